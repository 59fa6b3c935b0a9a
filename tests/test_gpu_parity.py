"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* Elementwise phases (momentum / Nesterov input, decay + apply + scatter):
  bit for bit against the same-order float32 reference.
* Orthogonalization: per-matrix relative Frobenius error of O against the
  fp64 oracle, <= 1e-4 (float32 products) and <= 2.5e-2 (bfloat16 MFMA).
* The whole step equals the composition of its phases bit for bit, and does
  not depend on descriptor order, shard layout or repetition.
"""

import numpy as np
import pytest

import workloads as wlm
from oracle import muon_oracle as mo
from oracle import same_order as so
from tests.gpu_helpers import (TOL, bits, covered_mask, host, mat, param_slices, rel_fro,
                               say)

pytestmark = pytest.mark.gpu

H = wlm.HYPER


@pytest.fixture(scope="module")
def nsf():
    import newton_schulz_flat_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def gpu_sync(torch):
    torch.cuda.synchronize()


# ------------------------------------------------------------------ front

@pytest.mark.parametrize("nesterov", [True, False])
@pytest.mark.parametrize("seed", [0, 1])
def test_front_bit_exact(nsf, torch, nesterov, seed):
    wl = wlm.small_mixed(seed, count=7, max_side=300)
    say("front", wl.name, nesterov, [(d.rows, d.cols) for d in wl.descs])
    _, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=0.01)
    g0, m0 = host(grads), host(mom)
    u = torch.full_like(grads, 7.0)
    nsf.muon_momentum(grads, mom, u, wl.descs, H["beta"], nesterov)
    gpu_sync(torch)
    m1, u1 = host(mom), host(u)
    cov = covered_mask(g0.size, wl.descs, "state")
    for d in wl.descs:
        want_m, want_u = so.front(mat(g0, d), mat(m0, d), H["beta"], nesterov)
        assert np.array_equal(bits(mat(m1, d)), bits(want_m))
        assert np.array_equal(bits(mat(u1, d)), bits(want_u))
    assert np.array_equal(m1[~cov], m0[~cov])
    assert np.all(u1[~cov] == 7.0)


# ------------------------------------------------------------------ apply

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shards", [1, 4])
def test_apply_bit_exact(nsf, torch, dtype, shards):
    wl = wlm.small_mixed(3 + shards, count=6, max_side=256, param_dtype=dtype, shards=shards)
    say("apply", wl.name, dtype, shards, [(d.rows, d.cols) for d in wl.descs])
    params, grads, _ = wlm.make_tensors(wl, "cuda")
    o = torch.randn(wl.n_state_elems, device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    w0 = host(params)
    nsf.muon_apply(params, o, wl.descs, H["lr"], H["weight_decay"])
    gpu_sync(torch)
    w1, oh = host(params), host(o)
    for d in wl.descs:
        want = so.apply(param_slices(w0, d), mat(oh, d).reshape(-1), H["lr"], H["weight_decay"],
                        dtype)
        assert np.array_equal(bits(param_slices(w1, d)), bits(want))
    cov = covered_mask(w0.size, wl.descs, "param")
    assert np.array_equal(bits(w1[~cov]), bits(w0[~cov]))


# ------------------------------------------------------- orthogonalization

# every tile class (64: shorter side < 160; 128: < 1024; 256), ragged shapes in each
SHAPES = [(1, 1), (1, 7), (7, 1), (3, 5), (64, 64), (65, 129), (129, 65), (130, 1000),
          (1000, 130), (256, 512), (300, 300), (768, 769), (200, 1500), (1536, 800),
          (1100, 1301), (1301, 1100)]


def _orth_case(nsf, torch, shapes, mode, ns_steps, seed=0):
    descs, off = [], 0
    for r, c in shapes:
        descs.append(wlm.Desc(off, r, c, off))
        off += (r * c + 63) // 64 * 64 + 64
    g = torch.Generator("cuda").manual_seed(100 + seed)
    u = torch.randn(off, device="cuda", generator=g) * 1e-3
    o = torch.full_like(u, 3.0)
    nsf.muon_orthogonalize(u, o, descs, ns_steps=ns_steps, mode=mode)
    gpu_sync(torch)
    return descs, host(u), host(o)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("ns_steps", [0, 1, 5])
def test_orthogonalize_parity(nsf, torch, mode, ns_steps):
    say("orthogonalize", mode, ns_steps, SHAPES)
    descs, uh, oh = _orth_case(nsf, torch, SHAPES, mode, ns_steps)
    worst = 0.0
    for d in descs:
        want = mo.newton_schulz(mat(uh, d).astype(np.float64), ns_steps)
        err = rel_fro(mat(oh, d), want)
        worst = max(worst, err)
        assert err <= TOL[mode], (d.rows, d.cols, err)
    say("worst rel err", worst)
    cov = covered_mask(uh.size, descs, "state")
    assert np.all(oh[~cov] == 3.0)


# bfloat16 rounding of X, A and B accumulates over iterations (the quintic does
# not converge to a fixed point, it keeps the singular values oscillating in its
# band): a simulation with bfloat16 storage and float32 sums gives ~2.4e-3 at 2
# iterations, ~1e-2 at 5, ~2.4e-2 at 10 and 4.9-5.3e-2 at 64 on these sizes.
# The 64-iteration bound below still separates an off-by-one iteration count,
# which changes O by 0.41-0.43 relative.
COUNT_TOL = {("f32", 2): TOL["f32"], ("f32", 3): TOL["f32"], ("f32", 10): TOL["f32"],
             ("f32", 64): TOL["f32"], ("bf16", 2): TOL["bf16"], ("bf16", 3): TOL["bf16"],
             ("bf16", 64): 0.1}


@pytest.mark.parametrize("mode,ns_steps", sorted(COUNT_TOL))
def test_orthogonalize_iteration_counts(nsf, torch, mode, ns_steps):
    shapes = [(3, 5), (65, 129), (129, 65), (256, 512), (768, 769), (1100, 1301)]
    say("orthogonalize iterations", mode, ns_steps, shapes)
    descs, uh, oh = _orth_case(nsf, torch, shapes, mode, ns_steps, seed=3)
    worst = 0.0
    for d in descs:
        want = mo.newton_schulz(mat(uh, d).astype(np.float64), ns_steps)
        err = rel_fro(mat(oh, d), want)
        worst = max(worst, err)
        assert err <= COUNT_TOL[(mode, ns_steps)], (d.rows, d.cols, err)
    say("worst rel err", worst)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_orthogonalize_maximum_side(nsf, torch, mode):
    """The largest accepted side, 2^20, as a 1 x 2^20 and a 2^20 x 1 matrix: one
    64-tile Gram product with 16384 K blocks, 16384 stage-X tiles."""
    n = 1 << 20
    say("orthogonalize maximum side", mode, n)
    descs, uh, oh = _orth_case(nsf, torch, [(1, n), (n, 1)], mode, 5)
    for d in descs:
        want = mo.newton_schulz(mat(uh, d).astype(np.float64), 5)
        err = rel_fro(mat(oh, d), want)
        say("maximum side", (d.rows, d.cols), err)
        assert err <= TOL[mode], (d.rows, d.cols, err)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_many_tiny_matrices(nsf, torch, mode):
    """3000 matrices with sides 1..24 in one call: the matrix search over the
    prefix tables and the grouped tile tables at large matrix counts."""
    rng = np.random.default_rng(31)
    shapes = [tuple(int(v) for v in rng.integers(1, 25, size=2)) for _ in range(3000)]
    say("many tiny matrices", mode, len(shapes))
    descs, uh, oh = _orth_case(nsf, torch, shapes, mode, 5, seed=7)
    worst = 0.0
    for d in descs:
        want = mo.newton_schulz(mat(uh, d).astype(np.float64), 5)
        worst = max(worst, rel_fro(mat(oh, d), want))
    say("many tiny worst rel err", mode, worst)
    assert worst <= TOL[mode]
    cov = covered_mask(uh.size, descs, "state")
    assert np.all(oh[~cov] == 3.0)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("rank", [1, 8, 64])
def test_rank_deficient(nsf, torch, rank, mode):
    """Rank-deficient inputs U = P Q (P 1024 x rank, Q rank x 1024; 256 x rank,
    rank x 512).  The exact O lives in U's column and row spaces; what the
    iteration does with U's null space is not unique in finite precision: each
    step multiplies a perturbation there by f'(0) = a, so rounding noise of
    relative size e (float32 products over K terms: about sqrt(K) 2^-24) grows
    to about a^5 e.  Checked: the projection of O onto U's column and row spaces
    against the fp64 oracle within the mode's tolerance; in float32 also the
    rest of O within a^5 sqrt(K) 2^-24 of ||O||.  With bfloat16 iterates the
    rest reaches the order of ||O|| (a property of the bfloat16 iteration: a
    CPU emulation gives 118% at rank 1, 15-35% at ranks 8-64), so only its
    size is reported."""
    say("rank deficient", mode, rank)
    shapes = [(1024, 1024), (256, 512)]
    descs, off = [], 0
    for r, c in shapes:
        descs.append(wlm.Desc(off, r, c, off))
        off += (r * c + 63) // 64 * 64 + 64
    g = torch.Generator("cuda").manual_seed(300 + rank)
    u = torch.zeros(off, device="cuda")
    for d in descs:
        p = torch.randn(d.rows, rank, device="cuda", generator=g)
        q = torch.randn(rank, d.cols, device="cuda", generator=g)
        u[d.offset:d.offset + d.rows * d.cols] = (p @ q).reshape(-1) * 1e-3
    o = torch.zeros_like(u)
    nsf.muon_orthogonalize(u, o, descs, mode=mode)
    gpu_sync(torch)
    uh, oh = host(u), host(o)
    a5 = 3.4445 ** 5
    for d in descs:
        u64 = mat(uh, d).astype(np.float64)
        want = mo.newton_schulz(u64, 5)
        pl, sv, qr = np.linalg.svd(u64, full_matrices=False)
        # the float32 input itself carries rounding noise (~1e-7 relative) in
        # the null space: count only the singular values above it
        k = int(np.sum(sv > sv[0] * 1e-5))
        pk, qk = pl[:, :k], qr[:k].T
        got = mat(oh, d).astype(np.float64)
        def project(m):
            return pk @ (pk.T @ m @ qk) @ qk.T
        in_range = project(got)
        err_range = rel_fro(in_range, project(want))
        rest = np.linalg.norm(got - in_range) / np.linalg.norm(want)
        bound = a5 * np.sqrt(max(d.rows, d.cols)) * 2.0 ** -24  # K of the Gram product
        say("rank", mode, rank, (d.rows, d.cols), "k", k, "range", err_range, "rest", rest,
            "bound", bound)
        assert k == rank
        assert err_range <= TOL[mode], (rank, d.rows, d.cols, err_range)
        if mode == "f32":
            assert rest <= bound, (rank, d.rows, d.cols, rest, bound)


def test_orthogonalize_long_float32_contraction(nsf, torch):
    """float32 products: a 1024 x 33000 matrix (256-tile size, but a contraction
    past 32768) runs on 128-tiles whose Gram product restarts its accumulation
    chains after 1024 K blocks; O stays within the float32 tolerance."""
    say("orthogonalize long float32 contraction")
    descs, uh, oh = _orth_case(nsf, torch, [(1024, 33000), (33000, 1024)], "f32", 5)
    for d in descs:
        want = mo.newton_schulz(mat(uh, d).astype(np.float64), 5)
        err = rel_fro(mat(oh, d), want)
        say("long contraction", (d.rows, d.cols), err)
        assert err <= TOL["f32"], (d.rows, d.cols, err)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_orthogonalize_in_place(nsf, torch, mode):
    shapes = [(100, 37), (37, 100), (256, 256)]
    descs, off = [], 0
    for r, c in shapes:
        descs.append(wlm.Desc(off, r, c, off))
        off += (r * c + 63) // 64 * 64
    u = torch.randn(off, device="cuda", generator=torch.Generator("cuda").manual_seed(7))
    o = torch.empty_like(u)
    say("orthogonalize in place", mode)
    u0 = host(u)
    nsf.muon_orthogonalize(u, o, descs, mode=mode)
    nsf.muon_orthogonalize(u, u, descs, mode=mode)
    gpu_sync(torch)
    cov = covered_mask(off, descs, "state")
    uh, oh = host(u), host(o)
    assert np.array_equal(bits(uh[cov]), bits(oh[cov]))
    assert np.array_equal(bits(uh[~cov]), bits(u0[~cov]))  # gaps untouched


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_orthogonalize_zero_matrix_gives_zero(nsf, torch, mode):
    descs = [wlm.Desc(0, 40, 70, 0), wlm.Desc(2816, 70, 40, 2816)]
    u = torch.zeros(2816 * 2, device="cuda")
    o = torch.full_like(u, 1.0)
    nsf.muon_orthogonalize(u, o, descs, mode=mode)
    gpu_sync(torch)
    oh = host(o)
    assert np.all(oh[:2800] == 0.0) and np.all(oh[2816:2816 + 2800] == 0.0)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_tall_is_transpose_of_wide(nsf, torch, mode):
    """NS(G^T) = NS(G)^T: the tall path transposes in and out."""
    r, c = 200, 530
    g = torch.randn(r * c, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    gt = g.view(r, c).t().contiguous().view(-1)
    u = torch.cat([g, gt])
    o = torch.empty_like(u)
    descs = [wlm.Desc(0, r, c, 0), wlm.Desc(r * c, c, r, r * c)]
    say("tall vs wide", mode)
    nsf.muon_orthogonalize(u, o, descs, mode=mode)
    gpu_sync(torch)
    oh = host(o)
    wide = oh[:r * c].reshape(r, c)
    tall = oh[r * c:].reshape(c, r) / np.float32(np.sqrt(c / r))
    assert rel_fro(tall.T, wide) <= (1e-6 if mode == "f32" else 1e-2)


# ---------------------------------------------------------- whole step

def _step_copies(wl, torch, momentum_std=0.0):
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=momentum_std)
    return params, grads, mom


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("dtype,shards", [("f32", 1), ("bf16", 1), ("bf16", 4)])
def test_step_equals_composition(nsf, torch, mode, dtype, shards):
    wl = wlm.small_mixed(11, count=6, max_side=280, param_dtype=dtype, shards=shards)
    say("step == composition", wl.name, mode, dtype, shards)
    params, grads, mom = _step_copies(wl, torch, momentum_std=1e-3)
    p2, m2 = params.clone(), mom.clone()
    nsf.muon_step(params, grads, mom, wl.descs, H["lr"], H["weight_decay"], H["beta"],
                  mode=mode)
    u = torch.zeros_like(grads)
    o = torch.zeros_like(grads)
    nsf.muon_momentum(grads, m2, u, wl.descs, H["beta"], True)
    nsf.muon_orthogonalize(u, o, wl.descs, mode=mode)
    nsf.muon_apply(p2, o, wl.descs, H["lr"], H["weight_decay"])
    gpu_sync(torch)
    assert np.array_equal(bits(host(mom)), bits(host(m2)))
    assert np.array_equal(bits(host(params)), bits(host(p2)))


# Tall matrices through both block shapes of the front pass (32 x 128 blocks of
# U where the iterate's padded row count is a multiple of 128, else 64 x 64) in
# the 64-, 128- and 256-tile classes; all but one have rows whose length is not
# a multiple of 4, which the fused update of the 64/128-tile kernels handles
# element by element.
TALL_SHAPES = [(900, 771), (700, 301), (650, 201), (400, 150), (333, 97), (1030, 1029),
               (512, 200)]


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tall_blocks_and_unaligned_rows(nsf, torch, mode, dtype):
    """M bit for bit against the same-order reference, O against the fp64 oracle,
    and the whole step bit for bit against its composition (whose apply kernel
    matches the same-order reference bit for bit)."""
    descs, off = [], 0
    for r, c in TALL_SHAPES:
        descs.append(wlm.Desc(off, r, c, off))
        off = (off + r * c + 63) // 64 * 64 + 64
    wl = wlm.Workload("tall_blocks", descs, dtype, off, off, 0.02, 1e-3,
                      [f"m{i}" for i in range(len(descs))])
    say("tall blocks / unaligned rows", mode, dtype, TALL_SHAPES)
    params, grads, mom = _step_copies(wl, torch, momentum_std=1e-3)
    w0, m0, gh = host(params), host(mom), host(grads)
    p1, m1 = params.clone(), mom.clone()
    nsf.muon_step(p1, grads, m1, descs, H["lr"], H["weight_decay"], H["beta"], mode=mode)
    p2, m2 = params.clone(), mom.clone()
    u = torch.zeros_like(grads)
    o = torch.zeros_like(grads)
    nsf.muon_momentum(grads, m2, u, descs, H["beta"], True)
    nsf.muon_orthogonalize(u, o, descs, mode=mode)
    nsf.muon_apply(p2, o, descs, H["lr"], H["weight_decay"])
    gpu_sync(torch)
    oh, w1, w2 = host(o), host(p1), host(p2)
    assert np.array_equal(bits(host(m1)), bits(host(m2)))
    assert np.array_equal(bits(w1), bits(w2))
    for d in descs:
        want_m, want_u = so.front(mat(gh, d), mat(m0, d), H["beta"], True)
        assert np.array_equal(bits(mat(host(m1), d)), bits(want_m)), (d.rows, d.cols)
        want_o = mo.newton_schulz(want_u.astype(np.float64), H["ns_steps"])
        err = rel_fro(mat(oh, d), want_o)
        assert err <= TOL[mode], (d.rows, d.cols, err)
        want_w = so.apply(mat(w0, d).ravel(), mat(oh, d).ravel(), H["lr"], H["weight_decay"], dtype)
        assert np.array_equal(bits(mat(w1, d).ravel()), bits(want_w)), (d.rows, d.cols)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_three_steps_against_oracle(nsf, torch, mode):
    """Three consecutive steps (so M != 0): M bit for bit against the same-order
    chain; the weight change W_before - W_after against the fp64 oracle."""
    wl = wlm.make_workload("single")
    small = wlm.small_mixed(21, count=4, max_side=200)
    for w in (wl, small):
        say("three steps", w.name, mode)
        params, grads, mom = _step_copies(w, torch)
        gh = host(grads)
        for t in range(3):
            w_before, m_before = host(params), host(mom)
            nsf.muon_step(params, grads, mom, w.descs, H["lr"], H["weight_decay"], H["beta"],
                          mode=mode)
            gpu_sync(torch)
            w_after, m_after = host(params), host(mom)
            lr, wd = mo.as_f32_value(H["lr"]), mo.as_f32_value(H["weight_decay"])
            for d in w.descs:
                want_m, want_u = so.front(mat(gh, d), mat(m_before, d), H["beta"], True)
                assert np.array_equal(bits(mat(m_after, d)), bits(want_m))
                o = mo.newton_schulz(want_u.astype(np.float64), H["ns_steps"])
                wb = param_slices(w_before, d).astype(np.float64).reshape(d.rows, d.cols)
                delta_want = wb * (lr * wd) + lr * o
                delta_got = wb - param_slices(w_after, d).astype(np.float64).reshape(
                    d.rows, d.cols)
                assert rel_fro(delta_got, delta_want) <= TOL[mode] + 1e-4, (t, d)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_descriptor_order_and_repeat_invariance(nsf, torch, mode):
    wl = wlm.small_mixed(5, count=8, max_side=260, param_dtype="bf16")
    say("order invariance", wl.name, mode)
    params, grads, mom = _step_copies(wl, torch, momentum_std=1e-3)
    runs = []
    for order in (list(range(wl.n)), list(reversed(range(wl.n))), list(range(wl.n))):
        p, m = params.clone(), mom.clone()
        nsf.muon_step(p, grads, m, [wl.descs[i] for i in order], H["lr"], H["weight_decay"],
                      H["beta"], mode=mode)
        gpu_sync(torch)
        runs.append((bits(host(p)), bits(host(m))))
    for r in runs[1:]:
        assert np.array_equal(r[0], runs[0][0]) and np.array_equal(r[1], runs[0][1])


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_sharded_equals_contiguous(nsf, torch, mode):
    """Scattering each update into 8 slices leaves the values unchanged."""
    sharded = wlm.small_mixed(9, count=5, max_side=240, param_dtype="bf16", shards=8)
    contiguous = wlm.Workload("c", [wlm.Desc(d.offset, d.rows, d.cols, d.offset)
                                    for d in sharded.descs], "bf16", sharded.n_state_elems,
                              sharded.n_state_elems, 0.02, 1e-3)
    say("sharded vs contiguous", mode)
    ps, grads, mom = _step_copies(sharded, torch, momentum_std=1e-3)
    pc = torch.zeros(contiguous.n_param_elems, dtype=torch.bfloat16, device="cuda")
    hs = host(ps)
    for ds, dc in zip(sharded.descs, contiguous.descs):
        n = ds.rows * ds.cols
        pc[dc.offset:dc.offset + n] = torch.from_numpy(
            param_slices(hs, ds).view(np.int16).copy()).view(torch.bfloat16).cuda()
    m2 = mom.clone()
    nsf.muon_step(ps, grads, mom, sharded.descs, H["lr"], H["weight_decay"], H["beta"], mode=mode)
    nsf.muon_step(pc, grads, m2, contiguous.descs, H["lr"], H["weight_decay"], H["beta"],
                  mode=mode)
    gpu_sync(torch)
    hs, hc = host(ps), host(pc)
    for ds, dc in zip(sharded.descs, contiguous.descs):
        n = ds.rows * ds.cols
        assert np.array_equal(param_slices(hs, ds), hc[dc.offset:dc.offset + n])


def test_empty_descriptor_list_is_noop(nsf, torch):
    t = torch.zeros(16, device="cuda")
    nsf.muon_step(t, t.clone(), t.clone(), [], 0.1, 0.1, 0.9)
    nsf.muon_orthogonalize(t, t, [])
    gpu_sync(torch)
    assert torch.all(t == 0).item()


def test_zero_gradient_decays_exactly(nsf, torch):
    wl = wlm.small_mixed(2, count=3, max_side=150, param_dtype="bf16")
    params, grads, mom = _step_copies(wl, torch)
    grads.zero_()
    w0 = host(params)
    say("zero gradient")
    nsf.muon_step(params, grads, mom, wl.descs, H["lr"], H["weight_decay"], H["beta"])
    gpu_sync(torch)
    w1 = host(params)
    for d in wl.descs:
        want = so.apply(param_slices(w0, d), np.zeros(d.rows * d.cols, np.float32), H["lr"],
                        H["weight_decay"], "bf16")
        assert np.array_equal(param_slices(w1, d), want)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_non_finite_gradient_stays_in_its_matrix(nsf, torch, mode, bad):
    """A NaN or infinite gradient element (no special handling: it propagates
    through the method's arithmetic) makes that matrix's whole update NaN, as
    in the fp64 oracle, and changes nothing else: the other matrices' weights
    and every other momentum element equal a clean run bit for bit."""
    wl = wlm.small_mixed(12, count=5, max_side=260, param_dtype="bf16", shards=2)
    params, grads, mom = _step_copies(wl, torch, momentum_std=1e-3)
    p_clean, m_clean = params.clone(), mom.clone()
    nsf.muon_step(p_clean, grads, m_clean, wl.descs, H["lr"], H["weight_decay"], H["beta"],
                  mode=mode)
    d_bad = wl.descs[2]
    at = d_bad.offset + (d_bad.rows * d_bad.cols) // 2
    g_bad = grads.clone()
    g_bad[at] = bad
    say("non-finite gradient", mode, bad, (d_bad.rows, d_bad.cols), at)
    nsf.muon_step(params, g_bad, mom, wl.descs, H["lr"], H["weight_decay"], H["beta"], mode=mode)
    gpu_sync(torch)
    w1, wc = host(params), host(p_clean)
    m1, mc = host(mom), host(m_clean)
    with np.errstate(invalid="ignore"):
        o_bad = mo.newton_schulz(np.where(np.arange(d_bad.rows * d_bad.cols) == (at - d_bad.offset),
                                          bad, 1.0).reshape(d_bad.rows, d_bad.cols), 5)
    assert np.isnan(o_bad).all()  # the oracle: the whole update is NaN
    for d in wl.descs:
        if d is d_bad:
            assert np.isnan(mo.bf16_bits_to_f64(param_slices(w1, d))).all(), d
        else:
            assert np.array_equal(param_slices(w1, d), param_slices(wc, d)), d
    diff = np.flatnonzero(bits(m1) != bits(mc))
    assert list(diff) == [at]
    if np.isnan(bad):
        assert np.isnan(m1[at])
    else:
        assert m1[at] == bad


# ------------------------------------------------------- batched workload

@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_batched_512_matrices_parity(nsf, torch, mode):
    """The 512-matrix mixed-shape workload in full: every matrix against the oracle."""
    wl = wlm.make_workload("batched")
    say("batched", wl.n, mode)
    _, grads, _ = _step_copies(wl, torch)
    o = torch.zeros_like(grads)
    nsf.muon_orthogonalize(grads, o, wl.descs, mode=mode)
    gpu_sync(torch)
    gh, oh = host(grads), host(o)
    worst = 0.0
    for d in wl.descs:
        err = rel_fro(mat(oh, d), mo.newton_schulz(mat(gh, d).astype(np.float64), 5))
        worst = max(worst, err)
    say("batched worst rel err", mode, worst)
    assert worst <= TOL[mode]
