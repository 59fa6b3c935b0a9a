"""Sizes beyond int32 element counts and beyond one launch grid (C ABI).

One matrix of more than 2^31 elements through muon_orthogonalize and
muon_step; and a set of more than 2^24 elementwise chunks through
muon_momentum and muon_apply, whose kernels then run as several launches.

2100 x 2^20 (the longest side the library takes): every kernel indexes it
with 64-bit offsets; bfloat16 products on 256-tiles, rows padded to 2304,
stage A contracting over K = 2^20.  The host cannot iterate on a matrix this
size, so the check uses the oracle's Gram form: every iterate of a wide
matrix is P U, and O = F U with F = newton_schulz_left_factor(U U^T, 5)
(pinned against the direct iteration and the singular-value closed form).
The fp64 Gram matrix U U^T is summed on the host over column chunks; then
sampled columns of O against F u_j (the first and last columns included: the
last rows' elements lie beyond 2^31), and every column at once through
||O||_F = sqrt(trace(F (U U^T) F^T)).
"""

import numpy as np
import pytest

import workloads as wlm
from oracle import muon_oracle as mo
from oracle import same_order as so
from tests.gpu_helpers import TOL, rel_fro, say

pytestmark = pytest.mark.gpu

ROWS, COLS = 2100, 2 ** 20  # 2,202,009,600 elements
CHUNK = 2 ** 16             # columns per host chunk


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


def test_matrix_beyond_int32_elements(nsf, torch):
    n = ROWS * COLS
    assert n > 2 ** 31
    descs = [(0, ROWS, COLS)]
    say("large matrix", ROWS, "x", COLS, "=", n, "elements")
    u = wlm._randn(n, 1.0, wlm.seed_of("large", 0, 0), "cuda")
    o = torch.empty_like(u)
    ws = torch.empty(nsf.muon_workspace_bytes(descs, "bf16"), dtype=torch.uint8, device="cuda")
    say("large matrix: muon_orthogonalize, workspace", ws.numel(), "bytes")
    nsf.muon_orthogonalize(u, o, descs, ns_steps=5, mode="bf16", workspace=ws)
    torch.cuda.synchronize()
    del ws
    torch.cuda.empty_cache()

    say("large matrix: host Gram sum")
    u2, o2 = u.view(ROWS, COLS), o.view(ROWS, COLS)
    uu = np.zeros((ROWS, ROWS))
    oo_trace = 0.0
    for j0 in range(0, COLS, CHUNK):
        ub = u2[:, j0:j0 + CHUNK].cpu().numpy().astype(np.float64)
        ob = o2[:, j0:j0 + CHUNK].cpu().numpy().astype(np.float64)
        assert np.isfinite(ob).all(), j0
        uu += ub @ ub.T
        oo_trace += float(np.sum(ob * ob))
    f = mo.newton_schulz_left_factor(uu, 5)

    rng = np.random.default_rng(11)
    cols = np.unique(np.concatenate([[0, 1, COLS - 2, COLS - 1],
                                     rng.choice(COLS, 2000, replace=False)]))
    idx = torch.from_numpy(cols).to("cuda")
    us = u2[:, idx].cpu().numpy().astype(np.float64)
    got = o2[:, idx].cpu().numpy().astype(np.float64)
    err_cols = rel_fro(got, f @ us)
    want_norm = float(np.sqrt(np.trace(f @ uu @ f.T)))
    err_norm = abs(np.sqrt(oo_trace) - want_norm) / want_norm
    say("large matrix: sampled columns", err_cols, "||O||", np.sqrt(oo_trace), "vs", want_norm)
    assert err_cols <= TOL["bf16"]
    assert err_norm <= TOL["bf16"]
    del u, o, u2, o2
    torch.cuda.empty_cache()


def test_step_beyond_int32_elements_sharded(nsf, torch):
    """The whole step (fused decay and update) on the same shape with float32
    master weights cut into 8 slices 4096 elements apart: slices start past
    2^31 in the params buffer.  M0 = 0, so M1 = G and U = G + beta G; the
    normalization removes U's scale, so O = F G with F from G G^T.  Checks: M
    equals G bit for bit everywhere, the gaps between slices are untouched,
    and the weight change at sampled columns against the oracle's
    decay-then-update with that O."""
    n = ROWS * COLS
    shards, gap = 8, 4096
    per = n // shards
    stride = per + gap
    h = wlm.HYPER
    descs = [(0, ROWS, COLS, 0, stride, shards)]
    say("large step", ROWS, "x", COLS, "in", shards, "slices of", per)
    params = torch.full((shards * stride,), 7.0, device="cuda")
    for s in range(shards):
        params[s * stride:s * stride + per] = wlm._randn(per, 0.02, wlm.seed_of("large", 1, s),
                                                          "cuda")
    grads = wlm._randn(n, 1e-3, wlm.seed_of("large", 2, 0), "cuda")
    mom = torch.zeros_like(grads)
    rng = np.random.default_rng(12)
    cols = np.unique(np.concatenate([[0, COLS - 1], rng.choice(COLS, 2000, replace=False)]))
    elem = (np.arange(ROWS)[:, None] * COLS + cols[None, :]).astype(np.int64)
    dst = (elem // per) * stride + elem % per
    dst_t = torch.from_numpy(dst.reshape(-1)).to("cuda")
    w_before = params[dst_t].cpu().numpy().astype(np.float64).reshape(dst.shape)
    ws = torch.empty(nsf.muon_workspace_bytes(descs, "bf16"), dtype=torch.uint8, device="cuda")
    say("large step: muon_step, workspace", ws.numel(), "bytes")
    nsf.muon_step(params, grads, mom, descs, h["lr"], h["weight_decay"], h["beta"],
                  ns_steps=5, mode="bf16", workspace=ws)
    torch.cuda.synchronize()
    del ws
    torch.cuda.empty_cache()
    assert torch.equal(mom, grads)
    for s in range(shards):
        assert bool((params[s * stride + per:(s + 1) * stride] == 7.0).all()), s
    w_after = params[dst_t].cpu().numpy().astype(np.float64).reshape(dst.shape)

    say("large step: host Gram sum")
    g2 = grads.view(ROWS, COLS)
    gg = np.zeros((ROWS, ROWS))
    for j0 in range(0, COLS, CHUNK):
        gb = g2[:, j0:j0 + CHUNK].cpu().numpy().astype(np.float64)
        gg += gb @ gb.T
    f = mo.newton_schulz_left_factor(gg, 5)
    idx = torch.from_numpy(cols).to("cuda")
    o = f @ g2[:, idx].cpu().numpy().astype(np.float64)
    lr, wd = mo.as_f32_value(h["lr"]), mo.as_f32_value(h["weight_decay"])
    want = w_before - mo.apply_update(w_before, o, lr, wd)
    err = rel_fro(w_before - w_after, want)
    say("large step: weight change at sampled columns", err)
    assert err <= TOL["bf16"] + 1e-4
    del params, grads, mom, g2
    torch.cuda.empty_cache()


def test_elementwise_over_two_launch_grids(nsf, torch):
    """A set of 8.59 G elements (8 matrices of 1024 x 2^20 and one of
    1024 x 1024) is more than 2^24 workgroups of 512 elements, so the momentum
    and apply kernels each run as two launches.  Sampled elements (the last of
    the first grid, the first of the second, the ends of the set, and random
    ones on both sides) bit-exact against the same-order float32 reference."""
    shapes = [(1024, 2 ** 20)] * 8 + [(1024, 1024)]
    descs, n = [], 0
    for r, c in shapes:
        descs.append((n, r, c))
        n += r * c
    first_grid = 2 ** 24 * 512  # elements the first launch covers
    assert n > first_grid
    h = wlm.HYPER
    say("two grids:", n, "elements")
    rng = np.random.default_rng(13)
    idx = np.unique(np.concatenate([
        [0, 1, first_grid - 5, first_grid - 1, first_grid, first_grid + 1, n - 2, n - 1],
        rng.integers(0, n, 20000), rng.integers(first_grid, n, 4000)])).astype(np.int64)
    idx_t = torch.from_numpy(idx).to("cuda")
    grads = wlm._randn(n, 1e-3, wlm.seed_of("grids", 0, 0), "cuda")
    mom = wlm._randn(n, 1e-3, wlm.seed_of("grids", 1, 0), "cuda")
    g_s = grads[idx_t].cpu().numpy()
    m_s = mom[idx_t].cpu().numpy()
    u = torch.empty_like(grads)
    say("two grids: muon_momentum")
    nsf.muon_momentum(grads, mom, u, descs, h["beta"], h["nesterov"])
    torch.cuda.synchronize()
    m1, u1 = so.front(g_s, m_s, h["beta"], h["nesterov"])
    assert np.array_equal(mom[idx_t].cpu().numpy().view(np.uint32), m1.view(np.uint32))
    assert np.array_equal(u[idx_t].cpu().numpy().view(np.uint32), u1.view(np.uint32))
    del grads, mom
    torch.cuda.empty_cache()

    params = wlm._randn(n, 0.02, wlm.seed_of("grids", 2, 0), "cuda").to(torch.bfloat16)
    torch.cuda.empty_cache()
    w_s = params[idx_t].view(torch.int16).cpu().numpy().view(np.uint16)
    o_s = u[idx_t].cpu().numpy()
    say("two grids: muon_apply")
    nsf.muon_apply(params, u, descs, h["lr"], h["weight_decay"])
    torch.cuda.synchronize()
    want = so.apply(w_s, o_s, h["lr"], h["weight_decay"], "bf16")
    got = params[idx_t].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    del params, u
    torch.cuda.empty_cache()
