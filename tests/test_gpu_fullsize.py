"""Full-size workloads on the GPU, checked on sampled matrices and by
properties that hold at any size.

* llama layer (the benchmarked workload, in the benchmark's launch
  configuration): the whole step equals its phase composition bit for bit;
  momentum and Nesterov input bit for bit for all 218 M elements; O of Wk, Wv,
  Wq, gate (tall) and down (K = 14336) -- every distinct shape -- against the
  fp64 oracle; for every matrix, two size-independent properties of the exact
  iteration:
    - trace identity: ||O||_F^2 / s^2 = sum_i f^5(sigma_i)^2, with sigma_i the
      singular values of the normalized input (eigenvalues of U U^T, float64);
    - symmetry: (O/s) X0^T is symmetric, because every iterate is a
      polynomial in X0 X0^T times X0.
* MoE set and the 224-matrix owner share: sampled matrices (including the
  7168 x 18432 dense matrix) orthogonalized on their own (grouping invariance)
  match the oracle, and the full step's
  weights for those matrices equal the same-order apply of that O bit for bit,
  across all 8 shard slices.
"""

import numpy as np
import pytest

import workloads as wlm
from oracle import muon_oracle as mo
from oracle import same_order as so
from tests.gpu_helpers import TOL, bits, host, mat, param_slices, rel_fro, say

pytestmark = pytest.mark.gpu
H = wlm.HYPER
A_, B_, C_ = 3.4445, -4.7750, 2.0315


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


def quintic5(x):
    for _ in range(5):
        x = A_ * x + B_ * x ** 3 + C_ * x ** 5
    return x


def properties(torch, u_flat, o_flat, d):
    """(relative error of the trace identity, relative asymmetry of (O/s) X0^T)."""
    u = u_flat[d.offset:d.offset + d.rows * d.cols].view(d.rows, d.cols).double()
    o = o_flat[d.offset:d.offset + d.rows * d.cols].view(d.rows, d.cols).double()
    s = mo.shape_scale(d.rows, d.cols)
    if d.rows > d.cols:
        u, o = u.t(), o.t()
    x0 = u / (torch.linalg.matrix_norm(u) + 1e-7)
    lam = torch.linalg.eigvalsh(x0 @ x0.t()).clamp_min(0)
    want = float((quintic5(lam.sqrt()) ** 2).sum())
    got = float((o / s).pow(2).sum())
    sym = (o / s) @ x0.t()
    asym = float(torch.linalg.matrix_norm(sym - sym.t()) / torch.linalg.matrix_norm(sym))
    return abs(got - want) / want, asym


def test_llama_layer_full_size(nsf, torch):
    wl = wlm.make_workload("llama")
    say("llama full size: generate")
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    m0 = host(mom)
    p_step, m_step = params.clone(), mom.clone()
    say("llama full size: muon_step (bf16 MFMA)")
    nsf.muon_step(p_step, grads, m_step, wl.descs, H["lr"], H["weight_decay"], H["beta"])
    u = torch.zeros_like(grads)
    o = torch.zeros_like(grads)
    say("llama full size: composition")
    nsf.muon_momentum(grads, mom, u, wl.descs, H["beta"], True)
    nsf.muon_orthogonalize(u, o, wl.descs)
    nsf.muon_apply(params, o, wl.descs, H["lr"], H["weight_decay"])
    torch.cuda.synchronize()
    assert torch.equal(p_step.view(torch.int16), params.view(torch.int16))
    assert torch.equal(m_step.view(torch.int32), mom.view(torch.int32))
    gh, mh, uh, oh = host(grads), host(mom), host(u), host(o)
    for d in wl.descs:
        want_m, want_u = so.front(mat(gh, d), mat(m0, d), H["beta"], True)
        assert np.array_equal(bits(mat(mh, d)), bits(want_m))
        assert np.array_equal(bits(mat(uh, d)), bits(want_u))
    # every distinct shape against the fp64 oracle element by element: 1024 x 4096,
    # 4096 x 4096, 14336 x 4096 (tall, scale sqrt(3.5)) and 4096 x 14336 (K = 14336)
    for name in ("wk", "wv", "wq", "gate", "down"):
        d = wl.descs[wl.names.index(name)]
        err = rel_fro(mat(oh, d), mo.newton_schulz(mat(uh, d).astype(np.float64), 5))
        say("llama oracle", name, err)
        assert err <= TOL["bf16"]
    for name, d in zip(wl.names, wl.descs):
        tr, asym = properties(torch, u, o, d)
        say("llama properties", name, tr, asym)
        assert tr <= 2 * TOL["bf16"] and asym <= TOL["bf16"]


def _sampled_check(nsf, torch, wl, oracle_names, property_names=(), mode="bf16"):
    """Full step on the whole workload; sampled matrices re-orthogonalized on
    their own must match the oracle (or the size-independent properties), and
    the full step's momentum and weights for them must equal the same-order
    phases fed that O."""
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    names = list(oracle_names) + list(property_names)
    sample = [wl.descs[wl.names.index(nm)] for nm in names]

    def slices(d):
        per = d.rows * d.cols // d.n_shards
        return np.concatenate([host(params[d.param_offset + k * d.shard_stride:
                                           d.param_offset + k * d.shard_stride + per])
                               for k in range(d.n_shards)])

    def state(t, d):
        return host(t[d.offset:d.offset + d.rows * d.cols]).reshape(d.rows, d.cols)

    w0 = [slices(d) for d in sample]
    g_s = [state(grads, d) for d in sample]
    m_s = [state(mom, d) for d in sample]
    say(wl.name, "full step", mode, wl.n, "matrices")
    nsf.muon_step(params, grads, mom, wl.descs, H["lr"], H["weight_decay"], H["beta"], mode=mode)
    torch.cuda.synchronize()
    fronts = [so.front(g, m, H["beta"], True) for g, m in zip(g_s, m_s)]
    descs, off = [], 0
    for d in sample:
        descs.append(wlm.Desc(off, d.rows, d.cols, off))
        off += (d.rows * d.cols + 63) // 64 * 64
    u_flat = np.zeros(off, np.float32)
    for dd, (_, u) in zip(descs, fronts):
        u_flat[dd.offset:dd.offset + dd.rows * dd.cols] = u.reshape(-1)
    ut = torch.from_numpy(u_flat).cuda()
    ot = torch.zeros_like(ut)
    say(wl.name, "sampled matrices on their own", names)
    nsf.muon_orthogonalize(ut, ot, descs, mode=mode)
    torch.cuda.synchronize()
    oh = host(ot)
    for nm, d, dd, (m1, u), w in zip(names, sample, descs, fronts, w0):
        n = d.rows * d.cols
        assert np.array_equal(bits(state(mom, d)), bits(m1)), nm
        o = oh[dd.offset:dd.offset + n]
        if nm in oracle_names:
            err = rel_fro(o.reshape(d.rows, d.cols), mo.newton_schulz(u.astype(np.float64), 5))
            say(wl.name, "oracle", nm, err)
            assert err <= TOL[mode], nm
        else:
            tr, asym = properties(torch, ut, ot, dd)
            say(wl.name, "properties", nm, tr, asym)
            assert tr <= 2 * TOL[mode] and asym <= TOL[mode], nm
        want = so.apply(w, o, H["lr"], H["weight_decay"], wl.param_dtype)
        assert np.array_equal(bits(slices(d)), bits(want)), nm


def test_moe_set_sampled(nsf, torch):
    wl = wlm.make_workload("moe")
    _sampled_check(nsf, torch, wl, ["expert_up0", "expert_down63", "dense_up"], ["dense_down"])


def test_owner_share_sampled(nsf, torch):
    wl = wlm.make_workload("owner")
    _sampled_check(nsf, torch, wl, ["l0.wk", "l5.wq", "l31.wv", "l12.down"])
