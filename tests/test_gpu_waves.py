"""Workspace-bounded waves and the compact U region, on the GPU.

A workspace smaller than muon_workspace_bytes (but at least
muon_workspace_min_bytes) runs the matrices in waves that each fit it.  Each
matrix's arithmetic does not depend on which wave it runs in, so results must
equal the one-wave run bit for bit; O is also checked against the fp64 oracle.
muon_step with ns_steps == 0 keeps U and O in a compact region overlaying the
Newton-Schulz intermediates; it must equal the composition of the phases bit
for bit.
"""

import numpy as np
import pytest

import workloads as wlm
from oracle import muon_oracle as mo
from oracle import same_order as so
from tests.gpu_helpers import TOL, bits, host, mat, param_slices, rel_fro, say

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


def _sizes(nsf, descs, mode):
    full = nsf.muon_workspace_bytes(descs, mode)
    low = nsf.muon_workspace_min_bytes(descs, mode)
    assert 0 < low < full, (low, full)
    return full, low


def _ws(torch, nbytes):
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("ns_steps", [5, 0])
@pytest.mark.parametrize("dtype,shards", [("bf16", 1), ("f32", 4)])
def test_step_in_waves_equals_one_wave(nsf, torch, mode, ns_steps, dtype, shards):
    wl = wlm.small_mixed(41 + shards, count=8, max_side=420, param_dtype=dtype, shards=shards)
    full, low = _sizes(nsf, wl.descs, mode)
    mid = (full + low) // 2
    say("waves", wl.name, mode, ns_steps, dtype, shards, "bytes", full, mid, low)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    runs = []
    for nbytes in (full, mid, low):
        p, m = params.clone(), mom.clone()
        nsf.muon_step(p, grads, m, wl.descs, H["lr"], H["weight_decay"], H["beta"],
                      ns_steps=ns_steps, mode=mode, workspace=_ws(torch, nbytes))
        torch.cuda.synchronize()
        runs.append((bits(host(p)), bits(host(m))))
    for r in runs[1:]:
        assert np.array_equal(r[0], runs[0][0]) and np.array_equal(r[1], runs[0][1])


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_orthogonalize_in_waves_against_oracle(nsf, torch, mode):
    """The smallest workspace (one matrix per wave for these shapes) against
    the one-wave run bit for bit and against the fp64 oracle."""
    shapes = [(600, 900), (900, 600), (300, 1200), (257, 513), (1024, 1024), (70, 90)]
    descs, off = [], 0
    for r, c in shapes:
        descs.append(wlm.Desc(off, r, c, off))
        off += (r * c + 63) // 64 * 64 + 64
    full, low = _sizes(nsf, descs, mode)
    say("orthogonalize in waves", mode, shapes, full, low)
    u = torch.randn(off, device="cuda", generator=torch.Generator("cuda").manual_seed(61)) * 1e-3
    o1 = torch.full_like(u, 5.0)
    o2 = torch.full_like(u, 5.0)
    nsf.muon_orthogonalize(u, o1, descs, mode=mode, workspace=_ws(torch, full))
    nsf.muon_orthogonalize(u, o2, descs, mode=mode, workspace=_ws(torch, low))
    torch.cuda.synchronize()
    uh, oh1, oh2 = host(u), host(o1), host(o2)
    assert np.array_equal(bits(oh1), bits(oh2))
    for d in descs:
        err = rel_fro(mat(oh2, d), mo.newton_schulz(mat(uh, d).astype(np.float64), 5))
        say("waves oracle", (d.rows, d.cols), err)
        assert err <= TOL[mode], (d.rows, d.cols, err)


def test_grouped_step_in_waves(nsf, torch):
    """Per-matrix optimizer groups and the bfloat16 model copy through waves."""
    wl = wlm.small_mixed(47, count=7, max_side=380, param_dtype="f32")
    descs = [wlm.Desc(d.offset, d.rows, d.cols, d.param_offset, d.shard_stride, d.n_shards,
                      k % 2) for k, d in enumerate(wl.descs)]
    table = nsf.group_table([(0.02, 0.01, 0.95, True), (0.01, 0.1, 0.9, False)], "cuda")
    full, low = _sizes(nsf, descs, "bf16")
    say("grouped waves", wl.name, full, low)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    runs = []
    for nbytes in (full, low):
        p, m = params.clone(), mom.clone()
        copy = torch.zeros(p.numel(), dtype=torch.bfloat16, device="cuda")
        nsf.muon_step_grouped(p, grads, m, descs, table, model_copy=copy,
                              workspace=_ws(torch, nbytes))
        torch.cuda.synchronize()
        runs.append((bits(host(p)), bits(host(m)), host(copy)))
    for a, b in zip(runs[0], runs[1]):
        assert np.array_equal(a, b)


def test_workspace_below_minimum_is_rejected(nsf, torch):
    wl = wlm.small_mixed(43, count=3, max_side=200)
    _, low = _sizes(nsf, wl.descs, "bf16")
    params, grads, mom = wlm.make_tensors(wl, "cuda")
    p0 = host(params)
    with pytest.raises(nsf.MuonError, match="WORKSPACE_TOO_SMALL"):
        nsf.muon_step(params, grads, mom, wl.descs, H["lr"], H["weight_decay"], H["beta"],
                      workspace=_ws(torch, low - 256))
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(params)), bits(p0))


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_without_iterations_equals_composition(nsf, torch, mode, dtype):
    """ns_steps == 0: U and O live in the compact region over the unused
    Newton-Schulz intermediates; the step equals momentum -> orthogonalize ->
    apply bit for bit, and M and W match the same-order reference."""
    wl = wlm.small_mixed(45, count=6, max_side=300, param_dtype=dtype)
    say("step ns_steps=0", wl.name, mode, dtype)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    w0, m0, gh = host(params), host(mom), host(grads)
    p1, m1 = params.clone(), mom.clone()
    nsf.muon_step(p1, grads, m1, wl.descs, H["lr"], H["weight_decay"], H["beta"], ns_steps=0,
                  mode=mode)
    p2, m2 = params.clone(), mom.clone()
    u = torch.zeros_like(grads)
    o = torch.zeros_like(grads)
    nsf.muon_momentum(grads, m2, u, wl.descs, H["beta"], True)
    nsf.muon_orthogonalize(u, o, wl.descs, ns_steps=0, mode=mode)
    nsf.muon_apply(p2, o, wl.descs, H["lr"], H["weight_decay"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(m1)), bits(host(m2)))
    assert np.array_equal(bits(host(p1)), bits(host(p2)))
    oh, w1 = host(o), host(p1)
    for d in wl.descs:
        want_m, want_u = so.front(mat(gh, d), mat(m0, d), H["beta"], True)
        assert np.array_equal(bits(mat(host(m1), d)), bits(want_m))
        err = rel_fro(mat(oh, d), mo.newton_schulz(want_u.astype(np.float64), 0))
        assert err <= TOL[mode], (d.rows, d.cols, err)
        want_w = so.apply(param_slices(w0, d), mat(oh, d).ravel(), H["lr"], H["weight_decay"],
                          dtype)
        assert np.array_equal(bits(param_slices(w1, d)), bits(want_w))
