"""GPU tests of muon_step_grouped (per-matrix optimizer groups read from a
device table, the optional bfloat16 model copy, and HIP-graph capture).

* With one group it equals muon_step bit for bit; with several groups every
  matrix equals muon_step called with its own group's scalars, bit for bit.
* Against the fp64 oracle: per-group weight changes within the GEMM mode's
  tolerance, momentum bit for bit against the same-order float32 chain.
* The model copy is the round-to-nearest-even bfloat16 of the updated
  float32 weights, bit for bit.
* A captured graph replayed with different group values between replays
  matches the same sequence of eager calls after every replay, and the fp64
  oracle and same-order chain with that replay's groups.
"""

import dataclasses

import numpy as np
import pytest

import workloads as wlm
from oracle import muon_oracle as mo
from oracle import same_order as so
from tests.gpu_helpers import TOL, bits, host, mat, param_slices, rel_fro, say

pytestmark = pytest.mark.gpu

H = wlm.HYPER
# three optimizer groups: (lr, weight_decay, beta, nesterov)
GROUPS = [(0.02, 0.01, 0.95, True), (0.005, 0.0, 0.9, False), (0.05, 0.1, 0.8, True)]


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


def with_groups(descs, n_groups):
    return [dataclasses.replace(d, group=k % n_groups) for k, d in enumerate(descs)]


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("dtype,shards", [("f32", 1), ("bf16", 1), ("bf16", 4)])
def test_one_group_equals_step(nsf, torch, mode, dtype, shards):
    wl = wlm.small_mixed(31, count=6, max_side=280, param_dtype=dtype, shards=shards)
    say("grouped, one group == step", wl.name, mode, dtype, shards)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    p2, m2 = params.clone(), mom.clone()
    table = nsf.group_table([(H["lr"], H["weight_decay"], H["beta"], True)], "cuda")
    nsf.muon_step(params, grads, mom, wl.descs, H["lr"], H["weight_decay"], H["beta"], mode=mode)
    nsf.muon_step_grouped(p2, grads, m2, wl.descs, table, mode=mode)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(params)), bits(host(p2)))
    assert np.array_equal(bits(host(mom)), bits(host(m2)))


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("ns_steps", [5, 0])
def test_groups_equal_separate_steps(nsf, torch, mode, ns_steps):
    wl = wlm.small_mixed(32, count=7, max_side=300, param_dtype="bf16", shards=2)
    descs = with_groups(wl.descs, len(GROUPS))
    say("grouped == per-group steps", wl.name, mode, ns_steps)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    p2, m2 = params.clone(), mom.clone()
    nsf.muon_step_grouped(params, grads, mom, descs, nsf.group_table(GROUPS, "cuda"),
                          ns_steps=ns_steps, mode=mode)
    for k, (lr, wd, beta, nest) in enumerate(GROUPS):
        sub = [d for d in descs if d.group == k]
        sub = [dataclasses.replace(d, group=0) for d in sub]
        nsf.muon_step(p2, grads, m2, sub, lr, wd, beta, nesterov=nest, ns_steps=ns_steps,
                      mode=mode)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(params)), bits(host(p2)))
    assert np.array_equal(bits(host(mom)), bits(host(m2)))


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_groups_against_oracle(nsf, torch, mode):
    """float32 weights: W_before - W_after against the fp64 oracle with each
    matrix's own group; M bit for bit against the same-order chain."""
    wl = wlm.small_mixed(33, count=6, max_side=240, param_dtype="f32")
    descs = with_groups(wl.descs, len(GROUPS))
    say("grouped vs oracle", wl.name, mode)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    w_before, m_before, gh = host(params), host(mom), host(grads)
    nsf.muon_step_grouped(params, grads, mom, descs, nsf.group_table(GROUPS, "cuda"), mode=mode)
    torch.cuda.synchronize()
    w_after, m_after = host(params), host(mom)
    for d in descs:
        lr, wd, beta, nest = GROUPS[d.group]
        want_m, want_u = so.front(mat(gh, d), mat(m_before, d), beta, nest)
        assert np.array_equal(bits(mat(m_after, d)), bits(want_m)), d
        o = mo.newton_schulz(want_u.astype(np.float64), H["ns_steps"])
        lr64, wd64 = mo.as_f32_value(lr), mo.as_f32_value(wd)
        wb = param_slices(w_before, d).astype(np.float64).reshape(d.rows, d.cols)
        delta_want = wb * (lr64 * wd64) + lr64 * o
        delta_got = wb - param_slices(w_after, d).astype(np.float64).reshape(d.rows, d.cols)
        assert rel_fro(delta_got, delta_want) <= TOL[mode] + 1e-4, d


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("ns_steps", [5, 0])
def test_model_copy_is_rounded_weights(nsf, torch, mode, ns_steps):
    wl = wlm.small_mixed(34, count=5, max_side=260, param_dtype="f32", shards=4)
    descs = with_groups(wl.descs, 2)
    say("model copy", wl.name, mode, ns_steps)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    p2, m2 = params.clone(), mom.clone()
    copy = torch.zeros(params.numel(), dtype=torch.bfloat16, device="cuda")
    table = nsf.group_table(GROUPS[:2], "cuda")
    nsf.muon_step_grouped(params, grads, mom, descs, table, ns_steps=ns_steps, mode=mode,
                          model_copy=copy)
    nsf.muon_step_grouped(p2, grads, m2, descs, table, ns_steps=ns_steps, mode=mode)
    torch.cuda.synchronize()
    # the copy does not change the master update
    assert np.array_equal(bits(host(params)), bits(host(p2)))
    w = host(params)
    c = host(copy)
    for d in descs:
        got = param_slices(c, d)
        want = so.f32_to_bf16_bits(param_slices(w, d))
        assert np.array_equal(got, want), d
    # elements outside every slice are left alone
    covered = np.zeros(params.numel(), bool)
    for d in descs:
        per = d.rows * d.cols // d.n_shards
        for k in range(d.n_shards):
            s = d.param_offset + k * d.shard_stride
            covered[s:s + per] = True
    assert not np.any(c[~covered])


def _check_against_oracle(descs, rows, w_before, m_before, gh, w_after, m_after, mode):
    """M bit for bit against the same-order chain; W_before - W_after against
    the fp64 oracle with each matrix's group (float32 weights)."""
    for d in descs:
        lr, wd, beta, nest = rows[d.group]
        want_m, want_u = so.front(mat(gh, d), mat(m_before, d), beta, nest)
        assert np.array_equal(bits(mat(m_after, d)), bits(want_m)), d
        o = mo.newton_schulz(want_u.astype(np.float64), H["ns_steps"])
        lr64, wd64 = mo.as_f32_value(lr), mo.as_f32_value(wd)
        wb = param_slices(w_before, d).astype(np.float64).reshape(d.rows, d.cols)
        delta_want = wb * (lr64 * wd64) + lr64 * o
        delta_got = wb - param_slices(w_after, d).astype(np.float64).reshape(d.rows, d.cols)
        assert rel_fro(delta_got, delta_want) <= TOL[mode] + 1e-4, d


def test_graph_capture_replays_follow_the_table(nsf, torch):
    """Capture one grouped step (float32 master weights, bfloat16 model copy,
    slices in two shards) in a HIP graph; replay it three times, changing the
    device group table between replays (eager work, with synchronization,
    outside the graph).  After every replay: the same eager call bit for bit,
    M bit for bit against the same-order chain, the weight change against the
    fp64 oracle, and the model copy equal to the rounded weights."""
    wl = wlm.small_mixed(35, count=6, max_side=300, param_dtype="f32", shards=2)
    descs = with_groups(wl.descs, 2)
    mode = "bf16"
    say("graph capture", wl.name)
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    pe, me = params.clone(), mom.clone()
    copy = torch.zeros(params.numel(), dtype=torch.bfloat16, device="cuda")
    copy_e = torch.zeros_like(copy)
    table = nsf.group_table(GROUPS[:2], "cuda")
    eager_table = table.clone()
    ws = torch.empty(nsf.muon_workspace_bytes(descs, mode), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws)
    # first call (plan build) outside capture, on throwaway copies
    nsf.muon_step_grouped(params.clone(), grads, mom.clone(), descs, table, workspace=ws,
                          model_copy=copy.clone())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            nsf.muon_step_grouped(params, grads, mom, descs, table, workspace=ws,
                                  model_copy=copy)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gh = host(grads)
    schedules = [GROUPS[:2], [GROUPS[2], GROUPS[1]], [(0.01, 0.05, 0.5, False), GROUPS[0]]]
    for rep, rows in enumerate(schedules):
        new = nsf.group_table(rows, "cuda")
        table.copy_(new)
        eager_table.copy_(new)
        torch.cuda.synchronize()
        w_before, m_before = host(params), host(mom)
        graph.replay()
        nsf.muon_step_grouped(pe, grads, me, descs, eager_table, workspace=ws_e,
                              model_copy=copy_e)
        torch.cuda.synchronize()
        w_after, m_after = host(params), host(mom)
        say("graph replay", rep, rows)
        assert np.array_equal(bits(w_after), bits(host(pe))), rep
        assert np.array_equal(bits(m_after), bits(host(me))), rep
        assert np.array_equal(host(copy), host(copy_e)), rep
        _check_against_oracle(descs, rows, w_before, m_before, gh, w_after, m_after, mode)
        c = host(copy)
        for d in descs:
            assert np.array_equal(param_slices(c, d),
                                  so.f32_to_bf16_bits(param_slices(w_after, d))), (rep, d)
