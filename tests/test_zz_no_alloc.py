"""muon_step_noalloc (no device allocation: every intermediate in the library's
fixed per-GPU scratch array) against muon_step, through the C ABI.

Results must equal muon_step's bit for bit: the same kernels run on the same
inputs, only the memory holding the intermediates differs.  Two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents and tables); a set whose matrices fill the scratch in waves (the
llama layer); and a matrix too large for the scratch, rejected before
anything is enqueued.
"""

import numpy as np
import pytest

import workloads as wlm
from tests.gpu_helpers import bits, host, say

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


def _both(nsf, torch, wl, mode, ns_steps=5):
    """(params, momentum) after muon_step and after muon_step_noalloc, as bits."""
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    p1, m1 = params.clone(), mom.clone()
    nsf.muon_step(p1, grads, m1, wl.descs, H["lr"], H["weight_decay"], H["beta"],
                  ns_steps=ns_steps, mode=mode)
    torch.cuda.synchronize()
    p2, m2 = params.clone(), mom.clone()
    nsf.muon_step_noalloc(p2, grads, m2, wl.descs, H["lr"], H["weight_decay"], H["beta"],
                          ns_steps=ns_steps, mode=mode)
    torch.cuda.synchronize()
    return (bits(host(p1)), bits(host(m1))), (bits(host(p2)), bits(host(m2)))


@pytest.mark.parametrize("mode", ["bf16", "f32"])
def test_two_calls_second_smaller(nsf, torch, mode):
    big = wlm.small_mixed(51, count=8, max_side=700, param_dtype="bf16", shards=2)
    small = wlm.small_mixed(52, count=3, max_side=150, param_dtype="f32")
    for wl in (big, small):
        say("noalloc", mode, wl.name, [(d.rows, d.cols) for d in wl.descs])
        want, got = _both(nsf, torch, wl, mode)
        assert np.array_equal(got[0], want[0]), wl.name
        assert np.array_equal(got[1], want[1]), wl.name


def test_same_set_again_and_no_iterations(nsf, torch):
    """The resident tables are reused by a repeated set; ns_steps == 0 runs
    through the compact U region of the scratch."""
    wl = wlm.small_mixed(53, count=5, max_side=400, param_dtype="bf16")
    for ns in (5, 5, 0):
        say("noalloc repeat", wl.name, ns)
        want, got = _both(nsf, torch, wl, "bf16", ns_steps=ns)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_llama_layer_in_waves(nsf, torch):
    """1.2 GB of intermediates run through the 312 MiB scratch in waves."""
    wl = wlm.make_workload("llama")
    say("noalloc llama layer")
    want, got = _both(nsf, torch, wl, "bf16")
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_too_large_matrix_is_rejected(nsf, torch):
    rows, cols = 4096, 16384
    n = rows * cols
    params = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    grads = torch.ones(n, device="cuda")
    mom = torch.zeros(n, device="cuda")
    say("noalloc too large", rows, cols)
    with pytest.raises(nsf.MuonError, match="WORKSPACE_TOO_SMALL"):
        nsf.muon_step_noalloc(params, grads, mom, [(0, rows, cols)], H["lr"],
                              H["weight_decay"], H["beta"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(mom).item() == 0


def test_graph_capture_with_resident_tables(nsf, torch):
    """A call whose descriptor set has its tables resident is captured into a
    HIP graph; every replay equals an eager muon_step bit for bit.  A call with
    another set under capture is rejected before anything is enqueued, and the
    resident tables stay in place (the graph still replays correctly); outside
    capture that other set then runs as usual."""
    wl = wlm.small_mixed(54, count=4, max_side=300, param_dtype="bf16")
    other = wlm.small_mixed(55, count=2, max_side=200, param_dtype="bf16")
    args = (H["lr"], H["weight_decay"], H["beta"])
    params, grads, mom = wlm.make_tensors(wl, "cuda", momentum_std=1e-3)
    pe, me = params.clone(), mom.clone()
    ws = torch.empty(nsf.muon_workspace_bytes(wl.descs, "bf16"), dtype=torch.uint8, device="cuda")
    say("noalloc graph", wl.name)
    # the set's tables become resident (eager call on throwaway copies)
    nsf.muon_step_noalloc(params.clone(), grads, mom.clone(), wl.descs, *args)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            nsf.muon_step_noalloc(params, grads, mom, wl.descs, *args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def replay_and_compare(tag):
        graph.replay()
        nsf.muon_step(pe, grads, me, wl.descs, *args, workspace=ws)
        torch.cuda.synchronize()
        say("noalloc graph replay", tag)
        assert np.array_equal(bits(host(params)), bits(host(pe))), tag
        assert np.array_equal(bits(host(mom)), bits(host(me))), tag

    replay_and_compare(0)
    replay_and_compare(1)
    # another set under capture: rejected, nothing enqueued, tables kept
    p2, g2, m2 = wlm.make_tensors(other, "cuda", momentum_std=1e-3)
    m2_before = host(m2)
    probe = torch.zeros(4, device="cuda")
    g_other = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g_other):
            with pytest.raises(nsf.MuonError, match="BAD_ARG"):
                nsf.muon_step_noalloc(p2, g2, m2, other.descs, *args)
            probe.add_(1.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(host(m2), m2_before)
    replay_and_compare(2)
    # outside capture the other set runs (its tables replace the resident ones)
    say("noalloc other set eager", other.name)
    want, got = _both(nsf, torch, other, "bf16")
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
