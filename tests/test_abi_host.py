"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, sizes workspaces, and rejects every invalid argument before touching
the GPU (these calls never reach a HIP call, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

import newton_schulz_flat_amd as nsf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_step.h")

ERR = {
    "NULL_POINTER": -1, "BAD_SHAPE": -2, "OUT_OF_BOUNDS": -3, "MISALIGNED": -4, "OVERLAP": -5,
    "ALIAS": -6, "BAD_ARG": -7, "WORKSPACE_TOO_SMALL": -8, "HIP": -9,
}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nsf.LIB_PATH):
        from newton_schulz_flat_amd import build
        build.build()
    return nsf.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(nsf.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.muon_status_string(0) == b"MUON_OK"
    for name, code in ERR.items():
        assert lib.muon_status_string(code) == ("MUON_ERR_" + name).encode()
    assert lib.muon_status_string(-1234) == b"MUON_ERR_UNKNOWN"


def descs(*items):
    return nsf.descs_array(items), len(items)


def ws_bytes(lib, items, mode=0):
    arr, n = descs(*items)
    out = ctypes.c_size_t(0)
    rc = lib.muon_workspace_bytes(arr, n, mode, ctypes.byref(out))
    return rc, out.value


def test_workspace_bytes_sizes(lib):
    rc, zero = ws_bytes(lib, [])
    assert rc == 0 and zero == 0
    rc, a = ws_bytes(lib, [(0, 256, 512)])
    assert rc == 0 and a % 256 == 0
    # two X iterates (bf16, 256 x 512 each) + A, B (256 x 256); the float32 U/O
    # region of ns_steps == 0 (4 B x 131072) overlays them
    assert a >= 2 * 2 * 256 * 512 + 2 * 2 * 256 * 256
    assert a < 4 * 131072 + 2 * 2 * 256 * 512 + 2 * 2 * 256 * 256
    rc, f = ws_bytes(lib, [(0, 256, 512)], mode=1)
    assert rc == 0 and f > a  # float32 intermediates are larger
    rc, two = ws_bytes(lib, [(0, 256, 512), (131072, 300, 17)])
    assert rc == 0 and two > a
    # the transposed shape needs the same intermediates
    assert ws_bytes(lib, [(0, 512, 256)])[1] == a


def ws_min_bytes(lib, items, mode=0):
    arr, n = descs(*items)
    out = ctypes.c_size_t(0)
    rc = lib.muon_workspace_min_bytes(arr, n, mode, ctypes.byref(out))
    return rc, out.value


def test_workspace_min_bytes(lib):
    one = [(0, 1024, 4096)]
    assert ws_min_bytes(lib, one) == ws_bytes(lib, one)  # one matrix: one wave either way
    many = [(k * 4096 * 1024, 1024, 4096) for k in range(6)] + [(6 * 4096 * 1024, 300, 17)]
    rc, lo = ws_min_bytes(lib, many)
    rc2, hi = ws_bytes(lib, many)
    assert rc == 0 and rc2 == 0 and lo < hi
    assert lo == ws_bytes(lib, [many[0]])[1]  # the largest single matrix
    assert ws_min_bytes(lib, [])[1] == 0
    arr, n = descs((0, 4, 4))
    assert lib.muon_workspace_min_bytes(arr, n, 0, None) == ERR["NULL_POINTER"]
    assert lib.muon_workspace_min_bytes(arr, n, 5, ctypes.byref(ctypes.c_size_t())) == ERR["BAD_ARG"]


@pytest.mark.parametrize("item,code", [
    ((0, 0, 5), "BAD_SHAPE"),
    ((0, 5, -1), "BAD_SHAPE"),
    ((0, 1 << 21, 4), "BAD_SHAPE"),
    ((0, (1 << 20) + 1, 1), "BAD_SHAPE"),   # one past the largest side
    ((0, 1, (1 << 20) + 1), "BAD_SHAPE"),
    ((0, 6, 6, 0, 20, 3), "BAD_SHAPE"),     # slice length 12 is not a multiple of 8
    ((0, 5, 5, 0, 0, 2), "BAD_SHAPE"),      # 25 % 2
    ((0, 8, 8, 0, 4, 4), "OVERLAP"),        # stride 4 < slice 16
    ((0, 8, 8, 0, 16, 0), "BAD_SHAPE"),     # n_shards 0
])
def test_workspace_bytes_rejects_bad_shapes(lib, item, code):
    rc, _ = ws_bytes(lib, [item])
    assert rc == ERR[code]
    assert lib.muon_last_error() != b""


def test_workspace_bytes_bounds_the_whole_set(lib):
    big = 1 << 17  # 2^17 x 2^17 = 2^34 elements, the largest matrix
    four = [(k << 34, big, big) for k in range(4)]           # 2^36 in total
    rc, b = ws_bytes(lib, four)
    assert rc == 0 and b > 0
    rc, _ = ws_bytes(lib, four + [(4 << 34, 1, 4)])          # four elements more
    assert rc == ERR["BAD_SHAPE"]
    assert b"in total" in lib.muon_last_error()


def test_workspace_bytes_accepts_largest_side(lib):
    for shape in [(0, 1 << 20, 1), (0, 1, 1 << 20)]:
        rc, b = ws_bytes(lib, [shape])
        assert rc == 0 and b > 0


def test_workspace_bytes_rejects_bad_mode_and_null(lib):
    arr, n = descs((0, 4, 4))
    out = ctypes.c_size_t()
    assert lib.muon_workspace_bytes(arr, n, 7, ctypes.byref(out)) == ERR["BAD_ARG"]
    assert lib.muon_workspace_bytes(arr, n, 0, None) == ERR["NULL_POINTER"]
    assert lib.muon_workspace_bytes(None, 1, 0, ctypes.byref(out)) == ERR["NULL_POINTER"]
    assert lib.muon_workspace_bytes(arr, -1, 0, ctypes.byref(out)) == ERR["BAD_ARG"]


# Fake device addresses: validation compares them as integers and never
# dereferences them.  Buffers are far apart so that they do not alias.
P, G, M, W = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000
BIG = 1 << 30


def step(lib, items, *, params=P, dtype=0, n_param=1 << 20, grads=G, momentum=M,
         n_state=1 << 20, lr=0.02, wd=0.01, beta=0.95, nesterov=1, ns=5, mode=0, ws=W,
         ws_size=BIG):
    arr, n = descs(*items)
    return lib.muon_step(params, dtype, n_param, grads, momentum, n_state, arr, n, lr, wd, beta,
                         nesterov, ns, mode, ws, ws_size, None)


GOOD = (0, 64, 32)


@pytest.mark.parametrize("kwargs,code", [
    (dict(params=None), "NULL_POINTER"),
    (dict(grads=None), "NULL_POINTER"),
    (dict(momentum=None), "NULL_POINTER"),
    (dict(ws=None), "NULL_POINTER"),
    (dict(dtype=5), "BAD_ARG"),
    (dict(mode=2), "BAD_ARG"),
    (dict(ns=-1), "BAD_ARG"),
    (dict(ns=65), "BAD_ARG"),
    (dict(nesterov=2), "BAD_ARG"),
    (dict(lr=float("nan")), "BAD_ARG"),
    (dict(wd=float("inf")), "BAD_ARG"),
    (dict(beta=float("-inf")), "BAD_ARG"),
    (dict(n_state=64 * 32 - 1), "OUT_OF_BOUNDS"),
    (dict(n_param=64 * 32 - 1), "OUT_OF_BOUNDS"),
    (dict(ws_size=1024), "WORKSPACE_TOO_SMALL"),
    (dict(ws=W + 16), "MISALIGNED"),
    (dict(grads=P + 64), "ALIAS"),
    (dict(momentum=G + 4 * 100), "ALIAS"),
    (dict(ws=M + 256), "ALIAS"),
])
def test_step_rejects(lib, kwargs, code):
    assert step(lib, [GOOD], **kwargs) == ERR[code]
    assert lib.muon_last_error() != b""


@pytest.mark.parametrize("items,kw,code", [
    ([(2, 8, 8)], {}, "MISALIGNED"),                       # state offset not 16-byte aligned
    ([(0, 8, 8, 2)], {}, "MISALIGNED"),                    # f32 param offset 2
    ([(0, 8, 8, 4)], dict(dtype=1), "MISALIGNED"),         # bf16 param offset 4 (8 bytes)
    ([(0, 8, 8, 8, 36, 2)], dict(dtype=1), "MISALIGNED"),  # bf16 slice 1 at element 44
    ([(-4, 8, 8)], {}, "OUT_OF_BOUNDS"),
    ([(0, 8, 8, -8)], {}, "OUT_OF_BOUNDS"),
    ([(0, 8, 8), (60, 2, 2, 100)], {}, "OVERLAP"),         # state ranges overlap
    ([(0, 8, 8, 0), (64, 8, 8, 32)], {}, "OVERLAP"),       # param ranges overlap
    ([(0, 8, 8, 0, 32, 2), (64, 4, 4, 40)], {}, "OVERLAP"),  # slice vs matrix
    ([(0, 8, 8, 0, 1 << 20, 2)], {}, "OUT_OF_BOUNDS"),     # slice 1 beyond params
    ([(0, 8, 8, 0, 0, 0, 1)], {}, "BAD_ARG"),              # group != 0 outside muon_step_grouped
])
def test_step_rejects_descriptors(lib, items, kw, code):
    arrs = []
    for it in items:
        arrs.append(it)
    if len(items[0]) == 7:  # group field set by hand
        arr = nsf.descs_array([items[0][:6]])
        arr[0].group = items[0][6]
        rc = lib.muon_step(P, 0, 1 << 20, G, M, 1 << 20, arr, 1, 0.02, 0.01, 0.95, 1, 5, 0, W,
                           BIG, None)
    else:
        rc = step(lib, arrs, **kw)
    assert rc == ERR[code], lib.muon_last_error()


def test_step_with_no_matrices_is_a_noop(lib):
    assert step(lib, [], params=None, grads=None, momentum=None, ws=None, ws_size=0) == 0


def test_phase_entry_points_validate(lib):
    arr, n = descs(GOOD)
    # momentum: aliasing u_out with grads
    assert lib.muon_momentum(G, M, G, 1 << 20, arr, n, 0.9, 1, None) == ERR["ALIAS"]
    assert lib.muon_momentum(G, M, None, 1 << 20, arr, n, 0.9, 1, None) == ERR["NULL_POINTER"]
    assert lib.muon_momentum(G, M, P, 100, arr, n, 0.9, 1, None) == ERR["OUT_OF_BOUNDS"]
    # orthogonalize: partial overlap of u and o_out is an alias, equality is in place
    assert lib.muon_orthogonalize(G, G + 16, 1 << 20, arr, n, 5, 0, W, BIG, None) == ERR["ALIAS"]
    assert lib.muon_orthogonalize(G, G, 1 << 20, arr, n, 5, 0, W, 16, None) == \
        ERR["WORKSPACE_TOO_SMALL"]
    assert lib.muon_orthogonalize(G, M, 1 << 20, arr, n, 99, 0, W, BIG, None) == ERR["BAD_ARG"]
    # apply
    assert lib.muon_apply(P, 0, 1 << 20, P, 1 << 20, arr, n, 0.1, 0.1, None) == ERR["ALIAS"]
    assert lib.muon_apply(P, 3, 1 << 20, G, 1 << 20, arr, n, 0.1, 0.1, None) == ERR["BAD_ARG"]
    assert lib.muon_apply(P, 0, 1 << 20, G, 1 << 20, arr, n, float("nan"), 0.1, None) == \
        ERR["BAD_ARG"]


def test_binding_refuses_cpu_tensors(lib):
    import torch
    t = torch.zeros(64 * 32)
    with pytest.raises((ValueError, TypeError)):
        nsf.muon_step(t, t, t, [GOOD], 0.02, 0.01, 0.95)


# ------------------------------------------------------------ muon_step_grouped

GR = 0x50_0000_0000   # fake device address of a group table
CP = 0x60_0000_0000   # fake device address of a bf16 model copy


def grouped(lib, items, *, params=P, dtype=0, n_param=1 << 20, copy=None, grads=G, momentum=M,
            n_state=1 << 20, groups=GR, n_groups=2, ns=5, mode=0, ws=W, ws_size=BIG):
    arr, n = descs(*items)
    return lib.muon_step_grouped(params, dtype, n_param, copy, grads, momentum, n_state, arr, n,
                                 groups, n_groups, ns, mode, ws, ws_size, None)


@pytest.mark.parametrize("items,kw,code", [
    ([(0, 8, 8, 0, 0, 1, 2)], {}, "BAD_ARG"),                   # group 2 of 2
    ([(0, 8, 8, 0, 0, 1, -1)], {}, "BAD_ARG"),                  # negative group
    ([(0, 8, 8)], dict(n_groups=0), "BAD_ARG"),
    ([(0, 8, 8)], dict(n_groups=65537), "BAD_ARG"),
    ([(0, 8, 8)], dict(groups=None), "NULL_POINTER"),
    ([(0, 8, 8)], dict(dtype=1, copy=CP), "BAD_ARG"),           # model copy needs f32 params
    ([(0, 8, 8)], dict(copy=CP + 8), "MISALIGNED"),
    ([(0, 8, 8)], dict(copy=P + 64), "ALIAS"),                  # copy inside params
    ([(0, 8, 8)], dict(groups=G + 64), "ALIAS"),                # group table inside grads
    ([(0, 8, 8)], dict(ns=65), "BAD_ARG"),
    ([(0, 8, 8)], dict(ws_size=16), "WORKSPACE_TOO_SMALL"),
])
def test_grouped_rejects(lib, items, kw, code):
    assert grouped(lib, items, **kw) == ERR[code], lib.muon_last_error()
    assert lib.muon_last_error() != b""


def test_grouped_accepts_groups_in_workspace_sizing(lib):
    # the workspace does not depend on groups: any group index >= 0 is sized
    assert ws_bytes(lib, [(0, 64, 32, 0, 0, 1, 7)]) == ws_bytes(lib, [(0, 64, 32)])
    assert ws_bytes(lib, [(0, 64, 32, 0, 0, 1, -1)])[0] == ERR["BAD_ARG"]


def test_grouped_no_matrices_is_a_noop(lib):
    assert grouped(lib, [], params=None, grads=None, momentum=None, groups=None, ws=None,
                   ws_size=0) == 0


def test_default_workspace_refused_under_capture(monkeypatch):
    """The default workspace cache cannot serve a call made under graph capture
    (a later, larger set could free it while the graph still points at it)."""
    import torch
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    with pytest.raises(RuntimeError, match="explicit workspace"):
        nsf.workspace_for([(0, 8, 8)], "bf16", "cuda:0")
