"""One matrix of more than 2^31 elements through muon_orthogonalize (C ABI).

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
