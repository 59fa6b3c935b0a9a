"""Shared helpers of the GPU tests: host copies, per-matrix views, tolerances."""

import sys

import numpy as np

#: Per-matrix relative Frobenius error bounds of O against the fp64 oracle.
#: float32 products: 1e-4; bfloat16 MFMA products (X, A, B stored bfloat16,
#: float32 accumulation and epilogues): 2.5e-2.
TOL = {"f32": 1e-4, "bf16": 2.5e-2}


def say(*args):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(*args, flush=True)
    sys.stdout.flush()


def host(t):
    """A torch tensor as a NumPy array; bfloat16 becomes uint16 bit patterns."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def mat(flat, d):
    n = d.rows * d.cols
    return flat[d.offset:d.offset + n].reshape(d.rows, d.cols)


def param_slices(flat, d):
    """The matrix's slices in the params buffer, concatenated (flattened matrix)."""
    n = d.rows * d.cols
    per = n // d.n_shards
    return np.concatenate([flat[d.param_offset + k * d.shard_stride:
                                d.param_offset + k * d.shard_stride + per]
                           for k in range(d.n_shards)])


def covered_mask(size, d_list, kind):
    m = np.zeros(size, bool)
    for d in d_list:
        n = d.rows * d.cols
        if kind == "state":
            m[d.offset:d.offset + n] = True
        else:
            per = n // d.n_shards
            for k in range(d.n_shards):
                s = d.param_offset + k * d.shard_stride
                m[s:s + per] = True
    return m


def rel_fro(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return num / den if den > 0 else num


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)
