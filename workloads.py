"""Seeded synthetic workloads for the flat-buffer Muon step.

This module only generates inputs (shapes, descriptors, random tensors); it
holds none of the step's arithmetic.  The tests and ``bench.py`` feed the same
generated tensors to the HIP path and to the CPU oracle.

Workloads (sizes of real models; values are synthetic, no dataset exists for
an optimizer step):

``single``   one float32 256 x 512 matrix; W, G ~ N(0, 0.02); M = 0.
``llama``    one Llama-style decoder layer (hidden 4096, 32 query / 8 key-value
             heads of 128, MLP 14336): Wq 4096x4096, Wk 1024x4096,
             Wv 1024x4096, Wo 4096x4096, gate 14336x4096, up 14336x4096,
             down 4096x14336; bfloat16 W ~ N(0, 0.02), float32 G ~ N(0, 1e-3),
             M = 0, contiguous in that order.
``batched``  512 float32 matrices whose sides are drawn independently,
             log-uniform on [128, 1024] and rounded to integers; one flat
             buffer, 256-byte aligned offsets; G ~ N(0, 1e-3).
``moe``      64 expert matrices 2048x7168 plus 64 of 7168x2048, and dense
             7168x18432 and 18432x7168 (a DeepSeek-V3-like set); bfloat16 W.
``owner``    one device's owner share of a 32-layer, 4096-hidden model: 32 x
             the ``llama`` layer (224 matrices) in layer-major flat G/M
             buffers, descriptors in a seeded random order, and every matrix's
             update scattered into 8 slices of 1/8 of the matrix each (slice k
             of every matrix lives in region k of the parameter buffer,
             standing in for 8 ranks' flat shards).

All use lr = 0.02, weight_decay = 0.01, beta = 0.95, Nesterov, 5 iterations.
Random tensors come from ``torch.Generator`` seeded per (workload, matrix,
kind), so any one matrix can be regenerated alone.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HYPER = dict(lr=0.02, weight_decay=0.01, beta=0.95, nesterov=True, ns_steps=5)
WORKLOADS = ("single", "llama", "batched", "moe", "owner")
_IDS = {name: i + 1 for i, name in enumerate(WORKLOADS)}
KIND_W, KIND_G, KIND_M = 0, 1, 2


@dataclass(frozen=True)
class Desc:
    offset: int
    rows: int
    cols: int
    param_offset: int
    shard_stride: int = 0
    n_shards: int = 1
    group: int = 0          # optimizer group (muon_step_grouped)


@dataclass
class Workload:
    name: str
    descs: list
    param_dtype: str          # "f32" or "bf16"
    n_param_elems: int
    n_state_elems: int
    w_std: float
    g_std: float
    names: list = field(default_factory=list)

    @property
    def n(self):
        return len(self.descs)

    def numel(self):
        return sum(d.rows * d.cols for d in self.descs)


def _align(v, a):
    return (v + a - 1) // a * a


def _contiguous(name, shapes, names, param_dtype, w_std, g_std):
    descs, off = [], 0
    for r, c in shapes:
        descs.append(Desc(off, r, c, off))
        off = _align(off + r * c, 64)
    return Workload(name, descs, param_dtype, off, off, w_std, g_std, list(names))


LLAMA_SHAPES = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
                (14336, 4096), (4096, 14336)]
LLAMA_NAMES = ["wq", "wk", "wv", "wo", "gate", "up", "down"]


def batched_shapes(count=512, seed=9):
    rng = np.random.default_rng([_IDS["batched"], 0, seed])
    lo, hi = math.log(128), math.log(1024)
    sides = np.rint(np.exp(rng.uniform(lo, hi, size=(count, 2)))).astype(int)
    return [(int(r), int(c)) for r, c in sides]


def make_workload(name: str, *, layers: int = 32, shards: int = 8) -> Workload:
    if name == "single":
        return _contiguous(name, [(256, 512)], ["w"], "f32", 0.02, 0.02)
    if name == "llama":
        return _contiguous(name, LLAMA_SHAPES, LLAMA_NAMES, "bf16", 0.02, 1e-3)
    if name == "batched":
        shapes = batched_shapes()
        return _contiguous(name, shapes, [f"m{i}" for i in range(len(shapes))], "f32", 0.02,
                           1e-3)
    if name == "moe":
        shapes = [(2048, 7168)] * 64 + [(7168, 2048)] * 64 + [(7168, 18432), (18432, 7168)]
        names = ([f"expert_up{i}" for i in range(64)] + [f"expert_down{i}" for i in range(64)]
                 + ["dense_up", "dense_down"])
        return _contiguous(name, shapes, names, "bf16", 0.02, 1e-3)
    if name == "owner":
        return owner_share(layers, shards)
    raise ValueError(f"unknown workload {name!r}")


def owner_share(layers=32, shards=8) -> Workload:
    shapes = LLAMA_SHAPES * layers
    names = [f"l{l}.{n}" for l in range(layers) for n in LLAMA_NAMES]
    state_off, off = [], 0
    for r, c in shapes:
        state_off.append(off)
        off = _align(off + r * c, 64)
    n_state = off
    slice_off, poff = [], 0
    for r, c in shapes:
        slice_off.append(poff)
        poff = _align(poff + r * c // shards, 64)
    region = poff
    descs = [Desc(state_off[i], r, c, slice_off[i], region, shards)
             for i, (r, c) in enumerate(shapes)]
    perm = np.random.default_rng([_IDS["owner"], 0, 9]).permutation(len(descs))
    return Workload("owner", [descs[i] for i in perm], "bf16", region * shards, n_state, 0.02,
                    1e-3, [names[i] for i in perm])


def seed_of(workload: str, matrix: int, kind: int) -> int:
    return (_IDS.get(workload, 99) * 1_000_003 + matrix) * 16 + kind


def _randn(n, std, seed, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(n, generator=g, device=device, dtype=torch.float32) * std


def make_tensors(wl: Workload, device="cuda", momentum_std: float = 0.0):
    """(params, grads, momentum) tensors on ``device``; params bf16 or f32.

    Matrix i's W, G (and M if momentum_std > 0) are drawn from generators
    seeded by (workload, i, kind), i being the descriptor's index in layer
    order (its position before any permutation is irrelevant: the seed uses
    the descriptor's state offset rank, which does not depend on order).
    """
    import torch
    pdt = torch.bfloat16 if wl.param_dtype == "bf16" else torch.float32
    params = torch.zeros(wl.n_param_elems, dtype=pdt, device=device)
    grads = torch.zeros(wl.n_state_elems, dtype=torch.float32, device=device)
    mom = torch.zeros(wl.n_state_elems, dtype=torch.float32, device=device)
    rank = {d.offset: k for k, d in enumerate(sorted(wl.descs, key=lambda d: d.offset))}
    for d in wl.descs:
        k = rank[d.offset]
        n = d.rows * d.cols
        w = _randn(n, wl.w_std, seed_of(wl.name, k, KIND_W), device).to(pdt)
        per = n // d.n_shards
        for s in range(d.n_shards):
            dst = d.param_offset + s * d.shard_stride
            params[dst:dst + per] = w[s * per:(s + 1) * per]
        grads[d.offset:d.offset + n] = _randn(n, wl.g_std, seed_of(wl.name, k, KIND_G), device)
        if momentum_std > 0:
            mom[d.offset:d.offset + n] = _randn(n, momentum_std, seed_of(wl.name, k, KIND_M),
                                                device)
    return params, grads, mom


def small_mixed(seed: int = 0, count: int = 6, max_side: int = 300, param_dtype="f32",
                shards: int = 1):
    """A small seeded workload of ragged shapes (parity tests at oracle speed).

    With shards > 1 every matrix's numel is made a multiple of 8 * shards and
    its slices are spread over ``shards`` regions with gaps between them.
    """
    rng = np.random.default_rng([77, seed])
    descs, off, poff = [], 0, 0
    shapes = []
    for _ in range(count):
        while True:
            r, c = (int(v) for v in rng.integers(1, max_side + 1, size=2))
            if shards == 1 or (r * c) % (8 * shards) == 0:
                break
        shapes.append((r, c))
    slice_offs = []
    for r, c in shapes:
        slice_offs.append(poff)
        poff = _align(poff + (r * c) // shards, 64) + (64 if shards > 1 else 0)
    region = poff
    for (r, c), so in zip(shapes, slice_offs):
        descs.append(Desc(off, r, c, so if shards > 1 else off, region if shards > 1 else 0,
                          shards))
        off = _align(off + r * c, 64) + 64  # gaps between matrices
    n_param = region * shards if shards > 1 else off
    return Workload(f"mixed{seed}", descs, param_dtype, n_param, off, 0.02, 1e-3,
                    [f"m{i}" for i in range(count)])
