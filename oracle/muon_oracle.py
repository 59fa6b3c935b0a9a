"""fp64 CPU oracle of one Muon optimizer step over flat buffers (test infrastructure only).

Sources (page title, then section):

* "Add initial Muon+M-FSDPv2 implementation" (Megatron-LM PR #6425), pseudocode
  block "Opt step": (1) update the optimizer state from the gradient and the
  state, (2) build the orthogonalization input from the state and, with
  Nesterov, the gradient, (4) orthogonalize the full matrix, (6) update the
  weights with the update.  Steps (3) and (5), the gather to the owner and the
  scatter back, are communication; on one device the "scatter back" is the
  write of each slice of the update to its destination in the flat buffer.
* "core.distributed.fsdp.src.megatron_fsdp.experimental.muon", class
  ``FsdpMuon``: ``_compute_momentum_inputs`` applies local weight decay,
  updates momentum and builds the orthogonalization inputs;
  ``_orthogonalize_updates`` replaces inputs by full orthogonalized updates;
  ``_apply_local_updates`` applies them to the (sharded) parameters.  Non-2-D
  parameters are not handled by this optimizer (class docstring,
  "Limitations").

The pages name the orthogonalization but not its algorithm.  This oracle uses
the quintic Newton-Schulz iteration that Muon is built on: Frobenius-normalize,
work on the wide orientation (transpose tall matrices), iterate
``X <- a X + (b A + c A^2) X`` with ``A = X X^T`` and
``(a, b, c) = (3.4445, -4.7750, 2.0315)``, then scale by
``sqrt(max(1, rows/cols))``.

Readings where the pages are silent (each is listed in the design notes):

* momentum is the SGD-style accumulator ``M <- beta M + G`` (an EMA form would
  only rescale M, and the normalization removes that scale from the update);
* the Nesterov input is ``G + beta M`` with the *updated* M (the state update is
  step 1, the input is built from it in step 2);
* weight decay is decoupled and multiplicative, ``W (1 - lr wd)``, applied
  before the update is subtracted;
* the normalization is ``X / (||X||_F + 1e-7)``;
* hyperparameters are rounded to float32 first (that is what the device sees)
  and then widened to float64.

Everything is computed in float64; inputs in float32 or bfloat16 convert to
float64 exactly.  Matrix products use NumPy's ``@`` on float64 arrays; no
blocking, fusion or reordering is added beyond the definitions above.

Pins (tests/test_oracle_pins.py): the momentum and decay closed forms on
constant and zero gradients, the singular-value closed form of the iteration
(``P diag(s) Q^T -> P diag(f^k(sigma)) Q^T``), exact rational values of the
scalar quintic on 1x1 inputs, rank-1 and orthogonal inputs, the output band of
the quintic, oddness / scale / orthogonal-equivariance / transposition
invariants, and layout equivalence of the flat-buffer scatter.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

#: Quintic Newton-Schulz coefficients (a, b, c) of Muon's orthogonalization.
NS_COEFFS = (3.4445, -4.7750, 2.0315)
#: Added to the Frobenius norm before dividing (keeps a zero matrix at zero).
NORM_EPS = 1e-7


@dataclass(frozen=True)
class MatrixDesc:
    """One 2-D parameter inside the flat buffers.

    ``offset``: position of the row-major rows x cols matrix in the flat
    gradient and momentum buffers.  ``param_offset``: position of its first
    slice in the flat parameter buffer.  The matrix is split into ``n_shards``
    contiguous slices of ``rows*cols/n_shards`` elements; slice ``k`` lives at
    ``param_offset + k*shard_stride`` in the parameter buffer (the owner's
    scatter of update slices to their shard destinations).
    """

    offset: int
    rows: int
    cols: int
    param_offset: int
    shard_stride: int = 0
    n_shards: int = 1


def as_f32_value(x: float) -> float:
    """A hyperparameter as the device sees it: rounded to float32, widened."""
    return float(np.float32(x))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 values (given as uint16 bit patterns)."""
    widened = bits.astype(np.uint32) << np.uint32(16)
    return widened.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Step (1) and (2) of "Opt step": state update and orthogonalization input.
# --------------------------------------------------------------------------

def momentum_update(grad: np.ndarray, momentum: np.ndarray, beta: float) -> np.ndarray:
    """Momentum state update ``M <- beta M + G`` (SGD-style accumulator)."""
    return beta * momentum + grad


def orthogonalization_input(grad: np.ndarray, new_momentum: np.ndarray, beta: float,
                            nesterov: bool) -> np.ndarray:
    """Input to the orthogonalization: ``G + beta M`` with Nesterov, else ``M``.

    ``new_momentum`` is the state *after* ``momentum_update`` of this step.
    """
    if nesterov:
        return grad + beta * new_momentum
    return new_momentum.copy()


# --------------------------------------------------------------------------
# Step (4) of "Opt step": orthogonalization of one full matrix.
# --------------------------------------------------------------------------

def shape_scale(rows: int, cols: int) -> float:
    """Update scale ``sqrt(max(1, rows/cols))`` from the original shape."""
    return math.sqrt(max(1.0, rows / cols))


def newton_schulz(update: np.ndarray, ns_steps: int) -> np.ndarray:
    """Quintic Newton-Schulz orthogonalization of one rows x cols matrix.

    Returns the full orthogonalized update in the original orientation,
    already multiplied by ``shape_scale(rows, cols)``.
    """
    rows, cols = update.shape
    tall = rows > cols
    # Work on the wide orientation so that A = X X^T is the small Gram matrix.
    x = np.ascontiguousarray(update.T if tall else update, dtype=np.float64)
    x = x / (np.linalg.norm(x) + NORM_EPS)  # Frobenius norm of the whole matrix
    a, b, c = NS_COEFFS
    for _ in range(ns_steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    out = np.ascontiguousarray(x.T) if tall else x
    return shape_scale(rows, cols) * out


def newton_schulz_left_factor(gram: np.ndarray, ns_steps: int) -> np.ndarray:
    """The same iteration for a wide or square U (rows <= cols), from its Gram
    matrix ``U U^T`` alone (float64, rows x rows): the matrix ``F`` with
    ``newton_schulz(U, ns_steps) == F @ U`` (the shape scale is 1 for such U).

    Every step multiplies the iterate on the left by ``a I + b A + c A^2`` with
    ``A = X X^T``; starting from ``X = U / (||U||_F + eps)`` each iterate is
    therefore ``X = P U`` with ``A = P (U U^T) P^T`` and ``||U||_F^2`` the
    trace of ``U U^T``.  For matrices too large to iterate on the host, the
    columns of the orthogonalized update are ``F u_j``.
    """
    p = np.eye(gram.shape[0]) / (math.sqrt(np.trace(gram)) + NORM_EPS)
    a, b, c = NS_COEFFS
    for _ in range(ns_steps):
        gram_x = p @ gram @ p.T
        poly = b * gram_x + c * (gram_x @ gram_x)
        p = a * p + poly @ p
    return p


# --------------------------------------------------------------------------
# Step (6) of "Opt step": decoupled decay and update of the weights.
# --------------------------------------------------------------------------

def apply_update(weight: np.ndarray, update: np.ndarray, lr: float,
                 weight_decay: float) -> np.ndarray:
    """``W <- W (1 - lr wd) - lr O`` (decay first, then the update)."""
    return weight * (1.0 - lr * weight_decay) - lr * update


# --------------------------------------------------------------------------
# The whole step over flat buffers.
# --------------------------------------------------------------------------

def _params_as_f64(params: np.ndarray, param_dtype: str) -> np.ndarray:
    if param_dtype == "bf16":
        if params.dtype != np.uint16:
            raise TypeError("bf16 parameters are passed as uint16 bit patterns")
        return bf16_bits_to_f64(params)
    if param_dtype == "f32":
        return params.astype(np.float64)
    raise ValueError(f"unknown param dtype {param_dtype!r}")


def gather_param(params64: np.ndarray, d: MatrixDesc) -> np.ndarray:
    """The rows x cols weight matrix assembled from its slices."""
    n = d.rows * d.cols
    per = n // d.n_shards
    parts = [params64[d.param_offset + k * d.shard_stride:
                      d.param_offset + k * d.shard_stride + per]
             for k in range(d.n_shards)]
    return np.concatenate(parts).reshape(d.rows, d.cols)


def scatter_param(params64: np.ndarray, d: MatrixDesc, weight: np.ndarray) -> None:
    """Write slice k of the flattened weight to ``param_offset + k*shard_stride``."""
    flat = weight.reshape(-1)
    per = flat.size // d.n_shards
    for k in range(d.n_shards):
        dst = d.param_offset + k * d.shard_stride
        params64[dst:dst + per] = flat[k * per:(k + 1) * per]


def step_matrix(weight: np.ndarray, grad: np.ndarray, momentum: np.ndarray, *, lr: float,
                weight_decay: float, beta: float, nesterov: bool, ns_steps: int):
    """One Muon step of one matrix, all arguments float64 rows x cols arrays.

    Hyperparameters must already be the float32-rounded values.
    Returns ``(new_weight, new_momentum, update)``.
    """
    new_m = momentum_update(grad, momentum, beta)
    u = orthogonalization_input(grad, new_m, beta, nesterov)
    o = newton_schulz(u, ns_steps)
    return apply_update(weight, o, lr, weight_decay), new_m, o


def muon_step(params: np.ndarray, grads: np.ndarray, momentum: np.ndarray, descs,
              *, lr: float, weight_decay: float, beta: float, nesterov: bool = True,
              ns_steps: int = 5, param_dtype: str = "f32", want_updates: bool = True):
    """One Muon step over flat buffers; every descriptor is a 2-D matrix.

    ``params`` is float32, or uint16 bfloat16 bit patterns when
    ``param_dtype == "bf16"``; ``grads`` and ``momentum`` are float32.
    Nothing is modified in place.  Returns ``(params64, momentum64, updates)``
    where ``updates[i]`` is descriptor ``i``'s full orthogonalized update
    (float64, rows x cols, scale included) if ``want_updates``.
    """
    lr, weight_decay, beta = (as_f32_value(v) for v in (lr, weight_decay, beta))
    p64 = _params_as_f64(params, param_dtype)
    m64 = momentum.astype(np.float64)
    updates = {}
    for i, d in enumerate(descs):
        n = d.rows * d.cols
        g = grads[d.offset:d.offset + n].astype(np.float64).reshape(d.rows, d.cols)
        m = m64[d.offset:d.offset + n].reshape(d.rows, d.cols)
        w = gather_param(p64, d)
        w_new, m_new, o = step_matrix(w, g, m, lr=lr, weight_decay=weight_decay, beta=beta,
                                      nesterov=nesterov, ns_steps=ns_steps)
        m64[d.offset:d.offset + n] = m_new.reshape(-1)
        scatter_param(p64, d, w_new)
        if want_updates:
            updates[i] = o
    return p64, m64, updates
