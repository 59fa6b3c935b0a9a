"""Same-order float32 reference of the elementwise phases (test infrastructure only).

The device's elementwise kernels are checked bit for bit against this module.
Each line below is one IEEE-754 binary32 operation with round-to-nearest-even;
NumPy float32 arithmetic never fuses a multiply and an add, so every product
and every sum is rounded on its own, exactly as in the device kernels (which
are compiled with floating-point contraction off).

Operation order (``fl`` = round to float32):

* momentum (step 1 of "Opt step", page "Add initial Muon+M-FSDPv2
  implementation"):       ``M1 = fl(fl(beta*M) + G)``
* orthogonalization input (step 2): ``U = fl(fl(beta*M1) + G)`` with Nesterov,
  else ``U = M1``
* decay factor, on the host: ``f = fl(1 - fl(lr*wd))``
* apply (step 6, and ``FsdpMuon._apply_local_updates`` on the page
  "core.distributed.fsdp.src.megatron_fsdp.experimental.muon"):
  ``W1 = fl(W*f)``, ``Wn = fl(W1 - fl(lr*O))`` where ``O`` is the float32
  orthogonalized update with its shape scale already applied; the result is
  stored as float32 or rounded once to bfloat16 (round to nearest even).

Pins (tests/test_oracle_pins.py): every operation is checked on random and
constructed inputs against exact rational arithmetic (``fractions.Fraction``)
followed by a brute-force correctly rounded conversion to float32; the
bfloat16 rounding is checked against the IEEE definition of round-to-nearest-
even on the bit pattern neighbours, including ties, infinities and NaN.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns uint16 bits.

    NaN maps to a quiet NaN with the same sign and top payload bits.
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    is_nan = np.isnan(x.astype(np.float32))
    quiet = ((bits >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return np.where(is_nan, quiet, rounded)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def front(grad: np.ndarray, momentum: np.ndarray, beta: float, nesterov: bool):
    """Momentum update and orthogonalization input; returns ``(M1, U)`` float32."""
    g = grad.astype(np.float32, copy=False)
    m = momentum.astype(np.float32, copy=False)
    b = F32(beta)
    m1 = (b * m) + g
    if nesterov:
        u = (b * m1) + g
    else:
        u = m1.copy()
    return m1.astype(np.float32), u.astype(np.float32)


def decay_factor(lr: float, weight_decay: float) -> np.float32:
    """``f = fl(1 - fl(lr*wd))`` computed in float32, as the host does."""
    return F32(F32(1.0) - F32(F32(lr) * F32(weight_decay)))


def apply(weight: np.ndarray, update: np.ndarray, lr: float, weight_decay: float,
          param_dtype: str) -> np.ndarray:
    """Decoupled decay and update of one slice of weights.

    ``weight`` is float32 values, or uint16 bfloat16 bits when
    ``param_dtype == "bf16"``; ``update`` is float32.  Returns the new weights
    in the same representation.
    """
    f = decay_factor(lr, weight_decay)
    l = F32(lr)
    w = bf16_bits_to_f32(weight) if param_dtype == "bf16" else weight.astype(np.float32)
    o = update.astype(np.float32, copy=False)
    w1 = w * f
    wn = w1 - (l * o)
    wn = wn.astype(np.float32)
    if param_dtype == "bf16":
        return f32_to_bf16_bits(wn)
    return wn

