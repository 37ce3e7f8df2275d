"""Seeded synthetic inputs shared by the GPU path, the oracle tests and the bench.

This module draws random numbers and rounds them to storage formats. It holds
none of the model's arithmetic, so the HIP path and the float64 oracle can both
take their inputs from here without sharing any code of the method itself.

Recipe (stated once, used everywhere):

* Weights: one ``numpy.random.default_rng(seed)`` (PCG64), tensors drawn in the
  canonical parameter order (wte, then per layer W_qkv, W_o, W_1, W_2, then
  W_lm), ``standard_normal * 0.02`` in float64, rounded to float32 by RNE and
  then, for bf16 models, to bf16 by RNE on the float32 bits. Optional
  tensors come after W_lm in the same stream: value-embedding tables take
  ``standard_normal * 0.5`` (so that the lookup is comparable to v), and the
  per-layer scalars take their initial values (resid_lambdas 1.0,
  x0_lambdas 0.1, ve_gates 1.0) plus ``0.1 * standard_normal``, a seeded
  perturbation that keeps every factor away from 0 and 1.
* Tokens: ``default_rng(seed)`` draws an int32 array [B, T+1]; ``idx`` is
  [:, :T] and ``targets`` is [:, 1:] (next-token targets). ``law="uniform"``
  draws ids uniformly from [0, V). ``law="zipf"`` draws ranks k = 1..V with
  P(k) proportional to k**-s (s = 1.1 by default) by inverse CDF
  (``searchsorted`` on the float64 cumulative; truncated at V) and returns
  id = k - 1, so frequent ids are small, like byte/merge order in a BPE vocab.
  The Zipf stream stands in for the FineWeb-EDU token stream the pages train
  on (aethryn.com, "Nanochat: full-stack LLM training in 8,000 lines for $72",
  section "Five training stages from raw text to chat assistant"), which is not
  available here.
"""
from __future__ import annotations

import numpy as np

WEIGHT_STD = 0.02


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16. NaN is not expected in inputs.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> 16) & 1
    rounded = (b + np.uint32(0x7FFF) + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_weights(shapes, seed: int = 0, dtype: str = "bf16", std: float = WEIGHT_STD):
    """Draw every parameter tensor in order into one flat buffer.

    ``shapes`` is a sequence of (name, rows, cols) in canonical order.
    Returns ``(storage, values)``: ``storage`` is the flat array in the
    model's storage format (float32, or uint16 bf16 bit patterns) and
    ``values`` is the same numbers as float32 (exactly representable).
    """
    rng = np.random.default_rng(seed)
    total = sum(int(r) * int(c) for _, r, c in shapes)
    vals = np.empty(total, dtype=np.float32)
    off = 0
    inits = {"resid_lambdas": 1.0, "x0_lambdas": 0.1, "ve_gates": 1.0}
    for name, r, c in shapes:
        n = int(r) * int(c)
        z = rng.standard_normal(n)
        if name in inits:
            vals[off:off + n] = (inits[name] + 0.1 * z).astype(np.float32)
        elif name.endswith(".ve"):
            vals[off:off + n] = (z * 0.5).astype(np.float32)
        else:
            vals[off:off + n] = (z * std).astype(np.float32)
        off += n
    if dtype == "f32":
        return vals, vals
    if dtype == "bf16":
        bits = f32_to_bf16_bits(vals)
        return bits, bf16_bits_to_f32(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def zipf_cdf(V: int, s: float = 1.1) -> np.ndarray:
    k = np.arange(1, V + 1, dtype=np.float64)
    w = k ** (-s)
    cdf = np.cumsum(w)
    return cdf / cdf[-1]


def make_tokens(B: int, T: int, V: int, law: str = "uniform", seed: int = 1, s: float = 1.1):
    """Return ``(idx, targets)``, both int32 [B, T], from one [B, T+1] draw."""
    rng = np.random.default_rng(seed)
    if law == "uniform":
        seq = rng.integers(0, V, size=(B, T + 1), dtype=np.int64)
    elif law == "zipf":
        u = rng.random(size=(B, T + 1))
        seq = np.searchsorted(zipf_cdf(V, s), u, side="right")
        seq = np.minimum(seq, V - 1)
    else:
        raise ValueError(f"unknown token law {law!r}")
    seq = seq.astype(np.int32)
    return np.ascontiguousarray(seq[:, :T]), np.ascontiguousarray(seq[:, 1:])
