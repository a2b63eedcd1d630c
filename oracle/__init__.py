"""CPU oracle for the affine Q4 group-32 quantized linear layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package. It shares no
code with the HIP library (``bit_group_quantized_amd``) and neither imports the
other.

The arithmetic lives in plain C (``q4_oracle.c``); this module only builds and
loads it and marshals numpy arrays. Every function cites the passage of the
pages it follows in the C source. Summary of what is computed:

* ``quantize(w)``: per 32-weight group along the input dimension, scale =
  (max - min)/15 and bias = min, both rounded to bf16; codes are
  ``clamp(rint((w - bias')/scale'), 0, 15)`` against the stored bf16 values;
  8 codes per uint32, low nibble first ("personaplex-edge-q4" model card,
  Release details table: affine Q4, group size 32, BF16 activations).
* ``unpack``: codes and ``w_hat = scale'*q + bias'``.
* ``matmul(x, ...)``: ``y = x . W_hat^T`` summed in float64 (the blog
  translation's MultiLinear figure: quantized product with transpose).
* ``multilinear_step``: the same product on rows ``[s*out, (s+1)*out)``.
* ``rope`` / ``attn_decode``: the rotary embedding at a position (rounded to
  bf16) and one query's attention per head over the KV cache (float64).
* ``rmsnorm`` / ``silu_mul``: the normalization before a layer's products and
  the gated FFN's product (with a residual sum, the parts fused around the
  products).
* ``embed_sum``: per frame, the sum over token streams of the dequantized
  embedding row each token selects (the blog translation's pipeline figure:
  17 streams summed into the step's input; embeddings stay packed).

Parity status of each function is recorded in the design notes; every function
here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_q4.so")
_lib = None

GROUP = 32


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle_q4.so``."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_quantize.argtypes = [P, I, I, P, P, P]
    lib.oracle_unpack.argtypes = [P, P, P, I, I, P, P]
    lib.oracle_matmul.argtypes = [P, I, P, P, P, I, I, P]
    lib.oracle_multilinear_step.argtypes = [P, I, P, P, P, I, I, I, I, P]
    lib.oracle_bf16_round.argtypes = [P, I, P]
    lib.oracle_embed_sum.argtypes = [P, I, I, P, P, P, P, I, P]
    lib.oracle_rope.argtypes = [P, I, I, I, ctypes.c_double, P]
    lib.oracle_rmsnorm.argtypes = [P, I, I, P, ctypes.c_double, P]
    lib.oracle_silu_mul.argtypes = [P, P, I, P]
    lib.oracle_attn_decode.argtypes = [P, P, P, I, I, I, I, P]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    for f in ("oracle_quantize", "oracle_unpack", "oracle_matmul", "oracle_multilinear_step",
              "oracle_bf16_round", "oracle_embed_sum", "oracle_rope", "oracle_attn_decode",
              "oracle_rmsnorm", "oracle_silu_mul"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc == 1:
        raise ValueError(f"{what}: invalid argument (shape or pointer)")
    if rc == 2:
        raise ValueError(f"{what}: non-finite input")
    if rc != 0:
        raise RuntimeError(f"{what}: oracle error {rc}")


def threads() -> int:
    return int(_load().oracle_threads())


def set_threads(t: int) -> None:
    _load().oracle_set_threads(int(t))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _check(_load().oracle_bf16_round(_ptr(a), a.size, _ptr(out)), "bf16_round")
    return out


def bf16_value(h: np.ndarray) -> np.ndarray:
    """fp32 values of bf16 bit patterns (exact widening)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize(w: np.ndarray):
    """Quantize fp32 W [n, k] -> (packed uint32 [n, k/8], scales uint16 [n, k/32],
    biases uint16 [n, k/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    packed = np.empty((n, k // 8), dtype=np.uint32)
    scales = np.empty((n, k // GROUP), dtype=np.uint16)
    biases = np.empty((n, k // GROUP), dtype=np.uint16)
    _check(_load().oracle_quantize(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(biases)), "quantize")
    return packed, scales, biases


def unpack(packed: np.ndarray, scales: np.ndarray, biases: np.ndarray, k: int):
    """Return (q uint8 [n, k], w_hat fp32 [n, k])."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    n = packed.shape[0]
    q = np.empty((n, k), dtype=np.uint8)
    w_hat = np.empty((n, k), dtype=np.float32)
    _check(_load().oracle_unpack(_ptr(packed), _ptr(scales), _ptr(biases), n, k, _ptr(q), _ptr(w_hat)),
           "unpack")
    return q, w_hat


def matmul(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, biases: np.ndarray, k: int) -> np.ndarray:
    """y = x . W_hat^T in float64. x_bits: bf16 bit patterns [m, k] (or [k])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    squeeze = x_bits.ndim == 1
    if squeeze:
        x_bits = x_bits[None, :]
    m = x_bits.shape[0]
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    n = packed.shape[0]
    if x_bits.shape[1] != k or packed.shape[1] * 8 != k:
        raise ValueError("shape mismatch")
    y = np.empty((m, n), dtype=np.float64)
    _check(_load().oracle_matmul(_ptr(x_bits), m, _ptr(packed), _ptr(scales), _ptr(biases), n, k, _ptr(y)),
           "matmul")
    return y[0] if squeeze else y


def multilinear_step(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                     num_steps: int, out: int, k: int, step: int) -> np.ndarray:
    """Product with the row block of codebook step ``step`` ([num_steps*out, k] weights)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    squeeze = x_bits.ndim == 1
    if squeeze:
        x_bits = x_bits[None, :]
    m = x_bits.shape[0]
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    if packed.shape[0] != num_steps * out:
        raise ValueError("packed rows must equal num_steps*out")
    y = np.empty((m, out), dtype=np.float64)
    _check(_load().oracle_multilinear_step(_ptr(x_bits), m, _ptr(packed), _ptr(scales), _ptr(biases),
                                           num_steps, out, k, step, _ptr(y)), "multilinear_step")
    return y[0] if squeeze else y


def embed_sum(tokens: np.ndarray, tables, dim: int) -> np.ndarray:
    """Sum over streams of the dequantized embedding rows the tokens select.

    tokens: int32 [frames, streams]; tables: one (packed, scales, biases) per
    stream, each [rows_t, dim] in the packed layout. A token outside [0, rows_t)
    adds nothing. Returns float64 [frames, dim] (the pipeline figure of the
    blog translation: the 17 token streams are summed into the step's input)."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    if tokens.ndim != 2 or tokens.shape[1] != len(tables):
        raise ValueError("tokens must be [frames, streams] with one table per stream")
    frames, streams = tokens.shape
    arrs = []
    for P, S, B in tables:
        P = np.ascontiguousarray(P, dtype=np.uint32)
        S = np.ascontiguousarray(S, dtype=np.uint16)
        B = np.ascontiguousarray(B, dtype=np.uint16)
        if P.shape[1] * 8 != dim or S.shape != (P.shape[0], dim // GROUP) or B.shape != S.shape:
            raise ValueError("table shape mismatch")
        arrs.append((P, S, B))
    VP = ctypes.c_void_p * streams
    pp = VP(*[a[0].ctypes.data for a in arrs])
    sp = VP(*[a[1].ctypes.data for a in arrs])
    bp = VP(*[a[2].ctypes.data for a in arrs])
    rows = np.array([a[0].shape[0] for a in arrs], dtype=np.int64)
    y = np.empty((frames, dim), dtype=np.float64)
    _check(_load().oracle_embed_sum(_ptr(tokens), frames, streams, ctypes.cast(pp, ctypes.c_void_p),
                                    ctypes.cast(sp, ctypes.c_void_p), ctypes.cast(bp, ctypes.c_void_p), _ptr(rows),
                                    dim, _ptr(y)), "embed_sum")
    return y


def rope(x_bits: np.ndarray, pos: int, theta: float = 10000.0) -> np.ndarray:
    """Rotary embedding of bf16 x [heads, D] at position pos, rounded to bf16
    (pairs (2i, 2i+1) turned by pos * theta^(-2i/D))."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    heads, d = x_bits.shape
    out = np.empty_like(x_bits)
    _check(_load().oracle_rope(_ptr(x_bits), heads, d, int(pos), float(theta), _ptr(out)), "rope")
    return out


def attn_decode(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, pos: int) -> np.ndarray:
    """Single-query attention per head over cache positions 0..pos, in float64.
    q: bf16 [heads, D] (rotated); k, v: bf16 [heads, cap, D]."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
    heads, cap, d = k_bits.shape
    if q_bits.shape != (heads, d) or v_bits.shape != k_bits.shape:
        raise ValueError("shape mismatch")
    out = np.empty((heads, d), dtype=np.float64)
    _check(_load().oracle_attn_decode(_ptr(q_bits), _ptr(k_bits), _ptr(v_bits), heads, d, cap, int(pos), _ptr(out)),
           "attn_decode")
    return out


def rmsnorm(x_bits: np.ndarray, g_bits: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row of bf16 x [m, k] with weight g [k], in double,
    rounded to bf16: (x * g) * 1/sqrt(mean(x^2) + eps), x * g exact."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    squeeze = x_bits.ndim == 1
    if squeeze:
        x_bits = x_bits[None, :]
    m, k = x_bits.shape
    g_bits = np.ascontiguousarray(g_bits, dtype=np.uint16)
    if g_bits.shape != (k,):
        raise ValueError("norm weight must be [k]")
    out = np.empty_like(x_bits)
    _check(_load().oracle_rmsnorm(_ptr(x_bits), m, k, _ptr(g_bits), float(eps), _ptr(out)), "rmsnorm")
    return out[0] if squeeze else out


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up elementwise in double (the gated FFN's product)."""
    gate = np.ascontiguousarray(gate, dtype=np.float64)
    up = np.ascontiguousarray(up, dtype=np.float64)
    if gate.shape != up.shape:
        raise ValueError("shape mismatch")
    out = np.empty_like(gate)
    _check(_load().oracle_silu_mul(_ptr(gate), _ptr(up), gate.size, _ptr(out)), "silu_mul")
    return out


def output_bits_bf16(y: np.ndarray) -> np.ndarray:
    """What a bf16 output tensor holds for the exact result y: bf16_rne(fl32(y))."""
    return bf16_round(np.asarray(y, dtype=np.float64).astype(np.float32))


def floored_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over outputs of |got - ref| / max(|ref|, 1e-3 * rms(ref)), per output row.

    "Max relative error" is ill-posed where the exact output is near zero; the
    floor of 1e-3 of the row's RMS is the reading used for the tolerances. The
    RMS is taken over each output row (one activation row's outputs) on its
    own, and every element is divided by its own |ref| (or the floor). An
    output that is not finite where the exact value is finite scores inf, so a
    NaN or inf can never pass a tolerance. Shapes must match."""
    got = np.atleast_2d(np.asarray(got, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch: got {got.shape}, ref {ref.shape}")
    if not np.all(np.isfinite(ref)):
        raise ValueError("reference values must be finite")
    if not np.all(np.isfinite(got)):
        return float("inf")
    worst = 0.0
    for g, r in zip(got, ref):
        if r.size == 0:
            continue
        rms = float(np.sqrt(np.mean(r * r)))
        floor = max(1e-3 * rms, np.finfo(np.float64).tiny)
        e = np.abs(g - r) / np.maximum(np.abs(r), floor)
        worst = max(worst, float(e.max()))
    return worst
