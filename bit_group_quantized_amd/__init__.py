"""Python binding of libq4, the gfx950 affine Q4 group-32 quantized linear library.

Argument marshalling only: every computation runs in the HIP kernels behind the
C ABI declared in ``include/q4.h``. PyTorch supplies device memory and the
current HIP stream; the functions here check dtypes/shapes for clear Python
errors, allocate outputs when none are given, and pass raw pointers.

Tensor conventions (torch dtypes holding the stored bit patterns):
  weights  w        float32 [n, k]            (input of q4_pack)
  packed            int32   [n, k/8]          (uint32 words, low nibble first)
  scales, biases    bfloat16 [n, k/32]
  activations x     bfloat16 [k] or [m, k]
  outputs y         bfloat16 or float32

There is no CPU fallback: if ``libq4.so`` is missing or no GPU is visible the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4.so")

Q4_OK, Q4_ERR_NULL, Q4_ERR_SHAPE, Q4_ERR_ALIGN, Q4_ERR_UNSUPPORTED, Q4_ERR_HIP = range(6)
Q4_OUT_BF16, Q4_OUT_F32 = 0, 1
GROUP = 32
MAX_M = 64  # Q4_MAX_M
MAX_K = 16384  # Q4_MAX_K

_lib = None

_EXPORTS = (
    "q4_layout_version", "q4_status_str", "q4_last_hip_error", "q4_pack", "q4_unpack", "q4_gemv",
    "q4_gemm_small", "q4_multilinear_step", "q4_chain_plan_bytes", "q4_chain_encode", "q4_chain_run",
    "q4_chain_encode_rows", "q4_chain_run_rows", "q4_chain_run_rows_noalloc", "q4_embed_sum",
    "q4_attn_workspace_bytes", "q4_attn_decode", "q4_chain_encode_ex", "q4_gemm_batch_blocks",
    "q4_gemm_batch_plan_bytes", "q4_gemm_batch_encode", "q4_gemm_batch_run",
)
EMBED_MAX_TABLES = 32  # Q4_EMBED_MAX_TABLES
CHAIN_WORKSPACE_BYTES = 131328


class _ChainMatrix(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("n", ctypes.c_int64)]


class _ChainStage(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("k", ctypes.c_int64), ("first_matrix", ctypes.c_int32),
                ("num_matrices", ctypes.c_int32)]


class _ChainMatrixEx(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("n", ctypes.c_int64), ("residual", ctypes.c_void_p)]


class _ChainStageEx(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("k", ctypes.c_int64), ("first_matrix", ctypes.c_int32),
                ("num_matrices", ctypes.c_int32), ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_double),
                ("gated", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _GemmBatchItem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("y", ctypes.c_void_p), ("n", ctypes.c_int64)]


class _EmbedTable(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("rows", ctypes.c_int64)]


class Q4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        msg = lib.q4_status_str(status).decode()
        if status == Q4_ERR_HIP:
            msg += f" (hipError {lib.q4_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def load():
    """Load libq4.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, V = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.q4_layout_version.restype = V
    lib.q4_status_str.argtypes = [V]
    lib.q4_status_str.restype = ctypes.c_char_p
    lib.q4_last_hip_error.restype = V
    lib.q4_pack.argtypes = [P, I, I, P, P, P, P]
    lib.q4_unpack.argtypes = [P, P, P, I, I, P, P, P]
    lib.q4_gemv.argtypes = [P, P, P, P, I, I, P, V, P]
    lib.q4_gemm_small.argtypes = [P, I, P, P, P, I, I, P, V, P]
    lib.q4_multilinear_step.argtypes = [P, I, P, P, P, I, I, I, I, P, V, P]
    lib.q4_chain_plan_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.q4_chain_plan_bytes.restype = ctypes.c_int64
    lib.q4_chain_encode.argtypes = [P, ctypes.c_int32, P, ctypes.c_int32, V, P, I]
    lib.q4_chain_run.argtypes = [P, V, P, P]
    lib.q4_chain_encode_rows.argtypes = [P, ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32, V, P, I]
    lib.q4_chain_run_rows.argtypes = [P, ctypes.c_int32, V, P, P]
    lib.q4_chain_encode_ex.argtypes = [P, ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32, V, P, I]
    lib.q4_chain_run_rows_noalloc.argtypes = [P, ctypes.c_int32, V, P, P]
    lib.q4_embed_sum.argtypes = [P, I, P, ctypes.c_int32, I, P, V, P]
    lib.q4_attn_workspace_bytes.argtypes = [I, I]
    lib.q4_attn_workspace_bytes.restype = ctypes.c_int64
    lib.q4_attn_decode.argtypes = [P, P, P, P, P, I, I, I, I, ctypes.c_double, P, V, P, I, P]
    lib.q4_gemm_batch_blocks.argtypes = [P, ctypes.c_int32]
    lib.q4_gemm_batch_blocks.restype = ctypes.c_int64
    lib.q4_gemm_batch_plan_bytes.argtypes = [ctypes.c_int32, I]
    lib.q4_gemm_batch_plan_bytes.restype = ctypes.c_int64
    lib.q4_gemm_batch_encode.argtypes = [P, ctypes.c_int32, I, I, V, P, I]
    lib.q4_gemm_batch_run.argtypes = [P, P, P]
    lib.q4_gemm_batch_encode.restype = V
    lib.q4_gemm_batch_run.restype = V
    for f in ("q4_pack", "q4_unpack", "q4_gemv", "q4_gemm_small", "q4_multilinear_step", "q4_chain_encode",
              "q4_chain_run", "q4_chain_encode_rows", "q4_chain_run_rows", "q4_chain_run_rows_noalloc", "q4_embed_sum",
              "q4_attn_decode", "q4_chain_encode_ex"):
        getattr(lib, f).restype = V
    _lib = lib
    return lib


def exported_symbols() -> Tuple[str, ...]:
    return _EXPORTS


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(fn: str, status: int) -> None:
    if status != Q4_OK:
        raise Q4Error(fn, status)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return Q4_OUT_BF16
    if dtype == torch.float32:
        return Q4_OUT_F32
    raise TypeError("output dtype must be torch.bfloat16 or torch.float32")


def q4_layout_version() -> int:
    return int(load().q4_layout_version())


def q4_status_str(status: int) -> str:
    return load().q4_status_str(int(status)).decode()


def q4_pack(w: torch.Tensor, packed: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
            biases: Optional[torch.Tensor] = None):
    """Quantize fp32 W [n, k] on the GPU -> (packed int32 [n, k/8], scales bf16, biases bf16).

    Outputs given by the caller must have exactly those shapes and sit on w's
    device (the library takes n and k from w and writes that many words)."""
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("w must be a tensor [n, k]")
    n, k = w.shape
    if k % GROUP:
        raise ValueError("k must be a multiple of 32")
    for t, name, shape in ((packed, "packed", (n, k // 8)), (scales, "scales", (n, k // GROUP)),
                           (biases, "biases", (n, k // GROUP))):
        if t is not None:
            if not isinstance(t, torch.Tensor) or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be [{shape[0]}, {shape[1]}] for w of shape [{n}, {k}]")
            if t.device != w.device:
                raise ValueError(f"{name} must be on w's device ({w.device})")
    _need(w, "w", torch.float32)
    dev = w.device
    packed = torch.empty((n, k // 8), dtype=torch.int32, device=dev) if packed is None else packed
    scales = torch.empty((n, k // GROUP), dtype=torch.bfloat16, device=dev) if scales is None else scales
    biases = torch.empty((n, k // GROUP), dtype=torch.bfloat16, device=dev) if biases is None else biases
    _need(packed, "packed", torch.int32)
    _need(scales, "scales", torch.bfloat16)
    _need(biases, "biases", torch.bfloat16)
    _check("q4_pack", load().q4_pack(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(biases), _ptr_stream(w)))
    return packed, scales, biases


def _ptr_stream(t: torch.Tensor):
    return ctypes.c_void_p(_stream(t))


def _check_matrix(packed, scales, biases):
    _need(packed, "packed", torch.int32)
    _need(scales, "scales", torch.bfloat16)
    _need(biases, "biases", torch.bfloat16)
    if packed.dim() != 2 or scales.dim() != 2 or biases.dim() != 2:
        raise ValueError("packed/scales/biases must be 2-D")
    n, k8 = packed.shape
    k = k8 * 8
    if scales.shape != (n, k // GROUP) or biases.shape != (n, k // GROUP):
        raise ValueError("scales/biases must be [n, k/32]")
    if scales.device != packed.device or biases.device != packed.device:
        raise ValueError("packed, scales and biases must be on one device")
    return n, k


def _same_device(ref: torch.Tensor, *ts) -> None:
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"every tensor of a call must be on {ref.device} (got {t.device})")


def q4_unpack(packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, want_codes: bool = True,
              want_weights: bool = True):
    """-> (codes uint8 [n, k] or None, w_hat float32 [n, k] or None)."""
    n, k = _check_matrix(packed, scales, biases)
    dev = packed.device
    q = torch.empty((n, k), dtype=torch.uint8, device=dev) if want_codes else None
    w = torch.empty((n, k), dtype=torch.float32, device=dev) if want_weights else None
    _check("q4_unpack", load().q4_unpack(_ptr(packed), _ptr(scales), _ptr(biases), n, k, _ptr(q), _ptr(w),
                                         _ptr_stream(packed)))
    return q, w


def q4_gemv(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
            out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [n] = x [k] . W_hat^T."""
    n, k = _check_matrix(packed, scales, biases)
    _need(x, "x", torch.bfloat16)
    if x.numel() != k:
        raise ValueError(f"x must hold k={k} elements")
    code = _out_code(out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((n,), dtype=out_dtype, device=x.device)
    _need(out, "out", out.dtype)
    if out.numel() != n:
        raise ValueError("out must hold n elements")
    _same_device(packed, x, out)
    _check("q4_gemv", load().q4_gemv(_ptr(x), _ptr(packed), _ptr(scales), _ptr(biases), n, k, _ptr(out), code,
                                     _ptr_stream(x)))
    return out


def q4_gemm_small(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                  out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y [m, n] = X [m, k] . W_hat^T for 1 <= m <= 64 (17..64: prefill)."""
    n, k = _check_matrix(packed, scales, biases)
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}]")
    m = x.shape[0]
    code = _out_code(out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _need(out, "out", out.dtype)
    if out.numel() != m * n:
        raise ValueError("out must hold m*n elements")
    _same_device(packed, x, out)
    _check("q4_gemm_small", load().q4_gemm_small(_ptr(x), m, _ptr(packed), _ptr(scales), _ptr(biases), n, k,
                                                 _ptr(out), code, _ptr_stream(x)))
    return out


class GemmBatchPlan:
    """An encoded product batch: the host and device copies of the plan plus
    what it references (kept alive here so the device pointers stay valid)."""

    def __init__(self, host_plan, device_plan: torch.Tensor, keep: list):
        self.host_plan = host_plan
        self.device_plan = device_plan
        self._keep = keep


def q4_gemm_batch_build(xs, mats, outs) -> GemmBatchPlan:
    """Encode independent products outs[i] [m, n_i] = xs[i] [m, k] . W_hat_i^T
    (mats[i] = (packed, scales, biases)) sharing m (5..16) and k, and upload
    the plan: q4_gemm_batch_run then runs them all in one launch."""
    if not (len(xs) == len(mats) == len(outs)) or not xs:
        raise ValueError("xs, mats and outs must be non-empty lists of one length")
    lib = load()
    m, k = xs[0].shape
    code = _out_code(outs[0].dtype)
    items, keep = [], []
    for x, (packed, scales, biases), out in zip(xs, mats, outs):
        n, kk = _check_matrix(packed, scales, biases)
        _need(x, "x", torch.bfloat16)
        _need(out, "out", outs[0].dtype)
        if x.dim() != 2 or tuple(x.shape) != (m, k) or kk != k:
            raise ValueError(f"every x must be [{m}, {k}] and every weight [n, {k}]")
        if out.numel() != m * n:
            raise ValueError("out must hold m*n elements")
        _same_device(xs[0], x, packed, out)
        items.append(_GemmBatchItem(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                    out.data_ptr(), n))
        keep += [x, packed, scales, biases, out]
    arr = (_GemmBatchItem * len(items))(*items)
    blocks = int(lib.q4_gemm_batch_blocks(ctypes.byref(arr), len(items)))
    nbytes = int(lib.q4_gemm_batch_plan_bytes(len(items), blocks))
    if nbytes <= 0:
        raise ValueError("batch outside the encoder's limits")
    host = (ctypes.c_uint8 * nbytes)()
    _check("q4_gemm_batch_encode", lib.q4_gemm_batch_encode(ctypes.byref(arr), len(items), m, k, code,
                                                            ctypes.byref(host), nbytes))
    plan = torch.empty(nbytes, dtype=torch.uint8, device=xs[0].device)
    plan.copy_(torch.frombuffer(bytearray(host), dtype=torch.uint8))
    return GemmBatchPlan(host, plan, keep)


def q4_gemm_batch_run(plan: GemmBatchPlan) -> None:
    """Run every product of the batch in one launch on the current stream."""
    _check("q4_gemm_batch_run", load().q4_gemm_batch_run(ctypes.byref(plan.host_plan), _ptr(plan.device_plan),
                                                         _ptr_stream(plan.device_plan)))


def q4_multilinear_step(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                        num_steps: int, step: int, out_dtype: torch.dtype = torch.bfloat16,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y [m, out] = X [m, k] . (rows [step*out, (step+1)*out) of W_hat)^T, weights [num_steps*out, k]."""
    rows, k = _check_matrix(packed, scales, biases)
    if num_steps <= 0 or rows % num_steps:
        raise ValueError("rows must be num_steps * out")
    out_rows = rows // num_steps
    _need(x, "x", torch.bfloat16)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    if x2.shape[1] != k:
        raise ValueError(f"x must have k={k} columns")
    m = x2.shape[0]
    code = _out_code(out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((m, out_rows) if x.dim() == 2 else (out_rows,), dtype=out_dtype, device=x.device)
    _need(out, "out", out.dtype)
    if out.numel() != m * out_rows:
        raise ValueError("out must hold m*out elements")
    _same_device(packed, x2, out)
    _check("q4_multilinear_step",
           load().q4_multilinear_step(_ptr(x2), m, _ptr(packed), _ptr(scales), _ptr(biases), num_steps, out_rows,
                                      k, int(step), _ptr(out), code, _ptr_stream(x)))
    return out


def q4_embed_sum(tokens: torch.Tensor, tables, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [frames, dim] = per frame, the sum over streams of the packed
    embedding row each token selects (tokens: int32 [frames, streams] on the
    device; tables: one (packed, scales, biases) per stream, [rows_t, dim]).
    A token outside [0, rows_t) adds nothing."""
    if not isinstance(tokens, torch.Tensor) or tokens.dim() != 2:
        raise ValueError("tokens must be [frames, streams]")
    frames, streams = tokens.shape
    if streams != len(tables) or not 1 <= streams <= EMBED_MAX_TABLES:
        raise ValueError(f"one table per stream (1..{EMBED_MAX_TABLES}): {streams} streams, {len(tables)} tables")
    dims = set()
    descs = []
    for t, (packed, scales, biases) in enumerate(tables):
        rows, dim = _check_matrix(packed, scales, biases)
        dims.add(dim)
        descs.append(_EmbedTable(packed.data_ptr(), scales.data_ptr(), biases.data_ptr(), rows))
    if len(dims) != 1:
        raise ValueError("every table must have the same dim")
    dim = dims.pop()
    _need(tokens, "tokens", torch.int32)
    code = _out_code(out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((frames, dim), dtype=out_dtype, device=tokens.device)
    _need(out, "out", out.dtype)
    if out.numel() != frames * dim:
        raise ValueError("out must hold frames*dim elements")
    _same_device(tokens, out, *[p for tb in tables for p in tb])
    arr = (_EmbedTable * streams)(*descs)
    _check("q4_embed_sum", load().q4_embed_sum(_ptr(tokens), frames, ctypes.byref(arr), streams, dim, _ptr(out), code,
                                               _ptr_stream(tokens)))
    return out


def q4_attn_workspace_bytes(heads: int, head_dim: int) -> int:
    return int(load().q4_attn_workspace_bytes(heads, head_dim))


def q4_attn_decode(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, pos: int, rope_theta: float = 10000.0,
                   out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One layer's decode attention: RoPE on q and k_new at pos, k and v written
    to the caches (bf16 [heads, cap, D]) at pos, then softmax(q.k/sqrt(D)).v
    per head over positions 0..pos -> out [heads, D]."""
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, torch.bfloat16)
    if k_cache.dim() != 3 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [heads, cap, D]")
    heads, cap, d = k_cache.shape
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        if t.numel() != heads * d:
            raise ValueError(f"{nm} must hold heads*D elements")
    code = _out_code(out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((heads, d), dtype=out_dtype, device=q.device)
    _need(out, "out", out.dtype)
    if out.numel() != heads * d:
        raise ValueError("out must hold heads*D elements")
    need = q4_attn_workspace_bytes(heads, d)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    _same_device(q, k_new, v_new, k_cache, v_cache, out, workspace)
    _check("q4_attn_decode", load().q4_attn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                                   heads, d, cap, int(pos), float(rope_theta), _ptr(out), code,
                                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _ptr_stream(q)))
    return out


# ---------------------------------------------------------------- chain executor

class ChainPlan:
    """An encoded chain: the device copy of the plan plus what it references
    (kept alive here so the device pointers in the plan stay valid)."""

    def __init__(self, device_plan: torch.Tensor, out_dtype: torch.dtype, keep: list, m: int = 1):
        self.device_plan = device_plan
        self.out_dtype = out_dtype
        self.m = m
        self._keep = keep


def q4_chain_workspace_bytes() -> int:
    return CHAIN_WORKSPACE_BYTES


def q4_chain_build(stages, out_dtype: Optional[torch.dtype] = None) -> ChainPlan:
    """Encode stages and upload the plan. A stage has .x, .mats (each
    .packed/.scales/.biases) and .outs, and optionally .norm (bf16 [k] RMSNorm
    weight) with .eps, .gated (True: two matrices gate, up; the output
    silu(gate) * up goes to outs[0], outs[1] may be None) and .residuals (one
    tensor or None per matrix, added to its product). All outputs and
    residuals share one dtype. Every stage's x is either a vector [k] (one
    activation row) or a matrix [m, k] with the same m (1..4) in every stage;
    each output then holds m*n elements."""
    lib = load()
    mats = []
    descs = []
    keep = []
    rows = None
    for si, st in enumerate(stages):
        if len(st.outs) != len(st.mats):
            raise ValueError(f"stage {si}: {len(st.mats)} matrices but {len(st.outs)} outputs")
        _need(st.x, "x", torch.bfloat16)
        m_st = 1 if st.x.dim() == 1 else st.x.shape[0]
        if st.x.dim() > 2:
            raise ValueError("x must be [k] or [m, k]")
        if rows is None:
            rows = m_st
        elif rows != m_st:
            raise ValueError("every stage must have the same number of activation rows")
        first = len(mats)
        k = st.x.shape[-1]
        gated = bool(getattr(st, "gated", False))
        residuals = getattr(st, "residuals", None) or [None] * len(st.mats)
        if len(residuals) != len(st.mats):
            raise ValueError(f"stage {si}: one residual (or None) per matrix")
        norm = getattr(st, "norm", None)
        eps = float(getattr(st, "eps", 0.0))
        if norm is not None:
            _need(norm, "norm", torch.bfloat16)
            if norm.numel() != k:
                raise ValueError("norm weight must hold k elements")
            _same_device(st.x, norm)
            keep.append(norm)
        for i, (m, y, r) in enumerate(zip(st.mats, st.outs, residuals)):
            n, km = _check_matrix(m.packed, m.scales, m.biases)
            if km != k:
                raise ValueError("every matrix of a stage must have the stage's k")
            written = not (gated and i == 1)
            if written:
                if out_dtype is None:
                    out_dtype = y.dtype
                _need(y, "y", out_dtype)
                if y.numel() != rows * n:
                    raise ValueError("output must hold m*n elements")
                _same_device(stages[0].x, st.x, m.packed, y)
                keep.append(y)
            elif y is not None:
                raise ValueError("a gated stage writes only its first matrix's output")
            if r is not None:
                if out_dtype is None:
                    out_dtype = r.dtype
                _need(r, "residual", out_dtype)
                if r.numel() != rows * n:
                    raise ValueError("residual must hold m*n elements")
                _same_device(st.x, r)
                keep.append(r)
            mats.append(_ChainMatrixEx(m.packed.data_ptr(), m.scales.data_ptr(), m.biases.data_ptr(),
                                       y.data_ptr() if written else None, n,
                                       None if r is None else r.data_ptr()))
            keep += [m.packed, m.scales, m.biases]
        descs.append(_ChainStageEx(st.x.data_ptr(), k, first, len(mats) - first,
                                   None if norm is None else norm.data_ptr(), eps, 1 if gated else 0, 0))
        keep.append(st.x)
    code = _out_code(out_dtype)
    ns, nm = len(descs), len(mats)
    nbytes = int(lib.q4_chain_plan_bytes(ns, nm))
    if nbytes <= 0:
        raise ValueError("empty chain")
    host = (ctypes.c_uint8 * nbytes)()
    sarr = (_ChainStageEx * ns)(*descs)
    marr = (_ChainMatrixEx * nm)(*mats)
    _check("q4_chain_encode_ex", lib.q4_chain_encode_ex(ctypes.byref(sarr), ns, ctypes.byref(marr), nm, rows,
                                                        code, ctypes.byref(host), nbytes))
    dev = stages[0].x.device
    host_t = torch.frombuffer(bytearray(host), dtype=torch.uint8)
    plan = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    plan.copy_(host_t)
    return ChainPlan(plan, out_dtype, keep, rows)


def q4_chain_run(plan: ChainPlan, workspace: torch.Tensor) -> None:
    """Run the chain on the current stream. workspace: zero-filled device tensor
    of at least CHAIN_WORKSPACE_BYTES (its word 0 reports barrier timeouts)."""
    if workspace.numel() * workspace.element_size() < CHAIN_WORKSPACE_BYTES or not workspace.is_cuda:
        raise ValueError("workspace must be a device tensor of >= %d bytes" % CHAIN_WORKSPACE_BYTES)
    _check("q4_chain_run_rows", load().q4_chain_run_rows(_ptr(plan.device_plan), plan.m, _out_code(plan.out_dtype),
                                                         _ptr(workspace), _ptr_stream(workspace)))


def q4_chain_run_noalloc(plan: ChainPlan, status_out: Optional[torch.Tensor] = None) -> None:
    """Run the chain on the current stream with the library's own device-global
    workspace (no workspace argument, no allocation). status_out: optional
    device int32 tensor of >= 1 element that receives the launch's status word
    (0 = ok). Calls that overlap in time on one device race."""
    if status_out is not None:
        _need(status_out, "status_out", torch.int32)
        if status_out.numel() < 1:
            raise ValueError("status_out must hold one element")
        _same_device(plan.device_plan, status_out)
    _check("q4_chain_run_rows_noalloc",
           load().q4_chain_run_rows_noalloc(_ptr(plan.device_plan), plan.m, _out_code(plan.out_dtype),
                                            _ptr(status_out), _ptr_stream(plan.device_plan)))
