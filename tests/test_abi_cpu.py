"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the GPU (every
call here fails validation, so no HIP call is made)."""
import ctypes
import os
import re
import struct

import pytest

import bit_group_quantized_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:q4_status|int64_t|int|const char\*)\s+(q4_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = header_functions()
    assert names == sorted(q4.exported_symbols())
    for want in ("q4_pack", "q4_unpack", "q4_gemv", "q4_gemm_small", "q4_multilinear_step"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q4.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_layout_version_and_status_strings():
    assert q4.q4_layout_version() == 1
    assert q4.q4_status_str(0) == "ok"
    assert q4.q4_status_str(q4.Q4_ERR_ALIGN) == "misaligned pointer"
    assert q4.q4_status_str(99) == "unknown status"


A16 = 0x10000   # a 16-byte aligned fake address: validation fails before any use
ODD = 0x10001
Y16 = 0x400000  # another one, far from A16 (chain outputs must not overlap their own input)


def _p(v):
    return ctypes.c_void_p(v)


@pytest.mark.parametrize("case,want", [
    (dict(x=0), q4.Q4_ERR_NULL),
    (dict(packed=0), q4.Q4_ERR_NULL),
    (dict(scales=0), q4.Q4_ERR_NULL),
    (dict(biases=0), q4.Q4_ERR_NULL),
    (dict(y=0), q4.Q4_ERR_NULL),
    (dict(k=0), q4.Q4_ERR_SHAPE),
    (dict(k=48), q4.Q4_ERR_SHAPE),
    (dict(n=-1), q4.Q4_ERR_SHAPE),
    (dict(dtype=7), q4.Q4_ERR_SHAPE),
    (dict(x=ODD), q4.Q4_ERR_ALIGN),
    (dict(packed=A16 + 4), q4.Q4_ERR_ALIGN),
    (dict(scales=ODD), q4.Q4_ERR_ALIGN),
    (dict(y=ODD), q4.Q4_ERR_ALIGN),
    (dict(k=32 * 1024), q4.Q4_ERR_UNSUPPORTED),
    (dict(k=q4.MAX_K + 32), q4.Q4_ERR_UNSUPPORTED),  # one group past the widest supported row
])
def test_gemv_validation(case, want):
    a = dict(x=A16, packed=A16, scales=A16, biases=A16, n=16, k=64, y=A16, dtype=0)
    a.update(case)
    st = q4.load().q4_gemv(_p(a["x"]), _p(a["packed"]), _p(a["scales"]), _p(a["biases"]), a["n"], a["k"],
                           _p(a["y"]), a["dtype"], None)
    assert st == want


@pytest.mark.parametrize("m,want", [(0, q4.Q4_ERR_SHAPE), (65, q4.Q4_ERR_SHAPE), (-3, q4.Q4_ERR_SHAPE)])
def test_gemm_small_rejects_m(m, want):
    st = q4.load().q4_gemm_small(_p(A16), m, _p(A16), _p(A16), _p(A16), 16, 64, _p(A16), 0, None)
    assert st == want


@pytest.mark.parametrize("steps,step,want", [
    (16, 16, q4.Q4_ERR_SHAPE), (16, -1, q4.Q4_ERR_SHAPE), (0, 0, q4.Q4_ERR_SHAPE)])
def test_multilinear_rejects_step(steps, step, want):
    st = q4.load().q4_multilinear_step(_p(A16), 1, _p(A16), _p(A16), _p(A16), steps, 8, 64, step, _p(A16), 0,
                                       None)
    assert st == want


def test_pack_and_unpack_validation():
    lib = q4.load()
    assert lib.q4_pack(None, 4, 64, _p(A16), _p(A16), _p(A16), None) == q4.Q4_ERR_NULL
    assert lib.q4_pack(_p(ODD), 4, 64, _p(A16), _p(A16), _p(A16), None) == q4.Q4_ERR_ALIGN
    assert lib.q4_pack(_p(A16), 4, 40, _p(A16), _p(A16), _p(A16), None) == q4.Q4_ERR_SHAPE
    assert lib.q4_unpack(_p(A16), _p(A16), _p(A16), 4, 64, None, None, None) == q4.Q4_ERR_NULL
    assert lib.q4_unpack(_p(A16), _p(A16), _p(A16), 4, 64, _p(ODD), None, None) == q4.Q4_ERR_ALIGN


def test_empty_calls_are_noops():
    lib = q4.load()
    assert lib.q4_gemv(_p(A16), _p(A16), _p(A16), _p(A16), 0, 64, _p(A16), 0, None) == q4.Q4_OK
    assert lib.q4_pack(_p(A16), 0, 64, _p(A16), _p(A16), _p(A16), None) == q4.Q4_OK
    assert lib.q4_multilinear_step(_p(A16), 2, _p(A16), _p(A16), _p(A16), 16, 0, 64, 3, _p(A16), 1, None) == q4.Q4_OK


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(4, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        q4.q4_pack(w)


def test_binding_checks_pack_output_shapes_before_any_call():
    """q4_pack takes n and k from w: outputs the caller passes must have exactly
    the shapes it writes (checked before the device, so a CPU run sees it)."""
    import torch
    w = torch.zeros(4, 64)
    with pytest.raises(ValueError, match=r"packed must be \[4, 8\]"):
        q4.q4_pack(w, packed=torch.zeros(4, 4, dtype=torch.int32))
    with pytest.raises(ValueError, match=r"scales must be \[4, 2\]"):
        q4.q4_pack(w, scales=torch.zeros(4, 1, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"biases must be \[4, 2\]"):
        q4.q4_pack(w, biases=torch.zeros(2, 2, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="multiple of 32"):
        q4.q4_pack(torch.zeros(4, 40))


def test_binding_chain_build_needs_one_output_per_matrix():
    import torch
    from types import SimpleNamespace
    mat = SimpleNamespace(packed=torch.zeros(4, 8, dtype=torch.int32), scales=torch.zeros(4, 2, dtype=torch.bfloat16),
                          biases=torch.zeros(4, 2, dtype=torch.bfloat16))
    st = SimpleNamespace(x=torch.zeros(64, dtype=torch.bfloat16), mats=[mat, mat], outs=[torch.zeros(4)])
    with pytest.raises(ValueError, match="2 matrices but 1 outputs"):
        q4.q4_chain_build([st])


def _chain(n_stages=2, k=256, n=16, x=A16, y=Y16, packed=A16):
    stages = (q4._ChainStage * n_stages)(*[q4._ChainStage(x, k, i, 1) for i in range(n_stages)])
    mats = (q4._ChainMatrix * n_stages)(*[q4._ChainMatrix(packed, A16, A16, y, n) for _ in range(n_stages)])
    return stages, mats


def _stage_field(buf, s, off):
    base = 64 + 64 * s
    return int.from_bytes(bytes(buf[base + off:base + off + 4]), "little", signed=True)


def test_chain_encode_validation_and_layout():
    lib = q4.load()
    assert lib.q4_chain_plan_bytes(0, 1) < 0
    nb = lib.q4_chain_plan_bytes(2, 2)
    assert nb == 64 + 2 * 64 + 2 * 48
    buf = (ctypes.c_uint8 * nb)()
    stages, mats = _chain()
    assert lib.q4_chain_encode(ctypes.byref(stages), 2, ctypes.byref(mats), 2, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    hdr = bytes(buf[:16])
    assert int.from_bytes(hdr[0:4], "little") == 0x34433451
    assert int.from_bytes(hdr[4:8], "little") == 2
    # too small a buffer, bad dtype, misaligned x, k not a multiple of 32, stage coverage errors
    assert lib.q4_chain_encode(ctypes.byref(stages), 2, ctypes.byref(mats), 2, 0, ctypes.byref(buf), nb - 1) == q4.Q4_ERR_SHAPE
    assert lib.q4_chain_encode(ctypes.byref(stages), 2, ctypes.byref(mats), 2, 5, ctypes.byref(buf), nb) == q4.Q4_ERR_SHAPE
    s2, m2 = _chain(x=ODD)
    assert lib.q4_chain_encode(ctypes.byref(s2), 2, ctypes.byref(m2), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_ALIGN
    s3, m3 = _chain(k=40)
    assert lib.q4_chain_encode(ctypes.byref(s3), 2, ctypes.byref(m3), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_SHAPE
    s4, m4 = _chain()
    s4[1].first_matrix = 0
    assert lib.q4_chain_encode(ctypes.byref(s4), 2, ctypes.byref(m4), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_SHAPE
    s6, m6 = _chain(k=96)  # 3 groups: one chunk, mostly past the row end
    assert lib.q4_chain_encode(ctypes.byref(s6), 2, ctypes.byref(m6), 2, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    # the LDS copy of the plan bounds stages and matrices
    big = lib.q4_chain_plan_bytes(385, 385)
    bigbuf = (ctypes.c_uint8 * big)()
    s9, m9 = _chain(n_stages=385)
    assert lib.q4_chain_encode(ctypes.byref(s9), 385, ctypes.byref(m9), 385, 0, ctypes.byref(bigbuf), big) == q4.Q4_ERR_UNSUPPORTED
    ok = lib.q4_chain_plan_bytes(384, 384)
    okbuf = (ctypes.c_uint8 * ok)()
    s10, m10 = _chain(n_stages=384)
    assert lib.q4_chain_encode(ctypes.byref(s10), 384, ctypes.byref(m10), 384, 0, ctypes.byref(okbuf), ok) == q4.Q4_OK
    s5, m5 = _chain(packed=0)
    assert lib.q4_chain_encode(ctypes.byref(s5), 2, ctypes.byref(m5), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_NULL
    s7, m7 = _chain(y=A16)  # a stage writing its own input
    assert lib.q4_chain_encode(ctypes.byref(s7), 2, ctypes.byref(m7), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_UNSUPPORTED
    s8, m8 = _chain(k=12288 + 256, n=64)  # wider than the executor's activation buffer
    assert lib.q4_chain_encode(ctypes.byref(s8), 2, ctypes.byref(m8), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_UNSUPPORTED


def test_chain_encode_rows_validation():
    """Several activation rows: the row count is checked and stored in the
    plan's header (int32 at byte 20), the executor's lower limits for 2..4
    rows are enforced, and buffer overlap is judged on m_rows rows."""
    lib = q4.load()
    nb = lib.q4_chain_plan_bytes(2, 2)
    buf = (ctypes.c_uint8 * nb)()

    def enc(stages, mats, m, ns=2, b=buf, size=nb):
        return lib.q4_chain_encode_rows(ctypes.byref(stages), ns, ctypes.byref(mats), ns, m, 0, ctypes.byref(b), size)

    stages, mats = _chain()
    for m in (0, 5, -1):
        assert enc(stages, mats, m) == q4.Q4_ERR_SHAPE
    for m in (1, 2, 3, 4):
        assert enc(stages, mats, m) == q4.Q4_OK
        assert int.from_bytes(bytes(buf[20:24]), "little") == m
    s1, m1 = _chain(k=11264, n=64)
    assert enc(s1, m1, 4) == q4.Q4_OK
    s2, m2 = _chain(k=11264 + 32, n=64)  # wider than the multi-row activation buffer
    assert enc(s2, m2, 2) == q4.Q4_ERR_UNSUPPORTED
    assert enc(s2, m2, 1) == q4.Q4_OK
    # y starts one bf16 row of x past x: disjoint for one row, overlapping for two
    s3, m3 = _chain(k=256, n=16, y=A16 + 2 * 256)
    assert enc(s3, m3, 1) == q4.Q4_OK
    assert enc(s3, m3, 2) == q4.Q4_ERR_UNSUPPORTED
    # the LDS plan tables hold 128 stages for several rows (384 for one)
    n129 = lib.q4_chain_plan_bytes(129, 129)
    b129 = (ctypes.c_uint8 * n129)()
    s4, m4 = _chain(n_stages=129)
    assert enc(s4, m4, 2, 129, b129, n129) == q4.Q4_ERR_UNSUPPORTED
    assert enc(s4, m4, 1, 129, b129, n129) == q4.Q4_OK
    n128 = lib.q4_chain_plan_bytes(128, 128)
    b128 = (ctypes.c_uint8 * n128)()
    s5, m5 = _chain(n_stages=128)
    assert enc(s5, m5, 4, 128, b128, n128) == q4.Q4_OK
    # 32 units of 4 rows per block: n up to 32 * 4 * 256 compute units
    s6, m6 = _chain(n=32 * 4 * 256)
    assert enc(s6, m6, 2) == q4.Q4_OK
    assert enc(s6, m6, 1) == q4.Q4_OK
    s7, m7 = _chain(n=32 * 4 * 256 + 4)
    assert enc(s7, m7, 2) == q4.Q4_ERR_UNSUPPORTED
    assert enc(s7, m7, 1) == q4.Q4_ERR_UNSUPPORTED


def test_chain_run_rows_validation():
    lib = q4.load()
    for m in (0, 5):
        assert lib.q4_chain_run_rows(_p(A16), m, 0, _p(A16), None) == q4.Q4_ERR_SHAPE
    assert lib.q4_chain_run_rows(None, 2, 0, _p(A16), None) == q4.Q4_ERR_NULL
    assert lib.q4_chain_run_rows(_p(A16), 2, 3, _p(A16), None) == q4.Q4_ERR_SHAPE


def test_chain_stage_geometry_and_dependencies():
    """Lanes per row and chunk count per stage, and the dependency flags the
    encoder derives from buffer overlap: stage 1 reads stage 0's output."""
    lib = q4.load()
    nb = lib.q4_chain_plan_bytes(3, 3)
    buf = (ctypes.c_uint8 * nb)()
    Y0, Y1, Y2 = 0x400000, 0x800000, 0xC00000
    stages = (q4._ChainStage * 3)(q4._ChainStage(A16, 4096, 0, 1), q4._ChainStage(Y0, 11264, 1, 1),
                                   q4._ChainStage(A16 + 0x100000, 2816, 2, 1))
    mats = (q4._ChainMatrix * 3)(q4._ChainMatrix(A16, A16, A16, Y0, 11264), q4._ChainMatrix(A16, A16, A16, Y1, 4096),
                                 q4._ChainMatrix(A16, A16, A16, Y2, 1024))
    assert lib.q4_chain_encode(ctypes.byref(stages), 3, ctypes.byref(mats), 3, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    # G, CH at byte offsets 8, 12; x_internal 24, sync_outputs 28
    # (16 lanes per row, chunks of 16 groups: CH = ceil(G / 16))
    assert [_stage_field(buf, 0, o) for o in (8, 12)] == [128, 8]
    assert [_stage_field(buf, 1, o) for o in (8, 12)] == [352, 22]
    assert [_stage_field(buf, 2, o) for o in (8, 12)] == [88, 6]     # ragged last chunk
    assert [_stage_field(buf, s, X_INTERNAL) for s in range(3)] == [0, 1, 0]
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(3)] == [1, 0, 0]


X_INTERNAL, SYNC_OUT = 24, 28  # byte offsets in a stage record of the plan


def test_chain_encoder_orders_overlapping_outputs():
    """A later stage that overwrites an earlier stage's outputs makes the
    earlier one store before its barrier (sync flag), as a later stage that
    reads them does; two outputs of one stage may not overlap; a later stage
    writing an earlier stage's input needs no flag."""
    lib = q4.load()
    nb = lib.q4_chain_plan_bytes(3, 3)
    buf = (ctypes.c_uint8 * nb)()
    X0, X1, X2, Y0, Y2 = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000

    def encode(xs, ys, per_stage=(1, 1, 1)):
        firsts = [sum(per_stage[:i]) for i in range(len(per_stage))]
        st = (q4._ChainStage * len(xs))(*[q4._ChainStage(x, 256, f, c) for x, f, c in zip(xs, firsts, per_stage)])
        mt = (q4._ChainMatrix * len(ys))(*[q4._ChainMatrix(A16, A16, A16, y, 16) for y in ys])
        return lib.q4_chain_encode(ctypes.byref(st), len(xs), ctypes.byref(mt), len(ys), 0, ctypes.byref(buf), nb)

    # stage 2 overwrites stage 0's outputs (bf16 [16] = 32 bytes at Y0): stage 0 syncs
    assert encode([X0, X1, X2], [Y0, Y2, Y0 + 16]) == q4.Q4_OK
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(3)] == [1, 0, 0]
    assert [_stage_field(buf, s, X_INTERNAL) for s in range(3)] == [0, 0, 0]
    # disjoint outputs: no flags
    assert encode([X0, X1, X2], [Y0, Y2, Y0 + 32]) == q4.Q4_OK
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(3)] == [0, 0, 0]
    # stage 2 writes stage 0's input: harmless, no flags
    assert encode([X0, X1, X2], [Y0, Y2, X0]) == q4.Q4_OK
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(3)] == [0, 0, 0]
    # stage 1 reads stage 0's output: stage 0 syncs, stage 1's x is internal
    assert encode([X0, Y0, X2], [Y0, Y2, Y0 + 64]) == q4.Q4_OK
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(3)] == [1, 0, 0]
    assert [_stage_field(buf, s, X_INTERNAL) for s in range(3)] == [0, 1, 0]
    # two matrices of one stage writing overlapping outputs are refused
    assert encode([X0, X1], [Y0, Y0 + 30, Y2], per_stage=(2, 1)) == q4.Q4_ERR_UNSUPPORTED
    assert encode([X0, X1], [Y0, Y0 + 32, Y2], per_stage=(2, 1)) == q4.Q4_OK


def test_chain_run_validation():
    lib = q4.load()
    assert lib.q4_chain_run(None, 0, _p(A16), None) == q4.Q4_ERR_NULL
    assert lib.q4_chain_run(_p(A16), 0, _p(A16 + 64), None) == q4.Q4_ERR_ALIGN
    assert lib.q4_chain_run(_p(A16 + 16), 0, _p(A16), None) == q4.Q4_ERR_ALIGN
    assert lib.q4_chain_run(_p(A16), 3, _p(A16), None) == q4.Q4_ERR_SHAPE


def test_chain_run_noalloc_validation():
    """The entry point without a workspace validates like q4_chain_run_rows
    (every call here fails before any HIP call)."""
    lib = q4.load()
    assert lib.q4_chain_run_rows_noalloc(None, 1, 0, None, None) == q4.Q4_ERR_NULL
    assert lib.q4_chain_run_rows_noalloc(_p(A16), 0, 0, None, None) == q4.Q4_ERR_SHAPE
    assert lib.q4_chain_run_rows_noalloc(_p(A16), 5, 0, None, None) == q4.Q4_ERR_SHAPE
    assert lib.q4_chain_run_rows_noalloc(_p(A16), 1, 2, None, None) == q4.Q4_ERR_SHAPE
    assert lib.q4_chain_run_rows_noalloc(_p(A16 + 16), 1, 0, None, None) == q4.Q4_ERR_ALIGN
    assert lib.q4_chain_run_rows_noalloc(_p(A16), 1, 0, _p(A16 + 2), None) == q4.Q4_ERR_ALIGN


def test_embed_sum_validation():
    """Host checks of the gather-sum (no HIP call: each call fails first)."""
    lib = q4.load()

    def tabs(n=2, rows=8, packed=A16, scales=A16):
        return (q4._EmbedTable * n)(*[q4._EmbedTable(packed, scales, A16, rows) for _ in range(n)])

    t = tabs()
    call = lambda tok=A16, frames=1, tb=t, n=2, dim=64, y=Y16, dt=0: lib.q4_embed_sum(
        _p(tok), frames, ctypes.byref(tb) if tb is not None else None, n, dim, _p(y), dt, None)
    assert call(tok=0) == q4.Q4_ERR_NULL
    assert call(y=0) == q4.Q4_ERR_NULL
    assert call(tb=tabs(packed=0)) == q4.Q4_ERR_NULL
    assert call(n=0) == q4.Q4_ERR_SHAPE
    assert call(n=33, tb=tabs(33)) == q4.Q4_ERR_SHAPE
    assert call(dim=48) == q4.Q4_ERR_SHAPE
    assert call(frames=-1) == q4.Q4_ERR_SHAPE
    assert call(dt=2) == q4.Q4_ERR_SHAPE
    assert call(tb=tabs(rows=0)) == q4.Q4_ERR_SHAPE
    assert call(tok=A16 + 2) == q4.Q4_ERR_ALIGN
    assert call(y=Y16 + 8) == q4.Q4_ERR_ALIGN
    assert call(tb=tabs(packed=A16 + 4)) == q4.Q4_ERR_ALIGN
    assert call(tb=tabs(rows=1 << 30), dim=4096) == q4.Q4_ERR_UNSUPPORTED  # past a 32-bit buffer range
    assert call(frames=0) == q4.Q4_OK


def test_attn_decode_validation():
    lib = q4.load()
    ws = lib.q4_attn_workspace_bytes(32, 128)
    assert ws > 0 and lib.q4_attn_workspace_bytes(0, 128) < 0
    W = 0x1000000  # a 256-byte aligned fake workspace address
    call = lambda q=A16, heads=32, d=128, cap=64, pos=3, theta=10000.0, out=Y16, dt=0, w=W, wb=ws: \
        lib.q4_attn_decode(_p(q), _p(A16), _p(A16), _p(A16), _p(A16), heads, d, cap, pos, theta, _p(out), dt,
                           _p(w), wb, None)
    assert call(q=0) == q4.Q4_ERR_NULL
    assert call(w=0) == q4.Q4_ERR_NULL
    assert call(pos=64) == q4.Q4_ERR_SHAPE
    assert call(pos=-1) == q4.Q4_ERR_SHAPE
    assert call(theta=0.0) == q4.Q4_ERR_SHAPE
    assert call(dt=3) == q4.Q4_ERR_SHAPE
    assert call(wb=ws - 1) == q4.Q4_ERR_SHAPE
    assert call(d=96) == q4.Q4_ERR_UNSUPPORTED
    assert call(q=A16 + 2) == q4.Q4_ERR_ALIGN
    assert call(w=W + 16) == q4.Q4_ERR_ALIGN


NORM_PTR, NORM_EPS, GATED = 32, 40, 48  # byte offsets in a stage record of the plan


def _stage_u64(buf, s, off):
    base = 64 + 64 * s
    return int.from_bytes(bytes(buf[base + off:base + off + 8]), "little")


def _encode_ex(stages, mats, rows=1, dtype=0):
    lib = q4.load()
    nb = lib.q4_chain_plan_bytes(len(stages), len(mats))
    buf = (ctypes.c_uint8 * nb)()
    st = (q4._ChainStageEx * len(stages))(*stages)
    mt = (q4._ChainMatrixEx * len(mats))(*mats)
    rc = lib.q4_chain_encode_ex(ctypes.byref(st), len(stages), ctypes.byref(mt), len(mats), rows, dtype,
                                ctypes.byref(buf), nb)
    return rc, buf


def _sx(x, k, first, count, norm=None, eps=1e-5, gated=0):
    return q4._ChainStageEx(x, k, first, count, norm, eps, gated, 0)


def _mx(y, n, residual=None):
    return q4._ChainMatrixEx(A16, A16, A16, y, n, residual)


def test_chain_encode_ex_records_the_fused_parts():
    """The norm weight, eps and gate flag land in the stage record; a gated
    stage's second matrix needs no output."""
    X0, G0, Y0, Y1, Y2 = 0x100000, 0x180000, 0x400000, 0x500000, 0x600000
    rc, buf = _encode_ex([_sx(X0, 256, 0, 1, norm=G0, eps=0.25), _sx(X0, 256, 1, 2, gated=1)],
                         [_mx(Y0, 64), _mx(Y1, 32), _mx(None, 32)])
    assert rc == q4.Q4_OK
    assert _stage_u64(buf, 0, NORM_PTR) == G0 and _stage_u64(buf, 1, NORM_PTR) == 0
    assert struct.unpack("<d", bytes(buf[64 + NORM_EPS:64 + NORM_EPS + 8]))[0] == 0.25
    assert [_stage_field(buf, s, GATED) for s in range(2)] == [0, 1]
    # q4_chain_encode_rows writes the same plan as the extended encoder without fused parts
    lib = q4.load()
    nb = lib.q4_chain_plan_bytes(2, 2)
    plain = (ctypes.c_uint8 * nb)()
    st = (q4._ChainStage * 2)(q4._ChainStage(X0, 256, 0, 1), q4._ChainStage(Y0, 64, 1, 1))
    mt = (q4._ChainMatrix * 2)(q4._ChainMatrix(A16, A16, A16, Y1, 64), q4._ChainMatrix(A16, A16, A16, Y2, 32))
    assert lib.q4_chain_encode_rows(ctypes.byref(st), 2, ctypes.byref(mt), 2, 1, 0, ctypes.byref(plain), nb) == 0
    rc, ex = _encode_ex([_sx(X0, 256, 0, 1, eps=0.0), _sx(Y0, 64, 1, 1, eps=0.0)], [_mx(Y1, 64), _mx(Y2, 32)])
    assert rc == q4.Q4_OK and bytes(ex) == bytes(plain)


@pytest.mark.parametrize("case,want", [
    ("gate_one_matrix", q4.Q4_ERR_SHAPE),
    ("gate_unequal_n", q4.Q4_ERR_SHAPE),
    ("gate_flag_2", q4.Q4_ERR_SHAPE),
    ("gate_residual_on_up", q4.Q4_ERR_SHAPE),
    ("norm_two_rows", q4.Q4_ERR_UNSUPPORTED),
    ("norm_misaligned", q4.Q4_ERR_ALIGN),
    ("eps_negative", q4.Q4_ERR_SHAPE),
    ("eps_nan", q4.Q4_ERR_SHAPE),
    ("residual_misaligned", q4.Q4_ERR_ALIGN),
    ("residual_is_other_output", q4.Q4_ERR_UNSUPPORTED),
    ("output_over_norm", q4.Q4_ERR_UNSUPPORTED),
    ("residual_in_place", q4.Q4_OK),
])
def test_chain_encode_ex_validation(case, want):
    X0, G0, Y0, Y1 = 0x100000, 0x180000, 0x400000, 0x500000
    stages = [_sx(X0, 256, 0, 2)]
    mats = [_mx(Y0, 32), _mx(Y1, 32)]
    rows = 1
    if case == "gate_one_matrix":
        stages = [_sx(X0, 256, 0, 1, gated=1)]
        mats = mats[:1]
    elif case == "gate_unequal_n":
        stages = [_sx(X0, 256, 0, 2, gated=1)]
        mats = [_mx(Y0, 32), _mx(None, 64)]
    elif case == "gate_flag_2":
        stages = [_sx(X0, 256, 0, 2, gated=2)]
    elif case == "gate_residual_on_up":
        stages = [_sx(X0, 256, 0, 2, gated=1)]
        mats = [_mx(Y0, 32), _mx(None, 32, residual=Y1)]
    elif case == "norm_two_rows":
        stages = [_sx(X0, 256, 0, 2, norm=G0)]
        rows = 2
    elif case == "norm_misaligned":
        stages = [_sx(X0, 256, 0, 2, norm=G0 + 2)]
    elif case == "eps_negative":
        stages = [_sx(X0, 256, 0, 2, norm=G0, eps=-1e-6)]
    elif case == "eps_nan":
        stages = [_sx(X0, 256, 0, 2, norm=G0, eps=float("nan"))]
    elif case == "residual_misaligned":
        mats = [_mx(Y0, 32, residual=Y1 + 1), _mx(Y1 + 64, 32)]
    elif case == "residual_is_other_output":
        mats = [_mx(Y0, 32, residual=Y1), _mx(Y1, 32)]
    elif case == "output_over_norm":
        stages = [_sx(X0, 256, 0, 2, norm=Y1)]
    elif case == "residual_in_place":
        mats = [_mx(Y0, 32, residual=Y0), _mx(Y1, 32, residual=Y1)]
    rc, _ = _encode_ex(stages, mats, rows=rows)
    assert rc == want


def test_chain_encode_ex_residual_dependencies():
    """A residual written by an earlier stage makes that stage store before its
    barrier; so does a later stage overwriting a residual an earlier stage
    reads. A residual no stage writes needs no flag."""
    X0, X1, R, Y0, Y1 = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    rc, buf = _encode_ex([_sx(X0, 256, 0, 1), _sx(X1, 256, 1, 1)], [_mx(Y0, 32), _mx(Y1, 32, residual=Y0)])
    assert rc == q4.Q4_OK
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(2)] == [1, 0]
    assert [_stage_field(buf, s, X_INTERNAL) for s in range(2)] == [0, 0]
    rc, buf = _encode_ex([_sx(X0, 256, 0, 1), _sx(X1, 256, 1, 1)], [_mx(Y0, 32, residual=R), _mx(R, 32)])
    assert rc == q4.Q4_OK
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(2)] == [1, 0]
    rc, buf = _encode_ex([_sx(X0, 256, 0, 1), _sx(X1, 256, 1, 1)], [_mx(Y0, 32, residual=R), _mx(Y1, 32, residual=R)])
    assert rc == q4.Q4_OK
    assert [_stage_field(buf, s, SYNC_OUT) for s in range(2)] == [0, 0]


def test_chain_encoder_picks_the_barrier_by_stage_size():
    """Plans whose stages average under 8 MB of weights use the device-counter
    barrier (2), larger ones the L2-flag barrier (1); header word 6."""
    def barrier(n, k, stages=4):
        rc, buf = _encode_ex([_sx(0x100000 * (s + 1), k, s, 1) for s in range(stages)],
                             [_mx(0x4000000 + 0x1000000 * s, n) for s in range(stages)])
        assert rc == q4.Q4_OK
        return int.from_bytes(bytes(buf[24:28]), "little")
    assert barrier(11264, 4096) == 1   # 28.8 MB per stage (a temporal FFN stage)
    assert barrier(1024, 1024) == 2    # 0.66 MB per stage (a Depformer attention stage)


NO_BARRIER = 52  # byte offset in a stage record of the plan


def test_chain_encoder_places_barriers_only_at_dependencies():
    """Stage s starts without a grid barrier unless it reads what a stage since
    the last barrier writes (x or residual), or writes what such a stage reads
    (x or residual) or writes. Independent stages, as in the temporal step with
    activations drawn per stage, run with none."""
    X0, X1, X2, X3, R, Y0, Y1, Y2, Y3 = (0x100000 * i for i in range(1, 10))

    def flags(xs, ys, res=(None,) * 4):
        rc, buf = _encode_ex([_sx(x, 256, i, 1) for i, x in enumerate(xs)],
                             [_mx(y, 128, residual=r) for y, r in zip(ys, res)])
        assert rc == q4.Q4_OK
        return [_stage_field(buf, s, NO_BARRIER) for s in range(len(xs))]

    # independent stages: no barrier anywhere
    assert flags([X0, X1, X2, X3], [Y0, Y1, Y2, Y3]) == [0, 1, 1, 1]
    # stage 2 reads stage 1's output: a barrier before stage 2 only
    assert flags([X0, X1, Y1, X3], [Y0, Y1, Y2, Y3]) == [0, 1, 0, 1]
    # stage 3 reads stage 0's output; a barrier before stage 2 already separates them
    assert flags([X0, X1, Y1, Y0], [Y0, Y1, Y2, Y3]) == [0, 1, 0, 1]
    # ... without it, stage 3 needs its own
    assert flags([X0, X1, X2, Y0], [Y0, Y1, Y2, Y3]) == [0, 1, 1, 0]
    # stage 2 overwrites stage 0's input (a write after a read)
    assert flags([X0, X1, X2, X3], [Y0, Y1, X0, Y3]) == [0, 1, 0, 1]
    # stage 3 overwrites stage 1's output (a write after a write)
    assert flags([X0, X1, X2, X3], [Y0, Y1, Y2, Y1]) == [0, 1, 1, 0]
    # stage 1 adds a residual stage 0 writes; stage 3 overwrites a residual stage 2 reads
    assert flags([X0, X1, X2, X3], [Y0, Y1, Y2, R], res=(None, Y0, R, None)) == [0, 0, 1, 0]
    # a residual no stage writes, read by two stages: no barrier
    assert flags([X0, X1, X2, X3], [Y0, Y1, Y2, Y3], res=(R, None, R, None)) == [0, 1, 1, 1]


def test_chain_encoder_barrier_kind_with_dependent_stages():
    """Counted per stretch between barriers: a chain whose every stage reads
    the last one's output, 0.66 MB per stage, takes the device-counter barrier
    (2); independent stages of 28.8 MB, one stretch of 115 MB, the L2-flag
    barrier (1)."""
    ys = [0x4000000 + 0x1000000 * s for s in range(4)]
    rc, buf = _encode_ex([_sx(0x100000 if s == 0 else ys[s - 1], 1024, s, 1) for s in range(4)],
                         [_mx(ys[s], 1024) for s in range(4)])
    assert rc == q4.Q4_OK
    assert int.from_bytes(bytes(buf[24:28]), "little") == 2
    assert [_stage_field(buf, s, NO_BARRIER) for s in range(4)] == [0, 0, 0, 0]


XOFF, XWAIT = 56, 60  # byte offsets in a stage record of the plan


def test_chain_encoder_places_activations_round_the_arena():
    """One row: each stage's activations get a region of the LDS arena (two
    buffers of the widest, 2 x 384 groups x 20 words), one after another round
    it; a region that does not fit at the end starts again at 0. xwait is the
    last earlier stage whose region overlaps. A normalized stage takes twice
    its size (its norm weights follow). Several rows: one buffer, offset 0."""
    ks = [4096, 4096, 4096, 11264] * 2          # the temporal layer's stages, twice
    xs = [0x100000 * (i + 1) for i in range(len(ks))]
    rc, buf = _encode_ex([_sx(x, k, i, 1) for i, (x, k) in enumerate(zip(xs, ks))],
                         [_mx(0x4000000 + 0x1000000 * i, 64) for i in range(len(ks))])
    assert rc == q4.Q4_OK
    size = [16 * (-(-k // 512)) * 20 for k in ks]  # 16 CH groups of 20 words
    assert size[:4] == [2560, 2560, 2560, 7040]
    assert [_stage_field(buf, s, XOFF) for s in range(8)] == [0, 2560, 5120, 7680, 0, 2560, 5120, 7680]
    assert [_stage_field(buf, s, XWAIT) for s in range(8)] == [-1, -1, -1, -1, 0, 1, 2, 3]
    # a normalized stage of k = 12288 fills the arena: its neighbours wait for it
    rc, buf = _encode_ex([_sx(0x100000, 4096, 0, 1), _sx(0x200000, 12288, 1, 1, norm=0x300000),
                          _sx(0x400000, 4096, 2, 1)],
                         [_mx(0x4000000 + 0x1000000 * i, 64) for i in range(3)])
    assert rc == q4.Q4_OK
    assert [_stage_field(buf, s, XOFF) for s in range(3)] == [0, 0, 0]
    assert [_stage_field(buf, s, XWAIT) for s in range(3)] == [-1, 0, 1]
    rc, buf = _encode_ex([_sx(x, k, i, 1) for i, (x, k) in enumerate(zip(xs[:3], ks[:3]))],
                         [_mx(0x4000000 + 0x1000000 * i, 64) for i in range(3)], rows=2)
    assert rc == q4.Q4_OK
    assert [_stage_field(buf, s, XOFF) for s in range(3)] == [0, 0, 0]
    assert [_stage_field(buf, s, XWAIT) for s in range(3)] == [-1, 0, 1]


def _batch(ns, x=None, scales=None, y=None):
    # fake, aligned device addresses: the encoder only validates and records them
    items = (q4._GemmBatchItem * len(ns))()
    for i, n in enumerate(ns):
        base = 0x100000 * (i + 1)
        items[i] = q4._GemmBatchItem(x if x is not None else base, base + 0x10000,
                                     scales if scales is not None else base + 0x20000, base + 0x30000,
                                     y if y is not None else base + 0x40000, n)
    return items


def test_gemm_batch_encode_validation_and_layout():
    lib = q4.load()
    ns = [16, 17, 1, 40]
    items = _batch(ns)
    blocks = lib.q4_gemm_batch_blocks(ctypes.byref(items), 4)
    assert blocks == 1 + 2 + 1 + 3
    nb = lib.q4_gemm_batch_plan_bytes(4, blocks)
    assert nb == (64 + 4 * 48 + 2 * blocks + 15) // 16 * 16
    buf = (ctypes.c_uint8 * nb)()
    assert lib.q4_gemm_batch_encode(ctypes.byref(items), 4, 8, 4096, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    raw = bytes(buf)
    magic, count, m, G, nblocks, dtype, gs, waves, sb16 = struct.unpack_from("<Iiiiiiiii", raw, 0)
    assert (magic, count, m, G, nblocks, dtype) == (0x51344742, 4, 8, 128, blocks, 0)
    assert (gs, waves, sb16) == (16, 8, 1)  # k = 4096: 16 groups per wave, 8 waves
    starts = [struct.unpack_from("<qqqqqii", raw, 64 + 48 * i) for i in range(4)]
    assert [s[5] for s in starts] == ns and [s[6] for s in starts] == [0, 1, 3, 4]
    assert starts[2][0] == 0x300000 and starts[2][4] == 0x340000
    owner = struct.unpack_from("<%dH" % blocks, raw, 64 + 4 * 48)
    assert owner == (0, 1, 1, 2, 3, 3, 3)
    # the groups-per-wave rule of q4_gemm_small: k = 11264 -> 32 per wave, 11 waves; k = 1024 -> 8, 4
    # and its edges: 16 per wave only while that gives 8..16 waves (k = 3584: 7 -> 8 per wave;
    # k = 8192: 16 waves; k = 8224: 17 -> 32 per wave)
    for k, want in ((11264, (32, 11)), (1024, (8, 4)), (3584, (8, 14)), (3840, (16, 8)), (8192, (16, 16)),
                    (8224, (32, 9)), (16384, (32, 16))):
        assert lib.q4_gemm_batch_encode(ctypes.byref(items), 4, 16, k, 1, ctypes.byref(buf), nb) == q4.Q4_OK
        assert struct.unpack_from("<ii", bytes(buf), 24) == want
    # scales not 16-byte aligned: one-group scale loads for the whole batch
    odd = _batch(ns, scales=0x100002)
    assert lib.q4_gemm_batch_encode(ctypes.byref(odd), 4, 8, 4096, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    assert struct.unpack_from("<i", bytes(buf), 32)[0] == 0
    # refusals
    assert lib.q4_gemm_batch_blocks(None, 4) < 0 and lib.q4_gemm_batch_blocks(ctypes.byref(items), 0) < 0
    assert lib.q4_gemm_batch_blocks(ctypes.byref(_batch([0])), 1) < 0
    assert lib.q4_gemm_batch_plan_bytes(4097, 10) < 0 and lib.q4_gemm_batch_plan_bytes(1, (1 << 24) + 1) < 0
    enc = lambda it, c, m, k, dt=0, n=nb: lib.q4_gemm_batch_encode(ctypes.byref(it), c, m, k, dt, ctypes.byref(buf), n)
    assert enc(items, 4, 4, 4096) == q4.Q4_ERR_SHAPE  # 1..4 rows are the GEMV kernel's
    assert enc(items, 4, 17, 4096) == q4.Q4_ERR_SHAPE
    assert enc(items, 0, 8, 4096) == q4.Q4_ERR_SHAPE
    assert enc(items, 4, 8, 4096, n=nb - 16) == q4.Q4_ERR_SHAPE
    assert enc(items, 4, 8, 4096, dt=2) == q4.Q4_ERR_SHAPE
    assert enc(items, 4, 8, 40) == q4.Q4_ERR_SHAPE
    assert enc(items, 4, 8, 16384 + 32) == q4.Q4_ERR_UNSUPPORTED
    assert enc(_batch(ns, x=0x100008), 4, 8, 4096) == q4.Q4_ERR_ALIGN
    assert enc(_batch(ns, y=0), 4, 8, 4096) == q4.Q4_ERR_NULL
    assert lib.q4_gemm_batch_encode(None, 4, 8, 4096, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_NULL


def test_gemm_batch_run_validation():
    lib = q4.load()
    junk = (ctypes.c_uint8 * 64)()
    assert lib.q4_gemm_batch_run(ctypes.byref(junk), 0x1000, None) == q4.Q4_ERR_SHAPE  # not an encoded plan
    assert lib.q4_gemm_batch_run(None, 0x1000, None) == q4.Q4_ERR_NULL
    items = _batch([32])
    nb = lib.q4_gemm_batch_plan_bytes(1, 2)
    buf = (ctypes.c_uint8 * nb)()
    assert lib.q4_gemm_batch_encode(ctypes.byref(items), 1, 5, 256, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    assert lib.q4_gemm_batch_run(ctypes.byref(buf), 0x1008, None) == q4.Q4_ERR_ALIGN
    assert lib.q4_gemm_batch_run(ctypes.byref(buf), None, None) == q4.Q4_ERR_NULL


def test_step_batches_refuse_dependent_stages_and_row_counts():
    import torch
    from bit_group_quantized_amd.step import Chain, Q4Matrix, Stage
    mat = Q4Matrix(torch.zeros(16, 8, dtype=torch.int32), torch.zeros(16, 2, dtype=torch.bfloat16),
                   torch.zeros(16, 2, dtype=torch.bfloat16))
    y0 = torch.zeros(8, 64, dtype=torch.bfloat16)
    first = Stage(torch.zeros(8, 64, dtype=torch.bfloat16), [mat], [y0[:, :16]])
    reads_y0 = Stage(y0, [mat], [torch.zeros(8, 16, dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="reads an output"):
        Chain([first, reads_y0]).prepare_batches()
    four_rows = Stage(torch.zeros(4, 64, dtype=torch.bfloat16), [mat], [torch.zeros(4, 16, dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="5..16 activation rows"):
        Chain([four_rows]).prepare_batches()


def _no_gpu() -> bool:
    import torch
    return torch.cuda.device_count() == 0  # (counts devices without initialising HIP)


@pytest.mark.skipif(not _no_gpu(), reason="only where no GPU exists: the calls below pass validation and launch")
def test_launch_failure_reports_hip_error():
    """With no device, a call that passes every host check fails at its launch:
    Q4_ERR_HIP, with the runtime's error kept for q4_last_hip_error()."""
    lib = q4.load()
    a = 0x10000000  # aligned stand-in addresses, never dereferenced: the launch fails first
    assert lib.q4_gemv(a, a + 0x100000, a + 0x200000, a + 0x300000, 64, 256, a + 0x400000, 0, None) == q4.Q4_ERR_HIP
    assert lib.q4_last_hip_error() != 0
    assert lib.q4_gemm_small(a, 8, a + 0x100000, a + 0x200000, a + 0x300000, 64, 256, a + 0x400000, 1,
                             None) == q4.Q4_ERR_HIP
    items = (q4._GemmBatchItem * 1)(q4._GemmBatchItem(a, a + 0x100000, a + 0x200000, a + 0x300000, a + 0x400000, 64))
    nb = lib.q4_gemm_batch_plan_bytes(1, 4)
    buf = (ctypes.c_uint8 * nb)()
    assert lib.q4_gemm_batch_encode(ctypes.byref(items), 1, 8, 256, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    assert lib.q4_gemm_batch_run(ctypes.byref(buf), a + 0x500000, None) == q4.Q4_ERR_HIP
    assert q4.q4_status_str(q4.Q4_ERR_HIP)
