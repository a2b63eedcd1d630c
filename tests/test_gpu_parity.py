"""GPU parity: the HIP library against the CPU oracle on seeded inputs.

Pack and unpack must be bit-exact; products must meet the floored relative
tolerance (1e-2 for bf16 outputs, 2e-3 for fp32 outputs). Inputs to each
product are the ORACLE's packed arrays, so product parity does not depend on
the GPU quantizer; expected values come only from ``oracle``.
"""
import numpy as np
import pytest
import torch

import bit_group_quantized_amd as q4
import oracle
import workloads
from helpers import (TOL_BF16, TOL_F32, bf16_bits_np, dev, out_np, packed_np, to_gpu_bf16_bits, to_gpu_f32,
                     upload_quantized)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    q4.load()


def _w(n, k, seed=0, item=0):
    return workloads.weights(seed, 9, 0, item, n, k)


def _x(m, k, seed=0, item=0):
    return workloads.activations(seed, 9, 0, item, m, k)


# shapes: (n, k) — several tiles plus ragged tails, and the pages' layer shapes
SMALL_SHAPES = [(1, 32), (5, 64), (37, 96), (100, 160), (257, 256), (300, 1056), (1000, 2048), (129, 4096)]
MODEL_SHAPES = [(4096, 4096), (11264, 4096), (4096, 11264), (1024, 1024), (2816, 1024), (1024, 2816)]


# ------------------------------------------------------------------ pack / unpack

@pytest.mark.parametrize("n,k", SMALL_SHAPES + MODEL_SHAPES)
def test_pack_bit_exact(n, k):
    w = _w(n, k, seed=n + k)
    P, S, B = oracle.quantize(w)
    gp, gs, gb = q4.q4_pack(to_gpu_f32(w))
    torch.cuda.synchronize()
    assert np.array_equal(packed_np(gp), P)
    assert np.array_equal(bf16_bits_np(gs), S)
    assert np.array_equal(bf16_bits_np(gb), B)


def _edge_weights():
    """Degenerate groups, exact-affine groups, exact ties of the code rounding,
    signed zeros, huge and tiny magnitudes."""
    r = np.random.default_rng(5)
    rows = []
    rows.append(np.full(64, 0.7, dtype=np.float32))                      # constant groups
    z = np.zeros(64, dtype=np.float32); z[3] = -0.0; z[40] = 1e-40; rows.append(z)
    a, s0 = -1.5, 0.25
    codes = np.concatenate([np.arange(16), np.arange(16)[::-1], r.integers(0, 16, 32)])
    codes[32] = 0; codes[33] = 15
    rows.append((a + s0 * codes).astype(np.float32))                        # exact affine
    t = np.zeros(64, dtype=np.float32)
    t[0] = 0.0; t[1] = 15 * 0.125                                           # scale 0.125, bias 0
    t[2:32] = (np.arange(30) % 15 + 0.5) * 0.125                            # exact half-way ties
    t[32:] = (r.integers(-1000, 1000, 32) * 0.5).astype(np.float32)
    rows.append(t)
    rows.append((r.standard_normal(64) * 1e30).astype(np.float32))
    rows.append((r.standard_normal(64) * 1e-30).astype(np.float32))
    big = r.standard_normal(64).astype(np.float32); big[5] = 300.0; rows.append(big)
    return np.stack(rows)


def test_pack_edge_cases_bit_exact():
    w = _edge_weights()
    P, S, B = oracle.quantize(w)
    gp, gs, gb = q4.q4_pack(to_gpu_f32(w))
    torch.cuda.synchronize()
    assert np.array_equal(packed_np(gp), P)
    assert np.array_equal(bf16_bits_np(gs), S)
    assert np.array_equal(bf16_bits_np(gb), B)


@pytest.mark.parametrize("n,k", [(37, 96), (4096, 4096), (7, 64)])
def test_unpack_bit_exact(n, k):
    w = _edge_weights() if n == 7 else _w(n, k, seed=3)
    P, S, B = oracle.quantize(w)
    q_ref, w_ref = oracle.unpack(P, S, B, w.shape[1])
    q, wh = q4.q4_unpack(*upload_quantized(P, S, B))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(wh.cpu().numpy().view(np.uint32), w_ref.view(np.uint32))


# ------------------------------------------------------------------ products

def _check(y_gpu: torch.Tensor, y_ref: np.ndarray, out_dtype):
    got = out_np(y_gpu).reshape(y_ref.shape)
    err = oracle.floored_rel_err(got, y_ref)
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    assert err <= tol, f"floored rel err {err:.3e} > {tol}"
    if out_dtype == torch.bfloat16:
        # a bf16 output is at most one rounding away from the exact value plus
        # the fp32 accumulation error
        assert err <= 2 ** -8 + TOL_F32
    return err


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,k", SMALL_SHAPES + MODEL_SHAPES)
def test_gemv_matches_oracle(n, k, out_dtype):
    w = _w(n, k, seed=7 * n + k)
    P, S, B = oracle.quantize(w)
    x = _x(1, k, seed=k)
    y_ref = oracle.matmul(x, P, S, B, k)
    y = q4.q4_gemv(to_gpu_bf16_bits(x[0]), *upload_quantized(P, S, B), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(y, y_ref[0], out_dtype)


@pytest.mark.parametrize("m", [2, 3, 4, 7, 16])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,k", [(37, 96), (300, 1056), (1000, 2048), (8197, 4096)] + MODEL_SHAPES)
def test_gemm_small_matches_oracle(n, k, m, out_dtype):
    w = _w(n, k, seed=n + 3 * k)
    P, S, B = oracle.quantize(w)
    x = _x(m, k, seed=m + k)
    y_ref = oracle.matmul(x, P, S, B, k)
    y = q4.q4_gemm_small(to_gpu_bf16_bits(x), *upload_quantized(P, S, B), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(y, y_ref, out_dtype)


# The host planner picks the kernel variant from k. The model shapes reach the
# GEMV with 64/32 lanes per row and the MFMA kernel with 8 (k = 1024, 2816),
# 16 (k = 4096) and 32 (k = 11264) groups per wave; these k reach the others:
# 16 lanes per row (G = 16, 48, 80 groups) and 16 groups per wave at 9..16
# waves (G = 129, 200, 256; m <= 4 take the GEMV, also 16 lanes).
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("k", [512, 1536, 2560])
def test_gemv_sixteen_lane_rows(k, out_dtype):
    n = 1000
    P, S, B = oracle.quantize(_w(n, k, seed=k + 1))
    x = _x(1, k, seed=k + 2)
    y = q4.q4_gemv(to_gpu_bf16_bits(x[0]), *upload_quantized(P, S, B), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(y, oracle.matmul(x, P, S, B, k)[0], out_dtype)


# With one activation row each lane keeps 8, 4 or 2 weight rows in flight,
# the most that still gives >= 8 blocks per compute unit (k = 2048: one lane
# per group, one row per wave): on 256 compute units 16421 rows take 8 (the
# last block ragged), 8197 rows take 4 and 1000 rows take 2.
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [16421, 8197, 1000])
def test_gemv_rows_in_flight(n, out_dtype):
    k = 2048
    P, S, B = oracle.quantize(_w(n, k, seed=n + 5))
    x = _x(1, k, seed=n + 6)
    y = q4.q4_gemv(to_gpu_bf16_bits(x[0]), *upload_quantized(P, S, B), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(y, oracle.matmul(x, P, S, B, k)[0], out_dtype)


@pytest.mark.parametrize("m", [1, 2, 4, 7, 16])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("k", [4128, 6400, 8192])
def test_gemm_small_sixteen_group_waves(k, m, out_dtype):
    n = 300
    P, S, B = oracle.quantize(_w(n, k, seed=k + 3))
    x = _x(m, k, seed=k + m)
    y = q4.q4_gemm_small(to_gpu_bf16_bits(x), *upload_quantized(P, S, B), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(y, oracle.matmul(x, P, S, B, k), out_dtype)


@pytest.mark.parametrize("m", [1, 2, 4, 7, 16, 50])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_products_on_edge_weights(m, out_dtype):
    """The pack edge cases (degenerate and exact-affine groups, exact code ties,
    subnormal and signed-zero inputs, magnitudes near 1e30 and 1e-30) as
    weights of a product, tiled to k = 4096 over 21 rows."""
    w = np.tile(_edge_weights(), (3, 64))
    k = w.shape[1]
    P, S, B = oracle.quantize(w)
    x = _x(m, k, seed=50 + m)
    gx = to_gpu_bf16_bits(x if m > 1 else x[0])
    if m == 1:
        y = q4.q4_gemv(gx, *upload_quantized(P, S, B), out_dtype=out_dtype)
    else:
        y = q4.q4_gemm_small(gx, *upload_quantized(P, S, B), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.matmul(x, P, S, B, k)
    _check(y, ref[0] if m == 1 else ref, out_dtype)


# Prefill (17..64 rows): one pass of the prefill kernel over 2..4 tiles of 16
# rows of x (ragged last tile included), at 8, 16 and 32 groups per wave
# (k = 4096, 6400 and 11264 among the shapes).
@pytest.mark.parametrize("m", [17, 24, 32, 33, 50, 64])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,k", [(37, 96), (300, 1056), (4096, 4096), (11264, 4096), (4096, 11264), (100, 16384),
                                 (64, 6400)])
def test_prefill_matches_oracle(n, k, m, out_dtype):
    P, S, B = oracle.quantize(_w(n, k, seed=n + 5 * k))
    x = _x(m, k, seed=m + 7 * k)
    y = q4.q4_gemm_small(to_gpu_bf16_bits(x), *upload_quantized(P, S, B), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(y, oracle.matmul(x, P, S, B, k), out_dtype)


def test_prefill_rows_equal_single_rows():
    """Row i of a 50-row prefill agrees with the GEMV of row i; the one-hot
    input in the last row selects a column exactly."""
    n, k, m = 4096, 4096, 50
    P, S, B = oracle.quantize(_w(n, k, seed=41))
    _, w_hat = oracle.unpack(P, S, B, k)
    gP, gS, gB = upload_quantized(P, S, B)
    x = _x(m, k, seed=42)
    x[m - 1] = 0
    x[m - 1, 777] = 0x3F80
    Y = q4.q4_gemm_small(to_gpu_bf16_bits(x), gP, gS, gB, out_dtype=torch.float32)
    for i in (0, 31, 32, 48):
        y = q4.q4_gemv(to_gpu_bf16_bits(x[i]), gP, gS, gB, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert oracle.floored_rel_err(out_np(Y[i]), out_np(y)) <= 2 * TOL_F32
    torch.cuda.synchronize()
    assert np.array_equal(Y[m - 1].cpu().numpy(), w_hat[:, 777])


@pytest.mark.parametrize("m", [1, 2, 16])
def test_one_hot_input_gives_exact_dequantized_column(m):
    """x = e_j in one activation row: y = w_hat[:, j] exactly in fp32 (pins the
    code, group, scale and bias indexing through the kernels)."""
    n, k = 160, 4096
    w = _w(n, k, seed=99)
    P, S, B = oracle.quantize(w)
    _, w_hat = oracle.unpack(P, S, B, k)
    gP, gS, gB = upload_quantized(P, S, B)
    for j in (0, 1, 7, 8, 31, 32, 33, 1000, 4095):
        x = np.zeros((m, k), dtype=np.uint16)
        x[m - 1, j] = 0x3F80
        gx = to_gpu_bf16_bits(x)
        y = q4.q4_gemm_small(gx, gP, gS, gB, out_dtype=torch.float32)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.array_equal(got[m - 1], w_hat[:, j]), j
        if m > 1:
            assert not got[: m - 1].any()


def test_gemm_rows_equal_gemv():
    """Each row of the small GEMM agrees with a GEMV of that row within tolerance."""
    n, k, m = 4096, 4096, 4
    w = _w(n, k, seed=17)
    P, S, B = oracle.quantize(w)
    gP, gS, gB = upload_quantized(P, S, B)
    x = _x(m, k, seed=5)
    Y = q4.q4_gemm_small(to_gpu_bf16_bits(x), gP, gS, gB, out_dtype=torch.float32)
    for i in range(m):
        y = q4.q4_gemv(to_gpu_bf16_bits(x[i]), gP, gS, gB, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert oracle.floored_rel_err(out_np(Y[i]), out_np(y)) <= 2 * TOL_F32


@pytest.mark.parametrize("m", [1, 4, 16])
def test_widest_k(m):
    """k at the library's limit (16384: 512 groups, the MFMA kernel's 32 groups
    per wave times 16 waves), with a ragged row count."""
    n, k = 100, q4.MAX_K
    P, S, B = oracle.quantize(_w(n, k, seed=31))
    x = _x(m, k, seed=32 + m)
    gx = to_gpu_bf16_bits(x if m > 1 else x[0])
    if m == 1:
        y = q4.q4_gemv(gx, *upload_quantized(P, S, B), out_dtype=torch.float32)
    else:
        y = q4.q4_gemm_small(gx, *upload_quantized(P, S, B), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matmul(x, P, S, B, k)
    _check(y, ref[0] if m == 1 else ref, torch.float32)


def test_deterministic():
    n, k = 11264, 4096
    w = _w(n, k, seed=23)
    P, S, B = oracle.quantize(w)
    gP, gS, gB = upload_quantized(P, S, B)
    x = to_gpu_bf16_bits(_x(1, k, seed=1)[0])
    X = to_gpu_bf16_bits(_x(16, k, seed=2))
    a = q4.q4_gemv(x, gP, gS, gB, out_dtype=torch.float32)
    b = q4.q4_gemv(x, gP, gS, gB, out_dtype=torch.float32)
    c = q4.q4_gemm_small(X, gP, gS, gB, out_dtype=torch.float32)
    d = q4.q4_gemm_small(X, gP, gS, gB, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(c.view(torch.int32), d.view(torch.int32))


# ------------------------------------------------------------------ product batch

def _batch_case(ns, k, m, out_dtype, seed):
    mats, xs, outs, refs = [], [], [], []
    for i, n in enumerate(ns):
        P, S, B = oracle.quantize(_w(n, k, seed=seed, item=i))
        x = _x(m, k, seed=seed + 1, item=i)
        refs.append(oracle.matmul(x, P, S, B, k))
        mats.append(upload_quantized(P, S, B))
        xs.append(to_gpu_bf16_bits(x))
        outs.append(torch.full((m, n), float("nan"), dtype=out_dtype, device=dev()))
    return mats, xs, outs, refs


# ragged row counts (1, 17, 40 rows: partial 16-row blocks), one-group-scale
# loads (k = 96, 1056: k not a multiple of 256) and the model's widths with 16
# (k = 4096) and 32 (k = 11264) groups per wave
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m", [5, 8, 16])
@pytest.mark.parametrize("ns,k", [([37, 1, 300, 16, 17], 96), ([129, 1000, 64], 1056),
                                  ([4096, 11264, 40], 4096), ([300, 4096], 11264)])
def test_gemm_batch_matches_oracle_and_single_calls(ns, k, m, out_dtype):
    mats, xs, outs, refs = _batch_case(ns, k, m, out_dtype, seed=31 * k + m)
    plan = q4.q4_gemm_batch_build(xs, mats, outs)
    q4.q4_gemm_batch_run(plan)
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    for o in outs:
        o.fill_(float("nan"))
    q4.q4_gemm_batch_run(plan)  # the same plan again: the same bits
    torch.cuda.synchronize()
    for i, n in enumerate(ns):
        _check(outs[i], refs[i], out_dtype)
        single = q4.q4_gemm_small(xs[i], *mats[i], out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(outs[i].view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           single.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)), f"item {i}"
        assert torch.equal(first[i].view(torch.uint8), outs[i].view(torch.uint8))


def test_gemm_batch_of_a_full_layer():
    """One temporal layer's seven matrices (q, k, v, o, gate, up at k = 4096;
    down at k = 11264) as two batches, against one call per matrix, bit for bit."""
    m = 16
    shapes = [(4096, 4096)] * 4 + [(11264, 4096)] * 2
    outs4, xs4, mats4, singles = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        w = _w(n, k, seed=5, item=i)
        mats4.append(upload_quantized(*oracle.quantize(w)))
        xs4.append(to_gpu_bf16_bits(_x(m, k, seed=6, item=i)))
        outs4.append(torch.empty((m, n), dtype=torch.bfloat16, device=dev()))
    Pd = upload_quantized(*oracle.quantize(_w(4096, 11264, seed=5, item=7)))
    xd = to_gpu_bf16_bits(_x(m, 11264, seed=6, item=7))
    yd = torch.empty((m, 4096), dtype=torch.bfloat16, device=dev())
    q4.q4_gemm_batch_run(q4.q4_gemm_batch_build(xs4, mats4, outs4))
    q4.q4_gemm_batch_run(q4.q4_gemm_batch_build([xd], [Pd], [yd]))
    torch.cuda.synchronize()
    for x, mat, y in zip(xs4 + [xd], mats4 + [Pd], outs4 + [yd]):
        ref = q4.q4_gemm_small(x, *mat)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_step_batches_equal_launches():
    """The step module's batch executor (one launch per k) against its
    one-launch-per-matrix executor on a chain of two widths, bit for bit."""
    from bit_group_quantized_amd.step import Chain, Q4Matrix, Stage
    m = 8
    stages = []
    for si, (ns, k) in enumerate([((300, 17), 1024), ((129,), 2816), ((64, 1000), 1024)]):
        mats = [Q4Matrix(*upload_quantized(*oracle.quantize(_w(n, k, seed=40 + si, item=j)))) for j, n in enumerate(ns)]
        stages.append(Stage(to_gpu_bf16_bits(_x(m, k, seed=50 + si)), mats))
    chain = Chain(stages)
    chain.run_launches()
    torch.cuda.synchronize()
    want = [y.clone() for st in stages for y in st.outs]
    for st in stages:
        for y in st.outs:
            y.fill_(float("nan"))
    chain.run_batches()
    torch.cuda.synchronize()
    assert len(chain._batches) == 2
    for got, ref in zip([y for st in stages for y in st.outs], want):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------------------------ MultiLinear

@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("out,k", [(1024, 1024), (2816, 1024), (1024, 2816), (40, 96)])
def test_multilinear_steps(out, k, m):
    steps = workloads.DEP_STEPS if out * k <= 2816 * 1024 else 4
    W = np.concatenate([_w(out, k, seed=200 + s, item=s) for s in range(steps)])
    P, S, B = oracle.quantize(W)
    gP, gS, gB = upload_quantized(P, S, B)
    x = _x(m, k, seed=out)
    gx = to_gpu_bf16_bits(x)
    for s in range(steps):
        y_ref = oracle.multilinear_step(x, P, S, B, steps, out, k, s)
        y = q4.q4_multilinear_step(gx, gP, gS, gB, steps, s, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check(y, y_ref, torch.float32)
        # the step is the product on that row block: bit-identical to a direct call
        blk = slice(s * out, (s + 1) * out)
        direct = q4.q4_gemm_small(gx, gP[blk].contiguous(), gS[blk].contiguous(), gB[blk].contiguous(),
                                  out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), direct.view(torch.int32))


def test_multilinear_out_of_range_step_raises():
    P, S, B = oracle.quantize(_w(64, 64))
    gP, gS, gB = upload_quantized(P, S, B)
    x = to_gpu_bf16_bits(_x(1, 64))
    with pytest.raises(q4.Q4Error):
        q4.q4_multilinear_step(x, gP, gS, gB, 4, 4)
