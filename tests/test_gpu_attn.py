"""GPU parity of the decode attention (q4_attn_decode) against the CPU oracle:
the new cache rows are the oracle's rotated k (bit for bit) and v; the other
rows are untouched; the output is within tolerance of the oracle's float64
attention over the oracle-built cache; one position returns v exactly; the
model's 32 heads x 128 and a 64-wide head; positions from 0 to a full cache."""
import numpy as np
import pytest
import torch

import bit_group_quantized_amd as q4
import oracle
import workloads
from helpers import TOL_BF16, TOL_F32, bf16_bits_np, out_np, to_gpu_bf16_bits

pytestmark = pytest.mark.gpu


def _case(heads, d, cap, pos, seed):
    q = workloads.activations(seed, 10, 0, 0, heads, d)
    k_new = workloads.activations(seed, 10, 0, 1, heads, d)
    v_new = workloads.activations(seed, 10, 0, 2, heads, d)
    k_cache = workloads.activations(seed, 10, 0, 3, heads * cap, d).reshape(heads, cap, d)
    v_cache = workloads.activations(seed, 10, 0, 4, heads * cap, d).reshape(heads, cap, d)
    return q, k_new, v_new, k_cache, v_cache


def _run(q, k_new, v_new, k_cache, v_cache, pos, out_dtype):
    gk, gv = to_gpu_bf16_bits(k_cache), to_gpu_bf16_bits(v_cache)
    heads, cap, d = k_cache.shape
    ws = torch.zeros(q4.q4_attn_workspace_bytes(heads, d), dtype=torch.uint8, device="cuda:0")
    out = q4.q4_attn_decode(to_gpu_bf16_bits(q), to_gpu_bf16_bits(k_new), to_gpu_bf16_bits(v_new), gk, gv, pos,
                            out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out, bf16_bits_np(gk), bf16_bits_np(gv), ws


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pos", [0, 1, 63, 64, 1000, 4095])
def test_model_heads_match_oracle(pos, out_dtype):
    heads, d, cap = 32, 128, 4096
    q, k_new, v_new, k_cache, v_cache = _case(heads, d, cap, pos, seed=pos)
    out, gk, gv, ws = _run(q, k_new, v_new, k_cache, v_cache, pos, out_dtype)
    k_rot = oracle.rope(k_new, pos)
    q_rot = oracle.rope(q, pos)
    # the new rows are the oracle's rotated k and the given v; no other row moves
    assert np.array_equal(gk[:, pos, :], k_rot)
    assert np.array_equal(gv[:, pos, :], v_new)
    others = [t for t in range(cap) if t != pos]
    assert np.array_equal(gk[:, others, :], k_cache[:, others, :])
    assert np.array_equal(gv[:, others, :], v_cache[:, others, :])
    # the rotated query (bf16 [heads][D] in the workspace, after the heads'
    # split counters, which the call leaves at zero)
    off = -(-heads * 4 // 256) * 256
    assert not ws[: heads * 4].any()
    assert np.array_equal(ws[off: off + heads * d * 2].cpu().numpy().view(np.uint16).reshape(heads, d), q_rot)
    k_ref, v_ref = k_cache.copy(), v_cache.copy()
    k_ref[:, pos, :] = k_rot
    v_ref[:, pos, :] = v_new
    ref = oracle.attn_decode(q_rot, k_ref, v_ref, pos)
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    assert oracle.floored_rel_err(out_np(out), ref) <= tol


@pytest.mark.parametrize("pos", [0, 5, 777])
def test_head_width_64(pos):
    heads, d, cap = 16, 64, 800
    q, k_new, v_new, k_cache, v_cache = _case(heads, d, cap, pos, seed=100 + pos)
    out, gk, gv, _ = _run(q, k_new, v_new, k_cache, v_cache, pos, torch.float32)
    k_rot, q_rot = oracle.rope(k_new, pos), oracle.rope(q, pos)
    assert np.array_equal(gk[:, pos, :], k_rot)
    k_ref, v_ref = k_cache.copy(), v_cache.copy()
    k_ref[:, pos, :] = k_rot
    v_ref[:, pos, :] = v_new
    assert oracle.floored_rel_err(out_np(out), oracle.attn_decode(q_rot, k_ref, v_ref, pos)) <= TOL_F32


def test_first_position_returns_the_new_value_exactly():
    heads, d, cap = 32, 128, 16
    q, k_new, v_new, k_cache, v_cache = _case(heads, d, cap, 0, seed=7)
    out, _, _, _ = _run(q, k_new, v_new, k_cache, v_cache, 0, torch.float32)
    assert np.array_equal(out.cpu().numpy(), oracle.bf16_value(v_new))


def test_full_cache_last_position():
    heads, d, cap = 32, 128, 3000
    pos = cap - 1
    q, k_new, v_new, k_cache, v_cache = _case(heads, d, cap, pos, seed=9)
    out, _, _, _ = _run(q, k_new, v_new, k_cache, v_cache, pos, torch.bfloat16)
    k_ref, v_ref = k_cache.copy(), v_cache.copy()
    k_ref[:, pos, :] = oracle.rope(k_new, pos)
    v_ref[:, pos, :] = v_new
    ref = oracle.attn_decode(oracle.rope(q, pos), k_ref, v_ref, pos)
    assert oracle.floored_rel_err(out_np(out), ref) <= TOL_BF16


def test_long_context_several_batches_per_split():
    """20001 positions: each of the 32 splits of a head takes ~626 positions,
    five batches of loads with the online softmax carried across them."""
    heads, d, cap = 32, 128, 20001
    pos = cap - 1
    q, k_new, v_new, k_cache, v_cache = _case(heads, d, cap, pos, seed=21)
    out, _, _, _ = _run(q, k_new, v_new, k_cache, v_cache, pos, torch.float32)
    k_ref, v_ref = k_cache.copy(), v_cache.copy()
    k_ref[:, pos, :] = oracle.rope(k_new, pos)
    v_ref[:, pos, :] = v_new
    ref = oracle.attn_decode(oracle.rope(q, pos), k_ref, v_ref, pos)
    assert oracle.floored_rel_err(out_np(out), ref) <= TOL_F32


def test_workspace_reused_across_calls():
    """One workspace for calls with different split counts (1, 32, 2 splits per
    head): the heads' counters come back to zero after every call."""
    heads, d, cap = 32, 128, 4096
    ws = torch.zeros(q4.q4_attn_workspace_bytes(heads, d), dtype=torch.uint8, device="cuda:0")
    for i, pos in enumerate((10, 4095, 100)):
        q, k_new, v_new, k_cache, v_cache = _case(heads, d, cap, pos, seed=30 + i)
        gk, gv = to_gpu_bf16_bits(k_cache), to_gpu_bf16_bits(v_cache)
        out = q4.q4_attn_decode(to_gpu_bf16_bits(q), to_gpu_bf16_bits(k_new), to_gpu_bf16_bits(v_new), gk, gv, pos,
                                out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert not ws[: heads * 4].any(), pos
        k_ref, v_ref = k_cache.copy(), v_cache.copy()
        k_ref[:, pos, :] = oracle.rope(k_new, pos)
        v_ref[:, pos, :] = v_new
        ref = oracle.attn_decode(oracle.rope(q, pos), k_ref, v_ref, pos)
        assert oracle.floored_rel_err(out_np(out), ref) <= TOL_F32, pos
