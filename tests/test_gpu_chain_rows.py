"""GPU parity of the persistent chain executor with 2..4 activation rows (several
conversations sharing every weight stream) against the CPU oracle.

* independent stages of the model's shapes, each row its own activation;
* a dependent chain where each stage's [m, k] activation IS the previous
  stage's bf16 [m, n] output, outputs pre-filled with a poison value;
* the chain against one q4_gemm_small launch per matrix on the same inputs;
* a plan encoded for one row count run with another is refused by the kernel;
* the small-GEMM step at m=4 (chain) and m=16 (per-matrix launches) exactly as
  the benchmark builds and runs it, sampled layers against the oracle.
"""
import numpy as np
import pytest
import torch

import bit_group_quantized_amd as q4
import oracle
import workloads
from bit_group_quantized_amd.step import Chain, Q4Matrix, Stage
from helpers import TOL_BF16, TOL_F32, bf16_bits_np, out_np, to_gpu_bf16_bits, upload_quantized

pytestmark = pytest.mark.gpu

SPECS = [  # (k, [n...])
    (4096, [4096, 4096, 1000]),
    (11264, [4096]),         # the widest activation the multi-row executor stages
    (1024, [1024, 37]),
    (4096, [11264]),
    (2816, [1024]),
    (256, [300]),            # 8 groups: one chunk, half of its lanes past the row end
    (6400, [128]),           # 200 groups: the last chunk ragged
    (96, [40]),              # 3 groups
    (4128, [70]),            # 129 groups
    (11264, [37]),           # 10 units: pieces of 22 chunks
]

_QUANT = {}


def _mat(n, k, seed, item):
    key = (n, k, seed, item)
    if key not in _QUANT:
        w = workloads.weights(seed, 8, 0, item, n, k)
        _QUANT[key] = oracle.quantize(w)
    P, S, B = _QUANT[key]
    return (P, S, B), Q4Matrix(*upload_quantized(P, S, B))


@pytest.mark.parametrize("m,out_dtype", [(2, torch.float32), (3, torch.bfloat16), (4, torch.float32),
                                         (4, torch.bfloat16)])
def test_independent_stages_rows(m, out_dtype):
    stages, refs = [], []
    item = 0
    for si, (k, ns) in enumerate(SPECS):
        x = workloads.activations(si, 8, 5, si, m, k)
        mats = []
        for n in ns:
            (P, S, B), mt = _mat(n, k, si, item)
            item += 1
            mats.append(mt)
            refs.append(oracle.matmul(x, P, S, B, k))
        stages.append(Stage(to_gpu_bf16_bits(x), mats))
    chain = Chain(stages, out_dtype)
    for _ in range(2):
        chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    outs = [y for st in stages for y in st.outs]
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    for y, ref in zip(outs, refs):
        assert tuple(y.shape) == ref.shape
        assert oracle.floored_rel_err(out_np(y), ref) <= tol


def _selector_matrix(n, k, pick):
    """Stored Q4 matrix whose row r has code 1 at input pick[r] and 0 elsewhere,
    scale 1.0 and bias 0.0 in every group: w_hat row r is the unit vector
    e_pick[r] (code of input 8j+t in bits [4t, 4t+4) of word j)."""
    packed = np.zeros((n, k // 8), dtype=np.uint32)
    packed[np.arange(n), pick // 8] = (np.uint32(1) << (4 * (pick % 8)).astype(np.uint32))
    scales = np.full((n, k // 32), 0x3F80, dtype=np.uint16)
    biases = np.zeros((n, k // 32), dtype=np.uint16)
    return packed, scales, biases


@pytest.mark.parametrize("m", [2, 4])
def test_dependent_chain_rows(m):
    """Stage s reads stage s-1's [m, n] bf16 output. Every output is an earlier
    integer input (bit-exact against the oracle); the rows differ, so a row
    read from the wrong conversation fails, and outputs start poisoned (1e4),
    so a stage that read its input before the previous one finished fails."""
    shapes = [(4096, 4096)] * 5 + [(11264, 4096), (4096, 11264), (4096, 4096), (1024, 4096), (4096, 1024)]
    r = np.random.default_rng(23 + m)
    x0 = workloads.bf16_bits_rne(r.integers(-64, 65, size=(m, shapes[0][1])).astype(np.float32))
    host, stages = [], []
    x = to_gpu_bf16_bits(x0)
    for (n, k) in shapes:
        P, S, B = _selector_matrix(n, k, r.integers(0, k, size=n))
        host.append((P, S, B))
        y = torch.full((m, n), 1.0e4, dtype=torch.bfloat16, device=x.device)
        stages.append(Stage(x, [Q4Matrix(*upload_quantized(P, S, B))], [y]))
        x = y
    chain = Chain(stages, torch.bfloat16)
    for rep in range(3):
        for st in stages:
            st.outs[0].fill_(1.0e4)
        chain.run_chain()
        torch.cuda.synchronize()
        assert chain.chain_status() == 0
        xr = x0
        for i, (n, k) in enumerate(shapes):
            P, S, B = host[i]
            y_ref = oracle.output_bits_bf16(oracle.matmul(xr, P, S, B, k))
            assert np.array_equal(bf16_bits_np(stages[i].outs[0]), y_ref), (rep, i)
            xr = y_ref


def test_rows_chain_matches_gemm_small_launches():
    """The chain at m=4 and one q4_gemm_small launch per matrix agree."""
    m = 4
    specs = [(4096, [4096, 4096]), (11264, [4096]), (4096, [11264])]
    stages = []
    for si, (k, ns) in enumerate(specs):
        x = workloads.activations(si, 8, 6, si, m, k)
        stages.append(Stage(to_gpu_bf16_bits(x), [_mat(n, k, 70 + si, j)[1] for j, n in enumerate(ns)]))
    chain = Chain(stages, torch.float32)
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    a = [y.clone() for st in stages for y in st.outs]
    chain.run_launches()
    torch.cuda.synchronize()
    b = [y for st in stages for y in st.outs]
    for u, v in zip(a, b):
        assert oracle.floored_rel_err(out_np(u), out_np(v)) <= 2 * TOL_F32


def test_plan_row_count_mismatch_is_refused():
    """A plan encoded for 2 rows launched as 3: the kernel checks the plan's
    row count before any load and reports status 2, writing nothing."""
    m = 2
    k, n = 1024, 256
    x = workloads.activations(3, 8, 7, 0, m, k)
    (P, S, B), mt = _mat(n, k, 3, 0)
    y = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda:0")
    chain = Chain([Stage(to_gpu_bf16_bits(x), [mt], [y])], torch.float32)
    chain.prepare_chain()
    chain._plan.m = 3
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 2
    assert bool((y == 7.0).all())
    chain._plan.m = 2
    chain._ws.zero_()
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    assert oracle.floored_rel_err(out_np(y), oracle.matmul(x, P, S, B, k)) <= TOL_F32


_STEP_QUANT = {}


def _step_weights(seed, layer, li):
    key = (seed, layer, li.item)
    if key not in _STEP_QUANT:
        w = workloads.weights(seed, workloads.CFG_STEP, layer, li.item, li.n, li.k)
        _STEP_QUANT[key] = oracle.quantize(w)
    return _STEP_QUANT[key]


@pytest.mark.parametrize("m", [4, 16])
def test_small_gemm_step_sampled_layers(m):
    """The small-GEMM step as the benchmark runs it: the temporal step's 224
    packed matrices against m activation rows per stage, in one chain launch
    for m=4 and one q4_gemm_small launch per matrix for m=16. Layers 0, 17 and
    31 are checked against the oracle on weights and activations rebuilt on
    the host."""
    import bench

    seed = 0
    dev = torch.device("cuda:0")
    base = bench.make_temporal_chain(seed, device=dev)
    rows = Chain(bench.make_small_gemm(base, m, seed, dev))
    if m <= 4:
        rows.run_chain()
        rows.run_chain()
    else:
        rows.run_launches()
    torch.cuda.synchronize()
    if m <= 4:
        assert rows.chain_status() == 0
    by_stage = {}
    for li in workloads.temporal_layer():
        by_stage.setdefault(li.stage, []).append(li)
    keys = sorted(by_stage)
    assert len(rows.stages) == workloads.TEMPORAL_LAYERS * len(keys)
    for layer in (0, 17, 31):
        for si, key in enumerate(keys):
            stage = rows.stages[layer * len(keys) + si]
            k = by_stage[key][0].k
            x = workloads.activations(seed, workloads.CFG_SMALL_GEMM, layer, 100 + key, m, k)
            assert np.array_equal(bf16_bits_np(stage.x), x)
            for li, y in zip(by_stage[key], stage.outs):
                P, S, B = _step_weights(seed, layer, li)
                ref = oracle.matmul(x, P, S, B, li.k)
                assert oracle.floored_rel_err(out_np(y), ref) <= TOL_BF16, (m, layer, li.name)
