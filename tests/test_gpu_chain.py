"""GPU parity of the persistent chain executor against the CPU oracle.

* independent stages of the model's shapes (several matrices per stage, mixed
  k, ragged row counts);
* a dependent chain where each stage's activation IS the previous stage's bf16
  output, with output buffers pre-filled with a poison value so that a stage
  reading its input before the previous stage finished cannot pass;
* the full 32-layer temporal step exactly as the benchmark runs it, with the
  packed weights (bit-exact) and outputs of sampled layers checked.
"""
import numpy as np
import pytest
import torch

import bit_group_quantized_amd as q4
import oracle
import workloads
from bit_group_quantized_amd.step import Chain, Q4Matrix, Stage
from helpers import TOL_BF16, TOL_F32, bf16_bits_np, out_np, packed_np, to_gpu_bf16_bits, upload_quantized

pytestmark = pytest.mark.gpu


def _mat(n, k, seed, item):
    w = workloads.weights(seed, 8, 0, item, n, k)
    P, S, B = oracle.quantize(w)
    return (P, S, B), Q4Matrix(*upload_quantized(P, S, B))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_independent_stages(out_dtype):
    specs = [  # (k, [n...])
        (4096, [4096, 4096, 1000]),
        (11264, [4096]),
        (1024, [1024, 37]),
        (4096, [11264, 11264]),
        (2816, [1024]),
        (256, [300]),    # 8 groups: one chunk, half of its lanes past the row end
        (6400, [128]),   # 200 groups: 13 chunks, the last one ragged
        (96, [40]),      # 3 groups
        (4128, [70]),    # 129 groups: an odd group count
        (11264, [37]),   # 10 units: blocks with one unit cut into pieces of 22 chunks
        (12288, [64]),   # the widest activation the executor stages
    ]
    stages, refs = [], []
    item = 0
    for si, (k, ns) in enumerate(specs):
        x = workloads.activations(si, 8, 1, si, 1, k)
        mats = []
        for n in ns:
            (P, S, B), m = _mat(n, k, si, item)
            item += 1
            mats.append(m)
            refs.append(oracle.matmul(x, P, S, B, k)[0])
        stages.append(Stage(to_gpu_bf16_bits(x[0]), mats))
    chain = Chain(stages, out_dtype)
    for _ in range(2):
        chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    outs = [y for st in stages for y in st.outs]
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    for y, ref in zip(outs, refs):
        assert oracle.floored_rel_err(out_np(y), ref) <= tol


def _selector_matrix(n, k, pick):
    """Stored Q4 matrix whose row r has code 1 at input pick[r] and 0 elsewhere,
    scale 1.0 and bias 0.0 in every group, so w_hat row r is the unit vector
    e_pick[r]. Words are written from the layout definition (code of input
    8j+t in bits [4t, 4t+4) of word j)."""
    packed = np.zeros((n, k // 8), dtype=np.uint32)
    packed[np.arange(n), pick // 8] = (np.uint32(1) << (4 * (pick % 8)).astype(np.uint32))
    scales = np.full((n, k // 32), 0x3F80, dtype=np.uint16)
    biases = np.zeros((n, k // 32), dtype=np.uint16)
    return packed, scales, biases


def test_dependent_chain_reads_previous_outputs():
    """Each stage's activation is the previous stage's bf16 output buffer. Row r of
    stage s selects input pick_s[r], so every output is exactly an earlier
    integer input and the whole chain is bit-exact against the oracle; all
    output buffers start poisoned (1e4), so a stage that read its input before
    the previous stage finished cannot match."""
    shapes = [(4096, 4096)] * 5 + [(11264, 4096), (4096, 11264), (4096, 4096), (1024, 4096), (4096, 1024)]
    r = np.random.default_rng(11)
    x0 = workloads.bf16_bits_rne(r.integers(-64, 65, size=shapes[0][1]).astype(np.float32))
    host, stages = [], []
    x = to_gpu_bf16_bits(x0)
    for (n, k) in shapes:
        P, S, B = _selector_matrix(n, k, r.integers(0, k, size=n))
        host.append((P, S, B))
        y = torch.full((n,), 1.0e4, dtype=torch.bfloat16, device=x.device)  # poison
        stages.append(Stage(x, [Q4Matrix(*upload_quantized(P, S, B))], [y]))
        x = y
    chain = Chain(stages, torch.bfloat16)
    for rep in range(3):
        for st in stages:
            st.outs[0].fill_(1.0e4)
        chain.run_chain()
        torch.cuda.synchronize()
        assert chain.chain_status() == 0
        xr = x0[None, :]
        for i, (n, k) in enumerate(shapes):
            P, S, B = host[i]
            y_ref = oracle.output_bits_bf16(oracle.matmul(xr, P, S, B, k)[0])
            assert np.array_equal(bf16_bits_np(stages[i].outs[0]), y_ref), (rep, i)
            xr = y_ref[None, :]


def test_interleaved_chains_barrier_every_other_stage():
    """Two dependent chains interleaved: stage s reads the output of stage
    s - 2, so the encoder puts a grid barrier before every even stage from 2
    on and none before the odd ones; the outputs stored in a stretch without a
    barrier (stage s - 2 before stage s - 1) must still be complete when the
    next barrier opens stage s. Selector matrices make the result bit-exact;
    outputs start poisoned."""
    shapes = [(4096, 4096), (11264, 4096), (4096, 4096), (4096, 11264), (1024, 4096), (4096, 4096),
              (4096, 1024), (4096, 4096), (4096, 4096), (1024, 4096)]
    r = np.random.default_rng(12)
    x0 = [workloads.bf16_bits_rne(r.integers(-64, 65, size=shapes[c][1]).astype(np.float32)) for c in range(2)]
    host, stages = [], []
    xs = [to_gpu_bf16_bits(x0[0]), to_gpu_bf16_bits(x0[1])]
    for s, (n, k) in enumerate(shapes):
        P, S, B = _selector_matrix(n, k, r.integers(0, k, size=n))
        host.append((P, S, B))
        y = torch.full((n,), 1.0e4, dtype=torch.bfloat16, device=xs[0].device)  # poison
        stages.append(Stage(xs[s % 2], [Q4Matrix(*upload_quantized(P, S, B))], [y]))
        xs[s % 2] = y
    chain = Chain(stages, torch.bfloat16)
    chain.run_chain()
    torch.cuda.synchronize()
    rec = chain._plan.device_plan.cpu().numpy()
    no_barrier = [int(rec[64 + 64 * s + 52]) for s in range(len(shapes))]  # the stage records' flag word
    assert no_barrier == [0, 1] * (len(shapes) // 2)
    for rep in range(3):
        for st in stages:
            st.outs[0].fill_(1.0e4)
        chain.run_chain()
        torch.cuda.synchronize()
        assert chain.chain_status() == 0
        xr = [x0[0][None, :], x0[1][None, :]]
        for i, (n, k) in enumerate(shapes):
            P, S, B = host[i]
            y_ref = oracle.output_bits_bf16(oracle.matmul(xr[i % 2], P, S, B, k)[0])
            assert np.array_equal(bf16_bits_np(stages[i].outs[0]), y_ref), (rep, i)
            xr[i % 2] = y_ref[None, :]


def test_chain_matches_per_call_launches():
    """The chain and one q4_gemv launch per matrix compute the same products."""
    specs = [(4096, [4096, 4096]), (11264, [4096]), (4096, [11264])]
    stages = []
    for si, (k, ns) in enumerate(specs):
        x = workloads.activations(si, 8, 3, si, 1, k)
        stages.append(Stage(to_gpu_bf16_bits(x[0]), [_mat(n, k, 70 + si, j)[1] for j, n in enumerate(ns)]))
    chain = Chain(stages, torch.float32)
    chain.run_chain()
    torch.cuda.synchronize()
    a = [y.clone() for st in stages for y in st.outs]
    chain.run_launches()
    torch.cuda.synchronize()
    b = [y for st in stages for y in st.outs]
    for u, v in zip(a, b):
        assert oracle.floored_rel_err(out_np(u), out_np(v)) <= 2 * TOL_F32


def _outputs_bits(chain):
    return [y.view(torch.int16).clone() for st in chain.stages for y in st.outs]


def _same_bits(a, b):
    return all(torch.equal(u, v) for u, v in zip(a, b))


@pytest.mark.timeout(600)
def test_full_temporal_step_every_layer():
    """The 32-layer step as the benchmark builds and runs it (seeded weights
    packed by q4_pack, bf16 outputs, one persistent launch). Every layer is
    rebuilt on the host: its packed weights compared bit for bit and every
    output against the oracle. A second launch gives bit-identical outputs."""
    import bench

    seed = 0
    chain = bench.make_temporal_chain(seed)
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    first = _outputs_bits(chain)
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    assert _same_bits(first, _outputs_bits(chain)), "a second launch changed the outputs"
    lin = workloads.temporal_layer()
    stages_per_layer = 4
    assert len(chain.stages) == workloads.TEMPORAL_LAYERS * stages_per_layer
    by_stage = {}
    for li in lin:
        by_stage.setdefault(li.stage, []).append(li)
    for layer in range(workloads.TEMPORAL_LAYERS):
        st0 = layer * stages_per_layer
        ws = dict(zip([li.name for li in lin],
                      workloads.weights_many([(seed, workloads.CFG_STEP, layer, li.item, li.n, li.k) for li in lin])))
        for si, st in enumerate(sorted(by_stage)):
            stage = chain.stages[st0 + si]
            x = workloads.activations(seed, workloads.CFG_STEP, layer, 100 + st, 1, by_stage[st][0].k)
            assert np.array_equal(bf16_bits_np(stage.x), x[0])
            for li, m, y in zip(by_stage[st], stage.mats, stage.outs):
                P, S, B = oracle.quantize(ws[li.name])
                assert np.array_equal(packed_np(m.packed), P)
                assert np.array_equal(bf16_bits_np(m.scales), S)
                assert np.array_equal(bf16_bits_np(m.biases), B)
                ref = oracle.matmul(x, P, S, B, li.k)[0]
                assert oracle.floored_rel_err(out_np(y), ref) <= TOL_BF16, (layer, li.name)
        del ws


@pytest.mark.timeout(600)
def test_depformer_frame_chain_every_step():
    """One Depformer frame as the benchmark runs it: 16 codebook steps x 6
    layers x 4 stages in one persistent launch, every matrix the step's row
    slice of its stacked packed tensor. Every layer is rebuilt on the host (the
    stacked weights compared bit for bit) and every output of every codebook
    step checked against the oracle on the step's rows. A second launch gives
    bit-identical outputs."""
    import bench

    seed = 0
    dev = torch.device("cuda:0")
    mats = bench.make_depformer(seed, dev)
    chain = bench.make_depformer_frame(mats, seed, device=dev)
    assert len(chain.stages) == workloads.DEP_STEPS * workloads.DEP_LAYERS * 4
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    first = _outputs_bits(chain)
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    assert _same_bits(first, _outputs_bits(chain)), "a second launch changed the outputs"
    lin = workloads.depformer_layer()
    by_stage = {}
    for li in lin:
        by_stage.setdefault(li.stage, []).append(li)
    for layer in range(workloads.DEP_LAYERS):
        quant = {}
        for li in lin:
            w = workloads.weights(seed, workloads.CFG_DEPFORMER, layer, li.item, workloads.DEP_STEPS * li.n, li.k)
            quant[li.name] = oracle.quantize(w)
            m = mats[(layer, li.name)]
            assert np.array_equal(packed_np(m.packed), quant[li.name][0])
            assert np.array_equal(bf16_bits_np(m.scales), quant[li.name][1])
            assert np.array_equal(bf16_bits_np(m.biases), quant[li.name][2])
        for step in range(workloads.DEP_STEPS):
            for si, st in enumerate(sorted(by_stage)):
                stage = chain.stages[(step * workloads.DEP_LAYERS + layer) * 4 + si]
                k = by_stage[st][0].k
                x = workloads.activations(seed, workloads.CFG_DEPFORMER, layer, 1000 + 4 * step + st, 1, k)
                assert np.array_equal(bf16_bits_np(stage.x), x[0])
                for li, y in zip(by_stage[st], stage.outs):
                    P, S, B = quant[li.name]
                    rows = slice(step * li.n, (step + 1) * li.n)
                    ref = oracle.matmul(x, P[rows], S[rows], B[rows], k)[0]
                    assert oracle.floored_rel_err(out_np(y), ref) <= TOL_BF16, (layer, step, li.name)
