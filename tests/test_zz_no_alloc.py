"""The chain entry point that allocates nothing (q4_chain_run_rows_noalloc,
workspace in a device-global array) against the entry point with a caller
workspace (q4_chain_run_rows): two calls in a row on one device, the second on
a smaller chain, each bit-identical to the workspace entry point (dependent
stages included) and, on stages with drawn inputs, within tolerance of the
oracle, with status 0 reported through status_out."""
import ctypes

import numpy as np
import pytest
import torch

import bit_group_quantized_amd as q4
import oracle
import workloads
from bit_group_quantized_amd.step import Q4Matrix, Stage
from helpers import TOL_BF16, out_np, to_gpu_bf16_bits, upload_quantized

pytestmark = pytest.mark.gpu

# (k, [n...], x from the previous stage's first output?)
BIG = [(4096, [4096, 4096, 1000], False), (4096, [11264], True), (11264, [4096], True), (1024, [37], False)]
SMALL = [(1024, [1024], False), (96, [40], False)]


def _build(specs, m, seed):
    dev = torch.device("cuda:0")
    mats, xs, host = [], [], []
    for si, (k, ns, dep) in enumerate(specs):
        x = workloads.activations(seed, 8, 40, si, m, k)
        xs.append(x)
        row = []
        for j, n in enumerate(ns):
            P, S, B = oracle.quantize(workloads.weights(seed, 8, 40, 10 * si + j, n, k))
            host.append((si, j, P, S, B))
            row.append(Q4Matrix(*upload_quantized(P, S, B)))
        mats.append(row)

    def stages():
        out, prev = [], None
        for si, (k, ns, dep) in enumerate(specs):
            shape = (m,) if m > 1 else ()
            outs = [torch.empty(shape + (n,), dtype=torch.bfloat16, device=dev) for n in ns]
            x = prev if dep else to_gpu_bf16_bits(xs[si] if m > 1 else xs[si][0])
            out.append(Stage(x, mats[si], outs))
            prev = outs[0]
        return out

    return stages, xs, host


def _refs(specs, xs, host):
    """Oracle values of the outputs of stages whose x is a drawn input. (A stage
    fed by the previous stage's bf16 output is checked only for bit-identity
    with the workspace entry point: its input is whatever the GPU rounded, and
    the oracle takes no input from the GPU.)"""
    refs = {}
    for si, j, P, S, B in host:
        k, _, dep = specs[si]
        if not dep:
            refs[(si, j)] = oracle.matmul(xs[si], P, S, B, k)
    return refs


@pytest.mark.parametrize("m", [1, 4])
def test_noalloc_matches_workspace_entry_point(m):
    lib = q4.load()
    dev = torch.device("cuda:0")
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    for call, specs in enumerate((BIG, SMALL)):
        make, xs, host = _build(specs, m, seed=call)
        ref_stages, got_stages = make(), make()
        plan_ref = q4.q4_chain_build(ref_stages)
        plan_got = q4.q4_chain_build(got_stages)
        ws = torch.zeros(q4.CHAIN_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev)
        q4.q4_chain_run(plan_ref, ws)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        st = lib.q4_chain_run_rows_noalloc(ctypes.c_void_p(plan_got.device_plan.data_ptr()), m, q4.Q4_OUT_BF16,
                                           ctypes.c_void_p(status.data_ptr()), stream)
        assert st == q4.Q4_OK, q4.q4_status_str(st)
        torch.cuda.synchronize()
        assert int(ws[0].item()) == 0
        assert int(status[0].item()) == 0, f"call {call}: status {int(status[0].item())}"
        status.fill_(-1)
        refs = _refs(specs, xs, host)
        for si, (a, b) in enumerate(zip(ref_stages, got_stages)):
            for j, (ya, yb) in enumerate(zip(a.outs, b.outs)):
                assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), (call, si, j)
                if (si, j) in refs:
                    ref = refs[(si, j)]
                    assert oracle.floored_rel_err(out_np(yb).reshape(ref.shape), ref) <= TOL_BF16, (call, si, j)

