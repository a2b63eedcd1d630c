"""GPU parity of the packed-embedding gather and stream sum (q4_embed_sum)
against the CPU oracle: the model's 17 streams (a text table of 32000 rows and
16 audio codebook tables of 2048 rows, width 4096), several frames, both
output dtypes; one stream returns the dequantized row bit for bit; tokens
outside a table add nothing; ragged widths."""
import numpy as np
import pytest
import torch

import bit_group_quantized_amd as q4
import oracle
import workloads
from helpers import TOL_BF16, TOL_F32, out_np, upload_quantized

pytestmark = pytest.mark.gpu

_TABLES = {}


def _tables(shapes, seed):
    key = (tuple(shapes), seed)
    if key not in _TABLES:
        ws = workloads.weights_many([(seed, 6, 0, t, rows, dim) for t, (rows, dim) in enumerate(shapes)])
        _TABLES[key] = [oracle.quantize(w) for w in ws]
    host = _TABLES[key]
    return host, [upload_quantized(*h) for h in host]


def _tokens(frames, rows, seed):
    r = np.random.default_rng(seed)
    return np.stack([[r.integers(0, n) for n in rows] for _ in range(frames)]).astype(np.int32)


def _run(tokens, gpu_tables, out_dtype):
    t = torch.from_numpy(tokens).to("cuda:0")
    y = q4.q4_embed_sum(t, gpu_tables, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out_np(y)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("frames", [1, 4, 16])
def test_model_streams_match_oracle(frames, out_dtype):
    shapes = [(workloads.TEXT_VOCAB, workloads.HIDDEN)] + [(workloads.AUDIO_CODEBOOK, workloads.HIDDEN)] * 16
    host, gpu = _tables(shapes, 0)
    tokens = _tokens(frames, [s[0] for s in shapes], seed=frames)
    ref = oracle.embed_sum(tokens, host, workloads.HIDDEN)
    got = _run(tokens, gpu, out_dtype)
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    assert oracle.floored_rel_err(got, ref) <= tol


def test_one_stream_returns_the_row_exactly():
    shapes = [(300, 1024)]
    host, gpu = _tables(shapes, 1)
    _, w_hat = oracle.unpack(*host[0], 1024)
    tokens = np.array([[0], [299], [17], [128]], dtype=np.int32)
    got = _run(tokens, gpu, torch.float32)
    assert np.array_equal(got.astype(np.float32), w_hat[tokens[:, 0]])


def test_tokens_outside_a_table_add_nothing():
    shapes = [(50, 256), (7, 256), (1000, 256)]
    host, gpu = _tables(shapes, 2)
    tokens = np.array([[-1, 3, 999], [50, -5, 0], [-1, 7, 1000], [49, 6, -2147483648]], dtype=np.int32)
    ref = oracle.embed_sum(tokens, host, 256)
    got = _run(tokens, gpu, torch.float32)
    assert not got[2].any() and not ref[2].any()
    assert oracle.floored_rel_err(got, ref) <= TOL_F32


@pytest.mark.parametrize("dim", [32, 96, 2080, 4128])
def test_ragged_widths(dim):
    """Widths whose group count is not a multiple of a block's 64 groups."""
    shapes = [(64, dim)] * 17
    host, gpu = _tables(shapes, 3)
    tokens = _tokens(3, [s[0] for s in shapes], seed=dim)
    ref = oracle.embed_sum(tokens, host, dim)
    got = _run(tokens, gpu, torch.bfloat16)
    assert oracle.floored_rel_err(got, ref) <= TOL_BF16
