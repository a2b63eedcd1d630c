"""GPU parity of the decoder-layer parts fused into the persistent chain
(RMSNorm of a stage's activation, the SwiGLU gate of a gate/up pair, the
residual sum) against the CPU oracle.

* independent fused stages at the model's widths and at ragged ones, against
  oracle.rmsnorm / oracle.silu_mul / oracle.matmul plus the residual;
* exact checks with selector matrices (each output row picks one input): the
  normalized activation the kernel stages is bit-identical to oracle.rmsnorm,
  and an in-place residual chain of the layer's shape is bit-exact;
* a dependent layer-shaped chain (norm -> q/k/v, o + residual in place,
  norm -> gate/up gated, down + residual in place) with poisoned buffers;
* gate and residual with several activation rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from bit_group_quantized_amd.step import Chain, Q4Matrix, Stage
from helpers import TOL_BF16, TOL_F32, bf16_bits_np, out_np, to_gpu_bf16_bits, upload_quantized

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _mat(n, k, seed, item):
    w = workloads.weights(seed, 9, 0, item, n, k)
    P, S, B = oracle.quantize(w)
    return (P, S, B), Q4Matrix(*upload_quantized(P, S, B))


def _gamma(k, seed):
    r = np.random.default_rng(seed)
    return workloads.bf16_bits_rne((1.0 + 0.25 * r.standard_normal(k)).astype(np.float32))


def _act(k, seed, scale=3.0):
    r = np.random.default_rng(seed)
    return workloads.bf16_bits_rne((scale * r.standard_normal(k)).astype(np.float32))


def _bf16_values(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_independent_fused_stages(out_dtype):
    """Every combination of the fused parts on stages of the model's widths
    and on ragged ones, each stage's inputs its own."""
    specs = [  # (k, [n...], norm, gated, residual)
        (4096, [4096, 4096, 1000], True, False, False),   # attention input: norm -> q, k, v
        (4096, [11264, 11264], True, True, False),        # FFN input: norm -> gate, up, gated
        (11264, [4096], False, False, True),              # down + residual
        (4096, [4096], False, False, True),               # o + residual
        (1024, [2816, 2816], True, True, False),          # the Depformer's widths
        (1024, [1024, 37], True, False, True),            # norm and residual together
        (96, [40], True, False, False),                   # 3 groups: one ragged chunk
        (4128, [70, 70], True, True, True),               # 129 groups, all three parts
        (12288, [64], True, False, False),                # the widest normalized activation
    ]
    stages, checks = [], []
    item = 0
    dev = torch.device("cuda:0")
    for si, (k, ns, norm, gated, res) in enumerate(specs):
        x = _act(k, 100 + si)
        g = _gamma(k, 200 + si) if norm else None
        xin = oracle.rmsnorm(x, g, EPS) if norm else x
        prods, mats = [], []
        for n in ns:
            (P, S, B), m = _mat(n, k, si, item)
            item += 1
            mats.append(m)
            prods.append(oracle.matmul(xin[None, :], P, S, B, k)[0])
        refs = [oracle.silu_mul(prods[0], prods[1])] if gated else prods
        resid = []
        for j, ref in enumerate(refs):
            if res:
                r_vals = np.random.default_rng(300 + 10 * si + j).standard_normal(ref.shape[0]) * 0.5
                r_t = torch.from_numpy(r_vals.astype(np.float32)).to(dev).to(out_dtype)
                resid.append(r_t)
                refs[j] = ref + r_t.double().cpu().numpy()
            else:
                resid.append(None)
        if gated:
            resid.append(None)
        st = Stage(to_gpu_bf16_bits(x), mats, norm=None if g is None else to_gpu_bf16_bits(g), eps=EPS,
                   gated=gated, residuals=resid)
        stages.append(st)
        checks.append((st, refs))
    chain = Chain(stages, out_dtype)
    for _ in range(2):
        chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    for si, (st, refs) in enumerate(checks):
        if st.gated:
            assert st.outs[1] is None
        for j, ref in enumerate(refs):
            err = oracle.floored_rel_err(out_np(st.outs[j]), ref)
            assert err <= tol, (si, j, err)


def _selector_matrix(n, k, pick):
    """Row r: code 1 at input pick[r], 0 elsewhere, scale 1.0 and bias 0.0 in
    every group, so w_hat row r is the unit vector e_pick[r]. Words are written
    from the layout definition (code of input 8j+t in bits [4t, 4t+4) of word j)."""
    packed = np.zeros((n, k // 8), dtype=np.uint32)
    packed[np.arange(n), pick // 8] = (np.uint32(1) << (4 * (pick % 8)).astype(np.uint32))
    scales = np.full((n, k // 32), 0x3F80, dtype=np.uint16)
    biases = np.zeros((n, k // 32), dtype=np.uint16)
    return packed, scales, biases


@pytest.mark.parametrize("k", [4096, 1024, 96, 12288])
def test_normalized_activation_is_bit_exact(k):
    """With a selector matrix the output is the normalized activation itself.
    x holds integers (its sum of squares is exact in any order), so the norm
    factor and every normalized value agree bit for bit with oracle.rmsnorm."""
    r = np.random.default_rng(k)
    x = workloads.bf16_bits_rne(r.integers(-64, 65, size=k).astype(np.float32))
    g = _gamma(k, k + 1)
    pick = np.concatenate([np.arange(k), r.integers(0, k, size=37)])
    P, S, B = _selector_matrix(pick.size, k, pick)
    st = Stage(to_gpu_bf16_bits(x), [Q4Matrix(*upload_quantized(P, S, B))], norm=to_gpu_bf16_bits(g), eps=EPS)
    chain = Chain([st], torch.bfloat16)
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    want = oracle.rmsnorm(x, g, EPS)[pick]
    assert np.array_equal(bf16_bits_np(st.outs[0]), want)


def _layer_chain(h, gammas, sels, poison=True):
    """Stages of one decoder layer on the hidden state h (bf16 [d], updated in
    place by the two residual products): norm -> (q, k, v); o(q) + h -> h;
    norm -> (gate, up) gated -> mid; down(mid) + h -> h."""
    dev = h.device
    d = h.numel()
    mk = lambda n: torch.full((n,), 1.0e4 if poison else 0.0, dtype=torch.bfloat16, device=dev)
    q, kk, v = mk(d), mk(d), mk(d)
    mid = mk(sels["gate"].n)
    stages = [
        Stage(h, [sels["q"], sels["k"], sels["v"]], [q, kk, v], norm=gammas[0], eps=EPS),
        Stage(q, [sels["o"]], [h], residuals=[h]),
        Stage(h, [sels["gate"], sels["up"]], [mid, None], norm=gammas[1], eps=EPS, gated=True),
        Stage(mid, [sels["down"]], [h], residuals=[h]),
    ]
    return stages, (q, kk, v, mid)


def test_dependent_layer_chain():
    """Two layers of the decoder's stage pattern, each stage reading what the
    previous one wrote (the hidden state is updated in place by the residual
    products; intermediate buffers start poisoned). Selector matrices keep the
    norm and residual stages exact; the gated product goes through silu, so
    from there on the check is the floored tolerance."""
    d, f = 4096, 11264
    r = np.random.default_rng(5)
    h0 = workloads.bf16_bits_rne(r.integers(-32, 33, size=d).astype(np.float32))
    layers = []
    for layer in range(2):
        picks = {nm: r.integers(0, kin, size=n) for nm, n, kin in
                 (("q", d, d), ("k", d, d), ("v", d, d), ("o", d, d), ("gate", f, d), ("up", f, d), ("down", d, f))}
        host = {nm: _selector_matrix(p.size, {"down": f}.get(nm, d), p) for nm, p in picks.items()}
        sels = {nm: Q4Matrix(*upload_quantized(*host[nm])) for nm in host}
        gam = [_gamma(d, 40 + 2 * layer), _gamma(d, 41 + 2 * layer)]
        layers.append((picks, sels, gam))
    h = to_gpu_bf16_bits(h0)
    stages, bufs = [], []
    for picks, sels, gam in layers:
        st, b = _layer_chain(h, [to_gpu_bf16_bits(gv) for gv in gam], sels)
        stages += st
        bufs.append(b)
    chain = Chain(stages, torch.bfloat16)
    for rep in range(2):
        h.copy_(to_gpu_bf16_bits(h0))
        for b in bufs:
            for t in b:
                t.fill_(1.0e4)
        chain.run_chain()
        torch.cuda.synchronize()
        assert chain.chain_status() == 0
        # the oracle's chain, layer by layer
        hr = h0.copy()
        for li, (picks, sels, gam) in enumerate(layers):
            xn = oracle.rmsnorm(hr, gam[0], EPS)
            q_ref = xn[picks["q"]]
            if li == 0:
                got_q = bf16_bits_np(bufs[li][0])
                assert np.array_equal(got_q, q_ref), rep
                assert np.array_equal(bf16_bits_np(bufs[li][1]), xn[picks["k"]]), rep
                assert np.array_equal(bf16_bits_np(bufs[li][2]), xn[picks["v"]]), rep
            h1 = oracle.output_bits_bf16(_bf16_values(hr) + _bf16_values(q_ref[picks["o"]]))
            xn2 = oracle.rmsnorm(h1, gam[1], EPS)
            mid = oracle.silu_mul(_bf16_values(xn2[picks["gate"]]), _bf16_values(xn2[picks["up"]]))
            if li == 0:
                assert oracle.floored_rel_err(out_np(bufs[li][3]), mid) <= TOL_BF16, rep
            mid_bits = oracle.output_bits_bf16(mid)
            hr = oracle.output_bits_bf16(_bf16_values(h1) + _bf16_values(mid_bits[picks["down"]]))
        err = oracle.floored_rel_err(out_np(h), _bf16_values(hr))
        assert err <= TOL_BF16, (rep, err)


def test_fused_chain_runs_are_identical():
    """The fused chain is deterministic: two runs give the same bits."""
    k, n = 4096, 11264
    x = _act(k, 7)
    (P, S, B), mg = _mat(n, k, 7, 0)
    (P2, S2, B2), mu = _mat(n, k, 7, 1)
    (P3, S3, B3), md = _mat(k, n, 7, 2)
    xt = to_gpu_bf16_bits(x)
    res = torch.zeros(k, dtype=torch.bfloat16, device=xt.device)
    mid = torch.empty(n, dtype=torch.bfloat16, device=xt.device)
    out = torch.empty(k, dtype=torch.bfloat16, device=xt.device)
    stages = [Stage(xt, [mg, mu], [mid, None], norm=to_gpu_bf16_bits(_gamma(k, 8)), eps=EPS, gated=True),
              Stage(mid, [md], [out], residuals=[res])]
    chain = Chain(stages, torch.bfloat16)
    chain.run_chain()
    torch.cuda.synchronize()
    a = (bf16_bits_np(mid).copy(), bf16_bits_np(out).copy())
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    assert np.array_equal(bf16_bits_np(mid), a[0]) and np.array_equal(bf16_bits_np(out), a[1])


@pytest.mark.parametrize("m", [2, 4])
def test_gate_and_residual_with_rows(m):
    """Several activation rows: the gate and the residual per row."""
    k, n = 4096, 2816
    dev = torch.device("cuda:0")
    x = workloads.activations(3, 9, 2, m, m, k)
    (Pg, Sg, Bg), mg = _mat(n, k, 11, m)
    (Pu, Su, Bu), mu = _mat(n, k, 12, m)
    (Pd, Sd, Bd), md = _mat(k, k, 13, m)
    r_vals = np.random.default_rng(m).standard_normal((m, k)).astype(np.float32)
    res = torch.from_numpy(r_vals).to(dev)
    mid = torch.empty((m, n), dtype=torch.float32, device=dev)
    out = torch.empty((m, k), dtype=torch.float32, device=dev)
    xt = to_gpu_bf16_bits(x).reshape(m, k)
    stages = [Stage(xt, [mg, mu], [mid, None], gated=True), Stage(xt, [md], [out], residuals=[res])]
    chain = Chain(stages, torch.float32)
    chain.run_chain()
    torch.cuda.synchronize()
    assert chain.chain_status() == 0
    ref_mid = oracle.silu_mul(oracle.matmul(x, Pg, Sg, Bg, k), oracle.matmul(x, Pu, Su, Bu, k))
    ref_out = oracle.matmul(x, Pd, Sd, Bd, k) + r_vals.astype(np.float64)
    for v in range(m):
        assert oracle.floored_rel_err(out_np(mid)[v], ref_mid[v]) <= TOL_F32, v
        assert oracle.floored_rel_err(out_np(out)[v], ref_out[v]) <= TOL_F32, v
