"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against something the pages or the mathematics fix:
hand-worked packed words, exactly representable affine groups, the
nearest-level property of the quantizer, the additive-noise law of uniform
rounding, the pages' sizes and validation gates, closed forms of the product
(one-hot input, constant codes), exact rational brute force on tiny shapes and a
library float64 product. None of them calls the HIP library.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16_exact(v: float) -> bool:
    """True when v is exactly a bf16 value (low 16 bits of its fp32 are zero)."""
    u = np.array([v], dtype=np.float32).view(np.uint32)[0]
    return float(np.float32(v)) == v and (u & 0xFFFF) == 0


def affine_group(a: float, s0: float, codes) -> np.ndarray:
    w = np.array([a + s0 * c for c in codes], dtype=np.float64)
    w32 = w.astype(np.float32)
    assert np.all(w32.astype(np.float64) == w), "group must be exact in fp32"
    return w32


# ---------------------------------------------------------------- layout

def test_hand_worked_words_roundtrip_through_quantizer():
    """Exact-affine groups whose codes spell each hand-worked word."""
    lines = [ln.split() for ln in open(os.path.join(GOLD, "pack_words.txt")) if ln.strip() and not ln.startswith("#")]
    for parts in lines:
        codes = [int(c) for c in parts[:8]]
        word = int(parts[8], 16)
        # Pad the group so that it holds both 0 and 15: then min = a, max = a + 15*s0
        # and the stored scale/bias are exactly s0, a.
        group_codes = codes + [0, 15] + [7] * 22
        w = affine_group(-1.5, 0.25, group_codes)[None, :]
        packed, scales, biases = oracle.quantize(w)
        assert packed[0, 0] == word, (codes, hex(packed[0, 0]), hex(word))
        assert oracle.bf16_value(scales)[0, 0] == 0.25
        assert oracle.bf16_value(biases)[0, 0] == -1.5


def test_hand_worked_words_unpack():
    """Unpack of the hand-worked words yields their codes (independent of the quantizer)."""
    lines = [ln.split() for ln in open(os.path.join(GOLD, "pack_words.txt")) if ln.strip() and not ln.startswith("#")]
    for parts in lines:
        codes = [int(c) for c in parts[:8]]
        word = int(parts[8], 16)
        packed = np.array([[word, 0, 0, 0]], dtype=np.uint32)
        one = np.array([[0x3F80]], dtype=np.uint16)   # scale 1.0
        zero = np.array([[0x0000]], dtype=np.uint16)  # bias 0.0
        q, w_hat = oracle.unpack(packed, one, zero, 32)
        assert list(q[0, :8]) == codes
        assert list(w_hat[0, :8]) == [float(c) for c in codes]
        assert not q[0, 8:].any()


def test_single_nibble_positions():
    """A code v at position t of a word lands in bits [4t, 4t+4)."""
    for t in range(8):
        for v in range(16):
            codes = [0] * 32
            codes[8 + t] = v        # second word of the group
            codes[0] = 0
            codes[31] = 15
            w = affine_group(2.0, 0.5, codes)[None, :]
            packed, _, _ = oracle.quantize(w)
            assert packed[0, 1] == (v << (4 * t))


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("seed", range(6))
def test_exact_affine_groups_are_reproduced_exactly(seed):
    """w = a + s0*c with bf16-exact a, s0 and codes spanning 0..15: the stored
    scale and bias are s0 and a, the codes are c and the round trip is exact."""
    r = np.random.default_rng(seed)
    rows, groups = 5, 6
    w = np.empty((rows, groups * 32), dtype=np.float32)
    codes = np.empty((rows, groups * 32), dtype=np.uint8)
    sc = np.empty((rows, groups)); bi = np.empty((rows, groups))
    for i in range(rows):
        for g in range(groups):
            s0 = float(2.0 ** r.integers(-8, 3)) * float(r.choice([1.0, 1.25, 1.5, 1.75]))
            a = float(r.integers(-64, 64)) * float(2.0 ** r.integers(-10, 2))
            assert bf16_exact(s0) and bf16_exact(a)
            c = r.integers(0, 16, size=32)
            c[r.integers(0, 32)] = 0
            c[(r.integers(1, 32) + 0) % 32] = 15
            if c.min() != 0:
                c[np.argmin(c)] = 0
            if c.max() != 15:
                c[np.argmax(c)] = 15
            w[i, g * 32:(g + 1) * 32] = affine_group(a, s0, c)
            codes[i, g * 32:(g + 1) * 32] = c
            sc[i, g] = s0; bi[i, g] = a
    packed, scales, biases = oracle.quantize(w)
    q, w_hat = oracle.unpack(packed, scales, biases, w.shape[1])
    assert np.array_equal(q, codes)
    assert np.array_equal(oracle.bf16_value(scales), sc.astype(np.float32))
    assert np.array_equal(oracle.bf16_value(biases), bi.astype(np.float32))
    assert np.array_equal(w_hat, w)


def _gaussian(n, k, seed=0):
    return workloads.weights(seed, 1, 0, 0, n, k)


def test_codes_pick_the_nearest_stored_level():
    """Each code selects the level s'*q + b' (q in 0..15, stored bf16 s', b')
    nearest to the weight, up to rounding of the fp32 quotient at exact ties."""
    w = _gaussian(256, 1024, seed=3)
    packed, scales, biases = oracle.quantize(w)
    q, _ = oracle.unpack(packed, scales, biases, w.shape[1])
    s = np.repeat(oracle.bf16_value(scales).astype(np.float64), 32, axis=1)
    b = np.repeat(oracle.bf16_value(biases).astype(np.float64), 32, axis=1)
    levels = b[..., None] + s[..., None] * np.arange(16, dtype=np.float64)  # exact in f64
    dist = np.abs(w.astype(np.float64)[..., None] - levels)
    chosen = np.take_along_axis(dist, q[..., None].astype(np.int64), axis=-1)[..., 0]
    best = dist.min(axis=-1)
    # slack: a few ulps of the quotient, expressed in weight units
    assert np.all(chosen - best <= 4 * 2.0 ** -23 * (np.abs(w) + 16 * s)), float((chosen - best).max())
    # and the reading matters: computing codes from the unrounded fp32 scale and
    # min (instead of the stored bf16 values) does pick a non-nearest level for
    # a measurable fraction of codes, so this pin separates the two readings.
    g = w.reshape(w.shape[0], -1, 32)
    mn = g.min(-1, keepdims=True); mx = g.max(-1, keepdims=True)
    s32 = ((mx - mn) / np.float32(15)).astype(np.float32)
    alt = np.clip(np.rint((g - mn) / s32), 0, 15).reshape(q.shape).astype(np.int64)
    alt_d = np.take_along_axis(dist, alt[..., None], axis=-1)[..., 0]
    assert np.mean(alt_d - best > 1e-9 * s) > 1e-3


def test_roundtrip_error_bound():
    """|w - w_hat| <= s'/2 for interior elements, and in general
    <= s'/2 + |b' - min| + 15|s' - s| (the bf16 rounding of the stored scale
    and bias can push an end element outside the level grid)."""
    w = _gaussian(512, 2048, seed=5).astype(np.float32)
    packed, scales, biases = oracle.quantize(w)
    _, w_hat = oracle.unpack(packed, scales, biases, w.shape[1])
    err = np.abs(w.astype(np.float64) - w_hat).reshape(w.shape[0], -1, 32)
    s_st = oracle.bf16_value(scales).astype(np.float64)[..., None]
    b_st = oracle.bf16_value(biases).astype(np.float64)[..., None]
    g = w.reshape(w.shape[0], -1, 32).astype(np.float64)
    mn = g.min(-1, keepdims=True); mx = g.max(-1, keepdims=True)
    s_exact = (mx - mn) / 15.0
    ulp = 2.0 ** -22 * np.abs(g)
    bound = s_st / 2 + np.abs(b_st - mn) + 15 * np.abs(s_st - s_exact) + ulp
    assert np.all(err <= bound)
    interior = (g > b_st) & (g < b_st + 15 * s_st)
    assert np.all(np.where(interior, err - (s_st / 2 + ulp), -1.0) <= 0)
    # the ratio |min|/s' stays small for these weights, far inside the range
    # where the end elements also satisfy the plain half-step bound
    assert float((np.abs(mn) / s_st).max()) < 50


def test_uniform_rounding_noise_law():
    """Rounding to a uniform grid leaves interior errors ~ U(-D/2, D/2), so their
    mean square is D^2/12 (D = stored scale). Truncation would give D^2/3, a
    wrong grid origin or step would shift it; a 2% band separates them."""
    w = _gaussian(1024, 4096, seed=7)
    packed, scales, biases = oracle.quantize(w)
    _, w_hat = oracle.unpack(packed, scales, biases, w.shape[1])
    e = (w.astype(np.float64) - w_hat).reshape(w.shape[0], -1, 32)
    g = w.reshape(w.shape[0], -1, 32)
    s = oracle.bf16_value(scales).astype(np.float64)[..., None]
    b = oracle.bf16_value(biases).astype(np.float64)[..., None]
    interior = (g > b + s / 2) & (g < b + 14.5 * s)
    ratio = float((e[interior] ** 2).sum() / (np.broadcast_to(s * s / 12, e.shape)[interior]).sum())
    assert 0.98 < ratio < 1.02, ratio
    mean_signed = float((e[interior] / np.broadcast_to(s, e.shape)[interior]).mean())
    assert abs(mean_signed) < 2e-3  # rounding is unbiased


def test_weight_error_statistics_pass_the_pages_gates():
    """Normalized RMSE and cosine against the unquantized weights, the two
    statistics the model card's validation table reports, on the 4096x4096
    synthetic matrix: both pass the card's gates, and the Gaussian value sits
    below the card's real-weight mean (real weights have heavier tails)."""
    gates = json.load(open(os.path.join(GOLD, "validation_gates.json")))
    w = workloads.weights(0, workloads.CFG_GEMV, 0, 0, 4096, 4096)
    packed, scales, biases = oracle.quantize(w)
    _, w_hat = oracle.unpack(packed, scales, biases, w.shape[1])
    wd = w.astype(np.float64); hd = w_hat.astype(np.float64)
    nrmse = np.linalg.norm(wd - hd) / np.linalg.norm(wd)
    cos = float((wd * hd).sum() / (np.linalg.norm(wd) * np.linalg.norm(hd)))
    assert nrmse <= gates["max_normalized_rmse_gate"]
    assert cos >= gates["min_cosine_gate"]
    assert nrmse < gates["printed_mean_normalized_rmse"]
    # Expected value from the noise law: per group MSE ~ (30/32) * D^2 / 12 with
    # D = range/15; E[range^2] of 32 standard normals by quadrature of the
    # range distribution (independent of the quantizer).
    from scipy import integrate, stats
    n = 32
    f = lambda r, x: n * (n - 1) * stats.norm.pdf(x) * stats.norm.pdf(x + r) * \
        (stats.norm.cdf(x + r) - stats.norm.cdf(x)) ** (n - 2)
    er2, _ = integrate.dblquad(lambda x, r: r * r * f(r, x), 0, 12, -8, 8)
    expected = np.sqrt((30 / 32) * er2 / 225 / 12)
    assert abs(nrmse / expected - 1) < 0.03, (nrmse, expected)
    # additive-noise model: cos = 1/sqrt(1 + nrmse^2) (error uncorrelated with W)
    assert abs(cos - 1 / np.sqrt(1 + nrmse ** 2)) < 2e-4


def test_degenerate_groups():
    """Constant group: zero stored scale, codes 0, bias = bf16(value); a range
    so small that the scale rounds to bf16 zero behaves the same."""
    w = np.zeros((3, 64), dtype=np.float32)
    w[0, :32] = 0.7
    w[0, 32:] = -3.0e-3
    w[1, :32] = 0.0
    w[1, 32:] = np.float32(1e-40)
    w[1, 40] = 0.0
    w[2, :] = 5.0
    packed, scales, biases = oracle.quantize(w)
    q, w_hat = oracle.unpack(packed, scales, biases, 64)
    assert not q.any()
    assert not scales.any()
    assert np.array_equal(biases, oracle.bf16_round(w.reshape(3, 2, 32).min(axis=-1)))
    assert w_hat[0, 0] == oracle.bf16_value(oracle.bf16_round(np.float32(0.7)))
    # 0.7 is not bf16-exact: the round-trip error is the bf16 rounding of the
    # bias, within 2^-9 relative
    assert abs(w_hat[0, 0] - 0.7) <= 0.7 * 2 ** -9


def test_bf16_rounding_hand_values_and_library():
    lines = [ln.split() for ln in open(os.path.join(GOLD, "bf16_rounding.txt")) if ln.strip() and not ln.startswith("#")]
    vals = np.array([float.fromhex(a) if "0x" in a else float(a) for a, _ in lines], dtype=np.float32)
    want = np.array([int(b, 16) for _, b in lines], dtype=np.uint16)
    assert np.array_equal(oracle.bf16_round(vals), want)
    import torch
    r = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * np.float32(10.0) ** \
        np.random.default_rng(1).integers(-30, 30, 100000).astype(np.float32)
    lib = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(r), lib)


def test_size_closed_form_matches_pages():
    """4 bits per weight plus a bf16 scale and bias per 32 weights = 5 bits per
    weight; with the card's parameter count this gives the card's packed size,
    and 16 bits per weight gives its BF16 source size."""
    rel = json.load(open(os.path.join(GOLD, "release_sizes.json")))
    p = rel["parameters"]
    assert round(p * 2 / 2 ** 30, 2) == rel["source_weights_gib"]
    assert round(p * 5 / 8 / 2 ** 30, 2) == rel["packed_language_model_gib"]
    n, k = 64, 256
    packed, scales, biases = oracle.quantize(_gaussian(n, k))
    assert packed.nbytes + scales.nbytes + biases.nbytes == n * k * 5 // 8


# ---------------------------------------------------------------- product

def _quantized(n, k, seed):
    w = _gaussian(n, k, seed)
    return oracle.quantize(w)


def test_one_hot_input_selects_a_column():
    n, k = 48, 256
    packed, scales, biases = _quantized(n, k, 11)
    _, w_hat = oracle.unpack(packed, scales, biases, k)
    for j in (0, 1, 7, 8, 31, 32, 100, 255):
        x = np.zeros(k, dtype=np.uint16)
        x[j] = 0x3F80  # 1.0
        y = oracle.matmul(x, packed, scales, biases, k)
        assert np.array_equal(y, w_hat[:, j].astype(np.float64))
        x[j] = 0xC000  # -2.0
        y = oracle.matmul(x, packed, scales, biases, k)
        assert np.array_equal(y, -2.0 * w_hat[:, j].astype(np.float64))


def test_constant_code_groups_closed_form():
    """All codes of a group equal c: y = sum_g (s_g*c_g + b_g) * X_g with X_g the
    group sum of x, computed here in exact rationals."""
    r = np.random.default_rng(2)
    n, k = 6, 160
    G = k // 32
    c = r.integers(0, 16, size=(n, G))
    packed = np.zeros((n, k // 8), dtype=np.uint32)
    for i in range(n):
        for g in range(G):
            word = 0
            for t in range(8):
                word |= int(c[i, g]) << (4 * t)
            packed[i, 4 * g:4 * g + 4] = word
    scales = oracle.bf16_round(r.uniform(1e-3, 1e-1, size=(n, G)).astype(np.float32))
    biases = oracle.bf16_round(r.uniform(-1, 1, size=(n, G)).astype(np.float32))
    x = workloads.activations(0, 1, 0, 0, 2, k)
    y = oracle.matmul(x, packed, scales, biases, k)
    xs = oracle.bf16_value(x)
    for m in range(2):
        for i in range(n):
            tot = Fraction(0)
            for g in range(G):
                Xg = sum(Fraction(float(v)) for v in xs[m, 32 * g:32 * g + 32])
                w_g = Fraction(float(oracle.bf16_value(scales[i, g]))) * int(c[i, g]) + \
                    Fraction(float(oracle.bf16_value(biases[i, g])))
                # w_hat is the fp32 rounding of s*c + b
                w_g = Fraction(float(np.float32(float(w_g))))
                tot += w_g * Xg
            assert abs(Fraction(y[m, i]) - tot) <= abs(tot) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


@pytest.mark.parametrize("k", [32, 64, 96, 256])
def test_bruteforce_exact_rationals(k):
    """Tiny shapes: decode every nibble of the words with Python integers,
    rebuild each weight and the dot product in exact rationals."""
    n = 5
    packed, scales, biases = _quantized(n, k, 100 + k)
    x = workloads.activations(3, 1, 0, k, 3, k)
    y = oracle.matmul(x, packed, scales, biases, k)
    xs = [[Fraction(float(v)) for v in row] for row in oracle.bf16_value(x)]
    for i in range(n):
        row_bytes = packed[i].astype("<u4").tobytes()
        codes = []
        for byte in row_bytes:           # little-endian: byte b holds codes 2b, 2b+1
            codes.append(byte & 0xF)
            codes.append(byte >> 4)
        assert len(codes) == k
        w = []
        for j, cde in enumerate(codes):
            s = Fraction(float(oracle.bf16_value(scales[i, j // 32])))
            b = Fraction(float(oracle.bf16_value(biases[i, j // 32])))
            w.append(Fraction(float(np.float32(float(s * cde + b)))))
        for m in range(3):
            exact = sum(wj * xj for wj, xj in zip(w, xs[m]))
            mag = sum(abs(wj * xj) for wj, xj in zip(w, xs[m]))
            assert abs(Fraction(y[m, i]) - exact) <= mag * k * Fraction(1, 2 ** 52)


def test_matches_library_float64_product():
    n, k = 300, 1024
    packed, scales, biases = _quantized(n, k, 21)
    _, w_hat = oracle.unpack(packed, scales, biases, k)
    x = workloads.activations(0, 1, 0, 0, 4, k)
    y = oracle.matmul(x, packed, scales, biases, k)
    ref = oracle.bf16_value(x).astype(np.float64) @ w_hat.astype(np.float64).T
    mag = np.abs(oracle.bf16_value(x).astype(np.float64)) @ np.abs(w_hat.astype(np.float64)).T
    assert np.all(np.abs(y - ref) <= mag * 1e-13)


# ---------------------------------------------------------------- MultiLinear

def test_multilinear_slices_rows_of_all_three_arrays():
    """Step s reads rows [s*out, (s+1)*out) of codes, scales and biases; rows are
    quantized independently, so packing the stack and slicing equals packing
    the slice; and each step's block is the one used."""
    steps, out, k = 4, 24, 96
    blocks = [(_gaussian(out, k, seed=40 + s) * np.float32(1 + s)) for s in range(steps)]
    W = np.concatenate(blocks, axis=0)
    P, S, B = oracle.quantize(W)
    x = workloads.activations(0, 4, 0, 0, 2, k)
    for s in range(steps):
        p, sc, bi = oracle.quantize(blocks[s])
        assert np.array_equal(P[s * out:(s + 1) * out], p)
        assert np.array_equal(S[s * out:(s + 1) * out], sc)
        assert np.array_equal(B[s * out:(s + 1) * out], bi)
        y_step = oracle.multilinear_step(x, P, S, B, steps, out, k, s)
        y_ref = oracle.matmul(x, p, sc, bi, k)
        assert np.array_equal(y_step, y_ref)
    # one-hot blocks identify the step: block s holds the constant s+1
    Wc = np.concatenate([np.full((out, k), s + 1, dtype=np.float32) for s in range(steps)])
    Pc, Sc, Bc = oracle.quantize(Wc)
    ones = np.full((1, k), 0x3F80, dtype=np.uint16)
    for s in range(steps):
        y = oracle.multilinear_step(ones, Pc, Sc, Bc, steps, out, k, s)
        assert np.all(y == (s + 1) * k)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 33), dtype=np.float32))
    w = np.zeros((2, 32), dtype=np.float32)
    w[1, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize(w)
    p, s, b = oracle.quantize(np.zeros((4, 32), dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.multilinear_step(np.zeros((1, 32), np.uint16), p, s, b, 2, 2, 32, 2)
    x = np.zeros((1, 32), dtype=np.uint16)
    x[0, 0] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        oracle.matmul(x, p, s, b, 32)


# ---------------------------------------------------------------- tolerance yardstick
# floored_rel_err is the measure every parity tolerance is stated in: per output
# row, max_n |got_n - ref_n| / max(|ref_n|, 1e-3 * rms(ref row)). Each case below is
# worked by hand and fails for one plausible slip in it.

def test_floored_rel_err_exact_match_is_zero():
    ref = np.array([[1.5, -2.25, 0.0, 3.0]])
    assert oracle.floored_rel_err(ref.copy(), ref) == 0.0


def test_floored_rel_err_divides_each_element_by_its_own_magnitude():
    # |1.01 - 1| / 1 = 0.01; dividing by max|ref| (100) instead would give 1e-4
    got = np.array([1.01, 100.0])
    ref = np.array([1.0, 100.0])
    assert oracle.floored_rel_err(got, ref) == pytest.approx(0.01, rel=1e-9)


def test_floored_rel_err_floor_applies_near_zero():
    # rms of [1e-9, 2, -2] is sqrt(8/3) (the 1e-18 term is below double precision
    # there), floor = 1e-3 * 1.6329931618554521; an error of 1e-5 at the
    # near-zero output scores 1e-5 / 1.6329931618554521e-3 = 0.0061237243569579
    # (without the floor it would be 1e4)
    ref = np.array([1e-9, 2.0, -2.0])
    got = ref + np.array([1e-5, 0.0, 0.0])
    assert oracle.floored_rel_err(got, ref) == pytest.approx(0.0061237243569579, rel=1e-9)


def test_floored_rel_err_rms_is_per_output_row():
    # row 1's rms is sqrt(2e-6 / 3) = 8.16496580927726e-4, so its floor is
    # 8.16496580927726e-7 and an error of 1e-8 at its zero output scores
    # 0.012247448713915890; an rms over both rows (~816) would score ~1.2e-11
    ref = np.array([[1000.0, -1000.0, 500.0], [1e-3, -1e-3, 0.0]])
    got = ref.copy()
    got[1, 2] = 1e-8
    assert oracle.floored_rel_err(got, ref) == pytest.approx(0.01224744871391589, rel=1e-9)
    # the worst row decides: an error of 1% in row 0 on top
    got[0, 0] = 1010.0
    assert oracle.floored_rel_err(got, ref) == pytest.approx(0.01224744871391589, rel=1e-9)
    got[0, 0] = 1020.0
    assert oracle.floored_rel_err(got, ref) == pytest.approx(0.02, rel=1e-9)


def test_floored_rel_err_non_finite_output_fails():
    ref = np.array([[1.0, 2.0, 3.0]])
    assert oracle.floored_rel_err(np.full((1, 3), np.nan), ref) == float("inf")
    assert oracle.floored_rel_err(np.array([[1.0, np.inf, 3.0]]), ref) == float("inf")
    assert oracle.floored_rel_err(np.array([[1.0, 2.0, -np.inf]]), ref) == float("inf")
    with pytest.raises(ValueError):
        oracle.floored_rel_err(np.zeros((1, 2)), ref)


# ---------------------------------------------------------------- embedding gather + stream sum
# (the blog translation's pipeline figure: 17 token streams, text + 8 user + 8
# assistant audio, summed into the temporal step's input; the model card's
# introduction: embeddings stay packed)

def _affine_table(rows, dim, a, s0, seed):
    """A table whose every group is exactly affine: w = a + s0 * code, codes
    drawn per element with 0 and 15 in every group (so the quantizer stores
    exactly s0 and a). Returns (weights fp32, codes int)."""
    r = np.random.default_rng(seed)
    codes = r.integers(0, 16, size=(rows, dim))
    codes[:, 0::32] = 0
    codes[:, 1::32] = 15
    w = (np.float64(a) + np.float64(s0) * codes).astype(np.float32)
    assert np.all(w.astype(np.float64) == np.float64(a) + np.float64(s0) * codes)
    return w, codes


def test_embed_single_stream_selects_the_dequantized_row():
    dim = 256
    w = _gaussian(40, dim, seed=60)
    table = oracle.quantize(w)
    _, w_hat = oracle.unpack(*table, dim)
    tokens = np.array([[0], [7], [39], [12]], dtype=np.int32)
    y = oracle.embed_sum(tokens, [table], dim)
    for f, tok in enumerate(tokens[:, 0]):
        assert np.array_equal(y[f], w_hat[tok].astype(np.float64))


def test_embed_sum_of_seventeen_affine_streams_closed_form():
    """17 streams of exactly affine tables (bias a_t, step s0_t): the sum is
    sum_t (a_t + s0_t * code_t[token_t][d]), exact in double (small dyadic
    values), written out from the construction, not from the oracle."""
    dim, streams = 128, 17
    params = [(-1.5 + 0.25 * t, 2.0 ** -(t % 5), 3 if t == 0 else 2) for t in range(streams)]
    tables, codes, rows_of = [], [], []
    for t, (a, s0, rows_scale) in enumerate(params):
        rows = 16 * rows_scale
        w, c = _affine_table(rows, dim, a, s0, seed=70 + t)
        P, S, B = oracle.quantize(w)
        assert np.all(oracle.bf16_value(S) == np.float32(s0)) and np.all(oracle.bf16_value(B) == np.float32(a))
        tables.append((P, S, B))
        codes.append(c)
        rows_of.append(rows)
    r = np.random.default_rng(80)
    tokens = np.stack([[r.integers(0, rows_of[t]) for t in range(streams)] for _ in range(3)]).astype(np.int32)
    y = oracle.embed_sum(tokens, tables, dim)
    for f in range(tokens.shape[0]):
        want = np.zeros(dim, dtype=np.float64)
        for t, (a, s0, _) in enumerate(params):
            want += a + s0 * codes[t][tokens[f, t]]
        assert np.array_equal(y[f], want)


def test_embed_tokens_outside_a_table_add_nothing():
    dim = 64
    t0 = oracle.quantize(_gaussian(5, dim, seed=90))
    t1 = oracle.quantize(_gaussian(9, dim, seed=91))
    _, w0 = oracle.unpack(*t0, dim)
    _, w1 = oracle.unpack(*t1, dim)
    tokens = np.array([[-1, 3], [5, 2], [4, 9], [-7, -1], [2, 8]], dtype=np.int32)
    y = oracle.embed_sum(tokens, [t0, t1], dim)
    assert np.array_equal(y[0], w1[3].astype(np.float64))
    assert np.array_equal(y[1], w1[2].astype(np.float64))      # token 5 is past table 0's 5 rows
    assert np.array_equal(y[2], w0[4].astype(np.float64))      # token 9 is past table 1's 9 rows
    assert not y[3].any()
    assert np.array_equal(y[4], w0[2].astype(np.float64) + w1[8].astype(np.float64))


# ---------------------------------------------------------------- rotary embedding + decode attention
# (blog translation, optimisation list: the RoPE offset is a step input; ONNX
# README, How to use: the step carries K and V caches [layers][1][32][T][128])

def _bits(vals):
    import torch
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_rope_position_zero_is_identity():
    x = workloads.activations(0, 7, 0, 0, 4, 64)
    assert np.array_equal(oracle.rope(x, 0), x)


def test_rope_hand_values():
    """One head of width 4, theta 10000: pair 0 turns by pos, pair 1 by
    pos / 100 (10000^(-2/4)); the unit vectors (1, 0) become (cos a, sin a).
    Values of cos and sin at 1, 0.01, 3, 0.03 written out."""
    x = _bits([[1.0, 0.0, 1.0, 0.0]])
    want1 = _bits([[0.5403023058681398, 0.8414709848078965, 0.9999500004166653, 0.009999833334166664]])
    want3 = _bits([[-0.9899924966004454, 0.1411200080598672, 0.9995500337489875, 0.02999550020249566]])
    assert np.array_equal(oracle.rope(x, 1), want1)
    assert np.array_equal(oracle.rope(x, 3), want3)
    # the second element of a pair: (0, 1) becomes (-sin a, cos a)
    y = _bits([[0.0, 1.0, 0.0, 1.0]])
    assert np.array_equal(oracle.rope(y, 1), _bits([[-0.8414709848078965, 0.5403023058681398,
                                                    -0.009999833334166664, 0.9999500004166653]]))


def test_rope_keeps_pair_norms_and_relative_positions():
    x = workloads.activations(0, 7, 0, 1, 8, 128)
    xv = oracle.bf16_value(x).astype(np.float64)
    for pos in (1, 17, 4095):
        r = oracle.bf16_value(oracle.rope(x, pos)).astype(np.float64)
        n0 = xv[:, 0::2] ** 2 + xv[:, 1::2] ** 2
        n1 = r[:, 0::2] ** 2 + r[:, 1::2] ** 2
        assert np.all(np.abs(n1 - n0) <= 2 ** -7 * n0 + 1e-30)
    # q . k after rotation depends on the distance of the positions only
    q = workloads.activations(0, 7, 0, 2, 1, 128)
    k = workloads.activations(0, 7, 0, 3, 1, 128)
    dots = []
    for shift in (0, 5, 100):
        qr = oracle.bf16_value(oracle.rope(q, 40 + shift)).astype(np.float64)
        kr = oracle.bf16_value(oracle.rope(k, 10 + shift)).astype(np.float64)
        dots.append(float((qr @ kr.T)[0, 0]))
    mag = float((np.abs(oracle.bf16_value(q)).astype(np.float64) @ np.abs(oracle.bf16_value(k)).astype(np.float64).T)[0, 0])
    assert max(dots) - min(dots) <= 2 ** -6 * mag


def test_attention_single_position_returns_its_value():
    heads, d, cap = 3, 64, 8
    q = workloads.activations(0, 7, 1, 0, heads, d)
    k = workloads.activations(0, 7, 1, 1, heads * cap, d).reshape(heads, cap, d)
    v = workloads.activations(0, 7, 1, 2, heads * cap, d).reshape(heads, cap, d)
    out = oracle.attn_decode(q, k, v, 0)
    assert np.array_equal(out, oracle.bf16_value(v[:, 0, :]).astype(np.float64))


def test_attention_equal_keys_average_the_values():
    heads, d, cap, pos = 2, 32, 16, 9
    q = workloads.activations(0, 7, 2, 0, heads, d)
    k = np.repeat(workloads.activations(0, 7, 2, 1, heads, d)[:, None, :], cap, axis=1)
    v = workloads.activations(0, 7, 2, 2, heads * cap, d).reshape(heads, cap, d)
    out = oracle.attn_decode(q, k, v, pos)
    mean = oracle.bf16_value(v[:, :pos + 1, :]).astype(np.float64).sum(axis=1) / (pos + 1)
    assert np.allclose(out, mean, rtol=1e-13, atol=1e-15)


def test_attention_two_positions_closed_form():
    """q = 2 e0, k0 = 0, k1 = 4 e0, D = 64: scores 0 and 2 * 4 / 8 = 1, so
    out = (v0 + e v1) / (1 + e); positions past pos are ignored."""
    import math
    d, cap = 64, 5
    q = np.zeros((1, d), np.uint16)
    q[0, 0] = _bits([2.0])[0]
    k = np.zeros((1, cap, d), np.uint16)
    k[0, 1, 0] = _bits([4.0])[0]
    k[0, 2:, 0] = _bits([100.0])[0]   # past pos: must not count
    v = workloads.activations(0, 7, 3, 0, cap, d).reshape(1, cap, d)
    out = oracle.attn_decode(q, k, v, 1)
    vv = oracle.bf16_value(v).astype(np.float64)
    want = (vv[0, 0] + math.e * vv[0, 1]) / (1.0 + math.e)
    assert np.allclose(out[0], want, rtol=1e-14, atol=1e-16)


# ---------------------------------------------------------------- RMSNorm and the gated product
# (GeekNews summary, audio pipeline; blog translation: RMSNorm and SwiGLU are
# among the model's reused parts)

def test_rmsnorm_of_a_constant_vector_is_the_weight():
    """x = c for every element: mean(x^2) = c^2, so out = g c / sqrt(c^2 + eps),
    which rounds to g for eps far below c^2."""
    k = 256
    g = workloads.activations(0, 11, 0, 0, 1, k)[0]
    for c in (1.0, -3.0, 0.125):
        x = np.full((1, k), _bits([c])[0], dtype=np.uint16)
        out = oracle.rmsnorm(x, g, 1e-6)
        want = g if c > 0 else _bits(-oracle.bf16_value(g))
        assert np.array_equal(out[0], want)


def test_rmsnorm_hand_values_and_scale_invariance():
    # x = (3, 4), g = 1, eps = 0: rms = sqrt(12.5); 3/sqrt(12.5) and 4/sqrt(12.5)
    x = _bits([[3.0, 4.0]])
    g = _bits([1.0, 1.0])
    assert np.array_equal(oracle.rmsnorm(x, g, 0.0), _bits([[0.848528137423857, 1.131370849898476]]))
    # scaling x by a power of two changes nothing (every step scales exactly)
    xr = workloads.activations(0, 11, 0, 1, 4, 1024)
    gr = workloads.activations(0, 11, 0, 2, 1, 1024)[0]
    xs = _bits(oracle.bf16_value(xr) * 8.0)
    assert np.array_equal(oracle.rmsnorm(xs, gr, 0.0), oracle.rmsnorm(xr, gr, 0.0))
    # with g = 1 the rows come out with unit mean square, up to bf16 rounding
    ones = _bits(np.ones(1024))
    y = oracle.bf16_value(oracle.rmsnorm(xr, ones, 0.0)).astype(np.float64)
    assert np.all(np.abs((y * y).mean(axis=1) - 1.0) < 2 ** -7)


def test_silu_mul_closed_forms():
    import math
    g = np.array([0.0, 1.0, -1.0, 20.0, -20.0, 2.5])
    u = np.array([3.0, 2.0, 2.0, 1.0, 1.0, -4.0])
    out = oracle.silu_mul(g, u)
    assert out[0] == 0.0
    assert out[1] == pytest.approx(2.0 * 0.7310585786300049, rel=1e-15)   # silu(1) = 1 / (1 + 1/e)
    assert out[2] == pytest.approx(2.0 * -0.2689414213699951, rel=1e-15)  # silu(-1) = -1 / (1 + e)
    assert out[3] == pytest.approx(20.0, rel=1e-8)                         # silu(t) -> t
    assert abs(out[4]) < 1e-7                                              # silu(t) -> 0
    assert out[5] == pytest.approx(-4.0 * 2.5 / (1.0 + math.exp(-2.5)), rel=1e-15)
