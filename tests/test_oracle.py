"""Pins for the fp64 CPU oracle, checked against facts fixed outside the oracle.

Every check here compares the oracle with something it does not compute itself: a
closed form derived by hand, an invariant of softmax attention, an independent library
routine (torch's CPU scaled_dot_product_attention or scipy's softmax in fp64), or exact
decimal arithmetic.  The attention function being pinned is exact softmax attention
(page "추론 최적화", section 6; co-design page, section "FlashAttention과 GEMM 모양"),
with grouped K/V heads (page "필수 LLM 최적화 기법(2)", section 1-1) and the
exactly-mergeable partial states of the LeanAttention digest (section "조각별로 합칠 수
있는 정확한 소프트맥스").
"""
import decimal
import math

import numpy as np
import pytest
import scipy.special
import torch

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def bf16_bits(x) -> np.ndarray:
    """float array -> bf16 bit patterns via torch's round-to-nearest-even conversion."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Independent decode through torch (library conversion), for building expectations."""
    return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def rand_bits(rng, shape, scale=1.0):
    return bf16_bits(rng.standard_normal(shape) * scale)


# ----------------------------------------------------------------------------- codec

def test_bf16_codec_known_patterns(oracle):
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x0000: 0.0, 0x3C00: 2.0 ** -7,
        0x4300: 128.0, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: math.inf, 0xFF80: -math.inf,
    }
    for bits, val in cases.items():
        assert oracle.bf16_to_f64(np.array([bits], dtype=np.uint16))[0] == val, hex(bits)
    neg0 = oracle.bf16_to_f64(np.array([0x8000], dtype=np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0


def test_bf16_codec_all_patterns_match_torch(oracle):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f64(allb)
    ref = bits_to_f64(allb)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


# ------------------------------------------------------------------ closed forms

def test_single_key_returns_its_value(oracle):
    rng = np.random.default_rng(1)
    B, Hq, KH, Hsz, S = 2, 8, 2, 128, 5
    q, k, v = rand_bits(rng, (B, Hq, Hsz)), rand_bits(rng, (B, KH, S, Hsz)), rand_bits(rng, (B, KH, S, Hsz))
    out = oracle.decode(q, k, v, [1, 1], Hq, KH, 1 / math.sqrt(Hsz))
    vf = bits_to_f64(v)
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(out[b, h], vf[b, h // 4, 0])


@pytest.mark.parametrize("k0, expect_w0", [(2.0, 1 / (1 + math.exp(-1.0))), (-6.0, 1 / (1 + math.exp(3.0)))])
def test_two_keys_logistic_closed_form(oracle, k0, expect_w0):
    # Hsz=4, scale 1/sqrt(4) = 1/2; q = e0, key0 = k0*e0, key1 = 0 -> s0 - s1 = k0/2,
    # so out = sigma(s0 - s1) v0 + sigma(s1 - s0) v1.
    Hsz = 4
    q = bf16_bits([[[1.0, 0, 0, 0]]])
    k = bf16_bits([[[[k0, 0, 0, 0], [0, 0, 0, 0]]]])
    v = bf16_bits([[[[1.0, -2.0, 0.5, 3.0], [-1.0, 4.0, 0.25, -3.0]]]])
    out = oracle.decode(q, k, v, [2], 1, 1, 0.5)
    vf = bits_to_f64(v)[0, 0]
    expect = expect_w0 * vf[0] + (1 - expect_w0) * vf[1]
    np.testing.assert_allclose(out[0, 0], expect, rtol=0, atol=1e-15)


def test_zero_query_gives_mean_of_values(oracle):
    rng = np.random.default_rng(2)
    B, Hq, KH, Hsz, S = 2, 4, 4, 64, 100
    q = bf16_bits(np.zeros((B, Hq, Hsz)))
    k, v = rand_bits(rng, (B, KH, S, Hsz)), rand_bits(rng, (B, KH, S, Hsz))
    sl = [37, 100]
    out = oracle.decode(q, k, v, sl, Hq, KH, 1 / 8)
    vf = bits_to_f64(v)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out[b, h], vf[b, h, : sl[b]].mean(axis=0), rtol=0, atol=1e-14)


def test_constant_values_return_the_constant(oracle):
    rng = np.random.default_rng(3)
    B, Hq, KH, Hsz, S = 3, 8, 2, 64, 77
    q, k = rand_bits(rng, (B, Hq, Hsz), 3.0), rand_bits(rng, (B, KH, S, Hsz))
    v = bf16_bits(np.full((B, KH, S, Hsz), -0.8125))
    out = oracle.decode(q, k, v, [77, 5, 60], Hq, KH, 1 / 8)
    np.testing.assert_allclose(out, -0.8125, rtol=0, atol=1e-15)


def test_identity_values_expose_weights_that_sum_to_one(oracle):
    # With Hsz >= L and v_j = e_j the output row is the softmax weight vector itself.
    rng = np.random.default_rng(4)
    Hsz, L = 64, 40
    q, k = rand_bits(rng, (1, 1, Hsz), 2.0), rand_bits(rng, (1, 1, L, Hsz))
    v = bf16_bits(np.eye(L, Hsz)[None, None])
    scale = 1 / 8
    out = oracle.decode(q, k, v, [L], 1, 1, scale)[0, 0]
    assert abs(out.sum() - 1.0) < 1e-12
    assert np.all(out[L:] == 0)
    scores = scale * (bits_to_f64(k)[0, 0] @ bits_to_f64(q)[0, 0])
    np.testing.assert_allclose(out[:L], scipy.special.softmax(scores), rtol=1e-12, atol=1e-15)


# -------------------------------------------------------------------- invariants

def test_key_permutation_invariance(oracle):
    rng = np.random.default_rng(5)
    Hq, KH, Hsz, L = 4, 1, 128, 333
    q, k, v = rand_bits(rng, (1, Hq, Hsz)), rand_bits(rng, (1, KH, L, Hsz)), rand_bits(rng, (1, KH, L, Hsz))
    perm = rng.permutation(L)
    a = oracle.decode(q, k, v, [L], Hq, KH, 1 / math.sqrt(Hsz))
    b = oracle.decode(q, k[:, :, perm], v[:, :, perm], [L], Hq, KH, 1 / math.sqrt(Hsz))
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_common_key_shift_invariance(oracle):
    # Adding one vector c to every key adds q.c to every score of a row; softmax is
    # unchanged.  Small integers keep k + c exact in bf16.
    rng = np.random.default_rng(6)
    Hq, Hsz, L = 4, 64, 50
    q = bf16_bits(rng.integers(-3, 4, (1, Hq, Hsz)))
    k = rng.integers(-8, 9, (1, 1, L, Hsz))
    c = rng.integers(-4, 5, (Hsz,))
    v = rand_bits(rng, (1, 1, L, Hsz))
    a = oracle.decode(q, bf16_bits(k), v, [L], Hq, 1, 0.125)
    b = oracle.decode(q, bf16_bits(k + c), v, [L], Hq, 1, 0.125)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_planted_huge_score_selects_its_value(oracle):
    # Score ~ +815 for one key: exp() of it overflows even fp64, so only a max-shifted
    # softmax returns the planted value; the margin to the next score is > 700.
    rng = np.random.default_rng(7)
    Hsz, L, hit = 128, 300, 123
    qf = np.zeros((1, 1, Hsz))
    qf[0, 0, 0] = 96.0
    kf = rng.standard_normal((1, 1, L, Hsz))
    kf[0, 0, :, 0] = np.clip(kf[0, 0, :, 0], -1, 1)
    kf[0, 0, hit, 0] = 96.0
    v = rand_bits(rng, (1, 1, L, Hsz))
    out = oracle.decode(bf16_bits(qf), bf16_bits(kf), v, [L], 1, 1, 1 / math.sqrt(Hsz))
    assert np.all(np.isfinite(out))
    np.testing.assert_array_equal(out[0, 0], bits_to_f64(v)[0, 0, hit])


def test_all_scores_hugely_negative_still_normalise(oracle):
    # Every score near -815: exp() underflows to 0 without the max shift.
    rng = np.random.default_rng(8)
    Hsz, L = 128, 64
    qf = np.zeros((1, 1, Hsz))
    qf[0, 0, 0] = 96.0
    qf[0, 0, 1] = 1.0
    kf = np.zeros((1, 1, L, Hsz))
    kf[0, 0, :, 0] = -96.0
    kf[0, 0, :, 1] = rng.integers(-4, 5, L)
    kshift = kf.copy()
    kshift[0, 0, :, 0] = 0.0
    v = rand_bits(rng, (1, 1, L, Hsz))
    a = oracle.decode(bf16_bits(qf), bf16_bits(kf), v, [L], 1, 1, 1 / math.sqrt(Hsz))
    b = oracle.decode(bf16_bits(qf), bf16_bits(kshift), v, [L], 1, 1, 1 / math.sqrt(Hsz))
    assert np.all(np.isfinite(a))
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_score_multiplier_equals_scaled_query(oracle):
    rng = np.random.default_rng(9)
    Hq, KH, Hsz, L = 8, 1, 128, 200
    qf = rng.standard_normal((1, Hq, Hsz))
    k, v = rand_bits(rng, (1, KH, L, Hsz)), rand_bits(rng, (1, KH, L, Hsz))
    s = 1 / math.sqrt(Hsz)
    a = oracle.decode(bf16_bits(qf), k, v, [L], Hq, KH, 8 * s)
    b = oracle.decode(bf16_bits(8 * bits_to_f64(bf16_bits(qf))), k, v, [L], Hq, KH, s)
    np.testing.assert_array_equal(a, b)


def test_empty_context_gives_zero_rows(oracle):
    rng = np.random.default_rng(10)
    q, k, v = rand_bits(rng, (2, 4, 64)), rand_bits(rng, (2, 2, 9, 64)), rand_bits(rng, (2, 2, 9, 64))
    out = oracle.decode(q, k, v, [0, 9], 4, 2, 0.125)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


# ------------------------------------------------------------ merge of partials

@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_arbitrary_splits_merge_to_full_result(oracle, seed):
    rng = np.random.default_rng(100 + seed)
    B, Hq, KH, Hsz, L = 1, 4, 2, 64, 517
    q, k, v = rand_bits(rng, (B, Hq, Hsz), 2.0), rand_bits(rng, (B, KH, L, Hsz)), rand_bits(rng, (B, KH, L, Hsz))
    scale = 1 / 8
    full = oracle.decode(q, k, v, [L], Hq, KH, scale)
    npieces = int(rng.integers(1, 12))
    cuts = np.sort(rng.integers(0, L + 1, npieces - 1))  # may repeat: empty pieces
    bounds = [0, *cuts.tolist(), L]
    for h in range(Hq):
        ms, ls, os_ = [], [], []
        for j0, j1 in zip(bounds[:-1], bounds[1:]):
            m, l, o = oracle.partial_state(q, k, v, Hq, KH, scale, 0, h, j0, j1)
            ms.append(m)
            ls.append(l)
            os_.append(o)
        order = rng.permutation(len(ms))  # merge is commutative
        merged = oracle.merge_states(np.array(ms)[order], np.array(ls)[order], np.array(os_)[order])
        np.testing.assert_allclose(merged, full[0, h], rtol=1e-12, atol=1e-13)


def test_partial_state_of_single_key(oracle):
    rng = np.random.default_rng(11)
    q, k, v = rand_bits(rng, (1, 1, 64)), rand_bits(rng, (1, 1, 10, 64)), rand_bits(rng, (1, 1, 10, 64))
    m, l, o = oracle.partial_state(q, k, v, 1, 1, 0.125, 0, 0, 3, 4)
    expect_m = 0.125 * float(bits_to_f64(q)[0, 0] @ bits_to_f64(k)[0, 0, 3])
    assert abs(m - expect_m) < 1e-13 and l == 1.0
    np.testing.assert_array_equal(o, bits_to_f64(v)[0, 0, 3])
    m, l, o = oracle.partial_state(q, k, v, 1, 1, 0.125, 0, 0, 4, 4)
    assert m == -math.inf and l == 0.0 and np.all(o == 0)


# --------------------------------------------------------------- GQA structure

def test_gqa_equals_mha_with_contiguously_repeated_kv(oracle):
    rng = np.random.default_rng(12)
    B, Hq, KH, Hsz, S = 2, 8, 2, 64, 50
    q, k, v = rand_bits(rng, (B, Hq, Hsz)), rand_bits(rng, (B, KH, S, Hsz)), rand_bits(rng, (B, KH, S, Hsz))
    sl = [37, 50]
    gqa = oracle.decode(q, k, v, sl, Hq, KH, 0.125)
    G = Hq // KH
    mha = oracle.decode(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), sl, Hq, Hq, 0.125)
    np.testing.assert_array_equal(gqa, mha)
    # the interleaved grouping (kv head = h % KH) is a different function
    inter = oracle.decode(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), sl, Hq, Hq, 0.125)
    assert np.abs(inter - gqa).max() > 1e-3


def test_g1_is_plain_mha(oracle):
    rng = np.random.default_rng(13)
    B, H, Hsz, S = 2, 4, 64, 30
    q, k, v = rand_bits(rng, (B, H, Hsz)), rand_bits(rng, (B, H, S, Hsz)), rand_bits(rng, (B, H, S, Hsz))
    out = oracle.decode(q, k, v, [30, 11], H, H, 0.125)
    qf, kf, vf = bits_to_f64(q), bits_to_f64(k), bits_to_f64(v)
    for b, L in enumerate([30, 11]):
        for h in range(H):
            w = scipy.special.softmax(0.125 * kf[b, h, :L] @ qf[b, h])
            np.testing.assert_allclose(out[b, h], w @ vf[b, h, :L], rtol=1e-12, atol=1e-14)


# ------------------------------------------------- independent library routine

@pytest.mark.parametrize("Hq,KH,Hsz", [(8, 2, 64), (8, 8, 128), (16, 1, 256), (6, 3, 64)])
def test_decode_matches_torch_sdpa_fp64(oracle, Hq, KH, Hsz):
    rng = np.random.default_rng(14 + Hq + KH + Hsz)
    B, S = 3, 45
    sl = [1, 17, 45]
    q, k, v = rand_bits(rng, (B, Hq, Hsz), 2.0), rand_bits(rng, (B, KH, S, Hsz)), rand_bits(rng, (B, KH, S, Hsz))
    scale = 1 / math.sqrt(Hsz)
    out = oracle.decode(q, k, v, sl, Hq, KH, scale)
    G = Hq // KH
    qt, kt, vt = (torch.from_numpy(bits_to_f64(x)) for x in (q, k, v))
    for b, L in enumerate(sl):
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[b][None, :, None, :], kt[b, :, :L].repeat_interleave(G, 0)[None],
            vt[b, :, :L].repeat_interleave(G, 0)[None], scale=scale)
        np.testing.assert_allclose(out[b], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_matches_torch_sdpa_causal_fp64(oracle):
    rng = np.random.default_rng(15)
    B, Hq, KH, ISL, Hsz = 2, 8, 2, 70, 64
    q, k, v = rand_bits(rng, (B, Hq, ISL, Hsz)), rand_bits(rng, (B, KH, ISL, Hsz)), rand_bits(rng, (B, KH, ISL, Hsz))
    out = oracle.prefill_causal(q, k, v, KH, 0.125)
    qt, kt, vt = (torch.from_numpy(bits_to_f64(x)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(Hq // KH, 1), vt.repeat_interleave(Hq // KH, 1), is_causal=True, scale=0.125)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_row0_is_v0_and_rows_match_decode(oracle):
    rng = np.random.default_rng(16)
    B, Hq, KH, ISL, Hsz = 1, 4, 2, 33, 128
    q, k, v = rand_bits(rng, (B, Hq, ISL, Hsz)), rand_bits(rng, (B, KH, ISL, Hsz)), rand_bits(rng, (B, KH, ISL, Hsz))
    scale = 1 / math.sqrt(Hsz)
    out = oracle.prefill_causal(q, k, v, KH, scale)
    vf = bits_to_f64(v)
    for h in range(Hq):
        np.testing.assert_array_equal(out[0, h, 0], vf[0, h // 2, 0])
    for i in [1, 7, 32]:
        dec = oracle.decode(np.ascontiguousarray(q[:, :, i]), k, v, [i + 1], Hq, KH, scale)
        np.testing.assert_allclose(out[0, :, i], dec[0], rtol=1e-13, atol=1e-15)


def test_prefill_row_subset_equals_full(oracle):
    rng = np.random.default_rng(17)
    B, Hq, KH, ISL, Hsz = 2, 4, 1, 40, 64
    q, k, v = rand_bits(rng, (B, Hq, ISL, Hsz)), rand_bits(rng, (B, KH, ISL, Hsz)), rand_bits(rng, (B, KH, ISL, Hsz))
    full = oracle.prefill_causal(q, k, v, KH, 0.125)
    rows = np.array([0, 5, 39, 40 * 5 + 17, B * Hq * ISL - 1])
    part = oracle.prefill_causal(q, k, v, KH, 0.125, rows=rows)
    flat_full, flat_part = full.reshape(-1, Hsz), part.reshape(-1, Hsz)
    np.testing.assert_array_equal(flat_part[rows], flat_full[rows])
    mask = np.ones(len(flat_part), bool)
    mask[rows] = False
    assert np.all(np.isnan(flat_part[mask]))


# ------------------------------------------------------ exact decimal brute force

def test_decimal_brute_force_tiny(oracle):
    """50-digit decimal evaluation of the attention sum on a tiny case (L=5, Hsz=3)."""
    decimal.getcontext().prec = 50
    rng = np.random.default_rng(18)
    Hsz, L = 3, 5
    q, k, v = rand_bits(rng, (1, 1, Hsz), 2.0), rand_bits(rng, (1, 1, L, Hsz), 2.0), rand_bits(rng, (1, 1, L, Hsz))
    out = oracle.decode(q, k, v, [L], 1, 1, 0.5)
    D = decimal.Decimal
    qf, kf, vf = bits_to_f64(q)[0, 0], bits_to_f64(k)[0, 0], bits_to_f64(v)[0, 0]
    s = [D("0.5") * sum(D(float(qf[d])) * D(float(kf[j, d])) for d in range(Hsz)) for j in range(L)]
    w = [x.exp() for x in s]
    tot = sum(w)
    for d in range(Hsz):
        exact = sum(w[j] * D(float(vf[j, d])) for j in range(L)) / tot
        assert abs(float(exact) - out[0, 0, d]) < 1e-14


# ------------------------------------------------------------ FP8 E4M3 KV cache

def test_fp8_e4m3_known_codes(oracle):
    # OCP E4M3: bias 7, 3 mantissa bits, exponent field 0 = subnormals, S.1111.111 = NaN
    cases = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x30: 0.5, 0xB8: -1.0, 0xC4: -3.0}
    for code, val in cases.items():
        assert oracle.fp8_e4m3_to_f64([code])[0] == val, hex(code)
    assert np.isnan(oracle.fp8_e4m3_to_f64([0x7F])[0]) and np.isnan(oracle.fp8_e4m3_to_f64([0xFF])[0])
    neg0 = oracle.fp8_e4m3_to_f64([0x80])[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0


def test_fp8_e4m3_all_codes_match_torch(oracle):
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], ref[~nan])


def fp8_codes(x) -> np.ndarray:
    """float array -> E4M3 codes via torch's round-to-nearest-even, saturating conversion."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def fp8_as_bf16_bits(codes) -> np.ndarray:
    """E4M3 codes -> the bf16 bit patterns of the same values (exact: E4M3 fits bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.5, 4.0), (0.0625, 0.25)])
def test_fp8_decode_equals_bf16_decode_of_the_same_values(oracle, k_scale, v_scale):
    # every E4M3 value is a bf16 value, and power-of-two scales are exact: the FP8 oracle
    # must reproduce the pinned bf16 oracle with the scale folded into q.k and out
    rng = np.random.default_rng(30)
    B, Hq, KH, Hsz, S = 2, 8, 2, 64, 90
    sl = [90, 37]
    q = rand_bits(rng, (B, Hq, Hsz))
    k8, v8 = fp8_codes(rng.standard_normal((B, KH, S, Hsz)) * 3), fp8_codes(rng.standard_normal((B, KH, S, Hsz)))
    got = oracle.decode_fp8(q, k8, v8, sl, Hq, KH, 0.125, k_scale, v_scale)
    ref = oracle.decode(q, fp8_as_bf16_bits(k8), fp8_as_bf16_bits(v8), sl, Hq, KH, 0.125 * k_scale) * v_scale
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_fp8_decode_closed_forms(oracle):
    rng = np.random.default_rng(31)
    Hsz = 64
    q = rand_bits(rng, (1, 4, Hsz))
    k8 = fp8_codes(rng.standard_normal((1, 1, 5, Hsz)))
    v8 = fp8_codes(rng.standard_normal((1, 1, 5, Hsz)))
    # one key: the scaled value itself
    out = oracle.decode_fp8(q, k8, v8, [1], 4, 1, 0.125, 1.0, 0.5)
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], 0.5 * oracle.fp8_e4m3_to_f64(v8[0, 0, 0]))
    # constant V: the constant, whatever the scores
    vc = np.full((1, 1, 5, Hsz), 0x3C, dtype=np.uint8)  # 1.5
    out = oracle.decode_fp8(q, k8, vc, [5], 4, 1, 0.125, 3.0, 2.0)
    np.testing.assert_allclose(out, 3.0, rtol=0, atol=1e-15)


# ------------------------------------------------------------- multi-token decode

def test_multi_gamma1_is_decode(oracle):
    rng = np.random.default_rng(70)
    B, Hq, KH, Hsz, S = 3, 8, 2, 64, 40
    sl = [40, 0, 17]
    q, k, v = rand_bits(rng, (B, Hq, 1, Hsz)), rand_bits(rng, (B, KH, S, Hsz)), rand_bits(rng, (B, KH, S, Hsz))
    a = oracle.decode_multi(q, k, v, sl, KH, 0.125)[:, :, 0]
    b = oracle.decode(np.ascontiguousarray(q[:, :, 0]), k, v, sl, Hq, KH, 0.125)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("gamma", [2, 4, 7])
def test_multi_equals_last_rows_of_causal_prefill(oracle, gamma):
    # gamma drafted positions checked at once are the last gamma rows of a causal prefill
    # over the whole context (the lecture: the target model scores them "like prefill")
    rng = np.random.default_rng(71 + gamma)
    Hq, KH, Hsz, L = 8, 2, 64, 29
    qf = rand_bits(rng, (1, Hq, L, Hsz))
    k, v = rand_bits(rng, (1, KH, L, Hsz)), rand_bits(rng, (1, KH, L, Hsz))
    pre = oracle.prefill_causal(qf, k, v, KH, 0.125)
    got = oracle.decode_multi(np.ascontiguousarray(qf[:, :, L - gamma:]), k, v, [L], KH, 0.125)
    np.testing.assert_allclose(got, pre[:, :, L - gamma:], rtol=1e-13, atol=1e-15)


def test_multi_matches_torch_sdpa_with_end_aligned_mask(oracle):
    rng = np.random.default_rng(73)
    B, Hq, KH, Hsz, S, gamma = 2, 8, 4, 64, 50, 5
    sl = [50, 23]
    q, k, v = rand_bits(rng, (B, Hq, gamma, Hsz)), rand_bits(rng, (B, KH, S, Hsz)), rand_bits(rng, (B, KH, S, Hsz))
    out = oracle.decode_multi(q, k, v, sl, KH, 0.125)
    qt, kt, vt = (torch.from_numpy(bits_to_f64(x)) for x in (q, k, v))
    for b, L in enumerate(sl):
        mask = torch.arange(L)[None, :] <= (L - gamma + torch.arange(gamma))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[b][None], kt[b, :, :L].repeat_interleave(Hq // KH, 0)[None],
            vt[b, :, :L].repeat_interleave(Hq // KH, 0)[None], attn_mask=mask, scale=0.125)
        np.testing.assert_allclose(out[b], ref[0].numpy(), rtol=1e-12, atol=1e-13)


def test_multi_first_draft_sees_the_prefix_only(oracle):
    # with V = e_j, the output of draft t is its weight vector: zero on keys after L - gamma + t
    rng = np.random.default_rng(74)
    Hsz, L, gamma = 64, 20, 4
    q = rand_bits(rng, (1, 1, gamma, Hsz), 2.0)
    k = rand_bits(rng, (1, 1, L, Hsz))
    v = bf16_bits(np.eye(L, Hsz)[None, None])
    out = oracle.decode_multi(q, k, v, [L], 1, 0.125)[0, 0]
    for t in range(gamma):
        last = L - gamma + t
        assert np.all(out[t, last + 1:] == 0) and out[t, last] > 0
        assert abs(out[t].sum() - 1.0) < 1e-12
