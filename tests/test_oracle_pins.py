"""Pins of the CPU oracle to things other than itself.

Each test ties one step of the oracle to a library routine, a closed form,
an invariant, a hand-derived table or brute force, chosen so that a dropped
term, a wrong sign or index, or a swapped operand in the oracle fails at
least one of them.  No GPU is involved.

Passages: "aclnnNsaCompress" page, Formula (compression);
"mindspore.ops.nsa_compress_attention" page, steps 1-7 (attention,
importance remap, group sum, top-k).
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(x) -> np.ndarray:
    """bf16 bit patterns of values that must already be bf16-representable."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    b = synth.bf16_bits(t)
    assert np.array_equal(oracle.bf16_to_f64(b), np.asarray(x, dtype=np.float64)), \
        "test input is not exactly representable in bfloat16"
    return b


def rand_bf16(rng, shape, std=1.0) -> np.ndarray:
    x = torch.tensor(rng.standard_normal(shape).astype(np.float32) * std).to(torch.bfloat16)
    return synth.bf16_bits(x)


def rand_f16(rng, shape, std=1.0) -> np.ndarray:
    """float16 bit patterns of normals, rounded by numpy."""
    return (rng.standard_normal(shape) * std).astype(np.float16).view(np.uint16)


def rand_bits(rng, shape, dtype, std=1.0) -> np.ndarray:
    return rand_f16(rng, shape, std) if dtype == "f16" else rand_bf16(rng, shape, std)


def widen_torch(b, dtype) -> torch.Tensor:
    """float64 values of bit patterns, widened by torch (not by the oracle)."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(tdt).to(torch.float64)


def starts_of(lens):
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)


def n_vis_of(t, l, d, n_cmp):
    """Number of compressed blocks i with i*d + l - 1 <= t (capped at n_cmp),
    counted by brute force."""
    return sum(1 for i in range(n_cmp) if i * d + l - 1 <= t)


def run_all(q, kc, vc, lens, N1, N2, scale, l, d, lsel, count):
    """Oracle steps 1-7 for every token of the given sequences."""
    actq = np.cumsum(lens).astype(np.int64)
    actc = oracle.cmp_prefix(lens, l, d)
    tokens = np.arange(int(sum(lens)), dtype=np.int64)
    return oracle.attention(q, tokens, kc, vc, actq, actc, N1, N2, scale, l, d, lsel, count)


# --------------------------------------------------------------------------
# bfloat16 rounding
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_on_float32_inputs():
    """For float32 inputs, one rounding step from double equals torch's
    float32 -> bfloat16 conversion (round to nearest, ties to even)."""
    rng = np.random.default_rng(0)
    mant = rng.standard_normal(200_000).astype(np.float32)
    expo = rng.integers(-140, 128, 200_000).astype(np.float32)
    with np.errstate(over="ignore"):
        x = (mant * np.exp2(expo)).astype(np.float32)
    tie_bits = (rng.integers(0, 2 ** 31, 50_000, dtype=np.uint64).astype(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, tie_bits.view(np.float32)])
    x = x[np.isfinite(x)]
    ref = synth.bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    got = oracle.to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,expect", [
    (1.0, 0x3F80), (-1.0, 0xBF80), (0.0, 0x0000), (-0.0, 0x8000),
    (1 + 2 ** -8, 0x3F80),            # tie -> even (down)
    (1 + 3 * 2 ** -8, 0x3F82),        # tie -> even (up)
    (1 + 2 ** -8 + 2 ** -40, 0x3F81), # just above a tie: up, in one step
    (2.0 ** -133, 0x0001),            # smallest subnormal
    (2.0 ** -134, 0x0000),            # tie between 0 and it -> 0
    (3 * 2.0 ** -134, 0x0002),        # tie between 1 and 2 subnormal steps -> 2
    (3.3895313892515355e38, 0x7F7F),  # largest finite
    (3.4e38, 0x7F80),                 # rounds past it -> inf
    (float("inf"), 0x7F80),
])
def test_bf16_rounding_special_values(x, expect):
    assert int(oracle.to_bf16(np.array([x]))[0]) == expect


def test_bf16_decode_all_patterns_match_torch():
    """Every finite bfloat16 pattern widens to torch's value (C decoder)."""
    allb = np.arange(65536, dtype=np.uint16)
    ref = widen_torch(allb, "bf16").numpy()
    lib = oracle._load()
    got = np.array([lib.nsa_oracle_bf16_to_double(int(h)) for h in allb])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


# --------------------------------------------------------------------------
# float16 (IEEE binary16) widening and rounding
# --------------------------------------------------------------------------

def test_f16_decode_all_patterns_match_numpy():
    """All 65536 binary16 patterns widen to numpy's float16 values, infinities
    and signed zeros included; NaN patterns decode to NaN."""
    allb = np.arange(65536, dtype=np.uint16)
    ref = allb.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(allb)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_rounding_matches_numpy_on_float64_inputs():
    """Doubles across the whole binary16 range, its subnormals, exact ties
    and the overflow edge round as numpy's double -> half conversion does
    (round to nearest, ties to even, in one step)."""
    rng = np.random.default_rng(10)
    mant = rng.standard_normal(200_000)
    expo = rng.integers(-28, 18, 200_000)
    x = mant * np.exp2(expo)
    # exact ties: halfway between neighbouring half values (normal and subnormal)
    h = rng.integers(0, 0x7BFF, 50_000, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = (lo + hi) / 2
    x = np.concatenate([x, ties, -ties, [65504.0, 65519.99, 65520.0, 2.0 ** -25, 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.to_f16(x)
    assert np.array_equal(got, ref)


def test_f16_rounding_matches_torch_on_float32_inputs():
    """For float32 inputs, one rounding step from double equals torch's
    float32 -> float16 conversion."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(100_000) * np.exp2(rng.integers(-27, 17, 100_000))).astype(np.float32)
    ref = synth.bits(torch.from_numpy(x).to(torch.float16))
    got = oracle.to_f16(x.astype(np.float64))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,expect", [
    (1.0, 0x3C00), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    (1 + 2 ** -11, 0x3C00),           # tie -> even (down)
    (1 + 3 * 2 ** -11, 0x3C02),       # tie -> even (up)
    (1 + 2 ** -11 + 2 ** -40, 0x3C01),  # just above a tie: up, in one step
    (2.0 ** -24, 0x0001),             # smallest subnormal
    (2.0 ** -25, 0x0000),             # tie between 0 and it -> 0
    (3 * 2.0 ** -25, 0x0002),         # tie between 1 and 2 subnormal steps -> 2
    (2.0 ** -14, 0x0400),             # smallest normal
    (2.0 ** -14 - 2.0 ** -25, 0x0400),  # tie between the largest subnormal and it -> even
    (65504.0, 0x7BFF),                # largest finite
    (65519.0, 0x7BFF),                # below the halfway point: stays finite
    (65520.0, 0x7C00),                # halfway to 2^16: ties to even -> inf
    (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
])
def test_f16_rounding_special_values(x, expect):
    assert int(oracle.to_f16(np.array([x]))[0]) == expect


def test_f16_rounding_nan():
    assert np.isnan(oracle.f16_to_f64(oracle.to_f16(np.array([float("nan")])))[0])


# --------------------------------------------------------------------------
# Compression ("aclnnNsaCompress", Formula)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,l,d,n", [(0, 32, 16, 0), (31, 32, 16, 0), (32, 32, 16, 1),
                                     (47, 32, 16, 1), (48, 32, 16, 2), (512, 32, 16, 31),
                                     (65536, 64, 32, 2047), (100, 16, 16, 6)])
def test_number_of_windows(T, l, d, n):
    """i runs over 0 .. floor((T-l)/d): counted by brute force over start rows."""
    brute = sum(1 for i in range(T + 1) if i * d + l <= T)
    assert brute == n
    assert oracle.n_cmp(T, l, d) == n


def test_compress_block_means_when_stride_equals_window():
    """l = d and w = 1/l: windows do not overlap and each output is the mean
    of its block, computed here with numpy reshape + mean."""
    rng = np.random.default_rng(1)
    l = d = 16
    lens = [16 * 5, 16 * 3 + 7, 9, 16]
    N, D = 3, 5
    x = rand_bf16(rng, (sum(lens), N, D))
    w = bits(np.full((l, N), 1.0 / l))
    got = oracle.compress(x, w, np.cumsum(lens), l, d)
    xf = oracle.bf16_to_f64(x)
    ref = []
    for s, T in zip(starts_of(lens), lens):
        nb = T // l
        ref.append(xf[s:s + nb * l].reshape(nb, l, N, D).mean(axis=1))
    ref = np.concatenate(ref)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("l,d", [(32, 16), (48, 16), (64, 32), (16, 16)])
def test_compress_impulse_response(l, d):
    """A single 1 at row r of head n, column e reaches output i exactly when
    row r lies in window i (rows i*d .. i*d+l-1), with the weight of its
    position in the window, and nowhere else -- not across sequences."""
    rng = np.random.default_rng(2)
    lens = [l + 3 * d + 5, l + d]
    N, D = 2, 3
    T = sum(lens)
    w = rand_bf16(rng, (l, N))
    wf = oracle.bf16_to_f64(w)
    starts = starts_of(lens)
    outs_per = [oracle.n_cmp(t, l, d) for t in lens]
    out_starts = np.concatenate([[0], np.cumsum(outs_per)[:-1]])
    for r in [0, 1, d, l - 1, l, lens[0] - 1, lens[0], T - 1]:
        n, e = r % N, (r * 7) % D
        xf = np.zeros((T, N, D))
        xf[r, n, e] = 1.0
        got = oracle.compress(bits(xf), w, np.cumsum(lens), l, d)
        expect = np.zeros_like(got)
        b = int(np.searchsorted(np.cumsum(lens), r, side="right"))
        rl = r - starts[b]
        for i in range(outs_per[b]):
            p = rl - i * d
            if 0 <= p < l:
                expect[out_starts[b] + i, n, e] = wf[p, n]
        assert np.array_equal(got, expect), f"impulse at row {r}"


def test_compress_constant_rows():
    """Rows constant along the sequence: every output is (sum_p w[p,n]) * c[n]."""
    rng = np.random.default_rng(3)
    l, d, N, D = 32, 16, 4, 6
    lens = [200, 77]
    c = np.array([1.5, -2.0, 0.25, 3.0])
    xf = np.broadcast_to(c[None, :, None], (sum(lens), N, D))
    w = rand_bf16(rng, (l, N))
    got = oracle.compress(bits(xf), w, np.cumsum(lens), l, d)
    expect = oracle.bf16_to_f64(w).sum(axis=0)[None, :, None] * c[None, :, None]
    np.testing.assert_allclose(got, np.broadcast_to(expect, got.shape), rtol=1e-13)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_compress_matches_numpy_weighted_windows(dtype):
    """Per element type: every output row is the numpy weighted sum of its
    window, on inputs widened by torch -- pins that the element type picks
    the matching decoder for both x and w."""
    rng = np.random.default_rng(12)
    l, d, N, D = 32, 16, 2, 8
    lens = [140, 33, 70]
    x = rand_bits(rng, (sum(lens), N, D), dtype)
    w = rand_bits(rng, (l, N), dtype, std=0.1)
    got = oracle.compress(x, w, np.cumsum(lens), l, d, dtype)
    xf, wf = widen_torch(x, dtype).numpy(), widen_torch(w, dtype).numpy()
    ref = []
    for s0, T in zip(starts_of(lens), lens):
        for i in range(oracle.n_cmp(T, l, d)):
            win = xf[s0 + i * d:s0 + i * d + l]                 # [l, N, D]
            ref.append(np.einsum("pn,pnd->nd", wf, win))
    ref = np.stack(ref)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_compress_is_linear():
    """compress(2x + y) = 2 compress(x) + compress(y) on small integers (exact)."""
    rng = np.random.default_rng(4)
    l, d, N, D = 32, 16, 2, 4
    lens = [150]
    xf = rng.integers(-8, 9, (150, N, D)).astype(np.float64)
    yf = rng.integers(-8, 9, (150, N, D)).astype(np.float64)
    w = bits(rng.integers(0, 4, (l, N)) / 4.0)
    a = oracle.compress(bits(2 * xf + yf), w, lens, l, d)
    b = 2 * oracle.compress(bits(xf), w, lens, l, d) + oracle.compress(bits(yf), w, lens, l, d)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# Steps 1-3: scaled scores, mask, softmax, output
# --------------------------------------------------------------------------

def _attention_case(seed, lens, N1, N2, D1, D2, l, d, kv_std=1.0, dtype="bf16"):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    T2 = int(oracle.cmp_prefix(lens, l, d)[-1])
    q = rand_bits(rng, (T, N1, D1), dtype)
    kc = rand_bits(rng, (T2, N2, D1), dtype, kv_std)
    vc = rand_bits(rng, (T2, N2, D2), dtype, kv_std)
    return q, kc, vc


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_attention_matches_torch_sdpa(dtype):
    """Rows with at least one visible block equal torch's scaled dot-product
    attention (float64, boolean mask built from the visibility rule);
    softmax max and sum equal torch's masked max and exp(logsumexp - max).
    Inputs are widened by torch for the reference, so the element type must
    reach every decode in the oracle."""
    lens = [40, 77, 130, 31]
    N1, N2, D1, D2, l, d, lsel, count = 6, 2, 16, 8, 32, 16, 64, 2
    scale = 0.3
    q, kc, vc = _attention_case(5, lens, N1, N2, D1, D2, l, d, dtype=dtype)
    actq = np.cumsum(lens).astype(np.int64)
    res = oracle.attention(q, np.arange(int(sum(lens)), dtype=np.int64), kc, vc, actq,
                           oracle.cmp_prefix(lens, l, d), N1, N2, scale, l, d, lsel, count,
                           dtype=dtype)
    qf, kf, vf = (widen_torch(a, dtype) for a in (q, kc, vc))
    actc = oracle.cmp_prefix(lens, l, d)
    cstarts = np.concatenate([[0], actc[:-1]])
    G = N1 // N2
    for b, (s, T) in enumerate(zip(starts_of(lens), lens)):
        nc = int(actc[b] - cstarts[b])
        if nc == 0:
            continue
        t = torch.arange(T)[:, None]
        i = torch.arange(nc)[None, :]
        mask = (i * d + l - 1) <= t                      # [T, nc]
        has = mask.any(dim=1)
        for h in range(N1):
            g = h // G
            qb = qf[s:s + T, h]
            kb = kf[cstarts[b]:cstarts[b] + nc, g]
            vb = vf[cstarts[b]:cstarts[b] + nc, g]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qb[None, None], kb[None, None], vb[None, None], attn_mask=mask[None, None],
                scale=scale)[0, 0]
            got = torch.from_numpy(res["out"][s:s + T, h])
            torch.testing.assert_close(got[has], ref[has], rtol=1e-12, atol=1e-13)
            sc = torch.where(mask, scale * (qb @ kb.T), torch.tensor(-float("inf"), dtype=torch.float64))
            mx = sc.max(dim=1).values
            lse = torch.logsumexp(sc, dim=1)
            torch.testing.assert_close(torch.from_numpy(res["max"][s:s + T, h])[has], mx[has],
                                       rtol=1e-13, atol=1e-13)
            torch.testing.assert_close(torch.from_numpy(res["sum"][s:s + T, h])[has],
                                       torch.exp(lse - mx)[has], rtol=1e-12, atol=0)


def _identity_value_case(lens, N1, N2, D1, l, d, seed=6, scale=0.5):
    """Values are unit vectors: output row h of token t is P_cmp itself."""
    T2 = int(oracle.cmp_prefix(lens, l, d)[-1])
    actc = oracle.cmp_prefix(lens, l, d)
    n_cmp_max = int(max(np.diff(np.concatenate([[0], actc]))))
    D2 = max(n_cmp_max, 1)
    rng = np.random.default_rng(seed)
    q = rand_bf16(rng, (sum(lens), N1, D1))
    kc = rand_bf16(rng, (T2, N2, D1))
    vcf = np.zeros((T2, N2, D2))
    for s, e in zip(np.concatenate([[0], actc[:-1]]), actc):
        for i in range(int(e - s)):
            vcf[s + i, :, i] = 1.0
    return q, kc, bits(vcf), D2, scale


def test_softmax_rows_sum_to_one():
    """With unit-vector values the output is P_cmp; each row with a visible
    block sums to 1 and equals scipy's softmax of the masked scores."""
    from scipy.special import softmax
    lens = [200, 95]
    N1, N2, D1, l, d = 4, 2, 8, 32, 16
    q, kc, vc, D2, scale = _identity_value_case(lens, N1, N2, D1, l, d)
    res = run_all(q, kc, vc, lens, N1, N2, scale, l, d, 64, 4)
    qf, kf = oracle.bf16_to_f64(q), oracle.bf16_to_f64(kc)
    actc = oracle.cmp_prefix(lens, l, d)
    cst = np.concatenate([[0], actc[:-1]])
    for b, (s, T) in enumerate(zip(starts_of(lens), lens)):
        nc = int(actc[b] - cst[b])
        for t in range(T):
            nv = n_vis_of(t, l, d, nc)
            for h in range(N1):
                P = res["out"][s + t, h]
                if nv == 0:
                    assert np.all(P == 0)
                    continue
                assert abs(P.sum() - 1.0) < 1e-13
                assert np.all(P[nv:] == 0)
                sc = scale * (kf[cst[b]:cst[b] + nv, h // (N1 // N2)] @ qf[s + t, h])
                np.testing.assert_allclose(P[:nv], softmax(sc), rtol=1e-12, atol=1e-15)


def test_identical_keys_closed_form():
    """All compressed keys equal: scores are equal, so the output is the mean
    of the visible values, the softmax sum is n_vis and the max is
    scale * <q, k>."""
    rng = np.random.default_rng(7)
    lens = [300, 64]
    N1, N2, D1, D2, l, d = 4, 1, 8, 8, 32, 16
    T2 = int(oracle.cmp_prefix(lens, l, d)[-1])
    q = rand_bf16(rng, (sum(lens), N1, D1))
    k1 = oracle.bf16_to_f64(rand_bf16(rng, (D1,)))
    kc = bits(np.broadcast_to(k1, (T2, N2, D1)))
    vc = rand_bf16(rng, (T2, N2, D2))
    scale = 0.25
    res = run_all(q, kc, vc, lens, N1, N2, scale, l, d, 64, 4)
    qf, vf = oracle.bf16_to_f64(q), oracle.bf16_to_f64(vc)
    actc = oracle.cmp_prefix(lens, l, d)
    cst = np.concatenate([[0], actc[:-1]])
    for b, (s, T) in enumerate(zip(starts_of(lens), lens)):
        nc = int(actc[b] - cst[b])
        for t in range(T):
            nv = n_vis_of(t, l, d, nc)
            for h in range(N1):
                if nv == 0:
                    assert np.all(res["out"][s + t, h] == 0)
                    assert res["max"][s + t, h] == -np.inf and res["sum"][s + t, h] == 0
                    continue
                np.testing.assert_allclose(res["out"][s + t, h], vf[cst[b]:cst[b] + nv, 0].mean(axis=0),
                                           rtol=1e-12, atol=1e-14)
                assert abs(res["sum"][s + t, h] - nv) < 1e-12 * nv
                assert abs(res["max"][s + t, h] - scale * float(qf[s + t, h] @ k1)) < 1e-13


def test_single_visible_block_and_empty_rows():
    """Tokens l-1 .. l+d-2 see only block 0: output = v_0, sum = 1,
    max = s_0.  Tokens before l-1 see nothing: output 0, max -inf, sum 0."""
    lens = [96]
    N1, N2, D1, D2, l, d = 2, 1, 8, 4, 32, 16
    q, kc, vc = _attention_case(8, lens, N1, N2, D1, D2, l, d)
    scale = 0.7
    res = run_all(q, kc, vc, lens, N1, N2, scale, l, d, 64, 2)
    qf, kf, vf = (oracle.bf16_to_f64(a) for a in (q, kc, vc))
    for t in range(l - 1):
        assert np.all(res["out"][t] == 0)
        assert np.all(res["max"][t] == -np.inf) and np.all(res["sum"][t] == 0)
    for t in range(l - 1, l + d - 1):
        for h in range(N1):
            assert np.array_equal(res["out"][t, h], vf[0, 0])
            assert res["sum"][t, h] == 1.0
            assert abs(res["max"][t, h] - scale * float(qf[t, h] @ kf[0, 0])) < 1e-14
    assert not np.array_equal(res["out"][l + d - 1, 0], vf[0, 0])


def test_gqa_head_to_group_mapping():
    """Query head h reads KV head floor(h / G): make KV head 1's values a
    constant, so exactly heads G..2G-1 output that constant."""
    rng = np.random.default_rng(9)
    lens = [120]
    N1, N2, D1, D2, l, d = 6, 2, 8, 4, 32, 16
    G = N1 // N2
    T2 = int(oracle.cmp_prefix(lens, l, d)[-1])
    q = rand_bf16(rng, (120, N1, D1))
    kc = rand_bf16(rng, (T2, N2, D1))
    vcf = oracle.bf16_to_f64(rand_bf16(rng, (T2, N2, D2)))
    vcf[:, 1, :] = 0.625
    res = run_all(q, kc, bits(vcf), lens, N1, N2, 0.4, l, d, 64, 2)
    for t in range(l - 1, 120):
        for h in range(N1):
            is_const = np.allclose(res["out"][t, h], 0.625, rtol=1e-14, atol=0)
            assert is_const == (h // G == 1), (t, h)


# --------------------------------------------------------------------------
# Steps 4-5: importance-score remap and the sum over a KV-head group
# --------------------------------------------------------------------------

def _load_coefficients():
    rows = {}
    with open(os.path.join(GOLDEN, "remap_coefficients.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            l, d, lsel, R, L2, *c = map(int, line)
            rows[(l, d, lsel)] = (R, L2, c)
    return rows


COEFFS = _load_coefficients()


def _p_and_pslc(lens, N1, N2, l, d, lsel, seed=10):
    """Oracle P_cmp (through unit-vector values) and its P_slc'."""
    q, kc, vc, D2, scale = _identity_value_case(lens, N1, N2, 8, l, d, seed=seed, scale=0.9)
    actc = oracle.cmp_prefix(lens, l, d)
    res = run_all(q, kc, vc, lens, N1, N2, scale, l, d, lsel, 3)
    return res, actc


@pytest.mark.parametrize("l,d,lsel", sorted(COEFFS))
def test_remap_scatter_form(l, d, lsel):
    """Scatter form: every compressed block i adds P_cmp[i] to select block
    j = (i + m + n) / R for each (m, n) that makes it an integer -- the
    page's gather sum read the other way round; summed over the group's
    heads."""
    lens = [23 * d + l, 7 * d + l + 3]
    N1, N2 = 4, 2
    G = N1 // N2
    R, L2 = lsel // d, l // d
    res, actc = _p_and_pslc(lens, N1, N2, l, d, lsel)
    cst = np.concatenate([[0], actc[:-1]])
    for b, (s, T) in enumerate(zip(starts_of(lens), lens)):
        nc = int(actc[b] - cst[b])
        S = -(-T // lsel)
        for t in range(T):
            for g in range(N2):
                acc = np.zeros(S + R + L2 + 2)
                for h in range(g * G, (g + 1) * G):
                    P = res["out"][s + t, h, :nc]
                    for i in range(nc):
                        for m in range(R):
                            for n in range(L2):
                                if (i + m + n) % R == 0:
                                    acc[(i + m + n) // R] += P[i]
                np.testing.assert_allclose(res["pslc"][s + t, g, :S], acc[:S], rtol=1e-13, atol=1e-15)
                assert np.all(res["pslc"][s + t, g, S:] == 0)


@pytest.mark.parametrize("l,d,lsel", sorted(COEFFS))
def test_remap_hand_derived_coefficients(l, d, lsel):
    """Stencil form with the coefficient table derived by hand (golden file):
    P_slc'[j] = sum_r c(r) * sum_h P_cmp^h[R*j - r]."""
    R, L2, c = COEFFS[(l, d, lsel)]
    assert R == lsel // d and L2 == l // d
    lens = [17 * d + l + 5]
    N1, N2 = 2, 1
    res, actc = _p_and_pslc(lens, N1, N2, l, d, lsel, seed=11)
    nc = int(actc[0])
    S = -(-lens[0] // lsel)
    for t in range(lens[0]):
        Psum = res["out"][t, :, :nc].sum(axis=0)
        for j in range(S):
            ref = sum(cr * Psum[R * j - r] for r, cr in enumerate(c) if 0 <= R * j - r < nc)
            assert abs(res["pslc"][t, 0, j] - ref) <= 1e-13 * max(1.0, abs(ref))


def test_remap_mass_invariant():
    """Each compressed block is counted floor(l/d) times over all select
    blocks, so a row whose remap stays inside the select range has
    sum_j P_slc'[j] = G * floor(l/d) (softmax rows sum to 1)."""
    wl = synth.small_variant(2, [700, 333])
    inp = synth.make_inputs(wl)
    b = {k: synth.bf16_bits(v) for k, v in inp.items()}
    res = oracle.run(wl, b["q"], b["k"], b["v"], b["w"])
    R, L2 = wl.lsel // wl.d, wl.l // wl.d
    H = R + L2 - 2
    G = wl.N1 // wl.N2
    actc = oracle.cmp_prefix(wl.seqlens, wl.l, wl.d)
    cst = np.concatenate([[0], actc[:-1]])
    checked = 0
    for bi, (s, T) in enumerate(zip(starts_of(wl.seqlens), wl.seqlens)):
        nc = int(actc[bi] - cst[bi])
        S = -(-T // wl.lsel)
        for t in range(T):
            nv = n_vis_of(t, wl.l, wl.d, nc)
            if nv == 0 or (nv - 1 + H) // R >= S:
                continue
            sums = res["pslc"][s + t].sum(axis=1)
            np.testing.assert_allclose(sums, G * L2, rtol=1e-12)
            checked += 1
    assert checked > 500


def test_remap_identical_keys_closed_form():
    """Identical keys make P_cmp uniform, 1/n_vis on the visible blocks, so
    P_slc'[j] = G * sum_r c(r) [0 <= R*j - r < n_vis] / n_vis."""
    rng = np.random.default_rng(12)
    l, d, lsel = 32, 16, 64
    R, L2, c = COEFFS[(l, d, lsel)]
    lens = [400]
    N1, N2 = 8, 2
    G = N1 // N2
    T2 = int(oracle.cmp_prefix(lens, l, d)[-1])
    q = rand_bf16(rng, (400, N1, 8))
    kc = bits(np.broadcast_to(oracle.bf16_to_f64(rand_bf16(rng, (8,))), (T2, N2, 8)))
    vc = rand_bf16(rng, (T2, N2, 4))
    res = run_all(q, kc, vc, lens, N1, N2, 0.3, l, d, lsel, 4)
    S = -(-400 // lsel)
    for t in range(400):
        nv = n_vis_of(t, l, d, T2)
        for j in range(S):
            ref = 0.0 if nv == 0 else G * sum(cr for r, cr in enumerate(c) if 0 <= R * j - r < nv) / nv
            for g in range(N2):
                assert abs(res["pslc"][t, g, j] - ref) <= 1e-12 * max(1.0, ref)


# --------------------------------------------------------------------------
# Steps 6-7: top-k mask and top-k
# --------------------------------------------------------------------------

def _check_topk_brute(res, lens, lsel, count):
    for s, T in zip(starts_of(lens), lens):
        S = -(-T // lsel)
        for t in range(T):
            for g in range(res["pslc"].shape[1]):
                valid = np.array([j for j in range(S) if j * lsel <= t])
                keys = res["pslc"][s + t, g, valid].astype(np.float32)
                order = valid[np.lexsort((valid, -keys))]     # score desc, index asc
                expect = np.full(count, -1, dtype=np.int32)
                expect[:min(count, len(order))] = order[:count]
                assert np.array_equal(res["topk"][s + t, g], expect), (s + t, g)


def test_topk_matches_brute_force_sort_tiny_workload():
    """Full sort (numpy lexsort on float32 scores) of the candidates of each
    row, on the tiny workload."""
    wl = synth.WORKLOADS[0]
    inp = synth.make_inputs(wl)
    b = {k: synth.bf16_bits(v) for k, v in inp.items()}
    res = oracle.run(wl, b["q"], b["k"], b["v"], b["w"])
    _check_topk_brute(res, wl.seqlens, wl.lsel, wl.count)


def test_topk_brute_force_gqa_varlen():
    wl = dataclasses.replace(synth.small_variant(4, [640, 300]), N1=8, D1=16, D2=16)
    inp = synth.make_inputs(wl)
    b = {k: synth.bf16_bits(v) for k, v in inp.items()}
    res = oracle.run(wl, b["q"], b["k"], b["v"], b["w"])
    _check_topk_brute(res, wl.seqlens, wl.lsel, wl.count)


def test_topk_forced_when_few_candidates():
    """With at most `count` candidates every candidate is picked, whatever
    the scores; the rest are -1."""
    wl = synth.WORKLOADS[0]
    inp = synth.make_inputs(wl)
    b = {k: synth.bf16_bits(v) for k, v in inp.items()}
    res = oracle.run(wl, b["q"], b["k"], b["v"], b["w"])
    for t in range(wl.count * wl.lsel):
        nvalid = t // wl.lsel + 1
        picks = res["topk"][t, 0]
        assert sorted(picks[:nvalid].tolist()) == list(range(nvalid))
        assert np.all(picks[nvalid:] == -1)
    assert np.array_equal(res["topk"][0, 0], [0, -1, -1, -1])


def test_topk_ties_go_to_lower_index():
    """Identical keys make interior importance scores exactly equal; the picks
    are the candidates sorted by (score desc, index asc) -- numpy lexsort."""
    rng = np.random.default_rng(13)
    l, d, lsel, count = 32, 16, 64, 4
    lens = [640]
    N1, N2 = 4, 1
    T2 = int(oracle.cmp_prefix(lens, l, d)[-1])
    q = rand_bf16(rng, (640, N1, 8))
    kc = bits(np.broadcast_to(oracle.bf16_to_f64(rand_bf16(rng, (8,))), (T2, N2, 8)))
    vc = rand_bf16(rng, (T2, N2, 4))
    res = run_all(q, kc, vc, lens, N1, N2, 0.3, l, d, lsel, count)
    ties = 0
    for t in range(640):
        row = res["pslc"][t, 0, : t // lsel + 1].astype(np.float32)
        ties += len(row) - len(np.unique(row))
    assert ties > 100
    _check_topk_brute(res, lens, lsel, count)


# --------------------------------------------------------------------------
# Explicit atten_mask / topk_mask (MindSpore page, Parameters: optional bool
# tensors of shape (S1, S2)).  Reading: one matrix shared by all sequences,
# indexed by (local query position, compressed entry or select block); a
# true element masks its pair out and replaces that step's positional rule.
# --------------------------------------------------------------------------

def _mask_case(seed, lens, N1, N2, D1, D2, l, d, lsel, extra_rows=3, extra_cols=5,
               p_masked=0.4):
    rng = np.random.default_rng(seed)
    q, kc, vc = _attention_case(seed, lens, N1, N2, D1, D2, l, d)
    actc = oracle.cmp_prefix(lens, l, d)
    nc_max = int(np.diff(np.concatenate([[0], actc])).max())
    s_max = max(-(-T // lsel) for T in lens)
    rows = max(lens) + extra_rows
    am = rng.random((rows, nc_max + extra_cols)) < p_masked
    tm = rng.random((rows, s_max + extra_cols)) < p_masked
    am[5, :] = True             # a row with every block masked
    am[7, :] = False            # a row that sees blocks the causal rule hides
    tm[6, :] = True             # a row with no top-k candidate
    return q, kc, vc, am, tm


def test_atten_mask_matches_torch_sdpa_and_literal_remap():
    """An explicit atten_mask: rows with a visible block equal torch's SDPA
    with the complementary boolean mask (torch's True = takes part); fully
    masked rows give 0 / -inf / 0; P_slc' is the literal remap formula over
    the masked softmax, summed over the group, computed here in numpy."""
    lens = [90, 41, 130]
    N1, N2, D1, D2, l, d, lsel, count = 4, 2, 16, 8, 32, 16, 64, 3
    scale = 0.4
    q, kc, vc, am, _ = _mask_case(21, lens, N1, N2, D1, D2, l, d, lsel)
    actq = np.cumsum(lens).astype(np.int64)
    actc = oracle.cmp_prefix(lens, l, d)
    res = oracle.attention(q, np.arange(sum(lens), dtype=np.int64), kc, vc, actq, actc, N1, N2,
                           scale, l, d, lsel, count, atten_mask=am)
    qf, kf, vf = (widen_torch(a, "bf16") for a in (q, kc, vc))
    cst = np.concatenate([[0], actc[:-1]])
    G, R, L2 = N1 // N2, lsel // d, l // d
    n_full_rows = n_empty = 0
    for b, (s, T) in enumerate(zip(starts_of(lens), lens)):
        nc = int(actc[b] - cst[b])
        S = -(-T // lsel)
        if nc == 0:
            continue
        vis = torch.from_numpy(~am[:T, :nc])
        has = vis.any(dim=1)
        pg = np.zeros((T, N2, nc))
        for h in range(N1):
            g = h // G
            qb = qf[s:s + T, h]
            kb = kf[cst[b]:cst[b] + nc, g]
            vb = vf[cst[b]:cst[b] + nc, g]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qb[None, None], kb[None, None], vb[None, None], attn_mask=vis[None, None],
                scale=scale)[0, 0]
            got = torch.from_numpy(res["out"][s:s + T, h])
            torch.testing.assert_close(got[has], ref[has], rtol=1e-12, atol=1e-13)
            assert torch.all(got[~has] == 0)
            assert np.all(np.isneginf(res["max"][s:s + T, h][~has.numpy()]))
            assert np.all(res["sum"][s:s + T, h][~has.numpy()] == 0)
            sc = torch.where(vis, scale * (qb @ kb.T), torch.tensor(-float("inf"), dtype=torch.float64))
            P = torch.softmax(sc, dim=1)
            P = torch.where(has[:, None], P, torch.zeros_like(P)).numpy()
            pg[:, g] += P
        n_full_rows += int(has.sum())
        n_empty += int((~has).sum())
        for t in range(T):
            for g in range(N2):
                for j in range(S):
                    ref = sum(pg[t, g, R * j - m - n] for m in range(R) for n in range(L2)
                              if 0 <= R * j - m - n < nc)
                    assert abs(res["pslc"][s + t, g, j] - ref) <= 1e-12 * max(1.0, ref)
    assert n_full_rows > 100 and n_empty >= 3


def test_topk_mask_matches_brute_force():
    """An explicit topk_mask: the candidates of row t are the j < ceil(T/l')
    with topk_mask[t, j] false; the picks are a full numpy sort of their
    float32 scores (descending, ties to the lower j), -1 padded."""
    lens = [200, 70]
    N1, N2, D1, D2, l, d, lsel, count = 4, 2, 16, 8, 32, 16, 16, 4
    q, kc, vc, _, tm = _mask_case(22, lens, N1, N2, D1, D2, l, d, lsel)
    actq = np.cumsum(lens).astype(np.int64)
    res = oracle.attention(q, np.arange(sum(lens), dtype=np.int64), kc, vc, actq,
                           oracle.cmp_prefix(lens, l, d), N1, N2, 0.3, l, d, lsel, count,
                           topk_mask=tm)
    short = 0
    for s, T in zip(starts_of(lens), lens):
        S = -(-T // lsel)
        for t in range(T):
            cand = np.array([j for j in range(S) if not tm[t, j]], dtype=np.int64)
            short += len(cand) < count
            for g in range(N2):
                keys = res["pslc"][s + t, g, cand].astype(np.float32)
                order = cand[np.lexsort((cand, -keys))]
                expect = np.full(count, -1, dtype=np.int32)
                expect[:min(count, len(order))] = order[:count]
                assert np.array_equal(res["topk"][s + t, g], expect), (s + t, g)
    assert short > 0


def test_masks_that_spell_the_positional_rules_change_nothing():
    """Masks built from the positional rules (block i masked iff
    i*d + l - 1 > t, select block j iff j*l' > t), with extra rows and
    columns, reproduce the mask-free results exactly: the mask is indexed
    (query position, column) and true means masked out."""
    lens = [150, 33, 260]
    N1, N2, D1, D2, l, d, lsel, count = 4, 1, 16, 8, 32, 16, 64, 3
    q, kc, vc = _attention_case(23, lens, N1, N2, D1, D2, l, d)
    actq = np.cumsum(lens).astype(np.int64)
    actc = oracle.cmp_prefix(lens, l, d)
    rows, cols = max(lens) + 4, int(actc[-1]) + 3
    t = np.arange(rows)[:, None]
    am = np.arange(cols)[None, :] * d + l - 1 > t
    tm = np.arange(cols)[None, :] * lsel > t
    tok = np.arange(sum(lens), dtype=np.int64)
    a = oracle.attention(q, tok, kc, vc, actq, actc, N1, N2, 0.3, l, d, lsel, count)
    b = oracle.attention(q, tok, kc, vc, actq, actc, N1, N2, 0.3, l, d, lsel, count,
                         atten_mask=am, topk_mask=tm)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    # a mask without a column for every compressed entry is refused
    with pytest.raises(ValueError):
        oracle.attention(q, tok, kc, vc, actq, actc, N1, N2, 0.3, l, d, lsel, count,
                         atten_mask=am[:, :2])


# --------------------------------------------------------------------------
# Selected-block attention (consumer of the top-k indices; interface of
# "lite_boost.ops.rain_fusion_attention").  Reading: token t, head h of
# group g attends to the raw keys s <= t of its sequence whose block
# floor(s / l') is listed in topk[t, g]; -1, out-of-range entries and
# repeats add nothing; no key -> output 0, lse -inf.
# --------------------------------------------------------------------------

def _sel_case(seed, lens, N1, N2, D1, D2, lsel, count, p_empty=0.05):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    q = rand_bf16(rng, (T, N1, D1))
    k = rand_bf16(rng, (T, N2, D1))
    v = rand_bf16(rng, (T, N2, D2))
    topk = np.full((T, N2, count), -1, dtype=np.int32)
    for s0, Tb in zip(starts_of(lens), lens):
        S = -(-Tb // lsel)
        for t in range(Tb):
            for g in range(N2):
                if rng.random() < p_empty:
                    continue
                n = int(rng.integers(1, count + 1))
                topk[s0 + t, g, :n] = rng.integers(0, S, n)   # repeats allowed, any order
    return q, k, v, topk


def test_select_attention_matches_torch_sdpa():
    """Rows against torch SDPA (float64) with the boolean mask 'key s <= t and
    block(s) listed'; lse against torch.logsumexp of the masked scores;
    rows with no key give 0 and -inf."""
    lens = [130, 77, 200]
    N1, N2, D1, D2, lsel, count = 4, 2, 16, 8, 32, 4
    scale = 0.35
    q, k, v, topk = _sel_case(40, lens, N1, N2, D1, D2, lsel, count)
    res = oracle.select_attention(q, k, v, topk, np.cumsum(lens), N1, N2, scale, lsel)
    qf, kf, vf = (widen_torch(a, "bf16") for a in (q, k, v))
    G = N1 // N2
    n_rows = n_empty = 0
    for s0, Tb in zip(starts_of(lens), lens):
        S = -(-Tb // lsel)
        t = np.arange(Tb)[:, None]
        s = np.arange(Tb)[None, :]
        for g in range(N2):
            sel = np.zeros((Tb, S), dtype=bool)
            for tt in range(Tb):
                for j in topk[s0 + tt, g]:
                    if 0 <= j < S:
                        sel[tt, j] = True
            mask = torch.from_numpy((s <= t) & sel[np.arange(Tb)[:, None], s // lsel])
            has = mask.any(dim=1)
            for hh in range(G):
                h = g * G + hh
                qb, kb, vb = qf[s0:s0 + Tb, h], kf[s0:s0 + Tb, g], vf[s0:s0 + Tb, g]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qb[None, None], kb[None, None], vb[None, None], attn_mask=mask[None, None],
                    scale=scale)[0, 0]
                got = torch.from_numpy(res["out"][s0:s0 + Tb, h])
                torch.testing.assert_close(got[has], ref[has], rtol=1e-12, atol=1e-13)
                assert torch.all(got[~has] == 0)
                sc = torch.where(mask, scale * (qb @ kb.T), torch.tensor(-float("inf"), dtype=torch.float64))
                lse = torch.logsumexp(sc, dim=1)
                gl = torch.from_numpy(res["lse"][s0:s0 + Tb, h])
                torch.testing.assert_close(gl[has], lse[has], rtol=1e-13, atol=1e-13)
                assert torch.all(torch.isneginf(gl[~has]))
            n_rows += int(has.sum())
            n_empty += int((~has).sum())
    assert n_rows > 500 and n_empty > 5


def test_select_attention_all_blocks_is_causal_attention():
    """Listing every block reduces to plain causal attention over the raw
    keys (torch SDPA with is_causal=True)."""
    lens = [150, 64]
    N1, N2, D1, D2, lsel = 4, 1, 16, 16, 32
    rng = np.random.default_rng(41)
    T = sum(lens)
    q, k, v = rand_bf16(rng, (T, N1, D1)), rand_bf16(rng, (T, N2, D1)), rand_bf16(rng, (T, N2, D2))
    S_max = max(-(-Tb // lsel) for Tb in lens)
    topk = np.tile(np.arange(S_max, dtype=np.int32)[::-1], (T, N2, 1))   # any order, every block
    res = oracle.select_attention(q, k, v, topk, np.cumsum(lens), N1, N2, 0.25, lsel)
    qf, kf, vf = (widen_torch(a, "bf16") for a in (q, k, v))
    for s0, Tb in zip(starts_of(lens), lens):
        for h in range(N1):
            ref = torch.nn.functional.scaled_dot_product_attention(
                qf[s0:s0 + Tb, h][None, None], kf[s0:s0 + Tb, 0][None, None],
                vf[s0:s0 + Tb, 0][None, None], is_causal=True, scale=0.25)[0, 0]
            torch.testing.assert_close(torch.from_numpy(res["out"][s0:s0 + Tb, h]), ref,
                                       rtol=1e-12, atol=1e-13)


def test_select_attention_identical_keys_closed_form():
    """Identical keys: uniform weights over the selected visible keys, so the
    output is their mean value and lse = scale*<q,k> + log(count of keys)."""
    lens = [300]
    N1, N2, D1, D2, lsel, count = 2, 1, 8, 4, 64, 2
    rng = np.random.default_rng(42)
    q = rand_bf16(rng, (300, N1, D1))
    k1 = oracle.bf16_to_f64(rand_bf16(rng, (D1,)))
    k = bits(np.broadcast_to(k1, (300, N2, D1)))
    v = rand_bf16(rng, (300, N2, D2))
    topk = np.full((300, N2, count), -1, dtype=np.int32)
    topk[:, 0, 0] = np.arange(300) // lsel          # own block
    topk[:, 0, 1] = 0                               # and the first
    res = oracle.select_attention(q, k, v, topk, lens, N1, N2, 0.5, lsel)
    qf, vf = oracle.bf16_to_f64(q), oracle.bf16_to_f64(v)
    for t in range(300):
        keys = [s for s in range(t + 1) if s // lsel in (t // lsel, 0)]
        for h in range(N1):
            np.testing.assert_allclose(res["out"][t, h], vf[keys, 0].mean(axis=0), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(res["lse"][t, h], 0.5 * qf[t, h] @ k1 + np.log(len(keys)),
                                       rtol=1e-12)


def test_select_attention_ignores_repeats_padding_and_out_of_range():
    """-1, repeats and indices past the sequence's last block change nothing."""
    lens = [200]
    N1, N2, D1, D2, lsel, count = 4, 2, 16, 8, 32, 6
    q, k, v, topk = _sel_case(43, lens, N1, N2, D1, D2, lsel, 3, p_empty=0.0)
    clean = np.full((200, N2, count), -1, dtype=np.int32)
    clean[:, :, :3] = topk
    noisy = clean.copy()
    noisy[:, :, 3] = topk[:, :, 0]                     # a repeat
    noisy[:, :, 4] = 7 + 100                           # past the last block (7)
    noisy[:, :, 5] = -5                                # negative
    a = oracle.select_attention(q, k, v, clean, lens, N1, N2, 0.3, lsel)
    b = oracle.select_attention(q, k, v, noisy, lens, N1, N2, 0.3, lsel)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


# --------------------------------------------------------------------------
# Backward (training use; the pages give no formulas): gradients of the
# compressed attention output and of the compression, against torch
# autograd of the forward written out in float64.
# --------------------------------------------------------------------------

def test_attention_backward_matches_torch_autograd():
    lens = [90, 41, 130]
    N1, N2, D1, D2, l, d = 6, 2, 16, 8, 32, 16
    scale = -0.3                                   # a negative scale too
    rng = np.random.default_rng(50)
    q, kc, vc = _attention_case(50, lens, N1, N2, D1, D2, l, d)
    do = rand_bf16(rng, (sum(lens), N1, D2))
    actq, actc = np.cumsum(lens), oracle.cmp_prefix(lens, l, d)
    res = oracle.attention_backward(q, kc, vc, do, actq, actc, N1, N2, scale, l, d)
    qf, kf, vf, dof = (widen_torch(a, "bf16").clone().requires_grad_(True) for a in (q, kc, vc, do))
    cst = np.concatenate([[0], actc[:-1]])
    G = N1 // N2
    loss = torch.zeros((), dtype=torch.float64)
    for b, (s0, T) in enumerate(zip(starts_of(lens), lens)):
        nc = int(actc[b] - cst[b])
        if nc == 0:
            continue
        t = torch.arange(T)[:, None]
        i = torch.arange(nc)[None, :]
        mask = (i * d + l - 1) <= t
        has = mask.any(dim=1)
        for h in range(N1):
            g = h // G
            sc = scale * (qf[s0:s0 + T, h] @ kf[cst[b]:cst[b] + nc, g].T)
            sc = torch.where(mask, sc, torch.tensor(-float("inf"), dtype=torch.float64))
            p = torch.softmax(sc[has], dim=1)
            out = p @ vf[cst[b]:cst[b] + nc, g]
            loss = loss + (out * dof.detach()[s0:s0 + T, h][has]).sum()
    loss.backward()
    np.testing.assert_allclose(res["dq"], qf.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["dkc"], kf.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["dvc"], vf.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.abs(res["dkc"]).max() > 0.1 and np.abs(res["dq"]).max() > 0.1


def test_compress_backward_matches_torch_autograd():
    rng = np.random.default_rng(51)
    l, d, N, D = 32, 16, 2, 8
    lens = [140, 33, 70]
    x = rand_bf16(rng, (sum(lens), N, D))
    w = rand_bf16(rng, (l, N), std=0.1)
    T2 = int(oracle.cmp_prefix(lens, l, d)[-1])
    dy = rng.standard_normal((T2, N, D))
    res = oracle.compress_backward(x, w, dy, np.cumsum(lens), l, d)
    xf = widen_torch(x, "bf16").clone().requires_grad_(True)
    wf = widen_torch(w, "bf16").clone().requires_grad_(True)
    ys = []
    for s0, T in zip(starts_of(lens), lens):
        for i in range(oracle.n_cmp(T, l, d)):
            ys.append(torch.einsum("pn,pnd->nd", wf, xf[s0 + i * d:s0 + i * d + l]))
    y = torch.stack(ys)
    (y * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(res["dx"], xf.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res["dw"], wf.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_backward_finite_differences():
    """Central differences of <attention_out, dout> in float64 along a few
    random directions of q, kc and vc match the oracle's gradients."""
    lens = [70]
    N1, N2, D1, D2, l, d, lsel = 2, 1, 8, 4, 32, 16, 64
    rng = np.random.default_rng(52)
    q, kc, vc = _attention_case(52, lens, N1, N2, D1, D2, l, d)
    do = rand_bf16(rng, (70, N1, D2))
    actq, actc = np.array([70]), oracle.cmp_prefix(lens, l, d)
    g = oracle.attention_backward(q, kc, vc, do, actq, actc, N1, N2, 0.5, l, d)
    dof = oracle.bf16_to_f64(do)
    base = [oracle.bf16_to_f64(a) for a in (q, kc, vc)]

    def f(qv, kv, vv):
        # the forward in float64 from float64 inputs: softmax over visible blocks
        tot = 0.0
        for t in range(70):
            nv = n_vis_of(t, l, d, kv.shape[0])
            for h in range(N1):
                if nv == 0:
                    continue
                sc = 0.5 * kv[:nv, 0] @ qv[t, h]
                pr = np.exp(sc - sc.max())
                pr /= pr.sum()
                tot += (pr @ vv[:nv, 0]) @ dof[t, h]
        return tot

    eps = 1e-5
    for which, key in enumerate(["dq", "dkc", "dvc"]):
        direction = rng.standard_normal(base[which].shape)
        plus = list(base); minus = list(base)
        plus[which] = base[which] + eps * direction
        minus[which] = base[which] - eps * direction
        fd = (f(*plus) - f(*minus)) / (2 * eps)
        assert abs(fd - float((g[key] * direction).sum())) <= 1e-6 * max(1.0, abs(fd)), key


def test_chunked_prefill_rows_equal_full_prefill_rows():
    """Chunked prefill (queries = the last Tq of Tkv key/value tokens, both
    causal rules aligned bottom-right) is the full prefill restricted to
    those rows: every output of a chunked query equals, bit for bit, the
    full-sequence output of the token at the same position.  And Tkv = Tq
    is the plain call."""
    rng = np.random.default_rng(2024)
    N1, N2, D1, D2, l, d, lsel, count, scale = 4, 2, 32, 32, 32, 16, 64, 4, 0.2
    kv_lens = [300, 181]
    q_lens = [77, 181]          # a chunk at the end of the first sequence, all of the second
    kc_all, vc_all, q_full = [], [], []
    for T in kv_lens:
        k = rand_bf16(rng, (T, N2, D1))
        v = rand_bf16(rng, (T, N2, D2))
        w = rand_bf16(rng, (l, N2), std=0.05)
        kc_all.append(oracle.round_to(oracle.compress(k, w, np.array([T]), l, d)))
        vc_all.append(oracle.round_to(oracle.compress(v, w, np.array([T]), l, d)))
        q_full.append(rand_bf16(rng, (T, N1, D1)))
    kc = np.concatenate(kc_all)
    vc = np.concatenate(vc_all)
    actc = oracle.cmp_prefix(kv_lens, l, d)
    full = oracle.attention(np.concatenate(q_full), np.arange(sum(kv_lens), dtype=np.int64), kc, vc,
                            np.cumsum(kv_lens), actc, N1, N2, scale, l, d, lsel, count)
    q_chunk = np.concatenate([qf[T - Tq:] for qf, T, Tq in zip(q_full, kv_lens, q_lens)])
    chunk = oracle.attention(q_chunk, np.arange(sum(q_lens), dtype=np.int64), kc, vc, np.cumsum(q_lens),
                             actc, N1, N2, scale, l, d, lsel, count, act_seq_kvlen=np.cumsum(kv_lens))
    rows = np.concatenate([s + np.arange(T - Tq, T) for s, T, Tq in zip(starts_of(kv_lens), kv_lens, q_lens)])
    for key in ("out", "max", "sum", "pslc", "topk"):
        assert np.array_equal(chunk[key], full[key][rows], equal_nan=True), key
    # the first chunk row of sequence 0 (position 223) sees blocks that a
    # top-left alignment (position 0) would not: the alignment matters
    assert np.isfinite(chunk["max"][0]).all()
    same = oracle.attention(q_chunk, np.arange(sum(q_lens), dtype=np.int64), kc, vc, np.cumsum(q_lens),
                            actc, N1, N2, scale, l, d, lsel, count, act_seq_kvlen=np.cumsum(q_lens))
    plain = oracle.attention(q_chunk, np.arange(sum(q_lens), dtype=np.int64), kc, vc, np.cumsum(q_lens),
                             actc, N1, N2, scale, l, d, lsel, count)
    for key in ("out", "max", "sum", "pslc", "topk"):
        assert np.array_equal(same[key], plain[key], equal_nan=True), key


def test_chunked_select_attention_rows_equal_full_prefill_rows():
    """Selected-block attention with chunked prefill (queries = the last Tq
    of Tkv key/value tokens, key s visible to query t iff s <= Tkv - Tq + t)
    is the full-sequence computation restricted to those rows, bit for bit,
    given the same block lists."""
    rng = np.random.default_rng(77)
    N1, N2, D1, D2, lsel, count, scale = 4, 2, 32, 32, 32, 3, 0.2
    kv_lens, q_lens = [250, 96], [70, 96]
    T = sum(kv_lens)
    k = rand_bf16(rng, (T, N2, D1))
    v = rand_bf16(rng, (T, N2, D2))
    q_full = rand_bf16(rng, (T, N1, D1))
    lists = np.empty((T, N2, count), dtype=np.int32)
    for s0, Tb in zip(starts_of(kv_lens), kv_lens):
        S = -(-Tb // lsel)
        lists[s0:s0 + Tb] = rng.integers(-1, S + 1, (Tb, N2, count))
    full = oracle.select_attention(q_full, k, v, lists, np.cumsum(kv_lens), N1, N2, scale, lsel)
    rows = np.concatenate([s + np.arange(Tb - Tq, Tb) for s, Tb, Tq in zip(starts_of(kv_lens), kv_lens, q_lens)])
    chunk = oracle.select_attention(np.ascontiguousarray(q_full[rows]), k, v, np.ascontiguousarray(lists[rows]),
                                    np.cumsum(q_lens), N1, N2, scale, lsel, act_seq_kvlen=np.cumsum(kv_lens))
    for key in ("out", "lse"):
        assert np.array_equal(chunk[key], full[key][rows], equal_nan=True), key
    # the rows sit at the end of a 250-token sequence: a top-left alignment
    # (query t at position t) would see far fewer keys and differ
    assert not np.array_equal(chunk["lse"][:5], full["lse"][:5])


def test_chunked_backward_equals_full_prefill_with_zero_gradient_elsewhere():
    """The backward with chunked prefill equals the full-sequence backward
    whose output gradient is zero on every row outside the chunk: such rows
    add exact zeros to d_key and d_value (dP = 0 and Delta = 0 there), so
    d_key, d_value and the chunk's d_query agree bit for bit."""
    rng = np.random.default_rng(78)
    N1, N2, D1, D2, l, d, scale = 4, 2, 32, 32, 32, 16, 0.3
    kv_lens, q_lens = [260, 130], [90, 1]
    T = sum(kv_lens)
    kc_all, vc_all = [], []
    for Tb in kv_lens:
        n = oracle.n_cmp(Tb, l, d)
        kc_all.append(rand_bf16(rng, (n, N2, D1)))
        vc_all.append(rand_bf16(rng, (n, N2, D2)))
    kc, vc = np.concatenate(kc_all), np.concatenate(vc_all)
    actc = oracle.cmp_prefix(kv_lens, l, d)
    q_full = rand_bf16(rng, (T, N1, D1))
    rows = np.concatenate([s + np.arange(Tb - Tq, Tb) for s, Tb, Tq in zip(starts_of(kv_lens), kv_lens, q_lens)])
    dout_full = np.zeros((T, N1, D2), dtype=np.uint16)       # bf16 +0
    dout_full[rows] = rand_bf16(rng, (len(rows), N1, D2))
    full = oracle.attention_backward(q_full, kc, vc, dout_full, np.cumsum(kv_lens), actc, N1, N2, scale, l, d)
    chunk = oracle.attention_backward(np.ascontiguousarray(q_full[rows]), kc, vc,
                                      np.ascontiguousarray(dout_full[rows]), np.cumsum(q_lens), actc, N1, N2,
                                      scale, l, d, act_seq_kvlen=np.cumsum(kv_lens))
    assert np.array_equal(chunk["dq"], full["dq"][rows])
    assert np.array_equal(chunk["dkc"], full["dkc"]) and np.array_equal(chunk["dvc"], full["dvc"])
    assert np.abs(chunk["dkc"]).sum() > 0 and np.abs(chunk["dvc"]).sum() > 0
