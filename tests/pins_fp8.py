"""Checks that pin the FP8 part of the oracle (oracle/fp8.py) to facts outside
itself: the E4M3 format's definition (bias 7, 3 mantissa bits, subnormals,
largest finite 448, NaN at S.1111.111, round to nearest even), Hadamard
algebra, exact-arithmetic identities of the quantisation, the plain attention
definition, and a hand-computed online-softmax example.

Each check takes the fp8 module (and the plain oracle for the attention
identities), so that tests/test_oracle_fp8_mutations.py can run them against
broken copies.  [P2] is 为什么Flash Attention能将注意力计算提速数倍而不损失精度,
whose Flash Attention 3 section names the FP8 forward and incoherent processing.
"""
from __future__ import annotations

import math

import numpy as np

import oracle


def _finite_codes(f):
    codes = np.arange(256, dtype=np.uint8)
    vals = f.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    return codes[ok], vals[ok]


# ------------------------------------------------------------ the format

def check_e4m3_closed_forms(f):
    """Values of named codes from the format's fields: value = (-1)^s (1 + m/8)
    2^(e - 7) for e >= 1, (-1)^s m 2^-9 for e = 0; S.1111.111 is NaN."""
    cases = {
        0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x09: 1.125 * 2.0 ** -6,
        0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x44: 3.0, 0x48: 4.0,
        0x70: 128.0, 0x77: 1.875 * 2.0 ** 7, 0x78: 256.0, 0x7E: 448.0,
        0x81: -(2.0 ** -9), 0xB8: -1.0, 0xFE: -448.0,
    }
    for code, want in cases.items():
        got = float(f.e4m3_decode(np.array([code], dtype=np.uint8))[0])
        assert got == want, (hex(code), got, want)
    nan = f.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(nan).all()
    z = f.e4m3_decode(np.array([0x80], dtype=np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0
    # 254 finite codes; the 127 non-negative magnitudes strictly increase
    codes, vals = _finite_codes(f)
    assert codes.size == 254
    pos = f.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6
    # between binades the spacing is 2^(e-3); subnormals are 2^-9 apart
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9, rtol=0, atol=0)


def check_e4m3_round_trip(f):
    """Encoding a code's own value gives the code back (both zeros kept)."""
    codes, vals = _finite_codes(f)
    back = f.e4m3_encode(vals)
    assert np.array_equal(back, codes), np.nonzero(back != codes)


def check_e4m3_nearest_even_brute_force(f):
    """For random values and for every midpoint between neighbours, the code is
    the nearest finite value by exhaustive search, ties to the even mantissa."""
    codes, vals = _finite_codes(f)
    rng = np.random.default_rng(11)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 4000))
    xs = np.concatenate([mags * rng.choice([-1.0, 1.0], mags.size), rng.uniform(-448, 448, 2000),
                         rng.uniform(-2.0 ** -6, 2.0 ** -6, 1000)])
    pos = f.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    xs = np.concatenate([xs, mids, -mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    got = f.e4m3_encode(xs)
    gv = f.e4m3_decode(got)
    for x, c, v in zip(xs, got, gv):
        dist = np.abs(vals - x)
        best = dist.min()
        assert abs(v - x) == best, (x, v)
        cands = codes[dist == best]
        if cands.size > 1:
            nonzero = [cc for cc in cands if (cc & 0x7F) != 0]
            even = [cc for cc in cands if (cc & 1) == 0]
            assert (c & 1) == 0 and c in even, (x, hex(c), [hex(e) for e in cands])
            del nonzero
    # the midpoints themselves go to the even neighbour
    lo = np.arange(126)
    even_side = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(f.e4m3_encode(mids).astype(np.int64), even_side)


def check_e4m3_range_limits(f):
    """448 is the largest finite value; 464 (the midpoint to the absent 480)
    ties to 448's even mantissa; anything rounding higher, inf or NaN is refused."""
    assert f.e4m3_encode(np.array([464.0]))[0] == 0x7E
    assert f.e4m3_encode(np.array([-464.0]))[0] == 0xFE
    for bad in (np.nextafter(464.0, np.inf), 500.0, np.inf, np.nan):
        try:
            f.e4m3_encode(np.array([bad]))
        except ValueError:
            continue
        raise AssertionError(f"{bad} was encoded")
    # values below half the smallest subnormal round to zero, with their sign
    z = f.e4m3_encode(np.array([2.0 ** -10, -(2.0 ** -10), 2.0 ** -11]))
    assert list(z) == [0x00, 0x80, 0x00]
    assert f.e4m3_encode(np.array([np.nextafter(2.0 ** -10, 1.0)]))[0] == 0x01


# ---------------------------------------------------- incoherent processing

def check_hadamard_algebra(f):
    """H_2 = [[1, 1], [1, -1]], H H^T = d I, and the butterfly equals the
    matrix product exactly on integers, for d = 64 and 128."""
    assert np.array_equal(f.hadamard_matrix(2), np.array([[1.0, 1.0], [1.0, -1.0]]))
    rng = np.random.default_rng(5)
    for d in (2, 8, 64, 128):
        h = f.hadamard_matrix(d)
        assert np.array_equal(h @ h.T, d * np.eye(d))
        # Sylvester order: entry (i, j) = (-1)^popcount(i & j)
        i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
        par = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
        assert np.array_equal(h, np.where(par, -1.0, 1.0))
        x = rng.integers(-50, 51, size=(6, d)).astype(np.float64)
        assert np.array_equal(f.fwht(x, np.float64), x @ h)
        # small integers stay exact in fp32 too; applying the transform twice gives d x
        assert np.array_equal(f.fwht(x, np.float32).astype(np.float64), x @ h)
        assert np.array_equal(f.fwht(f.fwht(x, np.float64), np.float64), d * x)


def check_fwht_fp32_butterfly_order(f):
    """The fp32 transform takes its rounding from the stated butterfly order
    (widths 1, 2, 4, ...): evaluated one pair at a time in np.float32 scalars
    on random non-integers, the result agrees bit for bit."""
    rng = np.random.default_rng(9)
    for d in (64, 128):
        x = rng.normal(size=(3, d)).astype(np.float32)
        got = f.fwht(x, np.float32)
        for r in range(3):
            y = [np.float32(t) for t in x[r]]
            w = 1
            while w < d:
                for i in range(d):
                    if i & w == 0:
                        a, b = y[i], y[i + w]
                        y[i], y[i + w] = np.float32(a + b), np.float32(a - b)
                w *= 2
            assert np.array_equal(np.array(y, dtype=np.float32), got[r])


def check_rotation_preserves_scores(f):
    """Incoherent processing keeps the score product: with y = (sigma o x) H
    for both operands, y_q . y_k = d (q . k) exactly (integer inputs)."""
    rng = np.random.default_rng(3)
    d = 128
    bits = int(rng.integers(0, 2 ** 62)) | (int(rng.integers(0, 2 ** 62)) << 64)
    sig = f.sign_vector(bits, d).astype(np.float64)
    assert set(np.unique(sig)) <= {-1.0, 1.0}
    assert all((sig[c] < 0) == bool((bits >> c) & 1) for c in range(d))
    q = rng.integers(-20, 21, size=(5, d)).astype(np.float64)
    k = rng.integers(-20, 21, size=(7, d)).astype(np.float64)
    yq = f.fwht(q * sig, np.float64)
    yk = f.fwht(k * sig, np.float64)
    assert np.array_equal(yq @ yk.T, d * (q @ k.T))


# ------------------------------------------------------------ quantisation

def _bf16_grid(x):
    """Round to the nearest bf16 value (so the inputs are what the GPU reads)."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def check_quantize_scaling(f):
    """amax is the head's largest |y|; that element becomes +-448 exactly;
    doubling the input keeps every code and doubles amax and the descale
    (power-of-two scaling is exact in fp32); a zero head gives zero codes and
    a zero descale; the dequantised values lie within half a code step."""
    rng = np.random.default_rng(21)
    x = _bf16_grid(rng.normal(size=(2, 3, 40, 64)) * 3)
    x[1, 2] = 0.0
    for rotate in (False, True):
        codes, amax, desc = f.quantize_heads(x, rotate=rotate, sign_bits=0x5A5A_1234)
        y = x.astype(np.float32)
        if rotate:
            y = f.fwht(y * f.sign_vector(0x5A5A_1234, 64), np.float32)
        assert np.array_equal(amax, np.abs(y).reshape(2, 3, -1).max(axis=-1))
        assert amax[1, 2] == 0 and desc[1, 2] == 0 and not codes[1, 2].any()
        for b in range(2):
            for h in range(3):
                if amax[b, h] == 0:
                    continue
                flat = np.abs(y[b, h]).ravel()
                i = int(np.argmax(flat))
                assert f.e4m3_decode(codes[b, h].ravel()[i:i + 1])[0] in (448.0, -448.0)
        c2, a2, d2 = f.quantize_heads(2 * x, rotate=rotate, sign_bits=0x5A5A_1234)
        assert np.array_equal(c2, codes) and np.array_equal(a2, 2 * amax) and np.array_equal(d2, 2 * desc)
        deq = f.dequantize_heads(codes, desc)
        unit = desc.astype(np.float64) * (np.sqrt(64) if rotate else 1.0)   # descale of the unrotated y
        yy = y.astype(np.float64) / (np.sqrt(64) if rotate else 1.0)
        tol = np.maximum(2.0 ** -4 * np.abs(yy), 2.0 ** -10 * (unit * (1 / np.sqrt(64) if rotate else 1.0))[:, :, None, None])
        assert np.all(np.abs(deq - yy) <= tol * (1 + 1e-6) + 1e-12)


def check_quantize_tiny_heads(f):
    """A head of bf16 subnormals: 448 / amax would overflow fp32, so amax is
    raised to 2^-117; every code is finite, the largest |y| maps to
    448 * amax / 2^-117 (a power-of-two step below 448), and the dequantised
    values lie within one code step of y.  A head at 2^-117 or above is not
    affected by the floor (scaling by 2^k keeps its codes)."""
    x = np.zeros((1, 2, 8, 64), dtype=np.float32)
    x[0, 0] = np.float32(2.0 ** -130) * np.arange(1, 513, dtype=np.float32).reshape(8, 64) / 512
    x[0, 1] = np.float32(2.0 ** -100) * np.arange(1, 513, dtype=np.float32).reshape(8, 64) / 512
    codes, amax, desc = f.quantize_heads(x)
    assert amax[0, 0] == np.float32(2.0 ** -117) and amax[0, 1] == np.float32(2.0 ** -100)
    assert np.all(np.isfinite(f.e4m3_decode(codes)))
    deq = f.dequantize_heads(codes, desc)
    step = 2.0 ** -3 * np.abs(x.astype(np.float64)) + desc.astype(np.float64)[:, :, None, None] * 2.0 ** -9
    assert np.all(np.abs(deq - x) <= step)
    top = f.e4m3_decode(codes[0, 0].ravel()[-1:])[0]
    assert top == 448.0 * 2.0 ** -13          # 2^-130 * 448 / 2^-117, exact in E4M3
    c2, _, _ = f.quantize_heads(x * np.float32(2.0 ** 20))
    assert np.array_equal(c2[0, 1], codes[0, 1])


def check_rotation_reduces_outlier_error(f):
    """The purpose stated on the page: with outlier channels shared by Q and K
    (two of 128 channels 20 times larger in both), quantising after the
    rotation gives scores closer to the exact ones than quantising directly.
    E4M3's error is relative, so the score error is about 2^-4 times the
    root of sum_c (q_c k_c)^2; coherent outliers concentrate that sum in a
    few channels and the rotation spreads it (seeded data)."""
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 1, 256, 128
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    for t in (q, k):
        t[..., [5, 77]] *= 20.0
    q, k = _bf16_grid(q), _bf16_grid(k)
    exact = q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T
    errs = {}
    for rotate in (False, True):
        cq, _, dq = f.quantize_heads(q, rotate, 0x1357_9BDF_2468_ACE0)
        ck, _, dk = f.quantize_heads(k, rotate, 0x1357_9BDF_2468_ACE0)
        s = f.dequantize_heads(cq, dq)[0, 0] @ f.dequantize_heads(ck, dk)[0, 0].T
        errs[rotate] = float(np.sqrt(np.mean((s - exact) ** 2)) / np.sqrt(np.mean(exact ** 2)))
    assert errs[True] * 2 < errs[False], errs


# ------------------------------------------------------------- attention

def check_fp8_attention_without_rounding_is_plain(f):
    """With the E4M3 step left out, the blocked running-maximum recurrence is
    the plain attention definition (causal, non-causal, ragged N)."""
    rng = np.random.default_rng(31)
    for N, causal in ((1, False), (70, True), (200, False), (129, True)):
        q, k, v = (rng.normal(size=(1, 2, N, 16)) for _ in range(3))
        o_ref, l_ref = oracle.attention(q, k, v, 0.3, causal)
        o, l = f.attention_fp8(q, k, v, 0.3, causal, round_p=False)
        assert np.abs(o - o_ref).max() < 1e-12 and np.abs(l - l_ref).max() < 1e-12


def check_fp8_attention_hand_example(f):
    """One query, keys with scores 0 and -ln 3 in the same block: P = (1, 1/3),
    E4M3(1/3) = 11/32 = 0.34375, so O = (v0 + 0.34375 v1) / (4/3) and
    LSE = ln(4/3).  With the second key 64 positions later (the next block)
    and score +ln 3, the running maximum moves: the first key's weight is
    carried by the exact factor 1/3 and the new key has P = 1, so O is the
    exact softmax average (v0/3 + v1) / (4/3)."""
    d = 4
    v = np.zeros((2, d))
    v[0] = [1.0, 0.0, 2.0, -1.0]
    v[1] = [0.0, 1.0, -2.0, 4.0]
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k = np.zeros((2, d))
    k[1, 0] = -math.log(3.0)
    o, lse = f.attention_fp8_head_rows(q, k, v, 1.0, False, [0])
    want = (v[0] + 0.34375 * v[1]) / (4.0 / 3.0)
    assert np.allclose(o[0], want, rtol=0, atol=1e-15), (o, want)
    assert abs(lse[0] - math.log(4.0 / 3.0)) < 1e-15
    # same two keys, the second one block later and larger
    k2 = np.zeros((65, d))
    v2 = np.zeros((65, d))
    v2[0], v2[64] = v[0], v[1]
    k2[64, 0] = math.log(3.0)
    k2[1:64, 0] = -1e9                      # other keys carry no weight
    o2, lse2 = f.attention_fp8_head_rows(q, k2, v2, 1.0, False, [0])
    want2 = (v[0] / 3.0 + v[1]) / (4.0 / 3.0)
    assert np.allclose(o2[0], want2, rtol=0, atol=1e-15), (o2, want2)
    assert abs(lse2[0] - (math.log(3.0) + math.log(4.0 / 3.0))) < 1e-14


def check_fp8_attention_bounds(f):
    """Dominant key: O is that key's V row exactly (its P is 1, every other P
    rounds to 0).  Random rows: |O - O_plain| <= sum_j max(2^-4 w_j,
    2^-10 / l) |v_j| (one E4M3 rounding per term, relative 2^-4 or absolute
    2^-10), and the LSE does not see the rounding at all."""
    rng = np.random.default_rng(41)
    N, d = 300, 32
    q, k, v = (rng.normal(size=(N, d)) for _ in range(3))
    k[123] = q[200] * 10.0
    o, _ = f.attention_fp8_head_rows(q, k, v, 1.0, False, [200])
    assert np.array_equal(o[0], v[123])
    rows = np.arange(0, N, 7)
    for causal in (False, True):
        o8, l8 = f.attention_fp8_head_rows(q, k, v, 0.25, causal, rows)
        o0, l0 = f.attention_fp8_head_rows(q, k, v, 0.25, causal, rows, round_p=False)
        assert np.array_equal(l8, l0)
        s = 0.25 * q[rows] @ k.T
        if causal:
            s = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, s)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        lsum = w.sum(axis=1, keepdims=True)
        bound = np.maximum(2.0 ** -4 * w / lsum, 2.0 ** -10 / lsum) @ np.abs(v)
        bound = np.where(np.isfinite(s).any(axis=1)[:, None], bound, 0)
        assert np.all(np.abs(o8 - o0) <= bound + 1e-12)
        assert np.abs(o8 - o0).max() > 0           # the rounding does act


ALL_CHECKS = [check_e4m3_closed_forms, check_e4m3_round_trip, check_e4m3_nearest_even_brute_force,
              check_e4m3_range_limits, check_hadamard_algebra, check_fwht_fp32_butterfly_order,
              check_rotation_preserves_scores, check_quantize_scaling, check_quantize_tiny_heads,
              check_rotation_reduces_outlier_error,
              check_fp8_attention_without_rounding_is_plain, check_fp8_attention_hand_example,
              check_fp8_attention_bounds]
