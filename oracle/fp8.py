"""FP8 forward: the E4M3 format, per-head quantisation with optional
incoherent processing, and attention on the quantised operands.

TEST INFRASTRUCTURE ONLY (see the package docstring for the page keys).

[P2 Flash Attention 3：拥抱Hopper架构, item 3] names an FP8 forward on the
FP8 matrix units, with "incoherent processing" to lower the quantisation
error, and nothing more.  The readings taken here, each the plainest one the
rest of the pages support:

  * Format: OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; subnormals down to 2^-9; the largest finite value is 448; the two
    codes S.1111.111 are NaN and there is no infinity.  Rounding is to the
    nearest representable value, ties to the even mantissa.  A value whose
    rounding would pass 448 is an error here: the quantisation below scales
    every operand into range, and P is at most 1.
  * Granularity: one scale per (batch, head) and tensor.  amax is the largest
    |y| over the head's N x d values, the quantisation multiplier is
    s = 448 / amax (fp32; s = 1 when amax = 0), each code is the E4M3
    rounding of the fp32 product y * s, and the dequantisation factor
    ("descale") is amax / 448 (fp32).  A non-zero amax below 2^-117 is
    raised to 2^-117 first, so that s stays finite (at most 1.75 2^125) for
    heads of tiny values such as bf16 subnormals.
  * Incoherent processing (Q and K only, the two operands of the score
    product): every row is multiplied by a random sign diagonal and by the
    d x d Sylvester-Hadamard matrix H (entries +-1) before the amax is
    taken: y = (sigma o x) H.  H H^T = d I, so the rotation spreads an
    outlier channel over all d channels while (Q' K'^T) / d = Q K^T exactly;
    the 1/sqrt(d) that makes it orthonormal is folded into the descale
    (descale = fp32(amax / 448) * fp32(1 / sqrt(d))), so the dequantised Q'
    and K' are the rotated rows and the score scale is unchanged.
    The transform is the fast Walsh-Hadamard butterfly, stages of width
    1, 2, 4, ... d/2, each pair (a, b) -> (a + b, a - b), in fp32.  The fp32
    rounding of these sums is part of the definition, because the codes are
    integers decided by it.
  * Attention on the quantised operands: the online softmax of
    [P1 在线Softmax] / [P2 在线Softmax技巧] over key blocks of 64, with one
    step added: the block's P = exp(s - m_new), taken against the running
    maximum (so P <= 1 and the largest weight seen so far is exactly 1), is
    rounded to E4M3 before the P V product.  The running sum l adds the
    unrounded P, so the logsumexp keeps fp32-level accuracy; only O carries
    the FP8 rounding of P.  Scores use the dequantised values:
    s_ij = scale * (descale_q q8_i) . (descale_k k8_j).

The integer results (codes, amax) are computed in the fp32 arithmetic the
definition fixes, so that they can be compared bit for bit; the attention is
fp64 on the exact dequantised values.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
AMAX_MIN = 2.0 ** -117       # smallest amax used for a non-zero head
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
FP8_TILE = 64


# ---------------------------------------------------------------- the format

def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * E4M3_MIN_SUBNORMAL, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code of each value, rounded to nearest, ties to even.

    Subnormal range (|x| < 2^-6): the value in units of 2^-9 rounded to an
    integer m in 0..8, code m (m = 8 is the smallest normal, code 8).  Normal
    range: |x| = q 2^(e-3) with q in [8, 16); q is rounded, a carry to 16
    moves to the next binade, code ((e + 7) << 3) | (q - 8).  np.rint rounds
    halves to even, and the scalings by powers of two are exact.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("E4M3 encode: non-finite input")
    a = np.abs(x)
    code = np.zeros(x.shape, dtype=np.int64)
    sub = a < E4M3_MIN_NORMAL
    code[sub] = np.rint(a[sub] / E4M3_MIN_SUBNORMAL).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        _, ex = np.frexp(a[nrm])            # a = f 2^ex, f in [0.5, 1)
        e = ex - 1                          # a in [2^e, 2^(e+1))
        q = np.rint(a[nrm] / np.ldexp(1.0, e - 3)).astype(np.int64)
        carry = q == 16
        e = e + carry
        q = np.where(carry, 8, q)
        biased = e + 7
        if np.any((biased > 15) | ((biased == 15) & (q - 8 == 7))):
            raise ValueError("E4M3 encode: value rounds past 448")
        code[nrm] = (biased << 3) | (q - 8)
    code = code | np.where(np.signbit(x), 128, 0)
    return code.astype(np.uint8)


def e4m3_round(x) -> np.ndarray:
    """x rounded to the nearest E4M3 value (float64)."""
    return e4m3_decode(e4m3_encode(x))


# ---------------------------------------------------- incoherent processing

def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester-Hadamard matrix of order d (a power of two): H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]]; entries +-1, H H^T = d I."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x, dtype=np.float32) -> np.ndarray:
    """Fast Walsh-Hadamard transform of every row (last axis, a power of two)
    in the arithmetic of `dtype`: stages of width w = 1, 2, 4, ..., each pair
    (x[i], x[i + w]) with i & w == 0 becomes (x[i] + x[i + w], x[i] - x[i + w]).
    Equals x @ H (Sylvester order) up to the rounding of the sums."""
    y = np.array(x, dtype=dtype, copy=True)
    d = y.shape[-1]
    lead = y.shape[:-1]
    w = 1
    while w < d:
        v = y.reshape(lead + (d // (2 * w), 2, w))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        y = v.reshape(lead + (d,))
        w *= 2
    return y


def sign_vector(sign_bits: int, d: int) -> np.ndarray:
    """The random sign diagonal: sigma_c = -1 where bit c of sign_bits is set."""
    return np.array([-1.0 if (sign_bits >> c) & 1 else 1.0 for c in range(d)], dtype=np.float32)


# ------------------------------------------------------------ quantisation

def quantize_heads(x, rotate: bool = False, sign_bits: int = 0):
    """Per-(batch, head) E4M3 quantisation of x [B, H, N, d] (values exactly
    representable in fp32, e.g. bf16).

    Returns (codes uint8 [B, H, N, d], amax float32 [B, H] (after the
    2^-117 floor), descale float32 [B, H]).  With `rotate`, each row is first transformed as
    y = fwht(sigma o x) in fp32 (sigma from sign_bits); see the module
    docstring for the scheme.
    """
    x32 = np.asarray(x, dtype=np.float32)
    B, H, N, d = x32.shape
    y = fwht(x32 * sign_vector(sign_bits, d), np.float32) if rotate else x32
    amax = np.abs(y).reshape(B, H, N * d).max(axis=-1).astype(np.float32)
    amax = np.where(amax > 0, np.maximum(amax, np.float32(AMAX_MIN)), amax).astype(np.float32)
    s = np.where(amax > 0, np.float32(E4M3_MAX) / np.where(amax > 0, amax, np.float32(1)),
                 np.float32(1)).astype(np.float32)
    prod = (y * s[:, :, None, None]).astype(np.float32)       # one fp32 product per element
    codes = e4m3_encode(prod)
    descale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    if rotate:
        descale = (descale * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
    return codes, amax, descale


def dequantize_heads(codes, descale) -> np.ndarray:
    """Exact values code * descale, float64 [B, H, N, d]."""
    return e4m3_decode(codes) * np.asarray(descale, dtype=np.float64)[:, :, None, None]


# ------------------------------------------------------------- attention

def attention_fp8_head_rows(q, k, v, scale: float, causal: bool, rows, round_p: bool = True,
                            tile: int = FP8_TILE):
    """O and LSE of the given query rows of one head, by the online softmax
    over key blocks of `tile` with P rounded to E4M3 (see the module
    docstring).  q, k, v are the dequantised float64 operands [N, d].

    Per block t of keys (the causal mask drops keys past the row):
        m_new = max(m, rowmax s_t);  alpha = exp(m - m_new)
        P = exp(s_t - m_new)                 (P <= 1)
        l = alpha l + rowsum P               (unrounded P)
        acc = alpha acc + E4M3(P) V_t        (round_p=False: P V_t)
    then O = acc / l and LSE = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    N, d = k.shape
    R = rows.size
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, v.shape[1]))
    qr = q[rows]
    last = rows.max() if causal else N - 1
    for start in range(0, last + 1, tile):
        kt = k[start:start + tile]
        s = scale * (qr @ kt.T)
        if causal:
            keys = start + np.arange(kt.shape[0])
            s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        bmax = s.max(axis=1)
        m_new = np.maximum(m, bmax)
        live = np.isfinite(m_new)
        alpha = np.where(live & np.isfinite(m), np.exp(m - np.where(live, m_new, 0.0)), 0.0)
        p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
        pr = e4m3_round(p) if round_p else p
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + pr @ v[start:start + tile]
        m = np.where(live, m_new, m)
    return acc / l[:, None], m + np.log(l)


def attention_fp8(q, k, v, scale: float, causal: bool, round_p: bool = True):
    """attention_fp8_head_rows over every row of every (batch, head) of
    dequantised [B, H, N, d] operands; returns (O, LSE) float64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, 256):
                rows = np.arange(r0, min(N, r0 + 256))
                o[b, h, rows], lse[b, h, rows] = attention_fp8_head_rows(
                    q[b, h], k[b, h], v[b, h], scale, causal, rows, round_p)
    return o, lse
