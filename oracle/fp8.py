"""FP8 attention with block quantization and incoherent processing, in fp64
(test infrastructure).

Sources:
  * FlashAttention from Scratch (ryhuang.blog), §10.3 "Treat FP8 as a second
    lesson": FA3 quantizes to FP8 with block quantization and incoherent
    processing; Q and K are multiplied by the same orthogonal matrix R, which
    leaves the scores unchanged before rounding and spreads a large component
    over the coordinates.
  * FlashAttention 1-4 (noviorlu.github.io), FlashAttention-3, point 3 "FP8
    with block quantization and incoherent processing": one FP8 scale per tile
    instead of one per tensor; the matrix is a Hadamard transform with random
    sign flips, M M^T = I, so (QM)(KM)^T = QK^T; a per-tensor scale is the
    baseline the block scheme improves on for inputs with outlier features.

Readings (the pages fix none of these details):
  * format: OCP FP8 E4M3 (largest finite 448, subnormals down to 2^-9, no
    infinity), rounding to nearest with ties to even -- the operand format of
    the gfx950 matrix cores;
  * blocks: one scale per 256 query rows of a head and per 64 keys of a head
    (the forward's query block and KV tile);
  * a block's scale is the smallest power of two 2^k with max|x| 2^-k <= 448,
    so scaling is exact and only the rounding to E4M3 loses information;
  * incoherent processing: x' = H (sigma * x) per row, with H the Sylvester
    Hadamard matrix (entries +-1, H H^T = D I) and sigma a vector of random
    signs shared by Q and K; the orthogonal matrix of the pages is
    M = diag(sigma) H / sqrt(D), whose 1/D in the scores goes into the
    softmax scale (the codes are those of the unnormalised x');
  * only Q and K are quantized: V and the probabilities stay as in the bf16
    forward (the pages discuss the outliers of Q and K).

The transform is exact in fp64 for bf16 inputs whose exponents span at most
38 binades (every partial sum of +-x terms is then representable), so the
rounding of x' to fp32, and of x' 2^-k to E4M3, are decisions taken on exact
values -- the same decisions any exact implementation takes.
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64, attention_forward

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code: sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal (M/8 * 2^-6); S.1111.111 is NaN."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def round_e4m3(x):
    """Round to the nearest E4M3 value, ties to even; |x| must be <= 448.

    Returns (values fp64, codes uint8).  In the binade [2^e, 2^(e+1)) the
    spacing is 2^(e-3) for e >= -6 and 2^-9 below (subnormals), so rounding
    is rint(|x| / spacing) * spacing, with rint's ties to even landing on an
    even mantissa; a result of exactly 2^(e+1) is the next binade's first
    value.  A zero result keeps the sign of x."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.all(a <= E4M3_MAX), "value outside the E4M3 range"
    _, E = np.frexp(np.where(a > 0, a, 1.0))          # a = f 2^E, f in [0.5, 1)
    binade = np.maximum(E - 1, -6)
    spacing = np.ldexp(1.0, binade - 3)
    mag = np.rint(a / spacing) * spacing
    neg = np.signbit(x)
    values = np.where(neg, -mag, mag)
    # Encode: subnormal (mag < 2^-6) -> M = mag / 2^-9; normal -> exponent and mantissa.
    _, E2 = np.frexp(np.where(mag > 0, mag, 1.0))
    eb = E2 - 1
    normal = mag >= 2.0 ** -6
    m_norm = np.where(normal, np.ldexp(mag, -eb) * 8 - 8, 0)
    code_norm = ((eb + 7) << 3) + m_norm.astype(np.int64)
    code_sub = (mag / 2.0 ** -9).astype(np.int64)
    codes = np.where(normal, code_norm, code_sub) + np.where(neg, 0x80, 0)
    return values, codes.astype(np.uint8)


def sylvester_hadamard(D: int) -> np.ndarray:
    """The D x D Hadamard matrix of Sylvester's construction (D a power of
    two): H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    assert D >= 1 and D & (D - 1) == 0, "D must be a power of two"
    H = np.ones((1, 1))
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    return H


def incoherent(x, signs):
    """x' = H (sigma * x) along the last axis, exactly in fp64 (H symmetric)."""
    x = as_f64(x)
    s = np.asarray(signs, dtype=np.float64)
    assert np.all(np.abs(s) == 1.0), "signs must be +-1"
    H = sylvester_hadamard(x.shape[-1])
    return (x * s) @ H


def block_scale_exponent(amax: float) -> int:
    """Smallest integer k with amax * 2^-k <= 448 (0 for an all-zero block)."""
    if amax == 0.0:
        return 0
    _, E = np.frexp(amax)                 # amax in [2^(E-1), 2^E)
    # 448 * 2^(E-9) = 0.875 * 2^E and 448 * 2^(E-10) < 2^(E-1) <= amax.
    return int(E - 9) if amax <= 0.875 * 2.0 ** E else int(E - 8)


def quantize_rows(x, block_rows, signs=None):
    """Block-quantize [..., L, D] rows to E4M3, one power-of-two scale per
    ``block_rows`` consecutive rows of each leading index.

    Returns (codes uint8 [..., L, D], scales fp64 [..., ceil(L / block_rows)],
    values fp64 [..., L, D] = code value * scale).  With ``signs``, the rows
    are first transformed by ``incoherent``; either way they are rounded to
    fp32 before the block maximum is taken."""
    x64 = incoherent(x, signs) if signs is not None else as_f64(x)
    x32 = x64.astype(np.float32).astype(np.float64)
    L = x32.shape[-2]
    nb = -(-L // block_rows)
    codes = np.zeros(x32.shape, dtype=np.uint8)
    values = np.zeros(x32.shape)
    scales = np.zeros(x32.shape[:-2] + (nb,))
    lead = x32.shape[:-2]
    for idx in np.ndindex(*lead):
        for j in range(nb):
            blk = x32[idx][j * block_rows:(j + 1) * block_rows]
            k = block_scale_exponent(float(np.abs(blk).max()) if blk.size else 0.0)
            v, c = round_e4m3(np.ldexp(blk, -k))
            codes[idx][j * block_rows:(j + 1) * block_rows] = c
            values[idx][j * block_rows:(j + 1) * block_rows] = np.ldexp(v, k)
            scales[idx + (j,)] = 2.0 ** k
    return codes, scales, values


def quantize_per_tensor(x):
    """The baseline of the pages: one power-of-two scale per whole tensor.
    Returns the dequantized values."""
    x32 = as_f64(x).astype(np.float32).astype(np.float64)
    k = block_scale_exponent(float(np.abs(x32).max()))
    v, _ = round_e4m3(np.ldexp(x32, -k))
    return np.ldexp(v, k)


def fp8_attention_forward(q, k, v, scale, causal=False, kv_lens=None, signs=None,
                          q_block=256, k_block=64, window=0):
    """Attention of the block-quantized Q and K (after incoherent processing
    when ``signs`` is given) with V as given: the definition evaluated in fp64
    on the dequantized values, with scores scale * Q'K'^T / D under the
    transform (M = diag(sigma) H / sqrt(D)).  Returns (O, LSE, qcodes,
    qscales, kcodes, kscales)."""
    qc, qs, qv = quantize_rows(q, q_block, signs)
    kc, ks, kv = quantize_rows(k, k_block, signs)
    D = qv.shape[-1]
    eff = scale / D if signs is not None else scale
    O, lse = attention_forward(qv, kv, as_f64(v), eff, causal, kv_lens, window=window)
    return O, lse, qc, qs, kc, ks
