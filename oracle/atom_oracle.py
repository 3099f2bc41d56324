"""CPU oracle for the Atom W4A4 mixed-precision quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code with the
HIP library (no kernels, headers, tables or helpers) and imports nothing from it.

Plain numpy, written for a reader to check against the pages by eye.  Sources, by page
title and section:

* "Atom: Low-bit Quantization for Efficient and Accurate LLM Serving" -- index page,
  section "Abstract (arXiv)": 4-bit weight-activation quantization built on 4-bit integer
  operators, mixed precision plus fine-grained quantization.
* Same title, curated summary page, method paragraph: weights grouped into small blocks
  with per-group scales; activations get a dedicated higher-precision outlier path.
* "Atom (mixed-precision block-outlier low-bit quantization for serving)" -- quantization
  record, Fields "Bits" (w4a4 with outlier channels at higher precision), "Weight group
  size" (128), "Activation scheme" (dense bulk 4-bit, a small set of outlier channels
  kept at higher precision) and "notes" (every contiguous run of 128 elements is one
  independently quantized group; a 128-channel high-precision group; effective bits ~4;
  integer operators, not FP4 tensor cores).

Readings taken where the pages are silent (each one is also a parameter of the HIP path):

* outlier statistic: sum of squares of each input channel over the calibration tokens,
  as the exactly rounded fp64 value; the 128 largest are outliers, ties to the lower
  channel index; one global set per layer shared by X and W;
* reorder: non-outlier channels ascending, then the outlier channels ascending;
* quantizer: symmetric absmax, no zero point, no clipping; INT4 codes in [-7, 7] for the
  bulk groups, INT8 codes in [-127, 127] for the outlier group;
* scale: fp32 correctly rounded ``absmax / qmax``, rounded to nearest-even fp16 and stored
  fp16, group-major ``[G, rows]``; codes ``clamp(rint_even(fl32(x / s)))``; a zero scale
  gives zero codes;
* packing: INT4 codes four bits each, in units of 16 consecutive codes stored in 8 bytes:
  the codes' OCP FP6 E2M3 encodings (value code/8, a subnormal) laid end to end make 96
  bits, and the last 32 of them are folded into the first 64 at the exponent bits, which
  are always zero for these codes (see ``pack_rows``); the 128 INT8 outlier codes are
  appended as the last 128 two's-complement bytes of each row;
* output: ``Y = sum_g acc_g * sx_g * sw_g`` rounded once to fp16 (round to nearest even).

W4A8 variant (a next step beside the path; the pages point to it only as the precision another
method's kernels target): activations get INT8 codes in every group (same scale rule with
qmax = 127, one byte per code), weights keep the W4 rule and are packed as offset-binary
nibbles (``pack_rows_w4a8``); the group products and the output are the same definitions.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 128          # quantization group: 128 contiguous elements (record, "Weight group size"; "notes")
OUTLIERS = 128       # high-precision outlier channels (record, "notes")
QMAX_INT4 = 7        # symmetric INT4 range for the dense bulk (record, "Bits")
QMAX_INT8 = 127      # symmetric INT8 range for the outlier group (higher precision; record, "Bits")


# --------------------------------------------------------------------------- shapes
def num_groups(K: int) -> int:
    """G = K / 128: groups 0..G-2 are INT4, group G-1 is the INT8 outlier group."""
    if K % GROUP or K < 2 * GROUP:
        raise ValueError(f"K={K} must be a multiple of {GROUP} and at least {2 * GROUP}")
    return K // GROUP


def row_bytes(K: int) -> int:
    """Bytes of one packed row: (K-128) INT4 codes at 2 per byte, then 128 INT8 codes."""
    num_groups(K)
    return (K - OUTLIERS) // 2 + OUTLIERS


# --------------------------------------------------------------------------- step: outlier selection
def channel_stat(X: np.ndarray) -> np.ndarray:
    """Per input channel, the sum of squares over the calibration rows.

    Every fp16 square is exact in fp64, and ``math.fsum`` returns the correctly rounded
    value of the exact sum, so the result does not depend on the summation order."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    sq = np.ascontiguousarray((X64 * X64).T)
    return np.array([math.fsum(sq[c].tolist()) for c in range(sq.shape[0])], dtype=np.float64)


def select_outliers(stat: np.ndarray, n: int = OUTLIERS) -> np.ndarray:
    """Indices (ascending) of the ``n`` channels with the largest statistic; ties go to the
    lower channel index."""
    stat = np.asarray(stat, dtype=np.float64)
    order = sorted(range(stat.shape[0]), key=lambda c: (-stat[c], c))
    return np.array(sorted(order[:n]), dtype=np.int64)


def make_perm(K: int, outliers: np.ndarray) -> np.ndarray:
    """Reordered channel j takes original channel perm[j]: the non-outlier channels in
    ascending order, then the outlier channels in ascending order (outliers at the tail)."""
    is_out = np.zeros(K, dtype=bool)
    is_out[np.asarray(outliers)] = True
    if is_out.sum() != OUTLIERS:
        raise ValueError("need exactly 128 distinct outlier channels")
    return np.concatenate([np.nonzero(~is_out)[0], np.nonzero(is_out)[0]]).astype(np.int32)


def outlier_perm(X_calib: np.ndarray) -> np.ndarray:
    """Calibration rows -> perm (statistic, top-128 selection, reorder)."""
    K = X_calib.shape[1]
    return make_perm(K, select_outliers(channel_stat(X_calib)))


# --------------------------------------------------------------------------- step: quantize one row set
def quantize_rows(X: np.ndarray, perm: np.ndarray, all_int8: bool = False):
    """Reorder the columns of fp16 ``X`` [rows, K] through ``perm`` and quantize each
    128-wide group of each row independently.

    Returns ``(codes int8 [rows, K], scales fp16 [G, rows])``: groups 0..G-2 hold INT4
    codes in [-7, 7], group G-1 (the 128 outlier channels) holds INT8 codes in [-127, 127].
    With ``all_int8`` (the W4A8 variant's activations) every group holds INT8 codes.
    """
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("X must be float16")
    rows, K = X.shape
    G = num_groups(K)
    perm = np.asarray(perm, dtype=np.int64)
    xr = X[:, perm].astype(np.float32).reshape(rows, G, GROUP)     # fp16 -> fp32 is exact

    qmax = np.full(G, QMAX_INT8 if all_int8 else QMAX_INT4, dtype=np.float32)
    qmax[G - 1] = QMAX_INT8
    a = np.max(np.abs(xr), axis=2)                                   # group absmax (exact)
    s32 = a / qmax[None, :]                                          # IEEE fp32 division
    s16 = s32.astype(np.float16)                                     # round to nearest even
    s = s16.astype(np.float32)[:, :, None]

    with np.errstate(divide="ignore", invalid="ignore"):
        t = xr / s                                                   # IEEE fp32 division
    q = np.rint(t)                                                   # ties to even
    q = np.clip(q, -qmax[None, :, None], qmax[None, :, None])
    q = np.where(s == 0.0, 0.0, q)
    return q.astype(np.int8).reshape(rows, K), np.ascontiguousarray(s16.T)


# --------------------------------------------------------------------------- step: pack / unpack
# INT4 packing unit: 16 codes -> 8 bytes.  Code c is written as the 6-bit FP6 E2M3 field of
# the value c/8: sign in bit 5, exponent bits 3-4 (zero: c/8 is a subnormal), |c| in bits 0-2.
UNIT = 16
FIELD = 6
_EXP_BITS = (3, 4)   # exponent positions inside a field


def _exponent_mask(word: int) -> int:
    """Bits of 32-bit word ``word`` (0, 1, 2) of the 96-bit field string that are exponent
    bits of some field, i.e. always zero for INT4 codes."""
    return sum(1 << b for b in range(32) if (32 * word + b) % FIELD in _EXP_BITS)


E0, E1, E2 = (_exponent_mask(w) for w in range(3))
# The third word's nonzero bits are exactly the exponent positions of the first two words,
# so it can be stored in them (a fact of the 6-bit period: 32 = 2 mod 6, 64 = 4 mod 6).
assert (0xFFFFFFFF & ~E2) == (E0 | E1) and (E0 & E1) == 0


def pack_rows(codes: np.ndarray) -> np.ndarray:
    """int8 codes [rows, K] -> packed bytes [rows, (K-128)/2 + 128].

    The first K-128 (INT4) codes go in units of 16 consecutive codes c0..c15, 8 bytes per
    unit, units in order.  Code c_i becomes the field f_i = |c_i| + 32 * (c_i < 0) at bits
    6i .. 6i+5 of a 96-bit string T = T0 + T1 * 2^32 + T2 * 2^64.  The stored words are
    w0 = T0 | (T2 & E0) and w1 = T1 | (T2 & E1), where E0 / E1 are the exponent-bit
    positions of T0 / T1 (zero there, since |c_i| <= 7 keeps every field a subnormal).
    w0 and w1 are written little-endian.  The 128 INT8 outlier codes follow as
    two's-complement bytes."""
    codes = np.asarray(codes, dtype=np.int8)
    rows, K = codes.shape
    klo = K - OUTLIERS
    q = codes[:, :klo].astype(np.int64).reshape(rows, klo // UNIT, UNIT)
    f = np.abs(q) + 32 * (q < 0)                                            # [row, unit, i]
    bits = (f[..., None] >> np.arange(FIELD)) & 1                          # [row, unit, i, b]
    bits = bits.reshape(rows, klo // UNIT, 3, 32)                          # bit 6i+b of T, by word
    T = (bits << np.arange(32, dtype=np.int64)).sum(axis=-1)               # [row, unit, word]
    w0 = T[..., 0] | (T[..., 2] & E0)
    w1 = T[..., 1] | (T[..., 2] & E1)
    words = np.stack([w0, w1], axis=-1).astype("<u4")                      # [row, unit, 2]
    body = words.view(np.uint8).reshape(rows, klo // 2)
    tail = codes[:, klo:].view(np.uint8)
    return np.ascontiguousarray(np.concatenate([body, tail], axis=1))


def unpack_rows(packed: np.ndarray, K: int) -> np.ndarray:
    """Inverse of :func:`pack_rows`."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    if packed.shape[1] != row_bytes(K):
        raise ValueError("packed row length does not match K")
    klo = K - OUTLIERS
    words = np.ascontiguousarray(packed[:, : klo // 2]).view("<u4").astype(np.int64).reshape(rows, klo // UNIT, 2)
    w0, w1 = words[..., 0], words[..., 1]
    T = np.stack([w0 & ~E0 & 0xFFFFFFFF, w1 & ~E1 & 0xFFFFFFFF, (w0 & E0) | (w1 & E1)], axis=-1)
    bits = (T[..., None] >> np.arange(32)) & 1                              # [row, unit, word, b]
    f = (bits.reshape(rows, klo // UNIT, UNIT, FIELD) << np.arange(FIELD)).sum(axis=-1)
    if np.any(f & 0b011000):
        raise ValueError("exponent bits set: not an INT4 code")
    mag, neg = f & 7, f >> 5
    out = np.empty((rows, K), dtype=np.int8)
    out[:, :klo] = np.where(neg == 1, -mag, mag).reshape(rows, klo)
    out[:, klo:] = packed[:, klo // 2:].view(np.int8)
    return out


# --------------------------------------------------------------------------- W4A8 variant: layouts
def pack_rows_a8(codes: np.ndarray) -> np.ndarray:
    """INT8 activation codes [rows, K] -> bytes [rows, K]: each code as one two's-complement
    byte, in reordered channel order."""
    codes = np.asarray(codes, dtype=np.int8)
    return np.ascontiguousarray(codes).view(np.uint8).copy()


def unpack_rows_a8(packed: np.ndarray, K: int) -> np.ndarray:
    """Inverse of :func:`pack_rows_a8`."""
    packed = np.asarray(packed, dtype=np.uint8)
    assert packed.shape[1] == K
    return packed.view(np.int8).copy()


def pack_rows_w4a8(codes: np.ndarray) -> np.ndarray:
    """W4 codes [rows, K] (INT4 in groups 0..G-2, INT8 in group G-1) -> bytes
    [rows, (K-128)/2 + 128] for the W4A8 GEMM.

    The K-128 INT4 codes go in blocks of 8 consecutive codes c_0..c_7, each block 4 bytes:
    byte j (j = 0..3) holds c_j + 8 in its low nibble and c_{j+4} + 8 in its high nibble
    (offset binary, values 1..15).  Masking a little-endian word with 0x0F0F0F0F gives the
    biased codes c_0..c_3 as bytes, shifting it right by 4 first gives c_4..c_7.  The 128
    INT8 codes follow as two's-complement bytes."""
    codes = np.asarray(codes, dtype=np.int8)
    rows, K = codes.shape
    klo = K - OUTLIERS
    q = codes[:, :klo].astype(np.int16) + 8
    if q.min(initial=8) < 1 or q.max(initial=8) > 15:
        raise ValueError("INT4 codes must lie in [-7, 7]")
    blk = q.reshape(rows, klo // 8, 8)
    body = (blk[:, :, :4] | (blk[:, :, 4:] << 4)).astype(np.uint8).reshape(rows, klo // 2)
    tail = np.ascontiguousarray(codes[:, klo:]).view(np.uint8)
    return np.ascontiguousarray(np.concatenate([body, tail], axis=1))


def unpack_rows_w4a8(packed: np.ndarray, K: int) -> np.ndarray:
    """Inverse of :func:`pack_rows_w4a8`."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    klo = K - OUTLIERS
    body = packed[:, :klo // 2].reshape(rows, klo // 8, 4).astype(np.int16)
    lo, hi = body & 0xF, body >> 4
    q = (np.concatenate([lo, hi], axis=2) - 8).reshape(rows, klo).astype(np.int8)
    tail = packed[:, klo // 2:].view(np.int8)
    return np.concatenate([q, tail], axis=1)


def quantize_act_a8(X: np.ndarray, perm: np.ndarray):
    """W4A8 runtime activation quantize: (bytes u8 [M, K], scales fp16 [G, M])."""
    q, s = quantize_rows(X, perm, all_int8=True)
    return pack_rows_a8(q), s


def pack_weights_w4a8(W: np.ndarray, perm: np.ndarray):
    """W4A8 offline weight pack: the W4 rule, offset-binary layout (u8 [N, row_bytes],
    scales fp16 [G, N])."""
    q, s = quantize_rows(W, perm)
    return pack_rows_w4a8(q), s


# --------------------------------------------------------------------------- the layer's two runtime calls
def quantize_act(X: np.ndarray, perm: np.ndarray):
    """Runtime activation quantize: (packed codes u8 [M, row_bytes], scales fp16 [G, M])."""
    q, s = quantize_rows(X, perm)
    return pack_rows(q), s


def pack_weights(W: np.ndarray, perm: np.ndarray):
    """Offline weight pack with the same rule: (packed u8 [N, row_bytes], scales fp16 [G, N])."""
    q, s = quantize_rows(W, perm)
    return pack_rows(q), s


# --------------------------------------------------------------------------- step: per-group integer products
def group_acc(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[g, m, n] = sum over the 128 channels k of group g of qx[m, k] * qw[n, k].

    Computed with an fp64 matmul per group: every partial sum is an integer of magnitude
    at most 128 * 127 * 127 < 2**53, so the fp64 result is exact; it is checked to be
    integral and to fit in int32."""
    qx = np.asarray(qx, dtype=np.int8)
    qw = np.asarray(qw, dtype=np.int8)
    M, K = qx.shape
    N = qw.shape[0]
    G = num_groups(K)
    out = np.empty((G, M, N), dtype=np.int64)
    for g in range(G):
        a = qx[:, g * GROUP:(g + 1) * GROUP].astype(np.float64)
        b = qw[:, g * GROUP:(g + 1) * GROUP].astype(np.float64)
        p = a @ b.T
        ip = p.astype(np.int64)
        if not np.array_equal(ip.astype(np.float64), p):
            raise AssertionError("non-integral group product")
        out[g] = ip
    if np.abs(out).max(initial=0) >= 2 ** 31:
        raise AssertionError("group product overflows int32")
    return out


# --------------------------------------------------------------------------- step: dequantised output
def _expand(scales: np.ndarray, K: int) -> np.ndarray:
    """fp16 scales [G, rows] -> fp64 [rows, K] (each scale repeated over its 128 channels)."""
    return np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64).T, GROUP, axis=1)[:, :K]


def gemm_ref(qx: np.ndarray, sx: np.ndarray, qw: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """Y64[m, n] = sum_g acc_g[m, n] * sx[g, m] * sw[g, n] in fp64.

    Written as one fp64 matmul of the dequantised operands: each product q * s is exact in
    fp64, so this is the same sum up to fp64 rounding order."""
    K = qx.shape[1]
    a = qx.astype(np.float64) * _expand(sx, K)
    b = qw.astype(np.float64) * _expand(sw, K)
    return a @ b.T


def gemm_ref_grouped(qx, sx, qw, sw) -> np.ndarray:
    """The same output written as the explicit sum over groups of scaled integer products."""
    acc = group_acc(qx, qw).astype(np.float64)
    sxd = np.asarray(sx, dtype=np.float16).astype(np.float64)
    swd = np.asarray(sw, dtype=np.float16).astype(np.float64)
    y = np.zeros(acc.shape[1:], dtype=np.float64)
    for g in range(acc.shape[0]):
        y += acc[g] * sxd[g][:, None] * swd[g][None, :]
    return y


def to_fp16(y64: np.ndarray) -> np.ndarray:
    """Round fp64 to fp16, nearest even."""
    return np.asarray(y64, dtype=np.float64).astype(np.float16)


def linear(X: np.ndarray, W: np.ndarray, perm: np.ndarray):
    """Whole layer: returns (Y fp16, Y64, (Xq, sx), (Wq, sw))."""
    qx, sx = quantize_rows(X, perm)
    qw, sw = quantize_rows(W, perm)
    y64 = gemm_ref(qx, sx, qw, sw)
    return to_fp16(y64), y64, (pack_rows(qx), sx), (pack_rows(qw), sw)


def effective_bits(K: int, scale_bytes: int = 2) -> float:
    """Bits per element of one quantized row including its per-group scales."""
    return (row_bytes(K) * 8 + num_groups(K) * scale_bytes * 8) / K
