"""Pins of the oracle's W4A8 variant (INT8 activations in every group, W4 weights).

The variant keeps the W4 rule for weights and uses the same scale rule with qmax = 127 for
every activation group (quantization record of "Atom (mixed-precision block-outlier low-bit
quantization for serving)", Fields "Bits", "Weight group size", "notes": per-group scales,
the 128-channel INT8 group).  Each test checks the oracle against something other than its
own code: hand-derived bytes, a closed-form error bound, exact rationals, brute-force sums.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import atom_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def test_w4a8_layout_hand_derived_bytes():
    fx = json.load(open(os.path.join(HERE, "golden", "w4a8_layout.json")))
    K = fx["K"]
    for row in fx["rows"]:
        codes = np.zeros((1, K), dtype=np.int8)
        codes[0, :16] = row["int4_codes_first_16"]
        codes[0, K - 128:K - 124] = row["int8_tail_first_4"]
        packed = O.pack_rows_w4a8(codes)
        assert packed.shape == (1, O.row_bytes(K))
        assert [int(b) for b in packed[0, :8]] == [int(h, 16) for h in row["packed_first_8"]]
        klo = (K - 128) // 2
        assert [int(b) for b in packed[0, klo:klo + 4]] == [int(h, 16) for h in row["packed_tail_first_4"]]
        # the rest of the INT4 body is zero codes, i.e. 0x88 bytes
        assert np.all(packed[0, 8:klo] == 0x88)


@pytest.mark.parametrize("K", [256, 1024, 4096])
def test_w4a8_layout_round_trip_and_nibble_positions(K):
    rng = np.random.default_rng(K)
    rows = 5
    q = np.concatenate([rng.integers(-7, 8, size=(rows, K - 128)), rng.integers(-127, 128, size=(rows, 128))],
                       axis=1).astype(np.int8)
    packed = O.pack_rows_w4a8(q)
    assert np.array_equal(O.unpack_rows_w4a8(packed, K), q)
    # code k of the body sits in byte 4 (k // 8) + (k % 4), high nibble when k % 8 >= 4
    for k in rng.choice(K - 128, 40, replace=False):
        byte = int(packed[2, 4 * (k // 8) + (k % 4)])
        nib = byte >> 4 if k % 8 >= 4 else byte & 15
        assert nib - 8 == int(q[2, k])


def test_a8_bytes_are_twos_complement():
    q = np.array([[-127, -1, 0, 1, 127] + [0] * 251], dtype=np.int8)
    b = O.pack_rows_a8(q)
    assert [int(v) for v in b[0, :5]] == [0x81, 0xFF, 0x00, 0x01, 0x7F]
    assert np.array_equal(O.unpack_rows_a8(b, 256), q)


@pytest.mark.parametrize("seed,K", [(0, 256), (1, 1024), (2, 4096)])
def test_a8_round_trip_bound(seed, K):
    """Every activation group INT8: |x - q s| <= s (1/2 + 2^-21) for normal scales, and the
    absmax element maps to +-127."""
    rng = np.random.default_rng(seed)
    M = 20
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp(rng.uniform(-8, 6, size=(M, 1))).astype(np.float32)
    x[:, rng.choice(K, 5, replace=False)] *= 30
    X = x.astype(np.float16)
    perm = rng.permutation(K).astype(np.int32)
    q, s16 = O.quantize_rows(X, perm, all_int8=True)
    G = K // 128
    xr = X[:, perm].astype(np.float64).reshape(M, G, 128)
    qg = q.astype(np.float64).reshape(M, G, 128)
    s = s16.astype(np.float64).T[:, :, None]
    assert np.all(np.abs(qg) <= 127)
    normal = np.broadcast_to(s >= 2.0 ** -14, xr.shape)
    err = np.abs(xr - qg * s)
    assert normal.any()
    assert np.all(err[normal] <= np.broadcast_to(s * (0.5 + 2.0 ** -21), xr.shape)[normal])
    a = np.abs(xr).max(axis=2)
    qa = np.take_along_axis(np.abs(qg), np.abs(xr).argmax(axis=2)[:, :, None], axis=2)[:, :, 0]
    ok = (a > 0) & (s[:, :, 0] >= 2.0 ** -14)
    assert np.all(qa[ok] == 127)


def test_a8_scale_is_fp16_of_absmax_over_127_within_half_ulp():
    x, _, _ = synth.make_linear(6, 512, 1, seed=5)
    _, s16 = O.quantize_rows(x, np.arange(512, dtype=np.int32), all_int8=True)
    for r in range(6):
        for g in range(4):
            a = Fraction(float(np.abs(x[r, g * 128:(g + 1) * 128].astype(np.float64)).max()))
            s = Fraction(float(s16[g, r]))
            ulp = Fraction(2) ** (math.frexp(float(s))[1] - 1 - 10)
            assert abs(s - a / 127) <= ulp / 2


@pytest.mark.parametrize("M,N,K", [(4, 5, 256), (7, 3, 384)])
def test_w4a8_group_products_and_output_brute_force(M, N, K):
    x, w, _ = synth.make_linear(M, K, N, seed=M * 31 + N)
    perm = np.random.default_rng(K).permutation(K).astype(np.int32)
    qx, sx = O.quantize_rows(x, perm, all_int8=True)
    qw, sw = O.quantize_rows(w, perm)
    acc = O.group_acc(qx, qw)
    G = K // 128
    y = np.zeros((M, N), dtype=object)
    for g in range(G):
        for m in range(M):
            for n in range(N):
                t = 0
                for k in range(g * 128, (g + 1) * 128):
                    t += int(qx[m, k]) * int(qw[n, k])
                assert acc[g, m, n] == t
                y[m, n] += Fraction(t) * Fraction(float(sx[g, m])) * Fraction(float(sw[g, n]))
    y64 = O.gemm_ref(qx, sx, qw, sw)
    exact = np.array([[float(v) for v in r] for r in y])
    assert np.allclose(y64, exact, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K", [256, 1152])
def test_w4a8_layer_calls_lossless_power_of_two_scales(K):
    """The variant's two calls on inputs built as s * q (power-of-two s per group, max|q| =
    qmax in every group): quantize_act_a8 must return every code as its two's-complement byte
    (INT8 in EVERY group, qmax 127) and the known scales; pack_weights_w4a8 the known W4 codes
    (INT4 bulk, INT8 last group) in the offset-binary layout whose bytes the hand-derived
    fixture pins.  A packer mix-up, a missing all-groups-INT8 switch or fp32-sized scales fail."""
    rng = np.random.default_rng(K + 5)
    G = K // 128

    def build(rows, qmaxes):
        q = np.concatenate([rng.integers(-qm, qm + 1, size=(rows, 128)) for qm in qmaxes], axis=1)
        s = np.ldexp(1.0, rng.integers(-12, 2, size=(rows, G)))
        for g, qm in enumerate(qmaxes):
            q[np.arange(rows), g * 128 + rng.integers(0, 128, size=rows)] = qm * rng.choice([-1, 1], size=rows)
        return (q.reshape(rows, G, 128) * s[:, :, None]).reshape(rows, K).astype(np.float16), q.astype(np.int8), s

    X, qx_true, sx_true = build(6, [127] * G)
    W, qw_true, sw_true = build(9, [7] * (G - 1) + [127])
    perm = np.arange(K, dtype=np.int32)
    xb, sx = O.quantize_act_a8(X, perm)
    assert xb.dtype == np.uint8 and xb.shape == (6, K)
    assert sx.dtype == np.float16 and sx.shape == (G, 6)
    np.testing.assert_array_equal(xb.view(np.int8), qx_true)
    np.testing.assert_array_equal(sx.astype(np.float64).T, sx_true)
    wb, sw = O.pack_weights_w4a8(W, perm)
    assert wb.dtype == np.uint8 and wb.shape == (9, O.row_bytes(K))
    assert sw.dtype == np.float16 and sw.shape == (G, 9)
    np.testing.assert_array_equal(O.unpack_rows_w4a8(wb, K), qw_true)
    np.testing.assert_array_equal(sw.astype(np.float64).T, sw_true)
    # byte-level: code k of the body in byte 4 (k // 8) + k % 4, biased by 8 (fixture layout)
    k = np.arange(K - 128)
    b = wb[:, 4 * (k // 8) + (k % 4)].astype(np.int16)
    nib = np.where(k % 8 >= 4, b >> 4, b & 15) - 8
    np.testing.assert_array_equal(nib, qw_true[:, :K - 128])
    np.testing.assert_array_equal(wb[:, (K - 128) // 2:].view(np.int8), qw_true[:, K - 128:])
    # the output of the variant: exact textbook product
    y64 = O.gemm_ref(xb.view(np.int8), sx, O.unpack_rows_w4a8(wb, K), sw)
    np.testing.assert_array_equal(y64, X.astype(np.float64) @ W.astype(np.float64).T)
