"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU needed).

Each test pins one step of the oracle to something other than itself: a closed-form
bound, an invariant, a special case that reduces to a library matmul, brute force on tiny
inputs, exact rational arithmetic, or the hand-worked fixture in ``tests/golden``.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import atom_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _h(hexstr):
    return np.array([int(hexstr, 16)], dtype=np.uint16).view(np.float16)[0]


# --------------------------------------------------------------------------- hand-worked rows
def test_worked_rows_fixture():
    """Codes, scales and bytes of five hand-derived rows (ties, outlier group, zero row,
    underflowing scale, subnormal scale where the clamp fires, and a unit whose 16 codes
    fill every FP6 field, including the folded third word)."""
    fx = json.load(open(os.path.join(GOLDEN, "worked_rows.json")))
    K = fx["K"]
    rows = fx["rows"]
    X = np.zeros((len(rows), K), dtype=np.float16)
    for r, row in enumerate(rows):
        for c, hx in row["x_fp16_hex"].items():
            X[r, int(c)] = _h(hx)
    perm = np.arange(K, dtype=np.int32)
    q, s = O.quantize_rows(X, perm)
    packed = O.pack_rows(q)
    for r, row in enumerate(rows):
        exp_s = [int(h, 16) for h in row["scales_fp16_hex"]]
        assert s[:, r].view(np.uint16).tolist() == exp_s, row["name"]
        exp_q = np.zeros(K, dtype=np.int8)
        for c, v in row["codes"].items():
            exp_q[int(c)] = v
        np.testing.assert_array_equal(q[r], exp_q, err_msg=row["name"])
        exp_b = np.zeros(O.row_bytes(K), dtype=np.uint8)
        for c, hx in row["packed_hex"].items():
            exp_b[int(c) if int(c) < 128 else int(c) - 128 + (K - 128) // 2] = int(hx, 16)
        np.testing.assert_array_equal(packed[r], exp_b, err_msg=row["name"])
    np.testing.assert_array_equal(O.unpack_rows(packed, K), q)


# --------------------------------------------------------------------------- P1 round-trip bound
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("K", [256, 384, 1024, 4096])
def test_p1_round_trip_bound(seed, K):
    rng = np.random.default_rng(seed)
    M = 24
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp(rng.uniform(-8, 6, size=(M, 1))).astype(np.float32)   # rows over many binades
    x[:, rng.choice(K, 5, replace=False)] *= 30
    X = x.astype(np.float16)
    perm = rng.permutation(K).astype(np.int32)
    q, s16 = O.quantize_rows(X, perm)
    G = K // 128
    xr = X[:, perm].astype(np.float64).reshape(M, G, 128)
    qg = q.astype(np.float64).reshape(M, G, 128)
    s = s16.astype(np.float64).T[:, :, None]
    qmax = np.array([7.0] * (G - 1) + [127.0])[None, :, None]
    normal = s >= 2.0 ** -14
    err = np.abs(xr - qg * s)
    assert np.all(np.abs(qg) <= qmax)
    mask = np.broadcast_to(normal, err.shape)
    bound = np.broadcast_to(s * (0.5 + 2.0 ** -21), err.shape)
    assert mask.any()
    assert np.all(err[mask] <= bound[mask])
    # the absmax element maps exactly to +-qmax
    a = np.abs(xr).max(axis=2)
    amax_idx = np.abs(xr).argmax(axis=2)
    qa = np.take_along_axis(np.abs(qg), amax_idx[:, :, None], axis=2)[:, :, 0]
    nz = a > 0
    assert np.all(qa[nz & normal[:, :, 0]] == np.broadcast_to(qmax[:, :, 0], qa.shape)[nz & normal[:, :, 0]])


def test_p1_scale_is_fp16_of_absmax_over_qmax_within_half_ulp():
    """The stored scale is the fp16 value nearest absmax/qmax (closed form, exact rationals)."""
    x, _, _ = synth.make_linear(8, 512, 1, seed=3)
    perm = np.arange(512, dtype=np.int32)
    _, s16 = O.quantize_rows(x, perm)
    for r in range(8):
        for g in range(4):
            a = Fraction(float(np.abs(x[r, g * 128:(g + 1) * 128].astype(np.float64)).max()))
            exact = a / (7 if g < 3 else 127)
            s = Fraction(float(s16[g, r]))
            # fp16 neighbours of s: spacing 2^(e-10) in the normal range
            e = math.frexp(float(s))[1] - 1
            ulp = Fraction(2) ** (e - 10)
            assert abs(s - exact) <= ulp / 2


# --------------------------------------------------------------------------- P2 brute force
@pytest.mark.parametrize("M,N,K", [(5, 7, 256), (9, 4, 384), (16, 32, 1024), (3, 3, 512)])
def test_p2_brute_force_group_products(M, N, K):
    x, w, _ = synth.make_linear(M, K, N, seed=M * 100 + N)
    perm = np.random.default_rng(K).permutation(K).astype(np.int32)
    qx, sx = O.quantize_rows(x, perm)
    qw, sw = O.quantize_rows(w, perm)
    acc = O.group_acc(qx, qw)
    G = K // 128
    brute = np.zeros((G, M, N), dtype=np.int64)
    for g in range(G):
        for m in range(M):
            for n in range(N):
                t = 0
                for k in range(g * 128, (g + 1) * 128):
                    t += int(qx[m, k]) * int(qw[n, k])
                brute[g, m, n] = t
    np.testing.assert_array_equal(acc, brute)
    y_grouped = O.gemm_ref_grouped(qx, sx, qw, sw)
    y = O.gemm_ref(qx, sx, qw, sw)
    assert np.max(np.abs(y - y_grouped)) <= 1e-12 * max(1.0, np.max(np.abs(y)))
    # exact rational evaluation of one output per case
    m, n = M - 1, N // 2
    exact = sum(Fraction(int(brute[g, m, n])) * Fraction(float(sx[g, m])) * Fraction(float(sw[g, n]))
                for g in range(G))
    assert abs(float(exact) - y_grouped[m, n]) <= 1e-12 * max(1.0, abs(float(exact)))


def test_p2_tiny_workload_brute_force():
    x, w, _ = synth.make_inputs(synth.get("T"))
    perm = O.outlier_perm(x)
    qx, sx = O.quantize_rows(x, perm)
    qw, sw = O.quantize_rows(w[:24], perm)
    acc = O.group_acc(qx, qw)
    ref = np.einsum("mgk,ngk->gmn", qx.astype(np.int64).reshape(16, 8, 128),
                    qw.astype(np.int64).reshape(24, 8, 128))
    np.testing.assert_array_equal(acc, ref)


# --------------------------------------------------------------------------- P3 lossless special case
@pytest.mark.parametrize("K", [256, 1024])
def test_p3_lossless_power_of_two_scales(K):
    """X and W built as s*q with s a power of two per group and max|q| = qmax: the oracle
    reproduces q and s exactly and Y64 equals the fp64 textbook X @ W.T exactly."""
    rng = np.random.default_rng(K)
    M, N = 12, 20
    G = K // 128

    def build(rows):
        q = rng.integers(-7, 8, size=(rows, K)).astype(np.int64)
        q[:, K - 128:] = rng.integers(-127, 128, size=(rows, 128))
        e = rng.integers(-10, 3, size=(rows, G))
        s = np.ldexp(1.0, e)
        for g in range(G):                      # force max|q| = qmax in each group
            qm = 7 if g < G - 1 else 127
            col = rng.integers(0, 128, size=rows)
            q[np.arange(rows), g * 128 + col] = qm * rng.choice([-1, 1], size=rows)
        x = (q.reshape(rows, G, 128) * s[:, :, None]).reshape(rows, K)
        return x.astype(np.float16), q.astype(np.int8), s

    X, qx_true, sx_true = build(M)
    W, qw_true, sw_true = build(N)
    assert np.array_equal(X.astype(np.float64), (qx_true.reshape(M, G, 128) * sx_true[:, :, None]).reshape(M, K))
    perm = np.arange(K, dtype=np.int32)
    qx, sx = O.quantize_rows(X, perm)
    qw, sw = O.quantize_rows(W, perm)
    np.testing.assert_array_equal(qx, qx_true)
    np.testing.assert_array_equal(qw, qw_true)
    np.testing.assert_array_equal(sx.astype(np.float64).T, sx_true)
    np.testing.assert_array_equal(sw.astype(np.float64).T, sw_true)
    y64 = O.gemm_ref_grouped(qx, sx, qw, sw)
    textbook = X.astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_array_equal(y64, textbook)
    np.testing.assert_array_equal(O.gemm_ref(qx, sx, qw, sw), textbook)
    assert np.array_equal(O.unpack_rows(O.pack_rows(qx), K), qx)
    # the layer's two calls: packed codes decode to the known codes, scales are the known ones
    xq, sx2 = O.quantize_act(X, perm)
    wq, sw2 = O.pack_weights(W, perm)
    np.testing.assert_array_equal(O.unpack_rows(xq, K), qx_true)
    np.testing.assert_array_equal(O.unpack_rows(wq, K), qw_true)
    np.testing.assert_array_equal(sx2.astype(np.float64).T, sx_true)
    np.testing.assert_array_equal(sw2.astype(np.float64).T, sw_true)
    # and the whole layer: Y64 is the textbook product, Y16 its fp16 rounding
    y16, y64b, (xq3, _), (wq3, _) = O.linear(X, W, perm)
    np.testing.assert_array_equal(y64b, textbook)
    np.testing.assert_array_equal(xq3, xq)
    np.testing.assert_array_equal(wq3, wq)
    np.testing.assert_array_equal(y16, textbook.astype(np.float16))


# --------------------------------------------------------------------------- P4 in-group permutation invariance
def test_p4_in_group_permutation_invariance():
    M, N, K = 10, 14, 768
    x, w, _ = synth.make_linear(M, K, N, seed=11)
    perm = O.outlier_perm(x)
    qx, sx = O.quantize_rows(x, perm)
    qw, sw = O.quantize_rows(w, perm)
    acc = O.group_acc(qx, qw)
    y = O.gemm_ref_grouped(qx, sx, qw, sw)
    rng = np.random.default_rng(5)
    perm2 = perm.copy()
    for g in range(K // 128):
        perm2[g * 128:(g + 1) * 128] = rng.permutation(perm[g * 128:(g + 1) * 128])
    qx2, sx2 = O.quantize_rows(x, perm2)
    qw2, sw2 = O.quantize_rows(w, perm2)
    np.testing.assert_array_equal(sx2, sx)
    np.testing.assert_array_equal(sw2, sw)
    np.testing.assert_array_equal(O.group_acc(qx2, qw2), acc)
    np.testing.assert_array_equal(O.gemm_ref_grouped(qx2, sx2, qw2, sw2), y)


# --------------------------------------------------------------------------- P5 bit accounting
@pytest.mark.parametrize("K,expected", [(1024, 4.625), (4096, 4.25), (8192, 4.1875), (11008, 4.171511627906977)])
def test_p5_effective_bits(K, expected):
    """Measured bytes of packed codes + fp16 scales per element.  The record's notes give
    'effective bit of 4' for group 128 with a 128-channel high-precision group; the exact
    count is (K-128)*4 + 128*8 code bits plus 16 scale bits per group, which rounds to 4
    for the Llama shapes (K >= 4096)."""
    X = np.ones((3, K), dtype=np.float16)
    xq, sx = O.quantize_act(X, np.arange(K, dtype=np.int32))
    measured = (xq.nbytes + sx.nbytes) * 8 / X.size
    assert measured == pytest.approx(expected, abs=1e-12)
    assert measured == pytest.approx(((K - 128) * 4 + 128 * 8 + (K // 128) * 16) / K, abs=1e-12)
    if K >= 4096:
        assert round(measured) == 4


@pytest.mark.parametrize("K,fp16_scales,fp32_scales", [(1024, 4.625, 4.75), (4096, 4.25, 4.375),
                                                       (8192, 4.1875, 4.3125), (11008, 4.1715, 4.2965)])
def test_p5_effective_bits_closed_form(K, fp16_scales, fp32_scales):
    """effective_bits against the bit-accounting table (INT4 bulk at 4 bits, the 128-channel
    group at 8 bits, one scale per 128-group; fp16 scales as stored, fp32 for comparison)."""
    assert O.effective_bits(K) == pytest.approx(fp16_scales, abs=5e-5)
    assert O.effective_bits(K, scale_bytes=4) == pytest.approx(fp32_scales, abs=5e-5)
    assert O.effective_bits(K) - O.effective_bits(K, scale_bytes=4) == pytest.approx(-16 / 128)


def test_to_fp16_rounds_once_to_nearest_even():
    """Y16 = fp16_rne(Y64) in one rounding, values worked out from the binary16 format: 11
    significant bits, largest finite 65504, subnormal spacing 2^-24."""
    u = 2.0 ** -10                                  # fp16 spacing on [1, 2)
    cases = [
        (1.0 + u / 2, 1.0),                         # tie -> even (1.0)
        (1.0 + 3 * u / 2, 1.0 + 2 * u),             # tie -> even (1 + 2u)
        (1.0 + u / 2 + 2.0 ** -40, 1.0 + u),        # just above the tie: up (a detour through fp32 would give 1.0)
        (-(1.0 + u / 2 + 2.0 ** -40), -(1.0 + u)),
        (65504.0, 65504.0),
        (65519.99, 65504.0),                        # below the overflow threshold 65520
        (65520.0, np.inf),                          # the tie above 65504 rounds to even = overflow
        (2.0 ** -25, 0.0),                          # half the smallest subnormal: tie -> even (0)
        (2.0 ** -25 + 2.0 ** -60, 2.0 ** -24),
        (3 * 2.0 ** -25, 2.0 ** -23),               # tie between 1 and 2 subnormal steps -> 2
        (0.1, 0.0999755859375),                     # nearest fp16 to 0.1 (0x2E66)
    ]
    y = O.to_fp16(np.array([c[0] for c in cases], dtype=np.float64))
    assert y.dtype == np.float16
    for (v, want), got in zip(cases, y.astype(np.float64)):
        assert got == want, (v, got, want)


# --------------------------------------------------------------------------- P6 a-priori error bound (quality)
@pytest.mark.parametrize("key", ["T"])
def test_p6_error_bound_vs_fp64(key):
    x, w, _ = synth.make_inputs(synth.get(key))
    perm = O.outlier_perm(x)
    _, y64, _, _ = O.linear(x, w, perm)
    qx, sx = O.quantize_rows(x, perm)
    qw, sw = O.quantize_rows(w, perm)
    K = x.shape[1]
    xr = x[:, perm].astype(np.float64)
    wr = w[:, perm].astype(np.float64)
    sxe = O._expand(sx, K)
    swe = O._expand(sw, K)
    bound = (np.abs(xr) / 2) @ swe.T + sxe @ (np.abs(wr) / 2).T + (sxe / 4) @ swe.T
    yfp = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.all(np.abs(y64 - yfp) <= bound * (1 + 4e-6) + 1e-12)
    # and the quantized layer is far closer to the fp64 product than the bound's scale
    assert np.sqrt(np.mean((y64 - yfp) ** 2)) < 0.25 * np.sqrt(np.mean(yfp ** 2))


# --------------------------------------------------------------------------- P7 outlier recovery + tail placement
@pytest.mark.parametrize("key", ["T", "B"])
def test_p7_seeded_outliers_recovered(key):
    x, _, idx = synth.make_inputs(synth.get(key), with_w=False)
    sel = O.select_outliers(O.channel_stat(x))
    np.testing.assert_array_equal(sel, idx)
    perm = O.make_perm(x.shape[1], sel)
    assert sorted(perm[-128:].tolist()) == idx.tolist()          # outliers land in the INT8 tail
    assert np.all(np.diff(perm[:-128]) > 0) and np.all(np.diff(perm[-128:]) > 0)
    assert sorted(perm.tolist()) == list(range(x.shape[1]))


def test_p7_laplace_outliers_inside_selection():
    x, _, idx = synth.make_inputs(synth.get("A"), with_w=False)
    sel = O.select_outliers(O.channel_stat(x))
    assert set(idx.tolist()) <= set(sel.tolist())
    assert len(idx) == 41


def test_p7_quant_only_outliers_recovered():
    x, idx, _ = synth.quant_only_x(rows=2048)
    sel = O.select_outliers(O.channel_stat(x))
    np.testing.assert_array_equal(sel, idx)


# --------------------------------------------------------------------------- statistic + selection rule
def test_channel_stat_is_correctly_rounded_exact_sum():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((37, 9)) * np.exp(rng.uniform(-12, 10, size=(37, 9)))).astype(np.float16)
    st = O.channel_stat(x)
    for c in range(9):
        exact = sum(Fraction(float(v)) ** 2 for v in x[:, c].astype(np.float64))
        assert st[c] == float(exact)                     # Fraction -> float rounds to nearest
    # order of the rows does not matter
    np.testing.assert_array_equal(O.channel_stat(x[::-1]), st)


def test_selection_ties_go_to_lower_index():
    stat = np.zeros(300)
    stat[::2] = 5.0                    # 150 tied channels, only 128 are taken
    sel = O.select_outliers(stat)
    np.testing.assert_array_equal(sel, np.arange(0, 256, 2))
    stat2 = np.arange(300, dtype=np.float64)
    np.testing.assert_array_equal(O.select_outliers(stat2), np.arange(172, 300))


# --------------------------------------------------------------------------- P8 edge groups
def test_p8_edge_groups():
    K = 512
    X = np.zeros((4, K), dtype=np.float16)
    X[1, :128] = np.float16(2.0 ** -24)          # scale underflows -> codes 0
    X[2, 128:256] = np.float16(1e-6)             # subnormal scale
    X[2, 130] = np.float16(-3e-7)
    X[3] = np.float16(1.0)
    perm = np.arange(K, dtype=np.int32)
    q, s = O.quantize_rows(X, perm)
    assert np.all(q[0] == 0) and np.all(s[:, 0] == 0)
    assert np.all(q[1, :128] == 0) and s[0, 1] == 0
    # subnormal scale: the fallback bound max(s*(1/2 + 2^-21), a - qmax*s)
    sv = float(s[1, 2])
    assert 0 < sv < 2.0 ** -14
    xr = X[2, 128:256].astype(np.float64)
    a = np.abs(xr).max()
    err = np.abs(xr - q[2, 128:256].astype(np.float64) * sv)
    assert np.all(err <= max(sv * (0.5 + 2.0 ** -21), a - 7 * sv) + 1e-30)
    assert np.all(q[3, :K - 128] == 7) and np.all(q[3, K - 128:] == 127)
    w = np.ones((2, K), dtype=np.float16)
    _, y64, _, _ = O.linear(X, w, perm)
    assert np.all(y64[0] == 0)


def test_shape_rules():
    assert O.row_bytes(4096) == 2112 and O.num_groups(4096) == 32
    assert O.row_bytes(11008) == 5568 and O.num_groups(11008) == 86
    for bad in (128, 100, 1000):
        with pytest.raises(ValueError):
            O.num_groups(bad)
