"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Bar: outlier statistic, perm, packed INT4/INT8 codes, fp16 scales and the per-group int32
accumulators are bit-exact; the fp16 output Y is within max(2e-3*|Y64|, 1e-2) of the
oracle's fp64 value.  Every input comes from ``synth`` (seeded); every expected value
from ``oracle``.  Calls go through the C ABI via the ctypes binding.
"""
import functools
import json
import os
import sys

import numpy as np
import pytest

import synth
from oracle import atom_oracle as O

torch = pytest.importorskip("torch")
import bit_quantized_gemm_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL, ATOL = 2e-3, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bq.load_library()           # fails loudly if the HIP library is missing


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_y_close(y16, y64, what):
    y = y16.astype(np.float64)
    err = np.abs(y - y64)
    tol = np.maximum(RTOL * np.abs(y64), ATOL)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                           f"worst err {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}")


# --------------------------------------------------------------------------- workload cache
@functools.lru_cache(maxsize=2)
def workload(key):
    w = synth.get(key)
    _say(f"[inputs] {key} {w.name}")
    x, wt, _ = synth.make_inputs(w)
    perm = O.outlier_perm(x)
    return w, x, wt, perm


# --------------------------------------------------------------------------- a0: statistic + selection
@pytest.mark.parametrize("key", ["T", "A", "B", "C"])
def test_channel_stat_and_perm_bitexact(key):
    w, x, _, perm = workload(key)
    _say(f"[a0] {key} M={w.M} K={w.K}")
    X = dev(x.view(np.float16))
    stat = bq.atom_channel_stat(X)
    p = bq.atom_select_outliers(stat)
    st_ref = O.channel_stat(x)
    np.testing.assert_array_equal(host(stat).view(np.uint64), st_ref.view(np.uint64))
    np.testing.assert_array_equal(host(p), perm)


def test_select_ties_and_order():
    """Ties go to the lower channel index; the perm is a stable partition."""
    K = 1024
    stat = np.zeros(K)
    stat[::3] = 2.0                     # 342 tied channels
    stat[5] = 7.0
    p = bq.atom_select_outliers(dev(stat))
    ref = O.make_perm(K, O.select_outliers(stat))
    np.testing.assert_array_equal(host(p), ref)


# --------------------------------------------------------------------------- a1/a2: quantize
def _check_rows(x, perm, q_dev, s_dev, rows=None, what=""):
    xs = x if rows is None else x[rows]
    qr, sr = O.quantize_rows(xs, perm)
    q = host(q_dev)
    s = host(s_dev)
    if rows is not None:
        q = q[rows]
        s = s[:, rows]
    np.testing.assert_array_equal(q, O.pack_rows(qr), err_msg=f"{what} codes")
    np.testing.assert_array_equal(s.view(np.uint16), sr.view(np.uint16), err_msg=f"{what} scales")


@pytest.mark.parametrize("key", ["T", "A", "B", "C"])
def test_quantize_act_bitexact(key):
    w, x, _, perm = workload(key)
    _say(f"[a2] {key}")
    Xq, sx = bq.atom_quantize_act(dev(x), dev(perm))
    _check_rows(x, perm, Xq, sx, what=f"{key} activations")


@pytest.mark.parametrize("key", ["T", "A", "B", "C"])
def test_pack_weights_bitexact(key):
    w, _, wt, perm = workload(key)
    _say(f"[a1] {key}")
    Wq, sw = bq.atom_pack_weights(dev(wt), dev(perm))
    _check_rows(wt, perm, Wq, sw, what=f"{key} weights")


def test_quantize_only_8192_bitexact():
    """The standalone 8192x8192 activation quantize (128 channels x30)."""
    x, _, _ = synth.quant_only_x()
    _say("[a2] Dq 8192x8192")
    perm = O.outlier_perm(x[:2048])     # calibration on a prefix keeps the oracle quick
    Xq, sx = bq.atom_quantize_act(dev(x), dev(perm))
    _check_rows(x, perm, Xq, sx, what="Dq")


def test_golden_rows_on_gpu():
    """The hand-worked rows of tests/golden/worked_rows.json, quantized on the GPU."""
    fx = json.load(open(os.path.join(GOLDEN, "worked_rows.json")))
    K = fx["K"]
    X = np.zeros((len(fx["rows"]), K), dtype=np.float16)
    for r, row in enumerate(fx["rows"]):
        for c, hx in row["x_fp16_hex"].items():
            X[r, int(c)] = np.array([int(hx, 16)], np.uint16).view(np.float16)[0]
    Xq, sx = bq.atom_quantize_act(dev(X), dev(np.arange(K, dtype=np.int32)))
    q, s = host(Xq), host(sx)
    for r, row in enumerate(fx["rows"]):
        assert s[:, r].view(np.uint16).tolist() == [int(h, 16) for h in row["scales_fp16_hex"]], row["name"]
        exp = np.zeros(O.row_bytes(K), np.uint8)
        for c, hx in row["packed_hex"].items():
            exp[int(c) if int(c) < 128 else int(c) - 128 + (K - 128) // 2] = int(hx, 16)
        np.testing.assert_array_equal(q[r], exp, err_msg=row["name"])


# --------------------------------------------------------------------------- a3/a4: group accumulators
@pytest.mark.parametrize("key", ["T", "A"])
def test_group_acc_bitexact(key):
    w, x, wt, perm = workload(key)
    _say(f"[acc] {key}")
    qx, _ = O.quantize_rows(x, perm)
    qw, _ = O.quantize_rows(wt, perm)
    Xq, _ = bq.atom_quantize_act(dev(x), dev(perm))
    Wq, _ = bq.atom_pack_weights(dev(wt), dev(perm))
    acc = host(bq.atom_gemm_group_acc(Xq, Wq, w.K))
    np.testing.assert_array_equal(acc, O.group_acc(qx, qw))


@pytest.mark.parametrize("key,extra_rows,ncols", [("B", 256, 384), ("C", 0, 256)])
def test_group_acc_bitexact_llama_shapes(key, extra_rows, ncols):
    """Per-group accumulators bit-exact on the real packed operands of the Llama-7B MLP shapes,
    with at least 1152 activation-side rows so the banded tile order (bands of 8 tile rows of
    128) runs past its first band: C with all 2048 token rows (two bands), B with its 1024 token
    rows followed by 256 of its packed weight rows (a partial second band of 2 tile rows)."""
    w, x, wt, perm = workload(key)
    _say(f"[acc] {key} llama shape, {w.M + extra_rows} x {ncols}")
    Pd = dev(perm)
    Xq, _ = bq.atom_quantize_act(dev(x), Pd)
    Wq, _ = bq.atom_pack_weights(dev(wt), Pd)
    A = torch.cat([Xq, Wq[:extra_rows]]).contiguous() if extra_rows else Xq
    Bm = Wq[:ncols].contiguous()
    acc = host(bq.atom_gemm_group_acc(A, Bm, w.K))
    qx, _ = O.quantize_rows(x, perm)
    qw, _ = O.quantize_rows(wt[:max(ncols, extra_rows)], perm)
    qa = np.concatenate([qx, qw[:extra_rows]]) if extra_rows else qx
    ref = O.group_acc(qa, qw[:ncols])
    assert acc.shape == ref.shape and acc.shape[1] >= 1152
    np.testing.assert_array_equal(acc, ref)


@pytest.mark.parametrize("M,N", [(15, 40), (45, 150)])
def test_oracle_packed_units_every_code_in_every_field(M, N):
    """The GEMMs read packed rows written by the oracle's packer (not by the GPU quantize):
    every INT4 code value sits in every field position of a 16-code unit, the folded third
    word included, and the INT8 group spans [-127, 127].  Group accumulators bit-exact and Y
    within tolerance, on the few-rows kernel (M = 15) and on the tiled kernel (M = 45):
    atom_gemm_group_acc runs the kernel atom_gemm runs for the shape."""
    K = 1152
    klo, G = K - O.OUTLIERS, K // O.GROUP
    _say(f"[units] M={M} N={N} K={K}")
    m, n, k = np.arange(M)[:, None], np.arange(N)[:, None], np.arange(K)[None, :]
    qx = ((m + k) % 15 - 7).astype(np.int8)                     # rows cycle through all 15 codes
    qw = ((n + 7 * k + k // 16) % 15 - 7).astype(np.int8)
    qx[:, klo:] = ((37 * m + 11 * k[:, klo:]) % 255 - 127).astype(np.int8)
    qw[:, klo:] = ((53 * n + 5 * k[:, klo:]) % 255 - 127).astype(np.int8)
    for i in range(16):                                          # coverage of the test itself
        assert len(np.unique(qx[:, :klo][:, i::16])) == 15 and len(np.unique(qw[:, :klo][:, i::16])) == 15
    Xq, Wq = dev(O.pack_rows(qx)), dev(O.pack_rows(qw))
    np.testing.assert_array_equal(host(bq.atom_gemm_group_acc(Xq, Wq, K)), O.group_acc(qx, qw))
    sx = (2.0 ** -(6 + (np.arange(G)[:, None] + m.T) % 5) * (1 + (m.T % 3) / 4)).astype(np.float16)
    sw = (2.0 ** -(4 + (2 * np.arange(G)[:, None] + n.T) % 7) * (1 + (n.T % 5) / 8)).astype(np.float16)
    Y = host(bq.atom_gemm(Xq, dev(sx), Wq, dev(sw), K))
    assert_y_close(Y, O.gemm_ref(qx, sx, qw, sw), f"units {M}x{N}")


@pytest.mark.parametrize("M,N,K", [(5, 8200, 1152), (16, 9000, 4224), (2, 11008, 4096)])
def test_few_rows_wide_n_accumulators_bitexact(M, N, K):
    """Few rows, many columns and at most 32 INT4 groups: the few-rows kernel's ranges of up to
    8 groups (4 waves per workgroup).  Per-group accumulators bit-exact against the oracle."""
    _say(f"[few rows acc] M={M} N={N} K={K}")
    x, wt, _ = synth.make_linear(M, K, N, seed=M + N + 7 * K)
    perm = np.random.default_rng(K + 1).permutation(K).astype(np.int32)
    Xq, _ = bq.atom_quantize_act(dev(x), dev(perm))
    Wq, _ = bq.atom_pack_weights(dev(wt), dev(perm))
    acc = host(bq.atom_gemm_group_acc(Xq, Wq, K))
    qx, _ = O.quantize_rows(x, perm)
    qw, _ = O.quantize_rows(wt, perm)
    np.testing.assert_array_equal(acc, O.group_acc(qx, qw))


# --------------------------------------------------------------------------- a5: output
@pytest.mark.parametrize("key", ["T", "A", "B", "C"])
def test_gemm_full_output(key):
    """Every element of Y for the tiny workload and the three Llama-7B shapes (the oracle's
    fp64 dequantise-then-matmul takes a few seconds at 2048 x 4096 x 11008)."""
    w, x, wt, perm = workload(key)
    _say(f"[Y] {key} full")
    Wq, sw = bq.atom_pack_weights(dev(wt), dev(perm))
    Y = host(bq.linear(dev(x), dev(perm), Wq, sw))
    _, y64, _, _ = O.linear(x, wt, perm)
    assert_y_close(Y, y64, key)


def test_gemm_llama70b_sampled():
    """Llama-70B MLP shape M=4096, K=8192, N=28672: codes of sampled rows bit-exact, Y sampled."""
    w = synth.get("D")
    _say("[Y] D sampled")
    x, wt, _ = synth.make_inputs(w)
    perm = O.outlier_perm(x[:1024])
    Xd, Pd = dev(x), dev(perm)
    Wq, sw = bq.atom_pack_weights(dev(wt), Pd)
    Xq, sx = bq.atom_quantize_act(Xd, Pd)
    Y = bq.atom_gemm(Xq, sx, Wq, sw, w.K)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(w.M, 256, replace=False))
    cols = np.sort(rng.choice(w.N, 1024, replace=False))
    _check_rows(x, perm, Xq, sx, rows=rows, what="D activations")
    _check_rows(wt, perm, Wq, sw, rows=cols, what="D weights")
    qx, sxr = O.quantize_rows(x[rows], perm)
    qw, swr = O.quantize_rows(wt[cols], perm)
    assert_y_close(host(Y)[np.ix_(rows, cols)], O.gemm_ref(qx, sxr, qw, swr), "D")
    # per-group accumulators bit-exact on a seeded slice: 1152 token rows (two tile-row bands)
    # against 384 weight rows, gathered from the packed operands of the full-size pack
    arows = np.sort(rng.choice(w.M, 1152, replace=False))
    acols = np.sort(rng.choice(w.N, 384, replace=False))
    ti = lambda a: torch.from_numpy(a).cuda()
    acc = host(bq.atom_gemm_group_acc(Xq.index_select(0, ti(arows)).contiguous(),
                                      Wq.index_select(0, ti(acols)).contiguous(), w.K))
    qxa, _ = O.quantize_rows(x[arows], perm)
    qwa, _ = O.quantize_rows(wt[acols], perm)
    np.testing.assert_array_equal(acc, O.group_acc(qxa, qwa))


def _exact_operands(M, N, K, seed):
    """Oracle-packed operands on which every step of the production GEMM is exact: codes in
    [-1, 1] (INT4 groups) and [-3, 3] (INT8 group), scales 2^-1 or 2^-2 by group and row.  Each
    term acc_g * sx * sw is then a multiple of 2^-4, every fp32 partial sum is exact, and Y is
    exactly representable in fp16 while |Y| < 64 (about 6 standard deviations here), so the
    kernel's Y must equal the oracle's bit for bit and a single accumulator off by one shows."""
    rng = np.random.default_rng(seed)
    klo, G = K - O.OUTLIERS, K // O.GROUP
    qx = rng.integers(-1, 2, size=(M, K), dtype=np.int8)
    qw = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    qx[:, klo:] = rng.integers(-3, 4, size=(M, O.OUTLIERS), dtype=np.int8)
    qw[:, klo:] = rng.integers(-3, 4, size=(N, O.OUTLIERS), dtype=np.int8)
    sx = np.where(rng.integers(0, 2, size=(G, M)) == 0, 0.5, 0.25).astype(np.float16)
    sw = np.where(rng.integers(0, 2, size=(G, N)) == 0, 0.5, 0.25).astype(np.float16)
    y64 = O.gemm_ref(qx, sx, qw, sw)
    inside = np.abs(y64) < 64
    assert inside.mean() > 0.999, "the exact window must hold nearly every output"
    return qx, sx, qw, sw, O.to_fp16(y64)


@pytest.mark.parametrize("key", ["A", "B", "C"])
def test_gemm_exact_y_llama_shapes(key):
    """The production GEMM of each Llama-7B shape (A: 64 x 64 tiles in two K parts; B: 688
    tiles of 128 x 128 over several rounds, later ones at priority 1; C: one round with fair
    turns), on operands where every fp32 step is exact: Y bit-identical to the oracle's, so the
    per-group integer sums inside the kernel that atom_gemm runs are exact at full size."""
    w = synth.get(key)
    _say(f"[exact Y] {key} {w.M}x{w.N}x{w.K}")
    qx, sx, qw, sw, y16 = _exact_operands(w.M, w.N, w.K, seed=11 + w.M)
    Y = host(bq.atom_gemm(dev(O.pack_rows(qx)), dev(sx), dev(O.pack_rows(qw)), dev(sw), w.K))
    np.testing.assert_array_equal(Y.view(np.uint16), y16.view(np.uint16))


@pytest.mark.parametrize("M,N,K", [(64, 4096, 11008), (16, 11008, 4096)])
def test_gemm_exact_y_split_and_few_rows(M, N, K):
    """The same exactness through split-K (atom_gemm and atom_gemm_ws) and the few-rows kernel
    (M <= 16) at Llama widths."""
    _say(f"[exact Y] M={M} N={N} K={K}")
    qx, sx, qw, sw, y16 = _exact_operands(M, N, K, seed=M + N + K)
    args = (dev(O.pack_rows(qx)), dev(sx), dev(O.pack_rows(qw)), dev(sw), K)
    need = bq.atom_gemm_workspace_bytes(M, N, K)
    outs = [host(bq.atom_gemm(*args))]
    if need:
        ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
        outs.append(host(bq.atom_gemm_ws(*args, ws)))
    for Y in outs:
        np.testing.assert_array_equal(Y.view(np.uint16), y16.view(np.uint16))


# --------------------------------------------------------------------------- ragged / edge shapes
RAGGED = [(1, 1, 256), (2, 3, 256), (37, 200, 384), (130, 129, 1152), (257, 513, 640), (16, 512, 1024),
          (128, 128, 256), (129, 255, 2048), (33, 70, 12416), (20, 48, 16384), (9, 40, 20480),
          # 288 tiles: one round, the fair-turns kernel; 860 tiles: several rounds, later ones at priority 1
          (1100, 4000, 640), (1200, 11000, 384)]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_shapes(M, N, K):
    _say(f"[ragged] M={M} N={N} K={K}")
    x, wt, _ = synth.make_linear(M, K, N, seed=M + N + K)
    perm = np.random.default_rng(K).permutation(K).astype(np.int32)
    Xd, Wd, Pd = dev(x), dev(wt), dev(perm)
    Xq, sx = bq.atom_quantize_act(Xd, Pd)
    Wq, sw = bq.atom_pack_weights(Wd, Pd)
    Y = bq.atom_gemm(Xq, sx, Wq, sw, K)
    acc = bq.atom_gemm_group_acc(Xq, Wq, K)
    qx, sxr = O.quantize_rows(x, perm)
    qw, swr = O.quantize_rows(wt, perm)
    np.testing.assert_array_equal(host(Xq), O.pack_rows(qx))
    np.testing.assert_array_equal(host(Wq), O.pack_rows(qw))
    np.testing.assert_array_equal(host(sx).view(np.uint16), sxr.view(np.uint16))
    np.testing.assert_array_equal(host(acc), O.group_acc(qx, qw))
    assert_y_close(host(Y), O.gemm_ref(qx, sxr, qw, swr), f"{M}x{N}x{K}")


def test_zero_and_degenerate_rows():
    M, N, K = 64, 96, 512
    x, wt, _ = synth.make_linear(M, K, N, seed=9)
    x[3] = 0                                   # all-zero token
    x[5, :] = np.float16(2.0 ** -24)           # scales underflow to zero
    x[7, :128] = np.float16(1e-6)              # subnormal scale in group 0
    wt[10] = 0                                 # all-zero weight row
    perm = np.arange(K, dtype=np.int32)
    Xq, sx = bq.atom_quantize_act(dev(x), dev(perm))
    Wq, sw = bq.atom_pack_weights(dev(wt), dev(perm))
    Y = host(bq.atom_gemm(Xq, sx, Wq, sw, K))
    y16, y64, (xq_r, sx_r), (wq_r, sw_r) = O.linear(x, wt, perm)
    np.testing.assert_array_equal(host(Xq), xq_r)
    np.testing.assert_array_equal(host(sx).view(np.uint16), sx_r.view(np.uint16))
    np.testing.assert_array_equal(host(Wq), wq_r)
    assert np.all(Y[3] == 0) and np.all(Y[5] == 0) and np.all(Y[:, 10] == 0)
    assert_y_close(Y, y64, "degenerate")


def test_max_k():
    M, N, K = 8, 40, bq.MAX_K
    x, wt, _ = synth.make_linear(M, K, N, seed=1)
    perm = np.random.default_rng(2).permutation(K).astype(np.int32)
    Xq, sx = bq.atom_quantize_act(dev(x), dev(perm))
    Wq, sw = bq.atom_pack_weights(dev(wt), dev(perm))
    Y = host(bq.atom_gemm(Xq, sx, Wq, sw, K))
    qx, sxr = O.quantize_rows(x, perm)
    qw, swr = O.quantize_rows(wt, perm)
    np.testing.assert_array_equal(host(Xq), O.pack_rows(qx))
    assert_y_close(Y, O.gemm_ref(qx, sxr, qw, swr), "max K")


def test_max_k_statistic_quantize_tiles_and_split():
    """K = ATOM_MAX_K through what a long K takes beyond the few-rows kernel: the statistic and
    the outlier selection (one flag byte per channel in LDS), the quantize's general
    instantiation (a 128 KiB staged row, more rows than resident workgroups), the 128 x 128
    kernel over 512 groups (accumulators bit-exact) and split-K."""
    M, N, K = 300, 136, bq.MAX_K
    x, wt, _ = synth.make_linear(M, K, N, seed=3)
    _say(f"[max K] M={M} N={N} K={K}")
    X = dev(x)
    p = bq.atom_select_outliers(bq.atom_channel_stat(X))
    perm = O.outlier_perm(x)
    np.testing.assert_array_equal(host(p), perm)
    Xq, sx = bq.atom_quantize_act(X, p)
    Wq, sw = bq.atom_pack_weights(dev(wt), p)
    qx, sxr = O.quantize_rows(x, perm)
    qw, swr = O.quantize_rows(wt, perm)
    np.testing.assert_array_equal(host(Xq), O.pack_rows(qx))
    np.testing.assert_array_equal(host(sx).view(np.uint16), sxr.view(np.uint16))
    np.testing.assert_array_equal(host(Wq), O.pack_rows(qw))
    acc = host(bq.atom_gemm_group_acc(Xq[:130], Wq, K))
    np.testing.assert_array_equal(acc, O.group_acc(qx[:130], qw))
    y64 = O.gemm_ref(qx, sxr, qw, swr)
    assert_y_close(host(bq.atom_gemm(Xq, sx, Wq, sw, K)), y64, "max K, whole tiles")
    need = bq.atom_gemm_workspace_bytes(M, N, K)
    assert need > 0, "this shape is expected to split"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert_y_close(host(bq.atom_gemm_ws(Xq, sx, Wq, sw, K, ws)), y64, "max K, split-K")


# --------------------------------------------------------------------------- determinism and streams
def test_deterministic_and_side_stream():
    w, x, wt, perm = workload("A")
    Xd, Pd = dev(x), dev(perm)
    Wq, sw = bq.atom_pack_weights(dev(wt), Pd)
    y1 = host(bq.linear(Xd, Pd, Wq, sw))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = bq.linear(Xd, Pd, Wq, sw, stream=s)
    s.synchronize()
    y2 = host(y2)
    np.testing.assert_array_equal(y1.view(np.uint16), y2.view(np.uint16))


# --------------------------------------------------------------------------- split-K (atom_gemm_ws)
# pieces per split tile: 7, 3, 2, 4, 5, 6, 8; every piece count has its own finalize instance
SPLIT = [(64, 128, 4096), (200, 300, 2048), (17, 130, 1152), (64, 4096, 11008), (17, 64, 3072), (40, 200, 3456),
         (33, 250, 4352)]


@pytest.mark.parametrize("M,N,K", SPLIT)
def test_gemm_ws_split_matches_oracle(M, N, K):
    """Shapes with few tiles take the split-K path; Y stays within the oracle tolerance."""
    need = bq.atom_gemm_workspace_bytes(M, N, K)
    assert need > 0, "this shape is expected to split"
    _say(f"[split-K] M={M} N={N} K={K} workspace={need}")
    x, wt, _ = synth.make_linear(M, K, N, seed=3 * M + N + K)
    perm = np.random.default_rng(K + 1).permutation(K).astype(np.int32)
    Xd, Wd, Pd = dev(x), dev(wt), dev(perm)
    Xq, sx = bq.atom_quantize_act(Xd, Pd)
    Wq, sw = bq.atom_pack_weights(Wd, Pd)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")   # contents must not matter
    Y = host(bq.atom_gemm_ws(Xq, sx, Wq, sw, K, ws))
    qx, sxr = O.quantize_rows(x, perm)
    qw, swr = O.quantize_rows(wt, perm)
    assert_y_close(Y, O.gemm_ref(qx, sxr, qw, swr), f"split {M}x{N}x{K}")
    Y2 = host(bq.atom_gemm_ws(Xq, sx, Wq, sw, K, ws))          # deterministic: splits summed in order
    np.testing.assert_array_equal(Y.view(np.uint16), Y2.view(np.uint16))


# Grids with few 128 x 128 tiles but enough of 64 x 64 run whole 64 x 64 tiles (no split, no
# scratch).  With at least 4 INT4 groups each workgroup splits K between two parts (K parts): the
# Llama-7B attention projection, ragged edges, odd and even INT4 group counts (the part with one
# group fewer passes one extra barrier: K = 640: 4 INT4 groups, 4096: 31, 1152: 8, 11008: 85),
# and shapes that split-K would otherwise take (128, 64 and 33 rows).  K = 256 and 512 leave
# too few groups to divide and run whole tiles of two waves.
TILE64 = [(256, 4096, 4096), (200, 4000, 640), (130, 5000, 1152), (100, 6100, 11008), (255, 3100, 4096),
          (128, 4096, 4096), (64, 4096, 4096), (33, 8448, 4096), (100, 2048, 4096), (200, 4000, 512), (255, 3100, 256)]


@pytest.mark.parametrize("M,N,K", TILE64)
def test_gemm_tile64_matches_oracle(M, N, K):
    _say(f"[64 x 64 tiles] M={M} N={N} K={K}")
    assert bq.atom_gemm_workspace_bytes(M, N, K) == 0
    x, wt, _ = synth.make_linear(M, K, N, seed=5 * M + N + K)
    perm = np.random.default_rng(K + 7).permutation(K).astype(np.int32)
    Xq, sx = bq.atom_quantize_act(dev(x), dev(perm))
    Wq, sw = bq.atom_pack_weights(dev(wt), dev(perm))
    Y = host(bq.atom_gemm(Xq, sx, Wq, sw, K))
    qx, sxr = O.quantize_rows(x, perm)
    qw, swr = O.quantize_rows(wt, perm)
    assert_y_close(Y, O.gemm_ref(qx, sxr, qw, swr), f"tile64 {M}x{N}x{K}")
    if N * M * (K // 128) <= 40_000_000:
        np.testing.assert_array_equal(host(bq.atom_gemm_group_acc(Xq, Wq, K)), O.group_acc(qx, qw))
    for y2 in (bq.atom_gemm(Xq, sx, Wq, sw, K), bq.atom_gemm_ws(Xq, sx, Wq, sw, K, None)):
        np.testing.assert_array_equal(Y.view(np.uint16), host(y2).view(np.uint16))


def test_gemm_ws_without_enough_scratch_is_atom_gemm():
    M, N, K = 64, 128, 4096
    x, wt, _ = synth.make_linear(M, K, N, seed=11)
    perm = np.arange(K, dtype=np.int32)
    Xq, sx = bq.atom_quantize_act(dev(x), dev(perm))
    Wq, sw = bq.atom_pack_weights(dev(wt), dev(perm))
    ref = host(bq.atom_gemm(Xq, sx, Wq, sw, K))
    small = torch.empty(bq.atom_gemm_workspace_bytes(M, N, K) - 16, dtype=torch.uint8, device="cuda")
    for ws in (None, small):
        y = host(bq.atom_gemm_ws(Xq, sx, Wq, sw, K, ws))
        np.testing.assert_array_equal(y.view(np.uint16), ref.view(np.uint16))



# --------------------------------------------------------------------------- few rows (M <= 16)
SMALL = [(1, 4096, 4096), (16, 11008, 4096), (16, 4096, 11008), (3, 131, 2048), (7, 37, 256), (16, 16, 1152),
         (5, 200, 32768), (12, 1000, 1408), (3, 9000, 2048), (16, 8200, 4224)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_gemm_small_m_matches_oracle(M, N, K):
    """M <= 16 runs the few-rows kernel (K ranges of 4, 6 or 8 INT4 groups, one wave each, added
    in LDS): Y against the oracle on up to 512 sampled columns (all of them for small N), and
    bit-identical on a second call and through atom_gemm_ws."""
    _say(f"[few rows] M={M} N={N} K={K}")
    assert bq.atom_gemm_workspace_bytes(M, N, K) == 0
    x, wt, _ = synth.make_linear(M, K, N, seed=M * 131 + N + K)
    perm = np.random.default_rng(K + 3).permutation(K).astype(np.int32)
    Xq, sx = bq.atom_quantize_act(dev(x), dev(perm))
    Wq, sw = bq.atom_pack_weights(dev(wt), dev(perm))
    Y = host(bq.atom_gemm(Xq, sx, Wq, sw, K))
    cols = np.arange(N) if N <= 512 else np.sort(np.random.default_rng(9).choice(N, 512, replace=False))
    qx, sxr = O.quantize_rows(x, perm)
    qw, swr = O.quantize_rows(wt[cols], perm)
    assert_y_close(Y[:, cols], O.gemm_ref(qx, sxr, qw, swr), f"few rows {M}x{N}x{K}")
    for y2 in (bq.atom_gemm(Xq, sx, Wq, sw, K), bq.atom_gemm_ws(Xq, sx, Wq, sw, K, None)):
        np.testing.assert_array_equal(Y.view(np.uint16), host(y2).view(np.uint16))


# --------------------------------------------------------------------------- HIP graph capture
def test_graph_capture_replays_match_eager():
    """The library allocates and synchronizes nothing, so quantize + GEMM can be captured in a
    HIP graph.  Six shapes cover the GEMM paths (64 x 64 tiles in K parts, split-K with its
    finalize kernel, whole 128 x 128 tiles in one partial round, in one full round with fair turns
    (512 tiles) and over several rounds with later ones at priority 1 (567 tiles), few rows); the
    graph is replayed several times with unrelated eager work and new inputs in between, and
    every replay must equal the eager result bit for bit."""
    cases = [(256, 4096, 4096), (64, 2048, 4096), (1024, 2048, 1024), (2048, 4096, 512), (1100, 8000, 384),
             (16, 2000, 11008)]
    st = torch.cuda.Stream()
    bufs = []
    for i, (M, N, K) in enumerate(cases):
        x, wt, _ = synth.make_linear(M, K, N, seed=40 + i)
        perm = dev(np.random.default_rng(i).permutation(K).astype(np.int32))
        Wq, sw = bq.atom_pack_weights(dev(wt), perm)
        need = bq.atom_gemm_workspace_bytes(M, N, K)
        b = dict(K=K, X=dev(x), perm=perm, Wq=Wq, sw=sw,
                 Xq=torch.empty((M, bq.atom_row_bytes(K)), dtype=torch.uint8, device="cuda"),
                 sx=torch.empty((K // 128, M), dtype=torch.float16, device="cuda"),
                 Y=torch.empty((M, N), dtype=torch.float16, device="cuda"),
                 ws=torch.empty(need, dtype=torch.uint8, device="cuda") if need else None)
        bufs.append(b)

    def step():
        for b in bufs:
            bq.atom_quantize_act(b["X"], b["perm"], Xq=b["Xq"], sx=b["sx"], stream=st)
            bq.atom_gemm_ws(b["Xq"], b["sx"], b["Wq"], b["sw"], b["K"], b["ws"], Y=b["Y"], stream=st)

    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()                                   # warm up (first-use queries happen outside capture)
    st.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for b in bufs:                           # new activations each replay, plus eager noise
            b["X"].mul_(-1.0 if rep % 2 else 1.0)
            torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(b["Y"]).copy() for b in bufs]
        with torch.cuda.stream(st):
            step()                               # eager on the same inputs
        st.synchronize()
        for i, b in enumerate(bufs):
            np.testing.assert_array_equal(got[i].view(np.uint16), host(b["Y"]).view(np.uint16),
                                          err_msg=f"replay {rep}, shape {cases[i]}")
