"""GPU parity of the W4A8 variant (INT8 activations in every group, W4 weights) against the
CPU oracle (needs an MI355X).

Bar as for W4A4: packed codes, scales and per-group int32 accumulators bit-exact; Y within
max(2e-3*|Y64|, 1e-2) of the oracle's fp64 value.  Inputs from ``synth`` (seeded), expected
values from ``oracle``; calls through the C ABI via the ctypes binding.
"""
import functools
import sys

import numpy as np
import pytest

import synth
from oracle import atom_oracle as O

torch = pytest.importorskip("torch")
import bit_quantized_gemm_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu
RTOL, ATOL = 2e-3, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bq.load_library()


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


@functools.lru_cache(maxsize=2)
def workload(key):
    w = synth.get(key)
    _say(f"[inputs] {key} {w.name}")
    x, wt, _ = synth.make_inputs(w)
    perm = O.outlier_perm(x)
    return x, wt, perm


def _quantized(x, wt, perm):
    Xd, Wd, Pd = dev(x), dev(wt), dev(perm)
    Xq, sx = bq.atom_quantize_act_a8(Xd, Pd)
    Wq, sw = bq.atom_pack_weights_w4a8(Wd, Pd)
    return Xq, sx, Wq, sw


@pytest.mark.parametrize("key", ["T", "A", "B", "C"])
def test_w4a8_quantize_act_bitexact(key):
    x, _, perm = workload(key)
    _say(f"[w4a8 quantize] {key}")
    Xq, sx = bq.atom_quantize_act_a8(dev(x), dev(perm))
    qr, sr = O.quantize_rows(x, perm, all_int8=True)
    np.testing.assert_array_equal(host(Xq), O.pack_rows_a8(qr), err_msg=f"{key} A8 codes")
    np.testing.assert_array_equal(host(sx).view(np.uint16), sr.view(np.uint16), err_msg=f"{key} A8 scales")


@pytest.mark.parametrize("key", ["T", "A"])
def test_w4a8_pack_weights_bitexact(key):
    _, wt, perm = workload(key)
    _say(f"[w4a8 pack] {key}")
    Wq, sw = bq.atom_pack_weights_w4a8(dev(wt), dev(perm))
    qr, sr = O.quantize_rows(wt, perm)
    np.testing.assert_array_equal(host(Wq), O.pack_rows_w4a8(qr), err_msg=f"{key} W4A8 weight bytes")
    np.testing.assert_array_equal(host(sw).view(np.uint16), sr.view(np.uint16), err_msg=f"{key} weight scales")
    # the same codes and scales as the W4A4 pack, in the other layout
    Wq4, sw4 = bq.atom_pack_weights(dev(wt), dev(perm))
    np.testing.assert_array_equal(O.unpack_rows(host(Wq4), wt.shape[1]), O.unpack_rows_w4a8(host(Wq), wt.shape[1]))
    np.testing.assert_array_equal(host(sw4).view(np.uint16), host(sw).view(np.uint16))


# the last shape has 65 INT4 groups: the LDS-DMA ring kernel (pieces of at least 64 groups)
@pytest.mark.parametrize("M,N,K", [(16, 512, 1024), (37, 200, 384), (130, 129, 1152), (1, 3, 256), (37, 200, 8448)])
def test_w4a8_group_acc_bitexact(M, N, K):
    _say(f"[w4a8 acc] M={M} N={N} K={K}")
    x, wt, _ = synth.make_linear(M, K, N, seed=7 * M + N + K)
    perm = np.random.default_rng(K).permutation(K).astype(np.int32)
    Xq, _, Wq, _ = _quantized(x, wt, perm)
    acc = host(bq.atom_gemm_w4a8_group_acc(Xq, Wq, K))
    qx, _ = O.quantize_rows(x, perm, all_int8=True)
    qw, _ = O.quantize_rows(wt, perm)
    np.testing.assert_array_equal(acc, O.group_acc(qx, qw))


@pytest.mark.parametrize("key", ["T", "A", "B", "C"])
def test_w4a8_gemm_full_output(key):
    x, wt, perm = workload(key)
    _say(f"[w4a8 gemm] {key}")
    Xq, sx, Wq, sw = _quantized(x, wt, perm)
    Y = host(bq.atom_gemm_w4a8(Xq, sx, Wq, sw, x.shape[1]))
    qx, sxr = O.quantize_rows(x, perm, all_int8=True)
    qw, swr = O.quantize_rows(wt, perm)
    assert_y_close(Y, O.gemm_ref(qx, sxr, qw, swr), f"W4A8 {key}")


@pytest.mark.parametrize("key", ["A", "B", "C"])
def test_w4a8_exact_y_llama_shapes(key):
    """The W4A8 GEMM at the Llama-7B shapes (register-staged tiles on A and B, the LDS-DMA ring
    on C's long K) on oracle-packed operands where every fp32 step is exact: activation and
    INT4 weight codes in [-1, 1], INT8 weight codes in [-3, 3], scales 2^-1 or 2^-2.  Every term
    is a multiple of 2^-4 and |Y| < 64 is exact in fp16, so Y must equal the oracle's bit for
    bit and a single per-group sum off by one (the offset-binary correction included) shows."""
    w = synth.get(key)
    M, N, K = w.M, w.N, w.K
    _say(f"[w4a8 exact Y] {key} {M}x{N}x{K}")
    rng = np.random.default_rng(23 + M)
    klo, G = K - O.OUTLIERS, K // O.GROUP
    qx = rng.integers(-1, 2, size=(M, K), dtype=np.int8)
    qw = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    qw[:, klo:] = rng.integers(-3, 4, size=(N, O.OUTLIERS), dtype=np.int8)
    sx = np.where(rng.integers(0, 2, size=(G, M)) == 0, 0.5, 0.25).astype(np.float16)
    sw = np.where(rng.integers(0, 2, size=(G, N)) == 0, 0.5, 0.25).astype(np.float16)
    y64 = O.gemm_ref(qx, sx, qw, sw)
    assert (np.abs(y64) < 64).mean() > 0.999, "the exact window must hold nearly every output"
    Y = host(bq.atom_gemm_w4a8(dev(O.pack_rows_a8(qx)), dev(sx), dev(O.pack_rows_w4a8(qw)), dev(sw), K))
    np.testing.assert_array_equal(Y.view(np.uint16), O.to_fp16(y64).view(np.uint16))


RAGGED = [(1, 1, 256), (3, 70, 256), (129, 255, 2048), (200, 300, 640), (33, 70, 12416), (9, 40, 32768),
          (33, 70, bq.MAX_K)]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_w4a8_ragged_shapes(M, N, K):
    _say(f"[w4a8 ragged] M={M} N={N} K={K}")
    x, wt, _ = synth.make_linear(M, K, N, seed=M + 3 * N + K)
    perm = np.random.default_rng(K + 5).permutation(K).astype(np.int32)
    Xq, sx, Wq, sw = _quantized(x, wt, perm)
    qx, sxr = O.quantize_rows(x, perm, all_int8=True)
    qw, swr = O.quantize_rows(wt, perm)
    np.testing.assert_array_equal(host(Xq), O.pack_rows_a8(qx))
    np.testing.assert_array_equal(host(Wq), O.pack_rows_w4a8(qw))
    Y = host(bq.atom_gemm_w4a8(Xq, sx, Wq, sw, K))
    assert_y_close(Y, O.gemm_ref(qx, sxr, qw, swr), f"W4A8 ragged {M}x{N}x{K}")
    Y2 = host(bq.atom_gemm_w4a8(Xq, sx, Wq, sw, K))
    np.testing.assert_array_equal(Y.view(np.uint16), Y2.view(np.uint16))


def test_w4a8_zero_rows():
    M, N, K = 40, 64, 512
    x, wt, _ = synth.make_linear(M, K, N, seed=2)
    x[5] = 0
    x[17, :128] = 0
    perm = np.arange(K, dtype=np.int32)
    Xq, sx, Wq, sw = _quantized(x, wt, perm)
    qx, sxr = O.quantize_rows(x, perm, all_int8=True)
    np.testing.assert_array_equal(host(Xq), O.pack_rows_a8(qx))
    np.testing.assert_array_equal(host(sx).view(np.uint16), sxr.view(np.uint16))
    Y = host(bq.atom_gemm_w4a8(Xq, sx, Wq, sw, K))
    assert np.all(Y[5] == 0)
    qw, swr = O.quantize_rows(wt, perm)
    assert_y_close(Y, O.gemm_ref(qx, sxr, qw, swr), "W4A8 zero rows")


# pieces per split tile 7, 3, 2, 4 (the attention projection), 5, 6, 8, and a 16-row batch; the
# last shape splits 255 INT4 groups three ways, so its pieces (85 groups) take the ring kernel
W8_SPLIT = [(64, 128, 4096), (200, 300, 2048), (17, 130, 1152), (256, 4096, 4096), (17, 64, 3072),
            (40, 200, 3456), (33, 250, 4352), (16, 512, 4096), (129, 5504, 32768)]


@pytest.mark.parametrize("M,N,K", W8_SPLIT)
def test_w4a8_split_k_matches_oracle(M, N, K):
    need = bq.atom_gemm_w4a8_workspace_bytes(M, N, K)
    assert need > 0, "this shape is expected to split"
    _say(f"[w4a8 split-K] M={M} N={N} K={K} workspace={need}")
    x, wt, _ = synth.make_linear(M, K, N, seed=5 * M + N + K)
    perm = np.random.default_rng(K + 3).permutation(K).astype(np.int32)
    Xq, sx, Wq, sw = _quantized(x, wt, perm)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")   # contents must not matter
    Y = host(bq.atom_gemm_w4a8_ws(Xq, sx, Wq, sw, K, ws))
    qx, sxr = O.quantize_rows(x, perm, all_int8=True)
    qw, swr = O.quantize_rows(wt, perm)
    assert_y_close(Y, O.gemm_ref(qx, sxr, qw, swr), f"W4A8 split {M}x{N}x{K}")
    Y2 = host(bq.atom_gemm_w4a8_ws(Xq, sx, Wq, sw, K, ws))
    np.testing.assert_array_equal(Y.view(np.uint16), Y2.view(np.uint16))
    Yu = host(bq.atom_gemm_w4a8_ws(Xq, sx, Wq, sw, K, None))           # no scratch: the unsplit kernel
    np.testing.assert_array_equal(Yu.view(np.uint16), host(bq.atom_gemm_w4a8(Xq, sx, Wq, sw, K)).view(np.uint16))
    assert_y_close(Yu, O.gemm_ref(qx, sxr, qw, swr), f"W4A8 unsplit {M}x{N}x{K}")
