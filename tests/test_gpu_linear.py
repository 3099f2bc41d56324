"""GPU parity of atom_linear, the activation quantize and the GEMM in one call (needs an MI355X).

Shapes whose GEMM runs whole 128 x 128 tiles (K <= 12288) take one persistent launch: every
workgroup quantizes its share of the activation rows, then runs its share of the output tiles,
each after the tile's rows are counted as quantized.  Other shapes run the two kernels back to back.  Bar: Xq and sx bit-exact
against the oracle, Y within max(2e-3 |Y64|, 1e-2) of the oracle's fp64 value and bit-identical
to atom_quantize_act + atom_gemm (the same tile code computes it); the workspace's control words
are zero again after every call.
"""
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
    err = np.abs(y16.astype(np.float64) - y64)
    tol = np.maximum(RTOL * np.abs(y64), ATOL)
    assert not (err > tol).any(), f"{what}: worst err {err.max():.3g}"


def control_words_zero(ws, M):
    n = 16 + (M + 63) // 64
    return not host(ws[:4 * n].view(torch.int32)).any()


def case(M, N, K, seed):
    x, wt, _ = synth.make_linear(M, K, N, seed=seed)
    perm = np.random.default_rng(seed + 1).permutation(K).astype(np.int32)
    Xd, Pd = dev(x), dev(perm)
    Wq, sw = bq.atom_pack_weights(dev(wt), Pd)
    return x, wt, perm, Xd, Pd, Wq, sw


# whole 128 x 128 tiles (one launch): the two Llama-7B MLP shapes, ragged rows and columns (a
# 64-row block of one row), each quantize instantiation (K <= 4096, <= 8192, <= 12288)
FUSED = [(1024, 11008, 4096), (2048, 4096, 11008), (1000, 2100, 1152), (2049, 2000, 4224), (1500, 2560, 8192)]
# the other plans (two launches): 64 x 64 tiles, split-K, few rows
OTHER = [(256, 4096, 4096), (64, 2048, 4096), (16, 4096, 4096)]


@pytest.mark.parametrize("M,N,K", FUSED + OTHER)
def test_linear_matches_oracle_and_two_launches(M, N, K):
    _say(f"[linear] M={M} N={N} K={K}")
    x, wt, perm, Xd, Pd, Wq, sw = case(M, N, K, seed=M + 3 * N + K)
    ws = torch.zeros(bq.atom_linear_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    Y, Xq, sx = bq.atom_linear(Xd, Pd, Wq, sw, ws)
    qx, sxr = O.quantize_rows(x, perm)
    np.testing.assert_array_equal(host(Xq), O.pack_rows(qx))
    np.testing.assert_array_equal(host(sx).view(np.uint16), sxr.view(np.uint16))
    cols = np.arange(N) if N <= 2100 else np.sort(np.random.default_rng(1).choice(N, 1024, replace=False))
    qw, swr = O.quantize_rows(wt[cols], perm)
    y = host(Y)
    assert_y_close(y[:, cols], O.gemm_ref(qx, sxr, qw, swr), f"linear {M}x{N}x{K}")
    # the same result as the two separate calls, bit for bit
    Xq2, sx2 = bq.atom_quantize_act(Xd, Pd)
    need = bq.atom_gemm_workspace_bytes(M, N, K)
    y2 = host(bq.atom_gemm_ws(Xq2, sx2, Wq, sw, K, torch.empty(need, dtype=torch.uint8, device="cuda") if need else None))
    np.testing.assert_array_equal(y.view(np.uint16), y2.view(np.uint16))
    assert control_words_zero(ws, M) and not bq.linear_timed_out(ws)
    # repeated calls on the same workspace: identical, and the workspace stays clean
    for _ in range(2):
        Y3, _, _ = bq.atom_linear(Xd, Pd, Wq, sw, ws)
        np.testing.assert_array_equal(host(Y3).view(np.uint16), y.view(np.uint16))
    assert control_words_zero(ws, M)


def test_linear_graph_replays_match_eager():
    """atom_linear captured in a HIP graph (no memset: the kernel resets its own
    counters), replayed with new activations and unrelated eager work in between."""
    M, N, K = 1024, 4096, 4096
    x, wt, perm, Xd, Pd, Wq, sw = case(M, N, K, seed=77)
    ws = torch.zeros(bq.atom_linear_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    Xq = torch.empty((M, bq.atom_row_bytes(K)), dtype=torch.uint8, device="cuda")
    sx = torch.empty((K // 128, M), dtype=torch.float16, device="cuda")
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        bq.atom_linear(Xd, Pd, Wq, sw, ws, Xq=Xq, sx=sx, Y=Y, stream=st)
    st.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        bq.atom_linear(Xd, Pd, Wq, sw, ws, Xq=Xq, sx=sx, Y=Y, stream=st)
    torch.cuda.synchronize()
    for rep in range(4):
        Xd.mul_(-1.0 if rep % 2 else 1.0)
        torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(Y).copy()
        with torch.cuda.stream(st):
            bq.atom_linear(Xd, Pd, Wq, sw, ws, Xq=Xq, sx=sx, Y=Y, stream=st)
        st.synchronize()
        np.testing.assert_array_equal(got.view(np.uint16), host(Y).view(np.uint16), err_msg=f"replay {rep}")
        assert control_words_zero(ws, M) and not bq.linear_timed_out(ws)


def test_linear_forced_wait_failure_sets_flag_and_recovers():
    """Word 10 < 0 makes every tile's wait give up at once (a host-forced failure of the bounded
    wait): the launch still completes, the sticky flag (word 9) is set and the counters are
    reset; with words 9 and 10 cleared, the next call is exact again."""
    M, N, K = 1024, 2048, 4096
    x, wt, perm, Xd, Pd, Wq, sw = case(M, N, K, seed=91)
    ws = torch.zeros(bq.atom_linear_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    words = ws.view(torch.int32)
    words[10] = -1
    bq.atom_linear(Xd, Pd, Wq, sw, ws)
    torch.cuda.synchronize()
    assert bq.linear_timed_out(ws)
    w = host(words)
    assert not w[:9].any() and not w[16:16 + (M + 63) // 64].any()
    words[9] = 0
    words[10] = 0
    Y, Xq, sx = bq.atom_linear(Xd, Pd, Wq, sw, ws)
    qx, sxr = O.quantize_rows(x, perm)
    qw, swr = O.quantize_rows(wt, perm)
    assert_y_close(host(Y), O.gemm_ref(qx, sxr, qw, swr), "after recovery")
    assert control_words_zero(ws, M) and not bq.linear_timed_out(ws)
