"""atom_gemm_noalloc, the entry point that allocates nothing (needs an MI355X).

For callers that cannot allocate device memory: the split-K scratch is a static buffer inside
the library.  Its output must equal atom_gemm_ws with a caller workspace, bit for bit (the same
kernels and the same plan), on two calls in a row, the second with a smaller input: the buffer
keeps the first call's partial tiles, which the second call must not depend on.
"""
import sys

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
import bit_quantized_gemm_amd as bq  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bq.load_library()


def _operands(M, N, K, seed):
    x, wt, _ = synth.make_linear(M, K, N, seed=seed)
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(K).astype(np.int32)).cuda()
    Xq, sx = bq.atom_quantize_act(torch.from_numpy(x).cuda(), perm)
    Wq, sw = bq.atom_pack_weights(torch.from_numpy(wt).cuda(), perm)
    return Xq, sx, Wq, sw


def test_noalloc_matches_workspace_entry_point_twice():
    # 64 x 4096 x 11008: 32 tiles in 8 split pieces (16.8 MB of partials); then 64 x 2048: 16 tiles in 7
    for M, N, K in [(64, 4096, 11008), (64, 2048, 4096)]:
        print(f"[noalloc] M={M} N={N} K={K}", flush=True)
        need = bq.atom_gemm_workspace_bytes(M, N, K)
        assert need > 0, "the shape must use split-K scratch"
        Xq, sx, Wq, sw = _operands(M, N, K, seed=M + N)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = bq.atom_gemm_ws(Xq, sx, Wq, sw, K, ws)
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        bq.atom_gemm_noalloc(Xq, sx, Wq, sw, K, Y=Y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Y.cpu().numpy().view(np.uint16), ref.cpu().numpy().view(np.uint16))
    sys.stdout.flush()
