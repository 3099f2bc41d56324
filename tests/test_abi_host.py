"""Host-side checks of the C ABI (no GPU needed, no kernel is ever launched).

The library must load, export every function declared in include/atom.h, and reject every
invalid argument on the host before it touches the HIP runtime.  The calls below pass fake
(never dereferenced) addresses and always fail validation, so nothing is enqueued.
"""
import ctypes
import os
import re
import sys

import pytest

import bit_quantized_gemm_amd as bq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "atom.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_OVERLAP, E_HIP, E_SCRATCH = 0, 1, 2, 3, 4, 5, 6


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(atom_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bq.lib_path()):
        pytest.skip("libatom.so not built (python -m bit_quantized_gemm_amd.build)")
    return bq.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 20
    assert sorted(bq.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants():
    text = open(HEADER).read()
    assert re.search(r"#define ATOM_GROUP 128\b", text)
    assert re.search(r"#define ATOM_OUTLIERS 128\b", text)
    assert re.search(rf"#define ATOM_MAX_K {bq.MAX_K}\b", text)
    assert re.search(r"#define ATOM_MAX_TILES \(1 << 26\)", text)


def test_shape_helpers(lib):
    assert bq.atom_row_bytes(4096) == 2112
    assert bq.atom_row_bytes(11008) == 5568
    assert bq.atom_row_bytes(256) == 192
    assert bq.atom_num_groups(4096) == 32
    assert bq.atom_num_groups(11008) == 86
    for bad in (0, 128, 200, 4100, bq.MAX_K + 128, -256):
        assert bq.atom_row_bytes(bad) == -E_SHAPE
        assert bq.atom_num_groups(bad) == -E_SHAPE
    assert bq.atom_row_bytes(32768) == (32768 - 128) // 2 + 128
    assert bq.atom_row_bytes(bq.MAX_K) == (bq.MAX_K - 128) // 2 + 128


def test_strerror(lib):
    for s in (OK, E_NULL, E_SHAPE, E_ALIGN, E_OVERLAP, E_HIP, E_SCRATCH, 99):
        msg = bq.atom_strerror(s)
        assert isinstance(msg, str) and msg
    assert bq.atom_strerror(OK) == "ok"


A = 0x10000000          # fake, aligned, disjoint device addresses (never dereferenced)
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000
S = None                # default stream


def _q(lib, X, perm, M, K, Q, Sc):
    return lib.atom_quantize_act(X, perm, M, K, Q, Sc, S)


def test_quantize_validation(lib):
    assert _q(lib, None, B, 4, 256, C, D) == E_NULL
    assert _q(lib, A, None, 4, 256, C, D) == E_NULL
    assert _q(lib, A, B, 4, 256, None, D) == E_NULL
    assert _q(lib, A, B, 4, 256, C, None) == E_NULL
    for K in (0, 128, 300, bq.MAX_K + 128):
        assert _q(lib, A, B, 4, K, C, D) == E_SHAPE
    for M in (0, -1, (1 << 24) + 1):
        assert _q(lib, A, B, M, 256, C, D) == E_SHAPE
    assert _q(lib, A + 8, B, 4, 256, C, D) == E_ALIGN
    assert _q(lib, A, B + 4, 4, 256, C, D) == E_ALIGN
    assert _q(lib, A, B, 4, 256, C + 2, D) == E_ALIGN
    assert _q(lib, A, B, 4, 256, C, D + 1) == E_ALIGN
    # Q starts inside X (X spans 4*256*2 = 2048 bytes)
    assert _q(lib, A, B, 4, 256, A + 1024, D) == E_OVERLAP
    # S overlaps perm (perm spans 1024 bytes)
    assert _q(lib, A, B, 4, 256, C, B + 512) == E_OVERLAP
    # S overlaps Q (Q spans 4*192 = 768 bytes)
    assert _q(lib, A, B, 4, 256, C, C + 512) == E_OVERLAP
    # same checks on the weight entry point
    assert lib.atom_pack_weights(A, B, 4, 300, C, D, S) == E_SHAPE
    assert lib.atom_pack_weights(A, None, 4, 256, C, D, S) == E_NULL


def test_gemm_validation(lib):
    g = lib.atom_gemm
    assert g(None, B, C, D, 4, 4, 256, E, S) == E_NULL
    assert g(A, B, C, D, 4, 4, 256, None, S) == E_NULL
    assert g(A, B, C, D, 0, 4, 256, E, S) == E_SHAPE
    assert g(A, B, C, D, 4, 0, 256, E, S) == E_SHAPE
    assert g(A, B, C, D, 4, 4, 384 + 64, E, S) == E_SHAPE
    assert g(A, B, C, D + 2, 4, 4, 256, E, S) == E_ALIGN
    assert g(A, B, C, D, 4, 4, 256, A + 16, S) == E_OVERLAP     # Y inside Xq
    assert g(A, B, C, D, 4, 4, 256, D, S) == E_OVERLAP          # Y on sw
    ga = lib.atom_gemm_group_acc
    assert ga(A, None, 4, 4, 256, E, S) == E_NULL
    assert ga(A, C, 4, 4, 200, E, S) == E_SHAPE
    assert ga(A, C, 4, 4, 256, E + 4, S) == E_ALIGN
    assert ga(A, C, 4, 4, 256, C + 64, S) == E_OVERLAP


def test_w4a8_validation(lib):
    qa = lib.atom_quantize_act_a8
    assert qa(None, B, 4, 256, C, D, S) == E_NULL
    assert qa(A, B, 4, 300, C, D, S) == E_SHAPE
    assert qa(A, B, 4, 256, C + 2, D, S) == E_ALIGN
    # the A8 row is K bytes: Q (4 x 256 bytes) reaches C + 1024
    assert qa(A, B, 4, 256, C, C + 1008, S) == E_OVERLAP
    pw = lib.atom_pack_weights_w4a8
    assert pw(A, None, 4, 256, C, D, S) == E_NULL
    assert pw(A, B, 4, 128, C, D, S) == E_SHAPE
    assert pw(A, B, 4, 256, C, C + 512, S) == E_OVERLAP      # sw inside Wq (4 x 192 bytes)
    g = lib.atom_gemm_w4a8
    assert g(None, B, C, D, 4, 4, 256, E, S) == E_NULL
    assert g(A, None, C, D, 4, 4, 256, E, S) == E_NULL
    assert g(A, B, C, D, 4, 0, 256, E, S) == E_SHAPE
    assert g(A, B, C, D + 2, 4, 4, 256, E, S) == E_ALIGN
    assert g(A, B, C, D, 4, 4, 256, A + 512, S) == E_OVERLAP    # Y inside Xq (4 x 256 bytes)
    assert lib.atom_gemm_w4a8_workspace_bytes(4, 4, 200) == -E_SHAPE
    assert lib.atom_gemm_w4a8_workspace_bytes(16, 4096, 4096) > 0          # no few-rows kernel: splits
    assert lib.atom_gemm_w4a8_workspace_bytes(2048, 4096, 4096) == 0
    gw = lib.atom_gemm_w4a8_ws
    need = lib.atom_gemm_w4a8_workspace_bytes(64, 128, 4096)
    assert gw(A, B, C, D, 64, 128, 4096, E, E + 4, need, S) == E_ALIGN     # misaligned workspace
    assert gw(A, B, C, D, 64, 128, 4096, E, A, need, S) == E_OVERLAP       # workspace over Xq
    ga = lib.atom_gemm_w4a8_group_acc
    assert ga(A, C, 4, 4, 256, None, S) == E_NULL
    assert ga(A, C, 4, 4, 200, E, S) == E_SHAPE
    assert ga(A, C, 4, 4, 256, E + 4, S) == E_ALIGN
    assert ga(A, C, 4, 4, 256, C + 64, S) == E_OVERLAP


def test_select_validation(lib):
    assert lib.atom_channel_stat(None, 4, 256, B, S) == E_NULL
    assert lib.atom_channel_stat(A, 0, 256, B, S) == E_SHAPE
    assert lib.atom_channel_stat(A, 4, 256, B + 8, S) == E_ALIGN
    assert lib.atom_channel_stat(A, 4, 256, A + 16, S) == E_OVERLAP
    assert lib.atom_select_outliers(None, 256, B, S) == E_NULL
    assert lib.atom_select_outliers(A, 100, B, S) == E_SHAPE
    assert lib.atom_select_outliers(A, 256, A + 1024, S) == E_OVERLAP


def test_binding_refuses_host_tensors():
    """The product path has no CPU fallback: host tensors are refused before any call."""
    torch = pytest.importorskip("torch")
    X = torch.zeros((4, 256), dtype=torch.float16)
    perm = torch.arange(256, dtype=torch.int32)
    if not os.path.exists(bq.lib_path()):
        with pytest.raises(bq.AtomError):
            bq.atom_quantize_act(X, perm)
        return
    with pytest.raises(bq.AtomError, match="ROCm device"):
        bq.atom_quantize_act(X, perm)
    with pytest.raises(bq.AtomError, match="ROCm device"):
        bq.atom_channel_stat(X)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bq, "_LIB", None)
    monkeypatch.setenv("ATOM_LIB", str(tmp_path / "nope.so"))
    with pytest.raises(bq.AtomError, match="not built"):
        bq.load_library()


def test_gemm_workspace_query(lib):
    # fp32 partial tiles of 128 x 128, tile-major: bytes = split tiles x pieces x 64 KiB
    T = 128 * 128 * 4
    # 256 x 4096 output = 2 x 32 tiles of 128 x 128 but 4 x 64 of 64 x 64: whole small tiles, no scratch
    assert bq.atom_gemm_workspace_bytes(256, 4096, 4096) == 0
    # 33 x 8448: 66 tiles of 128 x 128 but 132 of 64 x 64: K parts inside the workgroup, no scratch
    assert bq.atom_gemm_workspace_bytes(33, 8448, 4096) == 0
    # 64 x 4096, K = 11008: 64 tiles of 64 x 64 on a long K (86 groups): 32 tiles split eight ways
    assert bq.atom_gemm_workspace_bytes(64, 4096, 11008) == 32 * 8 * T
    assert bq.atom_gemm_workspace_bytes(64, 4096, 4096) == 0               # 64 small tiles, 32 groups: K parts
    assert bq.atom_gemm_workspace_bytes(64, 128, 4096) == 1 * 7 * T       # capped by 31 INT4 groups / 4
    # M <= 16: the few-rows kernel reduces its K ranges inside the workgroup: no scratch
    for M, N, K in [(1, 130, 1152), (1, 4096, 4096), (16, 4096, 11008), (3, 131, 2048), (16, 16, 32768)]:
        assert bq.atom_gemm_workspace_bytes(M, N, K) == 0
    assert bq.atom_gemm_workspace_bytes(17, 128, 4096) == 1 * 7 * T        # 17 rows: 128 x 128 tiles, split-K
    assert bq.atom_gemm_workspace_bytes(90 * 128, 64, 4096) == 0            # 180 small tiles: K parts
    assert bq.atom_gemm_workspace_bytes(17, 8000, 32768) == 63 * 5 * T       # 126 small tiles, long K: ceil(256 / 63) = 5
    # 128 tiles or more, or too few groups to divide: no scratch
    assert bq.atom_gemm_workspace_bytes(128 * 128, 128, 4096) == 0
    assert bq.atom_gemm_workspace_bytes(2048, 4096, 11008) == 0
    assert bq.atom_gemm_workspace_bytes(1024, 11008, 4096) == 0
    assert bq.atom_gemm_workspace_bytes(4, 4, 256) == 0
    assert bq.atom_gemm_workspace_bytes(4, 4, 1024) == 0                    # 7 INT4 groups: one piece of 4
    assert lib.atom_gemm_workspace_bytes(4, 4, 200) == -E_SHAPE
    assert lib.atom_gemm_workspace_bytes(0, 4, 256) == -E_SHAPE
    with pytest.raises(bq.AtomError):
        bq.atom_gemm_workspace_bytes(4, 4, 200)


def test_gemm_tile_limit(lib):
    # 2^24 x 2^24 output: 2^34 tiles of 128 x 128 -- rejected before anything is launched
    big = 1 << 24
    assert lib.atom_gemm(A, B, C, D, big, big, 256, E, S) == E_SHAPE
    assert lib.atom_gemm_ws(A, B, C, D, big, big, 256, E, None, 0, S) == E_SHAPE
    assert lib.atom_gemm_group_acc(A, C, big, big, 256, E, S) == E_SHAPE
    assert lib.atom_gemm_workspace_bytes(big, big, 256) == -E_SHAPE
    # 2^13 x 2^13 tile grid = 2^26 tiles: the largest accepted
    assert lib.atom_gemm_workspace_bytes(1 << 20, 1 << 20, 256) == 0


def test_gemm_ws_validation(lib):
    g = lib.atom_gemm_ws
    M, N, K = 64, 128, 4096
    need = bq.atom_gemm_workspace_bytes(M, N, K)
    F = 0x60000000
    assert g(A, B, C, D, M, N, K, None, F, need, S) == E_NULL
    assert g(A, B, C, D, M, N, 300, E, F, need, S) == E_SHAPE
    assert g(A, B, C, D, M, N, K, E, F + 8, need, S) == E_ALIGN       # workspace used, misaligned
    assert g(A, B, C, D, M, N, K, E, E + 64, need, S) == E_OVERLAP    # workspace over Y
    assert g(A, B, C, D, M, N, K, E, A + 16, need, S) == E_OVERLAP    # workspace over Xq


class _NoLaunch:
    """Stands in for the loaded library: the size helpers pass through, every entry point that
    would enqueue work fails the test if it is ever reached."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        if name in ("atom_row_bytes", "atom_num_groups", "atom_strerror", "atom_gemm_workspace_bytes",
                    "atom_gemm_w4a8_workspace_bytes"):
            return getattr(self._lib, name)

        def fail(*a):
            raise AssertionError(f"{name} was called with arguments the binding should have refused")
        return fail


def test_binding_rejects_mis_sized_tensors(lib, monkeypatch):
    """The C ABI cannot see buffer sizes, so the binding checks every tensor's shape against the
    sizes the call implies before calling it; a mis-sized tensor raises AtomError and nothing is
    enqueued (no entry point is reached)."""
    torch = pytest.importorskip("torch")
    monkeypatch.setattr(bq, "_LIB", _NoLaunch(lib))
    M, N, K = 4, 6, 384
    rb, G = bq.atom_row_bytes(K), bq.atom_num_groups(K)
    u8, f16, i32, f64 = torch.uint8, torch.float16, torch.int32, torch.float64
    z = torch.zeros
    X, W, perm = z((M, K), dtype=f16), z((N, K), dtype=f16), z((K,), dtype=i32)
    Xq, sx, Wq, sw = z((M, rb), dtype=u8), z((G, M), dtype=f16), z((N, rb), dtype=u8), z((G, N), dtype=f16)
    bad = [
        # quantize / pack outputs and perm
        lambda: bq.atom_quantize_act(X, z((K - 1,), dtype=i32)),
        lambda: bq.atom_quantize_act(X, perm, Xq=z((M, rb - 1), dtype=u8)),
        lambda: bq.atom_quantize_act(X, perm, sx=z((M, G), dtype=f16)),
        lambda: bq.atom_pack_weights(W, perm, Wq=z((N + 1, rb), dtype=u8)),
        lambda: bq.atom_quantize_act_a8(X, perm, Xq=z((M, rb), dtype=u8)),          # A8 rows are K bytes
        lambda: bq.atom_pack_weights_w4a8(W, perm, sw=z((G, N - 1), dtype=f16)),
        lambda: bq.atom_channel_stat(X, stat=z((K + 1,), dtype=f64)),
        lambda: bq.atom_select_outliers(z((K,), dtype=f64), perm=z((K - 2,), dtype=i32)),
        # GEMM operands against K
        lambda: bq.atom_gemm(Xq, sx, Wq, sw, K + 128),
        lambda: bq.atom_gemm(z((M, K), dtype=u8), sx, Wq, sw, K),                   # an A8 Xq to the W4A4 GEMM
        lambda: bq.atom_gemm(Xq, z((G, M + 1), dtype=f16), Wq, sw, K),
        lambda: bq.atom_gemm(Xq, sx, Wq, z((G - 1, N), dtype=f16), K),
        lambda: bq.atom_gemm(Xq, sx, z((N, rb + 16), dtype=u8), sw, K),
        lambda: bq.atom_gemm(Xq, sx, Wq, sw, K, Y=z((N, M), dtype=f16)),
        lambda: bq.atom_gemm_ws(Xq, sx, Wq, sw, K, z((8, 8), dtype=u8)),           # 2-D workspace
        lambda: bq.atom_gemm_ws(Xq, sx, Wq, sw, K, z((64,), dtype=u8), Y=z((M, N + 1), dtype=f16)),
        lambda: bq.atom_gemm_group_acc(Xq, Wq, K, acc=z((G, M, N - 1), dtype=i32)),
        lambda: bq.atom_gemm_w4a8(Xq, sx, Wq, sw, K),                               # a W4A4 Xq to the W4A8 GEMM
        lambda: bq.atom_gemm_w4a8_group_acc(z((M, K), dtype=u8), Wq, K, acc=z((G + 1, M, N), dtype=i32)),
        lambda: bq.atom_gemm_w4a8_ws(z((M, K), dtype=u8), sx, Wq, sw, K, None, Y=z((M,), dtype=f16)),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(bq.AtomError, match="shape|2-D|1-D"):
            call()
    # wrong dtype, and a non-contiguous tensor
    with pytest.raises(bq.AtomError, match="must be torch.float16"):
        bq.atom_gemm(Xq, sx.float(), Wq, sw, K)
    with pytest.raises(bq.AtomError, match="contiguous"):
        bq.atom_gemm(Xq, sx, Wq, sw, K, Y=z((N, M), dtype=f16).t())
    with pytest.raises(bq.AtomError, match="K=200"):
        bq.atom_gemm(Xq, sx, Wq, sw, 200)
    # correctly sized host tensors get as far as the device check, still without a call
    with pytest.raises(bq.AtomError, match="ROCm device"):
        bq.atom_gemm(Xq, sx, Wq, sw, K)
    with pytest.raises(bq.AtomError, match="ROCm device"):
        bq.atom_gemm_w4a8_ws(z((M, K), dtype=u8), sx, Wq, sw, K, z((16,), dtype=u8))


def test_gemm_noalloc_validation(lib):
    """atom_gemm_noalloc rejects bad arguments on the host before any HIP call (the calls below
    never reach the device: each fails validation)."""
    g = lib.atom_gemm_noalloc
    assert g(None, B, C, D, 4, 4, 256, E, S) == E_NULL
    assert g(A, B, C, D, 4, 4, 256, None, S) == E_NULL
    assert g(A, B, C, D, 4, 4, 300, E, S) == E_SHAPE
    assert g(A, B, C, D, 0, 4, 256, E, S) == E_SHAPE
    assert g(A, B, C, D + 2, 4, 4, 256, E, S) == E_ALIGN
    assert g(A, B, C, D, 4, 4, 256, A + 16, S) == E_OVERLAP     # Y inside Xq
    assert g(A, B, C, D, 64, 4096, 11008, C + 64, S) == E_OVERLAP   # a split shape: Y over Wq
    assert "static buffer" in bq.atom_strerror(E_SCRATCH)


def test_static_scratch_covers_every_split_plan(lib):
    """The static split-K scratch (24 MiB) holds the workspace of the largest split plan any valid
    shape asks for, so atom_gemm_noalloc never has to refuse a valid shape."""
    text = open(HEADER).read()
    cap = 24 << 20
    assert re.search(r"#define ATOM_STATIC_SCRATCH_BYTES \(24 << 20\)", text)
    worst = 0
    for M in (17, 33, 64, 100, 128, 129, 191, 192, 255, 256, 320, 384, 640):
        for N in range(64, 128 * 130, 64):
            worst = max(worst, bq.atom_gemm_workspace_bytes(M, N, bq.MAX_K))
    assert 0 < worst <= cap
    assert bq.atom_gemm_workspace_bytes(17, 8000, bq.MAX_K) == 315 * 128 * 128 * 4 == worst


def _local_includes(path, seen):
    """Every repository header a source includes, directly or through other headers."""
    for name in re.findall(r'^#include "([^"]+)"', open(path).read(), re.M):
        for d in (os.path.join(ROOT, "bit_quantized_gemm_amd", "csrc"), os.path.join(ROOT, "include")):
            p = os.path.join(d, name)
            if os.path.exists(p) and p not in seen:
                seen.add(p)
                _local_includes(p, seen)
    return seen


def test_bench_traffic_hash_covers_every_included_source():
    """bench.py reports the committed HBM-traffic counters only while the SHA-256 of the
    measured kernels' sources is unchanged: that hash must cover each kernel file and every
    repository header it includes, or a header edit would leave stale counters in the line."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    csrc = os.path.join(ROOT, "bit_quantized_gemm_amd", "csrc")
    for main, listed in (("gemm.hip", bench.GEMM_SRC), ("quantize.hip", bench.QUANT_SRC)):
        want = _local_includes(os.path.join(csrc, main), {os.path.join(csrc, main)})
        assert set(map(os.path.abspath, listed)) == want, main
    # the committed counters name the same files, in the order bench.py hashes them
    import json
    d = json.load(open(bench.TRAFFIC_FILE))
    assert [os.path.join(ROOT, f) for f in d["gemm_sources"]] == bench.GEMM_SRC
    assert [os.path.join(ROOT, f) for f in d["quantize_sources"]] == bench.QUANT_SRC


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and says why, before it
    imports torch or touches a device."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
