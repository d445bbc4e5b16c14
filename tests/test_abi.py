"""The C-ABI library loads, exports every declared symbol, and rejects invalid
arguments before touching the GPU (no compute call is made here)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")
HEADER_UNFUSED = os.path.join(ROOT, "include", "fa355_unfused.h")
LIB = os.path.join(ROOT, "exact_io_aware_12_amd", "libfa355.so")
LIB_UNFUSED = os.path.join(ROOT, "exact_io_aware_12_amd", "libfa355_unfused.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfa355.so not built")


def _declared(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"FA355_API\s+[\w\s\*]+?\b(fa_\w+)\s*\(", text)))


def _codes():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(FA_\w+)\s*=\s*(\d+)", text)}


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_12_amd import fa as mod
    mod.library()
    return mod


def test_header_declares_the_entry_points():
    assert _declared() == ["fa_bwd", "fa_bwd_kernel_name", "fa_bwd_noalloc",
                           "fa_bwd_workspace_bytes", "fa_decode_fwd",
                           "fa_decode_workspace_bytes", "fa_fa1_fwd", "fa_fa1_workspace_bytes",
                           "fa_fwd", "fa_fwd_kernel_name", "fa_fwd_persistent", "fa_strerror"]
    assert _declared(HEADER_UNFUSED) == ["fa_unfused_fwd", "fa_unfused_workspace_bytes"]


def test_fwd_kernel_name_follows_the_dispatch_rule(fa):
    # Two-group kernel: d = 128, causal N >= 8192 or non-causal N >= 4096, and
    # at least 256 of its 256-row workgroups (unless a split form applies);
    # otherwise the 128-row kernel.
    assert fa.fa_fwd_kernel_name(1, 16, 16384, 128, True) == "fa_fwd_pp_kernel"
    assert fa.fa_fwd_kernel_name(2, 32, 4096, 128, True) == "fa_fwd_kernel"
    assert fa.fa_fwd_kernel_name(2, 32, 4096, 128, False) == "fa_fwd_pp_kernel"
    assert fa.fa_fwd_kernel_name(2, 16, 2048, 128, True) == "fa_fwd_kernel"
    split = "fa_fwd_pp_kernel (keys split between the groups)"
    assert fa.fa_fwd_kernel_name(1, 1, 16384, 128, True) == split     # 128 tiles of 128 rows
    assert fa.fa_fwd_kernel_name(1, 2, 16384, 128, False) == split    # 256: one per CU
    assert fa.fa_fwd_kernel_name(1, 3, 1500, 128, True) == split
    paired = "fa_fwd_pp_kernel (keys split between the groups, two query tiles per workgroup)"
    # Causal, d = 128, N >= 4096, 257-512 tiles of 128 rows: two tiles per workgroup.
    assert fa.fa_fwd_kernel_name(1, 3, 16384, 128, True) == paired     # 384 tiles
    assert fa.fa_fwd_kernel_name(1, 8, 8192, 128, True) == paired      # 512 tiles
    assert fa.fa_fwd_kernel_name(1, 9, 4100, 128, True) == paired      # 297 tiles, ragged
    assert fa.fa_fwd_kernel_name(1, 3, 16384, 128, False) == "fa_fwd_kernel"   # non-causal
    assert fa.fa_fwd_kernel_name(1, 16, 4096, 128, True) == paired     # 512 tiles
    assert fa.fa_fwd_kernel_name(1, 17, 4096, 128, True) == "fa_fwd_kernel"    # 544 tiles
    assert fa.fa_fwd_kernel_name(1, 32, 2048, 128, True) == "fa_fwd_kernel"    # N < 4096
    assert fa.fa_fwd_kernel_name(1, 2, 1000, 128, True) == "fa_fwd_kernel"    # N < 1024
    assert fa.fa_fwd_kernel_name(1, 3, 16384, 64, True) == "fa_fwd_kernel"    # d = 64, 384 tiles
    assert fa.fa_fwd_kernel_name(1, 1, 16384, 64, True) == "fa_fwd_kernel (keys split between two groups)"
    assert fa.fa_fwd_kernel_name(4, 16, 2048, 64, True) == "fa_fwd_kernel"    # 1024 tiles
    assert fa.fa_fwd_kernel_name(1, 16, 16384, 64, True) == "fa_fwd_kernel"      # d = 64
    assert fa.fa_fwd_kernel_name(0, 16, 16384, 128, True) is None
    assert fa.fa_fwd_kernel_name(1, 16, 16384, 96, True) is None


def test_bwd_kernel_name_follows_the_dispatch_rule(fa):
    # dQ key split: causal grids of at most 512 query tiles of 128 rows,
    # non-causal grids of at most 256; both head dimensions.
    split = "fa_bwd_dq_kernel (keys split between two groups) + fa_bwd_dkdv_kernel"
    plain = "fa_bwd_dq_kernel + fa_bwd_dkdv_kernel"
    for d in (64, 128):
        assert fa.fa_bwd_kernel_name(2, 16, 2048, d, True) == split     # 512 tiles
        assert fa.fa_bwd_kernel_name(2, 16, 2048, d, False) == plain    # 512 > 256
        assert fa.fa_bwd_kernel_name(1, 33, 1000, d, False) == plain    # 264 > 256
        assert fa.fa_bwd_kernel_name(1, 32, 1024, d, False) == split    # 256
        assert fa.fa_bwd_kernel_name(4, 33, 500, d, True) == plain      # 528 > 512
        assert fa.fa_bwd_kernel_name(1, 1, 1, d, False) == split
    assert fa.fa_bwd_kernel_name(1, 1, 16, 96, True) is None
    assert fa.fa_bwd_kernel_name(1, 0, 16, 64, True) is None


def test_every_declared_symbol_is_exported():
    import torch  # noqa: F401  (torch's HIP runtime first, as the binding does)
    for header, path in ((HEADER, LIB), (HEADER_UNFUSED, LIB_UNFUSED)):
        lib = ctypes.CDLL(path)
        for name in _declared(header):
            assert hasattr(lib, name), (path, name)


def _needed(path):
    import subprocess
    out = subprocess.run(["readelf", "-d", path], capture_output=True, text=True, check=True)
    return re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out.stdout)


def test_fused_library_does_not_depend_on_rocblas():
    """libfa355.so needs the HIP runtime and the C/C++ runtimes only; rocBLAS
    is a dependency of the unfused comparator's library alone."""
    needed = _needed(LIB)
    assert any(n.startswith("libamdhip64") for n in needed), needed
    assert not any("rocblas" in n or "hipblas" in n for n in needed), needed
    assert any("rocblas" in n for n in _needed(LIB_UNFUSED))
    assert not any(n.startswith("libfa355") for n in _needed(LIB_UNFUSED))


def test_codes_match_binding(fa):
    codes = _codes()
    assert codes["FA_OK"] == fa.FA_OK == 0
    for n in ("NULL", "SHAPE", "HEADDIM", "SCALE", "ALIGN", "WORKSPACE", "HIP", "BLAS",
              "TOO_LARGE"):
        assert codes["FA_ERR_" + n] == getattr(fa, "FA_ERR_" + n)
        assert fa.fa_strerror(codes["FA_ERR_" + n]) not in ("", "unknown fa355 error code")
    assert fa.fa_strerror(99) == "unknown fa355 error code"


GOOD = 0x10000  # a 16-byte aligned dummy address; never dereferenced (calls fail validation)


def _fwd(fa, q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD, B=1, H=1, N=16, d=64, scale=0.125,
         causal=0):
    return fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fwd_null(fa, which):
    assert _fwd(fa, **{which: None}) == fa.FA_ERR_NULL


@pytest.mark.parametrize("B,H,N", [(0, 1, 16), (1, 0, 16), (1, 1, 0), (-1, 1, 16),
                                   (1024, 1024, 1024)])
def test_fwd_shape(fa, B, H, N):
    assert _fwd(fa, B=B, H=H, N=N) == fa.FA_ERR_SHAPE


@pytest.mark.parametrize("d", [0, 32, 96, 100, 256])
def test_fwd_headdim(fa, d):
    assert _fwd(fa, d=d) == fa.FA_ERR_HEADDIM


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_fwd_scale(fa, scale):
    assert _fwd(fa, scale=scale) == fa.FA_ERR_SCALE


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fwd_align(fa, which):
    assert _fwd(fa, **{which: GOOD + 8}) == fa.FA_ERR_ALIGN


def test_fwd_persistent_validation(fa):
    def call(q=GOOD, o=GOOD, B=1, N=16, d=64, scale=0.125):
        return fa.fa_fwd_persistent(q, GOOD, GOOD, o, GOOD, B, 1, N, d, scale, 1, None)
    assert call(q=None) == fa.FA_ERR_NULL
    assert call(N=0) == fa.FA_ERR_SHAPE
    assert call(B=1 << 20, N=1 << 12) == fa.FA_ERR_SHAPE
    assert call(d=96) == fa.FA_ERR_HEADDIM
    assert call(scale=math.nan) == fa.FA_ERR_SCALE
    assert call(o=GOOD + 2) == fa.FA_ERR_ALIGN


def test_workspace_bytes(fa):
    B, H, N, d = 2, 16, 2048, 128
    rows = B * H * N
    r256 = lambda x: (x + 255) // 256 * 256
    assert fa.fa_bwd_workspace_bytes(B, H, N, d) == r256(rows * 4)
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 64) == 256
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 48) == 0


def _bwd(fa, ws=GOOD, ws_bytes=None, B=1, H=1, N=16, d=64, scale=0.125, **ptrs):
    p = dict(q=GOOD, k=GOOD, v=GOOD, o=GOOD, dout=GOOD, lse=GOOD, dq=GOOD, dk=GOOD, dv=GOOD)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_bytes(1, 1, 16, 64)
    return fa.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"], p["dk"],
                     p["dv"], ws, ws_bytes, B, H, N, d, scale, 1, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"])
def test_bwd_null(fa, which):
    assert _bwd(fa, **{which: None}) == fa.FA_ERR_NULL


def test_bwd_workspace(fa):
    need = fa.fa_bwd_workspace_bytes(1, 1, 16, 64)
    assert _bwd(fa, ws=None) == fa.FA_ERR_WORKSPACE
    assert _bwd(fa, ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE


@pytest.mark.parametrize("which", ["q", "dout", "lse", "dv"])
def test_bwd_align(fa, which):
    assert _bwd(fa, **{which: GOOD + 4}) == fa.FA_ERR_ALIGN
    assert _bwd(fa, ws=GOOD + 8) == fa.FA_ERR_ALIGN


# ------------------------------------------------ fa_bwd_noalloc (static scratch)
def _bwd_na(fa, B=1, H=1, N=16, d=64, scale=0.125, **ptrs):
    p = dict(q=GOOD, k=GOOD, v=GOOD, o=GOOD, dout=GOOD, lse=GOOD, dq=GOOD, dk=GOOD, dv=GOOD)
    p.update(ptrs)
    return fa.fa_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"],
                             p["dk"], p["dv"], B, H, N, d, scale, 1, None)


def test_noalloc_limit_matches_header(fa):
    text = open(HEADER).read()
    m = re.search(r"#define\s+FA_BWD_NOALLOC_MAX_ROWS\s+(\d+)", text)
    assert m and int(m.group(1)) == fa.FA_BWD_NOALLOC_MAX_ROWS == 1 << 22


@pytest.mark.parametrize("B,H,N", [(1, 1, (1 << 22) + 1), (2, 32, 65537), (64, 64, 1025)])
def test_noalloc_rejects_rows_beyond_the_scratch(fa, B, H, N):
    # Rejected before any HIP call (no GPU here): too many rows for the
    # 16 MiB static scratch, though the shape itself is valid for fa_bwd.
    assert B * H * N > fa.FA_BWD_NOALLOC_MAX_ROWS
    assert _bwd_na(fa, B=B, H=H, N=N) == fa.FA_ERR_TOO_LARGE


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"])
def test_noalloc_null(fa, which):
    assert _bwd_na(fa, **{which: None}) == fa.FA_ERR_NULL


def test_noalloc_validation(fa):
    assert _bwd_na(fa, d=96) == fa.FA_ERR_HEADDIM
    assert _bwd_na(fa, N=0) == fa.FA_ERR_SHAPE
    assert _bwd_na(fa, scale=math.nan) == fa.FA_ERR_SCALE
    assert _bwd_na(fa, dk=GOOD + 2) == fa.FA_ERR_ALIGN


def test_bwd_shape_and_scale(fa):
    assert _bwd(fa, N=0) == fa.FA_ERR_SHAPE
    assert _bwd(fa, d=80) == fa.FA_ERR_HEADDIM
    assert _bwd(fa, scale=math.nan) == fa.FA_ERR_SCALE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from exact_io_aware_12_amd import fa as mod
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        mod.library()


def test_unfused_binding_fails_loudly_without_its_library(monkeypatch, tmp_path):
    from exact_io_aware_12_amd import fa as mod
    monkeypatch.setattr(mod, "_lib_unfused", None)
    monkeypatch.setattr(mod, "_LIB_UNFUSED_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        mod.library_unfused()


def test_single_hip_runtime_mapped():
    """Loaded through the binding, libfa355 binds to the libamdhip64 torch
    already mapped (same soname), so one HIP runtime serves both."""
    import subprocess
    import sys
    code = ("from exact_io_aware_12_amd import fa; fa.library(); "
            "m = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


# ---------------------------------------------------------------- unfused comparator
def _unf(fa, ws=GOOD, ws_bytes=None, B=1, H=1, N=16, d=64, scale=0.125, **ptrs):
    p = dict(q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = fa.fa_unfused_workspace_bytes(1, 1, 16, 64)
    return fa.fa_unfused_fwd(p["q"], p["k"], p["v"], p["o"], p["lse"], ws, ws_bytes, B, H, N,
                             d, scale, 1, None)


def test_unfused_workspace_bytes(fa):
    r256 = lambda x: (x + 255) // 256 * 256
    assert fa.fa_unfused_workspace_bytes(2, 16, 2048, 128) == r256(2 * 16 * 2048 * 2048 * 4)
    assert fa.fa_unfused_workspace_bytes(1, 1, 1, 64) == 256
    assert fa.fa_unfused_workspace_bytes(1, 0, 8, 64) == 0
    assert fa.fa_unfused_workspace_bytes(1, 1, 8, 96) == 0


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_unfused_null_and_align(fa, which):
    assert _unf(fa, **{which: None}) == fa.FA_ERR_NULL
    assert _unf(fa, **{which: GOOD + 4}) == fa.FA_ERR_ALIGN


def test_unfused_validation(fa):
    need = fa.fa_unfused_workspace_bytes(1, 1, 16, 64)
    assert _unf(fa, ws=None) == fa.FA_ERR_WORKSPACE
    assert _unf(fa, ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert _unf(fa, ws=GOOD + 8) == fa.FA_ERR_ALIGN
    assert _unf(fa, N=0) == fa.FA_ERR_SHAPE
    assert _unf(fa, d=32) == fa.FA_ERR_HEADDIM
    assert _unf(fa, scale=math.nan) == fa.FA_ERR_SCALE


# ---------------------------------------------------------------- loop-order comparator
def _fa1(fa, ws=GOOD, ws_bytes=None, B=1, H=1, N=16, d=64, scale=0.125, **ptrs):
    p = dict(q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = fa.fa_fa1_workspace_bytes(1, 1, 16, 64)
    return fa.fa_fa1_fwd(p["q"], p["k"], p["v"], p["o"], p["lse"], ws, ws_bytes, B, H, N, d,
                         scale, 1, None)


def test_fa1_workspace_bytes(fa):
    """fp32 running state per (head, 128-row query tile, wave of 32 rows): the
    O^T accumulator (d/2 registers) plus the running max and sum, 64 lanes
    each."""
    r256 = lambda x: (x + 255) // 256 * 256
    for B, H, N, d in [(1, 1, 1, 64), (2, 3, 129, 128), (1, 16, 16384, 128), (4, 16, 1000, 64)]:
        ntq = (N + 127) // 128
        assert fa.fa_fa1_workspace_bytes(B, H, N, d) == r256(B * H * ntq * 4 * (d // 2 + 2) * 64 * 4)
    assert fa.fa_fa1_workspace_bytes(1, 0, 8, 64) == 0
    assert fa.fa_fa1_workspace_bytes(1, 1, 8, 96) == 0


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fa1_null_and_align(fa, which):
    assert _fa1(fa, **{which: None}) == fa.FA_ERR_NULL
    assert _fa1(fa, **{which: GOOD + 4}) == fa.FA_ERR_ALIGN


def test_fa1_validation(fa):
    need = fa.fa_fa1_workspace_bytes(1, 1, 16, 64)
    assert _fa1(fa, ws=None) == fa.FA_ERR_WORKSPACE
    assert _fa1(fa, ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert _fa1(fa, ws=GOOD + 8) == fa.FA_ERR_ALIGN
    assert _fa1(fa, N=0) == fa.FA_ERR_SHAPE
    assert _fa1(fa, d=32) == fa.FA_ERR_HEADDIM
    assert _fa1(fa, scale=math.inf) == fa.FA_ERR_SCALE


# ---------------------------------------------------------------- decode
def _dec(fa, ws=GOOD, ws_bytes=None, B=1, H=1, Nq=1, Nk=100, d=128, scale=0.1, causal=1,
         **ptrs):
    p = dict(q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d)
    return fa.fa_decode_fwd(p["q"], p["k"], p["v"], p["o"], p["lse"], ws, ws_bytes, B, H, Nq,
                            Nk, d, scale, causal, None)


def test_decode_workspace_bytes(fa):
    # per split: Nq*d fp32 partial O plus Nq fp32 LSE; the split count depends
    # on B*H and Nk only
    w1 = fa.fa_decode_workspace_bytes(1, 1, 1, 100, 128)
    assert w1 == 512 + 256                      # 100 keys: one split (128 fp32 + 1 fp32)
    assert fa.fa_decode_workspace_bytes(16, 32, 4, 8192, 128) > 0
    assert fa.fa_decode_workspace_bytes(1, 1, 33, 100, 128) == 0   # Nq > 32
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 100, 96) == 0


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_decode_null_and_align(fa, which):
    assert _dec(fa, **{which: None}) == fa.FA_ERR_NULL
    assert _dec(fa, **{which: GOOD + 4}) == fa.FA_ERR_ALIGN


def test_decode_validation(fa):
    need = fa.fa_decode_workspace_bytes(1, 1, 1, 100, 128)
    assert _dec(fa, ws=None) == fa.FA_ERR_WORKSPACE
    assert _dec(fa, ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert _dec(fa, Nq=33, ws_bytes=1 << 20) == fa.FA_ERR_SHAPE
    assert _dec(fa, Nq=8, Nk=4, ws_bytes=1 << 20) == fa.FA_ERR_SHAPE     # causal needs Nq <= Nk
    assert _dec(fa, Nk=0, ws_bytes=1 << 20) == fa.FA_ERR_SHAPE
    assert _dec(fa, d=80, ws_bytes=1 << 20) == fa.FA_ERR_HEADDIM
    assert _dec(fa, scale=math.inf) == fa.FA_ERR_SCALE


# ---------------------------------------------------------------- sanitizers
def test_entry_points_under_address_and_ub_sanitizers(tmp_path):
    """The C entry points' host code (fa_api.cpp, fa_unfused_api.cpp) built by
    g++ with -fsanitize=address,undefined against stand-in launchers
    (tests/abi_host/stubs.cpp) and driven through valid and invalid calls
    (tests/abi_host/driver.cpp): every argument reaches the launcher intact,
    every invalid call is refused without a launch, and the sanitizers report
    nothing. CPU only; no GPU code is built."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(ROOT, "exact_io_aware_12_amd", "csrc")
    host = os.path.join(ROOT, "tests", "abi_host")
    exe = str(tmp_path / "abi_sanitized")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", os.path.join(csrc, "fa_api.cpp"),
           os.path.join(csrc, "fa_unfused_api.cpp"), os.path.join(host, "stubs.cpp"),
           os.path.join(host, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the environment may preload other libraries
    # ahead of the sanitizer runtime; that is harmless for this program.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ABI OK", r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
