"""The C-ABI library on the host: it loads, exports what include/fa.h declares,
and rejects bad arguments before touching the GPU (no kernel is launched by
any call in this file)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    from tiled_online_softmax_06_amd import fa, build_lib
    if not os.path.exists(fa.library_path()):
        build_lib.build()
    return fa.load_library()


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)


def _header_enum(name):
    text = open(HEADER).read()
    body = re.search(r"typedef enum \{([^{}]*)\}\s*" + name, text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return {k: int(v) for k, v in re.findall(r"(FA_\w+)\s*=\s*(\d+)", body)}


def test_exports_every_declared_function(lib):
    funcs = _header_functions()
    assert set(funcs) == {"fa_forward", "fa_forward_gqa", "fa_backward", "fa_forward_split", "fa_forward_fp8",
                          "fa_forward_split_noalloc", "fa_split_workspace_bytes", "fa_split_suggest", "fa_merge",
                          "fa_status_string", "fa_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for f in funcs:
        assert f in exported, f"{f} not exported"
        assert getattr(lib, f) is not None


def test_binding_constants_match_header():
    import torch
    from tiled_online_softmax_06_amd import fa
    dt = _header_enum("fa_dtype_t")
    assert fa.FA_DTYPE == {torch.float32: dt["FA_DTYPE_FP32"], torch.float16: dt["FA_DTYPE_FP16"],
                           torch.bfloat16: dt["FA_DTYPE_BF16"]}


def test_status_strings(lib):
    codes = _header_enum("fa_status_t")
    seen = set()
    for name, code in codes.items():
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status", name
        seen.add(s)
    assert len(seen) == len(codes)
    assert lib.fa_status_string(999).decode() == "unknown status"
    assert "gfx950" in lib.fa_version().decode()


# Fake, never dereferenced device addresses: every call below fails a check
# before any HIP call, so nothing is read or written through them.
A = 0x7F0000000000
MB = 1 << 20


def call(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
         B=1, H=1, N=128, d=64, scale=0.125, dtype=2):
    return lib.fa_forward(q, k, v, o, lse, B, H, N, d, scale, dtype, None)


def test_error_codes(lib):
    codes = _header_enum("fa_status_t")
    assert call(lib, B=-1) == codes["FA_ERR_BAD_SHAPE"]
    assert call(lib, N=-5) == codes["FA_ERR_BAD_SHAPE"]
    assert call(lib, d=-64) == codes["FA_ERR_BAD_SHAPE"]
    assert call(lib, B=1 << 40, H=1 << 40) == codes["FA_ERR_BAD_SHAPE"]       # size overflow
    assert call(lib, N=1 << 31) == codes["FA_ERR_BAD_SHAPE"]                  # 32-bit kernel index
    assert call(lib, N=1 << 24, d=128) == codes["FA_ERR_BAD_SHAPE"]           # 4 GiB per head > 32-bit offsets
    assert call(lib, N=1 << 23, d=64, dtype=0) == codes["FA_ERR_BAD_SHAPE"]
    assert call(lib, d=96) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    assert call(lib, d=256) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    assert call(lib, dtype=3) == codes["FA_ERR_UNSUPPORTED_DTYPE"]
    assert call(lib, dtype=-1) == codes["FA_ERR_UNSUPPORTED_DTYPE"]
    for bad in (math.nan, math.inf, -math.inf):
        assert call(lib, scale=bad) == codes["FA_ERR_BAD_SCALE"]
    # finite scales whose base-2 factor |scale| log2(e) overflows float32
    for bad in (3e38, -3e38, 2.4e38):
        assert call(lib, scale=bad) == codes["FA_ERR_BAD_SCALE"], bad
    for field in ("q", "k", "v", "o", "lse"):
        assert call(lib, **{field: None}) == codes["FA_ERR_NULL_POINTER"], field
    for field in ("q", "k", "v", "o"):
        assert call(lib, **{field: A + 8}) == codes["FA_ERR_MISALIGNED"], field
    assert call(lib, lse=A + 256 * MB + 2) == codes["FA_ERR_MISALIGNED"]
    # outputs overlapping an input or each other
    assert call(lib, o=A + 64) == codes["FA_ERR_ALIAS"]                       # O inside Q
    assert call(lib, o=A + 128 * MB) == codes["FA_ERR_ALIAS"]                 # O == V
    assert call(lib, lse=A + 192 * MB + 16) == codes["FA_ERR_ALIAS"]          # LSE inside O
    assert call(lib, lse=A + 64 * MB + 16384 - 16) == codes["FA_ERR_ALIAS"]   # LSE tail in K


def test_empty_problem_is_a_no_op(lib):
    for shape in ({"B": 0}, {"H": 0}, {"N": 0}):
        assert call(lib, q=None, k=None, v=None, o=None, lse=None, **shape) == 0


def call_gqa(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
             B=1, H=4, Hkv=2, N=128, d=64, scale=0.125, dtype=2):
    return lib.fa_forward_gqa(q, k, v, o, lse, B, H, Hkv, N, d, scale, dtype, None)


def test_gqa_error_codes(lib):
    codes = _header_enum("fa_status_t")
    lib.fa_forward_gqa.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    assert call_gqa(lib, Hkv=3) == codes["FA_ERR_BAD_SHAPE"]      # does not divide H
    assert call_gqa(lib, Hkv=0) == codes["FA_ERR_BAD_SHAPE"]
    assert call_gqa(lib, Hkv=-2) == codes["FA_ERR_BAD_SHAPE"]
    assert call_gqa(lib, Hkv=8) == codes["FA_ERR_BAD_SHAPE"]      # more K/V heads than query heads
    assert call_gqa(lib, d=80) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    assert call_gqa(lib, k=A + 64 * MB + 4) == codes["FA_ERR_MISALIGNED"]
    # O overlapping the (smaller) K: K spans B*Hkv*N*d*2 = 32 KiB here
    assert call_gqa(lib, o=A + 64 * MB + 32768 - 16) == codes["FA_ERR_ALIAS"]
    assert call_gqa(lib, q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    for bad in (math.nan, math.inf):
        assert call_gqa(lib, scale=bad) == codes["FA_ERR_BAD_SCALE"]


def call_bwd(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, do=A + 256 * MB, lse=A + 320 * MB,
             dws=A + 384 * MB, dq=A + 448 * MB, dk=A + 512 * MB, dv=A + 576 * MB,
             B=1, H=4, Hkv=2, N=128, d=64, scale=0.125, dtype=2):
    lib.fa_backward.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    return lib.fa_backward(q, k, v, o, do, lse, dws, dq, dk, dv, B, H, Hkv, N, d, scale, dtype, None)


def test_backward_error_codes(lib):
    codes = _header_enum("fa_status_t")
    assert call_bwd(lib, B=-1) == codes["FA_ERR_BAD_SHAPE"]
    assert call_bwd(lib, Hkv=3) == codes["FA_ERR_BAD_SHAPE"]
    assert call_bwd(lib, Hkv=0) == codes["FA_ERR_BAD_SHAPE"]
    assert call_bwd(lib, B=1 << 40, H=1 << 40) == codes["FA_ERR_BAD_SHAPE"]
    assert call_bwd(lib, N=1 << 24, d=64) == codes["FA_ERR_BAD_SHAPE"]       # 2 GiB per head
    assert call_bwd(lib, dtype=0) == codes["FA_ERR_UNSUPPORTED_DTYPE"]        # fp32: forward only
    assert call_bwd(lib, d=96) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    for bad in (math.nan, -math.inf):
        assert call_bwd(lib, scale=bad) == codes["FA_ERR_BAD_SCALE"]
    assert call_bwd(lib, scale=3e38) == codes["FA_ERR_BAD_SCALE"]      # scale log2(e) overflows float32
    for field in ("q", "k", "v", "o", "do", "lse", "dws", "dq", "dk", "dv"):
        assert call_bwd(lib, **{field: None}) == codes["FA_ERR_NULL_POINTER"], field
    for field in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        assert call_bwd(lib, **{field: A + 1024 * MB + 8}) == codes["FA_ERR_MISALIGNED"], field
    assert call_bwd(lib, dws=A + 384 * MB + 2) == codes["FA_ERR_MISALIGNED"]
    # outputs overlapping an input or each other (Q spans 64 KiB, K 32 KiB, LSE 2 KiB)
    assert call_bwd(lib, dq=A + 64) == codes["FA_ERR_ALIAS"]                   # dQ inside Q
    assert call_bwd(lib, dk=A + 256 * MB + 16) == codes["FA_ERR_ALIAS"]        # dK inside dO
    assert call_bwd(lib, dv=A + 512 * MB + 32768 - 16) == codes["FA_ERR_ALIAS"]  # dV tail of dK
    assert call_bwd(lib, dws=A + 320 * MB + 4) == codes["FA_ERR_ALIAS"]        # workspace inside LSE
    assert call_bwd(lib, dws=A + 448 * MB) == codes["FA_ERR_ALIAS"]            # workspace == dQ
    assert call_bwd(lib, q=None, k=None, v=None, o=None, do=None, lse=None, dws=None, dq=None,
                    dk=None, dv=None, N=0) == 0


def _split_lib(lib):
    lib.fa_forward_split.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.fa_split_workspace_bytes.argtypes = [ctypes.c_int64] * 5
    lib.fa_split_workspace_bytes.restype = ctypes.c_int64
    lib.fa_split_suggest.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.fa_split_suggest.restype = ctypes.c_int64
    lib.fa_merge.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 4 + [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return lib


def test_split_workspace_bytes(lib):
    """Ranges are whole 64-key tiles and never empty: ceil(N / kchunk) ranges
    with kchunk = 64 ceil(ceil(N / 64) / splits); bytes = B H ranges N (d+1) 4."""
    _split_lib(lib)
    for B, H, N, d, splits in ((1, 2, 16384, 128, 2), (1, 1, 1000, 64, 5), (1, 1, 100, 64, 5), (2, 3, 4097, 128, 7),
                               (1, 1, 64, 64, 4), (3, 1, 1, 128, 9), (1, 1, 8192, 64, 1)):
        tiles = -(-N // 64)
        s_ = min(splits, tiles)
        kchunk = 64 * -(-tiles // s_)
        ranges = -(-N // kchunk)
        want = 0 if ranges == 1 else B * H * ranges * N * (d + 1) * 4
        assert lib.fa_split_workspace_bytes(B, H, N, d, splits) == want, (B, H, N, d, splits)
    assert lib.fa_split_workspace_bytes(1, 1, 1000, 64, 0) == -1
    assert lib.fa_split_workspace_bytes(-1, 1, 1000, 64, 2) == -1
    assert lib.fa_split_workspace_bytes(1 << 40, 1 << 20, 1 << 10, 64, 8) == -1      # overflow
    assert lib.fa_split_workspace_bytes(0, 4, 1000, 64, 4) == 0


def test_split_suggest(lib):
    _split_lib(lib)
    assert lib.fa_split_suggest(2, 16, 8192, 128, 2) == 1       # 1024 workgroups already
    assert lib.fa_split_suggest(1, 2, 16384, 128, 2) == 2       # 128 workgroups -> 256
    assert lib.fa_split_suggest(1, 1, 8192, 128, 2) == 8        # 32 -> 256, 1024 keys per range
    assert lib.fa_split_suggest(1, 1, 1024, 128, 2) == 1        # tiny: a second launch costs more
    assert lib.fa_split_suggest(1, 1, 500, 64, 1) == 1          # too short to split
    assert lib.fa_split_suggest(4, 8, 1000, 64, 1) == 1         # a 19 us launch: a second launch costs more
    assert lib.fa_split_suggest(1, 2, 4096, 128, 2) == 8        # 32 workgroups -> 256
    assert lib.fa_split_suggest(1, 1, 8192, 96, 2) == 1         # unsupported d


def call_split(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, ws=A + 320 * MB,
               ws_bytes=1 << 30, B=1, H=2, Hkv=2, N=1000, d=64, splits=4, scale=0.125, dtype=2):
    return lib.fa_forward_split(q, k, v, o, lse, B, H, Hkv, N, d, scale, dtype, splits, ws, ws_bytes, None)


def test_split_error_codes(lib):
    codes = _header_enum("fa_status_t")
    _split_lib(lib)
    need = lib.fa_split_workspace_bytes(1, 2, 1000, 64, 4)
    assert call_split(lib, splits=0) == codes["FA_ERR_BAD_SHAPE"]
    assert call_split(lib, Hkv=3) == codes["FA_ERR_BAD_SHAPE"]
    assert call_split(lib, d=80) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    assert call_split(lib, scale=math.nan) == codes["FA_ERR_BAD_SCALE"]
    assert call_split(lib, ws=None) == codes["FA_ERR_WORKSPACE"]
    assert call_split(lib, ws_bytes=need - 1) == codes["FA_ERR_WORKSPACE"]
    assert call_split(lib, ws=A + 320 * MB + 4) == codes["FA_ERR_MISALIGNED"]
    assert call_split(lib, ws=A + 192 * MB - 1024) == codes["FA_ERR_ALIAS"]     # workspace runs into O
    assert call_split(lib, ws=A + 16) == codes["FA_ERR_ALIAS"]                  # workspace inside Q
    assert call_split(lib, o=A + 64) == codes["FA_ERR_ALIAS"]                   # the forward's own checks
    assert call_split(lib, q=None) == codes["FA_ERR_NULL_POINTER"]
    assert call_split(lib, N=0, q=None, k=None, v=None, o=None, lse=None, ws=None) == 0


def call_noalloc(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, B=1, H=2, Hkv=2,
                 N=1000, d=64, splits=4, scale=0.125, dtype=2):
    return lib.fa_forward_split_noalloc(q, k, v, o, lse, B, H, Hkv, N, d, scale, dtype, splits, None)


def test_split_noalloc_error_codes(lib):
    """The no-allocation key split checks its arguments like fa_forward_split
    and rejects sizes whose partial results exceed its fixed scratch, all
    before any GPU call."""
    codes = _header_enum("fa_status_t")
    _split_lib(lib)
    assert call_noalloc(lib, splits=0) == codes["FA_ERR_BAD_SHAPE"]
    assert call_noalloc(lib, Hkv=3) == codes["FA_ERR_BAD_SHAPE"]
    assert call_noalloc(lib, d=80) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    assert call_noalloc(lib, scale=math.nan) == codes["FA_ERR_BAD_SCALE"]
    assert call_noalloc(lib, q=None) == codes["FA_ERR_NULL_POINTER"]
    assert call_noalloc(lib, o=A + 64) == codes["FA_ERR_ALIAS"]
    # 8 heads x 4 ranges x 32768 rows x (128 + 1) floats = 541 MB > 64 MiB
    big = dict(B=1, H=8, Hkv=8, N=32768, d=128, splits=4, o=A + 1024 * MB, lse=A + 1536 * MB,
               k=A + 256 * MB, v=A + 512 * MB)
    assert lib.fa_split_workspace_bytes(1, 8, 32768, 128, 4) > (64 << 20)
    assert call_noalloc(lib, **big) == codes["FA_ERR_SCRATCH_LIMIT"]
    # the largest that fits: 2 heads x 2 ranges x 16384 rows x 129 floats = 32.25 MiB
    assert lib.fa_split_workspace_bytes(1, 2, 16384, 128, 2) <= (64 << 20)
    assert call_noalloc(lib, N=0, q=None, k=None, v=None, o=None, lse=None) == 0


def call_merge(lib, op=A, lp=A + 256 * MB, G=2, S=3, M=100, d=64, o=A + 512 * MB, lse=A + 768 * MB, dtype=2):
    return lib.fa_merge(op, lp, G, S, M, d, o, lse, dtype, None)


def test_merge_error_codes(lib):
    codes = _header_enum("fa_status_t")
    _split_lib(lib)
    assert call_merge(lib, S=0) == codes["FA_ERR_BAD_SHAPE"]
    assert call_merge(lib, G=-1) == codes["FA_ERR_BAD_SHAPE"]
    assert call_merge(lib, G=1 << 40, M=1 << 30) == codes["FA_ERR_BAD_SHAPE"]
    assert call_merge(lib, d=32) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    assert call_merge(lib, dtype=5) == codes["FA_ERR_UNSUPPORTED_DTYPE"]
    for field in ("op", "lp", "o", "lse"):
        assert call_merge(lib, **{field: None}) == codes["FA_ERR_NULL_POINTER"], field
    assert call_merge(lib, op=A + 4) == codes["FA_ERR_MISALIGNED"]
    assert call_merge(lib, lse=A + 768 * MB + 2) == codes["FA_ERR_MISALIGNED"]
    assert call_merge(lib, o=A + 1024) == codes["FA_ERR_ALIAS"]                 # O inside the O parts
    assert call_merge(lib, lse=A + 512 * MB + 64) == codes["FA_ERR_ALIAS"]      # LSE inside O
    assert call_merge(lib, lse=A + 256 * MB) == codes["FA_ERR_ALIAS"]           # LSE on the LSE parts
    assert call_merge(lib, M=0, op=None, lp=None, o=None, lse=None) == 0


def call_fp8(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, B=1, H=2, Hkv=2, N=1000,
             d=128, scale=0.1, dq=0.01, dk=0.01, dv=0.01, out=2):
    lib.fa_forward_fp8.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [ctypes.c_float] * 4 + [
        ctypes.c_int, ctypes.c_void_p]
    return lib.fa_forward_fp8(q, k, v, o, lse, B, H, Hkv, N, d, scale, dq, dk, dv, out, None)


def test_fp8_error_codes(lib):
    codes = _header_enum("fa_status_t")
    assert call_fp8(lib, N=-1) == codes["FA_ERR_BAD_SHAPE"]
    assert call_fp8(lib, Hkv=3) == codes["FA_ERR_BAD_SHAPE"]
    assert call_fp8(lib, N=1 << 25) == codes["FA_ERR_BAD_SHAPE"]              # 4 GiB per head > 32-bit offsets
    assert call_fp8(lib, out=7) == codes["FA_ERR_UNSUPPORTED_DTYPE"]
    assert call_fp8(lib, d=256) == codes["FA_ERR_UNSUPPORTED_HEAD_DIM"]
    for field in ("scale", "dq", "dk", "dv"):
        assert call_fp8(lib, **{field: math.inf}) == codes["FA_ERR_BAD_SCALE"], field
        assert call_fp8(lib, **{field: math.nan}) == codes["FA_ERR_BAD_SCALE"], field
    # finite factors whose product scale * dq * dk (times log2 e) overflows
    # float32, though each one alone is fine
    assert call_fp8(lib, scale=1e30, dq=1e10, dk=1e10) == codes["FA_ERR_BAD_SCALE"]
    assert call_fp8(lib, scale=-1e30, dq=1e5, dk=3e3) == codes["FA_ERR_BAD_SCALE"]
    # a product that underflows float32 is a valid (uniform-weight) call
    assert call_fp8(lib, N=0, scale=1e-30, dq=1e-20, dk=1e-20) == 0
    for field in ("q", "k", "v", "o", "lse"):
        assert call_fp8(lib, **{field: None}) == codes["FA_ERR_NULL_POINTER"], field
    assert call_fp8(lib, k=A + 64 * MB + 8) == codes["FA_ERR_MISALIGNED"]
    # O (bf16, 512,000 B) runs into LSE; Q is 256,000 B of codes
    assert call_fp8(lib, lse=A + 192 * MB + 511_000) == codes["FA_ERR_ALIAS"]
    assert call_fp8(lib, o=A + 255_984) == codes["FA_ERR_ALIAS"]
    assert call_fp8(lib, N=0, q=None, k=None, v=None, o=None, lse=None) == 0
