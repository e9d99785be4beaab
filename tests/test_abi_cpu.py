"""CPU-side checks of the C ABI: the library loads, exports every function
include/fa.h declares, and rejects bad arguments before launching anything.

Only argument combinations that fail validation are passed here (with fake,
never-dereferenced pointers), so no HIP call is made and no GPU is needed.
"""
import ctypes
import os
import re

import pytest
import torch

import exact_io_aware_forward_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)
MISALIGNED_LSE = ctypes.c_void_p(0x10002)   # LSE needs 4-byte alignment only

# These calls pass fake device pointers and rely on validation rejecting them
# before any launch.  Where a GPU is visible a mistaken case would launch a
# kernel on them, so the module only runs where none is (the CPU suite).
if torch.cuda.device_count() > 0:
    pytest.skip("argument-validation tests use fake pointers; run them without a GPU",
                allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    # FA_ABI_TEST_LIB names another build of the same C ABI to run these checks
    # on (tests/test_abi_sanitized.py: the host code under AddressSanitizer and
    # UndefinedBehaviorSanitizer).
    return fa.load_library(os.environ.get("FA_ABI_TEST_LIB", fa.LIB_PATH))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(fa.SYMBOLS)
    for name in names:
        assert hasattr(lib, name), name


def test_binding_exports_its_public_functions():
    public = {n for n, obj in vars(fa).items() if not n.startswith("_") and callable(obj)
              and getattr(obj, "__module__", None) == fa.__name__}
    assert public <= set(fa.__all__)
    assert all(hasattr(fa, n) for n in fa.__all__)


def fwd(lib, *, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=128, d=64, causal=0,
        scale=0.125, dtype=fa.FA_BF16):
    return lib.fa_forward(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, None)


def bwd(lib, *, ptr=FAKE, lse=None, B=1, H=1, N=128, d=64, causal=0, scale=0.125,
        dtype=fa.FA_BF16, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_backward_workspace_size(B, H, N, d)
    p = [ptr] * 9   # Q, K, V, O, dO, LSE, dQ, dK, dV
    if lse is not None:
        p[5] = lse
    return lib.fa_backward(*p, B, H, N, d, causal, scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=-0.5), fa.FA_ERR_UNSUPPORTED),
    (dict(o=MISALIGNED), fa.FA_ERR_INVALID_ARG),
    (dict(lse=MISALIGNED_LSE), fa.FA_ERR_INVALID_ARG),
    (dict(B=1 << 20, H=1 << 12), fa.FA_ERR_INVALID_ARG),
    (dict(N=1 << 23, d=128), fa.FA_ERR_UNSUPPORTED),     # one head of 2 GB
    (dict(N=1 << 24, d=64), fa.FA_ERR_UNSUPPORTED),         # N * d = 2^30
])
def test_forward_validation(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""


def test_blockmap_requires_codes_pointer(lib):
    assert lib.fa_forward_blockmap(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 1, 0.125,
                                   fa.FA_BF16, None, None) == fa.FA_ERR_INVALID_ARG


def test_backward_blockmap_requires_codes_pointers(lib):
    ws_bytes = 2 * 128 * 4
    for c1, c2 in ((None, FAKE), (FAKE, None)):
        assert lib.fa_backward_blockmap(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        1, 1, 128, 64, 1, 0.125, fa.FA_BF16, FAKE, ws_bytes,
                                        c1, c2, None) == fa.FA_ERR_INVALID_ARG
        assert lib.fa_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(ptr=None), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=4), fa.FA_ERR_WORKSPACE),
    (dict(ws=MISALIGNED), fa.FA_ERR_WORKSPACE),
    (dict(ptr=MISALIGNED), fa.FA_ERR_INVALID_ARG),
    (dict(lse=MISALIGNED_LSE), fa.FA_ERR_INVALID_ARG),
    (dict(N=-3), fa.FA_ERR_INVALID_ARG),
])
def test_backward_validation(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_workspace_size_is_two_floats_per_row(lib):
    assert lib.fa_backward_workspace_size(2, 16, 4096, 128) == 2 * 2 * 16 * 4096 * 4
    assert lib.fa_backward_workspace_size(0, 16, 4096, 128) == 0


def test_tile_config(lib):
    br, bc = ctypes.c_int(), ctypes.c_int()
    assert lib.fa_tile_config(0, 128, fa.FA_BF16, ctypes.byref(br), ctypes.byref(bc)) == fa.FA_OK
    assert br.value > 0 and bc.value > 0 and br.value % 32 == 0 and bc.value % 32 == 0
    assert lib.fa_tile_config(1, 64, fa.FA_F16, ctypes.byref(br), ctypes.byref(bc)) == fa.FA_OK
    assert lib.fa_tile_config(2, 64, fa.FA_F16, ctypes.byref(br), ctypes.byref(bc)) == fa.FA_OK
    assert lib.fa_tile_config(1, 64, fa.FA_F32, ctypes.byref(br), ctypes.byref(bc)) == \
        fa.FA_ERR_UNSUPPORTED
    # The forward without the causal mask: two 32-row blocks per wave (512 rows)
    # for 16-bit inputs at d = 64, the causal forward's 256 otherwise.
    for kid, d, dt, rows in ((0, 64, fa.FA_F16, 256), (3, 64, fa.FA_F16, 512), (3, 64, fa.FA_BF16, 512),
                             (3, 128, fa.FA_BF16, 256), (3, 64, fa.FA_F32, 256)):
        assert lib.fa_tile_config(kid, d, dt, ctypes.byref(br), ctypes.byref(bc)) == fa.FA_OK
        assert (br.value, bc.value) == (rows, 64)
    # dK/dV: 128-key tiles, 64 query rows at d = 128 and 32 at d = 64; dQ: 256
    # query rows, 32-key tiles at d = 128 and 64 at d = 64.
    for kid, d, rows, cols in ((1, 128, 64, 128), (1, 64, 32, 128), (2, 128, 256, 32), (2, 64, 256, 64)):
        assert lib.fa_tile_config(kid, d, fa.FA_BF16, ctypes.byref(br), ctypes.byref(bc)) == fa.FA_OK
        assert (br.value, bc.value) == (rows, cols)
    assert lib.fa_tile_config(4, 64, fa.FA_F16, ctypes.byref(br), ctypes.byref(bc)) == \
        fa.FA_ERR_INVALID_ARG
    assert lib.fa_tile_config(0, 96, fa.FA_F16, ctypes.byref(br), ctypes.byref(bc)) == \
        fa.FA_ERR_UNSUPPORTED


def test_strerror(lib):
    for s in (0, -1, -2, -3, -4, 99):
        assert lib.fa_strerror(s).decode()


def dec(lib, *, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Hkv=None, Nq=1, Nk=1000,
        d=128, causal=0, scale=0.125, dtype=fa.FA_BF16, splits=0, ws=FAKE, ws_bytes=None):
    Hkv = H if Hkv is None else Hkv
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_workspace_size(B, H, max(Hkv, 1), Nq, Nk, d, splits)
    return lib.fa_decode(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, dtype, splits, ws,
                         ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=5, Nk=4), fa.FA_ERR_INVALID_ARG),
    (dict(splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4, ws_bytes=1 << 20), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0, ws_bytes=1 << 20), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=33), fa.FA_ERR_UNSUPPORTED),
    (dict(H=8, Hkv=1, Nq=5, ws_bytes=1 << 20), fa.FA_ERR_UNSUPPORTED),   # 40 rows per kv head
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_UNSUPPORTED),
    (dict(k=MISALIGNED), fa.FA_ERR_INVALID_ARG),
    (dict(lse=MISALIGNED_LSE), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws=MISALIGNED), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(H=8, Hkv=2, Nq=4, ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(Nk=1 << 23, ws_bytes=1 << 30), fa.FA_ERR_UNSUPPORTED),   # a 2 GB cache head
])
def test_decode_validation(lib, kw, status):
    assert dec(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""


def test_decode_stage_validation(lib):
    ws = lib.fa_decode_workspace_size(1, 1, 1, 1, 64, 64, 0)
    assert lib.fa_decode_stage(2, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 64, 0, 0.125,
                               fa.FA_BF16, 0, FAKE, ws, None) == fa.FA_ERR_INVALID_ARG
    # the split stage needs Q, K, V but not O and LSE, the combine the reverse
    assert lib.fa_decode_stage(0, None, FAKE, FAKE, None, None, 1, 1, 1, 1, 64, 64, 0, 0.125,
                               fa.FA_BF16, 0, FAKE, ws, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_decode_stage(1, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 1, 1, 64, 64, 0, 0.125,
                               fa.FA_BF16, 0, FAKE, ws, None) == fa.FA_ERR_INVALID_ARG


def test_decode_split_count_and_workspace(lib):
    # 32 heads of a 128K cache: 8 slices fill 256 workgroups.
    assert lib.fa_decode_num_splits(1, 32, 32, 1, 131072, 128) == 8
    # grouped heads: 4 key/value heads need 64 slices for 256 workgroups
    assert lib.fa_decode_num_splits(1, 32, 4, 1, 131072, 128) == 64
    # short caches keep at least 16 tiles of 32 keys per slice, or one slice
    assert lib.fa_decode_num_splits(1, 1, 1, 1, 100, 128) == 1
    assert lib.fa_decode_num_splits(1, 1, 1, 1, 32 * 16 * 3, 128) == 3
    assert lib.fa_decode_num_splits(1, 1, 1, 1, 32 * 16 * 3 - 32, 128) == 2
    # many heads: no split
    assert lib.fa_decode_num_splits(64, 32, 32, 1, 131072, 128) == 1
    # no slice is ever empty, and an explicit count above the tile count is clamped
    # (one partial per slice; at most 512 slices; rows = H * Nq in every case)
    for nk, s in ((1000, 7), (1000, 31), (33, 5), (4, 4), (10 ** 6, 5000)):
        nt = -(-nk // 32)
        eff = min(s, nt, 512)
        tps = -(-nt // eff)
        eff = -(-nt // tps)
        assert lib.fa_decode_workspace_size(2, 3, 3, 4, nk, 64, s) == 2 * 3 * eff * 4 * (64 + 4) * 4
        assert lib.fa_decode_workspace_size(2, 6, 3, 4, nk, 64, s) == 2 * 6 * eff * 4 * (64 + 4) * 4
    assert lib.fa_decode_num_splits(1, 1, 1, 40, 1000, 128) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_decode_workspace_size(1, 1, 1, 2, 1, 128, 0) == 0


@pytest.mark.parametrize("H,Hkv", [(6, 4), (4, 0), (4, -2)])
def test_grouped_head_counts_are_validated(lib, H, Hkv):
    assert lib.fa_forward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, H, Hkv, 128, 64, 0, 0.125,
                              fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG
    ws = lib.fa_backward_workspace_size(1, H, 128, 64)
    assert lib.fa_backward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, H, Hkv,
                               128, 64, 0, 0.125, fa.FA_BF16, FAKE, ws, None) == \
        fa.FA_ERR_INVALID_ARG
    assert lib.fa_last_error().decode() != ""


def test_grouped_backward_workspace_size(lib):
    # One workgroup per (key/value head, key tile) while the grid is large enough:
    # the multi-head size.  Otherwise the smallest group split reaching 512
    # workgroups, with fp32 partial dK and dV after the per-row floats.
    assert lib.fa_backward_gqa_workspace_size(2, 16, 16, 4096, 128) == \
        lib.fa_backward_workspace_size(2, 16, 4096, 128)
    assert lib.fa_backward_gqa_workspace_size(2, 16, 8, 4096, 128) == \
        lib.fa_backward_workspace_size(2, 16, 4096, 128)          # 512 workgroups
    rows = 2 * 16 * 4096
    # B=2, Hkv=2: 128 workgroups -> split 4
    assert lib.fa_backward_gqa_workspace_size(2, 16, 2, 4096, 128) == \
        4 * (2 * rows + 2 * 4 * 2 * 2 * 4096 * 128)
    # B=2, Hkv=4: 256 workgroups -> split 2
    assert lib.fa_backward_gqa_workspace_size(2, 16, 4, 4096, 128) == \
        4 * (2 * rows + 2 * 2 * 2 * 4 * 4096 * 128)
    # a group of 3 on a tiny grid: split 3 (the whole group)
    assert lib.fa_backward_gqa_workspace_size(1, 3, 1, 100, 64) == \
        4 * ((2 * 300 + 3) // 4 * 4 + 2 * 3 * 1 * 100 * 64)
    # odd row count: the multi-head size is unchanged (no rounding)
    assert lib.fa_backward_gqa_workspace_size(1, 1, 1, 1, 64) == 8
    assert lib.fa_backward_gqa_workspace_size(1, 6, 4, 128, 64) == 0
    assert lib.fa_backward_gqa_workspace_size(1, 4, 2, 128, 96) == 0


def fp8q(lib, *, x=FAKE, rows=100, d=128, dtype=fa.FA_BF16, signs=FAKE, codes=FAKE, scales=FAKE):
    return lib.fa_fp8_quantize_rows(x, rows, d, dtype, signs, codes, scales, None)


@pytest.mark.parametrize("kw,status", [
    ({"x": None}, fa.FA_ERR_INVALID_ARG),
    ({"codes": None}, fa.FA_ERR_INVALID_ARG),
    ({"scales": None}, fa.FA_ERR_INVALID_ARG),
    ({"rows": -1}, fa.FA_ERR_INVALID_ARG),
    ({"rows": 1 << 31}, fa.FA_ERR_INVALID_ARG),
    ({"dtype": 7}, fa.FA_ERR_INVALID_ARG),
    ({"dtype": fa.FA_F32}, fa.FA_ERR_UNSUPPORTED),
    ({"d": 96}, fa.FA_ERR_UNSUPPORTED),
    ({"d": 256}, fa.FA_ERR_UNSUPPORTED),
    ({"x": MISALIGNED}, fa.FA_ERR_INVALID_ARG),
    ({"signs": MISALIGNED}, fa.FA_ERR_INVALID_ARG),
    ({"codes": ctypes.c_void_p(0x10004)}, fa.FA_ERR_INVALID_ARG),
    ({"scales": ctypes.c_void_p(0x10002)}, fa.FA_ERR_INVALID_ARG),
])
def test_fp8_quantize_validation(lib, kw, status):
    assert fp8q(lib, **kw) == status
    assert lib.fa_last_error().decode()


def test_fp8_quantize_zero_rows_launches_nothing(lib):
    # rows = 0 returns before any HIP call (the fake pointers are never used).
    assert fp8q(lib, rows=0) == fa.FA_OK
    assert fp8q(lib, rows=0, signs=None) == fa.FA_OK
    assert fp8q(lib, rows=0, x=None, codes=None, scales=None) == fa.FA_OK
    assert fp8q(lib, rows=0, d=96) == fa.FA_ERR_UNSUPPORTED


def test_noalloc_backward_rejects_inputs_beyond_its_scratch(lib):
    p = [FAKE] * 9
    # B * H * N = 2^20 + 1 rows: two floats each exceed the 8 MiB static array.
    assert lib.fa_backward_noalloc(*p, 1, 1, (1 << 20) + 1, 64, 0, 0.125, fa.FA_BF16,
                                   None) == fa.FA_ERR_WORKSPACE
    assert b"static array" in lib.fa_last_error()
    assert lib.fa_backward_noalloc(*p, 2, 8, (1 << 16) + 1, 128, 1, 0.125, fa.FA_F16,
                                   None) == fa.FA_ERR_WORKSPACE
    # the other checks come first, as in fa_backward
    assert lib.fa_backward_noalloc(*p, 0, 1, 64, 64, 0, 0.125, fa.FA_BF16,
                                   None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_backward_noalloc(*p, 1, 1, 64, 64, 0, 0.125, fa.FA_F32,
                                   None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_backward_noalloc(None, *p[1:], 1, 1, 64, 64, 0, 0.125, fa.FA_BF16,
                                   None) == fa.FA_ERR_INVALID_ARG


def fwd8(lib, *, qc=FAKE, qs=FAKE, kc=FAKE, ks=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=128,
         d=128, causal=1, scale=0.125, dtype=fa.FA_BF16):
    return lib.fa_forward_fp8(qc, qs, kc, ks, v, o, lse, B, H, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qc=None), fa.FA_ERR_INVALID_ARG),
    (dict(ks=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=9), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(kc=MISALIGNED), fa.FA_ERR_INVALID_ARG),
    (dict(v=MISALIGNED), fa.FA_ERR_INVALID_ARG),
    (dict(qs=ctypes.c_void_p(0x10002)), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 23), fa.FA_ERR_UNSUPPORTED),
])
def test_fp8_forward_validation(lib, kw, status):
    assert fwd8(lib, **kw) == status
