"""The C ABI on the host: the library loads, exports every declared entry point, and
rejects bad arguments before touching a device (no compute calls here)."""
import ctypes
import os
import re

import pytest
import torch

from long_sequence_attention_h3_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3attn.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first
WS = 0x20000    # 256-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    L = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = B.lib()
    for code, name in B.STATUS_NAMES.items():
        assert L.h3_status_string(code).decode().startswith(name)
    assert L.h3_status_string(99) == b"unknown h3_status"
    assert L.h3_version() >= 100


def shape(B_=1, H=2, D=128, S=1024, valid=(1000,), sin=None, sout=None):
    arr = (ctypes.c_int64 * len(valid))(*valid)
    s = B.Shape(B_, H, D, S, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)),
                H * D if sin is None else sin, H * D if sout is None else sout)
    s._keep = arr
    return s


def rope(n_1d=1000, sections=(0, 0, 0), grid=(0, 0, 0), theta=1e4):
    return B.make_rope(theta, n_1d, sections, grid)


def varlen(s, q=FAKE, ws=WS, ws_bytes=None, scale=0.088):
    L = B.lib()
    need = L.h3_attn_workspace_size(ctypes.byref(s)) if ws_bytes is None else ws_bytes
    return L.h3_attn_varlen(q, FAKE, FAKE, FAKE, scale, ctypes.byref(s), ws, need, None)


def layer(s, r, w=FAKE, whs=0, eps=1e-6):
    L = B.lib()
    need = L.h3_attn_workspace_size(ctypes.byref(s))
    return L.h3_attn_layer(FAKE, FAKE, FAKE, FAKE, w, w, whs, eps, ctypes.byref(r), 0.088,
                           ctypes.byref(s), WS, need, None)


def prologue(s, r, q_out=FAKE, eps=1e-6):
    return B.lib().h3_qk_rmsnorm_rope(FAKE, FAKE, q_out, FAKE, FAKE, FAKE, 0, eps,
                                      ctypes.byref(r), ctypes.byref(s), None)


def test_workspace_size_formula():
    """Tile images, then 8 pass-flag words per 256 query rows and head (room for up to 8
    key ranges) per batch, then, when some batch splits its keys into k > 1 ranges, the
    partial results of one batch: k*H*S rows of 128 floats, then k*H*S (max, sum) pairs."""
    L = B.lib()
    tile = 64 * 272 + 128 * 144  # padded K rows + padded V rows per 64-key tile

    def r256(nbytes):
        return (nbytes + 255) // 256 * 256

    def flags(words):
        return r256(words * 4)

    def part(k, H, S):
        return k * H * S * 128 * 4 + r256(k * H * S * 2 * 4)

    assert tile == 35840
    assert L.h3_attn_workspace_size(ctypes.byref(shape(H=42, S=58816, valid=(58758,)))) == \
        42 * 919 * tile + flags(8 * 42 * 230)
    assert L.h3_attn_workspace_size(ctypes.byref(shape(H=6, S=58816, valid=(58758,)))) == \
        6 * 919 * tile + flags(8 * 6 * 230) + part(2, 6, 58816)
    assert L.h3_attn_workspace_size(ctypes.byref(shape(H=2, S=1024, valid=(1000,)))) == \
        2 * 16 * tile + flags(8 * 2 * 4) + part(8, 2, 1024)
    assert L.h3_attn_workspace_size(ctypes.byref(shape(S=65, valid=(1,)))) == \
        2 * 2 * tile + flags(8 * 2 * 1)
    assert L.h3_attn_workspace_size(ctypes.byref(shape(B_=3, S=64, valid=(1, 2, 3)))) == \
        3 * 2 * 1 * tile + flags(3 * 8 * 2 * 1)
    assert L.h3_attn_workspace_size(ctypes.byref(shape(D=64))) == 0
    assert L.h3_attn_workspace_size(None) == 0


@pytest.mark.parametrize("H,S,N,k", [
    (2, 1024, 1000, 8),     # 8 query blocks: 8 key ranges of 2 tiles
    (8, 8192, 8150, 1),     # 256 blocks: one round on 256 compute units
    (6, 58816, 58758, 2),   # 1,380 blocks, 5.4 rounds: 2 ranges, 10.8 rounds
    (42, 58816, 58758, 1),  # 9,660 blocks, 37.7 rounds
    (42, 87552, 87500, 1),
    (2, 1024, 64, 1),       # one key tile cannot be split
    (2, 1024, 65, 2),
])
def test_key_range_splits(H, S, N, k):
    L = B.lib()
    assert L.h3_attn_splits(ctypes.byref(shape(H=H, S=S, valid=(N,))), 0) == k
    assert L.h3_attn_splits(ctypes.byref(shape(H=H, S=S, valid=(N,))), 1) == 0  # no batch 1
    assert L.h3_attn_splits(ctypes.byref(shape(D=64)), 0) == 0


@pytest.mark.parametrize("kwargs,code", [
    (dict(D=64), 4),                      # head_dim must be 128
    (dict(valid=(1025,)), 2),             # N > S
    (dict(valid=(-1,)), 2),               # N < 0
    (dict(sin=255), 2),                   # stride < H*D
    (dict(sin=260), 3),                   # stride not a multiple of 8 elements
    (dict(H=0), 2),
    (dict(B_=2, valid=(10, 2000)), 2),    # second batch N > S
])
def test_shape_validation(kwargs, code):
    assert varlen(shape(**kwargs)) == code


def test_pointer_and_workspace_validation():
    s = shape()
    assert varlen(s, q=0) == 1                       # NULL input
    assert varlen(s, q=FAKE + 2) == 3                # misaligned input
    assert varlen(s, ws=0) == 7                      # workspace missing
    assert varlen(s, ws_bytes=1000) == 7             # workspace too small
    assert varlen(s, ws=WS + 16) == 3                # workspace not 256-byte aligned
    assert varlen(s, scale=0.0) == 2                 # softmax scale must be > 0
    assert varlen(s, scale=float("nan")) == 2
    assert B.lib().h3_attn_varlen(FAKE, FAKE, FAKE, FAKE, 0.1, None, WS, 1, None) == 1


def test_rope_and_weight_validation():
    s = shape(valid=(1000,))
    assert layer(s, rope(n_1d=100)) == 4                        # 3-axis tokens, no sections
    assert layer(s, rope(n_1d=100, sections=(32, 48, 40), grid=(10, 10, 10))) == 4
    assert layer(s, rope(n_1d=100, sections=(40, 40, 48), grid=(10, 10, 10))) == 4  # not /16
    assert layer(s, rope(n_1d=100, sections=(32, 48, 48), grid=(8, 10, 10))) == 4   # grid small
    assert layer(s, rope(theta=0.0)) == 4
    assert layer(s, rope(), w=0) == 1
    assert layer(s, rope(), whs=64) == 2                       # per-head stride < D
    assert layer(s, rope(), eps=-1.0) == 2
    assert prologue(s, rope(), q_out=0) == 1
    # in place needs equal input and output strides
    s2 = shape(sin=512, sout=256)
    assert B.lib().h3_qk_rmsnorm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1e-6,
                                      ctypes.byref(rope()), ctypes.byref(s2), None) == 2


def test_stage_entry_points_validate():
    L = B.lib()
    s = shape()
    need = L.h3_attn_workspace_size(ctypes.byref(s))
    r = rope()
    assert L.h3_kv_pack(0, FAKE, None, 0, 0.0, None, 0.0, ctypes.byref(s), WS, need, None) == 1
    assert L.h3_kv_pack(FAKE, FAKE, None, 0, 0.0, None, 0.0, ctypes.byref(s), WS, need - 1,
                        None) == 7
    assert L.h3_kv_pack(FAKE, FAKE, FAKE, 0, 1e-6, None, 0.1, ctypes.byref(s), WS, need,
                        None) == 1
    # with w_k the softmax scale (the stored K's multiplier) must be positive and finite
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert L.h3_kv_pack(FAKE, FAKE, FAKE, 0, 1e-6, ctypes.byref(r), bad, ctypes.byref(s),
                            WS, need, None) == 2
    assert L.h3_attn_packed(FAKE, 0, None, 0, 0.0, None, 0.1, ctypes.byref(s), WS, need,
                            None) == 1
    assert L.h3_attn_packed(FAKE, FAKE, FAKE, 0, 1e-6, ctypes.byref(rope(n_1d=10)), 0.1,
                            ctypes.byref(s), WS, need, None) == 4
    assert L.h3_attn_packed(FAKE, FAKE, None, 0, 0.0, None, -1.0, ctypes.byref(s), WS, need,
                            None) == 2
    del r


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_valid_call_without_device_fails_loudly():
    L = B.lib()
    s = shape()
    assert varlen(s) == 5
    assert layer(s, rope()) == 5
    assert prologue(s, rope()) == 5
    need = L.h3_attn_workspace_size(ctypes.byref(s))
    assert L.h3_kv_pack(FAKE, FAKE, None, 0, 0.0, None, 0.0, ctypes.byref(s), WS, need,
                        None) == 5
    assert L.h3_kv_pack(FAKE, FAKE, FAKE, 0, 1e-6, ctypes.byref(rope()), 0.1, ctypes.byref(s),
                        WS, need, None) == 5
    assert L.h3_attn_packed(FAKE, FAKE, None, 0, 0.0, None, 0.1, ctypes.byref(s), WS, need,
                            None) == 5


def test_fp8_workspace_size_formula():
    L = B.lib()
    tile = 64 * 144 + 128 * 80  # K rows of 128 codes + 16 pad, V rows of 64 codes + 16 pad

    def words(n):  # n 4-byte words rounded up to 256 bytes
        return (n * 4 + 255) // 256 * 256

    assert tile == 19456
    f = L.h3_attn_fp8_workspace_size
    # tiles, then one V maximum per channel/head/batch, then one skip count per 256 rows
    assert f(ctypes.byref(shape(H=42, S=58816, valid=(58758,)))) == \
        42 * 919 * tile + words(42 * 128) + words(42 * 230)
    assert f(ctypes.byref(shape(S=65, valid=(1,)))) == 2 * 2 * tile + words(2 * 128) + words(2)
    assert f(ctypes.byref(shape(B_=3, S=64, valid=(1, 2, 3)))) == \
        3 * 2 * tile + words(3 * 256) + words(6)
    assert f(ctypes.byref(shape(D=64))) == 0
    assert f(None) == 0


def test_fp8_entry_points_validate():
    L = B.lib()
    s = shape()
    need = L.h3_attn_fp8_workspace_size(ctypes.byref(s))
    bf16_need = L.h3_attn_workspace_size(ctypes.byref(s))
    assert need < bf16_need
    assert L.h3_kv_pack_fp8(0, FAKE, None, 0, 0.0, None, ctypes.byref(s), WS, need, None) == 1
    assert L.h3_kv_pack_fp8(FAKE, FAKE, None, 0, 0.0, None, ctypes.byref(s), WS, need - 1,
                            None) == 7
    assert L.h3_kv_pack_fp8(FAKE, FAKE, None, 0, 0.0, None, ctypes.byref(s), WS + 16, need,
                            None) == 3
    assert L.h3_kv_pack_fp8(FAKE, FAKE, FAKE, 0, 1e-6, None, ctypes.byref(s), WS, need,
                            None) == 1
    assert L.h3_attn_packed_fp8(FAKE, 0, None, 0, 0.0, None, 0.1, 0.0, ctypes.byref(s), WS, need,
                                None) == 1
    assert L.h3_attn_packed_fp8(FAKE, FAKE, FAKE, 0, 1e-6, ctypes.byref(rope(n_1d=10)), 0.1,
                                0.0, ctypes.byref(s), WS, need, None) == 4
    assert L.h3_attn_packed_fp8(FAKE, FAKE, None, 0, 0.0, None, float("nan"), 0.0,
                                ctypes.byref(s), WS, need, None) == 2
    for bad in (-0.1, 1.0, float("nan")):  # Skip-Softmax threshold outside [0, 1)
        assert L.h3_attn_packed_fp8(FAKE, FAKE, None, 0, 0.0, None, 0.1, bad,
                                    ctypes.byref(s), WS, need, None) == 2
        assert L.h3_attn_varlen_fp8(FAKE, FAKE, FAKE, FAKE, 0.088, bad, ctypes.byref(s), WS,
                                    need, None) == 2
    assert L.h3_attn_varlen_fp8(FAKE, FAKE, FAKE, FAKE, 0.088, 0.0, ctypes.byref(shape(D=64)),
                                WS, need, None) == 4
    assert L.h3_attn_varlen_fp8(FAKE, FAKE, FAKE, FAKE, 0.088, 0.0, ctypes.byref(s), WS,
                                need - 1, None) == 7
    assert L.h3_attn_layer_fp8(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 1e-6, ctypes.byref(rope()),
                               0.088, 0.0, ctypes.byref(s), WS, need, None) == 1
    assert L.h3_attn_layer_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1e-6,
                               ctypes.byref(rope(n_1d=10)), 0.088, 0.0, ctypes.byref(s), WS,
                               need, None) == 4


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_fp8_valid_call_without_device_fails_loudly():
    L = B.lib()
    s = shape()
    need = L.h3_attn_fp8_workspace_size(ctypes.byref(s))
    assert L.h3_attn_varlen_fp8(FAKE, FAKE, FAKE, FAKE, 0.088, 0.0, ctypes.byref(s), WS, need,
                                None) == 5
    assert L.h3_attn_layer_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1e-6,
                               ctypes.byref(rope()), 0.088, 0.5, ctypes.byref(s), WS, need,
                               None) == 5
    assert L.h3_kv_pack_fp8(FAKE, FAKE, None, 0, 0.0, None, ctypes.byref(s), WS, need,
                            None) == 5
    assert L.h3_attn_packed_fp8(FAKE, FAKE, None, 0, 0.0, None, 0.1, 0.0, ctypes.byref(s), WS,
                                need, None) == 5


def rows_shape(B_=1, S=64, valid=(60,), C=128):
    arr = (ctypes.c_int64 * len(valid))(*valid)
    r = B.Rows(B_, S, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), C)
    r._keep = arr
    return r


@pytest.mark.parametrize("kwargs,code", [
    (dict(C=12), 4),          # hidden not a multiple of 8
    (dict(C=8200), 4),        # hidden above 8,192
    (dict(C=0), 2),
    (dict(valid=(65,)), 2),   # N > S
    (dict(valid=(-1,)), 2),
    (dict(B_=0), 2),
])
def test_block_shape_validation(kwargs, code):
    L = B.lib()
    r = rows_shape(**kwargs)
    assert L.h3_residual_norm_modulate(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1e-6, FAKE,
                                       ctypes.byref(r), None) == code


def test_block_pointer_validation():
    L = B.lib()
    r = rows_shape()
    f = L.h3_residual_norm_modulate
    assert f(0, FAKE, FAKE, FAKE, FAKE, 0, 1e-6, FAKE, ctypes.byref(r), None) == 1
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 0, 1e-6, FAKE, ctypes.byref(r), None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1e-6, FAKE, None, None) == 1
    assert f(FAKE + 4, FAKE, FAKE, FAKE, FAKE, 0, 1e-6, FAKE, ctypes.byref(r), None) == 3
    assert f(FAKE, FAKE + 2, FAKE, FAKE, FAKE, 0, 1e-6, FAKE, ctypes.byref(r), None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 1e-6, FAKE, ctypes.byref(r), None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 130, 1e-6, FAKE, ctypes.byref(r), None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, -1.0, FAKE, ctypes.byref(r), None) == 2


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_block_valid_call_without_device_fails_loudly():
    r = rows_shape()
    assert B.lib().h3_residual_norm_modulate(FAKE, None, None, FAKE, FAKE, 0, 1e-6, FAKE,
                                             ctypes.byref(r), None) == 5

