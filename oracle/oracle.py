"""ctypes wrapper of the fp64 CPU oracle (``h3_oracle.cpp``, ``h3_oracle_fp8.cpp``).

TEST INFRASTRUCTURE ONLY.  Importable by the tests, the smoke check and the
benchmark's CPU-baseline leg; the product package never imports it.

Inputs are numpy ``uint16`` arrays holding bf16 bit patterns (the exact values
the GPU path receives); outputs are numpy ``float64`` arrays.  The definitions
and the page passages they follow are documented in ``h3_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "h3_oracle.cpp"), os.path.join(_HERE, "h3_oracle_fp8.cpp"),
         os.path.join(_HERE, "h3_oracle_block.cpp"), os.path.join(_HERE, "h3_oracle_skip.cpp")]
_LIB = os.path.join(_HERE, "libh3oracle.so")

# Plain -O3 (vectorises the independent per-key / per-channel loops); no
# -ffast-math and no FMA contraction, so each product and sum is rounded as written.
GXX_CMD = ["g++", "-O3", "-std=c++17", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", *_SRCS, "-o", _LIB]


def build(force: bool = False) -> str:
    """Compile the oracle shared library (idempotent unless ``force``)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            [os.path.getmtime(f) for f in _SRCS] +
            [os.path.getmtime(os.path.join(_HERE, "h3_oracle.h"))]):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = GXX_CMD[:-1] + [tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class Rope(ctypes.Structure):
    """Oracle-side rotary descriptor (mirrors ``h3o_rope``)."""
    _fields_ = [("theta", ctypes.c_double), ("n_1d", ctypes.c_int64),
                ("sections", ctypes.c_int32 * 3), ("grid_t", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32)]


def make_rope(theta: float, n_1d: int, sections=(0, 0, 0), grid=(0, 0, 0)) -> Rope:
    r = Rope()
    r.theta = float(theta)
    r.n_1d = int(n_1d)
    for i in range(3):
        r.sections[i] = int(sections[i])
    r.grid_t, r.grid_h, r.grid_w = (int(g) for g in grid)
    return r


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.c_double
        I = ctypes.c_int
        _lib.h3o_widen_bf16.argtypes = [P, I64, P]
        _lib.h3o_widen_bf16.restype = None
        _lib.h3o_rmsnorm_row.argtypes = [P, P, I64, D, P]
        _lib.h3o_rmsnorm_row.restype = None
        _lib.h3o_rope_row.argtypes = [P, I64, I, P, P, D, P]
        _lib.h3o_rope_row.restype = I
        _lib.h3o_token_position.argtypes = [ctypes.POINTER(Rope), I64,
                                            ctypes.POINTER(I), P]
        _lib.h3o_token_position.restype = I
        _lib.h3o_prologue.argtypes = [P, I64, I64, I64, I64, P, I64, D,
                                      ctypes.POINTER(Rope), P, I64, I, P]
        _lib.h3o_prologue.restype = I
        _lib.h3o_attention.argtypes = [P, P, P, I64, I64, I64, I64, D, I, P]
        _lib.h3o_attention.restype = I
        _lib.h3o_attn_varlen.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, P, I64,
                                         I, P]
        _lib.h3o_attn_varlen.restype = I
        _lib.h3o_attn_layer.argtypes = [P, P, P, I64, I64, I64, I64, I64, P, P, I64, D,
                                        ctypes.POINTER(Rope), D, P, I64, I, P]
        _lib.h3o_attn_layer.restype = I
        _lib.h3o_e4m3.argtypes = [D]
        _lib.h3o_e4m3.restype = D
        _lib.h3o_round_bf16.argtypes = [D]
        _lib.h3o_round_bf16.restype = ctypes.c_uint16
        _lib.h3o_quantize_group.argtypes = [P, I64, P, P]
        _lib.h3o_quantize_group.restype = None
        _lib.h3o_attn_varlen_fp8.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, I64, D,
                                             P, I64, I, P, P]
        _lib.h3o_attn_varlen_fp8.restype = I
        _lib.h3o_attn_layer_fp8.argtypes = [P, P, P, I64, I64, I64, I64, I64, P, P, I64, D,
                                            ctypes.POINTER(Rope), D, I64, D, P, I64, I, P, P]
        _lib.h3o_attn_layer_fp8.restype = I
        _lib.h3o_attn_varlen_skip.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, I64, D,
                                              P, I64, I, P, P]
        _lib.h3o_attn_varlen_skip.restype = I
        _lib.h3o_attn_layer_skip.argtypes = [P, P, P, I64, I64, I64, I64, I64, P, P, I64, D,
                                             ctypes.POINTER(Rope), D, I64, D, P, I64, I, P, P]
        _lib.h3o_attn_layer_skip.restype = I
        _lib.h3o_residual_norm_modulate.argtypes = [P, P, P, P, P, I64, I64, I64, D, P, P]
        _lib.h3o_residual_norm_modulate.restype = I
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs must be passed as uint16 bit patterns")
    return a


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def widen_bf16(bits) -> np.ndarray:
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib().h3o_widen_bf16(_ptr(b), b.size, _ptr(out))
    return out


def rmsnorm_row(x, w, eps: float) -> np.ndarray:
    x = _f64(x)
    w = _f64(w)
    assert x.ndim == 1 and w.shape == x.shape
    y = np.empty_like(x)
    lib().h3o_rmsnorm_row(_ptr(x), _ptr(w), x.size, float(eps), _ptr(y))
    return y


def rope_row(x, mode: int, pos, sections=(0, 0, 0), theta: float = 10000.0) -> np.ndarray:
    x = _f64(x)
    p = _f64(list(pos) + [0.0] * (3 - len(pos)))
    s = np.ascontiguousarray(sections, dtype=np.int32)
    y = np.empty_like(x)
    _check(lib().h3o_rope_row(_ptr(x), x.size, int(mode), _ptr(p), _ptr(s), float(theta),
                              _ptr(y)), "rope_row")
    return y


def token_position(rope: Rope, i: int):
    mode = ctypes.c_int()
    pos = np.zeros(3, dtype=np.float64)
    _check(lib().h3o_token_position(ctypes.byref(rope), int(i), ctypes.byref(mode),
                                    _ptr(pos)), "token_position")
    return mode.value, pos


def prologue(x_bits, n_valid: int, w_bits, eps: float, rope: Rope, rows,
             w_head_stride: int = 0, threads: int | None = None) -> np.ndarray:
    """RMSNorm + RoPE of tokens ``rows`` of ``x_bits`` [S, H, D] -> [n_rows, H, D]."""
    x = _u16(x_bits)
    S, H, D = x.shape
    w = _u16(w_bits)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), dtype=np.float64)
    _check(lib().h3o_prologue(_ptr(x), H, D, H * D, int(n_valid), _ptr(w),
                              int(w_head_stride), float(eps), ctypes.byref(rope),
                              _ptr(rows), rows.size, threads or default_threads(),
                              _ptr(out)), "prologue")
    return out


def attention(q, k, v, scale: float, threads: int | None = None) -> np.ndarray:
    """Softmax attention on fp64 operands: q [R, H, D], k/v [N, H, D] -> [R, H, D]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    R, H, D = q.shape
    N = k.shape[0]
    assert k.shape == (N, H, D) and v.shape == (N, H, D)
    out = np.empty((R, H, D), dtype=np.float64)
    _check(lib().h3o_attention(_ptr(q), _ptr(k), _ptr(v), R, N, H, D, float(scale),
                               threads or default_threads(), _ptr(out)), "attention")
    return out


def attn_varlen(q_bits, k_bits, v_bits, n_valid: int, scale: float, rows,
                threads: int | None = None) -> np.ndarray:
    """Attention over bf16 [S, H, D] buffers (Q/K already prepared) -> [R, H, D]."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    S, H, D = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), dtype=np.float64)
    _check(lib().h3o_attn_varlen(_ptr(q), _ptr(k), _ptr(v), S, int(n_valid), H, D, H * D,
                                 float(scale), _ptr(rows), rows.size,
                                 threads or default_threads(), _ptr(out)), "attn_varlen")
    return out


def attn_layer(q_bits, k_bits, v_bits, n_valid: int, wq_bits, wk_bits, eps: float,
               rope: Rope, scale: float, rows, w_head_stride: int = 0,
               threads: int | None = None) -> np.ndarray:
    """RMSNorm + RoPE + attention over bf16 [S, H, D] buffers -> [R, H, D]."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    wq, wk = _u16(wq_bits), _u16(wk_bits)
    S, H, D = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), dtype=np.float64)
    _check(lib().h3o_attn_layer(_ptr(q), _ptr(k), _ptr(v), S, int(n_valid), H, D, H * D,
                                _ptr(wq), _ptr(wk), int(w_head_stride), float(eps),
                                ctypes.byref(rope), float(scale), _ptr(rows), rows.size,
                                threads or default_threads(), _ptr(out)), "attn_layer")
    return out


# ---- FP8 ("SAGE") variant


def e4m3(x: float) -> float:
    """Nearest FP8 E4M3 value of x (ties to even, saturating at +-448)."""
    return lib().h3o_e4m3(float(x))


def round_bf16(x: float) -> int:
    """Bits of the nearest bf16 of x (ties to even)."""
    return int(lib().h3o_round_bf16(float(x)))


def quantize_group(x) -> tuple[np.ndarray, float]:
    """One-scale FP8 quantization of bf16-valued inputs, decided in fp64: (codes, scale)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.size, dtype=np.float64)
    scale = ctypes.c_double()
    lib().h3o_quantize_group(_ptr(x), x.size, _ptr(codes), ctypes.byref(scale))
    return codes.reshape(x.shape), scale.value


FP8_P_TILE = 64  # keys per tile of the streamed softmax weights


def attn_varlen_fp8(q_bits, k_bits, v_bits, n_valid: int, scale: float, rows,
                    threads: int | None = None, p_tile: int = FP8_P_TILE,
                    skip_threshold: float = 0.0, with_wmax: bool = False):
    """FP8 attention over bf16 [S, H, D] buffers (Q/K already prepared) -> [R, H, D];
    P quantized against the running row maximum of ``p_tile``-key tiles; tiles below
    the running maximum by a factor under ``skip_threshold`` dropped per row.  With
    ``with_wmax`` returns (out, wmax): wmax [R, H] is each row's largest normalised
    weight."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    S, H, D = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), dtype=np.float64)
    wmax = np.empty((rows.size, H), dtype=np.float64)
    _check(lib().h3o_attn_varlen_fp8(_ptr(q), _ptr(k), _ptr(v), S, int(n_valid), H, D, H * D,
                                     float(scale), int(p_tile), float(skip_threshold),
                                     _ptr(rows), rows.size,
                                     threads or default_threads(), _ptr(out), _ptr(wmax)),
           "attn_varlen_fp8")
    return (out, wmax) if with_wmax else out


def attn_layer_fp8(q_bits, k_bits, v_bits, n_valid: int, wq_bits, wk_bits, eps: float,
                   rope: Rope, scale: float, rows, w_head_stride: int = 0,
                   threads: int | None = None, p_tile: int = FP8_P_TILE,
                   skip_threshold: float = 0.0, with_wmax: bool = False):
    """RMSNorm + RoPE (rounded to bf16) + FP8 attention over bf16 [S, H, D] buffers;
    ``with_wmax`` as for attn_varlen_fp8."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    wq, wk = _u16(wq_bits), _u16(wk_bits)
    S, H, D = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), dtype=np.float64)
    wmax = np.empty((rows.size, H), dtype=np.float64)
    _check(lib().h3o_attn_layer_fp8(_ptr(q), _ptr(k), _ptr(v), S, int(n_valid), H, D, H * D,
                                    _ptr(wq), _ptr(wk), int(w_head_stride), float(eps),
                                    ctypes.byref(rope), float(scale), int(p_tile),
                                    float(skip_threshold), _ptr(rows),
                                    rows.size, threads or default_threads(), _ptr(out),
                                    _ptr(wmax)),
           "attn_layer_fp8")
    return (out, wmax) if with_wmax else out


# ---- dense attention with Skip-Softmax (the "Skip-Softmax-only" control)

SKIP_P_TILE = 64  # keys per tile of the Skip-Softmax decision


def attn_varlen_skip(q_bits, k_bits, v_bits, n_valid: int, scale: float, rows,
                     skip_threshold: float, threads: int | None = None,
                     p_tile: int = SKIP_P_TILE, with_wmax: bool = False):
    """Dense attention over bf16 [S, H, D] buffers (Q/K already prepared) with tiles of
    ``p_tile`` keys dropped per row by the Skip-Softmax rule -> [R, H, D] (and, with
    ``with_wmax``, each row's largest normalised weight [R, H])."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    S, H, D = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), dtype=np.float64)
    wmax = np.empty((rows.size, H), dtype=np.float64)
    _check(lib().h3o_attn_varlen_skip(_ptr(q), _ptr(k), _ptr(v), S, int(n_valid), H, D, H * D,
                                      float(scale), int(p_tile), float(skip_threshold),
                                      _ptr(rows), rows.size, threads or default_threads(),
                                      _ptr(out), _ptr(wmax)), "attn_varlen_skip")
    return (out, wmax) if with_wmax else out


def attn_layer_skip(q_bits, k_bits, v_bits, n_valid: int, wq_bits, wk_bits, eps: float,
                    rope: Rope, scale: float, rows, skip_threshold: float,
                    w_head_stride: int = 0, threads: int | None = None,
                    p_tile: int = SKIP_P_TILE, with_wmax: bool = False):
    """fp64 RMSNorm + RoPE, then attention_varlen_skip's attention."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    wq, wk = _u16(wq_bits), _u16(wk_bits)
    S, H, D = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), dtype=np.float64)
    wmax = np.empty((rows.size, H), dtype=np.float64)
    _check(lib().h3o_attn_layer_skip(_ptr(q), _ptr(k), _ptr(v), S, int(n_valid), H, D, H * D,
                                     _ptr(wq), _ptr(wk), int(w_head_stride), float(eps),
                                     ctypes.byref(rope), float(scale), int(p_tile),
                                     float(skip_threshold), _ptr(rows), rows.size,
                                     threads or default_threads(), _ptr(out), _ptr(wmax)),
           "attn_layer_skip")
    return (out, wmax) if with_wmax else out


def residual_norm_modulate(x, a_bits, gate, shift, scale, n_valid: int, eps: float):
    """Gated residual update, LayerNorm and modulation of one sequence in fp64.
    x: fp32 [S, C]; a_bits: bf16 bits [S, C] or None; gate (or None), shift, scale:
    fp32 [C].  Returns (x_out, y) as float64 [S, C]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    S, C = x.shape
    a = None if a_bits is None else _u16(a_bits)
    g = None if gate is None else np.ascontiguousarray(gate, dtype=np.float32)
    sh = np.ascontiguousarray(shift, dtype=np.float32)
    sc = np.ascontiguousarray(scale, dtype=np.float32)
    x_out = np.empty((S, C), dtype=np.float64)
    y = np.empty((S, C), dtype=np.float64)
    _check(lib().h3o_residual_norm_modulate(_ptr(x), _ptr(a) if a is not None else None,
                                            _ptr(g) if g is not None else None, _ptr(sh),
                                            _ptr(sc), S, int(n_valid), C, float(eps),
                                            _ptr(x_out), _ptr(y)),
           "residual_norm_modulate")
    return x_out, y
