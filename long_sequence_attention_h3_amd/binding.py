"""Thin ctypes binding of libh3attn (include/h3attn.h).

Argument marshalling only: torch supplies device memory and the current stream,
every step of the layer runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: if ``libh3attn.so`` is missing or the device is not a gfx950,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libh3attn.so")

H3_OK = 0
STATUS_NAMES = {0: "H3_OK", 1: "H3_ERR_NULL", 2: "H3_ERR_SHAPE", 3: "H3_ERR_ALIGN",
                4: "H3_ERR_UNSUPPORTED", 5: "H3_ERR_DEVICE", 6: "H3_ERR_LAUNCH",
                7: "H3_ERR_WORKSPACE", 8: "H3_ERR_SCRATCH_LIMIT"}


class H3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Shape(ctypes.Structure):
    """``h3_shape``."""
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("seq_buf", ctypes.c_int64),
                ("seq_valid", ctypes.POINTER(ctypes.c_int64)),
                ("in_row_stride", ctypes.c_int64), ("out_row_stride", ctypes.c_int64)]


class Rope(ctypes.Structure):
    """``h3_rope``."""
    _fields_ = [("theta", ctypes.c_double), ("n_1d", ctypes.c_int64),
                ("sections", ctypes.c_int32 * 3), ("grid_t", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32)]


class Rows(ctypes.Structure):
    """``h3_rows``."""
    _fields_ = [("batch", ctypes.c_int32), ("seq_buf", ctypes.c_int64),
                ("seq_valid", ctypes.POINTER(ctypes.c_int64)), ("hidden", ctypes.c_int64)]


def make_rope(theta: float, n_1d: int, sections=(0, 0, 0), grid=(0, 0, 0)) -> Rope:
    r = Rope()
    r.theta = float(theta)
    r.n_1d = int(n_1d)
    for i in range(3):
        r.sections[i] = int(sections[i])
    r.grid_t, r.grid_h, r.grid_w = (int(g) for g in grid)
    return r


EXPORTED = ("h3_status_string", "h3_version", "h3_qk_rmsnorm_rope", "h3_attn_workspace_size",
            "h3_kv_pack", "h3_attn_packed", "h3_attn_varlen", "h3_attn_layer",
            "h3_attn_fp8_workspace_size", "h3_kv_pack_fp8", "h3_attn_packed_fp8",
            "h3_attn_varlen_fp8", "h3_attn_layer_fp8", "h3_residual_norm_modulate",
            "h3_attn_layer_noalloc", "h3_attn_layer_noalloc_max_workspace", "h3_attn_splits",
            "h3_attn_varlen_skip", "h3_attn_layer_skip")

_lib = None


def lib():
    """Load libh3attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m long_sequence_attention_h3_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        SH, RP = ctypes.POINTER(Shape), ctypes.POINTER(Rope)
        L.h3_status_string.argtypes = [ctypes.c_int]
        L.h3_status_string.restype = ctypes.c_char_p
        L.h3_version.argtypes = []
        L.h3_version.restype = ctypes.c_int
        L.h3_qk_rmsnorm_rope.argtypes = [P, P, P, P, P, P, I64, F, RP, SH, P]
        L.h3_qk_rmsnorm_rope.restype = ctypes.c_int
        L.h3_attn_workspace_size.argtypes = [SH]
        L.h3_attn_workspace_size.restype = SZ
        L.h3_attn_splits.argtypes = [SH, ctypes.c_int]
        L.h3_attn_splits.restype = ctypes.c_int
        L.h3_kv_pack.argtypes = [P, P, P, I64, F, RP, F, SH, P, SZ, P]
        L.h3_kv_pack.restype = ctypes.c_int
        L.h3_attn_packed.argtypes = [P, P, P, I64, F, RP, F, SH, P, SZ, P]
        L.h3_attn_packed.restype = ctypes.c_int
        L.h3_attn_varlen.argtypes = [P, P, P, P, F, SH, P, SZ, P]
        L.h3_attn_varlen.restype = ctypes.c_int
        L.h3_attn_layer.argtypes = [P, P, P, P, P, P, I64, F, RP, F, SH, P, SZ, P]
        L.h3_attn_layer.restype = ctypes.c_int
        L.h3_attn_varlen_skip.argtypes = [P, P, P, P, F, F, SH, P, SZ, P]
        L.h3_attn_varlen_skip.restype = ctypes.c_int
        L.h3_attn_layer_skip.argtypes = [P, P, P, P, P, P, I64, F, RP, F, F, SH, P, SZ, P]
        L.h3_attn_layer_skip.restype = ctypes.c_int
        L.h3_attn_layer_noalloc.argtypes = [P, P, P, P, P, P, I64, F, RP, F, SH, P]
        L.h3_attn_layer_noalloc.restype = ctypes.c_int
        L.h3_attn_layer_noalloc_max_workspace.argtypes = []
        L.h3_attn_layer_noalloc_max_workspace.restype = SZ
        L.h3_attn_fp8_workspace_size.argtypes = [SH]
        L.h3_attn_fp8_workspace_size.restype = SZ
        L.h3_kv_pack_fp8.argtypes = [P, P, P, I64, F, RP, SH, P, SZ, P]
        L.h3_kv_pack_fp8.restype = ctypes.c_int
        L.h3_attn_packed_fp8.argtypes = [P, P, P, I64, F, RP, F, F, SH, P, SZ, P]
        L.h3_attn_packed_fp8.restype = ctypes.c_int
        L.h3_attn_varlen_fp8.argtypes = [P, P, P, P, F, F, SH, P, SZ, P]
        L.h3_attn_varlen_fp8.restype = ctypes.c_int
        L.h3_attn_layer_fp8.argtypes = [P, P, P, P, P, P, I64, F, RP, F, F, SH, P, SZ, P]
        L.h3_attn_layer_fp8.restype = ctypes.c_int
        L.h3_residual_norm_modulate.argtypes = [P, P, P, P, P, I64, F, P,
                                                ctypes.POINTER(Rows), P]
        L.h3_residual_norm_modulate.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != H3_OK:
        msg = lib().h3_status_string(status).decode()
        raise H3Error(status, f"{what}: {msg}")


def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _row_stride(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a [B, S, H, D] or [S, H, D] bf16 device tensor whose heads
    and channels are packed and whose batches are S rows apart."""
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() == 3:
        t = t.unsqueeze(0)
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, S, H, D] or [S, H, D]")
    B, S, H, D = t.shape
    if t.stride(3) != 1 or t.stride(2) != D:
        raise ValueError(f"{name}: heads and channels must be packed")
    if B > 1 and t.stride(0) != S * t.stride(1):
        raise ValueError(f"{name}: batches must be S rows apart")
    return t.stride(1)


def _dims(t: torch.Tensor):
    return (1, *t.shape) if t.dim() == 3 else tuple(t.shape)


def _like(t: torch.Tensor, ref: torch.Tensor, name: str, ref_name: str = "q") -> int:
    """Row stride of ``t`` after checking that it is a bf16 tensor on ``ref``'s device with
    ``ref``'s [B, S, H, D] shape (so no kernel can read or write past its end)."""
    stride = _row_stride(t, name)
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, {ref_name} on {ref.device}")
    if _dims(t) != _dims(ref):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, {ref_name} {tuple(ref.shape)}")
    return stride


def _weight_stride(x: torch.Tensor, *ws) -> int:
    """w_head_stride for norm weights ``ws`` (all present, or all None -> 0): bf16 device
    tensors on ``x``'s device, each [D] (shared by the heads) or [H, D] with packed
    channels, all with the same shape and strides."""
    if all(w is None for w in ws):
        return 0
    if any(w is None for w in ws):
        raise ValueError("w_q and w_k must both be given")
    _, _, H, D = _dims(x)
    first = ws[0]
    for w in ws:
        if w.dtype != torch.bfloat16 or not _on_device(w) or w.device != x.device:
            raise ValueError(f"norm weights must be bf16 tensors on {x.device}")
        if w.shape != first.shape or w.stride() != first.stride():
            raise ValueError("w_q and w_k must have the same shape and strides")
    if first.dim() == 1:
        if first.shape != (D,) or first.stride(0) != 1:
            raise ValueError(f"shared norm weights must be a contiguous [{D}] tensor")
        return 0
    if first.dim() != 2 or first.shape != (H, D) or first.stride(1) != 1:
        raise ValueError(f"per-head norm weights must be [{H}, {D}] with packed channels")
    if first.stride(0) < D or first.stride(0) % 8:
        raise ValueError("per-head norm weights: head stride must be >= D and a multiple of 8")
    return first.stride(0)


class _Call:
    """Holds ctypes objects alive for the duration of a call."""

    def __init__(self, x: torch.Tensor, n_valid, in_stride: int, out_stride: int):
        B, S, H, D = _dims(x)
        if isinstance(n_valid, int):
            n_valid = [n_valid] * B
        if len(n_valid) != B:
            raise ValueError("n_valid must have one entry per batch")
        self.valid = (ctypes.c_int64 * B)(*[int(n) for n in n_valid])
        self.shape = Shape(B, H, D, S, ctypes.cast(self.valid, ctypes.POINTER(ctypes.c_int64)),
                           in_stride, out_stride)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def workspace_size(x: torch.Tensor, fp8: bool = False, n_valid=None) -> int:
    """Workspace bytes an attention call on a tensor shaped like ``x`` needs (``fp8``:
    the FP8 calls) for valid lengths ``n_valid`` (int or one per batch; default the
    buffer length S, which bounds the need of every N <= S)."""
    _, S, _, _ = _dims(x)
    c = _Call(x, S if n_valid is None else n_valid, x.shape[-2] * x.shape[-1],
              x.shape[-2] * x.shape[-1])
    f = lib().h3_attn_fp8_workspace_size if fp8 else lib().h3_attn_workspace_size
    return int(f(ctypes.byref(c.shape)))


def _workspace(q: torch.Tensor, call: _Call, workspace, fp8: bool = False):
    f = lib().h3_attn_fp8_workspace_size if fp8 else lib().h3_attn_workspace_size
    need = int(f(ctypes.byref(call.shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if not _on_device(workspace) or workspace.device != q.device or \
            not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous device tensor on {q.device}")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} "
                         f"bytes, {need} needed")
    return workspace


def qk_rmsnorm_rope(q, k, w_q, w_k, n_valid, eps: float, rope: Rope, q_out=None,
                    k_out=None, stream=None):
    """Fused per-head Q/K RMSNorm + RoPE (h3_qk_rmsnorm_rope).  Returns (q_out, k_out);
    pass ``q_out=q, k_out=k`` to work in place.  Output rows [N, S) are not written."""
    s_in = _row_stride(q, "q")
    if _like(k, q, "k") != s_in:
        raise ValueError("q and k must share a row stride")
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    s_out = _like(q_out, q, "q_out")
    if _like(k_out, q, "k_out") != s_out:
        raise ValueError("q_out and k_out must share a row stride")
    w_head_stride = _weight_stride(q, w_q, w_k)
    if w_q is None:
        raise ValueError("w_q and w_k are required")
    call = _Call(q, n_valid, s_in, s_out)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_qk_rmsnorm_rope(_p(q), _p(k), _p(q_out), _p(k_out), _p(w_q), _p(w_k),
                                    w_head_stride, float(eps), ctypes.byref(rope),
                                    ctypes.byref(call.shape), ctypes.c_void_p(st)),
           "h3_qk_rmsnorm_rope")
    return q_out, k_out


def attn_varlen(q, k, v, n_valid, softmax_scale: float, out=None, workspace=None,
                stream=None):
    """Attention over the valid tokens with pre-normalised, pre-rotated Q/K
    (h3_attn_varlen).  Output rows [N, S) are zero."""
    s_in, out, s_out = _qkv_strides(q, k, v, out)
    call = _Call(q, n_valid, s_in, s_out)
    ws = _workspace(q, call, workspace)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_varlen(_p(q), _p(k), _p(v), _p(out), float(softmax_scale),
                                ctypes.byref(call.shape), _p(ws), _nbytes(ws),
                                ctypes.c_void_p(st)), "h3_attn_varlen")
    return out


def attn_layer(q, k, v, w_q, w_k, n_valid, eps: float, rope: Rope, softmax_scale: float,
               out=None, workspace=None, stream=None):
    """The whole layer: Q/K RMSNorm + RoPE fused into attention (h3_attn_layer)."""
    s_in, out, s_out = _qkv_strides(q, k, v, out)
    if w_q is None or w_k is None:
        raise ValueError("w_q and w_k are required")
    w_head_stride = _weight_stride(q, w_q, w_k)
    call = _Call(q, n_valid, s_in, s_out)
    ws = _workspace(q, call, workspace)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_layer(_p(q), _p(k), _p(v), _p(out), _p(w_q), _p(w_k), w_head_stride,
                               float(eps), ctypes.byref(rope), float(softmax_scale),
                               ctypes.byref(call.shape), _p(ws), _nbytes(ws),
                               ctypes.c_void_p(st)), "h3_attn_layer")
    return out


def attn_varlen_skip(q, k, v, n_valid, softmax_scale: float, skip_threshold: float, out=None,
                     workspace=None, stream=None):
    """Dense attention with Skip-Softmax over pre-normalised, pre-rotated Q/K
    (h3_attn_varlen_skip); skip_threshold in (0, 1)."""
    s_in, out, s_out = _qkv_strides(q, k, v, out)
    call = _Call(q, n_valid, s_in, s_out)
    ws = _workspace(q, call, workspace)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_varlen_skip(_p(q), _p(k), _p(v), _p(out), float(softmax_scale),
                                     float(skip_threshold), ctypes.byref(call.shape), _p(ws),
                                     _nbytes(ws), ctypes.c_void_p(st)), "h3_attn_varlen_skip")
    return out


def attn_layer_skip(q, k, v, w_q, w_k, n_valid, eps: float, rope: Rope, softmax_scale: float,
                    skip_threshold: float, out=None, workspace=None, stream=None):
    """The whole layer with dense Skip-Softmax attention (h3_attn_layer_skip)."""
    s_in, out, s_out = _qkv_strides(q, k, v, out)
    if w_q is None or w_k is None:
        raise ValueError("w_q and w_k are required")
    w_head_stride = _weight_stride(q, w_q, w_k)
    call = _Call(q, n_valid, s_in, s_out)
    ws = _workspace(q, call, workspace)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_layer_skip(_p(q), _p(k), _p(v), _p(out), _p(w_q), _p(w_k),
                                    w_head_stride, float(eps), ctypes.byref(rope),
                                    float(softmax_scale), float(skip_threshold),
                                    ctypes.byref(call.shape), _p(ws), _nbytes(ws),
                                    ctypes.c_void_p(st)), "h3_attn_layer_skip")
    return out


def skip_counts(workspace, x: torch.Tensor) -> torch.Tensor:
    """Wave tiles (32 rows x 64 keys) each 256-row workgroup skipped in the last
    h3_attn_varlen_skip / h3_attn_layer_skip call with ``workspace`` for a tensor shaped
    like ``x``: [B, H, ceil(S / 256)] int32 (the pass-flag words of that call)."""
    B, S, H, D = _dims(x)
    img = B * H * ((S + 63) // 64) * 35840
    blocks = (S + 255) // 256
    per_batch = 8 * H * blocks
    words = workspace[img: img + 4 * B * per_batch].view(torch.int32).view(B, per_batch)
    return words[:, : H * blocks].reshape(B, H, blocks)


def attn_layer_noalloc(q, k, v, w_q, w_k, n_valid, eps: float, rope: Rope,
                       softmax_scale: float, out, stream=None):
    """h3_attn_layer with the library's static scratch as its workspace
    (h3_attn_layer_noalloc): the call allocates nothing; ``out`` must be given."""
    if out is None:
        raise ValueError("attn_layer_noalloc allocates nothing: pass out")
    s_in, out, s_out = _qkv_strides(q, k, v, out)
    if w_q is None or w_k is None:
        raise ValueError("w_q and w_k are required")
    w_head_stride = _weight_stride(q, w_q, w_k)
    call = _Call(q, n_valid, s_in, s_out)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_layer_noalloc(_p(q), _p(k), _p(v), _p(out), _p(w_q), _p(w_k),
                                       w_head_stride, float(eps), ctypes.byref(rope),
                                       float(softmax_scale), ctypes.byref(call.shape),
                                       ctypes.c_void_p(st)), "h3_attn_layer_noalloc")
    return out


def noalloc_max_workspace() -> int:
    """Bytes of the static scratch behind attn_layer_noalloc."""
    return int(lib().h3_attn_layer_noalloc_max_workspace())


def kv_pack(k, v, n_valid, workspace=None, w_k=None, eps: float = 0.0, rope: Rope | None = None,
            softmax_scale: float = 0.0, stream=None):
    """Stage 1 (h3_kv_pack): repack K (normalised + rotated, then multiplied by
    ``softmax_scale * log2(e)`` before rounding, when ``w_k`` is given) and V into a
    workspace for h3_attn_packed.  Returns the workspace."""
    s_in = _row_stride(k, "k")
    if _like(v, k, "v", "k") != s_in:
        raise ValueError("k and v must share a row stride")
    w_head_stride = _weight_stride(k, w_k)
    call = _Call(k, n_valid, s_in, s_in)
    ws = _workspace(k, call, workspace)
    st = _stream(k.device) if stream is None else stream
    _check(lib().h3_kv_pack(_p(k), _p(v), _p(w_k), w_head_stride, float(eps),
                            ctypes.byref(rope) if rope is not None else None,
                            float(softmax_scale), ctypes.byref(call.shape), _p(ws), _nbytes(ws),
                            ctypes.c_void_p(st)),
           "h3_kv_pack")
    return ws


def attn_packed(q, workspace, n_valid, softmax_scale: float, w_q=None, eps: float = 0.0,
                rope: Rope | None = None, out=None, stream=None):
    """Stage 2 (h3_attn_packed): attention of ``q`` (normalised + rotated in registers when
    ``w_q`` is given) against K/V packed by ``kv_pack``."""
    s_in = _row_stride(q, "q")
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    s_out = _like(out, q, "out")
    w_head_stride = _weight_stride(q, w_q)
    call = _Call(q, n_valid, s_in, s_out)
    _check_packed(q, call, workspace, fp8=False)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_packed(_p(q), _p(out), _p(w_q), w_head_stride, float(eps),
                                ctypes.byref(rope) if rope is not None else None,
                                float(softmax_scale), ctypes.byref(call.shape), _p(workspace),
                                _nbytes(workspace), ctypes.c_void_p(st)), "h3_attn_packed")
    return out


def _qkv_strides(q, k, v, out):
    """Row strides of q (shared by k and v) and out, after checking that k, v and out
    are bf16 tensors on q's device with q's shape; allocates out when it is None."""
    s_in = _row_stride(q, "q")
    for name, t in (("k", k), ("v", v)):
        if _like(t, q, name) != s_in:
            raise ValueError("q, k and v must share a row stride")
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    return s_in, out, _like(out, q, "out")


def _check_packed(q, call: _Call, workspace, fp8: bool):
    """A packed-stage workspace must be a device tensor on q's device."""
    if not isinstance(workspace, torch.Tensor) or not _on_device(workspace) or \
            workspace.device != q.device:
        raise ValueError(f"workspace must be a device tensor on {q.device}")


def attn_varlen_fp8(q, k, v, n_valid, softmax_scale: float, out=None, workspace=None,
                    stream=None, skip_threshold: float = 0.0):
    """FP8 (SAGE) attention over the valid tokens with pre-normalised, pre-rotated Q/K
    (h3_attn_varlen_fp8), with optional Skip-Softmax.  Output rows [N, S) are zero."""
    s_in, out, s_out = _qkv_strides(q, k, v, out)
    call = _Call(q, n_valid, s_in, s_out)
    ws = _workspace(q, call, workspace, fp8=True)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_varlen_fp8(_p(q), _p(k), _p(v), _p(out), float(softmax_scale),
                                    float(skip_threshold), ctypes.byref(call.shape), _p(ws),
                                    _nbytes(ws),
                                    ctypes.c_void_p(st)), "h3_attn_varlen_fp8")
    return out


def attn_layer_fp8(q, k, v, w_q, w_k, n_valid, eps: float, rope: Rope, softmax_scale: float,
                   out=None, workspace=None, stream=None, skip_threshold: float = 0.0):
    """The whole layer with FP8 attention: Q/K RMSNorm + RoPE fused (h3_attn_layer_fp8)."""
    s_in, out, s_out = _qkv_strides(q, k, v, out)
    if w_q is None or w_k is None:
        raise ValueError("w_q and w_k are required")
    w_head_stride = _weight_stride(q, w_q, w_k)
    call = _Call(q, n_valid, s_in, s_out)
    ws = _workspace(q, call, workspace, fp8=True)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_layer_fp8(_p(q), _p(k), _p(v), _p(out), _p(w_q), _p(w_k),
                                   w_head_stride, float(eps), ctypes.byref(rope),
                                   float(softmax_scale), float(skip_threshold),
                                   ctypes.byref(call.shape), _p(ws), _nbytes(ws),
                                   ctypes.c_void_p(st)), "h3_attn_layer_fp8")
    return out


def kv_pack_fp8(k, v, n_valid, workspace=None, w_k=None, eps: float = 0.0,
                rope: Rope | None = None, stream=None):
    """FP8 stage 1 (h3_kv_pack_fp8): quantize K (normalised + rotated when ``w_k`` is
    given) and V into FP8 tiles for h3_attn_packed_fp8.  Returns the workspace."""
    s_in = _row_stride(k, "k")
    if _like(v, k, "v", "k") != s_in:
        raise ValueError("k and v must share a row stride")
    w_head_stride = _weight_stride(k, w_k)
    call = _Call(k, n_valid, s_in, s_in)
    ws = _workspace(k, call, workspace, fp8=True)
    st = _stream(k.device) if stream is None else stream
    _check(lib().h3_kv_pack_fp8(_p(k), _p(v), _p(w_k), w_head_stride, float(eps),
                                ctypes.byref(rope) if rope is not None else None,
                                ctypes.byref(call.shape), _p(ws), _nbytes(ws),
                                ctypes.c_void_p(st)), "h3_kv_pack_fp8")
    return ws


def attn_packed_fp8(q, workspace, n_valid, softmax_scale: float, w_q=None, eps: float = 0.0,
                    rope: Rope | None = None, out=None, stream=None,
                    skip_threshold: float = 0.0):
    """FP8 stage 2 (h3_attn_packed_fp8): attention of ``q`` (normalised + rotated in
    registers when ``w_q`` is given) against FP8 tiles packed by ``kv_pack_fp8``."""
    s_in = _row_stride(q, "q")
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    s_out = _like(out, q, "out")
    w_head_stride = _weight_stride(q, w_q)
    call = _Call(q, n_valid, s_in, s_out)
    _check_packed(q, call, workspace, fp8=True)
    st = _stream(q.device) if stream is None else stream
    _check(lib().h3_attn_packed_fp8(_p(q), _p(out), _p(w_q), w_head_stride, float(eps),
                                    ctypes.byref(rope) if rope is not None else None,
                                    float(softmax_scale), float(skip_threshold),
                                    ctypes.byref(call.shape), _p(workspace), _nbytes(workspace),
                                    ctypes.c_void_p(st)), "h3_attn_packed_fp8")
    return out


def attn_splits(x: torch.Tensor, n_valid=None) -> list:
    """Key ranges per 256-row query block the bf16 attention calls use for each batch of
    a tensor shaped like ``x`` with valid lengths ``n_valid`` (default S)
    (h3_attn_splits)."""
    B, S, H, D = _dims(x)
    c = _Call(x, S if n_valid is None else n_valid, H * D, H * D)
    return [int(lib().h3_attn_splits(ctypes.byref(c.shape), b)) for b in range(B)]


def pass_flags(workspace, x: torch.Tensor, n_valid=None) -> torch.Tensor:
    """Which pass handled each workgroup in the last bf16 attention call with
    ``workspace`` for a tensor shaped like ``x`` with valid lengths ``n_valid`` (default
    S): [B, H, k, ceil(S / 256)] int32 for k key ranges per 256-row block (the same for
    every batch), 0 = the fast pass (scores provably bounded), 1 = the checked pass
    (layout documented with h3_attn_workspace_size)."""
    B, S, H, D = _dims(x)
    ks = attn_splits(x, n_valid)
    if len(set(ks)) != 1:
        raise ValueError(f"batches split their keys differently: {ks}")
    k = ks[0]
    img = B * H * ((S + 63) // 64) * 35840
    blocks = (S + 255) // 256
    per_batch = 8 * H * blocks  # flag words per batch (up to 8 key ranges)
    words = workspace[img: img + 4 * B * per_batch].view(torch.int32).view(B, per_batch)
    return words[:, : k * H * blocks].reshape(B, H, k, blocks)


def fp8_skip_counts(workspace, x: torch.Tensor) -> torch.Tensor:
    """Skip counts the last FP8 attention call left in ``workspace`` for a tensor shaped
    like ``x``: [B, H, ceil(S / 256)] int32, wave tiles (32 rows x 64 keys) skipped per
    256-row workgroup (layout documented with h3_attn_fp8_workspace_size)."""
    B, S, H, D = _dims(x)
    tiles = (S + 63) // 64
    img = B * H * tiles * 19456
    vamax = (B * H * D * 4 + 255) // 256 * 256
    blocks = (S + 255) // 256
    n = B * H * blocks
    return workspace[img + vamax: img + vamax + 4 * n].view(torch.int32).view(B, H, blocks)


def residual_norm_modulate(x, shift, scale, n_valid, eps: float = 1e-6, a=None, gate=None,
                           y=None, stream=None):
    """DiT block steps around attention (h3_residual_norm_modulate): with ``a``, the fp32
    residual stream ``x`` is updated in place to x + gate * a; then
    y = LayerNorm(x) * (1 + scale) + shift in bf16 is returned.  x: fp32 [B, S, C] or
    [S, C]; a: bf16 of the same shape or None; gate (or None), shift, scale: fp32 [C]
    (shared) or [B, C]."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 device tensor")
    xb = x if x.dim() == 3 else x.unsqueeze(0)
    B, S, C = xb.shape
    if a is not None and (a.dtype != torch.bfloat16 or a.shape != x.shape or
                          not a.is_contiguous()):
        raise ValueError("a must be a contiguous bf16 tensor shaped like x")
    vecs = [t for t in (gate, shift, scale) if t is not None]
    for t in vecs:
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape[-1] != C:
            raise ValueError("gate, shift and scale must be contiguous fp32 [..., C]")
    mod_stride = 0 if shift.dim() == 1 else C
    for t in vecs:
        if (0 if t.dim() == 1 else C) != mod_stride:
            raise ValueError("gate, shift and scale must all be [C] or all [B, C]")
    y = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device) if y is None else y
    if isinstance(n_valid, int):
        n_valid = [n_valid] * B
    valid = (ctypes.c_int64 * B)(*[int(n) for n in n_valid])
    rows = Rows(B, S, ctypes.cast(valid, ctypes.POINTER(ctypes.c_int64)), C)
    st = _stream(x.device) if stream is None else stream
    _check(lib().h3_residual_norm_modulate(_p(x), _p(a), _p(gate), _p(shift), _p(scale),
                                           mod_stride, float(eps), _p(y), ctypes.byref(rows),
                                           ctypes.c_void_p(st)), "h3_residual_norm_modulate")
    return y
