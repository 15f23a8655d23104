"""The binding rejects mismatched tensors before any library call.

Every attention call checks that k, v and out are bf16 tensors on q's device with q's
[B, S, H, D] shape, and that the norm weights are bf16 [D] or [H, D] tensors with the
same shape and strides for Q and K; otherwise a kernel could read or write past the end
of a shorter buffer, or apply w_q's head stride to a w_k of another layout.  Runs on the
CPU: the device check is replaced by one that accepts host tensors, and the library
loader by one that fails the test if it is reached.
"""
import pytest
import torch

from long_sequence_attention_h3_amd import binding as B


@pytest.fixture(autouse=True)
def host_tensors(monkeypatch):
    monkeypatch.setattr(B, "_on_device", lambda t: True)

    def no_lib():
        raise AssertionError("the library was called with invalid arguments")
    monkeypatch.setattr(B, "lib", no_lib)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


S, H, D = 128, 2, 128
ROPE = B.make_rope(1e4, S)


def good():
    return dict(q=t(1, S, H, D), k=t(1, S, H, D), v=t(1, S, H, D), w_q=t(D), w_k=t(D))


CALLS = {
    "attn_layer": lambda a: B.attn_layer(a["q"], a["k"], a["v"], a["w_q"], a["w_k"], S, 1e-6,
                                         ROPE, 0.088, out=a.get("out")),
    "attn_layer_fp8": lambda a: B.attn_layer_fp8(a["q"], a["k"], a["v"], a["w_q"], a["w_k"], S,
                                                 1e-6, ROPE, 0.088, out=a.get("out")),
    "attn_varlen": lambda a: B.attn_varlen(a["q"], a["k"], a["v"], S, 0.088, out=a.get("out")),
    "attn_varlen_fp8": lambda a: B.attn_varlen_fp8(a["q"], a["k"], a["v"], S, 0.088,
                                                   out=a.get("out")),
}
BAD = {
    "short k": dict(k=t(1, S - 64, H, D)),
    "short v": dict(v=t(1, S - 64, H, D)),
    "fewer heads in v": dict(v=t(1, S, 1, D)),
    "short out": dict(out=t(1, S // 2, H, D)),
    "fp16 v": dict(v=t(1, S, H, D, dtype=torch.float16)),
}


@pytest.mark.parametrize("call", sorted(CALLS))
@pytest.mark.parametrize("bad", sorted(BAD))
def test_mismatched_tensors_are_rejected(call, bad):
    a = dict(good(), **BAD[bad])
    with pytest.raises((ValueError, TypeError)):
        CALLS[call](a)


WEIGHTS_BAD = {
    "w_q per head, w_k shared": dict(w_q=t(H, D), w_k=t(D)),
    "w_q shared, w_k per head": dict(w_q=t(D), w_k=t(H, D)),
    "too few channels": dict(w_q=t(64), w_k=t(64)),
    "too few heads": dict(w_q=t(1, D), w_k=t(1, D)),
    "fp32 weights": dict(w_q=t(D, dtype=torch.float32), w_k=t(D, dtype=torch.float32)),
    "strided channels": dict(w_q=t(D, 2)[:, 0], w_k=t(D, 2)[:, 0]),
    "missing w_k": dict(w_k=None),
}


@pytest.mark.parametrize("call", ["attn_layer", "attn_layer_fp8"])
@pytest.mark.parametrize("bad", sorted(WEIGHTS_BAD))
def test_bad_norm_weights_are_rejected(call, bad):
    a = dict(good(), **WEIGHTS_BAD[bad])
    with pytest.raises((ValueError, TypeError)):
        CALLS[call](a)


def test_bad_weights_rejected_by_prologue_and_pack():
    a = good()
    with pytest.raises(ValueError):
        B.qk_rmsnorm_rope(a["q"], a["k"], t(H, D), t(D), S, 1e-6, ROPE)
    with pytest.raises(ValueError):
        B.qk_rmsnorm_rope(a["q"], t(1, S - 1, H, D), a["w_q"], a["w_k"], S, 1e-6, ROPE)
    with pytest.raises(ValueError):
        B.kv_pack(a["k"], t(1, S, H, D - 64), S)
    with pytest.raises(ValueError):
        B.kv_pack(a["k"], a["v"], S, w_k=t(3, D), eps=1e-6, rope=ROPE, softmax_scale=0.088)
    with pytest.raises(ValueError):
        B.kv_pack_fp8(a["k"], a["v"], S, w_k=t(D + 8), eps=1e-6, rope=ROPE)
    with pytest.raises(ValueError):
        B.attn_packed(a["q"], t(16, dtype=torch.uint8), S, 0.088, w_q=t(H + 1, D), eps=1e-6,
                      rope=ROPE)


def test_valid_arguments_reach_the_library(monkeypatch):
    """The same calls with consistent tensors pass validation (they stop at the library,
    which the fixture replaced)."""
    a = good()
    for name in ("attn_layer", "attn_varlen", "attn_layer_fp8", "attn_varlen_fp8"):
        with pytest.raises(AssertionError, match="library was called"):
            CALLS[name](a)
    per_head = dict(a, w_q=t(H, D), w_k=t(H, D))
    with pytest.raises(AssertionError, match="library was called"):
        CALLS["attn_layer"](per_head)
