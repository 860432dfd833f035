"""Thin ctypes binding of libmoedecode.so (the C ABI in include/moe_decode.h).

Argument marshalling only: every step of the decode path runs in the library's
HIP kernels. Tensors are torch device tensors (torch provides device memory and
streams); each wrapper passes their data pointers and the current HIP stream. A
missing library raises at first use: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoedecode.so")
_lib = None

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EWORKSPACE, MOE_EUNSUPPORTED, MOE_ELAUNCH = 0, -1, -2, -3, -4, -5
MOE_ETIMEOUT = -6
MOE_W_FP8_E4M3, MOE_W_BF16 = 0, 1
MOE_KV_BF16, MOE_KV_FP8 = 0, 1
MOE_ROUTER_BF16, MOE_ROUTER_FP8, MOE_ROUTER_EXPERT_MAJOR = 0, 1, 2

# Every symbol include/moe_decode.h declares.
EXPORTS = ("moe_decode_layer_workspace", "moe_decode_layer", "moe_decode_layer_status", "lm_head_argmax_workspace",
           "lm_head_argmax", "lm_head_argmax_bf16", "lm_head_argmax_noalloc", "lm_head_spec_sample_workspace", "lm_head_spec_sample",
           "spec_accept", "moe_add_rmsnorm", "moe_decode_step_workspace",
           "moe_decode_step_prepare", "moe_decode_step", "moe_decode_step_status", "moe_fp8_decode",
           "moe_hbm_read_probe", "moe_draft_step_workspace", "moe_draft_step", "moe_draft_step_status", "moe_kv_cache_bytes",
           "moe_kv_cache_write", "moe_attn_decode_workspace", "moe_attn_decode", "moe_strerror")


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, strerror(status), status))
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("num_experts", ctypes.c_int), ("top_k", ctypes.c_int),
                ("expert_width", ctypes.c_int), ("shared_width", ctypes.c_int), ("wtype", ctypes.c_int),
                ("router_type", ctypes.c_int)]


_P = ctypes.c_void_p


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("router_w", "router_bias", "gate_w", "up_w", "down_w", "gate_s",
                                  "up_s", "down_s", "sh_gate_w", "sh_up_w", "sh_down_w",
                                  "sh_gate_s", "sh_up_s", "sh_down_s", "router_s")]


class StepDesc(ctypes.Structure):
    _fields_ = [("layer", LayerDesc), ("num_layers", ctypes.c_int), ("vocab", ctypes.c_int),
                ("max_tokens", ctypes.c_int), ("eps", ctypes.c_float), ("spin_limit", ctypes.c_uint),
                ("flags", ctypes.c_uint)]


MOE_STEP_COOPERATIVE = 1
MOE_STEP_LM_BF16 = 2


class DraftDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("width", ctypes.c_int), ("ffn", ctypes.c_int), ("blocks", ctypes.c_int),
                ("vocab", ctypes.c_int), ("eps", ctypes.c_float), ("flags", ctypes.c_uint),
                ("spin_limit", ctypes.c_uint)]


MOE_DRAFT_CHAIN = 1


class DraftWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("pre_w", "pre_s", "gate_w", "gate_s", "up_w", "up_s", "down_w", "down_s", "gains",
                                  "table_w", "table_s", "post_w", "post_s")]


class AttnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("hidden", "q_heads", "kv_heads", "head_dim", "window", "capacity",
                                            "kv_type")]


class AttnWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("q_w", "q_s", "k_w", "k_s", "o_w", "o_s")]


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmoedecode.so is not built (%s); run "
                               "python -m fine_grained_moe_router_amd.build" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        I, S = ctypes.c_int, ctypes.c_size_t
        L.moe_decode_layer_workspace.restype = S
        L.moe_decode_layer_workspace.argtypes = [ctypes.POINTER(LayerDesc), I]
        L.moe_decode_layer.restype = I
        L.moe_decode_layer.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), I,
                                       _P, _P, _P, _P, _P, S, _P]
        L.moe_decode_layer_status.restype = I
        L.moe_decode_layer_status.argtypes = [ctypes.POINTER(LayerDesc), _P]
        L.lm_head_argmax_workspace.restype = S
        L.lm_head_argmax_workspace.argtypes = [I, I, I]
        L.lm_head_argmax.restype = I
        L.lm_head_argmax.argtypes = [I, I, I, _P, _P, _P, _P, _P, _P, S, _P]
        L.lm_head_spec_sample_workspace.restype = S
        L.lm_head_spec_sample_workspace.argtypes = [I, I, I]
        L.lm_head_spec_sample.restype = I
        L.lm_head_spec_sample.argtypes = [I, I, I, _P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_uint64,
                                          ctypes.c_uint64, _P, _P, _P, S, _P]
        L.lm_head_argmax_bf16.restype = I
        L.lm_head_argmax_bf16.argtypes = [I, I, I, _P, _P, _P, _P, _P, S, _P]
        L.lm_head_argmax_noalloc.restype = I
        L.lm_head_argmax_noalloc.argtypes = [I, I, I, _P, _P, _P, _P, _P, _P]
        L.spec_accept.restype = I
        L.spec_accept.argtypes = [I, _P, _P, _P, _P, _P]
        L.moe_add_rmsnorm.restype = I
        L.moe_add_rmsnorm.argtypes = [I, I, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
        L.moe_fp8_decode.restype = I
        L.moe_fp8_decode.argtypes = [I, _P, _P, _P, _P]
        L.moe_hbm_read_probe.restype = I
        L.moe_hbm_read_probe.argtypes = [_P, S, _P, _P]
        L.moe_decode_step_workspace.restype = S
        L.moe_decode_step_workspace.argtypes = [ctypes.POINTER(StepDesc)]
        L.moe_decode_step_prepare.restype = I
        L.moe_decode_step_prepare.argtypes = [ctypes.POINTER(StepDesc), ctypes.POINTER(LayerWeights), _P, S]
        L.moe_decode_step.restype = I
        L.moe_decode_step.argtypes = [ctypes.POINTER(StepDesc), I] + [_P] * 14 + [_P, S, _P]
        L.moe_decode_step_status.restype = I
        L.moe_decode_step_status.argtypes = [ctypes.POINTER(StepDesc), _P]
        L.moe_draft_step_workspace.restype = S
        L.moe_draft_step_workspace.argtypes = [ctypes.POINTER(DraftDesc)]
        L.moe_draft_step.restype = I
        L.moe_draft_step_status.restype = I
        L.moe_draft_step_status.argtypes = [ctypes.POINTER(DraftDesc), _P]
        L.moe_draft_step.argtypes = [ctypes.POINTER(DraftDesc), ctypes.POINTER(DraftWeights), I, _P, _P, _P, _P, _P,
                                     _P, S, _P]
        L.moe_kv_cache_bytes.restype = S
        L.moe_kv_cache_bytes.argtypes = [ctypes.POINTER(AttnDesc)]
        L.moe_kv_cache_write.restype = I
        L.moe_kv_cache_write.argtypes = [ctypes.POINTER(AttnDesc), I, I, _P, _P, _P]
        L.moe_attn_decode_workspace.restype = S
        L.moe_attn_decode_workspace.argtypes = [ctypes.POINTER(AttnDesc), I]
        L.moe_attn_decode.restype = I
        L.moe_attn_decode.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnWeights), I, I, _P, _P, _P, _P,
                                      _P, S, _P]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [I]
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


def layer_desc(shape, expert_dtype: str = "fp8", router_dtype: str = "bf16", expert_major: bool = False) -> LayerDesc:
    """expert_major: the router weights are passed [E][H] (MOE_ROUTER_EXPERT_MAJOR)."""
    rt = MOE_ROUTER_FP8 if router_dtype == "fp8" else MOE_ROUTER_BF16
    return LayerDesc(shape.hidden, shape.experts, shape.top_k, shape.width, shape.shared_width,
                     MOE_W_FP8_E4M3 if expert_dtype == "fp8" else MOE_W_BF16,
                     rt | (MOE_ROUTER_EXPERT_MAJOR if expert_major else 0))


def layer_weights(w: dict) -> LayerWeights:
    """LayerWeights from a dict of device tensors (keys as synth.layer_weights)."""
    keys = ("router_w", "router_b", "gate_w", "up_w", "down_w", "gate_s", "up_s", "down_s",
            "sh_gate_w", "sh_up_w", "sh_down_w", "sh_gate_s", "sh_up_s", "sh_down_s", "router_s")
    return LayerWeights(*[_ptr(w.get(k)) for k in keys])


def moe_decode_layer_workspace(desc: LayerDesc, max_M: int) -> int:
    return lib().moe_decode_layer_workspace(ctypes.byref(desc), int(max_M))


def moe_decode_layer(desc: LayerDesc, weights: LayerWeights, M: int, x, y, topk_idx, topk_w,
                     workspace, workspace_bytes: int, stream=None):
    st = lib().moe_decode_layer(ctypes.byref(desc), ctypes.byref(weights), int(M), _ptr(x), _ptr(y),
                                _ptr(topk_idx), _ptr(topk_w), _ptr(workspace), int(workspace_bytes),
                                _stream(stream))
    _check("moe_decode_layer", st)


def moe_decode_layer_status(desc: LayerDesc, workspace) -> int:
    """MOE_OK or MOE_ETIMEOUT (synchronous; clears the flag)."""
    return lib().moe_decode_layer_status(ctypes.byref(desc), _ptr(workspace))


def lm_head_argmax_workspace(max_M: int, H: int, V: int) -> int:
    return lib().lm_head_argmax_workspace(int(max_M), int(H), int(V))


def lm_head_argmax(M, H, V, x, w, w_s, token, max_logit, workspace, workspace_bytes, stream=None):
    st = lib().lm_head_argmax(int(M), int(H), int(V), _ptr(x), _ptr(w), _ptr(w_s), _ptr(token),
                              _ptr(max_logit), _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("lm_head_argmax", st)


def lm_head_spec_sample_workspace(max_M: int, H: int, V: int) -> int:
    return lib().lm_head_spec_sample_workspace(int(max_M), int(H), int(V))


def lm_head_spec_sample(M, H, V, x, w, w_s, temperature, draft, q, u_accept, seed, step, accepted_len, out_tokens,
                        workspace, workspace_bytes, stream=None):
    st = lib().lm_head_spec_sample(int(M), int(H), int(V), _ptr(x), _ptr(w), _ptr(w_s), float(temperature),
                                   _ptr(draft), _ptr(q), _ptr(u_accept), int(seed), int(step), _ptr(accepted_len),
                                   _ptr(out_tokens), _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("lm_head_spec_sample", st)


def lm_head_argmax_bf16(M, H, V, x, w, token, max_logit, workspace, workspace_bytes, stream=None):
    st = lib().lm_head_argmax_bf16(int(M), int(H), int(V), _ptr(x), _ptr(w), _ptr(token), _ptr(max_logit),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("lm_head_argmax_bf16", st)


def lm_head_argmax_noalloc(M, H, V, x, w, w_s, token, max_logit, stream=None):
    st = lib().lm_head_argmax_noalloc(int(M), int(H), int(V), _ptr(x), _ptr(w), _ptr(w_s), _ptr(token),
                                      _ptr(max_logit), _stream(stream))
    _check("lm_head_argmax_noalloc", st)


def spec_accept(num_draft, draft, target, accepted_len, out_tokens, stream=None):
    st = lib().spec_accept(int(num_draft), _ptr(draft), _ptr(target), _ptr(accepted_len),
                           _ptr(out_tokens), _stream(stream))
    _check("spec_accept", st)


def moe_add_rmsnorm(M, H, h_in, add0, add1, gain, eps, h_out, u_out, stream=None):
    st = lib().moe_add_rmsnorm(int(M), int(H), _ptr(h_in), _ptr(add0), _ptr(add1), _ptr(gain),
                               float(eps), _ptr(h_out), _ptr(u_out), _stream(stream))
    _check("moe_add_rmsnorm", st)


def moe_fp8_decode(n, codes, out_via_bf16, out_via_f32, stream=None):
    st = lib().moe_fp8_decode(int(n), _ptr(codes), _ptr(out_via_bf16), _ptr(out_via_f32),
                              _stream(stream))
    _check("moe_fp8_decode", st)


PROBE_GRID = 8192   # MOE_PROBE_GRID: words of the read probe's sink


def moe_hbm_read_probe(src, nbytes, sink, stream=None):
    st = lib().moe_hbm_read_probe(_ptr(src), int(nbytes), _ptr(sink), _stream(stream))
    _check("moe_hbm_read_probe", st)


def step_desc(shape, max_tokens: int, eps: float = 1e-6, spin_limit: int = 0,
              expert_dtype: str = "fp8", cooperative: bool = False, lm_bf16: bool = False,
              router_dtype: str = "bf16") -> StepDesc:
    return StepDesc(layer_desc(shape, expert_dtype, router_dtype), shape.layers, shape.vocab, max_tokens, eps,
                    spin_limit,
                    (MOE_STEP_COOPERATIVE if cooperative else 0) | (MOE_STEP_LM_BF16 if lm_bf16 else 0))


def moe_decode_step_workspace(desc: StepDesc) -> int:
    return lib().moe_decode_step_workspace(ctypes.byref(desc))


def moe_decode_step_prepare(desc: StepDesc, layers, workspace, workspace_bytes: int):
    """layers: a sequence of LayerWeights (host structs holding device pointers)."""
    arr = (LayerWeights * len(layers))(*layers)
    st = lib().moe_decode_step_prepare(ctypes.byref(desc), arr, _ptr(workspace), int(workspace_bytes))
    _check("moe_decode_step_prepare", st)


def moe_decode_step(desc: StepDesc, M, gains, lm_w, lm_s, x, noise, draft, token, max_logit,
                    accepted_len, out_tokens, y_layers, topk_idx, topk_w, x_final, workspace,
                    workspace_bytes, stream=None):
    st = lib().moe_decode_step(ctypes.byref(desc), int(M), _ptr(gains), _ptr(lm_w), _ptr(lm_s), _ptr(x),
                               _ptr(noise), _ptr(draft), _ptr(token), _ptr(max_logit), _ptr(accepted_len),
                               _ptr(out_tokens), _ptr(y_layers), _ptr(topk_idx), _ptr(topk_w),
                               _ptr(x_final), _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("moe_decode_step", st)


def moe_decode_step_status(desc: StepDesc, workspace) -> int:
    """MOE_OK or MOE_ETIMEOUT (synchronous; clears the flag)."""
    return lib().moe_decode_step_status(ctypes.byref(desc), _ptr(workspace))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zeroed device buffer of nbytes (torch allocations are 256-byte aligned)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def draft_desc(shape, eps: float = 1e-6, chain: bool = False, spin_limit: int = 0) -> DraftDesc:
    """chain: always run the chain of launches (MOE_DRAFT_CHAIN) instead of the one-launch form."""
    return DraftDesc(shape.hidden, shape.width, shape.ffn, shape.blocks, shape.vocab, eps,
                     MOE_DRAFT_CHAIN if chain else 0, int(spin_limit))


def draft_weights(w: dict) -> DraftWeights:
    """DraftWeights from a dict of device tensors (keys as synth.draft_head)."""
    return DraftWeights(*[_ptr(w[k]) for k in ("pre_w", "pre_s", "gate_w", "gate_s", "up_w", "up_s", "down_w",
                                                "down_s", "gains", "table_w", "table_s", "post_w", "post_s")])


def moe_draft_step_workspace(desc: DraftDesc) -> int:
    return lib().moe_draft_step_workspace(ctypes.byref(desc))


def moe_draft_step(desc: DraftDesc, weights: DraftWeights, gamma, tok0, hidden0, emb_w, emb_s, drafts, workspace,
                   workspace_bytes, stream=None):
    st = lib().moe_draft_step(ctypes.byref(desc), ctypes.byref(weights), int(gamma), _ptr(tok0), _ptr(hidden0),
                              _ptr(emb_w), _ptr(emb_s), _ptr(drafts), _ptr(workspace), int(workspace_bytes),
                              _stream(stream))
    _check("moe_draft_step", st)


def moe_draft_step_status(desc: DraftDesc, workspace) -> int:
    return lib().moe_draft_step_status(ctypes.byref(desc), _ptr(workspace))


def attn_desc(shape) -> AttnDesc:
    """AttnDesc from a synth.AttnShape."""
    return AttnDesc(shape.hidden, shape.q_heads, shape.kv_heads, shape.head_dim, shape.window, shape.capacity,
                    MOE_KV_FP8 if shape.kv_fp8 else MOE_KV_BF16)


def attn_weights(w: dict) -> AttnWeights:
    """AttnWeights from a dict of device tensors (keys as synth.attn_weights)."""
    return AttnWeights(*[_ptr(w[k]) for k in ("q_w", "q_s", "k_w", "k_s", "o_w", "o_s")])


def moe_kv_cache_bytes(desc: AttnDesc) -> int:
    return lib().moe_kv_cache_bytes(ctypes.byref(desc))


def moe_kv_cache_write(desc: AttnDesc, first_pos, n, k, cache, stream=None):
    st = lib().moe_kv_cache_write(ctypes.byref(desc), int(first_pos), int(n), _ptr(k), _ptr(cache), _stream(stream))
    _check("moe_kv_cache_write", st)


def moe_attn_decode_workspace(desc: AttnDesc, max_M: int) -> int:
    return lib().moe_attn_decode_workspace(ctypes.byref(desc), int(max_M))


def moe_attn_decode(desc: AttnDesc, weights: AttnWeights, M, pos, u, cache, out, o, workspace, workspace_bytes,
                    stream=None):
    st = lib().moe_attn_decode(ctypes.byref(desc), ctypes.byref(weights), int(M), int(pos), _ptr(u), _ptr(cache),
                               _ptr(out), _ptr(o), _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("moe_attn_decode", st)
