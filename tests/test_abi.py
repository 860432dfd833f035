"""The C-ABI library loads and exports every symbol include/*.h declares, and the
host-side validation rejects bad arguments before anything is enqueued (no GPU:
every call here fails validation, so no HIP call is made)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from fine_grained_moe_router_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, re.M):
            if m.group(1) not in ("if", "sizeof"):
                names.add(m.group(1))
    return names


def test_header_declares_the_binding_exports():
    assert declared_functions() == set(native.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = native.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", native._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    dyn = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert declared_functions() <= dyn


def test_strerror():
    for st in (0, -1, -2, -3, -4, -5):
        assert native.strerror(st) and native.strerror(st) != "unknown status"
    assert native.strerror(42) == "unknown status"


GEMMA = native.LayerDesc(2816, 128, 8, 704, 704, native.MOE_W_FP8_E4M3)
FAKE = 1 << 20          # a 16-byte-aligned non-null address (never dereferenced)


def fake_weights(**over):
    w = {k: FAKE for k, _ in native.LayerWeights._fields_}
    w["router_bias"] = None
    w.update(over)
    return native.LayerWeights(*[w[k] for k, _ in native.LayerWeights._fields_])


def call_layer(desc=GEMMA, weights=None, M=1, x=FAKE, y=FAKE, idx=None, wts=None, ws=FAKE,
               ws_bytes=None):
    L = native.lib()
    if weights is None:
        weights = fake_weights()
    if ws_bytes is None:
        ws_bytes = L.moe_decode_layer_workspace(ctypes.byref(desc), max(1, min(M, 8))) or 1 << 30
    return L.moe_decode_layer(ctypes.byref(desc), ctypes.byref(weights), M, x, y, idx, wts, ws,
                              ws_bytes, None)


def test_workspace_sizes():
    L = native.lib()
    w1 = L.moe_decode_layer_workspace(ctypes.byref(GEMMA), 1)
    w8 = L.moe_decode_layer_workspace(ctypes.byref(GEMMA), 8)
    assert 0 < w1 < w8 and w1 % 256 == 0 and w8 % 256 == 0
    assert L.moe_decode_layer_workspace(ctypes.byref(GEMMA), 0) == 0
    assert L.moe_decode_layer_workspace(ctypes.byref(GEMMA), 9) == 0
    assert L.moe_decode_layer_workspace(None, 1) == 0
    assert L.lm_head_argmax_workspace(5, 2816, 262144) > 0
    assert L.lm_head_argmax_workspace(5, 2817, 262144) == 0
    assert L.lm_head_argmax_workspace(5, 2816, 100) == 0


@pytest.mark.parametrize("field,value", [
    ("hidden", 0), ("hidden", 2800), ("hidden", 8192), ("num_experts", 0), ("num_experts", 257),
    ("top_k", 0), ("top_k", 17), ("expert_width", 700), ("expert_width", 0),
    ("shared_width", -64), ("shared_width", 100), ("wtype", 7)])
def test_layer_desc_validation(field, value):
    d = native.LayerDesc(*[getattr(GEMMA, f) for f, _ in native.LayerDesc._fields_])
    setattr(d, field, value)
    assert call_layer(desc=d, ws_bytes=1 << 30) == native.MOE_EINVAL


def test_top_k_above_experts_rejected():
    d = native.LayerDesc(256, 4, 5, 64, 64, 0)
    assert call_layer(desc=d, ws_bytes=1 << 30) == native.MOE_EINVAL


@pytest.mark.parametrize("M", [0, -1, 9, 100])
def test_token_count_validation(M):
    assert call_layer(M=M, ws_bytes=1 << 30) == native.MOE_EINVAL


def test_layer_pointer_validation():
    assert call_layer(x=None) == native.MOE_EINVAL
    assert call_layer(y=None) == native.MOE_EINVAL
    assert call_layer(x=FAKE + 8) == native.MOE_EALIGN
    assert call_layer(idx=FAKE + 2) == native.MOE_EALIGN
    assert call_layer(wts=FAKE + 1) == native.MOE_EALIGN
    assert call_layer(weights=fake_weights(gate_w=None)) == native.MOE_EINVAL
    assert call_layer(weights=fake_weights(down_s=FAKE + 2)) == native.MOE_EALIGN
    assert call_layer(weights=fake_weights(router_bias=FAKE + 4)) == native.MOE_EALIGN
    assert call_layer(weights=fake_weights(sh_up_w=None)) == native.MOE_EINVAL
    L = native.lib()
    assert L.moe_decode_layer(ctypes.byref(GEMMA), None, 1, FAKE, FAKE, None, None, FAKE,
                              1 << 30, None) == native.MOE_EINVAL


def test_layer_status_validation():
    L = native.lib()
    assert L.moe_decode_layer_status(None, FAKE) == native.MOE_EINVAL
    assert L.moe_decode_layer_status(ctypes.byref(GEMMA), None) == native.MOE_EWORKSPACE
    assert L.moe_decode_layer_status(ctypes.byref(GEMMA), FAKE + 16) == native.MOE_EWORKSPACE


def test_layer_workspace_validation():
    need = native.lib().moe_decode_layer_workspace(ctypes.byref(GEMMA), 5)
    assert call_layer(M=5, ws_bytes=need - 1) == native.MOE_EWORKSPACE
    assert call_layer(M=5, ws=None) == native.MOE_EWORKSPACE
    assert call_layer(M=5, ws=FAKE + 16) == native.MOE_EWORKSPACE     # not 256-byte aligned


def test_bf16_experts_pass_validation_without_scales():
    d = native.LayerDesc(2816, 128, 8, 704, 704, native.MOE_W_BF16)
    need = native.lib().moe_decode_layer_workspace(ctypes.byref(d), 1)
    assert need > 0
    # bf16 weights need no scales: with NULL scales the call gets past the weight checks
    # and stops at the (deliberately short) workspace, before anything is launched
    w = fake_weights(gate_s=None, up_s=None, down_s=None, sh_gate_s=None, sh_up_s=None, sh_down_s=None)
    assert call_layer(desc=d, weights=w, ws_bytes=need - 1) == native.MOE_EWORKSPACE
    # while FP8 weights without scales are rejected
    d8 = native.LayerDesc(2816, 128, 8, 704, 704, native.MOE_W_FP8_E4M3)
    assert call_layer(desc=d8, weights=w, ws_bytes=need) == native.MOE_EINVAL


def test_lm_head_validation():
    L = native.lib()
    ws = L.lm_head_argmax_workspace(5, 2816, 262144)
    f = lambda **k: L.lm_head_argmax(k.get("M", 5), k.get("H", 2816), k.get("V", 262144),
                                     k.get("x", FAKE), k.get("w", FAKE), k.get("s", FAKE),
                                     k.get("tok", FAKE), k.get("ml", None), k.get("ws", FAKE),
                                     k.get("wsb", ws), None)
    assert f(M=0) == native.MOE_EINVAL and f(M=9) == native.MOE_EINVAL
    assert f(H=100) == native.MOE_EINVAL and f(V=65) == native.MOE_EINVAL
    assert f(x=None) == native.MOE_EINVAL and f(tok=None) == native.MOE_EINVAL
    assert f(w=FAKE + 1) == native.MOE_EALIGN and f(ml=FAKE + 4) == native.MOE_EALIGN
    assert f(wsb=ws - 1) == native.MOE_EWORKSPACE and f(ws=None) == native.MOE_EWORKSPACE


def test_lm_head_bf16_validation():
    L = native.lib()
    ws = native.lm_head_argmax_workspace(5, 2816, 4096)
    assert L.lm_head_argmax_bf16(0, 2816, 4096, FAKE, FAKE, FAKE, None, FAKE, ws, None) == native.MOE_EINVAL
    assert L.lm_head_argmax_bf16(5, 2816, 4096, FAKE, None, FAKE, None, FAKE, ws, None) == native.MOE_EINVAL
    assert L.lm_head_argmax_bf16(5, 2816, 4096, FAKE, FAKE + 8, FAKE, None, FAKE, ws, None) == native.MOE_EALIGN
    assert L.lm_head_argmax_bf16(5, 2816, 4096, FAKE, FAKE, FAKE, None, FAKE, ws - 1, None) == native.MOE_EWORKSPACE


def test_lm_head_noalloc_validation():
    L = native.lib()
    assert L.lm_head_argmax_noalloc(0, 2816, 262144, FAKE, FAKE, FAKE, FAKE, None, None) == native.MOE_EINVAL
    assert L.lm_head_argmax_noalloc(9, 2816, 262144, FAKE, FAKE, FAKE, FAKE, None, None) == native.MOE_EINVAL
    assert L.lm_head_argmax_noalloc(1, 2816, 100, FAKE, FAKE, FAKE, FAKE, None, None) == native.MOE_EINVAL
    assert L.lm_head_argmax_noalloc(1, 2816, 4096, None, FAKE, FAKE, FAKE, None, None) == native.MOE_EINVAL
    assert L.lm_head_argmax_noalloc(1, 2816, 4096, FAKE + 2, FAKE, FAKE, FAKE, None, None) == native.MOE_EALIGN
    assert L.lm_head_argmax_noalloc(1, 2816, 4096, FAKE, FAKE, FAKE, FAKE, FAKE + 4, None) == native.MOE_EALIGN


def test_spec_sample_validation():
    L = native.lib()
    assert native.lm_head_spec_sample_workspace(5, 2816, 262144) > 0
    assert native.lm_head_spec_sample_workspace(5, 2816, (1 << 24) + 64) == 0
    assert native.lm_head_spec_sample_workspace(9, 2816, 4096) == 0
    ws = native.lm_head_spec_sample_workspace(5, 2816, 4096)
    args = lambda **o: [o.get(k, v) for k, v in (
        ("M", 5), ("H", 2816), ("V", 4096), ("x", FAKE), ("w", FAKE), ("s", FAKE), ("T", 0.7), ("d", FAKE),
        ("q", FAKE), ("u", FAKE), ("seed", 1), ("step", 2), ("n", FAKE), ("out", FAKE), ("ws", FAKE),
        ("wsb", ws), ("stream", None))]
    assert L.lm_head_spec_sample(*args(T=0.0)) == native.MOE_EINVAL
    assert L.lm_head_spec_sample(*args(T=-1.0)) == native.MOE_EINVAL
    assert L.lm_head_spec_sample(*args(M=0)) == native.MOE_EINVAL
    assert L.lm_head_spec_sample(*args(d=None)) == native.MOE_EINVAL
    assert L.lm_head_spec_sample(*args(q=None)) == native.MOE_EINVAL
    assert L.lm_head_spec_sample(*args(q=FAKE + 4)) == native.MOE_EALIGN
    assert L.lm_head_spec_sample(*args(out=FAKE + 2)) == native.MOE_EALIGN
    assert L.lm_head_spec_sample(*args(wsb=ws - 1)) == native.MOE_EWORKSPACE


def test_draft_step_validation():
    import synth
    L = native.lib()
    good = native.draft_desc(synth.MTP_HEAD)
    wsb = native.moe_draft_step_workspace(good)
    assert wsb > 0
    for k, v in (("hidden", 100), ("width", 128), ("ffn", 0), ("blocks", 65), ("vocab", 100), ("eps", -1.0),
                 ("width", 2304), ("width", 4352), ("ffn", 4352), ("ffn", 8704), ("ffn", 17408)):
        d = native.draft_desc(synth.MTP_HEAD)
        setattr(d, k, v)
        assert native.moe_draft_step_workspace(d) == 0, (k, v)
    # the largest splits: 32 lanes per gate/up row at width 4096, 64 lanes per down row
    for k, v in (("width", 2048), ("width", 2560), ("width", 4096), ("ffn", 4096), ("ffn", 4608), ("ffn", 8192),
                 ("ffn", 9216), ("ffn", 16384), ("hidden", 4096), ("hidden", 256)):
        d = native.draft_desc(synth.MTP_HEAD)
        setattr(d, k, v)
        assert native.moe_draft_step_workspace(d) > 0, (k, v)
    w = native.DraftWeights(*([FAKE] * 13))
    args = lambda **o: [o.get(k, v) for k, v in (
        ("d", ctypes.byref(good)), ("w", ctypes.byref(w)), ("g", 4), ("t", FAKE), ("h", FAKE), ("e", FAKE),
        ("s", FAKE), ("out", FAKE), ("ws", FAKE), ("wsb", wsb), ("st", None))]
    assert L.moe_draft_step(*args(g=0)) == native.MOE_EINVAL
    assert L.moe_draft_step(*args(g=8)) == native.MOE_EINVAL
    assert L.moe_draft_step(*args(t=None)) == native.MOE_EINVAL
    assert L.moe_draft_step(*args(h=FAKE + 2)) == native.MOE_EALIGN
    assert L.moe_draft_step(*args(out=FAKE + 2)) == native.MOE_EALIGN
    assert L.moe_draft_step(*args(wsb=wsb - 1)) == native.MOE_EWORKSPACE
    wbad = native.DraftWeights(*([FAKE] * 12 + [None]))
    assert L.moe_draft_step(*args(w=ctypes.byref(wbad))) == native.MOE_EINVAL


def test_draft_step_flags_and_status_validation():
    """MOE_DRAFT_CHAIN is the only flag; the workspace does not depend on it (a workspace
    serves both forms); the status call validates its arguments like the step's."""
    import synth
    L = native.lib()
    fused = native.draft_desc(synth.MTP_HEAD)
    chain = native.draft_desc(synth.MTP_HEAD, chain=True)
    assert chain.flags == native.MOE_DRAFT_CHAIN
    assert native.moe_draft_step_workspace(chain) == native.moe_draft_step_workspace(fused) > 0
    for bad in (2, 4, 0x80000000, 3):
        d = native.draft_desc(synth.MTP_HEAD)
        d.flags = bad
        assert native.moe_draft_step_workspace(d) == 0, bad
    # a spin limit is any value (0: the default)
    d = native.draft_desc(synth.MTP_HEAD, spin_limit=1)
    assert native.moe_draft_step_workspace(d) == native.moe_draft_step_workspace(fused)
    # the one-launch form's words and counter make the workspace larger than the chain alone
    # needs: a head the one-launch form does not take (width 2048) has none of them
    wide = native.draft_desc(synth.MTP_HEAD.__class__(hidden=2816, width=2048, ffn=4096, blocks=12, vocab=262144))
    assert 0 < native.moe_draft_step_workspace(wide)
    assert L.moe_draft_step_status(None, FAKE) == native.MOE_EINVAL
    assert native.moe_draft_step_status(fused, None) == native.MOE_EWORKSPACE
    assert native.moe_draft_step_status(fused, FAKE + 16) == native.MOE_EWORKSPACE
    d = native.draft_desc(synth.MTP_HEAD)
    d.flags = 2
    assert native.moe_draft_step_status(d, FAKE) == native.MOE_EINVAL


def test_spec_accept_validation():
    L = native.lib()
    assert L.spec_accept(-1, FAKE, FAKE, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.spec_accept(8, FAKE, FAKE, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.spec_accept(2, None, FAKE, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.spec_accept(2, FAKE, None, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.spec_accept(2, FAKE + 2, FAKE, FAKE, FAKE, None) == native.MOE_EALIGN


def test_add_rmsnorm_validation():
    L = native.lib()
    f = lambda **k: L.moe_add_rmsnorm(k.get("M", 1), k.get("H", 2816), k.get("h", FAKE),
                                      k.get("a0", FAKE), k.get("a1", None), k.get("g", FAKE),
                                      k.get("eps", 1e-6), k.get("ho", FAKE), k.get("u", FAKE), None)
    assert f(M=0) == native.MOE_EINVAL and f(H=2800) == native.MOE_EINVAL
    assert f(eps=-1.0) == native.MOE_EINVAL and f(eps=float("nan")) == native.MOE_EINVAL
    assert f(h=None) == native.MOE_EINVAL and f(a1=FAKE + 2) == native.MOE_EALIGN
    assert f(ho=None) == native.MOE_EINVAL and f(u=FAKE + 8) == native.MOE_EALIGN


def test_fp8_decode_validation():
    L = native.lib()
    assert L.moe_fp8_decode(0, FAKE, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.moe_fp8_decode(6, FAKE, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.moe_fp8_decode(256, None, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.moe_fp8_decode(256, FAKE, FAKE + 4, FAKE, None) == native.MOE_EALIGN


def test_hbm_read_probe_validation():
    L = native.lib()
    assert L.moe_hbm_read_probe(FAKE, 0, FAKE, None) == native.MOE_EINVAL
    assert L.moe_hbm_read_probe(FAKE, 24, FAKE, None) == native.MOE_EINVAL
    assert L.moe_hbm_read_probe(None, 4096, FAKE, None) == native.MOE_EINVAL
    assert L.moe_hbm_read_probe(FAKE + 8, 4096, FAKE, None) == native.MOE_EALIGN
    assert L.moe_hbm_read_probe(FAKE, 4096, FAKE + 4, None) == native.MOE_EALIGN


# ------------------------------------------------------------------ fused step

def step_desc(**over):
    import synth
    d = native.step_desc(synth.GEMMA4_26B_A4B, max_tokens=5)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def test_step_workspace_and_desc_validation():
    L = native.lib()
    d = step_desc()
    assert native.moe_decode_step_workspace(d) > 0
    for k, v in (("num_layers", 0), ("num_layers", 65), ("vocab", 100), ("max_tokens", 9), ("max_tokens", 0),
                 ("eps", -1.0), ("flags", 4), ("flags", 0x80000001)):
        assert native.moe_decode_step_workspace(step_desc(**{k: v})) == 0, k
    for f in (native.MOE_STEP_COOPERATIVE, native.MOE_STEP_LM_BF16, native.MOE_STEP_COOPERATIVE | native.MOE_STEP_LM_BF16):
        assert native.moe_decode_step_workspace(step_desc(flags=f)) > 0
    wide = step_desc()
    wide.layer.hidden = 3072                       # the fused step takes H <= 2816
    assert native.moe_decode_step_workspace(wide) == 0
    broad = step_desc()
    broad.layer.expert_width = 768                 # and routed rows of at most 704 columns
    assert native.moe_decode_step_workspace(broad) == 0
    assert L.moe_decode_step_workspace(None) == 0


def test_step_prepare_validation():
    d = step_desc()
    need = native.moe_decode_step_workspace(d)
    good = [fake_weights() for _ in range(d.num_layers)]
    with pytest.raises(native.MoeError) as e:
        native.moe_decode_step_prepare(d, good[:-1] + [fake_weights(up_w=None)], FAKE, need)
    assert e.value.status == native.MOE_EINVAL
    with pytest.raises(native.MoeError) as e:
        native.moe_decode_step_prepare(d, good, FAKE, need - 1)
    assert e.value.status == native.MOE_EWORKSPACE


def test_step_call_validation_through_the_binding():
    d = step_desc()
    need = native.moe_decode_step_workspace(d)

    def call(**k):
        args = dict(M=1, gains=FAKE, lm_w=FAKE, lm_s=FAKE, x=FAKE, noise=FAKE, draft=None, token=FAKE,
                    max_logit=None, accepted_len=FAKE, out_tokens=FAKE, y_layers=None, topk_idx=None,
                    topk_w=None, x_final=None, workspace=FAKE, workspace_bytes=need, stream=0)
        args.update(k)
        with pytest.raises(native.MoeError) as e:
            native.moe_decode_step(d, **args)
        return e.value.status

    assert call(M=0) == native.MOE_EINVAL and call(M=6) == native.MOE_EINVAL
    assert call(M=2) == native.MOE_EINVAL                       # drafts required for M > 1
    assert call(x=None) == native.MOE_EINVAL and call(token=None) == native.MOE_EINVAL
    assert call(x=FAKE + 2) == native.MOE_EALIGN and call(token=FAKE + 1) == native.MOE_EALIGN
    assert call(y_layers=FAKE + 8) == native.MOE_EALIGN
    assert call(workspace_bytes=need - 1) == native.MOE_EWORKSPACE


def test_step_status_validation():
    assert native.lib().moe_decode_step_status(None, FAKE) == native.MOE_EINVAL
    assert native.moe_decode_step_status(step_desc(), None) == native.MOE_EWORKSPACE


def test_attn_decode_validation():
    import synth
    L = native.lib()
    good = native.attn_desc(synth.GEMMA4_SLIDING)
    assert native.moe_kv_cache_bytes(good) == 2 * 8 * 1032 * 256
    fp8 = native.attn_desc(synth.GEMMA4_GLOBAL.with_(kv_fp8=True))
    n = 2 * 32768 * 512
    assert native.moe_kv_cache_bytes(fp8) == (n + 255) // 256 * 256 + 4 * 2 * 32768
    assert native.moe_attn_decode_workspace(good, 8) > 0 and native.moe_attn_decode_workspace(good, 9) == 0
    for k, v in (("hidden", 100), ("q_heads", 0), ("kv_heads", 3), ("head_dim", 64), ("head_dim", 96),
                 ("window", -1), ("capacity", 1030), ("kv_type", 2), ("window", 1 << 30)):
        d = native.attn_desc(synth.GEMMA4_SLIDING)
        setattr(d, k, v)
        assert native.moe_kv_cache_bytes(d) == 0, (k, v)
    d = native.attn_desc(synth.GEMMA4_SLIDING)
    d.q_heads, d.kv_heads = 32, 1            # 32 query heads per KV head: above 16
    assert native.moe_kv_cache_bytes(d) == 0
    w = native.AttnWeights(*([FAKE] * 6))
    wsb = native.moe_attn_decode_workspace(good, 5)
    call = lambda **o: L.moe_attn_decode(ctypes.byref(o.get("d", good)), ctypes.byref(o.get("w", w)), o.get("M", 5),
                                         o.get("pos", 100), o.get("u", FAKE), o.get("c", FAKE), o.get("out", FAKE),
                                         o.get("o", None), o.get("ws", FAKE), o.get("wsb", wsb), None)
    assert call(M=0) == native.MOE_EINVAL and call(M=9) == native.MOE_EINVAL and call(pos=-1) == native.MOE_EINVAL
    assert call(u=None) == native.MOE_EINVAL and call(u=FAKE + 2) == native.MOE_EALIGN
    assert call(c=FAKE + 16) == native.MOE_EALIGN           # the cache must be 256-byte aligned
    assert call(o=FAKE + 2) == native.MOE_EALIGN and call(wsb=wsb - 1) == native.MOE_EWORKSPACE
    assert call(w=native.AttnWeights(*([FAKE] * 5 + [None]))) == native.MOE_EINVAL
    g = native.attn_desc(synth.GEMMA4_GLOBAL)
    wsg = native.moe_attn_decode_workspace(g, 5)
    assert call(d=g, pos=32768 - 4, wsb=wsg) == native.MOE_EINVAL      # pos + M beyond a global cache
    assert L.moe_kv_cache_write(ctypes.byref(good), -1, 1, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.moe_kv_cache_write(ctypes.byref(good), 0, 0, FAKE, FAKE, None) == native.MOE_EINVAL
    assert L.moe_kv_cache_write(ctypes.byref(good), 0, 1, FAKE, FAKE + 16, None) == native.MOE_EALIGN


def test_fp8_router_validation():
    import synth
    L = native.lib()
    d = native.layer_desc(synth.TINY, "fp8", "fp8")
    assert native.moe_decode_layer_workspace(d, 1) > 0
    bad = native.layer_desc(synth.TINY, "fp8", "fp8")
    for rt in (4, 5, -1, 1 << 30):
        bad.router_type = rt
        assert native.moe_decode_layer_workspace(bad, 1) == 0
    # either type, expert-major: accepted on the fused geometry
    for rdt in ("bf16", "fp8"):
        assert native.moe_decode_layer_workspace(native.layer_desc(synth.TINY, "fp8", rdt, expert_major=True), 1) > 0
    # beyond the fused geometry: the per-layer kernels read a bf16 [H][E] router only
    wide_shape = synth.TINY.with_(hidden=512, width=768, shared_width=128)
    wide = native.layer_desc(wide_shape, "fp8", "fp8")
    assert native.moe_decode_layer_workspace(wide, 1) == 0
    wide_em = native.layer_desc(wide_shape, "fp8", "bf16", expert_major=True)
    assert native.moe_decode_layer_workspace(wide_em, 1) == 0
    assert native.moe_decode_layer_workspace(native.layer_desc(wide_shape, "fp8", "bf16"), 1) > 0
    w = native.LayerWeights(*([FAKE] * 14 + [None]))        # FP8 router without its scales
    wsb = native.moe_decode_layer_workspace(d, 1)
    st = L.moe_decode_layer(ctypes.byref(d), ctypes.byref(w), 1, FAKE, FAKE, None, None, FAKE, wsb, None)
    assert st == native.MOE_EINVAL
    w.router_s = FAKE + 2
    st = L.moe_decode_layer(ctypes.byref(d), ctypes.byref(w), 1, FAKE, FAKE, None, None, FAKE, wsb, None)
    assert st == native.MOE_EALIGN
    st = L.moe_decode_layer(ctypes.byref(wide), ctypes.byref(native.LayerWeights(*([FAKE] * 15))), 1, FAKE, FAKE,
                            None, None, FAKE, 1 << 30, None)
    assert st == native.MOE_EUNSUPPORTED
    st = L.moe_decode_layer(ctypes.byref(wide_em), ctypes.byref(native.LayerWeights(*([FAKE] * 15))), 1, FAKE, FAKE,
                            None, None, FAKE, 1 << 30, None)
    assert st == native.MOE_EUNSUPPORTED
    sd = native.step_desc(synth.TINY.with_(layers=2), 8, router_dtype="fp8")
    assert native.moe_decode_step_workspace(sd) > 0
