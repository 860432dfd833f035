"""CPU oracle for the batch-1 fine-grained MoE decode step (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
import this package. The GPU library never imports, links or calls it, and the two
share no source. The arithmetic lives in ``oracle.c`` (plain fp64 loops); this
module builds it with gcc, marshals numpy arrays into it and wires the stacked
decode step out of its routines.

Inputs are numpy arrays in storage formats: bf16 as uint16 bits, FP8 as uint8
OCP E4M3FN codes, scales as float32. Sources and readings are listed in
``oracle.c`` next to each routine; the stack wiring is described in
``stack_step`` below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fno-fast-math", "-ffp-contract=off"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP). Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int
            L.oracle_fp8_e4m3.restype = ctypes.c_double
            L.oracle_fp8_e4m3.argtypes = [ctypes.c_uint8]
            L.oracle_bf16.restype = ctypes.c_double
            L.oracle_bf16.argtypes = [ctypes.c_uint16]
            L.oracle_bf16_round.restype = ctypes.c_uint16
            L.oracle_bf16_round.argtypes = [ctypes.c_double]
            L.oracle_gelu_tanh.restype = ctypes.c_double
            L.oracle_gelu_tanh.argtypes = [ctypes.c_double]
            L.oracle_router.restype = None
            L.oracle_router.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
            L.oracle_moe_layer.restype = None
            L.oracle_moe_layer.argtypes = [I] * 7 + [P] * 22
            L.oracle_router_fp8.restype = None
            L.oracle_router_fp8.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P]
            L.oracle_lm_head.restype = None
            L.oracle_lm_head.argtypes = [I, I, I, P, P, P, P, P, P]
            L.oracle_lm_head_bf16.restype = None
            L.oracle_lm_head_bf16.argtypes = [I, I, I, P, P, P, P, P]
            L.oracle_lm_head_rows.restype = None
            L.oracle_lm_head_rows.argtypes = [I, I, I, P, P, P, P, P]
            L.oracle_spec_accept.restype = I
            L.oracle_spec_accept.argtypes = [I, P, P, P]
            L.oracle_add_rmsnorm.restype = None
            L.oracle_add_rmsnorm.argtypes = [I, I, P, P, P, P, ctypes.c_double, P, P]
            L.oracle_philox4x32_10.restype = None
            L.oracle_philox4x32_10.argtypes = [P, P, P]
            L.oracle_sample_uniform.restype = ctypes.c_double
            L.oracle_sample_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, I, I]
            L.oracle_lm_head_logits.restype = None
            L.oracle_lm_head_logits.argtypes = [I, I, I, P, P, P, P]
            L.oracle_spec_sample.restype = I
            L.oracle_spec_sample.argtypes = [I, I, P, ctypes.c_double, P, P, P, ctypes.c_uint64,
                                             ctypes.c_uint64, P, P, P]
            L.oracle_gemv_fp8.restype = None
            L.oracle_gemv_fp8.argtypes = [I, I, P, P, P, P]
            L.oracle_dense_mlp.restype = None
            L.oracle_dense_mlp.argtypes = [I, I, P, P, P, P, P, P, P, P]
            L.oracle_bf16_round_n.restype = None
            L.oracle_bf16_round_n.argtypes = [I, P, P]
            L.oracle_fp8_from_f32.restype = ctypes.c_uint8
            L.oracle_fp8_from_f32.argtypes = [ctypes.c_float]
            L.oracle_fp8_quant_row.restype = None
            L.oracle_fp8_quant_row.argtypes = [I, P, P, P]
            L.oracle_attn_decode.restype = I
            L.oracle_attn_decode.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, I, P, P, P, P, P, P,
                                             P, P, P]
            L.oracle_num_threads.restype = I
            L.oracle_num_threads.argtypes = []
            L.oracle_set_num_threads.restype = None
            L.oracle_set_num_threads.argtypes = [I]
            _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def fp8_e4m3(code: int) -> float:
    return lib().oracle_fp8_e4m3(int(code))


def bf16(bits: int) -> float:
    return lib().oracle_bf16(int(bits))


def bf16_round(v: float) -> int:
    return lib().oracle_bf16_round(float(v))


def gelu_tanh(z: float) -> float:
    return lib().oracle_gelu_tanh(float(z))


def router(u, W, bias, K):
    """u uint16 [M][H], W uint16 [H][E], bias f32 [E] or None -> dict(idx, w, gap, logits)."""
    u = _c(u, np.uint16)
    W = _c(W, np.uint16)
    bias = _c(bias, np.float32)
    M, H = u.shape
    E = W.shape[1]
    logits = np.empty((M, E), np.float64)
    idx = np.empty((M, K), np.int32)
    wts = np.empty((M, K), np.float64)
    gap = np.empty(M, np.float64)
    lib().oracle_router(M, H, E, K, _p(u), _p(W), _p(bias), _p(logits), _p(idx), _p(wts), _p(gap))
    return {"idx": idx, "w": wts, "gap": gap, "logits": logits}


def router_fp8(u, W8, s, bias, K):
    """u uint16 [M][H], W8 uint8 FP8 codes [H][E], s f32 [E], bias f32 [E] or None ->
    dict(idx, w, gap, logits) (oracle_router_fp8)."""
    u = _c(u, np.uint16)
    W8 = _c(W8, np.uint8)
    s = _c(s, np.float32)
    bias = _c(bias, np.float32)
    M, H = u.shape
    E = W8.shape[1]
    logits = np.empty((M, E), np.float64)
    idx = np.empty((M, K), np.int32)
    wts = np.empty((M, K), np.float64)
    gap = np.empty(M, np.float64)
    lib().oracle_router_fp8(M, H, E, K, _p(u), _p(W8), _p(s), _p(bias), _p(logits), _p(idx), _p(wts), _p(gap))
    return {"idx": idx, "w": wts, "gap": gap, "logits": logits}


def moe_layer(u, w: dict, K: int):
    """One MoE layer. u uint16 [M][H]; w: synth.weights_to_host(layer_weights(...)).

    Returns dict(idx [M][K] ascending, w [M][K], gap [M], logits [M][E],
    y fp64 [M][H], y_bf16 uint16 [M][H]).
    """
    u = _c(u, np.uint16)
    M, H = u.shape
    wtype = 0 if w["expert_dtype"] == "fp8" else 1
    edt = np.uint8 if wtype == 0 else np.uint16
    G = _c(w["gate_w"], edt)
    E, D, _ = G.shape
    shG = _c(w["sh_gate_w"], edt)
    Ds = 0 if shG is None else shG.shape[0]
    rfp8 = w.get("router_s") is not None
    args = dict(
        router_w=_c(w["router_w"], np.uint8 if rfp8 else np.uint16),
        router_s=_c(w.get("router_s"), np.float32), router_b=_c(w["router_b"], np.float32),
        G=G, U=_c(w["up_w"], edt), Dn=_c(w["down_w"], edt),
        gs=_c(w["gate_s"], np.float32), us=_c(w["up_s"], np.float32),
        ds=_c(w["down_s"], np.float32),
        shG=shG, shU=_c(w["sh_up_w"], edt), shD=_c(w["sh_down_w"], edt),
        shgs=_c(w["sh_gate_s"], np.float32), shus=_c(w["sh_up_s"], np.float32),
        shds=_c(w["sh_down_s"], np.float32))
    E_r = args["router_w"].shape[1]
    assert E_r == E
    idx = np.empty((M, K), np.int32)
    wts = np.empty((M, K), np.float64)
    gap = np.empty(M, np.float64)
    logits = np.empty((M, E), np.float64)
    y = np.empty((M, H), np.float64)
    yb = np.empty((M, H), np.uint16)
    lib().oracle_moe_layer(
        M, H, E, K, D, Ds, wtype, _p(u), _p(args["router_w"]), _p(args["router_s"]), _p(args["router_b"]),
        _p(args["G"]), _p(args["U"]), _p(args["Dn"]), _p(args["gs"]), _p(args["us"]),
        _p(args["ds"]), _p(args["shG"]), _p(args["shU"]), _p(args["shD"]),
        _p(args["shgs"]), _p(args["shus"]), _p(args["shds"]),
        _p(idx), _p(wts), _p(gap), _p(logits), _p(y), _p(yb))
    return {"idx": idx, "w": wts, "gap": gap, "logits": logits, "y": y, "y_bf16": yb}


def lm_head_argmax(x, Q, s):
    """x uint16 [M][H], Q uint8 [V][H], s f32 [V] -> (tok int32 [M], max_logit f64 [M], gap f64 [M])."""
    x = _c(x, np.uint16)
    Q = _c(Q, np.uint8)
    s = _c(s, np.float32)
    M, H = x.shape
    V = Q.shape[0]
    tok = np.empty(M, np.int32)
    ml = np.empty(M, np.float64)
    gap = np.empty(M, np.float64)
    lib().oracle_lm_head(M, H, V, _p(x), _p(Q), _p(s), _p(tok), _p(ml), _p(gap))
    return tok, ml, gap


def lm_head_argmax_bf16(x, W):
    """x uint16 [M][H], W uint16 (bf16 bits) [V][H] -> (tok int32 [M], max_logit f64 [M], gap f64 [M])."""
    x = _c(x, np.uint16)
    W = _c(W, np.uint16)
    M, H = x.shape
    V = W.shape[0]
    tok = np.empty(M, np.int32)
    ml = np.empty(M, np.float64)
    gap = np.empty(M, np.float64)
    lib().oracle_lm_head_bf16(M, H, V, _p(x), _p(W), _p(tok), _p(ml), _p(gap))
    return tok, ml, gap


def lm_head_rows(x, Q, s, rows):
    """Logits of the given vocab rows only: f64 [M][len(rows)]."""
    x = _c(x, np.uint16)
    Q = _c(Q, np.uint8)
    s = _c(s, np.float32)
    rows = _c(rows, np.int32)
    M, H = x.shape
    out = np.empty((M, len(rows)), np.float64)
    lib().oracle_lm_head_rows(M, H, len(rows), _p(rows), _p(x), _p(Q), _p(s), _p(out))
    return out


def spec_accept(draft, target):
    """draft int32 [gamma], target int32 [gamma+1] -> (n, out int32 [gamma+1])."""
    target = _c(target, np.int32)
    gamma = len(target) - 1
    draft = _c(draft, np.int32) if gamma > 0 else np.zeros(1, np.int32)
    out = np.empty(gamma + 1, np.int32)
    n = lib().oracle_spec_accept(gamma, _p(draft), _p(target), _p(out))
    return n, out


def philox4x32_10(ctr, key):
    """Philox4x32-10 of a 4-word counter under a 2-word key -> 4 uint32 words."""
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.empty(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def sample_uniform(seed: int, step: int, row: int, v: int) -> float:
    return lib().oracle_sample_uniform(int(seed), int(step), int(row), int(v))


def lm_head_logits(x, Q, s):
    """x uint16 [M][H], Q uint8 [V][H], s f32 [V] -> fp64 logits [M][V]."""
    x = _c(x, np.uint16)
    Q = _c(Q, np.uint8)
    s = _c(s, np.float32)
    M, H = x.shape
    V = Q.shape[0]
    out = np.empty((M, V), np.float64)
    lib().oracle_lm_head_logits(M, H, V, _p(x), _p(Q), _p(s), _p(out))
    return out


def spec_sample(logits, T, draft, q, u_acc, seed, step):
    """Stochastic speculative acceptance over target logits [M][V] (fp64) at temperature T:
    draft int32 [M-1], q f32 [M-1][V] (the drafter's distributions), u_acc f32 [M-1].
    Returns (n, out int32 [M], acc_margin f64 [M-1], samp_margin)."""
    logits = _c(logits, np.float64)
    M, V = logits.shape
    g = M - 1
    draft = _c(draft, np.int32) if g > 0 else np.zeros(1, np.int32)
    q = _c(q, np.float32) if g > 0 else np.zeros((1, V), np.float32)
    u = _c(u_acc, np.float32) if g > 0 else np.zeros(1, np.float32)
    out = np.empty(M, np.int32)
    am = np.empty(max(g, 1), np.float64)
    sm = np.empty(1, np.float64)
    n = lib().oracle_spec_sample(M, V, _p(logits), float(T), _p(draft), _p(q), _p(u), int(seed), int(step),
                                 _p(out), _p(am), _p(sm))
    return n, out, am[:g], float(sm[0])


def gemv_fp8(Q, s, x):
    """Q uint8 [N][K] FP8, s f32 [N], x uint16 bf16 [K] -> fp64 [N]."""
    Q = _c(Q, np.uint8)
    s = _c(s, np.float32)
    x = _c(x, np.uint16)
    N, K = Q.shape
    out = np.empty(N, np.float64)
    lib().oracle_gemv_fp8(N, K, _p(Q), _p(s), _p(x), _p(out))
    return out


def dense_mlp(u, G, U, Dn, sg, su, sd):
    """u uint16 [H]; G, U uint8 [F][H]; Dn uint8 [H][F]; scales f32 -> fp64 [H]."""
    u = _c(u, np.uint16)
    G, U, Dn = _c(G, np.uint8), _c(U, np.uint8), _c(Dn, np.uint8)
    sg, su, sd = _c(sg, np.float32), _c(su, np.float32), _c(sd, np.float32)
    F, H = G.shape
    out = np.empty(H, np.float64)
    lib().oracle_dense_mlp(H, F, _p(u), _p(G), _p(U), _p(Dn), _p(sg), _p(su), _p(sd), _p(out))
    return out


def bf16_round_n(v):
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_round_n(v.size, _p(v), _p(out))
    return out


def draft_step(tok0, hidden0, head, target_Q, target_s, gamma, eps=1e-6):
    """The MTP drafter's step, gamma drafts in sequence (page "LLM decoding", "The one-line
    shape bug that disabled the model's own drafter": the head's pre_projection takes 5632 =
    2 x 2816 inputs, the target's 2816-wide embedding of the token and a 2816-wide hidden
    state, down to its 1024-wide width; the head has its own 1024-wide embedding table;
    "Lever 2": a 430M head proposes the tokens the target then verifies). The rest of the
    head is not on the page; the reading taken (the body sized so the head holds about 430M
    parameters) is, per draft i = 1..gamma from the previous token t and hidden g:
        e   = bf16(s_t * dec(Q_target[t]))                 the target's (tied) embedding row
        z   = bf16(pre_proj([e | g]))                      5632 -> 1024
        for each block b: u = rmsnorm(z; g_b), z = bf16(z + mlp_b(u))      width 1024
        zf  = rmsnorm(z; g_final)
        d_i = argmax_v table(zf)[v]                        the head's own 262144 x 1024 table
        g   = bf16(post_proj(zf))                          1024 -> 2816, the next draft's hidden
    head: dict of numpy arrays (FP8 codes uint8, scales f32, gains bf16 uint16):
        pre_w [1024][5632], pre_s; blocks: list of dict(gain, gate_w, gate_s, up_w, up_s,
        down_w, down_s); final_gain; table_w [V][1024], table_s; post_w [2816][1024], post_s.
    Returns dict(drafts int32 [gamma], gaps f64 [gamma] (the argmax margins), z [gamma][1024],
    g [gamma][2816])."""
    t = int(tok0)
    g = np.ascontiguousarray(hidden0, np.uint16)
    H = g.shape[0]
    drafts, gaps, zs, gs = [], [], [], []
    dec = _fp8_values()
    for i in range(gamma):
        e = bf16_round_n(float(target_s[t]) * dec[target_Q[t]])
        x = np.concatenate([e, g])
        z = bf16_round_n(gemv_fp8(head["pre_w"], head["pre_s"], x))
        for b in head["blocks"]:
            _, u = add_rmsnorm(z[None, :], np.zeros_like(z)[None, :], None, b["gain"], eps)
            y = dense_mlp(u[0], b["gate_w"], b["up_w"], b["down_w"], b["gate_s"], b["up_s"], b["down_s"])
            z = bf16_round_n(_bf16_values(z) + y)
        _, zf = add_rmsnorm(z[None, :], np.zeros_like(z)[None, :], None, head["final_gain"], eps)
        tok, _, gap = lm_head_argmax(zf, head["table_w"], head["table_s"])
        t = int(tok[0])
        g = bf16_round_n(gemv_fp8(head["post_w"], head["post_s"], zf[0]))
        drafts.append(t)
        gaps.append(float(gap[0]))
        zs.append(z)
        gs.append(g)
    return {"drafts": np.array(drafts, np.int32), "gaps": np.array(gaps), "z": np.array(zs), "g": np.array(gs)}


def _fp8_values():
    return np.array([fp8_e4m3(c) for c in range(256)], np.float64)


def _bf16_values(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def add_rmsnorm(h, a0, a1, g, eps=1e-6):
    """h, a0, a1 uint16 [M][H] (a1 may be None), g uint16 [H] -> (h_out, u) uint16 [M][H]."""
    h = _c(h, np.uint16)
    a0 = _c(a0, np.uint16)
    a1 = _c(a1, np.uint16)
    g = _c(g, np.uint16)
    M, H = h.shape
    ho = np.empty_like(h)
    uo = np.empty_like(h)
    lib().oracle_add_rmsnorm(M, H, _p(h), _p(a0), _p(a1), _p(g), float(eps), _p(ho), _p(uo))
    return ho, uo


def stack_step(x, layers, noise, gains, lm_w, lm_s, K, eps=1e-6, draft=None, lm_bf16=False):
    """One decode step through a stack of MoE layers, then lm_head, argmax, acceptance.

    Wiring (the pages omit attention; the stacked workload replaces it by a residual
    add of noise and puts an RMSNorm before every layer and before the lm_head):
        h = x
        for l: h, u_l = add_rmsnorm(h, noise_l, y_{l-1}, g_l); y_l = moe_layer(u_l)
        h, x_f = add_rmsnorm(h, y_{L-1}, None, g_L)
        tok = argmax(lm_head(x_f)); (n, out) = spec_accept(draft, tok)
    layers: a list of host weight dicts (or a callable l -> dict, to fetch lazily).
    lm_bf16: lm_w holds bf16 bits [V][H] (no scales; lm_s ignored) instead of FP8 codes.
    Returns per-layer u, routing, gaps and y, plus the final tokens and gaps.
    """
    L = len(noise)
    h = np.ascontiguousarray(x, np.uint16)
    y_prev = None
    per = []
    for l in range(L):
        w = layers(l) if callable(layers) else layers[l]
        h_in = h
        h, u = add_rmsnorm(h, noise[l], y_prev, gains[l], eps)
        r = moe_layer(u, w, K)
        per.append({"h_in": h_in, "h": h, "u": u, "idx": r["idx"], "w": r["w"], "gap": r["gap"],
                    "y": r["y"], "y_bf16": r["y_bf16"]})
        y_prev = r["y_bf16"]
    h_last = h
    h, xf = add_rmsnorm(h, y_prev, None, gains[L], eps)
    tok, ml, gap = lm_head_argmax_bf16(xf, lm_w) if lm_bf16 else lm_head_argmax(xf, lm_w, lm_s)
    out = {"layers": per, "h_last": h_last, "x_final": xf, "h_final": h, "tok": tok,
           "max_logit": ml, "lm_gap": gap}
    if draft is not None:
        n, acc = spec_accept(draft, tok)
        out["accepted"] = n
        out["out_tokens"] = acc
    return out


def fp8_from_f32(v):
    """E4M3FN code (round to nearest even, saturating at 448) of one fp32 value."""
    return int(lib().oracle_fp8_from_f32(float(np.float32(v))))


def fp8_quant_rows(x):
    """The FP8 KV cache's quantiser over the last axis: x uint16 bf16 bits [..., n] ->
    (codes uint8 [..., n], scales f32 [...]), each row scale max|x| / 448 (fp32)."""
    x = _c(x, np.uint16)
    n = x.shape[-1]
    rows = x.reshape(-1, n)
    codes = np.empty(rows.shape, np.uint8)
    scales = np.empty(rows.shape[0], np.float32)
    L = lib()
    for i in range(rows.shape[0]):
        r = np.ascontiguousarray(rows[i])
        sc = np.empty(1, np.float32)
        cd = np.empty(n, np.uint8)
        L.oracle_fp8_quant_row(n, _p(r), _p(cd), _p(sc))
        codes[i] = cd
        scales[i] = sc[0]
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1])


def decode_kv(keys, kv_fp8):
    """Cached keys as the attention reads them, fp64: keys uint16 bf16 bits [..., dh] as
    written into the cache; for an FP8 cache each row is quantised and decoded
    (decode(code) * scale)."""
    keys = _c(keys, np.uint16)
    if not kv_fp8:
        return _bf16_values(keys)
    codes, scales = fp8_quant_rows(keys)
    return _fp8_values()[codes] * scales.astype(np.float64)[..., None]


def attn_decode(u, w, shape, M, pos, hist_keys, h0=0):
    """One attention layer of the decode step (oracle_attn_decode).
    u uint16 [M][H]; w: host dict q_w, q_s, k_w, k_s, o_w, o_s; shape with hidden, q_heads,
    kv_heads, head_dim, window, kv_fp8; hist_keys uint16 bf16 bits [pos - h0][kv_heads][head_dim],
    the keys written into the cache for positions h0 .. pos - 1 (decoded here as the cache
    holds them). Returns q, k (bf16 bits), k_codes / k_scales (FP8 cache), o (fp64), o_bf16,
    out (fp64), out_bf16."""
    u = _c(u, np.uint16)
    H, nq, nkv, dh = shape.hidden, shape.q_heads, shape.kv_heads, shape.head_dim
    fp8 = int(bool(shape.kv_fp8))
    hk = np.asarray(hist_keys, np.uint16).reshape(pos - h0, nkv, dh)
    hist = np.ascontiguousarray(decode_kv(hk, fp8).transpose(1, 0, 2), np.float64)   # [nkv][pos - h0][dh]
    NQ, NK = nq * dh, nkv * dh
    q = np.empty((M, NQ), np.uint16)
    k = np.empty((M, NK), np.uint16)
    kc = np.zeros((M, nkv, dh), np.uint8)
    ksc = np.zeros((M, nkv), np.float32)
    o = np.empty((M, NQ), np.float64)
    ob = np.empty((M, NQ), np.uint16)
    out = np.empty((M, H), np.float64)
    outb = np.empty((M, H), np.uint16)
    W = {k_: _c(v, np.uint8 if v.dtype == np.uint8 else np.float32) for k_, v in w.items()}
    rc = lib().oracle_attn_decode(M, H, nq, nkv, dh, shape.window, pos, fp8, _p(u), _p(W["q_w"]), _p(W["q_s"]),
                                  _p(W["k_w"]), _p(W["k_s"]), _p(W["o_w"]), _p(W["o_s"]), h0, _p(hist), _p(q),
                                  _p(k), _p(kc), _p(ksc), _p(o), _p(ob), _p(out), _p(outb))
    if rc != 0:
        raise ValueError("attn_decode: a position the tokens see lies below h0")
    return {"q": q, "k": k, "k_codes": kc, "k_scales": ksc, "o": o, "o_bf16": ob, "out": out, "out_bf16": outb}
