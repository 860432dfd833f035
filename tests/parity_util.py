"""Helpers shared by the GPU parity tests: moving seeded weights between host and
device, resampling step inputs until every decision is unambiguous in the
oracle, and the bf16 tolerance checks."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

TAU = 1e-3          # a routing or argmax decision is ambiguous when its fp64 margin is below this
REL_L2 = 2e-3       # bf16 outputs: relative L2 error bound ...
MAX_ABS = 1e-2      # ... and max absolute error bound, against the oracle's fp64 values


def to_device(w: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}


def bf16_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_bf16_output(got_bits, ref_f64, ref_bits=None, what="y", min_exact=0.99):
    got = bf16_f64(got_bits)
    err = rel_l2(got, ref_f64)
    mab = float(np.abs(got - ref_f64).max()) if got.size else 0.0
    assert err <= REL_L2, "%s rel-L2 %.3g > %.3g" % (what, err, REL_L2)
    assert mab <= MAX_ABS, "%s max-abs %.3g > %.3g" % (what, mab, MAX_ABS)
    if ref_bits is not None:
        exact = float((np.asarray(got_bits, np.uint16) == np.asarray(ref_bits, np.uint16)).mean())
        assert exact >= min_exact, "%s only %.4f of elements equal the oracle's bf16" % (what, exact)
    return err, mab


def unambiguous_layer_input(shape, M, w_host, step, tau=TAU, max_tries=200):
    """Resample the step's input (sub-seed 0, 1, ...) until no top-K decision has an
    oracle margin below tau. Returns (x bf16 CPU tensor, oracle result)."""
    for sub in range(max_tries):
        x = synth.hidden_inputs(shape, M, step, sub)
        r = oracle.moe_layer(synth.bits16(x), w_host, shape.top_k)
        if (r["gap"] >= tau).all():
            return x, r
    raise RuntimeError("no unambiguous input found")


def unambiguous_lm_input(shape, M, Q, s, step, tau=TAU, max_tries=200, tag="lm_x"):
    for sub in range(max_tries):
        x = synth.hidden_inputs(shape, M, step, sub, tag=tag)
        tok, ml, gap = oracle.lm_head_argmax(synth.bits16(x), Q, s)
        if (gap >= tau).all():
            return x, tok, ml
    raise RuntimeError("no unambiguous input found")


def stack_decisions_unambiguous(res, tau=TAU) -> bool:
    return all((l["gap"] >= tau).all() for l in res["layers"]) and (res["lm_gap"] >= tau).all()
