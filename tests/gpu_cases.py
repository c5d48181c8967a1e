"""Helpers shared by the GPU parity tests: marshal generated inputs into the library
and evaluate the CPU oracle on the same inputs (copied to the host)."""
from __future__ import annotations

import os

import numpy as np
import torch

import moe_synth as S
import oracle as O
import mixture_experts_ffn_03_amd as M

# Parity bar for the layer output (bf16 output vs the fp64 oracle before rounding).
MAX_ABS = 2e-2
REL_L2 = 5e-3
# Routing weights: fp32 exp/sigmoid/normalisation vs fp64; a few fp32 ulps per term over
# at most 1024 experts keeps the relative error well under this.
W_RTOL = 1e-5


def config_for(inp: S.LayerInputs, path=M.PATH_AUTO) -> M.MoeConfig:
    s = inp.spec
    return M.make_config(s.tokens, s.hidden, s.experts, s.top_k, s.inter, score_mode=s.score,
                         select_mode=s.select, renormalize=s.renormalize, has_shared=s.shared,
                         shared_inter=s.shared_inter, pre_norm=s.pre_norm, norm_eps=s.norm_eps,
                         vocab=s.vocab, path=path, zero_experts=s.zero_experts)


class LazyHost:
    """Per-expert host copies of a device tensor, fetched on first use."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return self.t[e].cpu().numpy()


def oracle_cache(ws: S.ExpertSet) -> O.DequantCache:
    parts = {}
    for n in ("gate", "up", "down"):
        w = getattr(ws, n)
        gs = None if w.global_scale is None else w.global_scale.cpu().numpy()
        packed = w.packed.view(torch.int16) if w.packed.dtype == torch.bfloat16 else w.packed
        parts[n] = (w.fmt, LazyHost(packed), None if w.scales is None else LazyHost(w.scales), gs)
    return O.DequantCache(parts["gate"], parts["up"], parts["down"])


def f32(t):
    return None if t is None else t.float().cpu().numpy()


def run_layer(inp: S.LayerInputs, path=M.PATH_AUTO, residual=True, stream=None):
    """Run moe_layer_forward; returns (out bf16, logits, ids, w, workspace)."""
    cfg = config_for(inp, path)
    T, E, K, H = inp.spec.tokens, inp.spec.experts, inp.spec.top_k, inp.spec.hidden
    dev = inp.x.device
    ws = M.alloc_workspace(cfg, dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((T, E + inp.spec.zero_experts), dtype=torch.float32, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out, ws,
                    norm_gamma=inp.gamma, logit_bias=inp.logit_bias,
                    correction_bias=inp.correction_bias, token_ids=inp.token_ids,
                    tid2eid=inp.tid2eid,
                    shared=M.expert_weights(inp.shared) if inp.shared is not None else None,
                    residual=inp.residual if residual else None, dbg_logits=logits, dbg_ids=ids,
                    dbg_w=w, stream=stream)
    return out, logits, ids, w, ws


def oracle_workers() -> int:
    """Host threads for the oracle's expert loop (at most 16: a GPU host's CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def oracle_layer(inp: S.LayerInputs, rows=None, residual=True, workers=1):
    s = inp.spec
    res = inp.residual if residual else torch.zeros_like(inp.residual)
    return O.layer_forward(
        f32(inp.x), f32(res), f32(inp.router_w), oracle_cache(inp.routed), s.top_k,
        score=s.score, select=s.select, renormalize=s.renormalize, logit_bias=f32(inp.logit_bias),
        correction_bias=f32(inp.correction_bias),
        token_ids=None if inp.token_ids is None else inp.token_ids.cpu().numpy(),
        tid2eid=None if inp.tid2eid is None else inp.tid2eid.cpu().numpy(),
        gamma=f32(inp.gamma), norm_eps=s.norm_eps,
        shared=oracle_cache(inp.shared) if inp.shared is not None else None, rows=rows,
        zero_experts=s.zero_experts, workers=workers)


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values at |v| (normal range): the largest error that the
    output's own final rounding to bf16 can contribute."""
    _, e = np.frexp(np.abs(v).astype(np.float64))
    return np.ldexp(1.0, e - 9)


def errors(got_bf16: np.ndarray, want: np.ndarray):
    """(max-abs error beyond the output's bf16 rounding, raw max-abs error, rel-L2 error)
    of a bf16 result against the fp64 oracle."""
    d = np.abs(got_bf16.astype(np.float64) - want)
    if not d.size:
        return 0.0, 0.0, 0.0
    beyond = np.maximum(d - bf16_half_ulp(want), 0.0)
    return float(beyond.max()), float(d.max()), \
        float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-300))


def assert_layer_close(got_bf16, want, resid=None, label=""):
    """Parity bar of the layer output: max-abs 2e-2 on the error beyond the output's own
    rounding to bf16 (a bf16 value cannot be closer to the exact result than half an
    ulp, 0.03 for |v| in [8, 16)), and rel-L2 5e-3 on the raw bf16 output."""
    mx, raw, rl = errors(got_bf16, want)
    msg = (f"{label}: max-abs beyond bf16 rounding {mx:.3e} (bar {MAX_ABS}; raw {raw:.3e}), "
           f"rel-L2 {rl:.3e} (bar {REL_L2})")
    if resid is not None:
        delta_got = got_bf16.astype(np.float64) - resid
        delta_want = want - resid
        rl_delta = float(np.linalg.norm(delta_got - delta_want) / max(np.linalg.norm(delta_want), 1e-300))
        msg += f", rel-L2 of the MoE delta {rl_delta:.3e}"
    print(msg, flush=True)
    assert mx <= MAX_ABS and rl <= REL_L2, msg
