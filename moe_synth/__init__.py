"""Seeded synthetic inputs for the FP4 mixture-of-experts feed-forward layer.

This module is shared by the tests, the benchmark and the smoke check. It draws
random tensors and encodes expert weights into the two 4-bit storage formats
named on the MoE module page (spark_model/layers/moe/mod.rs, docs of
``MoeLayer.experts_scale_kind`` and ``shared_experts_scale_kind``):

* NVFP4: packed E2M1 codes, one FP8-E4M3 scale per 16 values along K and one
  f32 global scale per (expert, projection) tensor;
* MXFP4: packed E2M1 codes, one E8M0 scale per 32 values along K, no global.

It holds none of the layer's arithmetic: nothing here decodes a code, routes a
token or evaluates an expert. The encoders are test-only and follow the public
OCP Microscaling (MX) v1.0 element definitions; they are the inverse of what the
layer consumes, written independently of both the CPU oracle and the HIP path.

Tensors are produced with ``torch`` on the requested device (CPU for the small
host-side tests, the GPU for the full-size workloads, where drawing several GB
of weights on the host would take minutes). The same seed gives different
values on CPU and GPU, because the two devices use different generators; each
is reproducible on its own.

Storage layout (shared by both sides of the boundary):
  FP4:  packed uint8 [E, N, K/2]  byte j of a row holds codes 2j (low nibble) and 2j+1 (high)
        scales uint8 [E, N, K/16] E4M3FN codes (NVFP4) or [E, N, K/32] E8M0 codes (MXFP4)
        global f32 [E]            NVFP4 only
  FP8:  packed uint8 [E, N, K]    E4M3FN codes
        scales f32 [E, ceil(N/128), ceil(K/128)]  one scale per 128 x 128 block
  BF16: packed bf16 [E, N, K], no scales
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

NVFP4 = 0
MXFP4 = 1
FP8 = 2
BF16 = 3
FP8_BLOCK = 128

SOFTMAX = 0
SIGMOID = 1
SQRT_SOFTPLUS = 2
SOFTMAX_BIAS = 3

TOPK = 0
HASH = 1


@dataclasses.dataclass
class LayerSpec:
    """Shape and routing description of one MoE layer workload."""

    name: str
    tokens: int
    hidden: int
    experts: int
    top_k: int
    inter: int
    fmt: int = NVFP4
    score: int = SOFTMAX
    select: int = TOPK
    renormalize: bool = False
    shared: bool = False
    shared_inter: int = 0
    shared_fmt: int = NVFP4
    pre_norm: bool = False
    norm_eps: float = 1e-6
    vocab: int = 0
    zipf_bias: float = 0.0          # exponent of the Zipf logit bias, 0 = none
    correction_bias: bool = False    # U(-0.1, 0.1) per-expert bias (sigmoid routing)
    zero_experts: int = 0            # zero-computation experts (router outputs E + Z)
    seed: int = 1000


def _cfg(**kw) -> LayerSpec:
    return LayerSpec(**kw)


# The five workloads: a tiny parity case, two decode shapes, a prefill shape with
# skewed expert loads and a hash-routed mixed-format layer.
WORKLOADS: Dict[str, LayerSpec] = {
    "tiny": _cfg(name="tiny", tokens=4, hidden=256, experts=8, top_k=2, inter=512,
                 fmt=NVFP4, score=SOFTMAX, renormalize=False, seed=1000),
    "qwen3_decode_t1": _cfg(name="qwen3_decode_t1", tokens=1, hidden=2048, experts=128, top_k=8,
                            inter=768, fmt=NVFP4, score=SOFTMAX, renormalize=True, seed=1001),
    "qwen3_decode_t8": _cfg(name="qwen3_decode_t8", tokens=8, hidden=2048, experts=128, top_k=8,
                            inter=768, fmt=NVFP4, score=SOFTMAX, renormalize=True, seed=1001),
    "dsv3_decode_t32": _cfg(name="dsv3_decode_t32", tokens=32, hidden=7168, experts=256, top_k=8,
                            inter=2048, fmt=NVFP4, score=SIGMOID, renormalize=True,
                            correction_bias=True, shared=True, shared_inter=2048,
                            shared_fmt=NVFP4, seed=1002),
    "prefill_zipf_t4096": _cfg(name="prefill_zipf_t4096", tokens=4096, hidden=4096, experts=64,
                               top_k=6, inter=1408, fmt=MXFP4, score=SOFTMAX, renormalize=False,
                               zipf_bias=1.1, seed=1003),
    "hash_mxfp4_t512": _cfg(name="hash_mxfp4_t512", tokens=512, hidden=4096, experts=256, top_k=6,
                            inter=2048, fmt=MXFP4, score=SOFTMAX, select=HASH, renormalize=True,
                            shared=True, shared_inter=2048, shared_fmt=NVFP4, pre_norm=True,
                            norm_eps=1e-6, vocab=32768, seed=1004),
}


def scaled(spec: LayerSpec, **changes) -> LayerSpec:
    """A copy of ``spec`` with some fields replaced (used for reduced-size parity cases)."""
    return dataclasses.replace(spec, **changes)


# ---------------------------------------------------------------------------
# Test-only encoders (OCP MX v1.0 element formats)
# ---------------------------------------------------------------------------

def _e2m1_encode_magnitude(a: torch.Tensor) -> torch.Tensor:
    """Round |w| (already divided by its block scale) to the nearest E2M1 magnitude code.

    The E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7). Ties go to
    the code with an even mantissa bit (codes 0, 2, 4, 6); values above 6 saturate.
    Each comparison below is one decision boundary between neighbouring codes:
    ``>`` where the tie rounds down, ``>=`` where it rounds up.
    """
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8) + (a > 1.25).to(torch.uint8)
            + (a >= 1.75).to(torch.uint8) + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
            + (a > 5.0).to(torch.uint8))
    return code


def _pack_codes(w_scaled: torch.Tensor) -> torch.Tensor:
    """Sign + magnitude codes of ``w_scaled`` [..., K] packed two per byte -> [..., K/2]."""
    mag = _e2m1_encode_magnitude(w_scaled.abs())
    code = mag | ((w_scaled < 0).to(torch.uint8) << 3)
    lo = code[..., 0::2]
    hi = code[..., 1::2]
    return (lo | (hi << 4)).contiguous()


def quantize_nvfp4(w: torch.Tensor):
    """Encode one fp32 tensor [N, K] as NVFP4: (packed [N,K/2], e4m3 scales [N,K/16], global f32).

    global = amax / (448 * 6), so the largest block scale reaches the E4M3 maximum;
    each 16-value block gets scale = E4M3(amax_block / (6 * global)) rounded to
    nearest even; codes are w / (scale * global) rounded onto the E2M1 grid.
    """
    n, k = w.shape
    assert k % 16 == 0
    amax = w.abs().max().float()
    gscale = (amax / (448.0 * 6.0)).item() if amax > 0 else 1.0
    gscale = float(torch.tensor(gscale, dtype=torch.float32))
    blocks = w.reshape(n, k // 16, 16)
    bmax = blocks.abs().amax(dim=-1)
    s = (bmax / (6.0 * gscale)).clamp(max=448.0).to(torch.float8_e4m3fn)
    s_val = s.to(torch.float32)
    denom = (s_val * gscale).unsqueeze(-1)
    safe = torch.where(denom > 0, denom, torch.ones_like(denom))
    ws = torch.where(denom > 0, blocks / safe, torch.zeros_like(blocks))
    packed = _pack_codes(ws.reshape(n, k))
    return packed, s.view(torch.uint8).contiguous(), gscale


def quantize_mxfp4(w: torch.Tensor):
    """Encode one fp32 tensor [N, K] as MXFP4: (packed [N,K/2], e8m0 scales [N,K/32]).

    Per OCP MX v1.0, the shared exponent of a 32-value block is
    floor(log2(amax_block)) - 2 (2 = the largest E2M1 exponent); codes are
    w / 2^X rounded onto the E2M1 grid, saturating at 6.
    """
    n, k = w.shape
    assert k % 32 == 0
    blocks = w.reshape(n, k // 32, 32)
    bmax = blocks.abs().amax(dim=-1)
    # frexp: bmax = m * 2^e with m in [0.5, 1) -> floor(log2 bmax) = e - 1
    _, e = torch.frexp(bmax)
    x = (e.to(torch.int32) - 1) - 2
    x = torch.where(bmax > 0, x, torch.full_like(x, -127)).clamp(-127, 127)
    code = (x + 127).to(torch.uint8)
    scale = torch.ldexp(torch.ones_like(bmax), x.to(bmax.dtype))
    ws = blocks / scale.unsqueeze(-1)
    packed = _pack_codes(ws.reshape(n, k))
    return packed, code.contiguous()


def quantize_fp8(w: torch.Tensor):
    """Encode one fp32 tensor [N, K] as FP8: (E4M3FN codes [N, K], fp32 scales
    [ceil(N/128), ceil(K/128)]). Each 128 x 128 block gets scale = amax_block / 448 (fp32),
    so its largest value maps to the E4M3 maximum; codes are w / scale rounded to nearest
    even by torch's float8_e4m3fn conversion (clamped to +-448 first)."""
    n, k = w.shape
    nb, kb = -(-n // FP8_BLOCK), -(-k // FP8_BLOCK)
    pad = torch.zeros((nb * FP8_BLOCK, kb * FP8_BLOCK), dtype=torch.float32, device=w.device)
    pad[:n, :k] = w
    blocks = pad.reshape(nb, FP8_BLOCK, kb, FP8_BLOCK)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    full = scale.repeat_interleave(FP8_BLOCK, 0).repeat_interleave(FP8_BLOCK, 1)[:n, :k]
    codes = (w / full).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).contiguous(), scale.contiguous()


def quantize(w: torch.Tensor, fmt: int):
    """(packed, scales, global) of one [N, K] fp32 tensor in storage format ``fmt``."""
    if fmt == NVFP4:
        return quantize_nvfp4(w)
    if fmt == MXFP4:
        packed, sc = quantize_mxfp4(w)
        return packed, sc, None
    if fmt == FP8:
        codes, sc = quantize_fp8(w)
        return codes, sc, None
    if fmt == BF16:
        return w.to(torch.bfloat16).contiguous(), None, None
    raise ValueError(f"unknown weight format {fmt}")


def storage_shapes(fmt: int, n: int, k: int):
    """((packed shape, dtype), (scales shape, dtype) or None) of one expert's [n, k] matrix."""
    if fmt in (NVFP4, MXFP4):
        return ((n, k // 2), torch.uint8), ((n, k // (16 if fmt == NVFP4 else 32)), torch.uint8)
    if fmt == FP8:
        return ((n, k), torch.uint8), ((-(-n // FP8_BLOCK), -(-k // FP8_BLOCK)), torch.float32)
    if fmt == BF16:
        return ((n, k), torch.bfloat16), None
    raise ValueError(f"unknown weight format {fmt}")


# ---------------------------------------------------------------------------
# Layer inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Fp4Weight:
    """One projection of all experts of a group, in storage form (any weight format; the
    layout of each format is in the module doc)."""

    fmt: int
    packed: torch.Tensor          # FP4 uint8 [E, N, K/2]; FP8 uint8 [E, N, K]; BF16 [E, N, K]
    scales: Optional[torch.Tensor]  # FP4 uint8 [E, N, K/16|32]; FP8 f32 [E, N/128, K/128]
    global_scale: Optional[torch.Tensor]  # f32 [E] (NVFP4) or None
    n: int
    k: int

    @property
    def experts(self) -> int:
        return self.packed.shape[0]


@dataclasses.dataclass
class ExpertSet:
    gate: Fp4Weight
    up: Fp4Weight
    down: Fp4Weight


@dataclasses.dataclass
class LayerInputs:
    spec: LayerSpec
    x: torch.Tensor                 # bf16 [T, H]
    residual: torch.Tensor          # bf16 [T, H]
    router_w: torch.Tensor          # bf16 [E, H]
    logit_bias: Optional[torch.Tensor]       # f32 [E]
    correction_bias: Optional[torch.Tensor]  # f32 [E]
    gamma: Optional[torch.Tensor]   # bf16 [H]
    token_ids: Optional[torch.Tensor]  # int32 [T]
    tid2eid: Optional[torch.Tensor]    # int64 [V, k]
    routed: ExpertSet
    shared: Optional[ExpertSet]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(g, shape, std, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _expert_set(g, device, experts: int, hidden: int, inter: int, fmt: int) -> ExpertSet:
    """Draw gate [I,H], up [I,H], down [H,I] per expert (expert-major) ~ N(0, 0.02), then encode."""
    parts = {}
    for name, (n, k) in (("gate", (inter, hidden)), ("up", (inter, hidden)), ("down", (hidden, inter))):
        (pshape, pdt), sdesc = storage_shapes(fmt, n, k)
        parts[name] = (
            torch.empty((experts,) + pshape, dtype=pdt, device=device),
            torch.empty((experts,) + sdesc[0], dtype=sdesc[1], device=device) if sdesc else None,
            torch.empty((experts,), dtype=torch.float32, device=device) if fmt == NVFP4 else None,
            n, k)
    for e in range(experts):
        for name in ("gate", "up", "down"):
            packed, sc, gs, n, k = parts[name]
            w = _normal(g, (n, k), 0.02, device)
            p, s, gg = quantize(w, fmt)
            packed[e].copy_(p)
            if sc is not None:
                sc[e].copy_(s)
            if gs is not None:
                gs[e] = gg
            del w
    return ExpertSet(**{name: Fp4Weight(fmt, p, s, gs, n, k) for name, (p, s, gs, n, k) in parts.items()})


def zipf_logit_bias(g, experts: int, exponent: float, device) -> torch.Tensor:
    """Per-expert additive router-logit bias ln(r^-a / sum_r r^-a), r = 1 + a seeded permutation."""
    perm = torch.randperm(experts, generator=g, device=device)
    r = (perm + 1).to(torch.float64)
    w = r.pow(-exponent)
    return torch.log(w / w.sum()).to(torch.float32)


def make_inputs(spec: LayerSpec, device="cpu", seed: Optional[int] = None,
                tokens: Optional[int] = None) -> LayerInputs:
    """Draw every input of one layer call from ``seed`` (default: the workload's seed).

    Draw order: x, residual, router weight, logit bias, correction bias, routed
    experts (expert-major; gate, up, down), shared expert, RMSNorm gamma, token
    ids, hash table. ``tokens`` overrides the token count (the weights do not
    depend on it, so two token counts with one seed share their weights only if
    drawn on the same device in the same order: x and residual come first and
    change the stream, so weights are drawn from a second generator).
    """
    seed = spec.seed if seed is None else seed
    T = spec.tokens if tokens is None else tokens
    H, E, K, I = spec.hidden, spec.experts, spec.top_k, spec.inter
    ga = _gen(device, seed)            # activations and token ids
    gw = _gen(device, seed + 7919)     # weights, biases and tables (independent of T)

    x = torch.randn((T, H), generator=ga, device=device).to(torch.bfloat16)
    residual = torch.randn((T, H), generator=ga, device=device).to(torch.bfloat16)
    NE = E + spec.zero_experts  # router outputs
    router_w = _normal(gw, (NE, H), 0.02, device).to(torch.bfloat16)
    logit_bias = zipf_logit_bias(gw, NE, spec.zipf_bias, device) if spec.zipf_bias > 0 else None
    corr = None
    if spec.correction_bias:
        corr = (torch.rand((NE,), generator=gw, device=device) * 0.2 - 0.1).to(torch.float32)
    routed = _expert_set(gw, device, E, H, I, spec.fmt)
    shared = _expert_set(gw, device, 1, H, spec.shared_inter, spec.shared_fmt) if spec.shared else None
    gamma = None
    if spec.pre_norm:
        gamma = (1.0 + 0.1 * torch.randn((H,), generator=gw, device=device)).to(torch.bfloat16)
    token_ids = tid2eid = None
    if spec.select == HASH:
        token_ids = torch.randint(0, spec.vocab, (T,), generator=ga, device=device, dtype=torch.int64).to(torch.int32)
        keys = torch.rand((spec.vocab, E), generator=gw, device=device)
        tid2eid = keys.argsort(dim=1)[:, :K].to(torch.int64).contiguous()
        del keys
    return LayerInputs(spec=dataclasses.replace(spec, tokens=T), x=x, residual=residual,
                       router_w=router_w, logit_bias=logit_bias, correction_bias=corr,
                       gamma=gamma, token_ids=token_ids, tid2eid=tid2eid,
                       routed=routed, shared=shared)


@dataclasses.dataclass
class Activations:
    x: torch.Tensor                  # bf16 [T, H]
    residual: torch.Tensor           # bf16 [T, H]
    token_ids: Optional[torch.Tensor]  # int32 [T] (hash routing)


def make_activations(spec: LayerSpec, device="cpu", seed: int = 0,
                     tokens: Optional[int] = None) -> Activations:
    """Another batch of layer activations (x, residual, token ids) with the workload's
    distributions, drawn from its own seed; used to vary the input between benchmark steps."""
    T = spec.tokens if tokens is None else tokens
    g = _gen(device, seed)
    x = torch.randn((T, spec.hidden), generator=g, device=device).to(torch.bfloat16)
    residual = torch.randn((T, spec.hidden), generator=g, device=device).to(torch.bfloat16)
    token_ids = None
    if spec.select == HASH:
        token_ids = torch.randint(0, spec.vocab, (T,), generator=g, device=device,
                                  dtype=torch.int64).to(torch.int32)
    return Activations(x, residual, token_ids)


def random_codes_weight(g, device, experts: int, n: int, k: int, fmt: int,
                        scale_codes: Optional[torch.Tensor] = None) -> Fp4Weight:
    """A weight tensor with uniformly random codes and scales (edge-case tests).

    E4M3 scales avoid the NaN code 0x7F/0xFF; E8M0 scales are drawn around 2^0. FP8: random
    non-NaN E4M3 codes and fp32 block scales in [2^-8, 2^0); BF16: N(0, 1) values.
    """
    if fmt == FP8:
        codes = torch.randint(0, 254, (experts, n, k), generator=g, device=device, dtype=torch.int32)
        codes = codes + (codes >= 0x7F).to(torch.int32)  # skip 0x7F (NaN); 0xFF is out of range
        (_, _), ((nb, kb), _) = storage_shapes(FP8, n, k)
        sc = torch.exp2(-8.0 * torch.rand((experts, nb, kb), generator=g, device=device))
        return Fp4Weight(fmt, codes.to(torch.uint8).contiguous(), sc.to(torch.float32).contiguous(),
                         None, n, k)
    if fmt == BF16:
        v = torch.randn((experts, n, k), generator=g, device=device, dtype=torch.float32)
        return Fp4Weight(fmt, v.to(torch.bfloat16).contiguous(), None, None, n, k)
    packed = torch.randint(0, 256, (experts, n, k // 2), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    if fmt == NVFP4:
        sc = torch.randint(0, 0x7F, (experts, n, k // 16), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
        gs = torch.rand((experts,), generator=g, device=device, dtype=torch.float32) + 0.5
    else:
        sc = torch.randint(117, 134, (experts, n, k // 32), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
        gs = None
    if scale_codes is not None:
        sc = scale_codes
    return Fp4Weight(fmt, packed.contiguous(), sc.contiguous(), gs, n, k)


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Raw uint16 storage of a bf16 tensor (as int16 view)."""
    return t.contiguous().view(torch.int16)


def count_unique_experts(ids: torch.Tensor, experts: int) -> int:
    v = ids.reshape(-1)
    v = v[(v >= 0) & (v < experts)]
    return int(torch.unique(v).numel())


def nbytes_fp4(n: int, k: int, fmt: int) -> float:
    """Storage bytes of one [n, k] expert matrix including its scales (and global for NVFP4)."""
    if fmt == FP8:
        return n * k + 4 * (-(-n // FP8_BLOCK)) * (-(-k // FP8_BLOCK))
    if fmt == BF16:
        return 2 * n * k
    return n * k / 2 + n * k / (16 if fmt == NVFP4 else 32) + (4 if fmt == NVFP4 else 0)


__all__ = [name for name in dir() if not name.startswith("_")] + ["_e2m1_encode_magnitude", "_pack_codes"]
_ = math
