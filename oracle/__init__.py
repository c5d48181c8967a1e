"""CPU oracle of the FP4 mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package. The
product path (the HIP library and its Python binding) never does, and shares no
code, table or helper with it.

The oracle is a plain, slow, direct evaluation of what the layer computes,
written from the MoE module pages of the Rust inference engine
(spark_model/layers/moe/mod.rs: the module doc and the field docs of
``MoeLayer``; spark_model/layers/moe/init.rs: the constructor's validation and
kernel set) and from the public OCP Microscaling v1.0 element definitions for
E2M1, E4M3 and E8M0. Expert weights come as NVFP4 or MXFP4 (FP4 codes with block
scales), FP8 (E4M3 codes with one fp32 scale per 128 x 128 block) or BF16. Floating point is evaluated in fp64 (numpy), except where
a decision is taken on a value the method defines in fp32 (router logits and
the sigmoid selection key), which are rounded to fp32 exactly as defined.

Layer (for every token t, top-k slots j):
    x_e      = bf16(RMSNorm(x))      if a pre-expert norm is configured, else x
    logits   = fp32(x . W_r^T + logit_bias)               (router sees raw x)
    ids, w   = select(score(logits))    (softmax | sigmoid+bias | sqrt-softplus+bias |
                                         softmax+bias | hash)
    y_{t,j}  = W_d[e] . (SiLU(W_g[e] . x_e[t]) * (W_u[e] . x_e[t]))
               (or x_e[t] for a zero-computation expert, ids E..E+Z-1)
    out[t]   = residual[t] + sum_j w[t,j] * y_{t,j} + y_shared[t]

Every function below cites the passage it follows. Readings of points the
pages leave open are listed in the design notes of the repository.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

NVFP4 = 0
MXFP4 = 1
FP8 = 2    # E4M3 (OCP "FN") elements, one fp32 scale per 128 x 128 block (N x K)
BF16 = 3   # bf16 elements, no scale
FP8_BLOCK = 128
SOFTMAX = 0
SIGMOID = 1
SQRT_SOFTPLUS = 2
SOFTMAX_BIAS = 3
TOPK = 0
HASH = 1

# ---------------------------------------------------------------------------
# Element formats (OCP MX v1.0 section 5.3; NVFP4/MXFP4 composition from the
# MoE module page, doc of MoeLayer.experts_scale_kind)
# ---------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.

    Exponent field 0 is subnormal: m * 2^(1-1) * 0.5. No infinities or NaN.
    """
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = m * 0.5
    else:
        mag = (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if s else mag


def e4m3fn_value(byte: int) -> float:
    """Value of an FP8 E4M3 ("FN": finite, bias 7) code: max 448, NaN at S.1111.111, no inf."""
    s = (byte >> 7) & 1
    e = (byte >> 3) & 15
    m = byte & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (-6)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e8m0_value(byte: int) -> float:
    """Value of an E8M0 scale code: 2^(byte-127); 0xFF is NaN."""
    if byte == 255:
        return math.nan
    return 2.0 ** (byte - 127)


_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3 = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)
_E8M0 = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; element 2j is the low nibble of byte j."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequant_fp4(packed: np.ndarray, scales: np.ndarray, fmt: int,
                global_scale: Optional[float] = None) -> np.ndarray:
    """Decode one FP4 matrix [N, K/2] (+ scales) to fp64 [N, K].

    NVFP4: value = e2m1 * e4m3(scale of its 16-block along K) * global (f32 per tensor).
    MXFP4: value = e2m1 * e8m0(scale of its 32-block along K).
    (MoE module page: doc of MoeLayer.experts_scale_kind.)
    """
    codes = unpack_codes(packed)
    n, k = codes.shape
    vals = _E2M1[codes]
    if fmt == NVFP4:
        blk = 16
        sv = _E4M3[np.asarray(scales, dtype=np.uint8)]
    elif fmt == MXFP4:
        blk = 32
        sv = _E8M0[np.asarray(scales, dtype=np.uint8)]
    else:
        raise ValueError(f"unknown FP4 format {fmt}")
    if sv.shape != (n, k // blk):
        raise ValueError(f"scale shape {sv.shape} does not match [{n}, {k // blk}]")
    out = vals * np.repeat(sv, blk, axis=1)
    if fmt == NVFP4:
        if global_scale is None:
            raise ValueError("NVFP4 needs a global scale")
        out = out * float(np.float32(global_scale))
    return out


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 (the upper 16 bits of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode one FP8 expert matrix [N, K] (E4M3 codes) to fp64: value = e4m3(code) *
    scale[n // 128, k // 128], the fp32 scales [ceil(N/128), ceil(K/128)] of 128 x 128
    blocks (the FP8 expert weights and block-scaled FP8 GEMMs of the MoE constructor and
    module pages, e.g. the FP8 pointer tables and fp8_gemm_t_blockscaled)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    sv = np.asarray(scales, dtype=np.float32).astype(np.float64)
    nb, kb = -(-n // FP8_BLOCK), -(-k // FP8_BLOCK)
    if sv.shape != (nb, kb):
        raise ValueError(f"scale shape {sv.shape} does not match [{nb}, {kb}]")
    full = np.repeat(np.repeat(sv, FP8_BLOCK, axis=0), FP8_BLOCK, axis=1)[:n, :k]
    return _E4M3[codes] * full


def dequant_weight(packed: np.ndarray, scales, fmt: int,
                   global_scale: Optional[float] = None) -> np.ndarray:
    """Decode one expert matrix in any storage format to fp64 [N, K]: FP4 (packed
    [N, K/2]), FP8 (codes [N, K] + block scales) or BF16 (bits [N, K]; the pages' BF16
    grouped GEMM for FP8-source models dequantised to BF16 at load)."""
    if fmt in (NVFP4, MXFP4):
        return dequant_fp4(packed, scales, fmt, global_scale)
    if fmt == FP8:
        return dequant_fp8(packed, scales)
    if fmt == BF16:
        return bf16_value(packed)
    raise ValueError(f"unknown weight format {fmt}")


# ---------------------------------------------------------------------------
# Router (MoE constructor page: router GEMM kernels with fp32 output and the
# top-K kernels; MoE module page: doc of dense_gemm_f32out and of
# correction_bias_dev / tid2eid_dev)
# ---------------------------------------------------------------------------


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Pre-expert RMSNorm: x * rsqrt(mean(x^2) + eps) * gamma, in fp64.

    Applied to the expert input only; the router reads the raw x
    (MoE module page: doc of MoeLayer.pre_expert_norm).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def router_logits(x: np.ndarray, router_w: np.ndarray,
                  logit_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 logits = round_fp32(x . W_r^T (+ bias)); the dot product is exact-ish in fp64."""
    l = np.asarray(x, dtype=np.float64) @ np.asarray(router_w, dtype=np.float64).T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)
    return l.astype(np.float32)


def _rank_order(keys: np.ndarray) -> np.ndarray:
    """Expert indices of one token, best first: larger key first, lower index on ties,
    NaN after everything (ties among NaN by index). -0 and +0 compare equal."""
    e = keys.shape[0]
    idx = np.arange(e)
    isnan = np.isnan(keys)
    k64 = np.where(isnan, 0.0, keys.astype(np.float64)) + 0.0  # -0 -> +0
    # lexsort: last key is primary
    return np.lexsort((idx, -k64, isnan.astype(np.int8)))


def select_topk(keys: np.ndarray, k: int) -> np.ndarray:
    """ids [T, k] int32 of the k largest keys per row, ordered best first (lowest index wins ties)."""
    keys = np.asarray(keys, dtype=np.float32)
    return np.stack([_rank_order(row)[:k] for row in keys]).astype(np.int32)


def softmax(logits: np.ndarray) -> np.ndarray:
    """p = exp(l - max) / sum exp(l - max) over all experts, in fp64."""
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l, axis=-1, keepdims=True)
    z = np.exp(l - m)
    return z / np.sum(z, axis=-1, keepdims=True)


def sigmoid_key(logits: np.ndarray, correction_bias: Optional[np.ndarray]) -> np.ndarray:
    """Selection key of sigmoid routing: fp32(sigmoid(l)) + bias, the addition in fp32.

    sigmoid is evaluated in fp64 and rounded once to fp32, so the key is the
    correctly rounded value (with overwhelming probability) on any platform.
    """
    s = (1.0 / (1.0 + np.exp(-np.asarray(logits, dtype=np.float64)))).astype(np.float32)
    if correction_bias is None:
        return s
    return (s + np.asarray(correction_bias, dtype=np.float32)).astype(np.float32)


def sqrt_softplus(logits: np.ndarray) -> np.ndarray:
    """sqrt(softplus(l)) = sqrt(ln(1 + e^l)) in fp64 (softplus via logaddexp, no overflow).

    The sqrt-softplus routing score of the constructor page (the DeepSeek-V4 top-K
    kernels moe_topk_sqrtsoftplus / _batched) and of the MoE module page (field docs of
    the sqrtsoftplus routing kernels).
    """
    return np.sqrt(np.logaddexp(0.0, np.asarray(logits, dtype=np.float64)))


def sqrt_softplus_key(logits: np.ndarray, correction_bias: Optional[np.ndarray]) -> np.ndarray:
    """Selection key of sqrt-softplus routing: fp32(sqrt(softplus(l))) + bias, the
    addition in fp32 (the score evaluated in fp64 and rounded once, as for sigmoid)."""
    s = sqrt_softplus(logits).astype(np.float32)
    if correction_bias is None:
        return s
    return (s + np.asarray(correction_bias, dtype=np.float32)).astype(np.float32)


def scores(logits: np.ndarray, score: int) -> np.ndarray:
    """The routing weight of every expert before selection, fp64."""
    l = np.asarray(logits, dtype=np.float32)
    if score == SOFTMAX:
        return softmax(l)
    if score == SIGMOID:
        return 1.0 / (1.0 + np.exp(-l.astype(np.float64)))
    if score == SQRT_SOFTPLUS:
        return sqrt_softplus(l)
    if score == SOFTMAX_BIAS:
        return softmax(l)
    raise ValueError(f"unknown score mode {score}")


def softmax_bias_key(logits: np.ndarray, correction_bias: Optional[np.ndarray]) -> np.ndarray:
    """Selection key of softmax+bias routing: fp32(softmax probability) + bias, the
    addition in fp32 (the probability evaluated in fp64 and rounded once)."""
    s = softmax(logits).astype(np.float32)
    if correction_bias is None:
        return s
    return (s + np.asarray(correction_bias, dtype=np.float32)).astype(np.float32)


def route(logits: np.ndarray, top_k: int, score: int = SOFTMAX, select: int = TOPK,
          renormalize: bool = False, correction_bias: Optional[np.ndarray] = None,
          token_ids: Optional[np.ndarray] = None, tid2eid: Optional[np.ndarray] = None,
          routed_scaling: float = 1.0):
    """Scores + top-K selection -> (ids [T,k] int32, weights [T,k] fp64).

    softmax: key = logit, weight = softmax probability of the chosen expert.
    sigmoid: key = sigmoid(logit) + correction bias (selection only),
             weight = unbiased sigmoid (MoE module page: doc of correction_bias_dev,
             "DeepSeek-V3 / MiniMax-M2 style").
    sqrt-softplus: key = sqrt(softplus(logit)) + correction bias (selection only),
             weight = unbiased sqrt(softplus(logit)) (the DeepSeek-V4 routing kernels of
             the constructor page; the bias handled as for sigmoid).
    softmax+bias: key = softmax probability + correction bias (selection only), weight
             = the probability (the LongCat softmax+bias top-K kernels of the
             constructor page; their logit width num_experts + zero_expert_num).
    hash:    ids = tid2eid[token] (MoE module page: doc of tid2eid_dev), weight =
             the score (softmax probability, sigmoid or sqrt-softplus) at those ids;
             an out-of-range token id or table entry gives id -1 and weight 0.
    Optional renormalisation divides the chosen weights by their sum; the routed
    scaling factor multiplies them afterwards.
    """
    logits = np.asarray(logits, dtype=np.float32)
    t, e = logits.shape
    if select == HASH:
        if tid2eid is None or token_ids is None:
            raise ValueError("hash routing needs token_ids and tid2eid")
        tid2eid = np.asarray(tid2eid)
        p = scores(logits, score)
        ids = np.full((t, top_k), -1, dtype=np.int32)
        w = np.zeros((t, top_k), dtype=np.float64)
        for i in range(t):
            tok = int(token_ids[i])
            if not 0 <= tok < tid2eid.shape[0]:
                continue
            for j in range(top_k):
                ex = int(tid2eid[tok, j])
                if 0 <= ex < e:
                    ids[i, j] = ex
                    w[i, j] = p[i, ex]
    elif score == SOFTMAX:
        ids = select_topk(logits, top_k)
        p = softmax(logits)
        w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    elif score in (SIGMOID, SQRT_SOFTPLUS, SOFTMAX_BIAS):
        key = {SIGMOID: sigmoid_key, SQRT_SOFTPLUS: sqrt_softplus_key,
               SOFTMAX_BIAS: softmax_bias_key}[score]
        ids = select_topk(key(logits, correction_bias), top_k)
        w = np.take_along_axis(scores(logits, score), ids.astype(np.int64), axis=1)
    else:
        raise ValueError(f"unknown score mode {score}")
    if renormalize:
        tot = w.sum(axis=1, keepdims=True)
        w = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    return ids, w * float(routed_scaling)


# ---------------------------------------------------------------------------
# Experts (MoE module page: module doc "gate+up, silu+down"; doc of moe_act_mul,
# SiLU by default) and the blend into the residual (weighted-sum blend kernel)
# ---------------------------------------------------------------------------


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def expert_ffn(xe: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """y = W_d . (SiLU(W_g . x) * (W_u . x)) for rows of xe [R, H]; weights dequantised fp64."""
    g = xe @ wg.T
    u = xe @ wu.T
    return (silu(g) * u) @ wd.T


class DequantCache:
    """Dequantised fp64 expert matrices, decoded on first use (the full tensors of
    a large layer do not fit in host memory at once)."""

    def __init__(self, gate, up, down):
        self.parts = {"gate": gate, "up": up, "down": down}
        self.cache = {}

    def get(self, e: int):
        if e not in self.cache:
            out = []
            for name in ("gate", "up", "down"):
                fmt, packed, scales, gs = self.parts[name]
                out.append(dequant_weight(packed[e], None if scales is None else scales[e],
                                          fmt, None if gs is None else gs[e]))
            self.cache[e] = tuple(out)
        return self.cache[e]

    def drop(self, e: int):
        self.cache.pop(e, None)


def experts_forward(xe: np.ndarray, ids: np.ndarray, w: np.ndarray, routed: DequantCache,
                    residual: np.ndarray, shared: Optional[DequantCache] = None,
                    rows: Optional[np.ndarray] = None,
                    num_experts: Optional[int] = None, workers: int = 1) -> np.ndarray:
    """out[t] = residual[t] + sum_j w[t,j] y_{t,j} + y_shared[t] in fp64, for tokens ``rows``.

    The sum runs over slots j in order, then the shared expert (weight 1, own
    format, same normalised input), then the residual. Slots with id -1 are skipped.
    With ``num_experts`` = E given, ids E and above are zero-computation experts: their
    y is the expert input itself (the constructor page's zero-expert add kernel, which
    folds their weights into one identity contribution per token).

    ``workers`` > 1 evaluates the experts on that many host threads (decoding a large
    layer's weights dominates the time). Each expert's rows are computed exactly as in
    the serial loop and stored in their own slots, and the sums are formed afterwards in
    the same fixed order, so the result does not depend on ``workers``.
    """
    xe = np.asarray(xe, dtype=np.float64)
    t_all = xe.shape[0]
    rows = np.arange(t_all) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), xe.shape[1]), dtype=np.float64)
    # group (row, slot) pairs by expert so each expert is decoded once
    by_expert = {}
    for ri, t in enumerate(rows):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e >= 0:
                by_expert.setdefault(e, []).append((ri, t, j))
    contrib = np.zeros((len(rows), ids.shape[1], xe.shape[1]), dtype=np.float64)
    if num_experts is not None:
        for e in [e for e in by_expert if e >= num_experts]:
            for ri, t, j in by_expert.pop(e):
                contrib[ri, j] = w[t, j] * xe[t]
    def one_expert(e):
        wg, wu, wd = routed.get(e)
        lst = by_expert[e]
        ts = np.array([t for _, t, _ in lst])
        y = expert_ffn(xe[ts], wg, wu, wd)
        for (ri, t, j), yy in zip(lst, y):
            contrib[ri, j] = w[t, j] * yy
        routed.drop(e)

    if workers > 1:
        import concurrent.futures
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, sorted(by_expert)))
    else:
        for e in sorted(by_expert):
            one_expert(e)
    for j in range(ids.shape[1]):
        out += contrib[:, j]
    if shared is not None:
        wg, wu, wd = shared.get(0)
        out += expert_ffn(xe[rows], wg, wu, wd)
    out += np.asarray(residual, dtype=np.float64)[rows]
    return out


def layer_forward(x, residual, router_w, routed: DequantCache, top_k: int, *,
                  score=SOFTMAX, select=TOPK, renormalize=False, logit_bias=None,
                  correction_bias=None, token_ids=None, tid2eid=None, gamma=None,
                  norm_eps=1e-6, shared: Optional[DequantCache] = None,
                  routed_scaling=1.0, rows=None, logits=None, zero_experts=0, workers=1):
    """Whole layer -> (out fp64 [len(rows), H], logits fp32, ids, w).

    ``logits`` may be given to route from fixed fp32 logits (used by the
    routing-parity checks); otherwise they are computed from x. With zero_experts = Z
    the router has E + Z outputs and its last Z experts are zero-computation experts.
    """
    x = np.asarray(x, dtype=np.float64)
    if logits is None:
        logits = router_logits(x, router_w, logit_bias)
    ids, w = route(logits, top_k, score, select, renormalize, correction_bias,
                   token_ids, tid2eid, routed_scaling)
    # the experts' input is a bf16 activation [T, H] (the boundary passes it as bf16), so
    # the normalised input is rounded once to bf16 before the expert GEMMs
    xe = bf16_round_f64(rms_norm(x, gamma, norm_eps)) if gamma is not None else x
    num_experts = np.asarray(logits).shape[1] - zero_experts if zero_experts else None
    out = experts_forward(xe, ids, w, routed, residual, shared, rows, num_experts, workers)
    return out, logits, ids, w


def bf16_round_f64(v: np.ndarray) -> np.ndarray:
    """Round fp64 values directly to the nearest bf16 value (8 significant bits, ties to
    even), returned as fp64. Normal range only (the activations here are far from the
    bf16 subnormal range); zeros, infinities and NaN pass through."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)  # np.round: half to even
    return np.where(np.isfinite(v) & (v != 0), r, v)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even), returned as fp32 (fp64 input is first
    rounded to fp32)."""
    f = np.asarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(f)
    out = r.astype(np.uint32).view(np.float32)
    return np.where(nan, f, out)
