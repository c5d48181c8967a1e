"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: expert ids bit-exact on identical fp32 logits; router logits bit-exact (fp64
accumulation on both sides, one rounding); layer output within max-abs 2e-2 and
rel-L2 5e-3 of the fp64 oracle (before its bf16 rounding).
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
import mixture_experts_ffn_03_amd as M
import zlib

from gpu_cases import (W_RTOL, assert_layer_close, config_for, f32, oracle_cache, oracle_layer,
                       oracle_workers, run_layer)

pytestmark = pytest.mark.gpu

DEV = "cuda"
PATHS = [pytest.param(M.PATH_DECODE, id="decode"), pytest.param(M.PATH_PREFILL, id="prefill")]
PATH_VALUES = [M.PATH_DECODE, M.PATH_PREFILL]


def _sync():
    torch.cuda.synchronize()


def _announce(*a):
    print("case:", *a, flush=True)


# ----------------------------------------------------------------------------- dequant

def _all_codes_weight(fmt):
    """256 rows (one per scale code) x 32 codes (0..15 twice); every block of a row has
    that row's scale code, so each code meets each scale."""
    blk = 16 if fmt == S.NVFP4 else 32
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)
    row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    packed = torch.from_numpy(np.tile(row, (256, 1))[None]).to(DEV)
    sc = np.repeat(np.arange(256, dtype=np.uint8).reshape(256, 1), 32 // blk, axis=1)
    scales = torch.from_numpy(sc[None]).to(DEV)
    gs = torch.tensor([0.3711], dtype=torch.float32, device=DEV) if fmt == S.NVFP4 else None
    return S.Fp4Weight(fmt, packed.contiguous(), scales.contiguous(), gs, 256, 32)


@pytest.mark.parametrize("fmt", [S.NVFP4, S.MXFP4])
@pytest.mark.parametrize("path", PATHS)
def test_dequant_every_code_times_every_scale(fmt, path):
    _announce("dequant", fmt, path)
    w = _all_codes_weight(fmt)
    out = torch.full((256, w.k), -7.0, dtype=torch.float32, device=DEV)
    M.debug_dequant(M.fp4_weight(w), 0, path, out)
    _sync()
    got = out.cpu().numpy()
    want = O.dequant_fp4(w.packed[0].cpu().numpy(), w.scales[0].cpu().numpy(), fmt,
                         None if w.global_scale is None else float(w.global_scale[0]))
    want32 = want.astype(np.float32)
    nan = np.isnan(want32)
    bad = ~nan & ~((got == want32) & (np.signbit(got) == np.signbit(want32)))
    bad |= nan & ~np.isnan(got)
    if bad.any():
        r, c = np.argwhere(bad)[0]
        pytest.fail(f"{bad.sum()} mismatches, first at scale code {r} code {c % 16}: "
                    f"got {got[r, c]!r} want {want32[r, c]!r}")


def test_dequant_random_block_layout():
    g = torch.Generator(device=DEV).manual_seed(3)
    for fmt in (S.NVFP4, S.MXFP4):
        w = S.random_codes_weight(g, DEV, 3, 96, 512, fmt)
        for e in range(3):
            for path in PATH_VALUES:
                out = torch.empty((96, 512), dtype=torch.float32, device=DEV)
                M.debug_dequant(M.fp4_weight(w), e, path, out)
                _sync()
                want = O.dequant_fp4(w.packed[e].cpu().numpy(), w.scales[e].cpu().numpy(), fmt,
                                     None if w.global_scale is None else float(w.global_scale[e]))
                assert np.array_equal(out.cpu().numpy(), want.astype(np.float32)), (fmt, e, path)


def _fp8_expected(codes, scales, path):
    """Device dequant of FP8 per path: decode GEMV = fp32(bf16(e4m3) * scale) (the bf16 of
    an E4M3 value is exact); MFMA operand = bf16_rne(fp32(e4m3 * scale)). numpy's float32
    multiply is correctly rounded, like the device's."""
    v = O.dequant_fp8(codes, np.ones_like(scales)).astype(np.float32)
    sc = np.repeat(np.repeat(scales.astype(np.float32), 128, 0), 128, 1)[:codes.shape[0], :codes.shape[1]]
    prod = v * sc
    if path == M.PATH_DECODE:
        return prod
    return torch.from_numpy(prod).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("path", PATHS)
def test_dequant_fp8_every_code_times_block_scales(path):
    _announce("dequant fp8", path)
    # 256 rows x 256 codes: row r holds every E4M3 code rotated by r; 2 x 2 blocks with
    # power-of-two and other fp32 scales
    codes = (np.arange(256)[None, :] + np.arange(256)[:, None]).astype(np.uint8)
    scales = np.array([[1.0, 2.0 ** -7], [np.float32(0.3711), np.float32(1e-3)]], dtype=np.float32)
    w = S.Fp4Weight(S.FP8, torch.from_numpy(codes[None].copy()).to(DEV),
                    torch.from_numpy(scales[None].copy()).to(DEV), None, 256, 256)
    out = torch.full((256, 256), -7.0, dtype=torch.float32, device=DEV)
    M.debug_dequant(M.fp4_weight(w), 0, path, out)
    _sync()
    got = out.cpu().numpy()
    want = _fp8_expected(codes, scales, path)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_dequant_fp8_bf16_random_layout():
    g = torch.Generator(device=DEV).manual_seed(4)
    for fmt in (S.FP8, S.BF16):
        w = S.random_codes_weight(g, DEV, 3, 200, 384, fmt)  # ragged 128-row blocks
        for e in range(3):
            for path in PATH_VALUES:
                out = torch.empty((200, 384), dtype=torch.float32, device=DEV)
                M.debug_dequant(M.fp4_weight(w), e, path, out)
                _sync()
                if fmt == S.FP8:
                    want = _fp8_expected(w.packed[e].cpu().numpy(), w.scales[e].cpu().numpy(), path)
                else:
                    want = w.packed[e].float().cpu().numpy()
                assert np.array_equal(out.cpu().numpy(), want), (fmt, e, path)


# ----------------------------------------------------------------------------- routing

def _route_gpu(cfg, logits=None, inp=None, corr=None, bias=None, token_ids=None, tid2eid=None):
    T, K, E = cfg.tokens, cfg.top_k, cfg.num_experts
    ws = M.alloc_workspace(cfg, DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    lo = torch.empty((T, E), dtype=torch.float32, device=DEV)
    M.route(cfg, None if inp is None else inp.x, None if inp is None else inp.router_w, ids, w, ws,
            logit_bias=bias, correction_bias=corr, token_ids=token_ids, tid2eid=tid2eid,
            logits_in=logits, logits_out=lo if logits is None else None)
    _sync()
    return ids.cpu().numpy(), w.cpu().numpy(), lo.cpu().numpy()


ROUTING_CASES = {
    "softmax_e8_k2": dict(E=8, K=2, score=S.SOFTMAX, renorm=False),
    "softmax_e128_k8_renorm": dict(E=128, K=8, score=S.SOFTMAX, renorm=True),
    "sigmoid_bias_e256_k8": dict(E=256, K=8, score=S.SIGMOID, renorm=True, corr=True),
    "softmax_e64_k6": dict(E=64, K=6, score=S.SOFTMAX, renorm=False),
    "softmax_e1024_k32": dict(E=1024, K=32, score=S.SOFTMAX, renorm=True),
    "sigmoid_e32_k32": dict(E=32, K=32, score=S.SIGMOID, renorm=False),
    "sqrtsp_bias_e256_k8": dict(E=256, K=8, score=S.SQRT_SOFTPLUS, renorm=True, corr=True),
    "sqrtsp_e64_k6": dict(E=64, K=6, score=S.SQRT_SOFTPLUS, renorm=False),
    "softmax_bias_e96_k8": dict(E=96, K=8, score=S.SOFTMAX_BIAS, renorm=False, corr=True),
}


def _tie_logits(T, E, seed):
    g = torch.Generator().manual_seed(seed)
    l = torch.randn((T, E), generator=g)
    l[: T // 4] = torch.randint(-2, 3, (T // 4, E), generator=g).float()  # many exact ties
    if T >= 8:
        l[T // 4] = 0.5                                  # all equal
        l[T // 4 + 1, ::2] = -0.0                        # signed zeros against +0
        l[T // 4 + 1, 1::2] = 0.0
        l[T // 4 + 2, ::3] = float("-inf")
    return l.float()


@pytest.mark.parametrize("name", sorted(ROUTING_CASES))
def test_route_ids_bitexact_on_identical_logits(name):
    c = ROUTING_CASES[name]
    _announce("route", name)
    T, E, K = 67, c["E"], c["K"]
    logits = _tie_logits(T, E, seed=zlib.crc32(name.encode()) % 1000)
    corr = (torch.rand(E, generator=torch.Generator().manual_seed(1)) * 0.2 - 0.1) if c.get("corr") else None
    cfg = M.make_config(T, 256, E, K, 256, score_mode=c["score"], renormalize=c["renorm"])
    ids, w, _ = _route_gpu(cfg, logits=logits.to(DEV), corr=None if corr is None else corr.to(DEV))
    oid, ow = O.route(logits.numpy(), K, c["score"], O.TOPK, c["renorm"],
                      None if corr is None else corr.numpy())
    assert np.array_equal(ids, oid)
    assert np.allclose(w, ow, rtol=W_RTOL, atol=1e-7)


def test_route_nan_logits_rank_last():
    T, E, K = 4, 64, 8
    logits = torch.randn((T, E))
    logits[0, :10] = float("nan")
    logits[1, :] = float("nan")
    cfg = M.make_config(T, 256, E, K, 256)
    ids, _, _ = _route_gpu(cfg, logits=logits.to(DEV))
    assert np.array_equal(ids, O.route(logits.numpy(), K)[0])


@pytest.mark.parametrize("score", [S.SOFTMAX, S.SIGMOID, S.SQRT_SOFTPLUS])
def test_hash_routing_and_bad_ids(score):
    T, E, K, V = 9, 16, 3, 50
    g = torch.Generator().manual_seed(4)
    logits = torch.randn((T, E), generator=g)
    table = torch.stack([torch.randperm(E, generator=g)[:K] for _ in range(V)]).to(torch.int64)
    table[7, 1] = E + 3   # bad table entry
    table[8, 0] = -5
    tok = torch.randint(0, V, (T,), generator=g).to(torch.int32)
    tok[2] = 7
    tok[3] = V + 1        # bad token id
    tok[4] = 8
    cfg = M.make_config(T, 256, E, K, 256, score_mode=score, select_mode=M.SELECT_HASH,
                        renormalize=True, vocab=V)
    ids, w, _ = _route_gpu(cfg, logits=logits.to(DEV), token_ids=tok.to(DEV), tid2eid=table.to(DEV))
    oid, ow = O.route(logits.numpy(), K, score, O.HASH, True, token_ids=tok.numpy(),
                      tid2eid=table.numpy())
    assert np.array_equal(ids, oid)
    assert np.allclose(w, ow, rtol=W_RTOL, atol=1e-7)


@pytest.mark.parametrize("name", ["tiny", "qwen3_decode_t8", "dsv3_decode_t32",
                                  "prefill_zipf_t4096", "hash_mxfp4_t512"])
def test_router_logits_bitexact(name):
    _announce("router logits", name)
    spec = S.WORKLOADS[name]
    if name in ("prefill_zipf_t4096", "hash_mxfp4_t512", "dsv3_decode_t32"):
        spec = S.scaled(spec, inter=64, shared_inter=64 if spec.shared else 0)  # weights unused
    inp = S.make_inputs(spec, device=DEV)
    cfg = config_for(inp)
    ids, w, lo = _route_gpu(cfg, inp=inp, corr=inp.correction_bias, bias=inp.logit_bias,
                            token_ids=inp.token_ids, tid2eid=inp.tid2eid)
    want = O.router_logits(f32(inp.x), f32(inp.router_w), f32(inp.logit_bias))
    nbad = int((lo != want).sum())
    assert nbad == 0, f"{nbad} of {want.size} logits differ"
    oid, ow = O.route(want, spec.top_k, spec.score, spec.select, spec.renormalize,
                      f32(inp.correction_bias),
                      None if inp.token_ids is None else inp.token_ids.cpu().numpy(),
                      None if inp.tid2eid is None else inp.tid2eid.cpu().numpy())
    assert np.array_equal(ids, oid)
    assert np.allclose(w, ow, rtol=W_RTOL, atol=1e-7)


# ----------------------------------------------------------------------------- layer

SMALL = {
    "tiny": S.WORKLOADS["tiny"],
    "qwen3_decode_t1": S.WORKLOADS["qwen3_decode_t1"],
    "qwen3_decode_t8": S.WORKLOADS["qwen3_decode_t8"],
    # reduced shapes of the larger workloads: several tiles per expert and ragged tails
    "dsv3_mini": S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=13, hidden=1024, experts=64,
                          inter=256, shared_inter=192),
    "zipf_mini": S.scaled(S.WORKLOADS["prefill_zipf_t4096"], tokens=301, hidden=512, experts=16,
                          inter=192),
    "hash_mini": S.scaled(S.WORKLOADS["hash_mxfp4_t512"], tokens=77, hidden=512, experts=32,
                          inter=256, shared_inter=128, vocab=1000),
    # sqrt-softplus scoring (with the correction bias; and weighting a hash layer)
    "sqrtsp_mini": S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=13, hidden=1024, experts=64,
                            inter=256, shared_inter=192, score=S.SQRT_SOFTPLUS),
    "hash_sqrtsp_mini": S.scaled(S.WORKLOADS["hash_mxfp4_t512"], tokens=40, hidden=512,
                                 experts=32, inter=256, shared_inter=128, vocab=1000,
                                 score=S.SQRT_SOFTPLUS),
    # K a multiple of 64 but not of 128 at 32-row prefill tiles (64-code stages)
    "oddk_mini": S.LayerSpec(name="oddk_mini", tokens=9, hidden=320, experts=16, top_k=4,
                             inter=192, fmt=S.MXFP4, seed=1078),
    # many slots (T * k >= 8192: the two-launch multi-block dispatch) with Zipf-skewed loads
    "many_slots_mini": S.scaled(S.WORKLOADS["prefill_zipf_t4096"], tokens=1500, hidden=256,
                                experts=16, inter=128),
    # few slots (5 tokens x 8) with zero-computation experts
    "zero_experts_small": S.LayerSpec(name="zero_experts_small", tokens=5, hidden=512,
                                      experts=48, top_k=8, inter=256, fmt=S.NVFP4,
                                      score=S.SOFTMAX_BIAS, renormalize=False,
                                      correction_bias=True, zero_experts=16, seed=1079),
    # FP8 (E4M3, 128 x 128 block scales) and BF16 expert weights, with an NVFP4 or FP8
    # shared expert; shapes not multiples of 128 exercise partial scale blocks
    "fp8_mini": S.LayerSpec(name="fp8_mini", tokens=11, hidden=640, experts=32, top_k=4,
                            inter=320, fmt=S.FP8, score=S.SIGMOID, renormalize=True,
                            correction_bias=True, shared=True, shared_inter=192,
                            shared_fmt=S.NVFP4, seed=1081),
    "fp8_prefill_mini": S.LayerSpec(name="fp8_prefill_mini", tokens=300, hidden=512, experts=8,
                                    top_k=3, inter=384, fmt=S.FP8, shared=True,
                                    shared_inter=256, shared_fmt=S.FP8, seed=1082),
    "bf16_mini": S.LayerSpec(name="bf16_mini", tokens=400, hidden=384, experts=12, top_k=3,
                             inter=256, fmt=S.BF16, seed=1083),
    "bf16_shared_mini": S.LayerSpec(name="bf16_shared_mini", tokens=9, hidden=256, experts=16,
                                    top_k=4, inter=128, fmt=S.BF16, shared=True,
                                    shared_inter=192, shared_fmt=S.BF16, seed=1084),
    # the fused top-K + bitmap dispatch (at most 16 tokens, more than 16 slots): 32 slots per
    # token (8 bitmap words per expert, several tiles per expert); 256 experts with a shared
    # expert; a hash layer (token errors read from LDS); 3 tokens of the Qwen3-like layer
    "wide_k_fused": S.LayerSpec(name="wide_k_fused", tokens=16, hidden=512, experts=64,
                                top_k=32, inter=128, fmt=S.NVFP4, renormalize=True, seed=1085),
    "fused_256": S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=16, hidden=256, experts=256,
                          inter=128, shared_inter=128, fmt=S.MXFP4),
    "hash_fused": S.scaled(S.WORKLOADS["hash_mxfp4_t512"], tokens=12, hidden=512, experts=32,
                           inter=256, shared_inter=128, vocab=1000),
    "qwen3_t3": S.scaled(S.WORKLOADS["qwen3_decode_t8"], tokens=3),
    # one token with top-K over at most 128 experts: the selection and the dispatch inside
    # the gate+up kernel; with a shared expert (its row first) and with MXFP4 weights
    "t1_fused_shared": S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=1, hidden=1024,
                                experts=64, inter=256, shared_inter=192),
    "t1_fused_mxfp4": S.LayerSpec(name="t1_fused_mxfp4", tokens=1, hidden=512, experts=128,
                                  top_k=6, inter=256, fmt=S.MXFP4, renormalize=True, seed=1092),
    # the other scores through the one-token kernel, whose expert blocks select with the lean
    # form (keys and rounds only) while one wave writes the full routing: sqrt-softplus with
    # a correction bias over 96 experts (two keys per lane, the last 32 lanes padding), and
    # softmax+bias over 40 experts (one key per lane), with no zero-computation experts
    "t1_fused_sqrtsp": S.LayerSpec(name="t1_fused_sqrtsp", tokens=1, hidden=512, experts=96,
                                   top_k=4, inter=256, fmt=S.NVFP4, score=S.SQRT_SOFTPLUS,
                                   renormalize=True, correction_bias=True, seed=1095),
    "t1_fused_softmax_bias": S.LayerSpec(name="t1_fused_softmax_bias", tokens=1, hidden=512,
                                         experts=40, top_k=5, inter=128, fmt=S.MXFP4,
                                         score=S.SOFTMAX_BIAS, correction_bias=True, seed=1096),
    # 40 tokens on the decode path: the shared expert's implicit list of ten 4-token tiles
    "dsv3_t40_mini": S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=40, hidden=1024,
                              experts=64, inter=256, shared_inter=192),
    # a shared expert of the routed format and sizes: multi-step decode gate+up at hidden
    # 2304 with a ragged last shared tile; one-step kernels with MXFP4 everywhere and ten
    # shared tiles
    "shared_merged_nv": S.LayerSpec(name="shared_merged_nv", tokens=13, hidden=2304,
                                    experts=32, top_k=4, inter=256, fmt=S.NVFP4,
                                    score=S.SIGMOID, renormalize=True, correction_bias=True,
                                    shared=True, shared_inter=256, shared_fmt=S.NVFP4,
                                    seed=1088),
    "shared_merged_mx": S.LayerSpec(name="shared_merged_mx", tokens=40, hidden=1024,
                                    experts=64, top_k=6, inter=192, fmt=S.MXFP4,
                                    score=S.SOFTMAX, renormalize=False, shared=True,
                                    shared_inter=192, shared_fmt=S.MXFP4, seed=1089),
    # MXFP4 at 32-row tiles with K a multiple of 512 (256-code stages, gate and up paired
    # across waves): routed experts on the dispatch's tile list, and a shared expert of few
    # tokens whose K is split over blocks (the split sums of the paired columns)
    "mx_k256_split": S.LayerSpec(name="mx_k256_split", tokens=20, hidden=4096, experts=8,
                                 top_k=2, inter=128, fmt=S.MXFP4, renormalize=True,
                                 shared=True, shared_inter=128, shared_fmt=S.MXFP4, seed=1093),
    # the same with NVFP4 (eight E4M3 scale bytes per lane half and stage): routed gate+up
    # over 16 stages, down over a single stage, a split-K shared expert
    "nv_k256_split": S.LayerSpec(name="nv_k256_split", tokens=20, hidden=4096, experts=8,
                                 top_k=2, inter=256, fmt=S.NVFP4, renormalize=True,
                                 shared=True, shared_inter=256, shared_fmt=S.NVFP4, seed=1094),
    # the library's limits, 1024 experts and 32 slots per token: 96 slots (the bitmap
    # dispatch, two words per expert) and 1280 slots (the block counting sort)
    "max_e1024_k32_t3": S.LayerSpec(name="max_e1024_k32_t3", tokens=3, hidden=256,
                                    experts=1024, top_k=32, inter=64, fmt=S.NVFP4,
                                    renormalize=True, seed=1086),
    "max_e1024_k32_t40": S.LayerSpec(name="max_e1024_k32_t40", tokens=40, hidden=256,
                                     experts=1024, top_k=32, inter=64, fmt=S.MXFP4,
                                     renormalize=False, seed=1087),
    # softmax+bias routing over 48 + 16 zero-computation experts (identity contributions)
    "zero_experts_mini": S.LayerSpec(name="zero_experts_mini", tokens=23, hidden=512,
                                     experts=48, top_k=8, inter=256, fmt=S.NVFP4,
                                     score=S.SOFTMAX_BIAS, renormalize=False,
                                     correction_bias=True, zero_experts=16, seed=1077),
}


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_parity_small(name, path):
    _announce("layer", name, path)
    inp = S.make_inputs(SMALL[name], device=DEV)
    out, logits, ids, w, ws = run_layer(inp, path=path)
    _sync()
    assert M.get_device_error(ws) == 0
    want, ologits, oids, ow = oracle_layer(inp)
    assert np.array_equal(logits.cpu().numpy(), ologits)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=W_RTOL, atol=1e-7)
    assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), f"{name}/{path}")


@pytest.mark.parametrize("path", PATHS)
def test_layer_without_residual_and_experts_entry(path):
    inp = S.make_inputs(SMALL["dsv3_mini"], device=DEV)
    out, logits, ids, w, ws = run_layer(inp, path=path, residual=False)
    want, _, _, _ = oracle_layer(inp, residual=False)
    assert_layer_close(out.float().cpu().numpy(), want, None, f"no-residual/{path}")
    # moe_experts_forward on the same routing and the normalised input equals the layer
    cfg = config_for(inp, path)
    out2 = torch.empty_like(out)
    M.experts_forward(cfg, inp.x, ids, w, M.expert_weights(inp.routed),
                      M.expert_weights(inp.shared), None, out2, ws)
    _sync()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("tokens", [1, 2, 4, 16])
def test_qwen3_shape_small_batches_and_experts_entry(tokens):
    """Qwen3-like decode layer at 1, 2, 4 and 16 tokens against the oracle; then
    moe_experts_forward builds its own dispatch from the ids in memory (the standalone
    dispatch kernel) where the layer's fused top-K built it from ids in LDS: same rows,
    same tiles, bit-identical outputs."""
    _announce("qwen3 shape", tokens)
    inp = S.make_inputs(S.scaled(SMALL["qwen3_decode_t8"], tokens=tokens), device=DEV)
    out, logits, ids, w, ws = run_layer(inp, path=M.PATH_DECODE, residual=False)
    _sync()
    assert M.get_device_error(ws) == 0
    want, ologits, oids, ow = oracle_layer(inp, residual=False)
    assert np.array_equal(logits.cpu().numpy(), ologits)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=W_RTOL, atol=1e-7)
    assert_layer_close(out.float().cpu().numpy(), want, None, f"qwen3 T={tokens}")
    cfg = config_for(inp, M.PATH_DECODE)
    out2 = torch.empty_like(out)
    M.experts_forward(cfg, inp.x, ids, w, M.expert_weights(inp.routed), None, None, out2, ws)
    _sync()
    assert M.get_device_error(ws) == 0
    assert torch.equal(out, out2)


def test_decode_long_rows_growing_lds():
    """Decode rows longer than 64 KB of staged activations, first hidden 10240 (80 KB of
    LDS) then 16384 (128 KB) on the same kernel instantiation: the second launch needs
    more LDS than the first and must still run (the kernel's limit is raised to the
    library's maximum, not to the first size seen)."""
    for hidden in (10240, 16384):
        _announce("decode long rows", hidden)
        spec = S.LayerSpec(name=f"long_rows_{hidden}", tokens=3, hidden=hidden, experts=4,
                           top_k=2, inter=64, fmt=S.NVFP4, seed=1091)
        inp = S.make_inputs(spec, device=DEV)
        out, logits, ids, w, ws = run_layer(inp, path=M.PATH_DECODE)
        _sync()
        assert M.get_device_error(ws) == 0
        want, ologits, oids, ow = oracle_layer(inp)
        assert np.array_equal(ids.cpu().numpy(), oids)
        assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), f"H={hidden}")


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_and_in_place(path):
    inp = S.make_inputs(SMALL["zipf_mini"], device=DEV)
    a = run_layer(inp, path=path)[0]
    b = run_layer(inp, path=path)[0]
    _sync()
    assert torch.equal(a, b)
    # out may alias the residual
    cfg = config_for(inp, path)
    ws = M.alloc_workspace(cfg, DEV)
    res = inp.residual.clone()
    M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), res, ws,
                    logit_bias=inp.logit_bias, residual=res)
    _sync()
    assert torch.equal(res, a)


@pytest.mark.parametrize("fmt", [S.NVFP4, S.MXFP4])
def test_prefill_partly_filled_tiles(fmt):
    """Expert row counts around the 32-row blocks of a 128-row prefill tile (1, 32, 33,
    64, 65, 96, 97, 127 rows in an expert's last tile, and an expert with no rows), so that
    the waves of a tile skip none, some or all of their row blocks."""
    counts = [129, 32, 33, 64, 65, 97, 127, 349, 0]  # 896 rows over 9 experts: 128-row tiles
    T, k = sum(counts) // 2, 2
    spec = S.LayerSpec(name="partial_tiles", tokens=T, hidden=512, experts=len(counts),
                       top_k=k, inter=192, fmt=fmt, seed=1090 + fmt)
    inp = S.make_inputs(spec, device=DEV)
    labels = np.repeat(np.arange(len(counts)), counts)
    oids = np.stack([labels[:T], labels[T:]], axis=1).astype(np.int32)  # distinct per token
    assert (oids[:, 0] != oids[:, 1]).all()
    rng = np.random.default_rng(7)
    ow = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    cfg = config_for(inp, M.PATH_PREFILL)
    ws = M.alloc_workspace(cfg, DEV)
    out = torch.empty_like(inp.x)
    M.experts_forward(cfg, inp.x, torch.from_numpy(oids).to(DEV), torch.from_numpy(ow).to(DEV),
                      M.expert_weights(inp.routed), None, inp.residual, out, ws)
    _sync()
    assert M.get_device_error(ws) == 0
    want = O.experts_forward(f32(inp.x), oids, ow.astype(np.float64),
                             oracle_cache(inp.routed), f32(inp.residual))
    assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), "partial-tiles")


def _distinct_pairs(T, E, rng):
    """[T, 2] expert ids, two distinct experts per token, Zipf-like expert popularity."""
    pop = 1.0 / np.arange(1, E + 1) ** 0.8
    pop /= pop.sum()
    first = rng.choice(E, size=T, p=pop)
    second = (first + 1 + rng.choice(E - 1, size=T)) % E
    return np.stack([first, second], axis=1).astype(np.int32)


@pytest.mark.parametrize("fmt", [S.NVFP4, S.MXFP4])
@pytest.mark.parametrize("shape", ["mt128", "mt64", "mt32_5stages"])
def test_prefill_persistent_down(fmt, shape):
    """Down projections on the persistent grid: more (row tile, column tile) items at
    hidden 4096 than the chip has block slots, so blocks claim further tiles from their
    XCD's counter and run the stage ring on from tile to tile, with ragged last tiles.
    Tile heights 128, 64 and 32 (the 32-row case with 5 stages of 128 codes, the fewest
    the persistent form takes)."""
    E, I, T = {"mt128": (8, 512, 2074), "mt64": (64, 512, 2048),
               "mt32_5stages": (128, 640, 2048)}[shape]
    _announce("persistent down", shape, fmt)
    spec = S.LayerSpec(name=f"persist_{shape}", tokens=T, hidden=4096, experts=E, top_k=2,
                       inter=I, fmt=fmt, seed=1200 + fmt)
    inp = S.make_inputs(spec, device=DEV)
    rng = np.random.default_rng(11)
    if shape == "mt128":
        counts = [2049, 1101, 513, 257, 129, 65, 33, 1]  # ragged last tiles, 39 tiles
        labels = np.repeat(np.arange(E), counts)
        oids = np.stack([labels[:T], labels[T:]], axis=1).astype(np.int32)
    else:
        oids = _distinct_pairs(T, E, rng)
    assert (oids[:, 0] != oids[:, 1]).all()
    ow = rng.uniform(0.1, 1.0, size=(T, 2)).astype(np.float32)
    # the launch is persistent: column tiles x tile bound above the resident slots
    mt = 128 if shape == "mt128" else (64 if shape == "mt64" else 32)
    tiles = sum(-(-int(c) // mt) for c in np.bincount(oids.ravel(), minlength=E))
    slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    assert (4096 // 256) * tiles > slots, (tiles, slots)
    cfg = config_for(inp, M.PATH_PREFILL)
    ws = M.alloc_workspace(cfg, DEV)
    out = torch.empty_like(inp.x)
    M.experts_forward(cfg, inp.x, torch.from_numpy(oids).to(DEV), torch.from_numpy(ow).to(DEV),
                      M.expert_weights(inp.routed), None, inp.residual, out, ws)
    _sync()
    assert M.get_device_error(ws) == 0
    want = O.experts_forward(f32(inp.x), oids, ow.astype(np.float64),
                             oracle_cache(inp.routed), f32(inp.residual),
                             workers=oracle_workers())
    assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), f"persist-{shape}")
    # a second call on the same workspace: the counters start again from zero
    out2 = torch.empty_like(out)
    M.experts_forward(cfg, inp.x, torch.from_numpy(oids).to(DEV), torch.from_numpy(ow).to(DEV),
                      M.expert_weights(inp.routed), None, inp.residual, out2, ws)
    _sync()
    assert torch.equal(out, out2)


def test_prefill_expert_output_range_is_flagged():
    """Routed prefill expert outputs are stored as fp16 between the down projection and the
    blend: an output that rounds past +-65504 saturates there and sets MOE_DEVERR_Y_RANGE
    (ordinary outputs set nothing)."""
    spec = S.LayerSpec(name="y_range", tokens=256, hidden=512, experts=8, top_k=2, inter=256,
                       fmt=S.NVFP4, seed=1400)
    inp = S.make_inputs(spec, device=DEV)
    cfg = config_for(inp, M.PATH_PREFILL)
    ws = M.alloc_workspace(cfg, DEV)
    out = torch.empty_like(inp.x)
    M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out, ws,
                    residual=inp.residual)
    assert M.get_device_error(ws) == 0
    inp.routed.down.global_scale.mul_(1e9)  # NVFP4 tensor scale: every expert output huge
    M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out, ws,
                    residual=inp.residual)
    assert M.get_device_error(ws) & M.DEVERR_Y_RANGE
    assert torch.isfinite(out.float()).all()  # saturated, not inf


def spec_e(inp):
    return inp.spec.experts


def test_bad_expert_ids_are_dropped_and_flagged():
    inp = S.make_inputs(SMALL["tiny"], device=DEV)
    cfg = config_for(inp, M.PATH_DECODE)
    ws = M.alloc_workspace(cfg, DEV)
    ids = torch.tensor([[0, 1], [9, 2], [-1, 3], [4, 5]], dtype=torch.int32, device=DEV)
    w = torch.full((4, 2), 0.5, dtype=torch.float32, device=DEV)
    out = torch.empty_like(inp.x)
    M.experts_forward(cfg, inp.x, ids, w, M.expert_weights(inp.routed), None, inp.residual, out, ws)
    assert M.get_device_error(ws) & M.DEVERR_EXPERT_ID
    oids = ids.cpu().numpy()
    oids = np.where((oids >= 0) & (oids < spec_e(inp)), oids, -1)  # dropped slots
    want = O.experts_forward(f32(inp.x), oids, w.cpu().numpy().astype(np.float64),
                             oracle_cache(inp.routed), f32(inp.residual))
    assert_layer_close(out.float().cpu().numpy(), want, None, "bad-ids")


@pytest.mark.parametrize("fmt", [S.NVFP4, S.MXFP4])
@pytest.mark.parametrize("tokens", [1, 2, 3])
def test_one_token_blend_inside_down(fmt, tokens):
    """A few tokens without a shared expert: the down kernel blends the slots itself (at three
    tokens some of its waves take two tiles). Slots of routed experts (one repeated within a
    token and across tokens), zero-computation experts and out-of-range ids (dropped,
    flagged), against the oracle; with and without a residual."""
    E, Z = 16, 4
    spec = S.LayerSpec(name="t1_blend", tokens=tokens, hidden=1024, experts=E, top_k=7,
                       inter=512, fmt=fmt, zero_experts=Z, seed=1300 + fmt)
    inp = S.make_inputs(spec, device=DEV)
    rows = [[3, E + 1, 5, 99, 0, E, 3], [7, 3, E + 2, 1, -4, 2, 5],
            [9, 11, 13, 3, E + 3, 15, 8]][:tokens]
    ws_ = [[0.3, 0.2, 0.15, 0.1, 0.1, 0.1, 0.05], [0.25, 0.2, 0.2, 0.15, 0.1, 0.06, 0.04],
           [0.2, 0.2, 0.15, 0.15, 0.1, 0.1, 0.1]][:tokens]
    ids = torch.tensor(rows, dtype=torch.int32, device=DEV)
    w = torch.tensor(ws_, dtype=torch.float32, device=DEV)
    cfg = config_for(inp, M.PATH_DECODE)
    ws = M.alloc_workspace(cfg, DEV)
    oids = ids.cpu().numpy()
    oids = np.where((oids >= 0) & (oids < E + Z), oids, -1)
    for residual in (inp.residual, None):
        _announce("one-token blend", fmt, residual is not None)
        out = torch.empty_like(inp.x)
        M.experts_forward(cfg, inp.x, ids, w, M.expert_weights(inp.routed), None, residual, out, ws)
        assert M.get_device_error(ws) & M.DEVERR_EXPERT_ID
        res = f32(residual) if residual is not None else np.zeros_like(f32(inp.x))
        want = O.experts_forward(f32(inp.x), oids, w.cpu().numpy().astype(np.float64),
                                 oracle_cache(inp.routed), res, num_experts=E)
        assert_layer_close(out.float().cpu().numpy(), want, None, "one-token blend")


HASH_GATHER = {
    "hash_mini": SMALL["hash_mini"],
    "hash_sqrtsp_mini": SMALL["hash_sqrtsp_mini"],
    "hash_sigmoid_mini": S.scaled(S.WORKLOADS["hash_mxfp4_t512"], tokens=50, hidden=512,
                                  experts=32, inter=256, shared_inter=128, vocab=1000,
                                  score=S.SIGMOID, renormalize=False, seed=1098),
    "hash_mxfp4_t512": S.WORKLOADS["hash_mxfp4_t512"],
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(HASH_GATHER))
def test_hash_layer_without_logits(name):
    """A hash-routed layer called without a logits output: its weights need only the k
    selected experts' logits (renormalised softmax, sigmoid, sqrt-softplus), so no router GEMM
    runs and the routing kernel forms just those dot products. Ids bit-exact, weights within
    the weight tolerance and the layer output within the bar, against the oracle."""
    _announce("hash without logits", name)
    inp = S.make_inputs(HASH_GATHER[name], device=DEV)
    cfg = config_for(inp)
    T, K, H = inp.spec.tokens, inp.spec.top_k, inp.spec.hidden
    ws = M.alloc_workspace(cfg, DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out, ws,
                    norm_gamma=inp.gamma, logit_bias=inp.logit_bias,
                    correction_bias=inp.correction_bias, token_ids=inp.token_ids,
                    tid2eid=inp.tid2eid,
                    shared=M.expert_weights(inp.shared) if inp.shared is not None else None,
                    residual=inp.residual, dbg_ids=ids, dbg_w=w)
    _sync()
    assert M.get_device_error(ws) == 0
    want, _, oids, ow = oracle_layer(inp, workers=oracle_workers())
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=W_RTOL, atol=1e-7)
    assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), name)


def test_hash_layer_without_logits_bad_ids():
    """The gathered-logit hash routing with an out-of-range token id and an out-of-range table
    entry: the token's slots and the bad entry's slot are dropped (id -1, weight 0), both error
    bits are set, and the other slots and the output match the oracle."""
    spec = SMALL["hash_mini"]
    inp = S.make_inputs(spec, device=DEV)
    inp.token_ids[5] = spec.vocab + 9
    row = int(inp.token_ids[11])
    inp.tid2eid[row, 2] = spec.experts + 40
    _announce("hash without logits, bad ids")
    cfg = config_for(inp)
    T, K, H = spec.tokens, spec.top_k, spec.hidden
    ws = M.alloc_workspace(cfg, DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out, ws,
                    norm_gamma=inp.gamma, correction_bias=inp.correction_bias,
                    token_ids=inp.token_ids, tid2eid=inp.tid2eid,
                    shared=M.expert_weights(inp.shared), residual=inp.residual, dbg_ids=ids,
                    dbg_w=w)
    _sync()
    err = M.get_device_error(ws)
    assert err & M.DEVERR_TOKEN_ID and err & M.DEVERR_TABLE
    got = ids.cpu().numpy()
    assert (got[5] == -1).all() and got[11, 2] == -1
    want, _, oids, ow = oracle_layer(inp)
    assert np.array_equal(got, oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=W_RTOL, atol=1e-7)
    assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), "hash bad ids")


@pytest.mark.parametrize("score", [S.SOFTMAX, S.SIGMOID])
def test_one_token_fused_topk_ties(score):
    """One token through the gate+up kernel that selects its own experts (a writer wave with
    the full top-K, and in each expert block a lean selection of the expert of its rank),
    with tied router logits: three experts share one router row and eight have a zero row
    (logit 0), so the top-k boundary falls inside tied groups. The ids, weights and layer
    output match the oracle's lowest-index tie-break."""
    spec = S.LayerSpec(name="t1_ties", tokens=1, hidden=512, experts=64, top_k=6, inter=256,
                       fmt=S.NVFP4, score=score, renormalize=True, seed=1097)
    inp = S.make_inputs(spec, device=DEV)
    rw = inp.router_w.clone()
    lg = (inp.x.float() @ rw.float().t())[0]
    best = int(torch.argmax(lg))
    assert float(lg[best]) > 0.0
    # the strongest row copied to two more experts; eight zero rows (logit exactly 0); every
    # other row the negated strongest one (logit exactly minus the top one)
    top = [best, (best + 17) % 64, (best + 33) % 64]
    rest = [e for e in range(64) if e not in top]
    zero = rest[20:28]
    neg = [e for e in rest if e not in zero]
    for e in top[1:]:
        rw[e] = rw[best]
    rw[zero] = 0
    rw[neg] = -rw[best]
    inp = dataclasses.replace(inp, router_w=rw)
    _announce("one-token ties", score)
    out, logits, ids, w, ws = run_layer(inp, path=M.PATH_DECODE)
    _sync()
    assert M.get_device_error(ws) == 0
    want, ologits, oids, ow = oracle_layer(inp)
    assert np.array_equal(logits.cpu().numpy(), ologits)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=W_RTOL, atol=1e-7)
    assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), "one-token ties")


def test_bad_expert_ids_many_slots():
    """Out-of-range ids among 9000 slots (multi-block dispatch): dropped, flagged, and the
    other slots still match the oracle."""
    spec = S.scaled(S.WORKLOADS["prefill_zipf_t4096"], tokens=1500, hidden=256, experts=16,
                    inter=128)
    inp = S.make_inputs(spec, device=DEV)
    rng = np.random.default_rng(11)
    T, k, E = spec.tokens, spec.top_k, spec.experts
    oids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    oids[7, 2] = E + 3
    oids[1400, 0] = -5
    ow = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    cfg = config_for(inp, M.PATH_PREFILL)
    ws = M.alloc_workspace(cfg, DEV)
    out = torch.empty_like(inp.x)
    M.experts_forward(cfg, inp.x, torch.from_numpy(oids).to(DEV), torch.from_numpy(ow).to(DEV),
                      M.expert_weights(inp.routed), None, inp.residual, out, ws)
    assert M.get_device_error(ws) & M.DEVERR_EXPERT_ID
    dropped = np.where((oids >= 0) & (oids < E), oids, -1)
    want = O.experts_forward(f32(inp.x), dropped, ow.astype(np.float64),
                             oracle_cache(inp.routed), f32(inp.residual))
    assert_layer_close(out.float().cpu().numpy(), want, None, "bad-ids-many")


# 77 tokens: top-K and dispatch launches; 6 and 2 tokens (36 and 12 slots): the fused
# kernel's bitmap dispatch
@pytest.mark.parametrize("tokens", [77, 6, 2])
def test_hash_layer_bad_token_flags_error(tokens):
    spec = S.scaled(SMALL["hash_mini"], tokens=tokens)
    inp = S.make_inputs(spec, device=DEV)
    bad = min(3, tokens - 1)
    inp.token_ids[bad] = spec.vocab + 5
    out, _, ids, _, ws = run_layer(inp, path=M.PATH_DECODE)
    err = M.get_device_error(ws)
    assert err & M.DEVERR_TOKEN_ID and not err & M.DEVERR_EXPERT_ID
    assert (ids[bad] == -1).all()
    want, _, _, _ = oracle_layer(inp)
    assert_layer_close(out.float().cpu().numpy(), want, None, "bad-token")


@pytest.mark.parametrize("tokens", [12, 2, 77])
def test_hash_layer_repeated_experts(tokens):
    """A hash table may name one expert twice for a token: both slots get their own row (in
    slot order) and weight, on every dispatch size."""
    _announce("hash repeated experts", tokens)
    spec = S.scaled(SMALL["hash_mini"], tokens=tokens)
    inp = S.make_inputs(spec, device=DEV)
    inp.tid2eid[:, 1] = inp.tid2eid[:, 0]
    inp.tid2eid[1::3, 5] = inp.tid2eid[1::3, 2]
    for path in PATH_VALUES:
        out, _, ids, w, ws = run_layer(inp, path=path)
        _sync()
        assert M.get_device_error(ws) == 0
        want, _, oids, ow = oracle_layer(inp)
        assert np.array_equal(ids.cpu().numpy(), oids)
        assert (oids[:, 0] == oids[:, 1]).any()
        assert np.allclose(w.cpu().numpy(), ow, rtol=W_RTOL, atol=1e-7)
        assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual),
                           f"hash-repeat/{tokens}/{path}")


def test_zero_tokens_is_a_noop():
    spec = S.scaled(SMALL["tiny"], tokens=0)
    inp = S.make_inputs(spec, device=DEV)
    out, *_ = run_layer(inp)
    _sync()
    assert out.shape == (0, spec.hidden)


def test_k_equals_e_dense_mixture():
    spec = S.scaled(SMALL["tiny"], tokens=5, experts=4, top_k=4)
    inp = S.make_inputs(spec, device=DEV)
    for path in PATH_VALUES:
        out = run_layer(inp, path=path)[0]
        want, *_ = oracle_layer(inp)
        assert_layer_close(out.float().cpu().numpy(), want, None, f"k=E/{path}")


# ----------------------------------------------------------------------------- full size

FULL = ["qwen3_decode_t1", "qwen3_decode_t8", "dsv3_decode_t32", "prefill_zipf_t4096",
        "hash_mxfp4_t512"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_layer_parity_full_size(name):
    """The workloads at their real sizes, in the launch configuration the benchmark uses
    (automatic path), every token against the oracle (its experts evaluated on several host
    threads). The printed line gives the raw max-abs error, the error beyond the output's
    own bf16 rounding (the bar) and the rel-L2 errors."""
    _announce("full", name)
    inp = S.make_inputs(S.WORKLOADS[name], device=DEV)
    out, logits, ids, w, ws = run_layer(inp)
    _sync()
    assert M.get_device_error(ws) == 0
    want, ologits, oids, ow = oracle_layer(inp, workers=oracle_workers())
    assert np.array_equal(logits.cpu().numpy(), ologits)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.allclose(w.cpu().numpy(), ow, rtol=W_RTOL, atol=1e-7)
    assert_layer_close(out.float().cpu().numpy(), want, f32(inp.residual), name)
