"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties one part of the oracle to something it cannot agree with by
construction: format tables from the OCP specifications (tests/golden), an
independent decoder (torch's float8 dtypes), library routines (torch softmax,
sigmoid, topk, silu, rms_norm, math.fsum), closed forms and special cases of the
method (k = E dense mixture, one-hot routing, zero-bias sigmoid = softmax
ranking, hash = softmax routing, exact power-of-two scaling), and brute-force
property checks on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import moe_synth as S
from conftest import read_golden


# ---------------------------------------------------------------- formats

def test_e2m1_table_matches_ocp():
    rows = read_golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = O.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_all_codes_match_torch_and_spec():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3fn_value(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    for code, val in read_golden("e4m3_spot_values.txt"):
        g = O.e4m3fn_value(code)
        assert (math.isnan(g) and math.isnan(val)) or g == val, hex(code)


def test_e8m0_all_codes_match_torch_and_spec():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([O.e8m0_value(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    for code, val in read_golden("e8m0_spot_values.txt"):
        g = O.e8m0_value(code)
        assert (math.isnan(g) and math.isnan(val)) or g == val, code


def _all_code_rows(blk):
    """One row per scale code, each row = codes 0..15 repeated to the block length."""
    codes = np.tile(np.arange(16, dtype=np.uint8), blk // 16)
    packed_row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return np.tile(packed_row, (256, 1)), codes


def test_nvfp4_exhaustive_e2m1_times_e4m3():
    packed, codes = _all_code_rows(16)
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    e2m1 = np.array([v for _, v in read_golden("e2m1_values.txt")])
    s = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for g in (1.0, 0.25, 2.0 ** 5, float(np.float32(0.3711))):
        got = O.dequant_fp4(packed, scales, O.NVFP4, g)
        want = e2m1[codes][None, :] * s[:, None] * g
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], want[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_mxfp4_exhaustive_e2m1_times_e8m0():
    packed, codes = _all_code_rows(32)
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    e2m1 = np.array([v for _, v in read_golden("e2m1_values.txt")])
    s = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = O.dequant_fp4(packed, scales, O.MXFP4)
    want = e2m1[codes][None, :] * s[:, None]
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_dequant_layout_rows_and_block_columns():
    # a non-square matrix with one distinct scale per (row, block): a transposed
    # operand or a wrong block index would move values between positions
    n, k = 3, 64
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sc = (120 + np.arange(n * 2).reshape(n, 2)).astype(np.uint8)
    got = O.dequant_fp4(packed, sc, O.MXFP4)
    e2m1 = np.array([v for _, v in read_golden("e2m1_values.txt")])
    for r in range(n):
        for c in range(k):
            assert got[r, c] == e2m1[codes[r, c]] * 2.0 ** (int(sc[r, c // 32]) - 127)


def test_fp8_every_code_times_block_scales():
    # every E4M3 code (torch's float8_e4m3fn decoder) times fp32 block scales, power of
    # two and not: the product is exact in fp64
    codes = np.tile(np.arange(256, dtype=np.uint8), (2, 1))  # [2, 256]: two k-blocks
    e4m3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for s0, s1 in ((1.0, 0.5), (2.0 ** -7, 3.0), (float(np.float32(0.3711)), float(np.float32(1e-3)))):
        sc = np.array([[s0, s1]], dtype=np.float32)
        got = O.dequant_fp8(codes, sc)
        want = np.concatenate([e4m3[:128] * float(np.float32(s0)), e4m3[128:] * float(np.float32(s1))])
        want = np.tile(want, (2, 1))
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], want[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_fp8_block_layout_rows_and_columns():
    # one distinct scale per 128 x 128 block of a ragged [300, 200] matrix: a swapped or
    # wrongly sized block index moves scales between positions
    n, k = 300, 200
    codes = np.full((n, k), 0x38, dtype=np.uint8)  # E4M3 1.0
    sc = (np.arange(3 * 2, dtype=np.float32).reshape(3, 2) + 1.0) * 0.25
    got = O.dequant_fp8(codes, sc)
    for r in (0, 127, 128, 255, 256, 299):
        for c in (0, 127, 128, 199):
            assert got[r, c] == sc[r // 128, c // 128]
    with pytest.raises(ValueError):
        O.dequant_fp8(codes, sc[:, :1])


def test_fp8_quantizer_round_trip_on_grid():
    """Values on the E4M3 grid of their block (block amax = 448 * scale) survive the
    test-only FP8 encoder exactly."""
    g = torch.Generator().manual_seed(9)
    n, k = 256, 384
    code = torch.randint(0, 0x7E, (n, k), generator=g, dtype=torch.int32).to(torch.uint8)
    sign = torch.randint(0, 2, (n, k), generator=g, dtype=torch.int32).to(torch.uint8) << 7
    code = code | sign
    vals = code.view(torch.float8_e4m3fn).float()
    scale = torch.tensor([[0.5, 2.0 ** -9, 3.0], [0.25, 1.0, 2.0 ** -3]], dtype=torch.float32)
    full = scale.repeat_interleave(128, 0).repeat_interleave(128, 1)
    vals[::128, ::128] = 448.0  # pin each block's amax
    w = vals * full
    c2, s2 = S.quantize_fp8(w)
    assert torch.equal(s2, scale)
    assert np.array_equal(O.dequant_fp8(c2.numpy(), s2.numpy()), w.double().numpy())


def test_bf16_weights_decode_to_their_values():
    v = torch.randn(5, 64, dtype=torch.float32).to(torch.bfloat16)
    bits = v.view(torch.int16).numpy()
    assert np.array_equal(O.dequant_weight(bits, None, O.BF16), v.double().numpy())


def test_quantizers_round_trip_on_grid():
    """On-grid weights survive the (independent) test-only encoders exactly."""
    g = torch.Generator().manual_seed(5)
    e2m1 = torch.tensor([v for _, v in read_golden("e2m1_values.txt")], dtype=torch.float32)
    # MXFP4: every 32-block holds a +-4 or +-6 so its shared exponent is exactly X
    n, k = 8, 128
    codes = torch.randint(0, 16, (n, k), generator=g)
    codes[:, ::32] = 6  # value 4.0 at the start of each block
    x = torch.randint(-10, 6, (n, k // 32), generator=g)
    w = e2m1[codes] * torch.pow(2.0, x.float()).repeat_interleave(32, dim=1)
    packed, sc = S.quantize_mxfp4(w)
    back = O.dequant_fp4(packed.numpy(), sc.numpy(), O.MXFP4)
    assert np.array_equal(back, w.double().numpy())
    # NVFP4: global chosen so that amax/(448*6) is a power of two; block amax = 6*s*g
    s_codes = torch.randint(0x30, 0x77, (n, k // 16), generator=g).to(torch.uint8)
    s_codes[0, 0] = 0x7E  # one block reaches the E4M3 maximum 448
    s_val = s_codes.view(torch.float8_e4m3fn).float()
    codes = torch.randint(0, 16, (n, k), generator=g)
    codes[:, ::16] = 7  # value 6.0 in every block: block amax = 6 * s * g
    gsc = 2.0 ** -12
    w = e2m1[codes] * s_val.repeat_interleave(16, dim=1) * gsc
    packed, sc, gg = S.quantize_nvfp4(w)
    assert gg == gsc
    back = O.dequant_fp4(packed.numpy(), sc.numpy(), O.NVFP4, gg)
    assert np.array_equal(back, w.double().numpy())


def test_quantizer_saturates_and_rounds_to_even():
    # direct check of the encoder's rounding, against hand-computed E2M1 ties
    a = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, 0.2])
    want = torch.tensor([0, 2, 2, 4, 4, 6, 6, 7, 7, 0], dtype=torch.uint8)
    assert torch.equal(S._e2m1_encode_magnitude(a), want)


# ---------------------------------------------------------------- router

def test_router_logits_one_hot_equals_router_column():
    torch.manual_seed(1)
    e, h = 8, 64
    wr = torch.randn(e, h).to(torch.bfloat16).float().numpy()
    for col in (0, 17, 63):
        x = np.zeros((1, h), dtype=np.float32)
        x[0, col] = 1.0
        assert np.array_equal(O.router_logits(x, wr)[0], wr[:, col])


def test_router_logits_correctly_rounded_against_fsum():
    torch.manual_seed(2)
    t, e, h = 4, 8, 256
    x = torch.randn(t, h).to(torch.bfloat16).float().numpy()
    wr = (torch.randn(e, h) * 0.02).to(torch.bfloat16).float().numpy()
    bias = (torch.randn(e) * 0.5).numpy().astype(np.float32)
    got = O.router_logits(x, wr, bias)
    for i in range(t):
        for j in range(e):
            exact = math.fsum([float(x[i, q]) * float(wr[j, q]) for q in range(h)] + [float(bias[j])])
            assert got[i, j] == np.float32(exact)


def test_rms_norm_matches_torch():
    torch.manual_seed(3)
    x = torch.randn(5, 96, dtype=torch.float64)
    gamma = 1 + 0.1 * torch.randn(96, dtype=torch.float64)
    ref = torch.nn.functional.rms_norm(x, (96,), gamma, eps=1e-6).numpy()
    assert np.allclose(O.rms_norm(x.numpy(), gamma.numpy(), 1e-6), ref, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- selection

def test_topk_all_equal_picks_lowest_indices():
    keys = np.full((3, 16), 0.25, dtype=np.float32)
    assert np.array_equal(O.select_topk(keys, 5), np.tile(np.arange(5), (3, 1)))


def test_topk_signed_zero_nan_and_inf():
    keys = np.array([[np.nan, -0.0, 0.0, -np.inf, np.nan, 1.0]], dtype=np.float32)
    assert O.select_topk(keys, 6)[0].tolist() == [5, 1, 2, 3, 0, 4]
    keys = np.array([[0.0, -0.0, -1.0, -0.0]], dtype=np.float32)
    assert O.select_topk(keys, 3)[0].tolist() == [0, 1, 3]


def test_topk_matches_torch_on_distinct_keys():
    torch.manual_seed(4)
    keys = torch.randn(64, 128)
    for k in (1, 6, 8, 128):
        ids = O.select_topk(keys.numpy(), k)
        assert np.array_equal(ids, torch.topk(keys, k, dim=1, sorted=True).indices.numpy())


def test_topk_brute_force_property_with_ties():
    """No unselected expert beats a selected one; order is key desc then index asc."""
    rng = np.random.default_rng(5)
    keys = rng.integers(-3, 4, size=(50, 12)).astype(np.float32)  # many ties
    for k in (1, 3, 12):
        ids = O.select_topk(keys, k)
        for r in range(keys.shape[0]):
            sel = list(ids[r])
            assert len(set(sel)) == k
            for a, b in zip(sel, sel[1:]):
                assert keys[r, a] > keys[r, b] or (keys[r, a] == keys[r, b] and a < b)
            for u in set(range(12)) - set(sel):
                last = sel[-1]
                assert keys[r, u] < keys[r, last] or (keys[r, u] == keys[r, last] and u > last)


def test_softmax_and_sigmoid_weights_match_torch():
    torch.manual_seed(6)
    logits = torch.randn(7, 32).float()
    ids, w = O.route(logits.numpy(), 4, O.SOFTMAX)
    p = torch.softmax(logits.double(), dim=1).numpy()
    assert np.allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-14)
    bias = (torch.rand(32) * 0.2 - 0.1).numpy().astype(np.float32)
    ids, w = O.route(logits.numpy(), 4, O.SIGMOID, correction_bias=bias)
    s = torch.sigmoid(logits.double()).numpy()
    assert np.allclose(w, np.take_along_axis(s, ids.astype(np.int64), 1), rtol=1e-14)
    # the bias moves selection but not the weights: unbiased sigmoid at the chosen ids
    key = (torch.sigmoid(logits.double()).float() + torch.from_numpy(bias)).numpy()
    assert np.array_equal(ids, torch.topk(torch.from_numpy(key), 4, dim=1).indices.numpy())


def test_renormalised_weights_sum_to_scaling():
    torch.manual_seed(7)
    logits = torch.randn(9, 64).numpy()
    _, w = O.route(logits, 8, O.SOFTMAX, renormalize=True, routed_scaling=2.5)
    assert np.allclose(w.sum(1), 2.5, rtol=1e-14)


def test_zero_bias_sigmoid_ranks_like_softmax():
    torch.manual_seed(8)
    logits = torch.randn(40, 256).numpy().astype(np.float32)
    a, _ = O.route(logits, 8, O.SOFTMAX)
    b, _ = O.route(logits, 8, O.SIGMOID, correction_bias=np.zeros(256, np.float32))
    assert np.array_equal(a, b)


def test_sqrt_softplus_score_closed_forms():
    # softplus(0) = ln 2; softplus(l) - softplus(-l) = l; exp(softplus(l)) - 1 = exp(l)
    assert O.sqrt_softplus(np.array([0.0]))[0] == math.sqrt(math.log(2.0))
    l = np.linspace(-30.0, 30.0, 121)
    s_pos, s_neg = O.sqrt_softplus(l), O.sqrt_softplus(-l)
    assert np.allclose(s_pos ** 2 - s_neg ** 2, l, rtol=0, atol=1e-13)
    mid = np.linspace(-8.0, 8.0, 33)
    assert np.allclose(np.expm1(O.sqrt_softplus(mid) ** 2), np.exp(mid), rtol=1e-13)
    # no overflow far out: sqrt(softplus(l)) -> sqrt(l) for large l, -> exp(l / 2) for very negative l
    big = O.sqrt_softplus(np.array([1000.0, -1000.0]))
    assert big[0] == math.sqrt(1000.0) and big[1] == 0.0
    assert np.all(np.diff(O.sqrt_softplus(np.linspace(-50, 50, 1001))) > 0)  # monotone


def test_sqrt_softplus_routing():
    torch.manual_seed(10)
    logits = torch.randn(40, 256).numpy().astype(np.float32)
    # monotone in the logit: with no bias it ranks like softmax
    a, _ = O.route(logits, 8, O.SOFTMAX)
    b, w = O.route(logits, 8, O.SQRT_SOFTPLUS, correction_bias=np.zeros(256, np.float32))
    assert np.array_equal(a, b)
    # the bias moves selection, not the weights (the unbiased score at the chosen ids)
    bias = (torch.rand(256) * 0.2 - 0.1).numpy().astype(np.float32)
    ids, w = O.route(logits, 8, O.SQRT_SOFTPLUS, correction_bias=bias)
    sp = torch.sqrt(torch.nn.functional.softplus(torch.from_numpy(logits).double())).numpy()
    assert np.allclose(w, np.take_along_axis(sp, ids.astype(np.int64), 1), rtol=1e-14)
    key = (torch.from_numpy(sp).float() + torch.from_numpy(bias)).numpy()
    assert np.array_equal(ids, torch.topk(torch.from_numpy(key), 8, dim=1).indices.numpy())
    # hash layers weighted by it: the table's ids, renormalised sqrt-softplus weights
    tok = np.arange(40, dtype=np.int32)
    table = np.tile(np.arange(6, dtype=np.int64), (40, 1)) * 7
    hid, hw = O.route(logits, 6, O.SQRT_SOFTPLUS, O.HASH, renormalize=True, token_ids=tok,
                      tid2eid=table)
    assert np.array_equal(hid, table.astype(np.int32))
    want = sp[:, ::7][:, :6]
    assert np.allclose(hw, want / want.sum(1, keepdims=True), rtol=1e-14)


def test_softmax_bias_routing():
    torch.manual_seed(12)
    logits = torch.randn(30, 96).numpy().astype(np.float32)
    # the probability is monotone in the logit: with no bias it ranks like softmax
    a, wa = O.route(logits, 6, O.SOFTMAX)
    b, wb = O.route(logits, 6, O.SOFTMAX_BIAS, correction_bias=np.zeros(96, np.float32))
    assert np.array_equal(a, b) and np.allclose(wa, wb, rtol=0, atol=0)
    # with a bias: selection on fp32(p) + bias, weights the unbiased probabilities
    bias = (torch.rand(96) * 0.02 - 0.01).numpy().astype(np.float32)
    ids, w = O.route(logits, 6, O.SOFTMAX_BIAS, correction_bias=bias)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1)
    key = (p.float() + torch.from_numpy(bias)).numpy()
    assert np.array_equal(ids, torch.topk(torch.from_numpy(key), 6, dim=1).indices.numpy())
    assert np.allclose(w, np.take_along_axis(p.numpy(), ids.astype(np.int64), 1), rtol=1e-14)


def test_zero_experts_add_the_expert_input():
    inp = _small_layer(seed=21, t=4, h=64, e=4, k=2, i=32)
    x = inp.x.double().numpy()
    res = inp.residual.double().numpy()
    rw = inp.router_w.float().numpy()
    z = 3  # router outputs 4 + 3; the last three are zero-computation experts
    rw_z = np.concatenate([rw, np.zeros((z, rw.shape[1]), np.float32)])
    # logits that select only zero experts: the output is residual + (sum of weights) * x
    lz = np.full((4, 7), -5.0, np.float32)
    lz[:, 4:] = [1.0, 2.0, 3.0]
    out, _, ids, w = O.layer_forward(x, res, rw_z, _cache(inp.routed), 2, renormalize=True,
                                     logits=lz, zero_experts=z)
    assert np.all(ids >= 4)
    assert np.allclose(out, res + x, rtol=0, atol=1e-12)
    # logits that never select a zero expert: the layer of the E real experts
    ln = np.concatenate([torch.randn(4, 4).numpy().astype(np.float32),
                         np.full((4, z), -np.inf, np.float32)], axis=1)
    o1, _, i1, w1 = O.layer_forward(x, res, rw_z, _cache(inp.routed), 2, logits=ln,
                                    zero_experts=z)
    o0, _, i0, w0 = O.layer_forward(x, res, rw, _cache(inp.routed), 2, logits=ln[:, :4])
    assert np.array_equal(i1, i0) and np.allclose(o1, o0, rtol=0, atol=0)


def test_hash_with_softmax_ids_reproduces_softmax_routing():
    torch.manual_seed(9)
    t, e, k, v = 6, 16, 3, 40
    logits = torch.randn(t, e).numpy().astype(np.float32)
    sid, sw = O.route(logits, k, O.SOFTMAX, renormalize=True)
    tok = np.arange(t, dtype=np.int32) * 5
    table = np.zeros((v, k), dtype=np.int64)
    table[tok] = sid
    hid, hw = O.route(logits, k, O.SOFTMAX, O.HASH, renormalize=True, token_ids=tok, tid2eid=table)
    assert np.array_equal(hid, sid)
    assert np.allclose(hw, sw, rtol=1e-15)


def test_hash_out_of_range_gives_empty_slots():
    logits = np.zeros((2, 4), np.float32)
    table = np.array([[0, 9], [1, 2]], np.int64)
    ids, w = O.route(logits, 2, O.SOFTMAX, O.HASH, renormalize=True,
                     token_ids=np.array([0, 7], np.int32), tid2eid=table)
    assert ids.tolist() == [[0, -1], [-1, -1]]
    assert w[0, 0] == 1.0 and w[0, 1] == 0 and np.all(w[1] == 0)


# ---------------------------------------------------------------- experts + combine

def _small_layer(seed=11, t=3, h=64, e=4, k=2, i=32, fmt=S.NVFP4, shared=False):
    spec = S.LayerSpec(name="pin", tokens=t, hidden=h, experts=e, top_k=k, inter=i, fmt=fmt,
                       shared=shared, shared_inter=i, seed=seed)
    return S.make_inputs(spec)


def _np_parts(ws):
    return {n: (getattr(ws, n).fmt, getattr(ws, n).packed.numpy(), getattr(ws, n).scales.numpy(),
                None if getattr(ws, n).global_scale is None else getattr(ws, n).global_scale.numpy())
            for n in ("gate", "up", "down")}


def _cache(ws):
    p = _np_parts(ws)
    return O.DequantCache(p["gate"], p["up"], p["down"])


def _torch_dense(inp):
    """All experts for all tokens with torch library ops, weights decoded by torch's float8."""
    e2m1 = torch.tensor([v for _, v in read_golden("e2m1_values.txt")], dtype=torch.float64)

    def deq(w):
        lo = (w.packed & 0xF).long()
        hi = (w.packed >> 4).long()
        codes = torch.stack([lo, hi], dim=-1).reshape(w.packed.shape[0], w.n, w.k)
        if w.fmt == S.NVFP4:
            s = w.scales.view(torch.float8_e4m3fn).double().repeat_interleave(16, dim=-1)
            return e2m1[codes] * s * w.global_scale.double()[:, None, None]
        s = w.scales.view(torch.float8_e8m0fnu).double().repeat_interleave(32, dim=-1)
        return e2m1[codes] * s

    wg, wu, wd = deq(inp.routed.gate), deq(inp.routed.up), deq(inp.routed.down)
    x = inp.x.double()
    g = torch.einsum("th,eih->eti", x, wg)
    u = torch.einsum("th,eih->eti", x, wu)
    y = torch.einsum("eti,ehi->eth", torch.nn.functional.silu(g) * u, wd)  # [E, T, H]
    return y


@pytest.mark.parametrize("fmt", [S.NVFP4, S.MXFP4])
def test_k_equals_e_softmax_is_dense_mixture(fmt):
    inp = _small_layer(fmt=fmt, e=4, k=4)
    out, logits, ids, w = O.layer_forward(inp.x.float().numpy(), inp.residual.float().numpy(),
                                          inp.router_w.float().numpy(), _cache(inp.routed), 4)
    y = _torch_dense(inp)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1)  # [T, E]
    want = inp.residual.double() + torch.einsum("te,eth->th", p, y)
    assert np.allclose(out, want.numpy(), rtol=1e-12, atol=1e-12)


def test_one_hot_routing_is_single_expert():
    inp = _small_layer(e=4, k=1)
    # a dominant router row makes expert 2 the only choice with weight ~1
    rw = inp.router_w.float().numpy().copy()
    x = inp.x.float().numpy()
    logits = np.zeros((x.shape[0], 4), np.float32)
    logits[:, 2] = 80.0
    out, _, ids, w = O.layer_forward(x, inp.residual.float().numpy(), rw, _cache(inp.routed), 1,
                                     logits=logits)
    assert np.all(ids == 2) and np.allclose(w, 1.0, rtol=1e-30, atol=1e-30)
    y = _torch_dense(inp)[2]
    assert np.allclose(out, (inp.residual.double() + y).numpy(), rtol=1e-12, atol=1e-12)


def test_zero_gate_gives_residual_exactly():
    inp = _small_layer(e=4, k=2)
    inp.routed.gate.packed.zero_()
    out, _, _, _ = O.layer_forward(inp.x.float().numpy(), inp.residual.float().numpy(),
                                   inp.router_w.float().numpy(), _cache(inp.routed), 2)
    assert np.array_equal(out, inp.residual.double().numpy())


def test_zero_weights_give_residual_exactly():
    inp = _small_layer(e=4, k=2)
    ids = np.array([[0, 1]] * 3, np.int32)
    out = O.experts_forward(inp.x.float().numpy(), ids, np.zeros((3, 2)), _cache(inp.routed),
                            inp.residual.float().numpy())
    assert np.array_equal(out, inp.residual.double().numpy())
    assert np.array_equal(O.bf16_round(out), inp.residual.float().numpy())


def test_power_of_two_global_scales_output_exactly():
    inp = _small_layer(e=4, k=2)
    x, r, rw = inp.x.float().numpy(), inp.residual.float().numpy(), inp.router_w.float().numpy()
    base, _, _, _ = O.layer_forward(x, np.zeros_like(r), rw, _cache(inp.routed), 2)
    inp.routed.down.global_scale.mul_(8.0)
    up8, _, _, _ = O.layer_forward(x, np.zeros_like(r), rw, _cache(inp.routed), 2)
    assert np.array_equal(up8, 8.0 * base)
    inp.routed.up.global_scale.mul_(0.5)  # linear in the up projection
    half, _, _, _ = O.layer_forward(x, np.zeros_like(r), rw, _cache(inp.routed), 2)
    assert np.allclose(half, 4.0 * base, rtol=1e-14, atol=1e-300)


def test_shared_expert_adds_with_weight_one():
    inp = _small_layer(e=4, k=2, shared=True)
    x, r, rw = inp.x.float().numpy(), inp.residual.float().numpy(), inp.router_w.float().numpy()
    with_s, _, _, _ = O.layer_forward(x, r, rw, _cache(inp.routed), 2, shared=_cache(inp.shared))
    without, _, _, _ = O.layer_forward(x, r, rw, _cache(inp.routed), 2)
    ys = _torch_dense(S.LayerInputs(**{**inp.__dict__, "routed": inp.shared}))[0]
    assert np.allclose(with_s - without, ys.numpy(), rtol=1e-11, atol=1e-12)


def test_pre_norm_feeds_experts_but_not_router():
    spec = S.LayerSpec(name="pin", tokens=3, hidden=64, experts=4, top_k=2, inter=32,
                       pre_norm=True, seed=12)
    inp = S.make_inputs(spec)
    x, r, rw = inp.x.float().numpy(), inp.residual.float().numpy(), inp.router_w.float().numpy()
    gamma = inp.gamma.float().numpy()
    out, logits, ids, w = O.layer_forward(x, r, rw, _cache(inp.routed), 2, gamma=gamma)
    assert np.array_equal(logits, O.router_logits(x, rw))
    xn = torch.nn.functional.rms_norm(inp.x.double(), (64,), inp.gamma.double(), eps=1e-6)
    xn = xn.to(torch.bfloat16).double().numpy()  # the expert input is a bf16 activation
    want = O.experts_forward(xn, ids, w, _cache(inp.routed), r)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def test_batching_invariance():
    inp = _small_layer(t=5, e=4, k=2)
    x, r, rw = inp.x.float().numpy(), inp.residual.float().numpy(), inp.router_w.float().numpy()
    full, _, _, _ = O.layer_forward(x, r, rw, _cache(inp.routed), 2)
    for t in range(5):
        one, _, _, _ = O.layer_forward(x[t:t + 1], r[t:t + 1], rw, _cache(inp.routed), 2)
        assert np.allclose(one[0], full[t], rtol=1e-13, atol=1e-13)


def test_rows_subset_equals_full():
    inp = _small_layer(t=6, e=4, k=2, shared=True)
    x, r, rw = inp.x.float().numpy(), inp.residual.float().numpy(), inp.router_w.float().numpy()
    full, _, _, _ = O.layer_forward(x, r, rw, _cache(inp.routed), 2, shared=_cache(inp.shared))
    sub, _, _, _ = O.layer_forward(x, r, rw, _cache(inp.routed), 2, shared=_cache(inp.shared),
                                   rows=np.array([4, 1]))
    assert np.allclose(sub, full[[4, 1]], rtol=1e-13, atol=1e-13)


def test_expert_threads_give_the_serial_result_bitwise():
    """The oracle's threaded expert loop (used on the full-size workloads) stores each
    expert's rows in their own slots and sums them afterwards in slot order, so any thread
    count gives exactly the serial result."""
    inp = _small_layer(t=9, e=6, k=3, shared=True)
    x, r, rw = inp.x.float().numpy(), inp.residual.float().numpy(), inp.router_w.float().numpy()
    one, _, _, _ = O.layer_forward(x, r, rw, _cache(inp.routed), 3, shared=_cache(inp.shared))
    many, _, _, _ = O.layer_forward(x, r, rw, _cache(inp.routed), 3, shared=_cache(inp.shared),
                                    workers=4)
    assert np.array_equal(one, many)


def test_bf16_round_f64_matches_torch_and_ties_to_even():
    torch.manual_seed(13)
    v = torch.randn(10000, dtype=torch.float64) * 10
    got = O.bf16_round_f64(v.numpy())
    assert np.array_equal(got, v.to(torch.bfloat16).double().numpy())
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 6.0 + 2 ** -6])
    assert O.bf16_round_f64(ties).tolist() == [1.0, 1.0 + 2 ** -6, -1.0, 6.0]
    # a value just above a tie must round up even though fp32 rounding would land on it
    assert O.bf16_round_f64(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0] == 1.0 + 2 ** -7


def test_bf16_round_ties_to_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -9], np.float32)
    got = O.bf16_round(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, ref)
