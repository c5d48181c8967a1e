"""Accuracy gate of the FP8-activation prefill variant (CPU only).

gfx950's block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) takes MXFP4 weights natively,
but its other operand must be FP8/FP6/FP4 too: the bf16 activations would have to be
quantised to MXFP8 (E4M3 elements, one E8M0 power-of-two scale per 32 along K, OCP MX v1.0).
These tests evaluate that variant with the oracle on the prefill workload's real H and I
(4096 x 1408, MXFP4 experts): quantising the expert inputs and the SiLU*up intermediates to
MXFP8 misses the layer's parity bar, while a hi + lo pair of MXFP8 values (two scaled MFMAs,
no faster than one bf16 MFMA) meets it. The default prefill path therefore keeps bf16
activations and bf16 MFMAs on exactly decoded weights.
"""
import numpy as np
import pytest

import moe_synth as S
import oracle as O
from gpu_cases import MAX_ABS, REL_L2, errors, f32, oracle_cache

_E4M3_MAX_EXP = 8  # emax of the E4M3 element format (largest finite 448 = 1.75 * 2^8)


def _e4m3_grid():
    vals = {O.e4m3fn_value(b) for b in range(128)}
    return np.array(sorted(v for v in vals if np.isfinite(v)))


_GRID = _e4m3_grid()


def _round_e4m3(a):
    """|a| to the nearest non-negative E4M3 value, ties to the even code, saturating."""
    a = np.minimum(np.abs(a), _GRID[-1])
    i = np.clip(np.searchsorted(_GRID, a), 1, len(_GRID) - 1)
    lo, hi = _GRID[i - 1], _GRID[i]
    up = (a - lo > hi - a) | ((a - lo == hi - a) & (i % 2 == 0))
    return np.where(up, hi, lo)


def mxfp8(x):
    """OCP MX quantisation of the last axis in blocks of 32: shared scale
    2^(floor(log2(amax)) - 8), elements rounded to E4M3; returns the decoded values."""
    x = np.asarray(x, np.float64)
    b = x.reshape(-1, 32)
    amax = np.abs(b).max(axis=1, keepdims=True)
    e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - _E4M3_MAX_EXP
    scale = np.ldexp(1.0, e.astype(np.int64))
    return (np.sign(b) * _round_e4m3(b / scale) * scale).reshape(x.shape)


def mxfp8_hi_lo(x):
    hi = mxfp8(x)
    return hi + mxfp8(np.asarray(x, np.float64) - hi)


def test_mxfp8_round_trip_on_grid():
    # values already on the E4M3 grid of their block survive unchanged
    rng = np.random.default_rng(3)
    codes = rng.choice(_GRID[1:], size=(4, 32)) * rng.choice([-1.0, 1.0], size=(4, 32))
    codes[:, 0] = 448.0  # block amax sets the scale to 2^0
    assert np.array_equal(mxfp8(codes), codes)
    # with the block scale 2^(floor(log2 amax) - 8), E4M3's half step is at most 2^-4 of the
    # block's amax, and saturating the largest elements at 448 costs less than 2^-3 of it
    x = rng.standard_normal((8, 64))
    q = mxfp8(x)
    blk_amax = np.abs(x.reshape(-1, 32)).max(axis=1).repeat(32).reshape(x.shape)
    assert np.all(np.abs(q - x) <= blk_amax * 2.0 ** -3)
    small = np.abs(x) < blk_amax / 2  # below the saturating binade: half a step
    assert np.all(np.abs(q - x)[small] <= blk_amax[small] * 2.0 ** -5)


@pytest.fixture(scope="module")
def prefill_case():
    spec = S.scaled(S.WORKLOADS["prefill_zipf_t4096"], tokens=16, experts=8)
    inp = S.make_inputs(spec)
    want, _, ids, w = O.layer_forward(
        f32(inp.x), f32(inp.residual), f32(inp.router_w), oracle_cache(inp.routed), spec.top_k,
        score=spec.score, renormalize=spec.renormalize, logit_bias=f32(inp.logit_bias))
    return spec, inp, want, ids, w


def _layer_with_quantised_activations(spec, inp, ids, w, q):
    cache = oracle_cache(inp.routed)
    x = f32(inp.x).astype(np.float64)
    moe = np.zeros_like(x)
    for e in range(spec.experts):
        sel = np.argwhere(ids == e)
        if not len(sel):
            continue
        wg, wu, wd = cache.get(e)
        xe = q(x[sel[:, 0]])
        h = q(O.bf16_round_f64(O.silu(xe @ wg.T) * (xe @ wu.T)))
        y = h @ wd.T
        for (t, j), yy in zip(sel, y):
            moe[t] += w[t, j] * yy
        cache.drop(e)
    return O.bf16_round_f64(f32(inp.residual).astype(np.float64) + moe)


def test_mxfp8_activations_miss_the_parity_bar(prefill_case):
    spec, inp, want, ids, w = prefill_case
    got = _layer_with_quantised_activations(spec, inp, ids, w, mxfp8)
    mx, _, rl = errors(got, want)
    assert mx > MAX_ABS or rl > REL_L2, (mx, rl)


def test_mxfp8_hi_lo_activations_meet_the_parity_bar(prefill_case):
    spec, inp, want, ids, w = prefill_case
    got = _layer_with_quantised_activations(spec, inp, ids, w, mxfp8_hi_lo)
    mx, _, rl = errors(got, want)
    assert mx <= MAX_ABS and rl <= REL_L2, (mx, rl)
