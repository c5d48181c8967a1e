"""moe_layer_forward_noalloc (the entry point for callers that cannot allocate device
memory) against moe_layer_forward with a caller workspace: both run the same kernels, so
the outputs and routing decisions must be bit-identical, on two calls in a row (the second
smaller than the first, leaving the first call's contents in the shared scratch array), on
both expert paths; an oversized config is refused before anything is launched."""
import pytest
import torch

import moe_synth as S
import mixture_experts_ffn_03_amd as M

from gpu_cases import config_for

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    # decode path: sigmoid + correction bias, a shared expert; then fewer tokens
    "dsv3_mini": (S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=13, hidden=1024, experts=64,
                           inter=256, shared_inter=192), 5, M.PATH_AUTO),
    # prefill path: Zipf-skewed loads, several tiles per expert; then fewer tokens
    "zipf_mini": (S.scaled(S.WORKLOADS["prefill_zipf_t4096"], tokens=301, hidden=512,
                           experts=16, inter=192), 120, M.PATH_AUTO),
    # hash routing with an RMSNorm'd expert input and a shared expert (prefill), then decode
    "hash_mini": (S.scaled(S.WORKLOADS["hash_mxfp4_t512"], tokens=77, hidden=512, experts=32,
                           inter=256, shared_inter=128, vocab=1000), 3, M.PATH_AUTO),
}


def _both(inp, path):
    """(out, logits, ids, w) from the workspace entry and from the no-allocation entry."""
    s = inp.spec
    cfg = config_for(inp, path)
    res = []
    for noalloc in (False, True):
        out = torch.empty((s.tokens, s.hidden), dtype=torch.bfloat16, device=DEV)
        logits = torch.empty((s.tokens, s.experts + s.zero_experts), dtype=torch.float32,
                             device=DEV)
        ids = torch.empty((s.tokens, s.top_k), dtype=torch.int32, device=DEV)
        w = torch.empty((s.tokens, s.top_k), dtype=torch.float32, device=DEV)
        kw = dict(norm_gamma=inp.gamma, logit_bias=inp.logit_bias,
                  correction_bias=inp.correction_bias, token_ids=inp.token_ids,
                  tid2eid=inp.tid2eid,
                  shared=M.expert_weights(inp.shared) if inp.shared is not None else None,
                  residual=inp.residual, dbg_logits=logits, dbg_ids=ids, dbg_w=w)
        if noalloc:
            M.layer_forward_noalloc(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out,
                                    **kw)
        else:
            ws = M.alloc_workspace(cfg, DEV)
            assert ws.numel() <= M.NOALLOC_SCRATCH_BYTES
            M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out, ws, **kw)
        res.append((out, logits, ids, w))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_matches_workspace_entry_twice(name):
    spec, smaller, path = CASES[name]
    for tokens in (spec.tokens, smaller):
        print(f"case: no-alloc {name} tokens={tokens}", flush=True)
        inp = S.make_inputs(S.scaled(spec, tokens=tokens), device=DEV)
        (o1, l1, i1, w1), (o2, l2, i2, w2) = _both(inp, path)
        assert torch.equal(l1, l2)
        assert torch.equal(i1, i2)
        assert torch.equal(w1, w2)
        assert torch.equal(o1, o2)


def test_noalloc_rejects_a_workspace_beyond_its_array():
    print("case: no-alloc oversized config", flush=True)
    small = S.make_inputs(CASES["zipf_mini"][0], device=DEV)
    tokens = 16384  # 98304 routed rows of fp32 expert outputs: 192 MiB of workspace
    cfg = M.make_config(tokens, small.spec.hidden, small.spec.experts, small.spec.top_k,
                        small.spec.inter, path=M.PATH_PREFILL)
    assert M.workspace_size(cfg) > M.NOALLOC_SCRATCH_BYTES
    out = torch.empty((tokens, small.spec.hidden), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((tokens, small.spec.hidden), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoeError) as ei:
        M.layer_forward_noalloc(cfg, x, small.router_w, M.expert_weights(small.routed), out)
    assert ei.value.status == -3  # MOE_ERR_WORKSPACE
