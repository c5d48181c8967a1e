"""HIP-graph capture of the layer, as bench.py replays decode layers: a graph holding two
layer calls on different inputs, replayed several times with eager work and host
synchronisation between the replays, gives bit-identical outputs to the eager calls at
every replay (the layer path records no memset, allocation or host synchronisation)."""
import pytest
import torch

import moe_synth as S
import mixture_experts_ffn_03_amd as M

from gpu_cases import config_for

pytestmark = pytest.mark.gpu

CASES = {
    # one token: top-K inside the gate+up kernel (a writer row and per-block lean selection),
    # the blend inside the down kernel
    "qwen3_decode_t1": S.WORKLOADS["qwen3_decode_t1"],
    "qwen3_decode_t8": S.WORKLOADS["qwen3_decode_t8"],
    # shared expert, sigmoid + correction bias, several tiles per expert; at 13 tokens the
    # shared expert's split-K MFMA launches run on the layer's stream
    "dsv3_mini": S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=13, hidden=1024, experts=64,
                          inter=256, shared_inter=192),
    # at 4 tokens it runs on the GEMV, on a side stream forked from the layer's stream and
    # joined before the blend (captured as a fork and a join)
    "dsv3_t4_mini": S.scaled(S.WORKLOADS["dsv3_decode_t32"], tokens=4, hidden=1024, experts=64,
                             inter=256, shared_inter=192),
    # hash routing from the selected experts' logits (no logits output), RMSNorm input
    "hash_mini": S.scaled(S.WORKLOADS["hash_mxfp4_t512"], tokens=40, hidden=512, experts=32,
                          inter=256, shared_inter=128, vocab=1000),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replay_matches_eager(name):
    print("case: graph replay", name, flush=True)
    spec = CASES[name]
    inp = S.make_inputs(spec, device="cuda")
    acts = [S.make_activations(spec, device="cuda", seed=spec.seed + 7 + 31 * b) for b in range(2)]
    cfg = config_for(inp, M.PATH_DECODE)
    ws = M.alloc_workspace(cfg, "cuda")
    T, H = spec.tokens, spec.hidden
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    routed = M.expert_weights(inp.routed)
    shared = M.expert_weights(inp.shared) if inp.shared is not None else None

    def call(b):
        a = acts[b]
        M.layer_forward(cfg, a.x, inp.router_w, routed, outs[b], ws, norm_gamma=inp.gamma,
                        logit_bias=inp.logit_bias, correction_bias=inp.correction_bias,
                        token_ids=a.token_ids, tid2eid=inp.tid2eid, shared=shared,
                        residual=a.residual)

    for b in range(2):
        call(b)
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    assert not torch.equal(want[0], want[1])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for b in range(2):
            call(b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for b in range(2):
            call(b)
    for rep in range(3):
        for o in outs:  # eager work between the replays
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for b in range(2):
            assert torch.equal(outs[b], want[b]), (rep, b)
    assert M.get_device_error(ws) == 0
    del graph
