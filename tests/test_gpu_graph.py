"""Capture of the layer's calls in a HIP graph (torch.cuda.CUDAGraph on a side
stream, through the C ABI): a training step (forward with saved state, then
the backward, whose weight and bias gradients run on the handle's second
stream, forked from and joined back into the captured stream) and a decode
step.  Each graph is replayed several times with eager work and
synchronisations between the replays, and every replay must reproduce the
eager results bit for bit (the same kernels on the same data)."""
from __future__ import annotations

import pytest

from gpt_causal_self_amd import gpt_attn as ga
from gpt_causal_self_amd.inputs import make_inputs
from layer_helpers import device_inputs

pytestmark = pytest.mark.gpu


def _replays_match(step, outs, s):
    import torch
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:  # eager work between the replays
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager run"


def test_graph_training_step_replays_match_eager():
    import torch
    B, T, C, H = 2, 200, 256, 4
    inp = make_inputs(B, T, C, H, bias=True, dtype="bf16", seed=41, with_dY=True)
    t = device_inputs(inp)
    layer = ga.Layer(C, H, B, T, "bf16")
    y = torch.empty_like(t["x"])
    g = {k: torch.empty_like(t[src]) for k, src in
         (("dx", "x"), ("dWa", "W_attn"), ("dba", "b_attn"), ("dWp", "W_proj"), ("dbp", "b_proj"))}

    def step(s):
        ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"],
                            H, y, stream=s, save_for_backward=True)
        ga.gpt_attn_backward(layer.h, t["x"], t["W_attn"], t["W_proj"], t["dY"], g["dx"],
                             g["dWa"], g["dba"], g["dWp"], g["dbp"], stream=s)

    _replays_match(step, [y, *g.values()], torch.cuda.Stream())
    layer.close()


def test_graph_decode_step_replays_match_eager():
    import torch
    B, C, H, cache_T = 3, 256, 4, 1100
    inp = make_inputs(B, 1, C, H, bias=True, dtype="bf16", seed=43)
    t = device_inputs(inp)
    layer = ga.Layer(C, H, B, 8, "bf16")
    gen = torch.Generator(device="cuda").manual_seed(3)
    kc = torch.randn((B, H, cache_T, C // H), device="cuda", generator=gen).to(torch.bfloat16)
    vc = torch.randn((B, H, cache_T, C // H), device="cuda", generator=gen).to(torch.bfloat16)
    xt = t["x"][:, 0].contiguous()
    yt = torch.empty_like(xt)
    pos = 1050  # two attention blocks: the merge of their partials is captured too

    def step(s):
        ga.gpt_attn_decode(layer.h, xt, t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"], H,
                           kc, vc, yt, pos, stream=s)

    _replays_match(step, [yt], torch.cuda.Stream())
    layer.close()


def test_graph_dropout_training_step_replays_match_eager():
    """The training step with dropout on: the forward also stores the keep
    bits that the backward reads; replays with the same seed reproduce the
    eager outputs and gradients bit for bit."""
    import torch
    B, T, C, H = 2, 200, 256, 4
    inp = make_inputs(B, T, C, H, bias=True, dtype="bf16", seed=47, with_dY=True)
    t = device_inputs(inp)
    layer = ga.Layer(C, H, B, T, "bf16")
    ga.gpt_attn_set_dropout(layer.h, 0.1, 2024)
    y = torch.empty_like(t["x"])
    g = {k: torch.empty_like(t[src]) for k, src in
         (("dx", "x"), ("dWa", "W_attn"), ("dba", "b_attn"), ("dWp", "W_proj"), ("dbp", "b_proj"))}

    def step(s):
        ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"],
                            H, y, stream=s, save_for_backward=True)
        ga.gpt_attn_backward(layer.h, t["x"], t["W_attn"], t["W_proj"], t["dY"], g["dx"],
                             g["dWa"], g["dba"], g["dWp"], g["dbp"], stream=s)

    _replays_match(step, [y, *g.values()], torch.cuda.Stream())
    layer.close()
