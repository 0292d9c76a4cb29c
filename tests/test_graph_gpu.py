"""The C-ABI entry points under HIP graph capture.

The library allocates nothing and clears nothing with memset: every launch
writes all of its outputs, so a captured forward + backward (outputs and the
backward workspace from the graph's memory pool) must replay to the same bits
as eager calls on the same inputs.  Each graph is replayed several times with
new inputs copied into its static tensors and eager work in between, and every
replay is compared with an eager run.
"""

import math

import pytest
import torch

from exact_attention_118_amd import synth

from test_parity_gpu import make, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up off the capture, as torch asks
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


@pytest.mark.parametrize("variant", ["plain", "dropout", "bias_map", "decode", "stored_ds"])
def test_graph_replays_match_eager(gpu_lib, variant):
    fa = gpu_lib
    say(f"graph capture {variant}")
    B, H, Nq, Nk, d = {"decode": (16, 8, 1, 4096, 128),
                       # enough heads and keys for the backward to store dS (three launches)
                       "stored_ds": (1, 128, 1024, 1024, 128)}.get(variant, (2, 4, 500, 500, 128))
    causal = variant != "decode"
    scale = 1.0 / math.sqrt(d)
    x = make(B, H, Nq, Nk, d, torch.bfloat16, seed=31)
    kw = {}
    if variant == "dropout":
        kw = dict(dropout_p=0.2, seed=99, offset=4)
    if variant == "bias_map":
        i = torch.arange(Nq, device="cuda")[:, None]
        j = torch.arange(Nk, device="cuda")[None, :]
        b = torch.randn((Nq, Nk), device="cuda")
        b[(i - j).abs() > 150] = float("-inf")
        full = torch.zeros((1, H, Nq, (Nk + 7) // 8 * 8), dtype=torch.bfloat16, device="cuda")
        full[..., :Nk] = b.to(torch.bfloat16)
        bias = full[..., :Nk]  # row stride a multiple of 8 elements
        kw = dict(bias=bias, tile_map=fa.fa_bias_tile_map(bias, B, H, Nq, Nk))

    def step():
        O, L = fa.forward(x["Q"], x["K"], x["V"], scale, causal, **kw)
        if variant == "decode":
            return (O, L)
        return (O, L) + tuple(fa.backward(x["Q"], x["K"], x["V"], O, L, x["dO"], scale, causal,
                                          **kw))

    g, outs = _capture(step)
    for rep, seed in enumerate((32, 33, 32)):
        new = make(B, H, Nq, Nk, d, torch.bfloat16, seed=seed)
        for k in x:
            x[k].copy_(new[k])
        g.replay()
        torch.cuda.synchronize()
        eager = step()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert bool(torch.isfinite(junk))
        for name, a, e in zip(("O", "L", "dQ", "dK", "dV"), outs, eager):
            assert torch.equal(a, e), (variant, rep, name)
