"""The C-ABI calls under HIP graph capture (torch.cuda.CUDAGraph).

The library enqueues kernels only (no allocation, copy, memset or
synchronisation), so a serving loop can capture its calls once and replay
them.  Each test captures a call sequence, replays the graph several times
with eager work and synchronisations in between, and checks every replay
against the eager result bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_delta_rule_58_amd as gdn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(x):
    return None if x is None else x.to(DEV)


def capture(fn):
    """Capture fn() on a side stream (after a warm-up call there), return the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_steps_graph_replay():
    B, H, d, steps = 4, 8, 128, 6
    rng = np.random.default_rng(31)
    k = torch.from_numpy(rng.standard_normal((steps, B, H, d)))
    inp = dict(
        q=torch.from_numpy(rng.standard_normal((steps, B, H, d))).to(torch.bfloat16),
        k=(k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16),
        v=torch.from_numpy(rng.standard_normal((steps, B, H, d))).to(torch.bfloat16),
        log_alpha=torch.from_numpy(
            -np.log1p(np.exp(rng.standard_normal((steps, B, H)) + 1.0))).float(),
        beta=torch.from_numpy(
            1.0 / (1.0 + np.exp(-rng.standard_normal((steps, B, H))))).float(),
        S0=torch.from_numpy(rng.standard_normal((B, H, d, d)) * 0.1).float())
    x = {n: dev(t) for n, t in inp.items()}
    say(f"decode graph: {steps} steps B={B} H={H} d={d}")
    S_e = x["S0"].clone()
    o_e = torch.empty((steps, B, H, d), device=DEV)
    for t in range(steps):
        gdn.step(x["q"][t], x["k"][t], x["v"][t], x["log_alpha"][t], x["beta"][t], S_e, o=o_e[t])
    torch.cuda.synchronize()

    S_g = x["S0"].clone()
    o_g = torch.empty_like(o_e)

    def run():
        for t in range(steps):
            gdn.step(x["q"][t], x["k"][t], x["v"][t], x["log_alpha"][t], x["beta"][t], S_g,
                     o=o_g[t])

    g = capture(run)
    for rep in range(3):
        S_g.copy_(x["S0"])           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(S_g, S_e), f"replay {rep}: state"
        assert torch.equal(o_g, o_e), f"replay {rep}: o"


def test_chunk_fwd_graph_replay():
    inp = gi.chunk_inputs(2, 200, 4, 128, 128, "bf16", s0_std=0.1, seed=32)
    x = {n: dev(t) for n, t in inp.items()}
    say("chunk_fwd graph: B=2 T=200 H=4 d=128")
    o_e, S_e = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S0=x["S0"])
    torch.cuda.synchronize()
    o_g = torch.empty_like(o_e)
    S_g = torch.empty_like(S_e)

    def run():
        gdn.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S0=x["S0"], o=o_g,
                      S_T=S_g)

    g = capture(run)
    for rep in range(3):
        o_g.fill_(float("nan"))
        S_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {rep}: o"
        assert torch.equal(S_g, S_e), f"replay {rep}: S_T"


def test_chunk_bwd_graph_replay():
    inp = gi.chunk_inputs(2, 150, 3, 128, 128, "bf16", s0_std=0.1, seed=33)
    x = {n: dev(t) for n, t in inp.items()}
    rng = np.random.default_rng(33)
    dO = torch.from_numpy(rng.standard_normal((2, 150, 3, 128))).float().to(DEV)
    dS_T = (torch.from_numpy(rng.standard_normal((2, 3, 128, 128)) * 0.1)).float().to(DEV)
    say("chunk_bwd graph: B=2 T=150 H=3 d=128")
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], dO)
    eager = gdn.chunk_bwd(*args, S0=x["S0"], dS_T=dS_T)
    torch.cuda.synchronize()
    ws = torch.empty(gdn.chunk_bwd_workspace_size(2, 150, 3, 128, 128), dtype=torch.uint8,
                     device=DEV)
    out = {}

    def run():
        out["g"] = gdn.chunk_bwd(*args, S0=x["S0"], dS_T=dS_T, workspace=ws)

    g = capture(run)
    for rep in range(3):
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), out["g"], eager):
            assert torch.equal(a, b), f"replay {rep}: {name}"


@pytest.mark.parametrize("which", ["kda", "kda_noalloc", "gdn2"])
def test_channel_forward_graph_replay(which):
    B, T, H, d = 2, 200, 3, 128
    if which == "gdn2":
        inp = gi.gdn2_inputs(B, T, H, d, d, "bf16", s0_std=0.1, seed=35)
        keys = ("q", "k", "v", "log_alpha", "erase", "write")
        fwd, size = gdn.gdn2_fwd, gdn.gdn2_fwd_workspace_size
    else:
        inp = gi.kda_inputs(B, T, H, d, d, "bf16", s0_std=0.1, seed=34)
        keys = ("q", "k", "v", "log_alpha", "beta")
        fwd, size = gdn.kda_fwd, gdn.kda_fwd_workspace_size
    x = {n: dev(t) for n, t in inp.items()}
    args = tuple(x[n] for n in keys)
    say(f"{which} graph: B={B} T={T} H={H} d={d}")
    o_e, S_e = fwd(*args, x["S0"])
    torch.cuda.synchronize()
    o_g = torch.empty_like(o_e)
    S_g = torch.empty_like(S_e)
    ws = torch.empty(size(B, T, H, d, d), dtype=torch.uint8, device=DEV)

    def run():
        if which == "kda_noalloc":   # workspace from the library's device array
            gdn.kda_fwd_noalloc(*args, x["S0"], o=o_g, S_T=S_g)
        else:
            fwd(*args, x["S0"], o=o_g, S_T=S_g, workspace=ws)

    g = capture(run)
    for rep in range(3):
        o_g.fill_(float("nan"))
        S_g.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {rep}: o"
        assert torch.equal(S_g, S_e), f"replay {rep}: S_T"
