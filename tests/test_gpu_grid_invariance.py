"""Results do not depend on the rest of the launch.

Every (sequence, head) chain, and every (chunk, head) pair of the prep and
gradient launches, is computed by its own workgroup from its own inputs, so
a batch row run alone, in a small batch, or inside a large one must give the
same bits.  The launches differ between those runs in their grid sizes, in
which workgroups share a CU or an XCD (the d_v slices of a head are paired on
one XCD only when the number of (unit, head) pairs is a multiple of 8), and
in how many pairs each persistent prep workgroup walks -- so this also checks
that no kernel's result depends on scheduling (a race on LDS or on the
workspace would show up as differing bits).  GPU runs are compared with each
other only; their parity with the oracle is tested elsewhere.
"""
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


def rows(inp, lo, hi, keys):
    """Batch rows lo..hi-1 of every [B, ...] input (and of S0, [B, H, ...])."""
    return {k: (None if inp[k] is None else inp[k][lo:hi].contiguous()) for k in keys}


def same(tag, a, b):
    assert a.shape == b.shape, tag
    assert torch.equal(a, b), f"{tag}: results differ between launches"


def test_chunk_fwd_rows_alone_and_in_batch():
    B, T, H, d = 8, 1000, 4, 128   # 8 x 4 = 32 (unit, head) pairs: XCD-paired slices
    inp = gi.chunk_inputs(B, T, H, d, d, "bf16", s0_std=0.1, seed=91)
    keys = ("q", "k", "v", "log_alpha", "beta", "S0")
    say(f"chunk_fwd B={B} T={T} H={H} d={d}: whole batch")
    o, st = gdn.chunk_fwd(*(dev(inp[k]) for k in keys))
    for lo, hi in ((0, 1), (3, 6), (7, 8)):   # 4, 12 (not a multiple of 8) and 4 pairs
        say(f"chunk_fwd rows {lo}..{hi - 1} alone")
        sub = rows(inp, lo, hi, keys)
        o2, st2 = gdn.chunk_fwd(*(dev(sub[k]) for k in keys))
        torch.cuda.synchronize()
        same(f"chunk_fwd o rows {lo}..{hi - 1}", o[lo:hi].cpu(), o2.cpu())
        same(f"chunk_fwd S_T rows {lo}..{hi - 1}", st[lo:hi].cpu(), st2.cpu())


@pytest.mark.parametrize("which", ["kda", "gdn2"])
def test_channel_forwards_rows_alone_and_in_batch(which):
    # 4 x 2048 / 64 x 16 = 2048 (chunk, head) pairs: each persistent GDN-2
    # prep workgroup walks eight of them in the whole batch, two alone
    B, T, H, d = 4, 2048, 16, 128
    if which == "kda":
        inp = gi.kda_inputs(B, T, H, d, d, "bf16", s0_std=0.1, seed=92)
        keys = ("q", "k", "v", "log_alpha", "beta", "S0")
        fwd = gdn.kda_fwd
    else:
        inp = gi.gdn2_inputs(B, T, H, d, d, "bf16", s0_std=0.1, seed=93)
        keys = ("q", "k", "v", "log_alpha", "erase", "write", "S0")
        fwd = gdn.gdn2_fwd
    say(f"{which} B={B} T={T} H={H} d={d}: whole batch")
    o, st = fwd(*(dev(inp[k]) for k in keys))
    for lo, hi in ((0, 1), (1, 3)):
        say(f"{which} rows {lo}..{hi - 1} alone")
        sub = rows(inp, lo, hi, keys)
        o2, st2 = fwd(*(dev(sub[k]) for k in keys))
        torch.cuda.synchronize()
        same(f"{which} o rows {lo}..{hi - 1}", o[lo:hi].cpu(), o2.cpu())
        same(f"{which} S_T rows {lo}..{hi - 1}", st[lo:hi].cpu(), st2.cpu())


def test_chunk_bwd_rows_alone_and_in_batch():
    B, T, H, d = 4, 700, 4, 128
    inp = gi.chunk_inputs(B, T, H, d, d, "bf16", s0_std=0.1, seed=94)
    dO = torch.randn((B, T, H, d), generator=torch.Generator().manual_seed(95))
    keys = ("q", "k", "v", "log_alpha", "beta", "S0")
    say(f"chunk_bwd B={B} T={T} H={H} d={d}: whole batch")
    g = [x.cpu() for x in gdn.chunk_bwd(*(dev(inp[k]) for k in keys[:5]), dev(dO),
                                        S0=dev(inp["S0"]))]
    for lo, hi in ((0, 1), (2, 4)):
        say(f"chunk_bwd rows {lo}..{hi - 1} alone")
        sub = rows(inp, lo, hi, keys)
        g2 = gdn.chunk_bwd(*(dev(sub[k]) for k in keys[:5]), dev(dO[lo:hi].contiguous()),
                           S0=dev(sub["S0"]))
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), g, g2):
            same(f"chunk_bwd {name} rows {lo}..{hi - 1}", a[lo:hi], b.cpu())


def test_step_rows_alone_and_in_batch():
    inp = gi.decode_inputs(16, 16, 128, 128, 2, "bf16", 1.0, 0.1, seed=96)
    t = 0
    S = dev(inp["S0"]).clone()
    say("step B=16 H=16 d=128: whole batch")
    o = gdn.step(dev(inp["q"][t]), dev(inp["k"][t]), dev(inp["v"][t]), dev(inp["log_alpha"][t]),
                 dev(inp["beta"][t]), S)
    for lo, hi in ((0, 1), (5, 11)):
        say(f"step rows {lo}..{hi - 1} alone")
        S2 = dev(inp["S0"][lo:hi]).clone()
        o2 = gdn.step(*(dev(inp[k][t][lo:hi].contiguous()) for k in ("q", "k", "v", "log_alpha",
                                                                     "beta")), S2)
        torch.cuda.synchronize()
        same(f"step o rows {lo}..{hi - 1}", o[lo:hi].cpu(), o2.cpu())
        same(f"step S rows {lo}..{hi - 1}", S[lo:hi].cpu(), S2.cpu())
