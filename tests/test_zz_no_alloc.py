"""gdn_kda_fwd_noalloc (workspace in the library's device array) against
gdn_kda_fwd (caller workspace) through the C ABI: two calls in a row, the
second smaller, each equal to the workspace entry point's result bit for bit
(the same kernels) and within the channel-wise decay forward's bar of the
fp64 oracle."""
import os

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_delta_rule_58_amd as gdn
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
THREADS = min(16, os.cpu_count() or 1)
TAU = 1e-3


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(x):
    return None if x is None else x.to(DEV)


def run_pair(tag, inp):
    args = [dev(inp[x]) for x in ("q", "k", "v", "log_alpha", "beta", "S0", "cu_seqlens")]
    say(f"{tag}: gdn_kda_fwd")
    o1, s1 = gdn.kda_fwd(*args)
    say(f"{tag}: gdn_kda_fwd_noalloc")
    o2, s2 = gdn.kda_fwd_noalloc(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(s1.cpu(), s2.cpu()), tag
    ro, rs = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                            inp["S0"], inp["cu_seqlens"], threads=THREADS)
    eo, es = gi.max_rel_err(o2, ro), gi.max_rel_err(s2, rs)
    say(f"{tag}: max err / RMS o {eo:.3e} S_T {es:.3e} (bar {TAU:g})")
    assert eo <= TAU and es <= TAU


def test_noalloc_matches_workspace_entry_point_twice():
    cap = gdn.kda_fwd_noalloc_max_workspace()
    big = gi.kda_inputs(2, 300, 4, 128, 128, "bf16", s0_std=0.1, seed=61)
    small = gi.kda_inputs(1, 70, 2, 128, 128, "bf16", s0_std=0.1, seed=62)
    assert gdn.kda_fwd_workspace_size(2, 300, 4, 128, 128) <= cap
    run_pair("noalloc call 1 (B=2 T=300 H=4)", big)
    run_pair("noalloc call 2, smaller (B=1 T=70 H=2)", small)


def test_noalloc_packed_and_d64():
    lens = [70, 0, 130, 1, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    run_pair("noalloc packed d=128", gi.kda_inputs(1, cu[-1], 2, 128, 128, "bf16", s0_std=0.1,
                                                    seed=63, cu_seqlens=cu))
    run_pair("noalloc d=64", gi.kda_inputs(2, 150, 3, 64, 64, "bf16", s0_std=0.1, seed=64))


def test_noalloc_rejects_shapes_beyond_the_array():
    cap = gdn.kda_fwd_noalloc_max_workspace()
    B, T, H = 1, 8192, 16          # 2048 chunk-heads at d = 128: 4x the array
    assert gdn.kda_fwd_workspace_size(B, T, H, 128, 128) > cap
    q = torch.zeros((B, T, H, 128), device=DEV, dtype=torch.bfloat16)
    la = torch.zeros((B, T, H, 128), device=DEV)
    be = torch.zeros((B, T, H), device=DEV)
    say("noalloc too large: expect GDN_ERR_WORKSPACE")
    with pytest.raises(gdn.GdnError) as ei:
        gdn.kda_fwd_noalloc(q, q, q, la, be)
    assert ei.value.code == 4 and "scratch" in str(ei.value)
