"""Parity of the backward pass (through the C ABI) with the fp64 oracle.

The GPU computes every gradient in fp32 from inputs that are exact in fp32
(bf16 inputs are upcast exactly), so its only error is fp32 rounding: the
bar is max |gpu - oracle| <= 1e-3 * RMS(oracle) per gradient (fp32
gradients); gradients returned in bf16 must be exactly the fp32 ones rounded
once.  The oracle is the
reverse-mode fp64 token recurrence ``oracle.bwd``; its pins are in
``tests/oracle_bwd_pins.py``.
"""
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
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(x):
    return None if x is None else x.to(DEV)


def grads_inputs(B, T, H, d, io, seed, s0_std=0.1, cu=None, dst=True, g_dtype=torch.float32):
    inp = gi.chunk_inputs(B, T, H, d, d, io, s0_std=s0_std, seed=seed, cu_seqlens=cu)
    rng = np.random.default_rng(seed + 7)
    units = B if cu is None else len(cu) - 1
    inp["dO"] = torch.from_numpy(rng.standard_normal((B, T, H, d))).to(g_dtype)
    inp["dS_T"] = (torch.from_numpy(rng.standard_normal((units, H, d, d)) * 0.1).float()
                   if dst else None)
    return inp


def compare(tag, inp, tau=TAU):
    say(f"{tag}: launch")
    g = gdn.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["log_alpha"]),
                      dev(inp["beta"]), dev(inp["dO"]), S0=dev(inp["S0"]),
                      cu_seqlens=dev(inp["cu_seqlens"]), dS_T=dev(inp["dS_T"]))
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"],
                     inp["cu_seqlens"], inp["dO"], inp["dS_T"], threads=THREADS)
    worst = 0.0
    for name, got, want in zip(NAMES, g, ref):
        got = got.cpu()
        err = gi.max_rel_err(got, want)
        worst = max(worst, err)
        say(f"{tag} {name}: max err / RMS = {err:.3e} (bar {tau:g})")
        assert np.all(np.isfinite(got.double().numpy())), f"{tag} {name}: non-finite"
        assert err <= tau, f"{tag} {name}: {err:.3e} > {tau:g}"
    return worst


def test_bwd_f32_d64_ragged():
    compare("bwd f32 d=64 T=150", grads_inputs(2, 150, 2, 64, "f32", seed=1))


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("T", [64, 200])
def test_bwd_bf16(d, T):
    compare(f"bwd bf16 d={d} T={T}", grads_inputs(2, T, 3, d, "bf16", seed=d + T))


def test_bwd_no_state_no_final_grad():
    compare("bwd S0=None dS_T=None",
            grads_inputs(2, 130, 2, 128, "bf16", seed=3, s0_std=0.0, dst=False))


def test_bwd_varlen_ragged():
    lens = [70, 0, 130, 1, 64, 200, 63]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    compare("bwd varlen", grads_inputs(1, cu[-1], 2, 128, "bf16", seed=4, cu=cu))


def test_bwd_weak_decay_long():
    inp = gi.chunk_inputs(1, 1024, 2, 128, 128, "bf16", alpha_mu=-4.0, s0_std=0.1, seed=5)
    rng = np.random.default_rng(5)
    inp["dO"] = torch.from_numpy(rng.standard_normal((1, 1024, 2, 128))).float()
    inp["dS_T"] = torch.from_numpy(rng.standard_normal((1, 2, 128, 128)) * 0.1).float()
    compare("bwd weak decay T=1024", inp)


def test_bwd_grad_dtype_bf16_is_rounded_f32():
    """With dO in bf16 the q, k, v gradients come back in bf16: the same fp32
    computation (dO upcast exactly), rounded once at the store.  (A bar
    against the oracle would have to allow for the heavy tail: rounding an
    element of 13x RMS to bf16 alone moves it by ~2.5% of RMS.)"""
    inp = grads_inputs(1, 150, 2, 128, "bf16", seed=6, g_dtype=torch.bfloat16)
    say("bwd bf16 gradients vs fp32 gradients")
    args = [dev(inp[x]) for x in ("q", "k", "v", "log_alpha", "beta")]
    g16 = gdn.chunk_bwd(*args, dev(inp["dO"]), S0=dev(inp["S0"]), dS_T=dev(inp["dS_T"]))
    g32 = gdn.chunk_bwd(*args, dev(inp["dO"]).float(), S0=dev(inp["S0"]),
                        dS_T=dev(inp["dS_T"]))
    torch.cuda.synchronize()
    for i in range(3):
        assert g16[i].dtype == torch.bfloat16
        assert torch.equal(g16[i], g32[i].to(torch.bfloat16)), NAMES[i]
    for i in range(3, 6):
        assert torch.equal(g16[i], g32[i]), NAMES[i]


def test_bwd_empty_sequence_passes_state_gradient():
    inp = grads_inputs(2, 0, 3, 128, "bf16", seed=8)
    say("bwd T=0")
    g = gdn.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["log_alpha"]),
                      dev(inp["beta"]), dev(inp["dO"]), S0=dev(inp["S0"]), dS_T=dev(inp["dS_T"]))
    torch.cuda.synchronize()
    assert torch.equal(g[5].cpu(), inp["dS_T"])


def test_bwd_deterministic():
    inp = grads_inputs(1, 200, 2, 128, "bf16", seed=9)
    say("bwd determinism")
    args = [dev(inp[x]) for x in ("q", "k", "v", "log_alpha", "beta", "dO")]
    a = gdn.chunk_bwd(*args, S0=dev(inp["S0"]), dS_T=dev(inp["dS_T"]))
    b = gdn.chunk_bwd(*args, S0=dev(inp["S0"]), dS_T=dev(inp["dS_T"]))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.slow
def test_bwd_headline_full():
    """The B=8 T=4096 H=16 d=128 bf16 workload, every gradient element."""
    w = gi.WORKLOADS[2]
    say("bwd full headline: generating inputs")
    inp = gi.workload_inputs(2)
    rng = np.random.default_rng(gi.SEED_BASE + 20)
    inp["dO"] = torch.from_numpy(
        rng.standard_normal((w["B"], w["T"], w["H"], w["dv"])).astype(np.float32))
    inp["dS_T"] = None
    compare("bwd headline full", inp)


@pytest.mark.parametrize("mode,param,shift", [("repeat", 16, 0.0), ("cluster", 1, 1.0)])
def test_bwd_structured_keys(mode, param, shift):
    """Keys repeated or nearly collinear inside a chunk (the worst-conditioned
    UT transforms; beta in (1, 2) with the clustered keys), weak decay."""
    inp = gi.structured_chunk_inputs(2, 300, 2, 128, 128, mode, param, "bf16", alpha_mu=-4.0,
                                     s0_std=0.1, beta_shift=shift, seed=71)
    rng = np.random.default_rng(72)
    inp["dO"] = torch.from_numpy(rng.standard_normal((2, 300, 2, 128))).float()
    inp["dS_T"] = torch.from_numpy(rng.standard_normal((2, 2, 128, 128)) * 0.1).float()
    compare(f"bwd keys {mode}({param}) beta+{shift}", inp)
