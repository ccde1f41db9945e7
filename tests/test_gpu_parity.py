"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bars (element-wise, max |gpu - oracle| <= tau * RMS(oracle), separately for
o and for the final states): tau = 1e-4 for fp32 inputs, 2e-2 for bf16
inputs with fp32 state and accumulation.  Every input is seeded and drawn by
gdn_inputs; the oracle sees the exact values the GPU sees (bf16 upcast).
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
TAU_F32, TAU_BF16 = 1e-4, 2e-2


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(x):
    return None if x is None else x.to(DEV)


def gpu_fwd(inp, chunk, o_dtype=torch.float32):
    cu = dev(inp["cu_seqlens"])
    o, st = gdn.chunk_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]),
                          dev(inp["log_alpha"]), dev(inp["beta"]), dev(inp["S0"]),
                          cu, chunk=chunk, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o.cpu(), st.cpu()


def ref_fwd(inp):
    return oracle.fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                      inp["S0"], inp["cu_seqlens"], threads=THREADS)


def check(name, got, ref, tau):
    err = gi.max_rel_err(got, ref)
    say(f"{name}: max err / RMS = {err:.3e} (bar {tau:g})")
    assert np.all(np.isfinite(got.double().numpy())), f"{name}: non-finite output"
    assert err <= tau, f"{name}: {err:.3e} > {tau:g}"
    return err


def compare_fwd(tag, inp, chunk, tau):
    say(f"{tag}: launch")
    o, st = gpu_fwd(inp, chunk)
    ro, rs = ref_fwd(inp)
    check(f"{tag} o", o, ro, tau)
    check(f"{tag} S_T", st, rs, tau)


# ---------------------------------------------------------------- decode step
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 36), (64, 200)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_step_small(dk, dv, io):
    d = gi.decode_inputs(3, 5, dk, dv, steps=4, dtype=io, seed=11)
    S = d["S0"].to(DEV).contiguous()
    S_ref = d["S0"]
    for t in range(4):
        say(f"step dk={dk} dv={dv} io={io} t={t}")
        o = gdn.step(dev(d["q"][t]), dev(d["k"][t]), dev(d["v"][t]),
                     dev(d["log_alpha"][t]), dev(d["beta"][t]), S)
        torch.cuda.synchronize()
        ro, S_ref = oracle.step(d["q"][t], d["k"][t], d["v"][t], d["log_alpha"][t],
                                d["beta"][t], S_ref, threads=THREADS)
        check("step o", o.cpu(), ro, TAU_F32)
        check("step S", S.cpu(), S_ref, TAU_F32)


def test_step_o_bf16_is_rounded_f32():
    d = gi.decode_inputs(2, 4, 128, 128, steps=1, seed=12)
    S1 = d["S0"].to(DEV).clone()
    S2 = d["S0"].to(DEV).clone()
    args = [dev(d[x][0]) for x in ("q", "k", "v", "log_alpha", "beta")]
    say("step o bf16 vs f32")
    o32 = gdn.step(*args, S1)
    o16 = gdn.step(*args, S2, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16))
    assert torch.equal(S1.cpu(), S2.cpu())


@pytest.mark.slow
def test_step_decode_workload_full():
    """256 consecutive steps, B=64, H=16, d=128, bf16 inputs, fp32 state.
    The oracle runs the same 256 tokens as one recurrence (step x T equals the
    forward over T tokens, pinned in the oracle tests)."""
    w = gi.WORKLOADS[4]
    d = gi.workload_inputs(4)
    S = d["S0"].to(DEV).contiguous()
    os_ = []
    qd, kd, vd = dev(d["q"]), dev(d["k"]), dev(d["v"])
    lad, bd = dev(d["log_alpha"]), dev(d["beta"])
    say("decode workload: 256 steps B=64 H=16 d=128")
    for t in range(w["steps"]):
        os_.append(gdn.step(qd[t], kd[t], vd[t], lad[t], bd[t], S))
    torch.cuda.synchronize()
    o = torch.stack(os_, 0).cpu()                       # [steps,B,H,dv]
    perm = lambda x: x.transpose(0, 1).contiguous()     # noqa: E731  [B,steps,...]
    ro, rs = oracle.fwd(perm(d["q"]), perm(d["k"]), perm(d["v"]), perm(d["log_alpha"]),
                        perm(d["beta"]), d["S0"], threads=THREADS)
    check("decode o (all steps)", perm(o), ro, TAU_BF16)
    check("decode final S", S.cpu(), rs, TAU_BF16)


# ------------------------------------------------------ chunk forward, fp32
def test_chunk_f32_workload0():
    w = gi.WORKLOADS[0]
    inp = gi.workload_inputs(0)
    compare_fwd("workload0 tiny f32", inp, w["chunk"], TAU_F32)


@pytest.mark.parametrize("dk", [16, 32, 64])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_f32_instances(dk, chunk):
    inp = gi.chunk_inputs(2, 100, 3, dk, dk, "f32", alpha_mu=0.0, s0_std=0.1, seed=dk + chunk)
    compare_fwd(f"f32 dk={dk} C={chunk} T=100", inp, chunk, TAU_F32)


def test_chunk_f32_varlen():
    lens = [37, 0, 64, 1, 90]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = gi.chunk_inputs(1, cu[-1], 2, 32, 32, "f32", s0_std=0.1, seed=5, cu_seqlens=cu)
    compare_fwd("f32 varlen", inp, 32, TAU_F32)


# ------------------------------------------------------ chunk forward, bf16 MFMA
@pytest.mark.parametrize("dk", [128, 64])
@pytest.mark.parametrize("T,s0", [(64, 0.0), (300, 0.1), (1000, 0.0)])
def test_chunk_mfma_small(dk, T, s0):
    inp = gi.chunk_inputs(2, T, 3, dk, dk, "bf16", alpha_mu=1.0, s0_std=s0, seed=T + dk)
    compare_fwd(f"mfma dk={dk} T={T} S0std={s0}", inp, 64, TAU_BF16)


def test_chunk_mfma_weak_decay():
    """alpha close to 1 (log alpha ~ -softplus(N(-4,1))): long memory, the state
    grows and nearly every token interacts with the whole chunk."""
    inp = gi.chunk_inputs(2, 640, 2, 128, 128, "bf16", alpha_mu=-4.0, s0_std=0.1, seed=3)
    compare_fwd("mfma weak decay", inp, 64, TAU_BF16)


def test_chunk_mfma_varlen_small():
    lens = [70, 0, 130, 1, 64, 200, 63]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = gi.chunk_inputs(1, cu[-1], 3, 128, 128, "bf16", s0_std=0.1, seed=6, cu_seqlens=cu)
    compare_fwd("mfma varlen ragged", inp, 64, TAU_BF16)


def test_chunk_empty_copies_state():
    for io, dk, C in (("bf16", 128, 64), ("f32", 16, 16)):
        inp = gi.chunk_inputs(2, 0, 3, dk, dk, io, s0_std=0.5, seed=7)
        say(f"empty T=0 {io}")
        o, st = gpu_fwd(inp, C)
        assert o.shape[1] == 0
        assert torch.equal(st, inp["S0"])
    inp = gi.chunk_inputs(1, 0, 2, 128, 128, "bf16", s0_std=0.0, seed=8, cu_seqlens=[0, 0, 0])
    say("empty varlen, no S0")
    _, st = gpu_fwd(inp, 64)
    assert torch.count_nonzero(st) == 0


def test_chunk_deterministic():
    inp = gi.chunk_inputs(2, 333, 4, 128, 128, "bf16", s0_std=0.1, seed=9)
    say("determinism: two runs")
    o1, s1 = gpu_fwd(inp, 64)
    o2, s2 = gpu_fwd(inp, 64)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_chunk_o_bf16_is_rounded_f32():
    inp = gi.chunk_inputs(1, 130, 2, 128, 128, "bf16", s0_std=0.1, seed=10)
    say("chunk o bf16 vs f32")
    o32, s32 = gpu_fwd(inp, 64)
    o16, s16 = gpu_fwd(inp, 64, o_dtype=torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s16, s32)


def test_chunk_split_resume():
    """Running [0,T1) then [T1,T) from the carried state matches the oracle."""
    inp = gi.chunk_inputs(2, 320, 2, 128, 128, "bf16", s0_std=0.1, seed=13)
    t1 = 150
    a = {k: (v[:, :t1].contiguous() if k in ("q", "k", "v", "log_alpha", "beta") else v)
         for k, v in inp.items()}
    say("split resume part 1")
    oa, sa = gpu_fwd(a, 64)
    b = {k: (v[:, t1:].contiguous() if k in ("q", "k", "v", "log_alpha", "beta") else v)
         for k, v in inp.items()}
    b["S0"] = sa
    say("split resume part 2")
    ob, sb = gpu_fwd(b, 64)
    ro, rs = ref_fwd(inp)
    check("split o", torch.cat([oa, ob], 1), ro, TAU_BF16)
    check("split S_T", sb, rs, TAU_BF16)


def test_step_matches_chunk_on_gpu():
    """T decode steps and one chunked forward agree (both against the oracle)."""
    inp = gi.chunk_inputs(2, 96, 3, 128, 128, "bf16", s0_std=0.1, seed=14)
    S = inp["S0"].to(DEV).clone()
    outs = []
    say("step x 96 vs chunk")
    for t in range(96):
        outs.append(gdn.step(*(dev(inp[x][:, t].contiguous())
                               for x in ("q", "k", "v", "log_alpha", "beta")), S))
    torch.cuda.synchronize()
    o_step = torch.stack(outs, 1).cpu()
    o_chunk, s_chunk = gpu_fwd(inp, 64)
    ro, rs = ref_fwd(inp)
    check("steps o", o_step, ro, TAU_F32)
    check("steps S", S.cpu(), rs, TAU_F32)
    check("chunk o", o_chunk, ro, TAU_BF16)
    check("chunk S", s_chunk, rs, TAU_BF16)


def test_chunk_guard_bands():
    """Writes stay inside o and S_T: sentinels around both are untouched."""
    inp = gi.chunk_inputs(2, 130, 3, 128, 128, "bf16", s0_std=0.1, seed=15)
    B, T, H, dv, dk = 2, 130, 3, 128, 128
    pad = 64
    n_o, n_s = B * T * H * dv, B * H * dv * dk
    ob = torch.full((n_o + 2 * pad,), 12345.0, device=DEV)
    sb = torch.full((n_s + 2 * pad,), 12345.0, device=DEV)
    o = ob[pad:pad + n_o].view(B, T, H, dv)
    st = sb[pad:pad + n_s].view(B, H, dv, dk)
    say("guard bands")
    gdn.chunk_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["log_alpha"]),
                  dev(inp["beta"]), dev(inp["S0"]), o=o, S_T=st)
    torch.cuda.synchronize()
    for buf in (ob, sb):
        c = buf.cpu()
        assert torch.all(c[:pad] == 12345.0) and torch.all(c[-pad:] == 12345.0)


# ------------------------------------------------------ full-size workloads
@pytest.mark.slow
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_workload_full(wid):
    w = gi.WORKLOADS[wid]
    say(f"workload {wid} ({w['name']}) full size: generating inputs")
    inp = gi.workload_inputs(wid)
    compare_fwd(f"workload {wid} full", inp, w["chunk"], TAU_BF16)
