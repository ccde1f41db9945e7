"""Degenerate gates on the GPU: no decay and nothing written.

With log alpha = 0 and beta = 0 (for Gated DeltaNet-2: erase = write = 0)
every term of the update vanishes, so the state passes through unchanged
and each read-out is o_t = S0 q_t ("Gated Delta Networks: Improving Mamba2
with Delta Rule", research-map summary, section "Approach": alpha_t = 1
keeps the state and beta_t = 0 writes nothing; "Gated DeltaNet-2:
Decoupling Erase and Write in Linear Attention", abstract: the erase and
write gates scale the removed and the added terms).  In the kernels every
decay is then exp2(0) = 1 exactly and the factors that carry beta (erase,
write) are exactly zero, so the final state must equal S0 bit for bit; o is
checked against S0 q computed in fp64 and against the oracle, at the
parity bars of each path.  With the decays kept and nothing written, the
state only decays: S_t = S0 Diag(e^{G_t}) with G_t the prefix sum of log
alpha (per key channel for the channel-wise rules), a closed form that the
pure-decay tests compare o and the final state with.
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


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(x):
    return None if x is None else x.to(DEV)


def frozen(inp):
    """The same inputs with log alpha = 0 and every write gate 0."""
    out = dict(inp)
    for name in ("log_alpha", "beta", "erase", "write"):
        if out.get(name) is not None:
            out[name] = torch.zeros_like(out[name])
    return out


def s0_q(inp):
    """o_t = S0 q_t in fp64, per sequence (S0 [U, H, dv, dk], q [B, T, H, dk])."""
    q = inp["q"].double().numpy()
    S0 = inp["S0"].double().numpy()
    o = np.zeros(q.shape[:3] + (S0.shape[2],))
    cu = inp["cu_seqlens"]
    if cu is None:
        return np.einsum("bhvk,bthk->bthv", S0, q)
    cu = [int(x) for x in cu]
    for u in range(len(cu) - 1):
        o[0, cu[u]:cu[u + 1]] = np.einsum("hvk,thk->thv", S0[u], q[0, cu[u]:cu[u + 1]])
    return o


def check(tag, o, st, inp, ref_o, tau):
    S0 = inp["S0"]
    assert torch.equal(st.cpu(), S0), f"{tag}: S_T differs from S0"
    for name, want in (("o vs S0 q", s0_q(inp)), ("o vs oracle", ref_o)):
        err = gi.max_rel_err(o.cpu(), want)
        say(f"{tag} {name}: max err / RMS = {err:.3e} (bar {tau:g})")
        assert err <= tau, f"{tag} {name}: {err:.3e} > {tau:g}"


@pytest.mark.parametrize("io,d,chunk,tau", [("bf16", 128, 64, 2e-2), ("bf16", 64, 64, 2e-2),
                                            ("f32", 32, 32, 1e-4)])
def test_chunk_fwd_frozen_state(io, d, chunk, tau):
    inp = frozen(gi.chunk_inputs(2, 150, 3, d, d, io, s0_std=0.5, seed=71))
    tag = f"chunk_fwd {io} d={d} C={chunk}"
    say(f"{tag}: launch")
    o, st = gdn.chunk_fwd(*(dev(inp[n]) for n in ("q", "k", "v", "log_alpha", "beta", "S0")),
                          chunk=chunk)
    torch.cuda.synchronize()
    ro, _ = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"],
                       threads=THREADS)
    check(tag, o, st, inp, ro, tau)


def test_chunk_fwd_frozen_state_varlen():
    lens = [70, 0, 130, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = frozen(gi.chunk_inputs(1, cu[-1], 2, 128, 128, "bf16", s0_std=0.5, seed=72,
                                 cu_seqlens=cu))
    say("chunk_fwd varlen: launch")
    o, st = gdn.chunk_fwd(*(dev(inp[n]) for n in ("q", "k", "v", "log_alpha", "beta", "S0")),
                          dev(inp["cu_seqlens"]))
    torch.cuda.synchronize()
    ro, _ = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"],
                       inp["cu_seqlens"], threads=THREADS)
    check("chunk_fwd varlen", o, st, inp, ro, 2e-2)


def test_kda_fwd_frozen_state():
    inp = frozen(gi.kda_inputs(2, 150, 3, 128, 128, "bf16", s0_std=0.5, seed=73))
    say("kda_fwd: launch")
    o, st = gdn.kda_fwd(*(dev(inp[n]) for n in ("q", "k", "v", "log_alpha", "beta", "S0")))
    torch.cuda.synchronize()
    ro, _ = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                           inp["S0"], threads=THREADS)
    check("kda_fwd", o, st, inp, ro, 1e-3)


def test_gdn2_fwd_frozen_state():
    inp = frozen(gi.gdn2_inputs(2, 150, 3, 128, 128, "bf16", s0_std=0.5, seed=74))
    say("gdn2_fwd: launch")
    o, st = gdn.gdn2_fwd(*(dev(inp[n]) for n in ("q", "k", "v", "log_alpha", "erase", "write",
                                                 "S0")))
    torch.cuda.synchronize()
    ro, _ = oracle.gdn2_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["erase"],
                            inp["write"], inp["S0"], threads=THREADS)
    check("gdn2_fwd", o, st, inp, ro, 1e-3)


def test_step_frozen_state():
    rng = np.random.default_rng(75)
    B, H, d = 3, 4, 128
    k = rng.standard_normal((B, H, d))
    q = torch.from_numpy(rng.standard_normal((B, H, d))).to(torch.bfloat16)
    kk = torch.from_numpy(k / np.linalg.norm(k, axis=-1, keepdims=True)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, H, d))).to(torch.bfloat16)
    zeros = torch.zeros((B, H), dtype=torch.float32)
    S0 = torch.from_numpy(rng.standard_normal((B, H, d, d)) * 0.5).float()
    S = dev(S0).clone()
    say("step: launch")
    o = gdn.step(dev(q), dev(kk), dev(v), dev(zeros), dev(zeros), S)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), S0), "step: S differs from S0"
    want = np.einsum("bhvk,bhk->bhv", S0.double().numpy(), q.double().numpy())
    err = gi.max_rel_err(o.cpu(), want)
    say(f"step o vs S0 q: max err / RMS = {err:.3e} (bar 1e-4)")
    assert err <= 1e-4


def no_writes(inp):
    """The same inputs with every write gate 0 (decays kept)."""
    out = dict(inp)
    for name in ("beta", "erase", "write"):
        if out.get(name) is not None:
            out[name] = torch.zeros_like(out[name])
    return out


def decayed(inp, channelwise):
    """Pure decay in fp64: S_t = S0 Diag(e^{G_t}) with G_t the prefix sum of
    log alpha (a scalar per token for the scalar rule, per key channel
    otherwise); returns (o_t = S_t q_t for every token, S_T)."""
    q = inp["q"].double().numpy()
    la = inp["log_alpha"].double().numpy()
    S0 = inp["S0"].double().numpy()
    G = np.cumsum(la, axis=1)                      # [B, T, H] or [B, T, H, dk]
    eG = np.exp(G) if channelwise else np.exp(G)[..., None]
    o = np.einsum("bhvk,bthk->bthv", S0, eG * q)
    last = eG[:, -1]                               # [B, H, dk] or [B, H, 1]
    S_T = S0 * last[:, :, None, :]
    return o, S_T


@pytest.mark.parametrize("which", ["chunk", "kda", "gdn2"])
def test_pure_decay_matches_closed_form(which):
    # weak decays (log alpha = -softplus(N(-4, 1)), about -0.02 per token), so
    # the state keeps a few per cent of S0 over the 150 tokens
    B, T, H, d = 2, 150, 3, 128
    if which == "chunk":
        inp = no_writes(gi.chunk_inputs(B, T, H, d, d, "bf16", alpha_mu=-4.0, s0_std=0.5, seed=76))
        args = ("q", "k", "v", "log_alpha", "beta", "S0")
        fwd, tau = gdn.chunk_fwd, 2e-2
    elif which == "kda":
        inp = no_writes(gi.kda_inputs(B, T, H, d, d, "bf16", alpha_mu=-4.0, s0_std=0.5, seed=77))
        args = ("q", "k", "v", "log_alpha", "beta", "S0")
        fwd, tau = gdn.kda_fwd, 1e-3
    else:
        inp = no_writes(gi.gdn2_inputs(B, T, H, d, d, "bf16", alpha_mu=-4.0, s0_std=0.5, seed=78))
        args = ("q", "k", "v", "log_alpha", "erase", "write", "S0")
        fwd, tau = gdn.gdn2_fwd, 1e-3
    say(f"{which} pure decay: launch")
    o, st = fwd(*(dev(inp[n]) for n in args))
    torch.cuda.synchronize()
    want_o, want_s = decayed(inp, which != "chunk")
    for name, got, want in (("o", o, want_o), ("S_T", st, want_s)):
        err = gi.max_rel_err(got.cpu(), want)
        say(f"{which} pure decay {name}: max err / RMS = {err:.3e} (bar {tau:g})")
        assert err <= tau, f"{which} pure decay {name}: {err:.3e} > {tau:g}"


def overwrite_inputs(which, B, T, H, d, seed):
    """alpha = 1, beta = 1 (GDN-2: erase = write = 1) and keys that are
    distinct basis vectors e_j of the key space: each token replaces column j
    of the state by its value, S <- S (I - e_j e_j^T) + v e_j^T (the delta
    rule's exact overwrite).  Returns the inputs and the basis index of every
    token, [B, T, H]."""
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([rng.permutation(d)[:T] for _ in range(H)], axis=-1)
                    for _ in range(B)])                       # [B, T, H]
    k = np.zeros((B, T, H, d))
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    bf = torch.bfloat16
    inp = dict(q=torch.from_numpy(rng.standard_normal((B, T, H, d))).to(bf),
               k=torch.from_numpy(k).to(bf),
               v=torch.from_numpy(rng.standard_normal((B, T, H, d))).to(bf),
               S0=torch.from_numpy(rng.standard_normal((B, H, d, d)) * 0.5).float(),
               cu_seqlens=None)
    if which == "chunk":
        inp["log_alpha"] = torch.zeros((B, T, H))
        inp["beta"] = torch.ones((B, T, H))
    else:
        inp["log_alpha"] = torch.zeros((B, T, H, d))
        if which == "kda":
            inp["beta"] = torch.ones((B, T, H))
        else:
            inp["erase"] = torch.ones((B, T, H, d))
            inp["write"] = torch.ones((B, T, H, d))
    return inp, idx


def overwritten(inp, idx):
    """Token by token in fp64: column idx[t] of S becomes v_t; o_t = S_t q_t."""
    q = inp["q"].double().numpy()
    v = inp["v"].double().numpy()
    S = inp["S0"].double().numpy().copy()
    B, T, H, _ = q.shape
    o = np.zeros(v.shape)
    for t in range(T):
        for b in range(B):
            for h in range(H):
                S[b, h, :, idx[b, t, h]] = v[b, t, h]
                o[b, t, h] = S[b, h] @ q[b, t, h]
    return o, S


@pytest.mark.parametrize("which,d,T,tau", [("chunk", 128, 100, 2e-2), ("chunk", 64, 60, 2e-2),
                                           ("kda", 128, 100, 1e-3), ("gdn2", 128, 100, 1e-3)])
def test_exact_overwrite_with_basis_keys(which, d, T, tau):
    # The scalar-gate chunk kernel forms K S^T from the hi (bf16) part of the
    # state only, so an overwritten column keeps its old lo part, about 2^-9
    # of |S0|: some 1e-2 of RMS at most, inside that path's bar.  The KDA and
    # GDN-2 launches carry every operand as a hi + lo pair (near 1e-5).
    inp, idx = overwrite_inputs(which, 2, T, 2, d, seed=79 + d)
    if which == "gdn2":
        args, fwd = ("q", "k", "v", "log_alpha", "erase", "write", "S0"), gdn.gdn2_fwd
    else:
        args = ("q", "k", "v", "log_alpha", "beta", "S0")
        fwd = gdn.chunk_fwd if which == "chunk" else gdn.kda_fwd
    say(f"{which} exact overwrite d={d} T={T}: launch")
    o, st = fwd(*(dev(inp[n]) for n in args))
    torch.cuda.synchronize()
    want_o, want_s = overwritten(inp, idx)
    for name, got, want in (("o", o, want_o), ("S_T", st, want_s)):
        err = gi.max_rel_err(got.cpu(), want)
        say(f"{which} exact overwrite {name}: max err / RMS = {err:.3e} (bar {tau:g})")
        assert err <= tau, f"{which} exact overwrite {name}: {err:.3e} > {tau:g}"


def frozen_grads(inp, dO, dS_T):
    """Gradients of <dO, o> + <dS_T, S_T> at alpha = 1, beta = 0, in fp64.
    There o_t = S0 q_t and S_T = S0, so dq_t = S0^T dO_t, dS0 = sum_t dO_t
    q_t^T + dS_T, and every path to k or v carries a factor beta: dk = dv =
    0.  d log alpha_s scales S_t for t >= s: dla_s = sum_{t>=s} <dO_t, o_t>
    + <dS_T, S0>.  d beta_s adds (v_s - S0 k_s) k_s^T to every later state:
    dbeta_s = sum_{t>=s} (dO_t . u_s)(k_s . q_t) + u_s^T dS_T k_s with
    u_s = v_s - S0 k_s."""
    q, k, v = (inp[n].double().numpy() for n in ("q", "k", "v"))
    S0 = inp["S0"].double().numpy()
    dO = dO.double().numpy()
    dST = dS_T.double().numpy()
    o = np.einsum("bhvk,bthk->bthv", S0, q)
    dq = np.einsum("bhvk,bthv->bthk", S0, dO)
    dS0 = np.einsum("bthv,bthk->bhvk", dO, q) + dST
    c = np.einsum("bthv,bthv->bth", dO, o)                       # <dO_t, o_t>
    tail = np.flip(np.cumsum(np.flip(c, 1), 1), 1)              # sum over t >= s
    dla = tail + np.einsum("bhvk,bhvk->bh", dST, S0)[:, None, :]
    u = v - np.einsum("bhvk,bshk->bshv", S0, k)                  # u_s
    du = np.einsum("bthv,bshv->bsth", dO, u)                     # dO_t . u_s  [b, s, t, h]
    kq = np.einsum("bshk,bthk->bsth", k, q)                      # k_s . q_t
    T = q.shape[1]
    later = np.triu(np.ones((T, T)))[None, :, :, None]           # t >= s
    dbeta = (du * kq * later).sum(2) + np.einsum("bshv,bhvk,bshk->bsh", u, dST, k)
    return dq, dla, dbeta, dS0


def test_bwd_frozen_state_closed_form():
    B, T, H, d = 2, 150, 2, 128
    inp = frozen(gi.chunk_inputs(B, T, H, d, d, "bf16", s0_std=0.5, seed=83))
    rng = np.random.default_rng(84)
    dO = torch.from_numpy(rng.standard_normal((B, T, H, d))).float()
    dS_T = torch.from_numpy(rng.standard_normal((B, H, d, d)) * 0.1).float()
    say(f"chunk_bwd alpha=1 beta=0 B={B} T={T} H={H} d={d}: launch")
    g = gdn.chunk_bwd(*(dev(inp[n]) for n in ("q", "k", "v", "log_alpha", "beta")), dev(dO),
                      S0=dev(inp["S0"]), dS_T=dev(dS_T))
    torch.cuda.synchronize()
    dq, dk, dv, dla, dbeta, dS0 = (x.cpu() for x in g)
    want = dict(zip(("dq", "dlog_alpha", "dbeta", "dS0"), frozen_grads(inp, dO, dS_T)))
    for name, got in (("dq", dq), ("dlog_alpha", dla), ("dbeta", dbeta), ("dS0", dS0)):
        err = gi.max_rel_err(got, want[name])
        say(f"bwd frozen {name}: max err / RMS = {err:.3e} (bar 1e-3)")
        assert err <= 1e-3, f"bwd frozen {name}: {err:.3e} > 1e-3"
    scale = float(np.sqrt(np.mean(want["dq"] ** 2)))
    for name, got in (("dk", dk), ("dv", dv)):
        m = float(got.abs().max())
        say(f"bwd frozen {name}: max |x| = {m:.3e} (zero expected)")
        assert m <= 1e-6 * scale, f"bwd frozen {name}: {m:.3e} is not zero"
