"""Parity of the Gated DeltaNet-2 forward, through the C ABI, with the fp64
oracle ``oracle.gdn2_fwd`` (pins in tests/test_oracle_gdn2.py).

The GPU computes the chunk factors in fp32 and every product of the
sequential launch from hi + lo bf16 pairs (about 16 mantissa bits per
operand, three piece products), so the bar is max |gpu - oracle| <= 1e-3 *
RMS(oracle) on o and on the final states.
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


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(x):
    return None if x is None else x.to(DEV)


def run(inp, o_dtype=torch.float32):
    o, st = gdn.gdn2_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["log_alpha"]),
                         dev(inp["erase"]), dev(inp["write"]), dev(inp["S0"]),
                         dev(inp["cu_seqlens"]), o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, st


def compare(tag, inp, tau=TAU):
    say(f"{tag}: launch")
    o, st = run(inp)
    ro, rs = oracle.gdn2_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["erase"],
                             inp["write"], inp["S0"], inp["cu_seqlens"], threads=THREADS)
    for name, got, want in (("o", o.cpu(), ro), ("S_T", st.cpu(), rs)):
        err = gi.max_rel_err(got, want)
        say(f"{tag} {name}: max err / RMS = {err:.3e} (bar {tau:g})")
        assert np.all(np.isfinite(got.double().numpy())), f"{tag} {name}: non-finite"
        assert err <= tau, f"{tag} {name}: {err:.3e} > {tau:g}"


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("T", [64, 200])
def test_gdn2_bf16(d, T):
    compare(f"gdn2 bf16 d={d} T={T}", gi.gdn2_inputs(2, T, 3, d, d, "bf16", s0_std=0.1,
                                                     seed=d + T))


def test_gdn2_f32_d64_ragged():
    compare("gdn2 f32 d=64 T=150", gi.gdn2_inputs(2, 150, 2, 64, 64, "f32", s0_std=0.1, seed=3))


def test_gdn2_varlen_ragged():
    lens = [70, 0, 130, 1, 64, 200, 63]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    compare("gdn2 varlen", gi.gdn2_inputs(1, cu[-1], 2, 128, 128, "bf16", s0_std=0.1, seed=4,
                                          cu_seqlens=cu))


def test_gdn2_extreme_channels():
    inp = gi.gdn2_inputs(1, 256, 2, 128, 128, "bf16", alpha_mu=2.0, alpha_sd=5.0, s0_std=0.1,
                         seed=5)
    compare("gdn2 extreme channel decays", inp)


def test_gdn2_decays_at_the_term_threshold():
    """Per-channel decays of about e^-3 per token put the decay span of a
    16-token diagonal block around e^-60, the limit above which the prep
    forms the block term by term: in one launch some diagonal blocks take the
    rescaled product and the others the term-by-term path (19 of 64 here)."""
    inp = gi.gdn2_inputs(1, 512, 2, 128, 128, "bf16", alpha_mu=3.0, alpha_sd=1.0, s0_std=0.1,
                         seed=81)
    compare("gdn2 decays at the term threshold", inp)


def test_gdn2_scalar_gates_match_kda():
    """b_t = w_t = beta_t in every channel: gdn_kda_fwd's rule (both GPU runs
    against each other; each is checked against its oracle elsewhere).  The
    two launches factor the chunk differently and form their products from
    hi + lo bf16 pairs, so they agree to the sum of their own errors (each
    about 1e-4 of RMS here), held to the parity bar."""
    inp = gi.kda_inputs(1, 200, 2, 128, 128, "bf16", s0_std=0.1, seed=6)
    b = inp["beta"][..., None]
    g2 = dict(inp, erase=b.expand(1, 200, 2, 128).contiguous(),
              write=b.expand(1, 200, 2, 128).contiguous())
    say("gdn2 with scalar gates vs kda")
    o2, s2 = run(g2)
    ok, sk = gdn.kda_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["log_alpha"]),
                         dev(inp["beta"]), dev(inp["S0"]))
    torch.cuda.synchronize()
    e1, e2 = gi.max_rel_err(o2.cpu(), ok.cpu()), gi.max_rel_err(s2.cpu(), sk.cpu())
    say(f"gdn2 vs kda: o {e1:.2e}, S {e2:.2e}")
    assert e1 <= TAU and e2 <= TAU


@pytest.mark.slow
def test_gdn2_headline_shape_full():
    say("gdn2 full: generating inputs")
    inp = gi.gdn2_inputs(8, 4096, 16, 128, 128, "bf16", alpha_mu=1.0, seed=gi.SEED_BASE + 40)
    compare("gdn2 full 1.3b-layer shape", inp)


@pytest.mark.parametrize("mode,param", [("repeat", 16), ("cluster", 1)])
def test_gdn2_structured_keys(mode, param):
    """Keys repeated or nearly collinear inside a chunk, weak channel decays."""
    inp = gi.gdn2_inputs(2, 300, 2, 128, 128, "bf16", alpha_mu=-4.0, s0_std=0.1, seed=75)
    inp["k"] = gi.structured_chunk_inputs(2, 300, 2, 128, 128, mode, param, "bf16", seed=76)["k"]
    compare(f"gdn2 keys {mode}({param})", inp)
