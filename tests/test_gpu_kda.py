"""Parity of the channel-wise decay (KDA) forward, through the C ABI, with
the fp64 oracle ``oracle.kda_fwd`` (pins in tests/test_oracle_kda.py).

The GPU computes A, P and T in fp32 and every product of the sequential
launch from hi + lo bf16 pairs (about 16 mantissa bits per operand, three
piece products), so the bar is max |gpu - oracle| <= 1e-3 * RMS(oracle) on o
and on the final states.
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


def compare(tag, inp, o_dtype=torch.float32, tau=TAU):
    say(f"{tag}: launch")
    o, st = gdn.kda_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["log_alpha"]),
                        dev(inp["beta"]), dev(inp["S0"]), dev(inp["cu_seqlens"]),
                        o_dtype=o_dtype)
    torch.cuda.synchronize()
    ro, rs = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                            inp["S0"], inp["cu_seqlens"], threads=THREADS)
    for name, got, want in (("o", o.cpu(), ro), ("S_T", st.cpu(), rs)):
        err = gi.max_rel_err(got, want)
        say(f"{tag} {name}: max err / RMS = {err:.3e} (bar {tau:g})")
        assert np.all(np.isfinite(got.double().numpy())), f"{tag} {name}: non-finite"
        assert err <= tau, f"{tag} {name}: {err:.3e} > {tau:g}"


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("T", [64, 200])
def test_kda_bf16(d, T):
    compare(f"kda bf16 d={d} T={T}", gi.kda_inputs(2, T, 3, d, d, "bf16", s0_std=0.1, seed=d + T))


def test_kda_f32_d64_ragged():
    compare("kda f32 d=64 T=150", gi.kda_inputs(2, 150, 2, 64, 64, "f32", s0_std=0.1, seed=3))


def test_kda_varlen_ragged():
    lens = [70, 0, 130, 1, 64, 200, 63]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    compare("kda varlen", gi.kda_inputs(1, cu[-1], 2, 128, 128, "bf16", s0_std=0.1, seed=4,
                                        cu_seqlens=cu))


def test_kda_strong_and_weak_channels():
    """Per-channel decays from ~e^-12 to ~1 per token: the intra-chunk
    products must stay finite and exact (operands are rescaled in blocks)."""
    inp = gi.kda_inputs(1, 256, 2, 128, 128, "bf16", alpha_mu=2.0, alpha_sd=5.0, s0_std=0.1,
                        seed=5)
    compare("kda extreme channel decays", inp)


def test_kda_decays_at_the_term_threshold():
    """Per-channel decays of about e^-3 per token put the decay span of a
    16-token diagonal block around e^-60, the limit above which the prep
    forms the block term by term: in one launch some diagonal blocks take the
    rescaled product and the others the term-by-term path (19 of 64 here)."""
    inp = gi.kda_inputs(1, 512, 2, 128, 128, "bf16", alpha_mu=3.0, alpha_sd=1.0, s0_std=0.1,
                        seed=81)
    compare("kda decays at the term threshold", inp)


def test_kda_uniform_channels_match_scalar_rule():
    """Equal channels: the same rule as gdn_chunk_fwd (both against the oracle)."""
    inp = gi.chunk_inputs(2, 200, 2, 128, 128, "bf16", s0_std=0.1, seed=6)
    kin = dict(inp, log_alpha=inp["log_alpha"][..., None].expand(2, 200, 2, 128).contiguous())
    compare("kda uniform channels", kin)


def test_kda_o_bf16_is_rounded_f32():
    inp = gi.kda_inputs(1, 130, 2, 128, 128, "bf16", s0_std=0.1, seed=7)
    say("kda o bf16 vs f32")
    args = [dev(inp[x]) for x in ("q", "k", "v", "log_alpha", "beta", "S0")]
    o32, s32 = gdn.kda_fwd(*args)
    o16, s16 = gdn.kda_fwd(*args, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s16, s32)


@pytest.mark.slow
def test_kda_headline_shape_full():
    """B=8 T=4096 H=16 d=128 bf16 with channel-wise decays, every element."""
    say("kda full: generating inputs")
    inp = gi.kda_inputs(8, 4096, 16, 128, 128, "bf16", alpha_mu=1.0, seed=gi.SEED_BASE + 30)
    compare("kda full 1.3b-layer shape", inp)


@pytest.mark.parametrize("mode,param,shift", [("repeat", 16, 0.0), ("cluster", 1, 1.0)])
def test_kda_structured_keys(mode, param, shift):
    """Keys repeated or nearly collinear inside a chunk, weak channel decays."""
    inp = gi.kda_inputs(2, 300, 2, 128, 128, "bf16", alpha_mu=-4.0, s0_std=0.1, seed=73)
    sk = gi.structured_chunk_inputs(2, 300, 2, 128, 128, mode, param, "bf16", seed=74,
                                    beta_shift=shift)
    inp["k"], inp["beta"] = sk["k"], sk["beta"]
    compare(f"kda keys {mode}({param}) beta+{shift}", inp)
