"""Benchmark of the gated-delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one gdn_chunk_fwd over the 1.3B-layer-shaped workload (B=8,
T=4096, H=16, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 gates, fp32 o and
state) with every input already resident in HBM.  The JSON line reports:
  value       whole-job tokens/s (B*T tokens per step);
  roofline    the chunk kernel against the HBM roofline (its algorithmic
              arithmetic intensity is below the bf16 MFMA ridge point), with
              the launch time measured by HIP events on the launch stream;
  mfma        the same launches against the dense bf16 MFMA peak;
  decode      gdn_step on B=64, H=16, d=128 (fp32 state in place): HBM GB/s
              with the state evicted from the caches before each step
              ("cold"), and back to back ("warm");
  backward    gdn_chunk_bwd on the same workload: ms, tokens/s and its fp32
              MFMA roofline (the arithmetic its kernels execute);
  kda_forward the channel-wise decay forward (gdn_kda_fwd) on the same
              shape: ms, tokens/s, fp32 MFMA roofline;
  gdn2_forward the Gated DeltaNet-2 forward (gdn_gdn2_fwd) on the same shape;
  fused_prologue the same forward on raw projections with the input
              prologue (L2 norm of q, k; gate activations) inside the kernel,
              beside the same prologue done as separate torch ops;
  cpu_baseline the fp64 CPU oracle timed on a bounded sample of the same
              workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gated-delta chunk-fwd tokens/s at B8 T4096 H16 d128; % MFMA peak; decode GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published
MFMA_FP32_PEAK_TFS = 157.3     # MI355X dense fp32 (matrix and vector), published
PMC_FILE = os.path.join(ROOT, "profiles", "chunk_mfma_b8_t4096_h16_d128_traffic.json")


def kernel_source_sha256() -> str:
    """Hash of the chunk kernel's sources (the kernel file and its header)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("chunk_mfma.hip", "gdn_common.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_58_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def flops_per_token_head(C: int, dk: int, dv: int) -> float:
    """Algorithmic flops of the chunk algorithm per (token, head): K K^T
    (strict lower), forward substitution, U, W, Delta + state update + Q S^T,
    Q K^T (with diagonal) and P Delta; 2 flops per multiply-add."""
    L, Lp = C * (C - 1) // 2, C * (C + 1) // 2
    macs = (L * dk + C * (C - 1) * (C - 2) // 6 + L * dv + L * dk + 3 * C * dk * dv
            + Lp * dk + Lp * dv)
    return 2.0 * macs / C


def bytes_chunk_fwd(B, T, H, dk, dv, io_bytes=2, o_bytes=4, with_s0=False,
                    units=None) -> float:
    """Algorithmic HBM bytes of one forward over B*T tokens: q, k, v, gates read
    once, o and the final states written once (initial states read once if
    given); `units` states (default B: one per batch row or packed sequence)."""
    per_th = (2 * dk + dv) * io_bytes + dv * o_bytes + 8
    units = B if units is None else units
    states = units * H * dv * dk * 4 * (2 if with_s0 else 1)
    return B * T * H * per_th + states


PREHEAT_MS = 250.0   # GPU time run before each leg's counted warm-up
MIN_TIMED = 10       # timed calls of every sub-leg, at least


def set_preheat(ms: float) -> None:
    global PREHEAT_MS
    PREHEAT_MS = ms


def preheat(torch, fn, min_ms=None):
    """Run fn back to back until at least min_ms of GPU time has passed.  The
    GPU needs tens of milliseconds of sustained load to reach its steady
    clock; without this a short counted warm-up ends while the clock is still
    ramping.  Returns (GPU ms, calls)."""
    min_ms = PREHEAT_MS if min_ms is None else min_ms
    stream = torch.cuda.current_stream()
    total, calls = 0.0, 0
    while total < min_ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(4):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
        calls += 4
    return total, calls


def time_calls(torch, fn, n, warm=0):
    """ms per call of fn over n back-to-back calls (HIP events on the stream
    the calls are launched on), after a pre-heat and `warm` untimed calls."""
    preheat(torch, fn)
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def run_decode(args, torch, gi, gdn, dev):
    """Time gdn_step on the decode workload; returns the JSON sub-object."""
    wd = gi.WORKLOADS[4]
    print("[bench] decode: workload 4", file=sys.stderr, flush=True)
    dh = gi.workload_inputs(4)
    dd = {k: v.to(dev) for k, v in dh.items()}
    S = dd["S0"].clone()
    Bd, Hd = wd["B"], wd["H"]
    od = torch.empty((Bd, Hd, wd["dv"]), device=dev, dtype=torch.float32)
    nsteps = min(args.decode_steps, wd["steps"])

    def dstep(t):
        gdn.step(dd["q"][t], dd["k"][t], dd["v"][t], dd["log_alpha"][t], dd["beta"][t], S, o=od)

    preheat(torch, lambda: dstep(0))
    torch.cuda.synchronize()
    S.copy_(dd["S0"])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(nsteps):
        dstep(t)
    e1.record(stream)
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / nsteps
    # Evict the state from L2 and the 256 MB MALL by READING 1 GiB before each
    # timed step (a write-based flush would leave dirty lines that drain to
    # HBM during the timed step).
    flush = torch.zeros(1 << 28, device=dev, dtype=torch.float32)
    torch.cuda.synchronize()
    cold = []
    for t in range(args.cold_steps):
        flush.sum()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record(stream)
        dstep(t)
        eb.record(stream)
        torch.cuda.synchronize()
        cold.append(ea.elapsed_time(eb) * 1e3)
    del flush
    cold.sort()
    cold_us = cold[len(cold) // 2]
    # the same steps replayed from one HIP graph (a serving loop captures its
    # decode steps once): no launch gaps between steps, state in the MALL
    gsteps = min(nsteps, 64)
    S.copy_(dd["S0"])
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for t in range(gsteps):
            dstep(t)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(gsteps):
            dstep(t)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / gsteps
    del graph
    dbytes = (2 * Bd * Hd * wd["dv"] * wd["dk"] * 4 + Bd * Hd * (2 * wd["dk"] + wd["dv"]) * 2
              + Bd * Hd * wd["dv"] * 4 + Bd * Hd * 8)
    decode = {
        "workload": f"{wd['name']}: B={Bd} H={Hd} d_k=d_v={wd['dk']}, bf16 q/k/v, fp32 state",
        "bytes_per_step": dbytes,
        "us_per_step_cold": round(cold_us, 2),
        "GB_s_cold": round(dbytes / (cold_us * 1e-6) / 1e9, 1),
        "frac_hbm_cold": round(dbytes / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "us_per_step_warm": round(warm_us, 2),
        "GB_s_warm": round(dbytes / (warm_us * 1e-6) / 1e9, 1),
        "us_per_step_graph": round(graph_us, 2),
        "GB_s_graph": round(dbytes / (graph_us * 1e-6) / 1e9, 1),
        "note": "cold = 1 GiB cache-evicting read before each timed step (median of "
                f"{args.cold_steps}); warm = {nsteps} steps back to back, state resident in "
                f"MALL; graph = {gsteps} steps replayed from one captured HIP graph",
    }

    if args.only == "decode":
        print(json.dumps({"decode": decode}))
    return decode


def bwd_flops_per_chunk_head(d: int, C: int = 64) -> float:
    """fp32 MFMA flops the backward launches execute per (chunk, head): the
    tiles of each product, 2 flop per multiply-add (prep: the lower 10 of 16
    tiles of K K^T and Q K^T; states: K S^T, T Z, the update; dstates: P^T dO,
    K dS'^T, T^T dDelta, two update products; sprod: three C x d x d
    products; grads: ten C-row products and two C^3 ones)."""
    cdd = 2.0 * C * d * d
    ccd = 2.0 * C * C * d
    prep = 2 * 10 * 2.0 * 16 * 16 * d
    states = cdd + ccd + cdd
    dstates = ccd + cdd + ccd + 2 * cdd
    sprod = 3 * cdd
    grads = 10 * ccd + 2 * 2.0 * C ** 3
    return prep + states + dstates + sprod + grads


def run_backward(args, torch, gi, gdn, dev, w, host):
    """Time gdn_chunk_bwd on the same workload (dO ~ N(0,1) fp32, no final
    state gradient), workspace and inputs resident."""
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["chunk"]
    print("[bench] backward", file=sys.stderr, flush=True)
    d = {k: (v.to(dev) if v is not None else None) for k, v in host.items()}
    g = torch.Generator(device=dev).manual_seed(gi.SEED_BASE + 20)
    dO = torch.randn((B, T, H, dv), device=dev, dtype=torch.float32, generator=g)
    nbytes = gdn.chunk_bwd_workspace_size(B, T, H, dk, dv, C)
    ws = torch.empty(nbytes, device=dev, dtype=torch.uint8)
    steps, warm = max(MIN_TIMED, args.steps // 10), max(1, args.warmup // 10)

    def step():
        gdn.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dO, S0=d["S0"],
                      chunk=C, workspace=ws)

    ms = time_calls(torch, step, steps, warm)
    nch = B * H * ((T + C - 1) // C)
    fl = bwd_flops_per_chunk_head(dk, C) * nch
    tfs = fl / (ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "steps": steps, "workspace_bytes": nbytes,
            "roofline": {"bound": "mfma", "achieved": round(tfs, 1),
                         "peak": MFMA_FP32_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tfs / MFMA_FP32_PEAK_TFS, 4), "dtype": "f32",
                         "flops_per_step": fl},
            "note": "gdn_chunk_bwd = 5 launches (prep, states, dstates, sprod, grads); "
                    "fp32-accurate products, counted as fp32 MFMA work (those with a bf16 "
                    "input operand run on the bf16 MFMA, the fp32 side as three exact bf16 "
                    "pieces; sprod's fp32 x fp32 products as six products of such pieces); "
                    "dO fp32 ~ N(0,1), dS_T = 0"}


def kda_flops_per_chunk_head(d: int, C: int = 64):
    """MFMA flops of gdn_kda_fwd per (chunk, head), as (fp32 products of the
    prep, fp32-accurate products of the sequential launch).  Prep: the 6
    blocks below the diagonal of A and of P (16 x 16 x d each), on the fp32
    MFMA.  Sequential launch: (K o e^G) S^T and (Q o e^G) S^T (C x d x d
    each), T diag(beta) Z and P Delta (C x C x d each), the state update
    (d x C x d); each runs on the bf16 MFMA as three piece products of hi + lo
    pairs.  The diagonal blocks of A and P (term-by-term VALU) are not
    counted."""
    cdd = 2.0 * C * d * d
    ccd = 2.0 * C * C * d
    prep = 2 * 6 * 2.0 * 16 * 16 * d
    return prep, 2 * cdd + 2 * ccd + cdd


def channel_fwd_bytes(B, T, H, dk, dv, gate_floats_per_th, io_bytes=2, o_bytes=4):
    """Algorithmic HBM bytes of a channel-wise forward: q, k, v once, the
    fp32 gates once (gate_floats_per_th per token-head: d_k for KDA's decay
    and beta; d_k + d_k + d_v for GDN-2's decay, erase and write), o once, the
    final states once.  The workspace its two launches pass between them is
    not algorithmic and is reported beside it."""
    per_th = (2 * dk + dv) * io_bytes + dv * o_bytes + 4 * gate_floats_per_th
    return B * T * H * per_th + B * H * dv * dk * 4


def hbm_roofline(nbytes, ms, ws_bytes):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
            "workspace_bytes_written_and_read": ws_bytes,
            "frac_with_workspace": round((nbytes + 2 * ws_bytes) / (ms * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4)}


def run_kda(args, torch, gi, gdn, dev, w):
    """Time gdn_kda_fwd on the headline shape with channel-wise decays
    (log alpha = -softplus(N(1,1)) per channel), inputs resident."""
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["chunk"]
    print("[bench] channel-wise decay forward", file=sys.stderr, flush=True)
    inp = gi.kda_inputs(B, T, H, dk, dv, "bf16", alpha_mu=1.0, seed=gi.SEED_BASE + 30)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
    st = torch.empty((B, H, dv, dk), device=dev, dtype=torch.float32)
    ws = torch.empty(gdn.kda_fwd_workspace_size(B, T, H, dk, dv, C), device=dev,
                     dtype=torch.uint8)
    steps, warm = max(MIN_TIMED, args.steps // 4), max(1, args.warmup // 4)

    def step():
        gdn.kda_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, chunk=C, o=o,
                    S_T=st, workspace=ws)

    ms = time_calls(torch, step, steps, warm)
    nch = B * H * ((T + C - 1) // C)
    f_prep, f_seq = kda_flops_per_chunk_head(dk, C)
    hbm = hbm_roofline(channel_fwd_bytes(B, T, H, dk, dv, dk + 1), ms, ws.numel())
    bf16_tfs = 3 * f_seq * nch / (ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "steps": steps, "roofline": hbm,
            "mfma_executed": {"bf16_piece_products_tflops": round(bf16_tfs, 1),
                              "frac_of_bf16_peak": round(bf16_tfs / MFMA_BF16_PEAK_TFS, 4),
                              "prep_f32_tflops": round(f_prep * nch / (ms * 1e-3) / 1e12, 1),
                              "flops_per_step": {"prep_f32": f_prep * nch,
                                                 "sequential_fp32_accurate": f_seq * nch}},
            "note": "gdn_kda_fwd = prep (fp32 MFMA blocks of A and P, T by the blocked "
                    "inverse; writes the sequential launch's operands as bf16 hi + lo pairs, "
                    "rows dense) + sequential launch (bf16 MFMA, three piece products per "
                    "product; operand regions copied global->LDS three phases ahead). HBM-bound "
                    "on the workspace round trip: see frac_with_workspace. bf16 q/k/v, fp32 "
                    "channel-wise log alpha [B,T,H,d_k], fp32 o and state"}


def gdn2_flops_per_chunk_head(d: int, C: int = 64):
    """MFMA flops of gdn_gdn2_fwd per (chunk, head), as (fp32 products of the
    prep, fp32-accurate products of the sequential launch).  Prep, on the fp32
    MFMA: the 6 blocks below the diagonal of each of A_e, A_k, P_e, P_k, the
    folds M = P_e T_e, N1 = T_e A_k, N2 (C^3 each), F1 and Qh (C x C x d
    each).  Sequential launch, each product as three bf16 piece products of
    hi + lo pairs: F1 S^T, Qh S^T (C x d x d), N1 Z, N2 Z (C^2 x d) and the two
    update products (d x C x d).  Diagonal blocks (term-by-term VALU) are not
    counted."""
    cdd = 2.0 * C * d * d
    ccd = 2.0 * C * C * d
    prep = 4 * 6 * 2.0 * 16 * 16 * d + 3 * 2.0 * C ** 3 + 2 * ccd
    return prep, 2 * cdd + 2 * ccd + 2 * cdd


def run_gdn2(args, torch, gi, gdn, dev, w):
    """Time gdn_gdn2_fwd on the headline shape (channel-wise decays, erase and
    write gates sigmoid(N(0,1))), inputs resident."""
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["chunk"]
    print("[bench] Gated DeltaNet-2 forward", file=sys.stderr, flush=True)
    inp = gi.gdn2_inputs(B, T, H, dk, dv, "bf16", alpha_mu=1.0, seed=gi.SEED_BASE + 40)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
    st = torch.empty((B, H, dv, dk), device=dev, dtype=torch.float32)
    ws = torch.empty(gdn.gdn2_fwd_workspace_size(B, T, H, dk, dv, C), device=dev,
                     dtype=torch.uint8)
    steps, warm = max(MIN_TIMED, args.steps // 4), max(1, args.warmup // 4)

    def step():
        gdn.gdn2_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["erase"], d["write"], None,
                     chunk=C, o=o, S_T=st, workspace=ws)

    ms = time_calls(torch, step, steps, warm)
    nch = B * H * ((T + C - 1) // C)
    f_prep, f_seq = gdn2_flops_per_chunk_head(dk, C)
    hbm = hbm_roofline(channel_fwd_bytes(B, T, H, dk, dv, 2 * dk + dv), ms, ws.numel())
    bf16_tfs = 3 * f_seq * nch / (ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "steps": steps, "roofline": hbm,
            "mfma_executed": {"bf16_piece_products_tflops": round(bf16_tfs, 1),
                              "frac_of_bf16_peak": round(bf16_tfs / MFMA_BF16_PEAK_TFS, 4),
                              "prep_f32_tflops": round(f_prep * nch / (ms * 1e-3) / 1e12, 1),
                              "frac_of_f32_peak_prep": round(f_prep * nch / (ms * 1e-3) / 1e12
                                                             / MFMA_FP32_PEAK_TFS, 4),
                              "flops_per_step": {"prep_f32": f_prep * nch,
                                                 "sequential_fp32_accurate": f_seq * nch}},
            "note": "gdn_gdn2_fwd = prep (fp32 MFMA: channel-weighted blocks, T_e, the folds "
                    "F1, Qh, N1, N2; writes the sequential launch's operands as bf16 hi + lo "
                    "pairs, rows dense) + sequential launch (bf16 MFMA, three piece "
                    "products per product, five phases, operand regions copied global->LDS "
                    "ahead of use). bf16 q/k/v, fp32 log alpha and erase gates [B,T,H,d_k], "
                    "write gates [B,T,H,d_v]"}


def run_prologue(args, torch, gi, gdn, dev, w, plain_ms):
    """Time the forward with the fused input prologue on raw projections of
    the same workload (q, k unnormalised, gates as pre-activations), and, for
    comparison, the same prologue as separate torch ops before a plain call."""
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["chunk"]
    print("[bench] fused prologue: raw inputs", file=sys.stderr, flush=True)
    raw = gi.raw_chunk_inputs(B, T, H, dk, dv, "bf16", alpha_mu=w["alpha_mu"],
                              seed=gi.SEED_BASE + 2)
    d = {k: (v.to(dev) if v is not None else None) for k, v in raw.items()}
    o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
    st = torch.empty((B, H, dv, dk), device=dev, dtype=torch.float32)
    steps, warm = max(MIN_TIMED, args.steps // 2), max(1, args.warmup // 2)

    def fused():
        gdn.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, chunk=C,
                      o=o, S_T=st, norm_qk=True, gates=True)

    def separate():
        F = torch.nn.functional
        q = F.normalize(d["q"].float(), dim=-1, eps=1e-6).to(torch.bfloat16)
        k = F.normalize(d["k"].float(), dim=-1, eps=1e-6).to(torch.bfloat16)
        la = -F.softplus(d["log_alpha"])
        be = torch.sigmoid(d["beta"])
        gdn.chunk_fwd(q, k, d["v"], la, be, None, chunk=C, o=o, S_T=st)

    res = {}
    for name, fn, n in (("fused", fused, steps), ("separate", separate, MIN_TIMED)):
        res[name] = time_calls(torch, fn, n, warm)
    fms = res["fused"]
    return {"ms_per_step": round(fms, 4), "tokens_per_s": round(B * T / (fms * 1e-3), 1),
            "vs_plain_call": round(fms / plain_ms, 4),
            "separate_torch_prologue_ms_per_step": round(res["separate"], 4),
            "kernel": "chunk_mfma_kernel<128,float,3>", "steps": steps,
            "inputs": "raw projections of the same workload: q, k ~ N(0,1) unnormalised, "
                      "gate pre-activations a ~ N(1,1), b ~ N(0,1)"}


def run_other_workloads(args, torch, gi, gdn, dev, headline_ns_per_th):
    """The mid workload (B=4 T=2048 H=8 d=64) and the packed long-context
    workload (8 sequences of 1 024-16 384 tokens, 65 536 in all, H=16 d=128)
    through the same entry point: ms per call, tokens/s and the HBM fraction
    of their algorithmic bytes; for the packed one also the time per
    token-head relative to the headline workload's (a longest sequence that
    sets the launch time shows up as a ratio above 1)."""
    out = {}
    for wid in (1, 3):
        w = gi.WORKLOADS[wid]
        print(f"[bench] workload {wid} ({w['name']})", file=sys.stderr, flush=True)
        host = gi.workload_inputs(wid)
        d = {k: (v.to(dev) if v is not None else None) for k, v in host.items()}
        B, T, H = d["q"].shape[:3]
        dk, dv = w["dk"], w["dv"]
        cu = d["cu_seqlens"]
        units = B if cu is None else cu.shape[0] - 1
        o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
        st = torch.empty((units, H, dv, dk), device=dev, dtype=torch.float32)

        def fn():
            gdn.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], cu,
                          chunk=w["chunk"], o=o, S_T=st)

        ms = time_calls(torch, fn, max(MIN_TIMED, args.steps // 4), 2)
        nbytes = bytes_chunk_fwd(B, T, H, dk, dv, with_s0=d["S0"] is not None, units=units)
        gbs = nbytes / (ms * 1e-3) / 1e9
        rec = {"workload": w["name"], "ms_per_call": round(ms, 4),
               "tokens_per_s": round(B * T / (ms * 1e-3), 1),
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "algorithmic_bytes": nbytes}}
        if cu is not None:
            lens = [int(b - a) for a, b in zip(host["cu_seqlens"][:-1], host["cu_seqlens"][1:])]
            rec["seq_lens"] = lens
            rec["ns_per_token_head"] = round(ms * 1e6 / (B * T * H), 4)
            rec["vs_headline_per_token_head"] = round(
                ms * 1e6 / (B * T * H) / headline_ns_per_th, 3)
        else:
            rec["note"] = "35 MB of algorithmic bytes: resident in the 256 MB MALL between calls"
        out[w["name"]] = rec
        del d, o, st
    return out


def cpu_info():
    """CPU model, logical CPUs and the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_available": avail}


def run_cpu_baseline(args, host, B, T, H):
    """The fp64 oracle on a bounded sample of the headline workload (batch
    rows, every head and token), at the threads this process may use (16 at
    most) and at one thread."""
    import oracle
    info = cpu_info()
    rows = max(1, min(args.cpu_rows, B))
    threads = max(1, min(16, info["cpus_available"] or 1))
    sub = {k: (v[:rows] if v is not None else None) for k, v in host.items()
           if k != "cu_seqlens"}

    def timed(n_rows, nthreads, seconds):
        part = {k: (v[:n_rows] if v is not None else None) for k, v in sub.items()}
        reps, ct = 0, 0.0
        while ct < seconds and (reps == 0 or ct / reps * (reps + 1) <= 3 * seconds):
            c0 = time.perf_counter()
            oracle.fwd(part["q"], part["k"], part["v"], part["log_alpha"], part["beta"],
                       part["S0"], threads=nthreads)
            ct += time.perf_counter() - c0
            reps += 1
        return reps * n_rows * T / ct, reps, ct

    print(f"[bench] cpu baseline: oracle on {rows} batch row(s), {threads} threads, "
          f">= {args.cpu_seconds:g} s, then 1 row on 1 thread", file=sys.stderr, flush=True)
    v, reps, ct = timed(rows, threads, args.cpu_seconds)
    v1, reps1, ct1 = timed(1, 1, args.cpu_seconds / 2)
    return {"value": round(v, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "threads": threads, "value_1thread": round(v1, 1), **info,
            "sample": f"{rows} of {B} batch rows (all {H} heads x {T} tokens), fp64 token "
                      f"recurrence, run {reps} times in {ct:.2f} s on {threads} threads; "
                      f"1 row on 1 thread {reps1} times in {ct1:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--cold-steps", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8,
                    help="batch rows of the workload the CPU oracle runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle until it has run this long")
    ap.add_argument("--only", choices=["all", "chunk", "decode", "kda", "gdn2", "bwd"],
                    default="all",
                    help="run one part only (for profiling); the JSON line needs 'all'")
    ap.add_argument("--preheat-ms", type=float, default=PREHEAT_MS,
                    help="GPU time run before each leg's counted warm-up (0 for counter "
                         "passes, which should see few dispatches)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a device-to-device copy of this many MiB (a "
                         "known-size kernel for calibrating HBM byte counters)")
    args = ap.parse_args()
    set_preheat(args.preheat_ms)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the "
              "path has no multi-GPU component to measure.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gdn_inputs as gi
    import gated_delta_rule_58_amd as gdn

    dev = "cuda:0"
    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {args.copy_mib} MiB x3", file=sys.stderr, flush=True)
        del src, dst
    if args.only == "decode":
        run_decode(args, torch, gi, gdn, dev)
        return
    w = gi.WORKLOADS[2]
    if args.only in ("kda", "gdn2", "bwd"):   # one leg alone (for profiling)
        if args.only == "bwd":
            leg = run_backward(args, torch, gi, gdn, dev, w, gi.workload_inputs(2))
        else:
            leg = (run_kda if args.only == "kda" else run_gdn2)(args, torch, gi, gdn, dev, w)
        print(json.dumps(leg))
        return
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["chunk"]
    print(f"[bench] inputs: workload 2 {w['name']} B={B} T={T} H={H} d={dk}", file=sys.stderr,
          flush=True)
    host = gi.workload_inputs(2)
    d = {k: (v.to(dev) if v is not None else None) for k, v in host.items()}
    o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
    st = torch.empty((B, H, dv, dk), device=dev, dtype=torch.float32)

    def step():
        gdn.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                      chunk=C, o=o, S_T=st)

    pre_ms, pre_calls = preheat(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} chunk_fwd steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    tokens = B * T
    value = tokens / (ms * 1e-3)

    nbytes = bytes_chunk_fwd(B, T, H, dk, dv, with_s0=d["S0"] is not None)
    gbs = nbytes / (ms * 1e-3) / 1e9
    fl = flops_per_token_head(C, dk, dv) * B * T * H
    tfs = fl / (ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(PMC_FILE):
        with open(PMC_FILE) as f:
            pmc = json.load(f)
        # counters taken on another version of the kernel source do not count
        if pmc.get("kernel_source_sha256") == kernel_source_sha256():
            traffic = pmc.get("hbm_bytes_per_launch")

    if args.only == "chunk":
        print(json.dumps({"chunk_ms_per_step": round(ms, 4), "tokens_per_s": round(value, 1),
                          "GB_s": round(gbs, 1)}))
        return
    others = run_other_workloads(args, torch, gi, gdn, dev, ms * 1e6 / (B * T * H))
    prologue = run_prologue(args, torch, gi, gdn, dev, w, ms)
    backward = run_backward(args, torch, gi, gdn, dev, w, host)
    kda = run_kda(args, torch, gi, gdn, dev, w)
    gdn2 = run_gdn2(args, torch, gi, gdn, dev, w)
    decode = run_decode(args, torch, gi, gdn, dev)

    # ---------------- CPU oracle baseline ----------------
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(args, host, B, T, H)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "preheat_ms": round(pre_ms, 1),
        "preheat_calls": pre_calls,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w['name']}: B={B} T={T} H={H} d_k=d_v={dk} chunk={C}, "
                               "bf16 q/k/v, fp32 gates/state/o",
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": dk, "d_v": dv,
                   "chunk": C, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "chunk_mfma_kernel<128,float,0>",
                     "algorithmic_bytes": nbytes},
        "mfma": {"achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                 "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "algorithmic_flops": fl},
        "other_workloads": others,
        "decode": decode,
        "fused_prologue": prologue,
        "backward": backward,
        "kda_forward": kda,
        "gdn2_forward": gdn2,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
