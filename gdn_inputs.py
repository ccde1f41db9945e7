"""Seeded synthetic inputs for the gated-delta-rule workloads.

This module only draws random numbers in the shapes and distributions of the
workloads; it holds none of the recurrence's arithmetic.  Both the GPU tests
and the CPU oracle consume its output, so the two sides always see the same
values.

The pages describe the models only as 400M-1.3B-parameter Gated DeltaNet
layers and print no shapes, so the shapes below stand in for them (one
attention-sized layer: 16 heads of width 128 at 1.3B, 8 heads of width 64
for a mid-sized one).  Recipe per workload (numpy PCG64, seed 58000 + id,
draw order: packed lengths (if any), q, k, v, beta logits, alpha logits, S0):

* q, k ~ N(0,1), L2-normalised per (token, head) over d_k in fp64 (no
  epsilon), then cast to the I/O dtype with round-to-nearest-even;
* v ~ N(0,1), cast the same way;
* beta = sigmoid(x), x ~ N(0,1), fp32;
* log alpha = -softplus(x), x ~ N(mu,1) (mu = 0 for the tiny and mid
  workloads, 1 for the 1.3B-shaped ones), fp32, so alpha is in (0,1);
* S0 = 0, or ~ N(0, 0.1^2) in fp32 where the workload starts from a state.

The ``raw_*`` generators draw the same numbers in the same order but stop
before the normalisation and the gate activations, for the path's fused
input prologue: q, k ~ N(0,1) cast to the I/O dtype as they are, and the
gate pre-activations b ~ N(0,1) (for beta) and a ~ N(mu,1) (for alpha) in
fp32, returned under the names ``beta`` and ``log_alpha``.
"""
from __future__ import annotations

import numpy as np
import torch

SEED_BASE = 58000

WORKLOADS = {
    0: dict(name="tiny-f32", B=1, T=64, H=1, dk=16, dv=16, chunk=16,
            dtype="f32", alpha_mu=0.0, s0_std=0.0),
    1: dict(name="mid-bf16", B=4, T=2048, H=8, dk=64, dv=64, chunk=64,
            dtype="bf16", alpha_mu=0.0, s0_std=0.1),
    2: dict(name="1.3b-layer-bf16", B=8, T=4096, H=16, dk=128, dv=128,
            chunk=64, dtype="bf16", alpha_mu=1.0, s0_std=0.0),
    3: dict(name="varlen-long-bf16", n_seqs=8, total=65536, lmin=1024,
            lmax=16384, H=16, dk=128, dv=128, chunk=64, dtype="bf16",
            alpha_mu=1.0, s0_std=0.0),
    4: dict(name="decode-b64", B=64, H=16, dk=128, dv=128, steps=256,
            dtype="bf16", alpha_mu=1.0, s0_std=0.1),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(x).to(TORCH_DTYPE[dtype])


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _neg_softplus(x: np.ndarray) -> np.ndarray:
    return -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def packed_lengths(rng: np.random.Generator, n: int, total: int, lo: int,
                   hi: int) -> list[int]:
    """n lengths in [lo, hi] summing to total: draw n-1 uniformly, set the
    last to the remainder, redraw all while the remainder is out of range."""
    while True:
        head = rng.integers(lo, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return [int(x) for x in head] + [last]


def chunk_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
                 alpha_mu: float = 1.0, s0_std: float = 0.0, seed: int = 0,
                 cu_seqlens=None, rng: np.random.Generator | None = None):
    """Inputs of one chunked forward.  With cu_seqlens (B must be 1) S0 has one
    state per packed sequence.  Returns a dict of CPU torch tensors."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q = _cast(_unit_rows(rng, (B, T, H, dk)), dtype)
    k = _cast(_unit_rows(rng, (B, T, H, dk)), dtype)
    v = _cast(rng.standard_normal((B, T, H, dv)), dtype)
    beta = torch.from_numpy(_sigmoid(rng.standard_normal((B, T, H)))).float()
    log_alpha = torch.from_numpy(
        _neg_softplus(rng.normal(alpha_mu, 1.0, (B, T, H)))).float()
    units = B if cu_seqlens is None else len(cu_seqlens) - 1
    S0 = None
    if s0_std > 0:
        S0 = torch.from_numpy(rng.normal(0.0, s0_std, (units, H, dv, dk))).float()
    cu = None
    if cu_seqlens is not None:
        cu = torch.tensor(list(cu_seqlens), dtype=torch.int32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S0=S0,
                cu_seqlens=cu)


def raw_chunk_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
                     alpha_mu: float = 1.0, s0_std: float = 0.0, seed: int = 0,
                     cu_seqlens=None, rng: np.random.Generator | None = None):
    """Like chunk_inputs, but q, k unnormalised and the gates as
    pre-activations (a under "log_alpha", b under "beta")."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q = _cast(rng.standard_normal((B, T, H, dk)), dtype)
    k = _cast(rng.standard_normal((B, T, H, dk)), dtype)
    v = _cast(rng.standard_normal((B, T, H, dv)), dtype)
    b = torch.from_numpy(rng.standard_normal((B, T, H))).float()
    a = torch.from_numpy(rng.normal(alpha_mu, 1.0, (B, T, H))).float()
    units = B if cu_seqlens is None else len(cu_seqlens) - 1
    S0 = None
    if s0_std > 0:
        S0 = torch.from_numpy(rng.normal(0.0, s0_std, (units, H, dv, dk))).float()
    cu = None
    if cu_seqlens is not None:
        cu = torch.tensor(list(cu_seqlens), dtype=torch.int32)
    return dict(q=q, k=k, v=v, log_alpha=a, beta=b, S0=S0, cu_seqlens=cu)


def structured_keys(rng: np.random.Generator, B: int, T: int, H: int, dk: int,
                    mode: str, param: float, window: int = 64,
                    cos: float = 0.99) -> np.ndarray:
    """Keys [B,T,H,dk] (fp64, unit rows) with the structure of repeated tokens,
    drawn per (batch row, head) and per `window` consecutive tokens (windows
    start at token 0, so with the chunk length as window they are the chunks):

    * "repeat": runs of `param` consecutive tokens share one random unit key;
    * "scatter": the window draws window/param distinct unit keys and each
      token takes one of them uniformly at random (repeats at any distance);
    * "cluster": the window draws `param` random unit directions u_j; each
      token takes one of them at random and its key is u_j + e n,
      renormalised, with n a random unit vector and e = sqrt(1/cos^2 - 1), so
      the key is at cosine about `cos` from its direction (keys of one
      cluster are nearly collinear).
    """
    k = np.empty((B, T, H, dk))
    eps = np.sqrt(1.0 / cos ** 2 - 1.0)
    for b in range(B):
        for h in range(H):
            for t0 in range(0, T, window):
                n = min(window, T - t0)
                if mode == "repeat":
                    g = int(param)
                    base = _unit_rows(rng, ((n + g - 1) // g, dk))
                    x = base[np.arange(n) // g]
                elif mode == "scatter":
                    base = _unit_rows(rng, (max(1, window // int(param)), dk))
                    x = base[rng.integers(0, base.shape[0], n)]
                elif mode == "cluster":
                    base = _unit_rows(rng, (int(param), dk))
                    x = base[rng.integers(0, int(param), n)] + eps * _unit_rows(rng, (n, dk))
                    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
                else:
                    raise ValueError(f"unknown key structure {mode!r}")
                k[b, t0:t0 + n, h] = x
    return k


def structured_chunk_inputs(B: int, T: int, H: int, dk: int, dv: int, mode: str,
                            param: float, dtype: str = "bf16", alpha_mu: float = 1.0,
                            s0_std: float = 0.0, beta_shift: float = 0.0,
                            seed: int = 0, cu_seqlens=None, window: int = 64):
    """chunk_inputs with the keys replaced by `structured_keys` (drawn after
    everything else, from the same generator, per packed sequence when
    cu_seqlens is given so windows start at each sequence start), and
    beta + beta_shift (a shift of 1 gives beta in (1, 2))."""
    rng = np.random.default_rng(seed)
    inp = chunk_inputs(B, T, H, dk, dv, dtype, alpha_mu, s0_std, seed, cu_seqlens, rng=rng)
    if cu_seqlens is None:
        k = structured_keys(rng, B, T, H, dk, mode, param, window)
    else:
        k = np.empty((1, T, H, dk))
        for s in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
            if e > a:
                k[:, a:e] = structured_keys(rng, 1, e - a, H, dk, mode, param, window)
    inp["k"] = _cast(k, dtype)
    if beta_shift:
        inp["beta"] = inp["beta"] + float(beta_shift)
    return inp


def kda_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
               alpha_mu: float = 1.0, alpha_sd: float = 1.0, s0_std: float = 0.0,
               seed: int = 0, cu_seqlens=None):
    """Inputs of the channel-wise decay forward: as chunk_inputs, with
    log_alpha [B,T,H,dk] = -softplus(N(alpha_mu, alpha_sd)) per channel."""
    rng = np.random.default_rng(seed)
    inp = chunk_inputs(B, T, H, dk, dv, dtype, alpha_mu, s0_std, seed, cu_seqlens, rng=rng)
    inp["log_alpha"] = torch.from_numpy(
        _neg_softplus(rng.normal(alpha_mu, alpha_sd, (B, T, H, dk)))).float()
    return inp


def gdn2_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
                alpha_mu: float = 1.0, alpha_sd: float = 1.0, s0_std: float = 0.0,
                seed: int = 0, cu_seqlens=None):
    """Inputs of the Gated DeltaNet-2 forward: as kda_inputs, plus erase
    [B,T,H,dk] = sigmoid(N(0,1)) and write [B,T,H,dv] = sigmoid(N(0,1))."""
    inp = kda_inputs(B, T, H, dk, dv, dtype, alpha_mu, alpha_sd, s0_std, seed, cu_seqlens)
    rng = np.random.default_rng(seed + 12345)
    inp["erase"] = torch.from_numpy(_sigmoid(rng.standard_normal((B, T, H, dk)))).float()
    inp["write"] = torch.from_numpy(_sigmoid(rng.standard_normal((B, T, H, dv)))).float()
    return inp


def raw_decode_inputs(B: int, H: int, dk: int, dv: int, steps: int,
                      dtype: str = "bf16", alpha_mu: float = 1.0,
                      s0_std: float = 0.1, seed: int = 0):
    """Like decode_inputs, with unnormalised q, k and gate pre-activations."""
    rng = np.random.default_rng(seed)
    q = _cast(rng.standard_normal((steps, B, H, dk)), dtype)
    k = _cast(rng.standard_normal((steps, B, H, dk)), dtype)
    v = _cast(rng.standard_normal((steps, B, H, dv)), dtype)
    b = torch.from_numpy(rng.standard_normal((steps, B, H))).float()
    a = torch.from_numpy(rng.normal(alpha_mu, 1.0, (steps, B, H))).float()
    S0 = torch.from_numpy(rng.normal(0.0, s0_std, (B, H, dv, dk))).float()
    return dict(q=q, k=k, v=v, log_alpha=a, beta=b, S0=S0)


def decode_inputs(B: int, H: int, dk: int, dv: int, steps: int,
                  dtype: str = "bf16", alpha_mu: float = 1.0,
                  s0_std: float = 0.1, seed: int = 0):
    """Inputs of `steps` consecutive decode steps: q,k [steps,B,H,dk],
    v [steps,B,H,dv], gates [steps,B,H], initial state [B,H,dv,dk]."""
    rng = np.random.default_rng(seed)
    q = _cast(_unit_rows(rng, (steps, B, H, dk)), dtype)
    k = _cast(_unit_rows(rng, (steps, B, H, dk)), dtype)
    v = _cast(rng.standard_normal((steps, B, H, dv)), dtype)
    beta = torch.from_numpy(_sigmoid(rng.standard_normal((steps, B, H)))).float()
    log_alpha = torch.from_numpy(
        _neg_softplus(rng.normal(alpha_mu, 1.0, (steps, B, H)))).float()
    S0 = torch.from_numpy(rng.normal(0.0, s0_std, (B, H, dv, dk))).float()
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S0=S0)


def workload_inputs(wid: int):
    """The full-size inputs of workload `wid` (0-4)."""
    w = WORKLOADS[wid]
    seed = SEED_BASE + wid
    if wid == 4:
        return decode_inputs(w["B"], w["H"], w["dk"], w["dv"], w["steps"],
                             w["dtype"], w["alpha_mu"], w["s0_std"], seed)
    if wid == 3:
        rng = np.random.default_rng(seed)
        lens = packed_lengths(rng, w["n_seqs"], w["total"], w["lmin"], w["lmax"])
        cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
        return chunk_inputs(1, w["total"], w["H"], w["dk"], w["dv"],
                            w["dtype"], w["alpha_mu"], w["s0_std"],
                            cu_seqlens=cu, rng=rng)
    return chunk_inputs(w["B"], w["T"], w["H"], w["dk"], w["dv"], w["dtype"],
                        w["alpha_mu"], w["s0_std"], seed)


def max_rel_err(x, ref) -> float:
    """max |x - ref| / RMS(ref), both upcast to fp64 (the parity statistic)."""
    x = np.asarray(x.detach().cpu().double().numpy() if hasattr(x, "detach") else x,
                   dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return float(np.max(np.abs(x - ref)) / rms) if x.size else 0.0
