"""Seeded synthetic inputs shaped like Wan2.1 self-attention (Q, K, V per head).

This module draws random numbers and nothing else: it holds none of the
attention method's arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any computation.

Recipe (the pages measure on Wan2.1-T2V activations from VBench prompts, which
are not available here; these mixtures stand in for them):

* one numpy ``Generator(Philox)`` per head, seeded by
  ``SeedSequence(seed).spawn(H)[h]``;
* ``n_centers`` centres mu_c ~ center_std * N(0, I_d), shared by Q and K of the
  head, so a query mostly attends to keys of its own centre;
* a component z_t per token from the prior w (uniform, or Zipf w_c ~ (c+1)^-a);
* with a latent grid (T, Y, X): ``n_anchors`` anchors uniform in the unit cube,
  each with a component from w; a token takes the component of its nearest
  anchor (normalised coordinates) with probability ``locality``, else a fresh
  draw from w (random 3-D locality bias);
* q_t = q_scale * (mu_z + noise_std * eps), k_t = mu_z + noise_std * eps',
  v_t ~ N(0, I_d);
* optionally (``norm_spread`` s > 0) every q_t and k_t is scaled by its own
  log-normal factor exp(s * g), g ~ N(0, 1), drawn after everything above (so
  the other draws are unchanged): a wide spread of |q| |k|, as with the
  large-norm outlier tokens of real activations;
* cast to the requested dtype (bf16 uses round-to-nearest-even).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch


def _head(ss, N, d, n_centers, grid, locality, n_anchors, zipf, q_scale,
          center_std, noise_std, norm_spread=0.0):
    rng = np.random.Generator(np.random.Philox(ss))
    mu = rng.standard_normal((n_centers, d)) * center_std
    if zipf:
        w = (np.arange(n_centers) + 1.0) ** (-float(zipf))
    else:
        w = np.ones(n_centers)
    w = w / w.sum()
    fresh = rng.choice(n_centers, size=N, p=w)
    if grid is not None:
        T, Y, X = grid
        assert T * Y * X == N, "grid does not match the token count"
        t = np.arange(N)
        coords = np.stack([(t // (Y * X)) / T, ((t // X) % Y) / Y, (t % X) / X], axis=1)
        anchors = rng.random((n_anchors, 3))
        anchor_comp = rng.choice(n_centers, size=n_anchors, p=w)
        d2 = ((coords[:, None, :] - anchors[None, :, :]) ** 2).sum(-1)
        near = anchor_comp[np.argmin(d2, axis=1)]
        keep = rng.random(N) < locality
        z = np.where(keep, near, fresh)
    else:
        z = fresh
    q = q_scale * (mu[z] + noise_std * rng.standard_normal((N, d)))
    k = mu[z] + noise_std * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    if norm_spread:
        q = q * np.exp(norm_spread * rng.standard_normal((N, 1)))
        k = k * np.exp(norm_spread * rng.standard_normal((N, 1)))
    return (q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
            z.astype(np.int32))


def make_qkv(H: int, N: int, d: int, *, n_centers: int = 64, grid=None,
             locality: float = 0.75, n_anchors: int = 64, zipf=None,
             q_scale: float = 1.0, center_std: float = 1.0,
             noise_std: float = 0.3, seed: int = 0, dtype: str = "bf16",
             B: int = 1, threads: int | None = None, norm_spread: float = 0.0):
    """Return (q, k, v, comp) as CPU tensors of shape [B, H, N, d] (comp: [B, H, N]).

    ``dtype`` is "bf16" or "f32". Batch b uses seed ``seed + b``.
    """
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    q = torch.empty((B, H, N, d), dtype=tdt)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    comp = torch.empty((B, H, N), dtype=torch.int32)
    jobs = []
    for b in range(B):
        for h, ss in enumerate(np.random.SeedSequence(seed + b).spawn(H)):
            jobs.append((b, h, ss))

    def run(job):
        b, h, ss = job
        qh, kh, vh, zh = _head(ss, N, d, n_centers, grid, locality, n_anchors,
                               zipf, q_scale, center_std, noise_std, norm_spread)
        q[b, h] = torch.from_numpy(qh).to(tdt)
        k[b, h] = torch.from_numpy(kh).to(tdt)
        v[b, h] = torch.from_numpy(vh).to(tdt)
        comp[b, h] = torch.from_numpy(zh)

    nthr = threads or min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    if nthr <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(run, jobs))
    return q, k, v, comp


def structured_values(comp, d: int, *, n_centers: int = 64, seed: int = 0, noise_std: float = 0.3,
                      dtype: str = "bf16"):
    """Values that carry the keys' cluster structure: v_t = nu_{z_t} + noise_std * eps,
    with nu_c ~ N(0, I_d) drawn per (batch, head) from their own seeded stream.  comp
    is the component index per token ([B, H, N], as returned by make_qkv).  Used by
    the error-vs-density study: with values independent of the keys (v ~ N(0, I)) the
    dense output of a near-uniform row is close to zero and a relative error says
    little, while real values carry structure that a skipped region contributes."""
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    B, H, N = comp.shape
    v = torch.empty((B, H, N, d), dtype=tdt)
    for b in range(B):
        for h, ss in enumerate(np.random.SeedSequence([seed + b, 7919]).spawn(H)):
            rng = np.random.Generator(np.random.Philox(ss))
            nu = rng.standard_normal((n_centers, d))
            eps = rng.standard_normal((N, d))
            v[b, h] = torch.from_numpy((nu[comp[b, h].numpy()] + noise_std * eps).astype(np.float32)).to(tdt)
    return v


def make_workload(w: dict, *, seed: int = 0, threads: int | None = None, H=None, N=None):
    """Inputs for a workload dict from ``workloads.WORKLOADS`` (optionally fewer heads/tokens)."""
    H = H or w["H"]
    N = N or w["N"]
    grid = w.get("grid") if N == w["N"] else None
    return make_qkv(H, N, w["d"], n_centers=w["n_centers"], grid=grid,
                    locality=w.get("locality", 0.75), zipf=w.get("zipf"),
                    q_scale=w.get("q_scale", 1.0), seed=seed, dtype=w["dtype"],
                    B=w.get("B", 1), threads=threads, norm_spread=w.get("norm_spread", 0.0))
