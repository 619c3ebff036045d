"""GPU path vs the CPU oracle, stage by stage, through the C ABI.

Bars: block lists, sample indices, permutations and offsets bit-exact given the
same upstream inputs; k-means labels equal except near-ties (fp64 distance gap
< 1e-5); centroids within fp32 rounding; pi and offsets within 1e-6; attention
output max-abs <= 2e-2 (bf16) / <= 1e-4 (fp32), LSE <= 4.0e-3 (bf16) / 1e-4 (fp32).

The bf16 LSE bar follows from the arithmetic: the attention kernel sums the
bf16-rounded weights that its P.V product uses (so O is an exact convex
combination of V rows).  bf16 carries 8 significant bits, so rounding a
non-negative term to the nearest bf16 changes it by a relative 2^-8 at most, and
the sum of such terms likewise: |d LSE| <= ln(1 + 2^-8) = 3.90e-3, plus fp32
round-off.  A row whose sum is dominated by one weight reaches that bound.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_means_amd import isg
from block_sparse_attention_means_amd.synth import make_qkv, make_workload
from block_sparse_attention_means_amd.workloads import WORKLOADS, budget_keys

pytestmark = pytest.mark.gpu

LSE_TOL_BF16 = 4.0e-3

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def f32(t):
    return t.float().cpu().numpy()


def npy(t):
    return t.cpu().numpy()


def _inputs(H, N, d, dtype, seed=0, n_centers=12, q_scale=1.0, zipf=None):
    q, k, v, _ = make_qkv(H, N, d, n_centers=n_centers, dtype=dtype, seed=seed, q_scale=q_scale, zipf=zipf)
    return q, k, v


# ------------------------------------------------------------------ clustering
def _near_tie_ok(orc, x, cent, lab_gpu, lab_orc, tol=1e-5):
    bad = np.nonzero(lab_gpu != lab_orc)[0]
    gaps = []
    for t in bad:
        dg = orc.sqdist(x[t], cent[lab_gpu[t]])
        do = orc.sqdist(x[t], cent[lab_orc[t]])
        gaps.append(dg - do)
    gaps = np.array(gaps)
    if len(bad):
        say(f"  k-means label mismatches: {len(bad)} / {len(x)}, max fp64 gap {gaps.max():.3e}")
    return len(bad) == 0 or gaps.max() < tol


@pytest.mark.parametrize("dtype,d,N,C", [("f32", 64, 2048, 8), ("f32", 64, 2048, 32), ("bf16", 128, 3000, 50),
                                         ("bf16", 16, 1500, 256), ("bf16", 64, 777, 13), ("bf16", 128, 300, 2),
                                         ("bf16", 128, 8192, 4096), ("bf16", 16, 500, 2), ("bf16", 16, 2000, 3),
                                         ("bf16", 16, 4000, 33), ("bf16", 16, 6000, 300)])
def test_cluster_one_round_stagewise(orc, dtype, d, N, C):
    """Assign given identical centroids (near-tie rule); update given identical labels;
    stable permutation and offsets bit-exact given the labels; gathers exact."""
    say(f"cluster 1 round dtype={dtype} d={d} N={N} C={C}")
    q, k, v = _inputs(2, N, d, dtype, seed=d + C)
    x = f32(k)
    init = x[:, :, (np.arange(C) * N) // C].copy()
    r = isg.isg_cluster(k.to(DEV), C, 1, init=torch.from_numpy(init).to(DEV), companion=v.to(DEV))
    torch.cuda.synchronize()
    for h in range(2):
        lab_g = npy(r["labels"][0, h])
        lab_o = orc.kmeans_assign(x[0, h], init[0, h])
        assert _near_tie_ok(orc, x[0, h], init[0, h], lab_g, lab_o)
        if dtype == "bf16" and d == 16:
            # every re-decision at d = 16 sums in the exact definition's order and
            # rounding, so the labels are the oracle's argmin itself
            assert np.array_equal(lab_g, lab_o)
        cent_o, cnt = orc.kmeans_update(x[0, h], lab_g, init[0, h])
        cent_g = npy(r["centroids"][0, h])
        assert np.allclose(cent_g, cent_o, rtol=1e-6, atol=1e-6)
        perm_o, off_o = orc.stable_sort(lab_g, C)
        assert np.array_equal(npy(r["perm"][0, h]), perm_o)
        assert np.array_equal(npy(r["offsets"][0, h]), off_o)
        assert torch.equal(r["x_perm"][0, h].cpu(), k[0, h][torch.from_numpy(perm_o).long()])
        assert torch.equal(r["companion_perm"][0, h].cpu(), v[0, h][torch.from_numpy(perm_o).long()])


@pytest.mark.parametrize("d,C", [(16, 30), (16, 29), (16, 285), (128, 30), (128, 61), (128, 285)])
def test_cluster_padding_rows_never_kept(orc, d, C):
    """Centroid counts that leave the last 32-row tile partly padding (C mod 32 in
    28..31: the second half-wave's rows j + 4 fall past C while rows j do not),
    on zero-mean keys of magnitude ~3e15: most tokens then have every real
    centroid farther than |x|^2 + 1e30, the padding rows' screening value.  The
    labels must still be real centroids and the oracle's fp64 argmin (exactly at
    d = 16, up to fp64 near-ties wider)."""
    N = 2000
    say(f"cluster padding rows d={d} C={C}")
    g = np.random.default_rng(C + d)
    xb = torch.from_numpy(g.standard_normal((1, 2, N, d)) * 3e15).to(torch.bfloat16)
    x = f32(xb)
    src = (np.arange(C) * N) // C
    r = isg.isg_cluster(xb.to(DEV), C, 1, want_perm=False)
    torch.cuda.synchronize()
    for h in range(2):
        lab_g = npy(r["labels"][0, h])
        assert lab_g.min() >= 0 and lab_g.max() < C
        init = x[0, h][src]
        lab_o = orc.kmeans_assign(x[0, h], init)
        if d == 16:
            assert np.array_equal(lab_g, lab_o)
        else:
            assert _near_tie_ok(orc, x[0, h], init, lab_g, lab_o)


@pytest.mark.parametrize("factor", [100.0, 300.0])
def test_cluster_large_norms_first_round(orc, factor):
    """Keys scaled by 100-300 (|x|^2 up to ~1e7, so the fp32 screening error of a
    distance exceeds 1): in the first round from data-point centroids, where each
    strided token's own centroid is at distance 0, the labels equal the oracle's
    fp64 argmin except near-ties, and every strided token takes its own centroid."""
    N, d, C = 4096, 128, 256
    say(f"cluster large norms x{factor}")
    _, k, _ = _inputs(2, N, d, "bf16", seed=17)
    ks = (k.float() * factor).to(torch.bfloat16)
    x = f32(ks)
    src = (np.arange(C) * N) // C
    r = isg.isg_cluster(ks.to(DEV), C, 1, want_perm=False)
    torch.cuda.synchronize()
    for h in range(2):
        init = x[0, h][src]
        lab_g = npy(r["labels"][0, h])
        lab_o = orc.kmeans_assign(x[0, h], init)
        say(f"  head {h}: |x|^2 up to {float((x[0, h].astype(np.float64) ** 2).sum(-1).max()):.3e}, "
            f"{int((lab_g != lab_o).sum())} labels differ")
        assert _near_tie_ok(orc, x[0, h], init, lab_g, lab_o)
        own = lab_g[src]
        assert all(own[j] == j or orc.sqdist(x[0, h][src[j]], init[own[j]]) == 0.0 for j in range(C))


@pytest.mark.parametrize("dtype,d,N,C", [("f32", 64, 2048, 8), ("bf16", 128, 4096, 100), ("bf16", 16, 8192, 256)])
def test_cluster_five_rounds(orc, dtype, d, N, C):
    """End to end after 5 rounds: every round's labels checked against the oracle's
    assignment from the GPU's previous centroids (near-tie rule); final agreement with
    the oracle's own 5-round run reported."""
    say(f"cluster 5 rounds dtype={dtype} d={d} N={N} C={C}")
    q, k, v = _inputs(1, N, d, dtype, seed=7)
    x = f32(q)
    kg = q.to(DEV)
    prev = x[:, :, (np.arange(C) * N) // C].copy()
    for it in range(1, 6):
        r = isg.isg_cluster(kg, C, 1, init=torch.from_numpy(prev).to(DEV))
        lab_o = orc.kmeans_assign(x[0, 0], prev[0, 0])
        assert _near_tie_ok(orc, x[0, 0], prev[0, 0], npy(r["labels"][0, 0]), lab_o)
        prev = npy(r["centroids"])
    full = isg.isg_cluster(kg, C, 5)
    assert np.array_equal(npy(full["labels"]), npy(r["labels"]))
    assert np.array_equal(npy(full["centroids"]), prev)
    o = orc.cluster(x, C, 5)
    agree = (o["labels"] == npy(full["labels"])).mean()
    say(f"  5-round label agreement with the oracle's own run: {agree:.6f}")
    assert agree > 0.99


def test_cluster_strided_input_matches_contiguous():
    """[B,N,H,d] input through element strides gives the same result as [B,H,N,d]."""
    q, k, v = _inputs(3, 1000, 128, "bf16", seed=3)
    kg = k.to(DEV)
    strided = kg.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    a = isg.isg_cluster(kg, 20, 3)
    b = isg.isg_cluster(strided, 20, 3)
    for key in ("labels", "perm", "offsets", "centroids", "x_perm"):
        assert torch.equal(a[key], b[key]), key


# ------------------------------------------------------------------ scores and selection
def _clustered(H, N, d, dtype, Cq, Ck, seed=0, q_scale=1.0, zipf=None, n_centers=12):
    q, k, v = _inputs(H, N, d, dtype, seed=seed, q_scale=q_scale, zipf=zipf, n_centers=n_centers)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    cq = isg.isg_cluster(qg, Cq, 5)
    ck = isg.isg_cluster(kg, Ck, 5, companion=vg)
    return (q, k, v), cq, ck


def test_probs_bit_exact(orc):
    (q, k, v), cq, ck = _clustered(3, 4096, 128, "bf16", 16, 64)
    scale = isg.default_scale(128)
    S_g, pi_g = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale)
    S_o, pi_o = orc.probs(npy(cq["centroids"]), npy(ck["centroids"]), npy(ck["offsets"]), scale)
    assert np.array_equal(npy(S_g), S_o)
    assert np.abs(npy(pi_g) - pi_o).max() <= 1e-6


@pytest.mark.parametrize("E,m,mode,seed", [(400, 400, "importance", 0), (400, 400, "importance", 17),
                                           (400, 400, "uniform", 3), (0, 300, "importance", 1),
                                           (4096, 200, "importance", 0), (256, 4096, "importance", 0),
                                           (1000, 0, "importance", 0), (100, 2000, "uniform", 9)])
def test_select_sample_bit_exact(orc, E, m, mode, seed):
    say(f"select E={E} m={m} mode={mode} seed={seed}")
    (q, k, v), cq, ck = _clustered(2, 4096, 128, "bf16", 16, 64)
    scale = isg.default_scale(128)
    S_g, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
    g = isg.isg_select_sample(S_g, ck["offsets"], 4096, E, m, mode=mode, seed=seed, call_id=5)
    o = orc.select_sample(npy(S_g), npy(ck["offsets"]), 4096, E, m, mode=isg.MODES[mode], seed=seed, call_id=5)
    for key in ("exact_groups", "n_exact", "n_sample"):
        assert np.array_equal(npy(g[key]), o[key]), key
    ns = o["n_sample"]
    gi_, go_ = npy(g["sample_idx"]), o["sample_idx"]
    bi_, bo_ = npy(g["sample_bias"]), o["sample_bias"]
    for b in range(ns.shape[0]):
        for h in range(ns.shape[1]):
            for i in range(ns.shape[2]):
                n = ns[b, h, i]
                assert np.array_equal(gi_[b, h, i, :n], go_[b, h, i, :n])
                assert np.abs(bi_[b, h, i, :n] - bo_[b, h, i, :n]).max(initial=0) <= 1e-6


def _ties_case(seed, B=1, H=2, Cq=8, Ck=300, N=6000):
    """Scores drawn from a few values (exact ties, -0 and +0) and key groups cut at
    repeated points (many empty groups)."""
    rng = np.random.default_rng(seed)
    offs = np.zeros((B, H, Ck + 1), np.int32)
    for b in range(B):
        for h in range(H):
            offs[b, h, 1:Ck] = np.sort(rng.choice(np.arange(0, N + 1, 37), size=Ck - 1))
            offs[b, h, Ck] = N
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 2.0], np.float32)
    S = rng.choice(vals, size=(B, H, Cq, Ck)).astype(np.float32)
    pi = rng.choice(np.array([0.0, 1e-3, 1e-2, 5e-2], np.float32), size=(B, H, Cq, Ck)).astype(np.float32)
    return S, pi, offs, N


@pytest.mark.parametrize("rule,mode,E,m", [("budget", "importance", 1500, 500), ("budget", "uniform", 800, 700),
                                           ("budget", "importance", 0, 4000), ("topp", "importance", 0, 500),
                                           ("topp", "uniform", 0, 300)])
def test_select_ties_signed_zeros_empty_groups(orc, rule, mode, E, m):
    """Group ranking with exact score ties, -0 against +0 and empty groups (score or
    pi descending, group id ascending, empty groups last), lists and samples
    bit-exact against the oracle."""
    say(f"select ties rule={rule} mode={mode} E={E} m={m}")
    S, pi, offs, N = _ties_case(31)
    Sg, pig, og = torch.from_numpy(S).to(DEV), torch.from_numpy(pi).to(DEV), torch.from_numpy(offs).to(DEV)
    if rule == "budget":
        g = isg.isg_select_sample(Sg, og, N, E, m, mode=mode, seed=3, call_id=1)
        o = orc.select_sample(S, offs, N, E, m, mode=isg.MODES[mode], seed=3, call_id=1)
    else:
        g = isg.isg_select_sample_topp(Sg, pig, og, N, 0.6, m, mode=mode, seed=3, call_id=1)
        o = orc.select_sample_topp(S, pi, offs, N, 0.6, m, mode=isg.MODES[mode], seed=3, call_id=1)
    for key in ("exact_groups", "n_exact", "n_sample"):
        assert np.array_equal(npy(g[key]), o[key]), key
    ns = o["n_sample"]
    for b in range(ns.shape[0]):
        for h in range(ns.shape[1]):
            for i in range(ns.shape[2]):
                n = ns[b, h, i]
                assert np.array_equal(npy(g["sample_idx"])[b, h, i, :n], o["sample_idx"][b, h, i, :n])
                assert np.abs(npy(g["sample_bias"])[b, h, i, :n] - o["sample_bias"][b, h, i, :n]).max(
                    initial=0) <= 1e-6


# ------------------------------------------------------------------ attention
def _attn_case(orc, H, N, d, dtype, Cq, Ck, E, m, seed=0, q_scale=1.0, zipf=None, mode="importance"):
    (q, k, v), cq, ck = _clustered(H, N, d, dtype, Cq, Ck, seed=seed, q_scale=q_scale, zipf=zipf)
    scale = isg.default_scale(d)
    S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
    sel = isg.isg_select_sample(S, ck["offsets"], N, E, m, mode=mode, seed=seed)
    o_p, lse_p = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                                   ck["offsets"], sel, scale)
    torch.cuda.synchronize()
    selo = {kk: npy(vv) for kk, vv in sel.items() if kk != "m"}
    oo, lo = orc.attention(f32(cq["x_perm"]), f32(ck["x_perm"]), f32(ck["companion_perm"]), npy(cq["offsets"]),
                           npy(ck["offsets"]), selo, m, scale)
    return (q, k, v), cq, ck, sel, o_p, lse_p, oo, lo


@pytest.mark.parametrize("H,N,d,dtype,Cq,Ck,E,m", [
    (2, 4096, 128, "bf16", 8, 32, 512, 512),     # several 128-row tiles per group, ragged tails
    (1, 3001, 128, "bf16", 5, 40, 300, 257),     # odd sizes everywhere
    (2, 2048, 64, "bf16", 8, 32, 256, 256),
    (1, 2048, 64, "f32", 8, 32, 512, 512),       # the tiny fp32 shape
    (1, 1500, 128, "f32", 7, 20, 200, 100),
    (2, 4096, 128, "bf16", 64, 128, 100, 300),   # many small groups
])
def test_attention_given_lists(orc, H, N, d, dtype, Cq, Ck, E, m):
    say(f"attention H={H} N={N} d={d} {dtype} Cq={Cq} Ck={Ck} E={E} m={m}")
    *_, o_p, lse_p, oo, lo = _attn_case(orc, H, N, d, dtype, Cq, Ck, E, m)
    err = np.abs(f32(o_p) - oo).max()
    lerr = _lse_report(f"max|O-O_oracle| = {err:.3e}", npy(lse_p), lo)
    if dtype == "bf16":
        assert err <= 2e-2 and lerr <= LSE_TOL_BF16
    else:
        assert err <= 1e-4 and lerr <= 1e-4


@pytest.mark.parametrize("H,N,Cq,Ck,E,m", [
    (1, 2048, 8, 64, 1, 0),        # exact set = the top group only, no samples: one 64-column tile
    (3, 2048, 8, 64, 1, 16),       # one tile; odd head count, so tile pairs mix heads
    (1, 3001, 13, 64, 40, 40),     # one or two tiles per group, ragged query groups
    (3, 1500, 5, 48, 100, 60),     # two or three tiles; odd tile counts per head
])
def test_attention_short_column_lists(orc, H, N, Cq, Ck, E, m):
    """Column lists of one to three 64-column tiles: the paired-tile kernel's
    pipeline prologue and epilogue, tile pairs that cross heads or end in an
    empty slot, and the loads past the end of a list."""
    say(f"short lists H={H} N={N} Cq={Cq} Ck={Ck} E={E} m={m}")
    *_, sel, o_p, lse_p, oo, lo = _attn_case(orc, H, N, 128, "bf16", Cq, Ck, E, m)
    cols = npy(sel["n_sample"]).max()
    err = np.abs(f32(o_p) - oo).max()
    lerr = _lse_report(f"max samples per group {cols}; max|O-O_oracle| = {err:.3e}", npy(lse_p), lo)
    assert np.isfinite(f32(o_p)).all()
    assert err <= 2e-2 and lerr <= LSE_TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
def test_attention_extreme_logit_range_falls_back(orc, d):
    """Queries and keys anti-aligned with large norms: the Cauchy-Schwarz bound sits
    thousands of log2 units above every logit.  The one-tile kernel (d = 64) keeps
    its fixed reference there, every weight underflows and each tile is recomputed
    by the rescaling kernel; the paired-tile kernel (d = 128) anchors its reference
    to the first tile's largest logit and needs no fallback.  Both outputs match."""
    H, N, Cq, Ck = 1, 2048, 8, 32
    g = torch.Generator().manual_seed(5)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = (200.0 * u + 0.05 * torch.randn(1, H, N, d, generator=g)).to(torch.bfloat16)
    k = (-200.0 * u + 0.05 * torch.randn(1, H, N, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(1, H, N, d, generator=g).to(torch.bfloat16)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = isg.default_scale(d)
    cq = isg.isg_cluster(qg, Cq, 5)
    ck = isg.isg_cluster(kg, Ck, 5, companion=vg)
    S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
    sel = isg.isg_select_sample(S, ck["offsets"], N, 300, 300, seed=1)
    nfb = torch.zeros(1, device=DEV, dtype=torch.int32)
    o_p, lse_p = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                                   ck["offsets"], sel, scale, n_fallback_tiles=nfb)
    torch.cuda.synchronize()
    selo = {kk: npy(vv) for kk, vv in sel.items() if kk != "m"}
    oo, lo = orc.attention(f32(cq["x_perm"]), f32(ck["x_perm"]), f32(ck["companion_perm"]), npy(cq["offsets"]),
                           npy(ck["offsets"]), selo, 300, scale)
    assert np.isfinite(f32(o_p)).all()
    err = np.abs(f32(o_p) - oo).max()
    n_fb = int(nfb.item())
    say(f"  extreme range d={d}: max|O-O_oracle| {err:.3e}, LSE range {lo.min():.1f}..{lo.max():.1f}, "
        f"{n_fb} tiles through the fallback")
    assert (n_fb > 0) if d == 64 else (n_fb == 0)
    assert err <= 2e-2
    assert lo.max() < -1000  # the case really is extreme
    # |LSE| ~ 3500 here: fp32 logits carry ~1e-7 relative error on top of the bf16 bar
    assert np.abs(npy(lse_p) - lo).max() <= LSE_TOL_BF16 + 1e-6 * np.abs(lo).max()


@pytest.mark.parametrize("d", [64, 128])
def test_attention_fallback_mixed_heads_many_tiles(orc, d):
    """One extreme head among three ordinary ones, with more query tiles than the
    fallback has work-groups.  d = 64: every tile of the extreme head is flagged and
    the rescaling pass walks them with a persistent grid, leaving the others alone;
    d = 128: the anchored reference handles the extreme head directly."""
    H, N, Cq, Ck = 4, 16384, 8, 32
    g = torch.Generator().manual_seed(11)
    q, k, v = _inputs(H, N, d, "bf16", seed=13)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q[0, 2] = (200.0 * u + 0.05 * torch.randn(N, d, generator=g)).to(torch.bfloat16)
    k[0, 2] = (-200.0 * u + 0.05 * torch.randn(N, d, generator=g)).to(torch.bfloat16)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = isg.default_scale(d)
    cq = isg.isg_cluster(qg, Cq, 5)
    ck = isg.isg_cluster(kg, Ck, 5, companion=vg)
    S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
    sel = isg.isg_select_sample(S, ck["offsets"], N, 300, 300, seed=2)
    nfb = torch.zeros(1, device=DEV, dtype=torch.int32)
    o_p, lse_p = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                                   ck["offsets"], sel, scale, n_fallback_tiles=nfb)
    torch.cuda.synchronize()
    n_fb = int(nfb.item())
    n_tiles = int(((np.diff(npy(cq["offsets"]), axis=-1) + 127) // 128)[0, 2].sum())
    say(f"  d={d}: {n_fb} tiles through the fallback ({n_tiles} query tiles in the extreme head)")
    assert (n_fb == n_tiles) if d == 64 else (n_fb == 0)
    selo = {kk: npy(vv) for kk, vv in sel.items() if kk != "m"}
    oo, lo = orc.attention(f32(cq["x_perm"]), f32(ck["x_perm"]), f32(ck["companion_perm"]), npy(cq["offsets"]),
                           npy(ck["offsets"]), selo, 300, scale)
    assert np.isfinite(f32(o_p)).all()
    err = np.abs(f32(o_p) - oo).max()
    lerr = np.abs(npy(lse_p) - lo)
    say(f"  mixed heads: max|O-O_oracle| {err:.3e}, extreme head LSE {lo[0, 2].min():.1f}..{lo[0, 2].max():.1f}")
    assert lo[0, 2].max() < -1000 and lo[0, [0, 1, 3]].min() > -1000
    assert err <= 2e-2
    assert lerr[0, [0, 1, 3]].max() <= LSE_TOL_BF16
    assert lerr[0, 2].max() <= LSE_TOL_BF16 + 1e-6 * np.abs(lo[0, 2]).max()


@pytest.mark.parametrize("H", [1, 3])
def test_attention_rescaling_pass_after_anchor(orc, H):
    """Hand-built lists (d = 128): key group 0 is anti-aligned with every query and
    comes first in the column list, key group 1 is aligned with large norms, so
    the logits of the second tile exceed the first tile's by thousands of log2
    units.  The anchored reference overflows there, every tile is flagged, and the
    listed tiles are recomputed by the paired-tile kernel with a running maximum
    (an odd number of tiles per head leaves one pair half-empty)."""
    N, d, nq = 640, 128, 384
    g = torch.Generator().manual_seed(23)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = (40.0 * u + 0.3 * torch.randn(1, H, N, d, generator=g)).to(torch.bfloat16)
    k = 0.3 * torch.randn(1, H, N, d, generator=g)
    k[:, :, :64] += -40.0 * u
    k[:, :, 64:128] += 60.0 * u
    k = k.to(torch.bfloat16)
    v = torch.randn(1, H, N, d, generator=g).to(torch.bfloat16)
    # query groups: [0, nq) and [nq, N); key groups: [0, 64), [64, 128), [128, N)
    qo = torch.tensor([0, nq, N], dtype=torch.int32).repeat(1, H, 1)
    ko = torch.tensor([0, 64, 128, N], dtype=torch.int32).repeat(1, H, 1)
    eg = torch.full((1, H, 2, 3), -1, dtype=torch.int32)
    eg[..., 0], eg[..., 1] = 0, 1
    sel = dict(exact_groups=eg, n_exact=torch.full((1, H, 2), 2, dtype=torch.int32),
               sample_idx=torch.zeros((1, H, 2, 1), dtype=torch.int32),
               sample_bias=torch.zeros((1, H, 2, 1), dtype=torch.float32),
               n_sample=torch.zeros((1, H, 2), dtype=torch.int32), m=0)
    scale = isg.default_scale(d)
    dev = {kk: (vv.to(DEV) if torch.is_tensor(vv) else vv) for kk, vv in sel.items()}
    nfb = torch.zeros(1, device=DEV, dtype=torch.int32)
    o_p, lse_p = isg.isg_attention(q.to(DEV), k.to(DEV), v.to(DEV), qo.to(DEV), ko.to(DEV), dev, scale,
                                   n_fallback_tiles=nfb)
    torch.cuda.synchronize()
    n_tiles = H * ((nq + 127) // 128 + (N - nq + 127) // 128)
    oo, lo = orc.attention(f32(q), f32(k), f32(v), npy(qo), npy(ko), {kk: npy(vv) if torch.is_tensor(vv) else vv
                                                                      for kk, vv in sel.items() if kk != "m"},
                           0, scale)
    err = np.abs(f32(o_p) - oo).max()
    lerr = np.abs(npy(lse_p) - lo).max()
    say(f"  H={H}: {int(nfb.item())} of {n_tiles} tiles through the rescaling pass; max|O-O_oracle| {err:.3e}, "
        f"max|LSE-LSE_oracle| {lerr:.3e}, LSE {lo.min():.0f}..{lo.max():.0f}")
    assert int(nfb.item()) == n_tiles
    assert np.isfinite(f32(o_p)).all()
    assert err <= 2e-2 and lerr <= LSE_TOL_BF16 + 1e-6 * np.abs(lo).max()


def test_attention_high_entropy_zipf(orc):
    """Near-uniform attention (Q scaled by 0.2) with Zipf cluster sizes."""
    *_, o_p, lse_p, oo, lo = _attn_case(orc, 2, 4096, 128, "bf16", 16, 64, 300, 300, q_scale=0.2, zipf=1.2)
    assert np.abs(f32(o_p) - oo).max() <= 2e-2
    assert np.abs(npy(lse_p) - lo).max() <= LSE_TOL_BF16


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_all_selected_equals_dense(orc, dtype, d):
    """E = 100 %: the GPU output is dense softmax attention (fp32: within 1e-5)."""
    N = 2048
    (q, k, v), cq, ck, sel, o_p, lse_p, oo, lo = _attn_case(orc, 1, N, d, dtype, 8, 32, N, 64)
    assert np.all(npy(sel["n_sample"]) == 0)
    o, lse = isg.isg_unpermute(o_p, lse_p, cq["perm"])
    od, ld = orc.dense(f32(q), f32(k), f32(v), isg.default_scale(d))
    err = np.abs(f32(o) - od).max()
    say(f"  all-selected vs dense: {err:.3e}")
    assert err <= (1e-5 if dtype == "f32" else 2e-2)
    assert np.abs(npy(lse) - ld).max() <= (1e-5 if dtype == "f32" else LSE_TOL_BF16)


def test_every_skipped_token_weight_one(orc):
    N = 2048
    (q, k, v), cq, ck, sel, o_p, lse_p, oo, lo = _attn_case(orc, 1, N, 64, "f32", 8, 32, 0, N)
    o, _ = isg.isg_unpermute(o_p, lse_p, cq["perm"])
    od, _ = orc.dense(f32(q), f32(k), f32(v), isg.default_scale(64))
    assert np.abs(f32(o) - od).max() <= 1e-5


def test_unpermute_exact_and_strided(orc):
    B, H, N, d = 1, 3, 1000, 128
    o_p = torch.randn(B, H, N, d, device=DEV).to(torch.bfloat16)
    lse_p = torch.randn(B, H, N, device=DEV)
    perm = torch.stack([torch.randperm(N) for _ in range(H)])[None].to(torch.int32).to(DEV)
    o, lse = isg.isg_unpermute(o_p, lse_p, perm)
    ref_o, ref_l = orc.unpermute(f32(o_p).astype(np.float64), npy(lse_p).astype(np.float64), npy(perm))
    assert np.array_equal(f32(o), ref_o.astype(np.float32)) and np.array_equal(npy(lse), ref_l.astype(np.float32))
    out = torch.empty(B, N, H, d, device=DEV, dtype=torch.bfloat16)
    isg.isg_unpermute(o_p, None, perm, out=out.permute(0, 2, 1, 3))
    assert torch.equal(out.permute(0, 2, 1, 3), o)


# ------------------------------------------------------------------ whole path
def test_pipeline_tiny_config_vs_oracle(orc):
    """The tiny fp32 workload end to end; the oracle re-runs every step after the
    clustering from the GPU's clustering."""
    w = WORKLOADS["tiny_f32"]
    q, k, v, _ = make_workload(w)
    N = w["N"]
    E = budget_keys(0.25, N)
    m = budget_keys(0.25, N)
    r = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), w["Cq"], w["Ck"], w["iters"], E, m, seed=0)
    torch.cuda.synchronize()
    # the oracle's own 5-round clustering: labels agree (a near-tie in one round may
    # move a later centroid, so a few differences are allowed, each checked per round
    # by test_cluster_five_rounds)
    for c, x, C_ in (("cq", q, w["Cq"]), ("ck", k, w["Ck"])):
        oc = orc.cluster(f32(x), C_, 5)
        agree = (oc["labels"] == npy(r[c]["labels"])).mean()
        say(f"  tiny: {c} label agreement with the oracle's own clustering {agree:.5f}")
        assert agree >= 0.999, c
    S, _ = orc.probs(npy(r["cq"]["centroids"]), npy(r["ck"]["centroids"]), npy(r["ck"]["offsets"]), r["scale"])
    assert np.array_equal(S, npy(r["scores"]))
    sel = orc.select_sample(S, npy(r["ck"]["offsets"]), N, E, m, seed=0)
    for key in ("exact_groups", "n_exact", "n_sample", "sample_idx"):
        assert np.array_equal(sel[key], npy(r["sel"][key])), key
    o_p, lse_p = orc.attention(f32(r["cq"]["x_perm"]), f32(r["ck"]["x_perm"]), f32(r["ck"]["companion_perm"]),
                               npy(r["cq"]["offsets"]), npy(r["ck"]["offsets"]), sel, m, r["scale"])
    o, lse = orc.unpermute(o_p, lse_p, npy(r["cq"]["perm"]))
    assert np.abs(f32(r["o"]) - o).max() <= 1e-4
    assert np.abs(npy(r["lse"]) - lse).max() <= 1e-4


@pytest.mark.parametrize("d", [64, 128])
def test_key_norm_from_clustering_matches_attention_pass(d):
    """K's per-head largest squared row norm, fused into the last k-means update,
    against a plain fp32 reduction; and attention given it against attention
    that runs its own key-norm pass: equal bit for bit (the same arithmetic)."""
    H, N = 3, 3001
    say(f"key norms H={H} N={N} d={d}")
    q, k, v = _inputs(H, N, d, "bf16", seed=5)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    cq = isg.isg_cluster(qg, 7, 3)
    ck = isg.isg_cluster(kg, 20, 3, companion=vg, want_max_sqnorm=True)
    mx = ck["max_sqnorm"]
    ref = (kg.float() ** 2).sum(-1).amax(-1)
    rel = ((mx - ref).abs() / ref).max().item()
    say(f"  max relative difference to the fp32 reduction {rel:.2e}")
    assert rel <= 1e-5
    scale = isg.default_scale(d)
    S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
    sel = isg.isg_select_sample(S, ck["offsets"], N, 300, 200)
    args = (cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"], sel, scale)
    o_a, l_a = isg.isg_attention(*args)
    o_b, l_b = isg.isg_attention(*args, k_max_sqnorm=mx)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_attention_token_order_equals_unpermute(dtype, d):
    """Attention given the query permutation writes rows in token order: equal bit
    for bit to the permuted-order call followed by isg_unpermute (the paired-tile
    kernel, the one-tile bf16 kernel and the fp32 kernel)."""
    H, N = 2, 2500
    say(f"token-order attention H={H} N={N} d={d} {dtype}")
    q, k, v = _inputs(H, N, d, dtype, seed=9)
    r = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), 9, 24, 3, 250, 150, seed=1, fuse_unpermute=False)
    cq, ck = r["cq"], r["ck"]
    o, lse = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"],
                               r["sel"], r["scale"], k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"])
    torch.cuda.synchronize()
    assert torch.equal(o, r["o"]) and torch.equal(lse, r["lse"])


def _same_lists_and_samples(o, g):
    """Exact lists and counts equal; samples equal up to each group's n_sample
    (the entries past it are not written)."""
    for key in ("exact_groups", "n_exact", "n_sample"):
        assert np.array_equal(o[key], npy(g[key])), key
    ns, gi = o["n_sample"], npy(g["sample_idx"])
    for idx in np.ndindex(*ns.shape):
        n = ns[idx]
        assert np.array_equal(o["sample_idx"][idx][:n], gi[idx][:n]), ("sample_idx", idx)


def test_pipeline_batch_of_two_vs_oracle(orc):
    """B = 2 with ragged N: each batch's clustering equals a B = 1 run on its own
    data bit for bit, the permuted copies are exact gathers, and scores, lists,
    samples (whose counter carries the batch index), attention and un-permute
    match the oracle re-run from the GPU's clustering."""
    B, H, N, d, Cq, Ck, E, m = 2, 2, 3001, 128, 8, 40, 300, 257
    q, k, v, _ = make_qkv(H, N, d, n_centers=12, dtype="bf16", seed=21, B=B)
    r = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), Cq, Ck, 5, E, m, seed=4)
    torch.cuda.synchronize()
    for b in range(B):
        one = isg.isg_cluster(k[b:b + 1].to(DEV), Ck, 5, companion=v[b:b + 1].to(DEV))
        for key in ("labels", "centroids", "perm", "offsets", "x_perm", "companion_perm"):
            assert torch.equal(one[key][0].cpu(), r["ck"][key][b].cpu()), (b, key)
        for h in range(H):
            pk = r["ck"]["perm"][b, h].long().cpu()
            assert torch.equal(r["ck"]["x_perm"][b, h].cpu(), k[b, h][pk])
            pq = r["cq"]["perm"][b, h].long().cpu()
            assert torch.equal(r["cq"]["x_perm"][b, h].cpu(), q[b, h][pq])
    S, _ = orc.probs(npy(r["cq"]["centroids"]), npy(r["ck"]["centroids"]), npy(r["ck"]["offsets"]), r["scale"])
    assert np.array_equal(S, npy(r["scores"]))
    sel = orc.select_sample(S, npy(r["ck"]["offsets"]), N, E, m, seed=4)
    _same_lists_and_samples(sel, r["sel"])
    o_p, lse_p = orc.attention(f32(r["cq"]["x_perm"]), f32(r["ck"]["x_perm"]), f32(r["ck"]["companion_perm"]),
                               npy(r["cq"]["offsets"]), npy(r["ck"]["offsets"]), sel, m, r["scale"])
    o, lse = orc.unpermute(o_p, lse_p, npy(r["cq"]["perm"]))
    err = np.abs(f32(r["o"]) - o).max()
    lerr = np.abs(npy(r["lse"]) - lse).max()
    say(f"  B=2: max|O-O_oracle| = {err:.3e}, max|LSE-LSE_oracle| = {lerr:.3e}")
    assert err <= 2e-2 and lerr <= LSE_TOL_BF16


@pytest.mark.parametrize("H,N,d,dtype,Cq,Ck,E,m", [
    (1, 1, 128, "bf16", 1, 1, 1, 0),       # one token
    (2, 5, 64, "f32", 1, 1, 0, 5),         # one group each side, every key sampled
    (1, 64, 128, "bf16", 64, 64, 10, 10),  # C = N: a group per token
    (1, 200, 128, "bf16", 4, 8, 200, 0),   # exact budget covers every key
    (1, 130, 64, "bf16", 3, 5, 20, 20),    # d = 64 (the one-tile kernel), ragged
])
def test_pipeline_degenerate_shapes(orc, H, N, d, dtype, Cq, Ck, E, m):
    """Degenerate shapes through the whole path against the oracle re-run from the
    GPU's clustering: scores, lists and samples bit-exact, output within the bar."""
    say(f"degenerate H={H} N={N} d={d} {dtype} Cq={Cq} Ck={Ck} E={E} m={m}")
    q, k, v = _inputs(H, N, d, dtype, seed=N + d)
    r = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), Cq, Ck, 5, E, m, seed=6)
    torch.cuda.synchronize()
    for c, x in (("cq", q), ("ck", k)):
        for h in range(H):
            pp = r[c]["perm"][0, h].long().cpu()
            assert torch.equal(torch.sort(pp).values, torch.arange(N)), c
            assert torch.equal(r[c]["x_perm"][0, h].cpu(), x[0, h][pp]), c
    S, _ = orc.probs(npy(r["cq"]["centroids"]), npy(r["ck"]["centroids"]), npy(r["ck"]["offsets"]), r["scale"])
    assert np.array_equal(S, npy(r["scores"]))
    sel = orc.select_sample(S, npy(r["ck"]["offsets"]), N, E, m, seed=6)
    _same_lists_and_samples(sel, r["sel"])
    o_p, lse_p = orc.attention(f32(r["cq"]["x_perm"]), f32(r["ck"]["x_perm"]), f32(r["ck"]["companion_perm"]),
                               npy(r["cq"]["offsets"]), npy(r["ck"]["offsets"]), sel, m, r["scale"])
    o, lse = orc.unpermute(o_p, lse_p, npy(r["cq"]["perm"]))
    err = np.abs(f32(r["o"]) - o).max()
    lerr = np.abs(npy(r["lse"]) - lse).max()
    say(f"  max|O-O_oracle| = {err:.3e}, max|LSE-LSE_oracle| = {lerr:.3e}")
    if dtype == "bf16":
        assert err <= 2e-2 and lerr <= LSE_TOL_BF16
    else:
        assert err <= 1e-4 and lerr <= 1e-4


def test_pipeline_max_groups(orc):
    """Cq = Ck = 1024 (the most groups selection and attention take): 32 centroid
    tiles in the assign, a 1024-key ranking sort, one tile table slot per group;
    lists and samples bit-exact, output within the bar."""
    H, N, d, Cq, Ck, E, m = 1, 8192, 128, 1024, 1024, 600, 600
    q, k, v = _inputs(H, N, d, "bf16", seed=29, n_centers=64)
    r = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), Cq, Ck, 5, E, m, seed=8)
    torch.cuda.synchronize()
    assert int(npy(r["ck"]["labels"]).max()) < Ck and int(npy(r["cq"]["labels"]).max()) < Cq
    S, _ = orc.probs(npy(r["cq"]["centroids"]), npy(r["ck"]["centroids"]), npy(r["ck"]["offsets"]), r["scale"])
    assert np.array_equal(S, npy(r["scores"]))
    sel = orc.select_sample(S, npy(r["ck"]["offsets"]), N, E, m, seed=8)
    _same_lists_and_samples(sel, r["sel"])
    o_p, lse_p = orc.attention(f32(r["cq"]["x_perm"]), f32(r["ck"]["x_perm"]), f32(r["ck"]["companion_perm"]),
                               npy(r["cq"]["offsets"]), npy(r["ck"]["offsets"]), sel, m, r["scale"])
    o, lse = orc.unpermute(o_p, lse_p, npy(r["cq"]["perm"]))
    err = np.abs(f32(r["o"]) - o).max()
    lerr = np.abs(npy(r["lse"]) - lse).max()
    say(f"  1024 groups: max|O-O_oracle| = {err:.3e}, max|LSE-LSE_oracle| = {lerr:.3e}")
    assert err <= 2e-2 and lerr <= LSE_TOL_BF16


def test_pipeline_deterministic():
    q, k, v = _inputs(2, 4096, 128, "bf16", seed=11)
    a = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), 16, 64, 5, 400, 400, seed=3)
    b = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), 16, 64, 5, 400, 400, seed=3)
    for key in ("o", "lse", "scores"):
        assert torch.equal(a[key], b[key]), key
    for key in ("centroids", "labels", "perm"):
        assert torch.equal(a["cq"][key], b["cq"][key]) and torch.equal(a["ck"][key], b["ck"][key]), key


@pytest.mark.parametrize("mode", ["importance", "uniform"])
def test_unbiased_over_1000_seeds_gpu(orc, mode):
    """GPU path, tiny shape: the mean over 1,000 seeds of e^LSE and O e^LSE converges
    to the dense denominator and numerator (z-score test as for the oracle), for the
    importance proposal and for the uniform one."""
    say(f"unbiasedness over 1000 seeds, {mode}")
    N, d, Cq, Ck, E, m = 512, 64, 4, 16, 64, 48
    q, k, v = _inputs(1, N, d, "f32", seed=2, q_scale=0.5, n_centers=6)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = isg.default_scale(d)
    cq = isg.isg_cluster(qg, Cq, 5)
    ck = isg.isg_cluster(kg, Ck, 5, companion=vg)
    S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
    od, ld = orc.dense(f32(q), f32(k), f32(v), scale)
    Dh, Nh = [], []
    for s in range(1000):
        sel = isg.isg_select_sample(S, ck["offsets"], N, E, m, seed=s, mode=mode)
        o_p, lse_p = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                                       ck["offsets"], sel, scale)
        o, lse = isg.isg_unpermute(o_p, lse_p, cq["perm"])
        Dh.append(lse[0, 0])
        Nh.append(o[0, 0])
    lse_all = torch.stack(Dh).double().cpu().numpy()
    o_all = torch.stack(Nh).double().cpu().numpy()
    d_rel = np.exp(lse_all - ld[0, 0][None])
    n_rel = o_all * d_rel[:, :, None]
    for x, target in ((d_rel, 1.0), (n_rel, od[0, 0])):
        z = (x.mean(0) - target) / (x.std(0, ddof=1) / math.sqrt(x.shape[0]))
        zs = seed_summary_z(x, target)
        say(f"  z: max {np.abs(z).max():.2f}, frac>4 {np.mean(np.abs(z) > 4):.4f}, seed-summary z {zs:.2f}")
        assert np.mean(np.abs(z) > 4) <= 1e-3 and abs(zs) < 4


def seed_summary_z(x, target):
    """z-score of the mean over seeds of a per-seed summary: each seed's estimates,
    standardised per element by their spread over the seeds, averaged over the
    elements.  Elements of one query group share a sample, so their per-element z
    are correlated and their plain mean is not N(0, 1/#elements); the seeds are
    independent, so this summary's z is N(0, 1) when the estimator is unbiased.
    Elements with no spread (a fully enumerated skipped region) are left out."""
    x = np.asarray(x, np.float64)
    t = np.broadcast_to(np.asarray(target, np.float64), x.shape[1:]).reshape(-1)
    x = x.reshape(x.shape[0], -1)
    sd = x.std(0, ddof=1)
    keep = sd > 1e-12 * np.maximum(np.abs(t), 1e-300)
    T = ((x[:, keep] - t[keep]) / sd[keep]).mean(1)
    return float(T.mean() / (T.std(ddof=1) / math.sqrt(x.shape[0])))


# ------------------------------------------------------------------ full sizes, sampled checks
_WORKLOAD_CACHE = {}


def _workload_inputs(name):
    """Host inputs of a named workload, kept for the next test of the same workload
    (one workload at a time)."""
    if name not in _WORKLOAD_CACHE:
        _WORKLOAD_CACHE.clear()
        q, k, v, _ = make_workload(WORKLOADS[name])
        _WORKLOAD_CACHE[name] = (q, k, v)
    return _WORKLOAD_CACHE[name]


def _last_round_near_ties(orc, x_dev, x_host, C, iters, final, heads, ntok=2000, seed=0):
    """k-means at full size: the centroids before the last round come from a call
    with iters - 1 rounds, and one more round from them (given centroids)
    reproduces the final labels and centroids bit for bit.  A sample of tokens of
    each checked head is then assigned by the oracle (fp64) from those centroids:
    labels equal except near-ties (fp64 gap < 1e-5)."""
    prev = isg.isg_cluster(x_dev, C, iters - 1, want_perm=False)
    last = isg.isg_cluster(x_dev, C, 1, init=prev["centroids"], want_perm=False)
    torch.cuda.synchronize()
    assert torch.equal(last["labels"], final["labels"])
    assert torch.equal(last["centroids"], final["centroids"])
    N = x_dev.shape[2]
    rng = np.random.default_rng(seed)
    for h in heads:
        toks = np.sort(rng.choice(N, min(ntok, N), replace=False))
        xs = x_host[0, h][torch.from_numpy(toks)].float().numpy()
        cent = npy(prev["centroids"][0, h])
        lab_g = npy(final["labels"][0, h])[toks]
        lab_o = orc.kmeans_assign(xs, cent)
        say(f"  head {h}: {len(toks)} tokens, C={C}: {int((lab_g != lab_o).sum())} labels differ from the "
            f"oracle's assignment")
        assert _near_tie_ok(orc, xs, cent, lab_g, lab_o)
        # centroids are the means of the final groups (a few groups)
        lab = npy(final["labels"][0, h])
        xh = x_host[0, h].float().numpy()
        for j in rng.choice(C, 4, replace=False):
            mem = xh[lab == j].astype(np.float64)
            if len(mem):
                assert np.allclose(npy(final["centroids"][0, h, j]), mem.mean(0), rtol=1e-6, atol=1e-6)


def _lse_report(tag, lg, lo):
    e = np.abs(np.asarray(lg, np.float64) - np.asarray(lo, np.float64)).ravel()
    p50, p99, p999 = np.percentile(e, [50, 99, 99.9])
    say(f"  {tag}: |LSE - LSE_oracle| p50 {p50:.2e}  p99 {p99:.2e}  p99.9 {p999:.2e}  max {e.max():.2e}")
    return float(e.max())


def _full_size_check(orc, name, E_share, S_share, heads, groups_per_head=3, mode="importance", max_rows=None,
                     all_groups_head=None, expect_fallback=None, top_p=None):
    w = WORKLOADS[name]
    N, d, Cq, Ck = w["N"], w["d"], w["Cq"], w["Ck"]
    say(f"full size {name}: inputs")
    q, k, v = _workload_inputs(name)
    E, m = budget_keys(E_share, N), budget_keys(S_share, N)
    say(f"full size {name}: pipeline E={E} m={m} mode={mode} top_p={top_p}")
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    r = isg.pipeline(qg, kg, vg, Cq, Ck, w["iters"], E, m, seed=0, mode=mode, pq=w.get("pq"), top_p=top_p)
    torch.cuda.synchronize()
    qo_all = npy(r["cq"]["offsets"])
    ko_all = npy(r["ck"]["offsets"])
    n_tiles = int(((np.diff(qo_all, axis=-1) + 127) // 128).sum())
    n_fb = int(r["n_fallback_tiles"].item())
    say(f"  {n_fb} of {n_tiles} query tiles went to the rescaling fallback")
    assert 0 <= n_fb <= n_tiles
    if expect_fallback is not None:
        assert (n_fb > 0) == expect_fallback
    # k-means of Q and of K: the last round against the oracle on sampled tokens
    say(f"full size {name}: k-means of Q and K, last round against the oracle")
    _last_round_near_ties(orc, qg, q, Cq, w["iters"], r["cq"], heads, seed=1)
    _last_round_near_ties(orc, kg, k, Ck, w["iters"], r["ck"], heads, seed=2)
    # every head: permutations are the stable sort of the labels
    for c, C_ in (("cq", Cq), ("ck", Ck)):
        for h in heads:
            perm_o, off_o = orc.stable_sort(npy(r[c]["labels"][0, h]), C_)
            assert np.array_equal(perm_o, npy(r[c]["perm"][0, h]))
            assert np.array_equal(off_o, npy(r[c]["offsets"][0, h]))
    # every head: scores, lists, sample indices bit-exact and offsets within 1e-6, from the GPU's centroids
    S, pi_o = orc.probs(npy(r["cq"]["centroids"]), npy(r["ck"]["centroids"]), ko_all, r["scale"])
    assert np.array_equal(S, npy(r["scores"]))
    if top_p is not None:
        # the exact set's size is decided on pi, so both sides decide on the GPU's
        # pi, which itself is checked against the oracle's
        pi_g = npy(r["pi"])
        assert np.abs(pi_g.astype(np.float64) - pi_o).max() <= 1e-6
    votes = None
    if mode == "votes":
        pq = r["pq"]
        votes = npy(pq["votes"])
        rng = np.random.default_rng(1)
        for h in heads:
            hs = slice(h, h + 1)
            kbar = orc.pq_kbar(npy(pq["k_codes"][:, :, hs]), npy(pq["k_codebooks"][:, :, hs]),
                               npy(r["ck"]["perm"][:, hs]), ko_all[:, hs])
            assert np.array_equal(kbar, npy(pq["kbar"][:, hs]))
            tables = orc.pq_tables(npy(pq["q_codebooks"][:, :, hs]), kbar, r["scale"])
            assert np.array_equal(tables, npy(pq["tables"][:, hs]))
            i0 = int(rng.integers(0, Cq - 3))
            vo = orc.pq_votes(npy(pq["q_codes"][:, :, hs]), tables, npy(r["cq"]["perm"][:, hs]),
                              qo_all[:, hs, i0:i0 + 4], ko_all[:, hs], E)
            say(f"  head {h}: PQ votes of groups {i0}..{i0 + 2} vs the oracle")
            assert np.array_equal(vo[0, 0], votes[0, h, i0:i0 + 3])
    if top_p is not None:
        sel = orc.select_sample_topp(S, pi_g, ko_all, N, top_p, m, seed=0, mode=isg.MODES[mode])
        say(f"  top-p {top_p}: exact key groups per query group {int(np.median(sel['n_exact']))} (median)")
    else:
        sel = orc.select_sample(S, ko_all, N, E, m, seed=0, mode=isg.MODES[mode], votes=votes)
    for key in ("exact_groups", "n_exact", "n_sample"):
        assert np.array_equal(sel[key], npy(r["sel"][key])), key
    written = np.arange(max(m, 1))[None, None, None, :] < sel["n_sample"][..., None]
    gi_ = npy(r["sel"]["sample_idx"])
    assert np.array_equal(np.where(written, gi_, 0), np.where(written, sel["sample_idx"], 0))
    del gi_
    db = np.where(written, npy(r["sel"]["sample_bias"]).astype(np.float64) - sel["sample_bias"], 0.0)
    say(f"  sample offsets: max |GPU - oracle| {np.abs(db).max():.2e} over {int(sel['n_sample'].sum())} draws")
    assert np.abs(db).max() <= 1e-6
    del db, written
    # attention from the oracle's own lists: every group of one head, a few groups of the others
    rng = np.random.default_rng(0)
    for h in heads:
        sizes = np.diff(qo_all[0, h])
        nz = np.nonzero(sizes)[0]
        if max_rows is not None:  # keep the oracle's share of the work bounded at long sequences
            nz = nz[sizes[nz] <= max_rows]
        if h == all_groups_head:
            pick = list(nz)
        else:
            pick = [nz[np.argmax(sizes[nz])], nz[np.argmin(sizes[nz])]] + list(
                rng.choice(nz, groups_per_head - 2, replace=False))
        gm = np.zeros((1, 1, Cq), np.uint8)
        gm[0, 0, pick] = 1
        sl = lambda t: t[:, h:h + 1]
        oo, lo = orc.attention(f32(sl(r["cq"]["x_perm"])), f32(sl(r["ck"]["x_perm"])),
                               f32(sl(r["ck"]["companion_perm"])), qo_all[:, h:h + 1], ko_all[:, h:h + 1],
                               {kk: vv[:, h:h + 1] for kk, vv in sel.items() if kk != "m"}, m, r["scale"],
                               group_mask=gm)
        # the step writes O and LSE in token order: row r of the permuted order is o[perm[r]]
        ph = r["cq"]["perm"][0, h].long()
        og, lg = f32(r["o"][0, h][ph]), npy(r["lse"][0, h][ph])
        rows = np.concatenate([np.arange(qo_all[0, h, i], qo_all[0, h, i + 1]) for i in pick])
        err = np.abs(og[rows] - oo[0, 0, rows]).max()
        lerr = _lse_report(f"head {h}, {len(pick)} groups, {len(rows)} rows: max|O-O_oracle| {err:.3e}",
                           lg[rows], lo[0, 0, rows])
        assert err <= 2e-2 and lerr <= LSE_TOL_BF16


def test_full_size_480p(orc):
    _full_size_check(orc, "wan1.3b_480p", 0.08, 0.08, heads=[0, 6, 11], all_groups_head=6)


def test_full_size_1p3b_720p_16_16(orc):
    _full_size_check(orc, "wan1.3b_720p", 0.16, 0.16, heads=[0, 6, 11], groups_per_head=4)


def test_full_size_14b_720p(orc):
    _full_size_check(orc, "wan14b_720p", 0.08, 0.08, heads=[0, 20, 39], groups_per_head=4, all_groups_head=20)


@pytest.mark.parametrize("share", [0.04, 0.32])
def test_full_size_14b_720p_sweep(orc, share):
    """The budget sweep's ends at the headline shape: 4+4 % (m = 3,024) and 32+32 %
    (m = 24,192 draws per query group)."""
    _full_size_check(orc, "wan14b_720p", share, share, heads=[0, 20, 39], groups_per_head=4)


def test_full_size_14b_720p_uniform(orc):
    """The uniform variant (every skipped key equally likely) at the headline shape, 8+8 %."""
    _full_size_check(orc, "wan14b_720p", 0.08, 0.08, heads=[0, 39], groups_per_head=4, mode="uniform")


def test_full_size_14b_720p_topp(orc):
    """Top-p sizing (p = 0.9) with an 8 % sample at the headline shape."""
    _full_size_check(orc, "wan14b_720p", 0.0, 0.08, heads=[0, 39], groups_per_head=4, top_p=0.9)


def test_full_size_14b_720p_wide_norms(orc):
    """Token norms spread log-normally (|q| |k| over a wide range), so many rows sit
    far below the Cauchy-Schwarz bound (29 % of the query tiles needed the
    rescaling fallback with the bound as the reference): the reference anchored to
    the first tile's maximum keeps every tile on the fast path, and the output stays
    within the bar on every checked group."""
    _full_size_check(orc, "wan14b_720p_wide_norms", 0.08, 0.08, heads=[0, 20, 39], groups_per_head=6)


def test_full_size_14b_720p_wider_norms_rescaling_pass(orc):
    """A log-normal norm spread of 0.6: some rows' logits run so far past the first
    tile's that their sums would overflow around the anchored reference; those
    tiles are flagged and recomputed by the running-maximum pass, and every checked
    group stays within the bar."""
    _full_size_check(orc, "wan14b_720p_wider_norms", 0.08, 0.08, heads=[0, 20, 39], groups_per_head=6,
                     expect_fallback=True)


# ------------------------------------------------------------------ product-quantised votes
def _pq_stage(orc, qc, qcb, kc, kcb, cq, ck, E, scale):
    """Oracle Kbar, tables and votes from the GPU's codes (stage by stage), and the GPU's."""
    g = isg.isg_pq_votes(qc, qcb, kc, kcb, cq["perm"], cq["offsets"], ck["perm"], ck["offsets"], E, scale)
    torch.cuda.synchronize()
    kbar = orc.pq_kbar(npy(kc), npy(kcb), npy(ck["perm"]), npy(ck["offsets"]))
    tables = orc.pq_tables(npy(qcb), kbar, scale)
    votes = orc.pq_votes(npy(qc), tables, npy(cq["perm"]), npy(cq["offsets"]), npy(ck["offsets"]), E)
    return g, kbar, tables, votes


@pytest.mark.parametrize("H,N,d,P,Cc,Cq,Ck,E", [
    (2, 2000, 128, 8, 64, 10, 50, 200),     # one key group per lane
    (2, 3000, 128, 8, 128, 12, 100, 300),   # two per lane
    (1, 3000, 128, 8, 64, 8, 200, 0),       # exact_keys 0: only the top group
    (1, 4096, 128, 8, 256, 16, 500, 400),   # the 500-group shape
    (1, 5000, 64, 4, 32, 8, 1000, 500),     # sixteen per lane
    (1, 2048, 128, 8, 64, 8, 64, 4096),     # every group fits
])
def test_pq_votes_stagewise(orc, H, N, d, P, Cc, Cq, Ck, E):
    """Kbar, tables and votes bit-exact against the oracle given the same codes."""
    say(f"pq votes H={H} N={N} d={d} P={P} Cc={Cc} Cq={Cq} Ck={Ck} E={E}")
    (q, k, v), cq, ck = _clustered(H, N, d, "bf16", Cq, Ck, seed=P + Ck)
    qc, qcb = isg.pq_codebooks(q.to(DEV), P, Cc, 3)
    kc, kcb = isg.pq_codebooks(k.to(DEV), P, Cc, 3)
    scale = isg.default_scale(d)
    g, kbar, tables, votes = _pq_stage(orc, qc, qcb, kc, kcb, cq, ck, E, scale)
    assert np.array_equal(npy(g["kbar"]), kbar)
    assert np.array_equal(npy(g["tables"]), tables)
    assert np.array_equal(npy(g["votes"]), votes)
    assert (votes.sum(-1) >= np.diff(npy(cq["offsets"]), axis=-1)).all()


@pytest.mark.parametrize("N,E", [(1_100_000, 200_000), (20_000, 19_999)])
def test_pq_votes_unequal_groups_and_long_rows(orc, N, E):
    """Query groups of very unequal size (Zipf component prior), so the fixed query
    chunks of the votes kernel cross group boundaries (and skip any empty group); at
    N = 1.1 million tokens the group sizes no longer fit the packed 20-bit sums and
    the search runs without its early exit; E = N - 1 leaves one key out."""
    H, d, P, Cc, Cq, Ck = 1, 16, 1, 16, 40, 32
    say(f"pq votes unequal groups N={N} E={E}")
    (q, k, v), cq, ck = _clustered(H, N, d, "bf16", Cq, Ck, seed=17, q_scale=0.3, zipf=1.2)
    nq = np.diff(npy(cq["offsets"])[0, 0])
    say(f"  query group sizes: max {nq.max()}, mean {nq.mean():.0f}, empty {(nq == 0).sum()}")
    qc, qcb = isg.pq_codebooks(q.to(DEV), P, Cc, 3)
    kc, kcb = isg.pq_codebooks(k.to(DEV), P, Cc, 3)
    scale = isg.default_scale(d)
    g, kbar, tables, votes = _pq_stage(orc, qc, qcb, kc, kcb, cq, ck, E, scale)
    assert np.array_equal(npy(g["tables"]), tables)
    assert np.array_equal(npy(g["votes"]), votes)


def test_pq_votes_sixteen_subspaces(orc):
    """P = 16 subspaces of 16 dims (d = 256), more than one batch of table rows per
    query: codes and codebooks are given directly (random), the group structure
    comes from a real clustering; Kbar, tables and votes bit-exact."""
    H, N, Cq, Ck, P, Cc, ds, E = 1, 3000, 8, 100, 16, 32, 16, 300
    (q, k, v), cq, ck = _clustered(H, N, 128, "bf16", Cq, Ck, seed=33)
    g = torch.Generator().manual_seed(33)
    qc = torch.randint(0, Cc, (P, 1, H, N), generator=g, dtype=torch.int32).to(DEV)
    kc = torch.randint(0, Cc, (P, 1, H, N), generator=g, dtype=torch.int32).to(DEV)
    qcb = torch.randn((P, 1, H, Cc, ds), generator=g).to(DEV)
    kcb = torch.randn((P, 1, H, Cc, ds), generator=g).to(DEV)
    scale = isg.default_scale(P * ds)
    gv, kbar, tables, votes = _pq_stage(orc, qc, qcb, kc, kcb, cq, ck, E, scale)
    assert np.array_equal(npy(gv["kbar"]), kbar)
    assert np.array_equal(npy(gv["tables"]), tables)
    assert np.array_equal(npy(gv["votes"]), votes)


def test_pq_votes_all_scores_tied(orc):
    """Every key has the same codes, so every group mean (and score) is equal: the
    ranking is by group id alone, and the exact-set rule stops part-way."""
    H, N, d, P, Cc, Cq, Ck = 1, 3000, 128, 8, 32, 8, 100
    (q, k, v), cq, ck = _clustered(H, N, d, "bf16", Cq, Ck, seed=5)
    qc, qcb = isg.pq_codebooks(q.to(DEV), P, Cc, 2)
    kc = torch.zeros_like(qc)
    kcb = qcb.clone()
    scale = isg.default_scale(d)
    for E in (0, 7, 250, 1234):
        g, _, _, votes = _pq_stage(orc, qc, qcb, kc, kcb, cq, ck, E, scale)
        assert np.array_equal(npy(g["votes"]), votes), E


@pytest.mark.parametrize("B,dtype,P,Cc", [(1, "bf16", 8, 64), (2, "bf16", 8, 256), (1, "f32", 2, 40),
                                           (2, "bf16", 1, 16), (1, "bf16", 8, 300)])
def test_pq_codebooks_strided_and_vs_oracle(orc, B, dtype, P, Cc):
    """isg_pq_codebooks (subspace-major copy, then the rounds over every subspace,
    batch and head at once) equals isg_cluster on each subspace alone, bit for
    bit, through a strided view of the input.  For bf16 16-dim subspaces with at
    most 256 codewords the means come from exact integer sums, isg_cluster's from
    fp64 sums in sorted order: on these inputs both sums are exact, so the two
    agree bit for bit.  Agreement with the oracle's own k-means of each subspace
    is reported and bounded."""
    H, N, d = 2, 3000, 128
    say(f"pq codebooks B={B} {dtype} P={P} Cc={Cc}")
    xs = [_inputs(H, N, d, dtype, seed=21 + b)[0] for b in range(B)]
    q = torch.stack([x[0] for x in xs])  # [B, H, N, d]
    # a strided view: every token row padded to 2 d elements
    big = torch.zeros((B, H, N, 2 * d), dtype=q.dtype, device=DEV)
    big[..., :d] = q.to(DEV)
    qg = big[..., :d]
    codes, cbs = isg.pq_codebooks(qg, P, Cc, 3)
    ds = d // P
    for s in sorted({0, P // 2, P - 1}):
        r = isg.isg_cluster(qg[..., s * ds:(s + 1) * ds].contiguous(), Cc, 3)
        assert torch.equal(r["labels"], codes[s]) and torch.equal(r["centroids"], cbs[s]), s
    oc, ocb = orc.pq_codebooks(f32(q), P, Cc, 3)
    agree = (oc == npy(codes)).mean()
    say(f"  PQ code agreement with the oracle's own k-means: {agree:.5f}")
    assert agree > 0.97
    if dtype == "bf16" and d // P == 16:
        # labels decided in the exact definition's arithmetic and means from exact
        # sums: the whole k-means equals the oracle's, round after round
        assert agree == 1.0 and np.array_equal(npy(cbs), ocb)


@pytest.mark.parametrize("N,Cc", [(700, 256), (3000, 64), (20000, 200), (5, 3), (8193, 256), (140000, 256)])
def test_pq_codebooks_integer_means_wide_span(N, Cc):
    """The integer-sum update of bf16 16-dim subspaces on values spread over 2^60
    (each element times 2^u, u uniform in [-60, 0]): the fixed-point grid then
    drops the low bits of the smallest values, so the means are checked against
    the exact mean of each group (math.fsum, fp64), within one fp32 ulp plus the
    grid's bound, with the labels of one round (from the data-point start, the
    same assign as isg_cluster) equal to isg_cluster's.  Two calls agree bit for
    bit: integer sums do not depend on the order of the atomics."""
    say(f"pq integer means wide span N={N} Cc={Cc}")
    H, d, P = 2, 64, 4
    g = np.random.default_rng(N + Cc)
    x = g.standard_normal((1, H, N, d)) * np.exp2(g.uniform(-60, 0, (1, H, N, d)))
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xg = xb.to(DEV)
    codes, cbs = isg.pq_codebooks(xg, P, Cc, 1)
    codes2, cbs2 = isg.pq_codebooks(xg, P, Cc, 1)
    assert torch.equal(codes, codes2) and torch.equal(cbs, cbs2)
    xv = xb.to(torch.float64).numpy()
    L = 0
    while (1 << L) <= N:
        L += 1
    lim = min(62 - L, 51)
    c_np, cb_np = npy(codes), npy(cbs)
    for s in range(P):
        sub = xg[..., s * 16:(s + 1) * 16]
        r = isg.isg_cluster(sub.contiguous(), Cc, 1)
        assert torch.equal(r["labels"], codes[s]), s
        for h in range(H):
            xs = xv[0, h, :, s * 16:(s + 1) * 16]
            bits = xb[0, h, :, s * 16:(s + 1) * 16].contiguous().view(torch.int16).numpy().astype(np.int64)
            E = max(int(((bits >> 7) & 0xFF).max()), 1)
            grid = 2.0 ** -(126 - E + lim)
            lab = c_np[s, 0, h]
            for j in np.unique(lab):
                rows = xs[lab == j]
                n = len(rows)
                exact = np.array([math.fsum(rows[:, e]) / n for e in range(16)])
                got = cb_np[s, 0, h, j].astype(np.float64)
                ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
                assert np.all(np.abs(got - exact) <= ulp + grid * (n / 2 + 1) / n), (s, h, j)


def test_pipeline_votes_mode_vs_oracle(orc):
    """Votes mode end to end: the oracle re-runs PQ votes, selection (mode 2) and
    attention from the GPU's clustering and codes."""
    H, N, d, Cq, Ck, E, m, P, Cc = 2, 4096, 128, 16, 64, 400, 400, 8, 64
    q, k, v = _inputs(H, N, d, "bf16", seed=8, q_scale=0.5, zipf=1.2)
    r = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), Cq, Ck, 3, E, m, mode="votes", pq=(P, Cc), seed=4)
    torch.cuda.synchronize()
    pq = r["pq"]
    kbar = orc.pq_kbar(npy(pq["k_codes"]), npy(pq["k_codebooks"]), npy(r["ck"]["perm"]), npy(r["ck"]["offsets"]))
    tables = orc.pq_tables(npy(pq["q_codebooks"]), kbar, r["scale"])
    votes = orc.pq_votes(npy(pq["q_codes"]), tables, npy(r["cq"]["perm"]), npy(r["cq"]["offsets"]),
                         npy(r["ck"]["offsets"]), E)
    assert np.array_equal(votes, npy(pq["votes"]))
    sel = orc.select_sample(npy(r["scores"]), npy(r["ck"]["offsets"]), N, E, m, mode=2, votes=votes, seed=4)
    for key in ("exact_groups", "n_exact", "n_sample", "sample_idx"):
        assert np.array_equal(sel[key], npy(r["sel"][key])), key
    o_p, lse_p = orc.attention(f32(r["cq"]["x_perm"]), f32(r["ck"]["x_perm"]), f32(r["ck"]["companion_perm"]),
                               npy(r["cq"]["offsets"]), npy(r["ck"]["offsets"]), sel, m, r["scale"])
    o, lse = orc.unpermute(o_p, lse_p, npy(r["cq"]["perm"]))
    assert np.abs(f32(r["o"]) - o).max() <= 2e-2
    assert np.abs(npy(r["lse"]) - lse).max() <= LSE_TOL_BF16


def test_full_size_14b_720p_pq_votes(orc):
    _full_size_check(orc, "wan14b_720p_stress_pq", 0.08, 0.08, heads=[0, 39], groups_per_head=3, mode="votes")


# ------------------------------------------------------------------ top-p exact-set sizing
@pytest.mark.parametrize("p,m,mode", [(1e-6, 400, "importance"), (0.5, 400, "importance"), (0.9, 400, "uniform"),
                                      (0.99, 300, "importance"), (1.0, 200, "importance"), (2.0, 100, "uniform"),
                                      (0.9, 4096, "importance"), (0.7, 0, "importance")])
def test_select_topp_bit_exact(orc, p, m, mode):
    """Lists and samples of the top-p rule bit-exact against the oracle given the GPU's pi."""
    say(f"select top-p p={p} m={m} mode={mode}")
    (q, k, v), cq, ck = _clustered(2, 4096, 128, "bf16", 16, 64, zipf=1.2, q_scale=0.5)
    scale = isg.default_scale(128)
    S, pi = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale)
    g = isg.isg_select_sample_topp(S, pi, ck["offsets"], 4096, p, m, mode=mode, seed=7, call_id=2)
    o = orc.select_sample_topp(npy(S), npy(pi), npy(ck["offsets"]), 4096, p, m, mode=isg.MODES[mode], seed=7,
                               call_id=2)
    for key in ("exact_groups", "n_exact", "n_sample"):
        assert np.array_equal(npy(g[key]), o[key]), key
    ns = o["n_sample"]
    for b in range(ns.shape[0]):
        for h in range(ns.shape[1]):
            for i in range(ns.shape[2]):
                n = ns[b, h, i]
                assert np.array_equal(npy(g["sample_idx"])[b, h, i, :n], o["sample_idx"][b, h, i, :n])
                assert np.abs(npy(g["sample_bias"])[b, h, i, :n] - o["sample_bias"][b, h, i, :n]).max(
                    initial=0) <= 1e-6


def test_pipeline_topp_vs_oracle(orc):
    """Top-p sizing end to end: lists from the GPU's pi, attention and un-permute against the oracle."""
    H, N, d, Cq, Ck, m = 2, 4096, 128, 16, 64, 300
    q, k, v = _inputs(H, N, d, "bf16", seed=19, q_scale=0.5, zipf=1.2)
    r = isg.pipeline(q.to(DEV), k.to(DEV), v.to(DEV), Cq, Ck, 3, 0, m, top_p=0.8, seed=5)
    torch.cuda.synchronize()
    sel = orc.select_sample_topp(npy(r["scores"]), npy(r["pi"]), npy(r["ck"]["offsets"]), N, 0.8, m, seed=5)
    for key in ("exact_groups", "n_exact", "n_sample", "sample_idx"):
        assert np.array_equal(sel[key], npy(r["sel"][key])), key
    o_p, lse_p = orc.attention(f32(r["cq"]["x_perm"]), f32(r["ck"]["x_perm"]), f32(r["ck"]["companion_perm"]),
                               npy(r["cq"]["offsets"]), npy(r["ck"]["offsets"]), sel, m, r["scale"])
    o, lse = orc.unpermute(o_p, lse_p, npy(r["cq"]["perm"]))
    assert np.abs(f32(r["o"]) - o).max() <= 2e-2
    assert np.abs(npy(r["lse"]) - lse).max() <= LSE_TOL_BF16


# ------------------------------------------------------------------ error against density (trend checks)
def _density_errors(orc, zipf, q_scale, seed=3):
    """Relative L2 error of GPU calls against the oracle's dense rows (fp64), for
    exact-only (E+S exact) and exact+importance / exact+uniform at matched density."""
    from block_sparse_attention_means_amd.synth import structured_values
    H, N, d, Cq, Ck = 2, 8192, 64, 16, 64
    q, k, v, comp = make_qkv(H, N, d, n_centers=16, q_scale=q_scale, zipf=zipf, seed=seed, dtype="bf16")
    v = structured_values(comp, d, n_centers=16, seed=seed, dtype="bf16")
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = isg.default_scale(d)
    cq = isg.isg_cluster(qg, Cq, 5)
    ck = isg.isg_cluster(kg, Ck, 5, companion=vg)
    S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
    rows = np.random.default_rng(1).choice(N, 128, replace=False)
    od, _ = orc.dense(f32(q), f32(k), f32(v), scale, rows=rows)
    out = {}
    for share in (0.04, 0.08, 0.16):
        E = budget_keys(share, N)
        res = {}
        for name, e2, m2, mode in (("exact_only", budget_keys(2 * share, N), 0, "importance"),
                                   ("importance", E, E, "importance"), ("uniform", E, E, "uniform")):
            errs = []
            for s in range(1 if m2 == 0 else 3):
                sel = isg.isg_select_sample(S, ck["offsets"], N, e2, m2, mode=mode, seed=s)
                o_p, lse_p = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                                               ck["offsets"], sel, scale)
                o, _ = isg.isg_unpermute(o_p, lse_p, cq["perm"])
                og = f32(o)[:, :, rows]
                errs.append(np.linalg.norm(og - od) / np.linalg.norm(od))
            res[name] = float(np.mean(errs))
        out[share] = res
        say(f"  share {share}: " + ", ".join(f"{kk} {vv:.4f}" for kk, vv in res.items()))
    return out


@pytest.mark.parametrize("zipf,q_scale", [(None, 1.0), (1.2, 0.2)])
def test_error_against_density_trends(orc, zipf, q_scale):
    """With values that carry the keys' structure, exact + importance sample beats
    exact-only at matched density (the unbiased estimate keeps the skipped region's
    contribution), and its error falls as the budget grows."""
    out = _density_errors(orc, zipf, q_scale)
    shares = sorted(out)
    for sh in shares:
        assert out[sh]["importance"] < out[sh]["exact_only"], sh
    assert out[shares[-1]]["importance"] < out[shares[0]]["importance"]


def test_long_sequence_84_frames(orc):
    """Sequence-length scaling: 84 latent frames (N = 302,400) at 8+8 %, checked like
    the full-size cases (query groups of at most 1,500 rows go to the oracle)."""
    _full_size_check(orc, "wan14b_720p_84f", 0.08, 0.08, heads=[0, 1], groups_per_head=3, max_rows=1500)


@pytest.mark.parametrize("P,Cc", [(16, 32), (2, 64), (4, 300)])
def test_pq_votes_other_subspace_widths(orc, P, Cc):
    """Subspace widths 8, 64 and 32 dims (random codes and codebooks): Kbar, tables and
    votes bit-exact, through both table kernels."""
    H, N, d, Cq, Ck, E = 2, 3000, 128, 10, 80, 250
    say(f"pq votes P={P} Cc={Cc}")
    (q, k, v), cq, ck = _clustered(H, N, d, "bf16", Cq, Ck, seed=P)
    rng = np.random.default_rng(P)
    ds = d // P
    qc = torch.from_numpy(rng.integers(0, Cc, (P, 1, H, N)).astype(np.int32)).to(DEV)
    kc = torch.from_numpy(rng.integers(0, Cc, (P, 1, H, N)).astype(np.int32)).to(DEV)
    qcb = torch.from_numpy(rng.standard_normal((P, 1, H, Cc, ds)).astype(np.float32)).to(DEV)
    kcb = torch.from_numpy(rng.standard_normal((P, 1, H, Cc, ds)).astype(np.float32)).to(DEV)
    g, kbar, tables, votes = _pq_stage(orc, qc, qcb, kc, kcb, cq, ck, E, isg.default_scale(d))
    assert np.array_equal(npy(g["kbar"]), kbar)
    assert np.array_equal(npy(g["tables"]), tables)
    assert np.array_equal(npy(g["votes"]), votes)
