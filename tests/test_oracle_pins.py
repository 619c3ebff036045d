"""Pins of the CPU oracle to things other than itself (library routines, closed
forms, invariants, brute force, statistics).  No GPU needed.

Each test names what it pins and which plausible mistake it would catch.
"""
import math

import numpy as np
import pytest
import scipy.cluster.vq as vq
import scipy.stats
import torch

from block_sparse_attention_means_amd.synth import make_qkv


# ---------------------------------------------------------------- Philox / table
@pytest.mark.parametrize("ctr,key", [
    ([1, 0, 0, 0], [0, 0]),
    ([1, 7, 3, 0], [0, 0]),
    ([5, 99, 39, 1], [123456789, 42]),
    ([2**63 + 5, 2**64 - 1, 2**40, 12345], [2**64 - 1, 2**63 - 1]),
])
def test_philox_matches_numpy(orc, ctr, key):
    """Raw Philox4x64-10 block equals numpy's Philox (a library implementation of
    the same published generator).  numpy bumps its counter before producing a
    block, so block c corresponds to numpy state counter c - 1."""
    bg = np.random.Philox(counter=np.array([ctr[0] - 1] + ctr[1:], np.uint64),
                          key=np.array(key, np.uint64))
    ref = bg.random_raw(4).astype(np.uint64)
    got = orc.philox4x64_10(ctr, key)
    assert np.array_equal(got, ref)


def test_philox_differs_per_word_and_counter(orc):
    a = orc.philox4x64_10([1, 0, 0, 0], [0, 0])
    b = orc.philox4x64_10([2, 0, 0, 0], [0, 0])
    c = orc.philox4x64_10([1, 0, 0, 0], [1, 0])
    assert len(set(a.tolist()) | set(b.tolist()) | set(c.tolist())) == 12


def test_proposal_table(orc):
    """tbl[k] = round(2^31 * 2^(-k/256)): monotone, endpoints, and within half a unit
    of numpy's exp2 (independent libm path)."""
    t = orc.proposal_table().astype(np.int64)
    assert t[0] == 2**31
    assert np.all(np.diff(t) < 0)
    exact = np.exp2(31.0 - np.arange(256) / 256.0)
    assert np.all(np.abs(t - exact) <= 0.5)
    # one more grid step past the end halves the first entry
    assert abs(t[255] * 2 ** (-1 / 256) - 2**30) < 1.0


# ---------------------------------------------------------------- k-means
def _kmeans2_step(data64, cent32):
    with np.errstate(all="ignore"):
        import warnings
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            c, lab = vq.kmeans2(data64, cent32.astype(np.float64), iter=1, minit="matrix",
                                missing="warn")
    return c, lab


@pytest.mark.parametrize("n,d,C", [(400, 8, 10), (2048, 64, 32), (300, 16, 40)])
def test_kmeans_step_matches_scipy(orc, n, d, C):
    """One Lloyd round (assign, update; empty keeps its centroid) equals scipy's
    kmeans2(iter=1) -- labels exactly, centroids after rounding to fp32."""
    rng = np.random.default_rng(n + d + C)
    x = (rng.standard_normal((n, d)) + 3 * rng.standard_normal((6, d))[rng.integers(0, 6, n)])
    x = x.astype(np.float32)
    cent = x[(np.arange(C) * n) // C].copy()
    for _ in range(4):
        c_ref, lab_ref = _kmeans2_step(x.astype(np.float64), cent)
        lab = orc.kmeans_assign(x, cent)
        assert np.array_equal(lab, lab_ref)
        c_new, cnt = orc.kmeans_update(x, lab, cent)
        assert np.array_equal(c_new, c_ref.astype(np.float32))
        assert np.array_equal(cnt, np.bincount(lab, minlength=C))
        cent = c_new


def test_kmeans_empty_cluster_keeps_centroid(orc):
    x = np.array([[0.0], [0.1], [10.0], [10.1]], np.float32)
    cent = np.array([[0.0], [10.0], [100.0]], np.float32)
    lab = orc.kmeans_assign(x, cent)
    assert lab.tolist() == [0, 0, 1, 1]
    c, cnt = orc.kmeans_update(x, lab, cent)
    assert cnt.tolist() == [2, 2, 0]
    assert c[2, 0] == 100.0
    assert abs(c[0, 0] - 0.05) < 1e-7 and abs(c[1, 0] - 10.05) < 1e-6


def test_kmeans_tie_goes_to_lowest_index(orc):
    x = np.array([[1.0, 0.0]], np.float32)
    cent = np.array([[0.0, 1.0], [1.0, 1.0], [1.0, -1.0]], np.float32)
    assert orc.kmeans_assign(x, cent).tolist() == [1]


def test_cluster_invariants(orc):
    """Whole clustering step: strided init, objective never increases, labels are the
    argmin against the centroids of the previous round, each final centroid is the mean
    of its final group, perm is the stable sort by label, offsets the prefix of counts,
    x_perm/companion gathered by perm."""
    q, k, v, _ = make_qkv(2, 1024, 16, n_centers=8, dtype="f32", seed=3)
    q = q.numpy()
    v = v.numpy()
    C = 12
    prev_obj = np.inf
    cent = q[:, :, (np.arange(C) * 1024) // C].copy()
    for iters in range(1, 6):
        r = orc.cluster(q, C, iters, companion=v)
        x0 = q[0, 0].astype(np.float64)
        c0 = r["centroids"][0, 0].astype(np.float64)
        lab = r["labels"][0, 0]
        obj = ((x0 - c0[lab]) ** 2).sum()
        assert obj <= prev_obj * (1 + 1e-9)
        prev_obj = obj
    for bh in [(0, 0), (0, 1)]:
        x = q[bh].astype(np.float64)
        lab = r["labels"][bh]
        cen = r["centroids"][bh]
        for j in range(C):
            mem = x[lab == j]
            if len(mem):
                assert np.allclose(cen[j], mem.mean(0), rtol=0, atol=1e-6)
        perm = r["perm"][bh]
        assert np.array_equal(perm, np.argsort(lab, kind="stable"))
        assert np.array_equal(r["offsets"][bh], np.concatenate([[0], np.cumsum(np.bincount(lab, minlength=C))]))
        assert np.array_equal(r["x_perm"][bh], q[bh][perm])
        assert np.array_equal(r["companion_perm"][bh], v[bh][perm])
    # labels are the argmin against the centroids of the round before the last
    r4 = orc.cluster(q, C, 4)
    r5 = orc.cluster(q, C, 5)
    lab_ref = orc.kmeans_assign(q[0, 1], r4["centroids"][0, 1])
    assert np.array_equal(lab_ref, r5["labels"][0, 1])
    # explicit init equals strided init
    r_init = orc.cluster(q, C, 5, init=cent)
    assert np.array_equal(r_init["labels"], r5["labels"])


def test_stable_sort_matches_numpy(orc):
    rng = np.random.default_rng(1)
    lab = rng.integers(0, 37, 5000).astype(np.int32)
    perm, off = orc.stable_sort(lab, 40)
    assert np.array_equal(perm, np.argsort(lab, kind="stable"))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(lab, minlength=40))]))


# ---------------------------------------------------------------- scores and pi
def _groups(rng, Ck, N, n_empty=0):
    counts = rng.multinomial(N - 0, np.ones(Ck) / Ck)
    if n_empty:
        counts[rng.choice(Ck, n_empty, replace=False)] = 0
        counts[0] += N - counts.sum()
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return counts, off


def test_probs_closed_form(orc):
    """S_ij is the scaled centroid dot product (fp32 rounding only); pi is the
    size-weighted softmax: sums to 1, ratios n_j/n_j' e^(S_ij - S_ij'), empty -> 0."""
    rng = np.random.default_rng(7)
    B, H, Cq, Ck, d = 1, 2, 5, 16, 64
    cq = rng.standard_normal((B, H, Cq, d)).astype(np.float32)
    ck = rng.standard_normal((B, H, Ck, d)).astype(np.float32)
    offs = []
    for _ in range(H):
        counts, off = _groups(rng, Ck, 500, n_empty=3)
        offs.append(off)
    ko = np.stack(offs)[None]
    scale = np.float32(1 / math.sqrt(d))
    S, pi = orc.probs(cq, ck, ko, scale)
    ref = np.einsum("bhid,bhjd->bhij", cq.astype(np.float64), ck.astype(np.float64)) * float(scale)
    assert np.allclose(S, ref, rtol=0, atol=2e-6 * np.abs(ref).max())
    n = np.diff(ko, axis=-1)[:, :, None, :].astype(np.float64)
    assert np.allclose(pi.sum(-1), 1.0, atol=1e-12)
    assert np.all(pi[np.broadcast_to(n == 0, pi.shape)] == 0)
    i, j1, j2 = 2, 4, 9
    for h in range(H):
        if n[0, h, 0, j1] and n[0, h, 0, j2]:
            ratio = pi[0, h, i, j1] / pi[0, h, i, j2]
            want = n[0, h, 0, j1] / n[0, h, 0, j2] * math.exp(float(S[0, h, i, j1]) - float(S[0, h, i, j2]))
            assert abs(ratio / want - 1) < 1e-12


# ---------------------------------------------------------------- exact set
def _brute_exact(S, counts, E, votes=None):
    ne = [j for j in range(len(counts)) if counts[j] > 0]
    if votes is None:
        order = sorted(ne, key=lambda j: (-float(S[j]), j))
    else:
        order = sorted(ne, key=lambda j: (-int(votes[j]), -float(S[j]), j))
    taken, cum = [], 0
    for p, j in enumerate(order):
        if p > 0 and cum + counts[j] > E:
            break
        taken.append(j)
        cum += counts[j]
    return sorted(taken)


@pytest.mark.parametrize("E", [0, 1, 40, 120, 333, 999, 1000])
def test_exact_set_brute_force(orc, E):
    rng = np.random.default_rng(E)
    Ck, N = 24, 1000
    counts, off = _groups(rng, Ck, N, n_empty=4)
    S = np.round(rng.standard_normal((1, 1, 6, Ck)), 1).astype(np.float32)   # rounding makes ties
    r = orc.select_sample(S, off[None, None], N, E, m=10)
    for i in range(6):
        want = _brute_exact(S[0, 0, i], counts, E)
        got = r["exact_groups"][0, 0, i, :r["n_exact"][0, 0, i]].tolist()
        assert got == want
        assert np.all(r["exact_groups"][0, 0, i, len(got):] == -1)
        # top group always present; budget respected unless it is the top group alone
        top = min((j for j in range(Ck) if counts[j]), key=lambda j: (-float(S[0, 0, i, j]), j))
        assert top in got
        tot = counts[got].sum()
        assert tot <= E or len(got) == 1
    if E >= N:
        assert all(r["n_exact"][0, 0] == (counts > 0).sum())


# ---------------------------------------------------------------- sampler
def _tiny_selection(orc, seed=0, E=60, m=40, N=600, Ck=16, mode=0):
    rng = np.random.default_rng(11)
    counts, off = _groups(rng, Ck, N, n_empty=2)
    S = (1.5 * rng.standard_normal((1, 1, 3, Ck))).astype(np.float32)
    r = orc.select_sample(S, off[None, None], N, E, m, mode=mode, seed=seed)
    return S, counts, off, r


def test_sample_rows_in_skipped_groups(orc):
    S, counts, off, r = _tiny_selection(orc)
    for i in range(3):
        ex = set(r["exact_groups"][0, 0, i, :r["n_exact"][0, 0, i]].tolist())
        rows = r["sample_idx"][0, 0, i, :r["n_sample"][0, 0, i]]
        g = np.searchsorted(off, rows, side="right") - 1
        assert r["n_sample"][0, 0, i] == 40
        assert all(counts[x] > 0 and x not in ex for x in g)
        assert np.all((rows >= 0) & (rows < 600))


def test_sample_deterministic_and_seeded(orc):
    _, _, _, a = _tiny_selection(orc, seed=5)
    _, _, _, b = _tiny_selection(orc, seed=5)
    _, _, _, c = _tiny_selection(orc, seed=6)
    assert np.array_equal(a["sample_idx"], b["sample_idx"])
    assert not np.array_equal(a["sample_idx"], c["sample_idx"])


@pytest.mark.parametrize("mode", [0, 1])
def test_sample_offsets_match_pi(orc, mode):
    """Offset b = -ln(m p) with p the per-key draw probability.  Importance mode:
    p = pi~_g / n_g with pi~ = pi renormalised over the skipped groups, up to the
    2^(-1/256) quantisation of the proposal (relative error < 0.2 %) where the weight is
    not floored; uniform mode: p = 1/M exactly."""
    S, counts, off, r = _tiny_selection(orc, mode=mode)
    m = 40
    for i in range(3):
        ex = set(r["exact_groups"][0, 0, i, :r["n_exact"][0, 0, i]].tolist())
        skip = [j for j in range(16) if counts[j] > 0 and j not in ex]
        w = np.array([counts[j] * math.exp(float(S[0, 0, i, j])) for j in skip])
        pt = w / w.sum()
        M = sum(counts[j] for j in skip)
        rows = r["sample_idx"][0, 0, i]
        bias = r["sample_bias"][0, 0, i]
        g = np.searchsorted(off, rows, side="right") - 1
        for t in range(m):
            p_key = math.exp(-float(bias[t])) / m
            if mode == 1:
                assert abs(p_key * M - 1) < 1e-6
            else:
                k = skip.index(g[t])
                want = pt[k] / counts[g[t]]
                # floor-1 weights only hit groups ~ e^-21 below the max; none here
                assert abs(p_key / want - 1) < 2e-3


def test_sample_frequencies_chi_square(orc):
    """Draw frequencies per group follow the probabilities implied by the offsets
    (n_g e^{-b}/m): chi-square goodness of fit over 200 seeds x 400 draws; keys inside
    a group are drawn uniformly."""
    m, i = 400, 1
    rows, bias = [], []
    for s in range(200):
        S, counts, off, r = _tiny_selection(orc, m=m, seed=s)
        assert r["n_sample"][0, 0, i] == m
        rows.append(r["sample_idx"][0, 0, i])
        bias.append(r["sample_bias"][0, 0, i].astype(np.float64))
    rows, bias = np.concatenate(rows), np.concatenate(bias)
    g = np.searchsorted(off, rows, side="right") - 1
    groups = np.unique(g)
    obs = np.array([(g == j).sum() for j in groups])
    p = np.array([counts[j] * math.exp(-bias[g == j][0]) / m for j in groups])
    ex = set(r["exact_groups"][0, 0, i, :r["n_exact"][0, 0, i]].tolist())
    skip = [j for j in range(16) if counts[j] > 0 and j not in ex]
    assert abs(p.sum() - 1) < 1e-5 and len(groups) == len(skip)
    chi2, pval = scipy.stats.chisquare(obs, p / p.sum() * obs.sum())
    assert pval > 1e-4
    j = groups[np.argmax(obs)]
    kk = rows[g == j] - off[j]
    _, pv2 = scipy.stats.chisquare(np.bincount(kk, minlength=counts[j]))
    assert pv2 > 1e-4


def test_enumeration_when_budget_covers_skipped(orc):
    S, counts, off, r = _tiny_selection(orc, E=60, m=600)
    for i in range(3):
        ex = set(r["exact_groups"][0, 0, i, :r["n_exact"][0, 0, i]].tolist())
        want = [row for j in range(16) if counts[j] and j not in ex for row in range(off[j], off[j + 1])]
        ns = r["n_sample"][0, 0, i]
        assert r["sample_idx"][0, 0, i, :ns].tolist() == want
        assert np.all(r["sample_bias"][0, 0, i, :ns] == 0)


# ---------------------------------------------------------------- attention
def _sdpa_ref(q, k, v, bias, scale):
    """torch fp64 scaled_dot_product_attention with an additive mask, plus logsumexp."""
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))
    vt = torch.from_numpy(v.astype(np.float64))
    bt = torch.from_numpy(bias.astype(np.float64))[None, :].expand(q.shape[0], -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                                         attn_mask=bt[None], scale=scale)[0]
    lse = torch.logsumexp(qt @ kt.T * scale + bt, dim=-1)
    return o.numpy(), lse.numpy()


def _clustered(orc, H=1, N=512, d=16, Cq=4, Ck=16, seed=0):
    q, k, v, _ = make_qkv(H, N, d, n_centers=6, dtype="f32", seed=seed)
    q, k, v = q.numpy(), k.numpy(), v.numpy()
    cq = orc.cluster(q, Cq, 5)
    ck = orc.cluster(k, Ck, 5, companion=v)
    scale = float(np.float32(1 / math.sqrt(d)))
    S, pi = orc.probs(cq["centroids"], ck["centroids"], ck["offsets"], scale)
    return q, k, v, cq, ck, S, scale


def test_attention_on_lists_matches_sdpa(orc):
    """Attention over an exact set + sample with duplicates and offsets equals torch
    SDPA (fp64) over the gathered columns with the offsets as an additive mask."""
    q, k, v, cq, ck, S, scale = _clustered(orc)
    N = q.shape[2]
    sel = orc.select_sample(S, ck["offsets"], N, 100, 37, seed=3)
    o_p, lse_p = orc.attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                               ck["offsets"], sel, 37, scale)
    ko = ck["offsets"][0, 0]
    for i in range(4):
        eg = sel["exact_groups"][0, 0, i, :sel["n_exact"][0, 0, i]]
        cols = [r for j in eg for r in range(ko[j], ko[j + 1])]
        ns = sel["n_sample"][0, 0, i]
        cols += sel["sample_idx"][0, 0, i, :ns].tolist()
        bias = np.concatenate([np.zeros(len(cols) - ns), sel["sample_bias"][0, 0, i, :ns]])
        rows = slice(cq["offsets"][0, 0, i], cq["offsets"][0, 0, i + 1])
        o_ref, lse_ref = _sdpa_ref(cq["x_perm"][0, 0, rows], ck["x_perm"][0, 0, cols],
                                   ck["companion_perm"][0, 0, cols], bias, scale)
        assert np.allclose(o_p[0, 0, rows], o_ref, rtol=0, atol=1e-12)
        assert np.allclose(lse_p[0, 0, rows], lse_ref, rtol=0, atol=1e-12)
        assert len(set(sel["sample_idx"][0, 0, i, :ns].tolist())) < ns   # duplicates exercised


def test_dense_matches_sdpa(orc):
    q, k, v, _ = make_qkv(2, 300, 32, n_centers=5, dtype="f32", seed=1)
    q, k, v = q.numpy(), k.numpy(), v.numpy()
    scale = float(np.float32(0.17))   # the oracle takes the fp32 scale
    o, lse = orc.dense(q, k, v, scale)
    for h in range(2):
        o_ref, lse_ref = _sdpa_ref(q[0, h], k[0, h], v[0, h], np.zeros(300), scale)
        assert np.allclose(o[0, h], o_ref, atol=1e-12) and np.allclose(lse[0, h], lse_ref, atol=1e-12)
    rows = np.array([0, 17, 299], np.int32)
    o2, lse2 = orc.dense(q, k, v, scale, rows=rows)
    assert np.allclose(o2, o[:, :, rows], atol=0) and np.allclose(lse2, lse[:, :, rows], atol=0)


def _full(orc, q, k, v, cq, ck, S, scale, E, m, seed=0, mode=0):
    N = q.shape[2]
    sel = orc.select_sample(S, ck["offsets"], N, E, m, mode=mode, seed=seed)
    o_p, lse_p = orc.attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                               ck["offsets"], sel, m, scale)
    o, lse = orc.unpermute(o_p, lse_p, cq["perm"])
    return sel, o, lse


def test_all_selected_equals_dense(orc):
    """Selecting every block (E = 100 %) is dense softmax attention (to 1e-5 in the
    pages' fp32 terms; the fp64 oracle meets it to round-off)."""
    q, k, v, cq, ck, S, scale = _clustered(orc)
    N = q.shape[2]
    sel, o, lse = _full(orc, q, k, v, cq, ck, S, scale, E=N, m=16)
    assert np.all(sel["n_sample"] == 0)
    o_ref, lse_ref = _sdpa_ref(q[0, 0], k[0, 0], v[0, 0], np.zeros(N), scale)
    assert np.abs(o[0, 0] - o_ref).max() < 1e-12
    assert np.abs(lse[0, 0] - lse_ref).max() < 1e-12


def test_every_skipped_token_weight_one_is_exact(orc):
    """Top group exact + a budget m >= M that enumerates the skipped keys once with
    offset 0 reproduces dense attention."""
    q, k, v, cq, ck, S, scale = _clustered(orc)
    N = q.shape[2]
    sel, o, lse = _full(orc, q, k, v, cq, ck, S, scale, E=0, m=N)
    assert np.all(sel["n_exact"] == 1)
    assert np.all(sel["n_sample"] + np.array([
        np.diff(ck["offsets"][0, 0])[sel["exact_groups"][0, 0, i, 0]] for i in range(4)]) == N)
    o_ref, lse_ref = _sdpa_ref(q[0, 0], k[0, 0], v[0, 0], np.zeros(N), scale)
    assert np.abs(o[0, 0] - o_ref).max() < 1e-12
    assert np.abs(lse[0, 0] - lse_ref).max() < 1e-12


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


def _unbiased_stats(orc, bias_tamper=None, seeds=1000, mode=0):
    q, k, v, cq, ck, S, scale = _clustered(orc, N=256, d=16, Cq=4, Ck=16, seed=2)
    q = q * 0.5   # softer attention so the skipped region carries real mass
    cq = orc.cluster(q, 4, 5)
    S, _ = orc.probs(cq["centroids"], ck["centroids"], ck["offsets"], scale)
    N = q.shape[2]
    o_ref, lse_ref = _sdpa_ref(q[0, 0], k[0, 0], v[0, 0], np.zeros(N), scale)
    E, m = 32, 24
    Dh, Nh = [], []
    for s in range(seeds):
        sel = orc.select_sample(S, ck["offsets"], N, E, m, mode=mode, seed=s)
        if bias_tamper is not None:
            bias_tamper(sel, ck["offsets"])
        o_p, lse_p = orc.attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                                   ck["offsets"], sel, m, scale)
        o, lse = orc.unpermute(o_p, lse_p, cq["perm"])
        d_rel = np.exp(lse[0, 0] - lse_ref)
        Dh.append(d_rel)
        Nh.append(o[0, 0] * d_rel[:, None])
    Dh, Nh = np.array(Dh), np.array(Nh)

    def z(x, target):
        mu = x.mean(0)
        se = x.std(0, ddof=1) / math.sqrt(x.shape[0])
        return (mu - target) / np.maximum(se, 1e-300)

    return (z(Dh, 1.0).ravel(), seed_summary_z(Dh, 1.0)), (z(Nh, o_ref).ravel(), seed_summary_z(Nh, o_ref))


@pytest.mark.parametrize("mode", [0, 1])
def test_unbiased_over_1000_seeds(orc, mode):
    """The mean over 1,000 seeds of the denominator (e^LSE) and numerator (O e^LSE)
    estimates converges to the dense ones: per-element z-scores, fraction |z| > 4 at
    most 0.1 %, and the seed-level summary's z within 4."""
    for zz, zs in _unbiased_stats(orc, mode=mode):
        print(f"mode {mode}: max |z| {np.abs(zz).max():.2f}, summary z {zs:.2f}")
        assert np.mean(np.abs(zz) > 4) <= 1e-3
        assert abs(zs) < 4


def test_unbiased_negative_control(orc):
    """Planted mistake (offset from the group probability, without the 1/n_g of the
    key within the group): the same statistic must flag it."""
    def tamper(sel, ko):
        off = ko[0, 0]
        n = np.diff(off)
        for i in range(sel["sample_idx"].shape[2]):
            ns = sel["n_sample"][0, 0, i]
            rows = sel["sample_idx"][0, 0, i, :ns]
            g = np.searchsorted(off, rows, side="right") - 1
            sel["sample_bias"][0, 0, i, :ns] -= np.log(n[g]).astype(np.float32)
    (zd, zsd), (zn, zsn) = _unbiased_stats(orc, bias_tamper=tamper, seeds=200)
    assert np.mean(np.abs(zd) > 4) > 0.5
    assert abs(zsd) > 10


def test_unpermute_inverts_perm(orc):
    rng = np.random.default_rng(0)
    perm = np.stack([rng.permutation(50) for _ in range(3)]).astype(np.int32)[None]
    o_p = rng.standard_normal((1, 3, 50, 4))
    lse_p = rng.standard_normal((1, 3, 50))
    o, lse = orc.unpermute(o_p, lse_p, perm)
    for h in range(3):
        assert np.array_equal(o[0, h][perm[0, h]], o_p[0, h])
        assert np.array_equal(lse[0, h][perm[0, h]], lse_p[0, h])


def test_error_falls_with_sample_size(orc):
    """Reconstruction error of the sampled estimate falls as the sample grows
    (trend check over 32 seeds per budget)."""
    q, k, v, cq, ck, S, scale = _clustered(orc, N=512, d=16, Cq=4, Ck=16, seed=4)
    N = q.shape[2]
    o_ref, _ = _sdpa_ref(q[0, 0], k[0, 0], v[0, 0], np.zeros(N), scale)
    errs = []
    for m in (8, 32, 128):
        e = []
        for s in range(32):
            _, o, _ = _full(orc, q, k, v, cq, ck, S, scale, E=32, m=m, seed=s)
            e.append(np.linalg.norm(o[0, 0] - o_ref) / np.linalg.norm(o_ref))
        errs.append(np.mean(e))
    assert errs[0] > errs[1] > errs[2]


# ---------------------------------------------------------------- product-quantised voting
def _pq_case(orc, exact_pq=False, same_query=False, seed=0):
    """Tiny head: Cq query groups, Ck key groups, P subspaces of ds dims."""
    rng = np.random.default_rng(seed)
    H, N, P, ds, Cc, Cq, Ck = 1, 240, 4, 4, 16, 4, 12
    d = P * ds
    if exact_pq:
        # every sub-vector is one of Cc distinct codewords, so 16-means recovers them
        words = rng.standard_normal((P, Cc, ds)) * 3
        qi = rng.integers(0, Cc, (N, P))
        ki = rng.integers(0, Cc, (N, P))
        q = np.concatenate([words[s][qi[:, s]] for s in range(P)], 1)
        k = np.concatenate([words[s][ki[:, s]] for s in range(P)], 1)
    else:
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d))
    q = q.astype(np.float32)[None, None]
    k = k.astype(np.float32)[None, None]
    cq = orc.cluster(q, Cq, 5)
    if same_query:
        # every query of a group equals its group's centroid (then re-quantised exactly)
        q = cq["centroids"][0, 0][cq["labels"][0, 0]][None, None].astype(np.float32)
    ck = orc.cluster(k, Ck, 5)
    return q, k, cq, ck, P, Cc


def test_pq_exact_quantisation_reproduces_centroid_ranking(orc):
    """When every query of a group equals the group's centroid and the quantisation
    is exact, each query's per-group scores are the centroid scores, so every query of
    group i votes for exactly the exact set that the centroid ranking selects."""
    rng = np.random.default_rng(3)
    H, N, P, ds, Cq, Ck = 1, 240, 4, 4, 4, 12
    d = P * ds
    k = (rng.standard_normal((N, d)) * 2).astype(np.float32)[None, None]
    ck = orc.cluster(k, Ck, 5)
    # queries: Cq distinct vectors, each repeated; quantisation of both is exact when the
    # number of distinct sub-vectors is <= Cc
    qv = (rng.standard_normal((Cq, d)) * 2).astype(np.float32)
    lab = np.repeat(np.arange(Cq), N // Cq)
    q = qv[lab][None, None]
    cq = orc.cluster(q, Cq, 5)
    Cc = 256
    # keys: at most N distinct sub-vectors per subspace (<= Cc) -> exact codebooks
    qc, qcb = orc.pq_codebooks(q, P, Cc, 5)
    kc, kcb = orc.pq_codebooks(k, P, Cc, 5)
    for s in range(P):
        assert np.array_equal(qcb[s, 0, 0][qc[s, 0, 0]], q[0, 0][:, s * ds:(s + 1) * ds])
        assert np.array_equal(kcb[s, 0, 0][kc[s, 0, 0]], k[0, 0][:, s * ds:(s + 1) * ds])
    scale = 0.25
    kbar = orc.pq_kbar(kc, kcb, ck["perm"], ck["offsets"])
    cent = ck["centroids"][0, 0]
    assert np.allclose(kbar[0, 0], cent, atol=1e-5)
    tables = orc.pq_tables(qcb, kbar, scale)
    E = 60
    votes = orc.pq_votes(qc, tables, cq["perm"], cq["offsets"], ck["offsets"], E)
    S, _ = orc.probs(cq["centroids"], ck["centroids"], ck["offsets"], scale)
    sel = orc.select_sample(S, ck["offsets"], N, E, 0)
    n_q = np.diff(cq["offsets"][0, 0])
    for i in range(Cq):
        ex = set(sel["exact_groups"][0, 0, i, :sel["n_exact"][0, 0, i]].tolist())
        got = {j for j in range(Ck) if votes[0, 0, i, j] > 0}
        assert got == ex
        assert all(votes[0, 0, i, j] == n_q[i] for j in got)
    # votes mode then reproduces the exact set
    selv = orc.select_sample(S, ck["offsets"], N, E, 0, mode=2, votes=votes)
    assert np.array_equal(selv["exact_groups"], sel["exact_groups"])


def _pq_reference(q, k, cq, ck, P, kc, kcb, qc, qcb, scale):
    """Direct fp64 numpy evaluation of the PQ reading: reconstructed keys and queries
    (codewords per subspace), key-group means in fp64, per-query group scores."""
    ko = ck["offsets"][0, 0]
    n_k = np.diff(ko)
    krec = np.concatenate([kcb[s, 0, 0][kc[s, 0, 0]] for s in range(P)], 1).astype(np.float64)
    qrec = np.concatenate([qcb[s, 0, 0][qc[s, 0, 0]] for s in range(P)], 1).astype(np.float64)
    kperm = krec[ck["perm"][0, 0]]
    gmean = np.stack([kperm[ko[j]:ko[j + 1]].mean(0) if n_k[j] else np.zeros(q.shape[-1]) for j in range(len(n_k))])
    return n_k, qrec, gmean, scale * (qrec @ gmean.T)


def _walk(sc, n_k, E, stop_at_equal=False):
    """The exact-set rule on one query's ranking (score desc, group asc): the groups
    taken, and the smallest score gap between neighbours among the ranked groups the
    walk looked at (the taken ones, the one that stopped it, and the next one)."""
    order = sorted([j for j in range(len(n_k)) if n_k[j]], key=lambda j: (-sc[j], j))
    taken, cum = [], 0
    for p_, j in enumerate(order):
        over = cum + n_k[j] >= E if stop_at_equal else cum + n_k[j] > E
        if p_ > 0 and over:
            break
        cum += n_k[j]
        taken.append(j)
    look = order[:min(len(order), len(taken) + 2)]
    gaps = [abs(sc[look[p]] - sc[look[p + 1]]) for p in range(len(look) - 1)]
    return taken, (min(gaps) if gaps else np.inf)


@pytest.mark.parametrize("seed,scale", [(4, 0.5), (8, 0.3), (13, 1.0)])
def test_pq_votes_brute_force(orc, seed, scale):
    """Votes against a direct fp64 numpy evaluation of the same reading on a tiny head.
    Every query whose ranking has no two groups within 1e-5 up to where the budget walk
    stops must vote exactly as the direct evaluation (the table path sums in fp32 in
    another order, which can only swap groups closer than that); the remaining
    near-tie queries are counted and bound the difference.  The budget sits exactly
    at a cumulative group size of one query, so a >= for > slip in the rule changes
    the votes (negative control on the reference)."""
    q, k, cq, ck, P, Cc = _pq_case(orc, seed=seed)
    qc, qcb = orc.pq_codebooks(q, P, Cc, 5)
    kc, kcb = orc.pq_codebooks(k, P, Cc, 5)
    kbar = orc.pq_kbar(kc, kcb, ck["perm"], ck["offsets"])
    tables = orc.pq_tables(qcb, kbar, scale)
    n_k, qrec, gmean, sc = _pq_reference(q, k, cq, ck, P, kc, kcb, qc, qcb, scale)
    qo = cq["offsets"][0, 0]
    t0 = cq["perm"][0, 0, 0]
    order0 = sorted([j for j in range(len(n_k)) if n_k[j]], key=lambda j: (-sc[t0, j], j))
    E = int(n_k[order0[0]] + n_k[order0[1]] + n_k[order0[2]])
    votes = orc.pq_votes(qc, tables, cq["perm"], cq["offsets"], ck["offsets"], E)[0, 0]
    Cq_, Ck_ = votes.shape
    want = np.zeros((Cq_, Ck_), np.int64)
    slip = np.zeros((Cq_, Ck_), np.int64)
    near = np.zeros(Cq_, np.int64)
    for i in range(Cq_):
        for r in range(qo[i], qo[i + 1]):
            t = cq["perm"][0, 0, r]
            taken, gap = _walk(sc[t], n_k, E)
            for j in _walk(sc[t], n_k, E, stop_at_equal=True)[0]:
                slip[i, j] += 1
            if gap > 1e-5:
                for j in taken:
                    want[i, j] += 1
            else:
                near[i] += 1
    print(f"PQ votes seed {seed}: {int(near.sum())} of {int(qo[-1])} queries have a near-tie in their ranking")
    resid = votes.astype(np.int64) - want
    for i in range(Cq_):
        if near[i] == 0:
            assert np.array_equal(resid[i], np.zeros(Ck_)), i
        else:
            assert (resid[i] >= 0).all() and (resid[i] <= near[i]).all(), i
    assert near.sum() <= 0.05 * qo[-1]
    assert np.all(votes.sum(1) >= np.diff(qo))
    assert not np.array_equal(slip, votes)


def test_pq_kbar_and_tables_against_numpy(orc):
    """Kbar = fp64 mean of each key group's reconstructed sub-vectors (0 for an empty
    group) and M_s[a][j] = scale <cw^q_{s,a}, Kbar_{j,s}>, both against direct numpy fp64
    within 1e-6 relative (the oracle rounds to fp32; its tables are an fp32 fma chain)."""
    q, k, cq, ck, P, Cc = _pq_case(orc, seed=6)
    qc, qcb = orc.pq_codebooks(q, P, Cc, 5)
    kc, kcb = orc.pq_codebooks(k, P, Cc, 5)
    ko = ck["offsets"].copy()
    ko[0, 0, 4] = ko[0, 0, 3]  # group 3 empty (its rows join group 4)
    kbar = orc.pq_kbar(kc, kcb, ck["perm"], ko)
    ck2 = dict(ck, offsets=ko)
    scale = 0.37
    n_k, _, gmean, _ = _pq_reference(q, k, cq, ck2, P, kc, kcb, qc, qcb, scale)
    assert n_k[3] == 0 and np.all(kbar[0, 0, 3] == 0)
    big = np.abs(gmean).max()
    assert np.allclose(kbar[0, 0], gmean, rtol=1e-6, atol=1e-6 * big)
    tables = orc.pq_tables(qcb, kbar, scale)
    ds = q.shape[-1] // P
    kb = kbar[0, 0].astype(np.float64).reshape(len(n_k), P, ds)
    want = scale * np.einsum("sae,jse->saj", qcb[:, 0, 0].astype(np.float64), kb)
    assert tables.shape[-3:] == want.shape
    assert np.allclose(tables[0, 0], want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
    # a dropped subspace term or a transposed operand would be far off
    assert not np.allclose(tables[0, 0][1:], want[:-1], rtol=1e-3)


# ---------------------------------------------------------------- top-p exact-set sizing
def test_topp_exact_set_brute_force(orc):
    """Top-p rule against a direct Python evaluation: groups by (pi desc, j asc), taken
    until the fp64 running sum of pi reaches p; the taken mass reaches p and dropping the
    last taken group falls short of it (minimality); the first group is always taken."""
    rng = np.random.default_rng(11)
    B, H, Cq, Ck, N = 1, 2, 3, 40, 2000
    q = rng.standard_normal((B, H, Cq, 16)).astype(np.float32)
    k = rng.standard_normal((B, H, Ck, 16)).astype(np.float32)
    sizes = rng.multinomial(N, rng.dirichlet(np.ones(Ck) * 0.5), size=(B, H))
    sizes[0, 0, 5] = 0  # an empty group
    ko = np.concatenate([np.zeros((B, H, 1), np.int64), np.cumsum(sizes, -1)], -1).astype(np.int32)
    S, pi = orc.probs(q, k, ko, 0.7)
    for p in (1e-6, 0.3, 0.8, 0.95, 0.999, 1.0, 2.0):
        sel = orc.select_sample_topp(S, pi, ko, N, p, 0)
        for h in range(H):
            for i in range(Cq):
                P = pi[0, h, i].astype(np.float64)
                ne = [j for j in range(Ck) if sizes[0, h, j] > 0]
                order = sorted(ne, key=lambda j: (-float(pi[0, h, i, j]), j))
                want, mass = [], 0.0
                for j in order:
                    want.append(j)
                    mass += float(pi[0, h, i, j])
                    if mass >= p:
                        break
                got = sel["exact_groups"][0, h, i, :sel["n_exact"][0, h, i]].tolist()
                assert got == sorted(want), (p, h, i)
                assert order[0] in got
                tm = sum(P[j] for j in got)
                assert tm >= min(p, sum(P[j] for j in ne)) - 1e-12
                if len(got) > 1:
                    assert tm - P[want[-1]] < p


def test_topp_one_reaches_dense_and_sample_covers_rest(orc):
    """p = 1 (up to fp32 rounding of pi) keeps essentially every group; the sample then
    draws only from groups outside the exact set, as in the budget rule."""
    rng = np.random.default_rng(12)
    N, d, Cq, Ck = 512, 16, 4, 12
    x = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    cq = orc.cluster(x, Cq, 3)
    ck = orc.cluster(x, Ck, 3)
    S, pi = orc.probs(cq["centroids"], ck["centroids"], ck["offsets"], 0.25)
    sel = orc.select_sample_topp(S, pi, ck["offsets"], N, 0.5, 300, seed=3)
    ko = ck["offsets"][0, 0]
    for i in range(Cq):
        ex = set(sel["exact_groups"][0, 0, i, :sel["n_exact"][0, 0, i]].tolist())
        grp = np.searchsorted(ko, sel["sample_idx"][0, 0, i, :sel["n_sample"][0, 0, i]], side="right") - 1
        assert not (set(grp.tolist()) & ex)
    full = orc.select_sample_topp(S, pi, ck["offsets"], N, 2.0, 0)
    nonempty = int((np.diff(ko) > 0).sum())
    assert (full["n_exact"] == nonempty).all()
