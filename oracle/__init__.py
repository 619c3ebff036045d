"""ctypes wrapper of the CPU oracle (oracle/isg_oracle.c).

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  Inputs are numpy
arrays (bf16 values are passed as their exact fp32 values); outputs are fp64
where the oracle computes in fp64.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import LIB, build

_lib = None


def lib():
    """The compiled oracle; ISG_ORACLE_LIB names another build of the same source
    (the sanitizer test's)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ISG_ORACLE_LIB") or LIB
        if path == LIB and not os.path.exists(LIB):
            build()
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


_p = C.c_void_p
_i = C.c_int
_i64 = C.c_int64
_u64 = C.c_uint64
_f = C.c_float


def _declare(L):
    L.orc_num_threads.restype = _i
    L.orc_philox4x64_10.argtypes = [_p, _p, _p]
    L.orc_proposal_table.argtypes = [_p]
    L.orc_kmeans_assign.argtypes = [_p, _i64, _i, _i64, _p, _i, _p, _p]
    L.orc_sqdist.argtypes = [_p, _p, _i]
    L.orc_sqdist.restype = C.c_double
    L.orc_kmeans_update.argtypes = [_p, _i64, _i, _i64, _p, _i, _p, _p, _p]
    L.orc_stable_sort.argtypes = [_p, _i64, _i, _p, _p]
    L.orc_cluster.argtypes = [_p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]
    L.orc_probs.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p]
    L.orc_select_sample.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _u64, _u64,
                                    _p, _p, _p, _p, _p]
    L.orc_select_sample_topp.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _u64, _u64,
                                         _p, _p, _p, _p, _p]
    L.orc_attention.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p,
                                _i, _f, _p, _p, _p]
    L.orc_dense.argtypes = [_p, _p, _p, _i, _i, _i, _i, _f, _p, _i, _p, _p]
    L.orc_unpermute.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p, _p]
    L.orc_pq_kbar.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p]
    L.orc_pq_tables.argtypes = [_p, _p, _i, _i, _i, _i, _i, _i, _f, _p]
    L.orc_pq_votes.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p]


def _c(a, dtype):
    """Contiguous array of the given dtype (no copy when already so)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return lib().orc_num_threads()


def philox4x64_10(counter, key):
    ctr = _c(counter, np.uint64)
    k = _c(key, np.uint64)
    out = np.zeros(4, np.uint64)
    lib().orc_philox4x64_10(_ptr(ctr), _ptr(k), _ptr(out))
    return out


def proposal_table():
    t = np.zeros(256, np.uint32)
    lib().orc_proposal_table(_ptr(t))
    return t


def kmeans_assign(x, cent, with_dist=False):
    x = _c(x, np.float32)
    cent = _c(cent, np.float32)
    n, d = x.shape
    lab = np.zeros(n, np.int32)
    bd = np.zeros(n, np.float64) if with_dist else None
    lib().orc_kmeans_assign(_ptr(x), n, d, d, _ptr(cent), cent.shape[0], _ptr(lab), _ptr(bd))
    return (lab, bd) if with_dist else lab


def sqdist(xrow, crow):
    xrow = _c(xrow, np.float32)
    crow = _c(crow, np.float32)
    return lib().orc_sqdist(_ptr(xrow), _ptr(crow), xrow.shape[0])


def kmeans_update(x, labels, cent_prev):
    x = _c(x, np.float32)
    labels = _c(labels, np.int32)
    cent_prev = _c(cent_prev, np.float32)
    n, d = x.shape
    C_ = cent_prev.shape[0]
    out = np.zeros_like(cent_prev)
    cnt = np.zeros(C_, np.int32)
    lib().orc_kmeans_update(_ptr(x), n, d, d, _ptr(labels), C_, _ptr(cent_prev), _ptr(out), _ptr(cnt))
    return out, cnt


def stable_sort(labels, C_):
    labels = _c(labels, np.int32)
    perm = np.zeros(labels.shape[0], np.int32)
    off = np.zeros(C_ + 1, np.int32)
    lib().orc_stable_sort(_ptr(labels), labels.shape[0], C_, _ptr(perm), _ptr(off))
    return perm, off


def cluster(x, C_, iters, init=None, companion=None, want_perm=True):
    """x: [B,H,N,d].  Returns dict(centroids, labels, perm, offsets, x_perm, companion_perm)."""
    x = _c(x, np.float32)
    B, H, N, d = x.shape
    cent = np.zeros((B, H, C_, d), np.float32) if init is None else _c(init, np.float32).copy()
    lab = np.zeros((B, H, N), np.int32)
    perm = np.zeros((B, H, N), np.int32)
    off = np.zeros((B, H, C_ + 1), np.int32)
    xp = np.zeros_like(x) if want_perm else None
    comp = None if companion is None else _c(companion, np.float32)
    cp = None if comp is None else np.zeros_like(comp)
    lib().orc_cluster(_ptr(x), B, H, N, d, C_, iters, 0 if init is None else 1, _ptr(comp),
                      _ptr(cent), _ptr(lab), _ptr(perm), _ptr(off), _ptr(xp), _ptr(cp))
    return dict(centroids=cent, labels=lab, perm=perm, offsets=off, x_perm=xp, companion_perm=cp)


def probs(cq, ck, k_offsets, scale):
    cq = _c(cq, np.float32)
    ck = _c(ck, np.float32)
    ko = _c(k_offsets, np.int32)
    B, H, Cq, d = cq.shape
    Ck = ck.shape[2]
    S = np.zeros((B, H, Cq, Ck), np.float32)
    pi = np.zeros((B, H, Cq, Ck), np.float64)
    lib().orc_probs(_ptr(cq), _ptr(ck), _ptr(ko), B, H, Cq, Ck, d, float(scale), _ptr(S), _ptr(pi))
    return S, pi


def select_sample(scores, k_offsets, N, exact_keys, m, mode=0, seed=0, call_id=0, votes=None):
    S = _c(scores, np.float32)
    ko = _c(k_offsets, np.int32)
    B, H, Cq, Ck = S.shape
    vt = None if votes is None else _c(votes, np.int32)
    eg = np.zeros((B, H, Cq, Ck), np.int32)
    ne = np.zeros((B, H, Cq), np.int32)
    mm = max(m, 1)
    si = np.zeros((B, H, Cq, mm), np.int32)
    sb = np.zeros((B, H, Cq, mm), np.float32)
    ns = np.zeros((B, H, Cq), np.int32)
    lib().orc_select_sample(_ptr(S), _ptr(ko), _ptr(vt), B, H, Cq, Ck, N, int(exact_keys), int(m),
                            int(mode), seed, call_id, _ptr(eg), _ptr(ne), _ptr(si), _ptr(sb), _ptr(ns))
    return dict(exact_groups=eg, n_exact=ne, sample_idx=si, sample_bias=sb, n_sample=ns)


def select_sample_topp(scores, pi, k_offsets, N, top_p, m, mode=0, seed=0, call_id=0):
    """Exact set by the top-p rule (groups by pi desc until the running pi reaches top_p), then the sample."""
    S = _c(scores, np.float32)
    P = _c(pi, np.float32)
    ko = _c(k_offsets, np.int32)
    B, H, Cq, Ck = S.shape
    eg = np.zeros((B, H, Cq, Ck), np.int32)
    ne = np.zeros((B, H, Cq), np.int32)
    mm = max(m, 1)
    si = np.zeros((B, H, Cq, mm), np.int32)
    sb = np.zeros((B, H, Cq, mm), np.float32)
    ns = np.zeros((B, H, Cq), np.int32)
    lib().orc_select_sample_topp(_ptr(S), _ptr(P), _ptr(ko), B, H, Cq, Ck, N, float(top_p), int(m), int(mode),
                                 seed, call_id, _ptr(eg), _ptr(ne), _ptr(si), _ptr(sb), _ptr(ns))
    return dict(exact_groups=eg, n_exact=ne, sample_idx=si, sample_bias=sb, n_sample=ns)


def attention(q_p, k_p, v_p, q_offsets, k_offsets, sel, m, scale, group_mask=None):
    q_p = _c(q_p, np.float32)
    k_p = _c(k_p, np.float32)
    v_p = _c(v_p, np.float32)
    B, H, N, d = q_p.shape
    qo = _c(q_offsets, np.int32)
    ko = _c(k_offsets, np.int32)
    Cq = qo.shape[-1] - 1
    Ck = ko.shape[-1] - 1
    eg = _c(sel["exact_groups"], np.int32)
    ne = _c(sel["n_exact"], np.int32)
    si = _c(sel["sample_idx"], np.int32)
    sb = _c(sel["sample_bias"], np.float32)
    ns = _c(sel["n_sample"], np.int32)
    mm = si.shape[-1]
    gm = None if group_mask is None else _c(group_mask, np.uint8)
    o = np.zeros((B, H, N, d), np.float64)
    lse = np.zeros((B, H, N), np.float64)
    lib().orc_attention(_ptr(q_p), _ptr(k_p), _ptr(v_p), B, H, N, d, Cq, Ck, _ptr(qo), _ptr(ko),
                        _ptr(eg), _ptr(ne), _ptr(si), _ptr(sb), _ptr(ns), mm, float(scale),
                        _ptr(gm), _ptr(o), _ptr(lse))
    return o, lse


def dense(q, k, v, scale, rows=None):
    q = _c(q, np.float32)
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    B, H, N, d = q.shape
    rr = None if rows is None else _c(rows, np.int32)
    R = N if rr is None else rr.shape[0]
    o = np.zeros((B, H, R, d), np.float64)
    lse = np.zeros((B, H, R), np.float64)
    lib().orc_dense(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), _ptr(rr), R, _ptr(o), _ptr(lse))
    return o, lse


def unpermute(o_p, lse_p, perm_q):
    o_p = _c(o_p, np.float64)
    lse_p = _c(lse_p, np.float64)
    pq = _c(perm_q, np.int32)
    B, H, N, d = o_p.shape
    o = np.zeros_like(o_p)
    lse = np.zeros_like(lse_p)
    lib().orc_unpermute(_ptr(o_p), _ptr(lse_p), _ptr(pq), B, H, N, d, _ptr(o), _ptr(lse))
    return o, lse


def pipeline(q, k, v, Cq, Ck, iters, exact_keys, m, mode=0, seed=0, call_id=0, scale=None):
    """All steps in order on [B,H,N,d] inputs; returns every intermediate."""
    d = q.shape[-1]
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    cq = cluster(q, Cq, iters)
    ck = cluster(k, Ck, iters, companion=v)
    S, pi = probs(cq["centroids"], ck["centroids"], ck["offsets"], scale)
    sel = select_sample(S, ck["offsets"], q.shape[2], exact_keys, m, mode, seed, call_id)
    o_p, lse_p = attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"],
                           ck["offsets"], sel, m, scale)
    o, lse = unpermute(o_p, lse_p, cq["perm"])
    return dict(cq=cq, ck=ck, scores=S, pi=pi, sel=sel, o_p=o_p, lse_p=lse_p, o=o, lse=lse,
                scale=scale)


# ---------------------------------------------------------------- product-quantised voting
def pq_codebooks(x, P, Cc, iters):
    """Codes [P,B,H,N] and codebooks [P,B,H,Cc,d/P] from k-means of each subspace."""
    x = _c(x, np.float32)
    B, H, N, d = x.shape
    ds = d // P
    codes = np.zeros((P, B, H, N), np.int32)
    cbs = np.zeros((P, B, H, Cc, ds), np.float32)
    for s in range(P):
        r = cluster(np.ascontiguousarray(x[..., s * ds:(s + 1) * ds]), Cc, iters, want_perm=False)
        codes[s] = r["labels"]
        cbs[s] = r["centroids"]
    return codes, cbs


def pq_kbar(k_codes, k_cb, perm_k, k_offsets):
    k_codes = _c(k_codes, np.int32)
    k_cb = _c(k_cb, np.float32)
    pk = _c(perm_k, np.int32)
    ko = _c(k_offsets, np.int32)
    P, B, H, N = k_codes.shape
    Cc, ds = k_cb.shape[-2:]
    Ck = ko.shape[-1] - 1
    kbar = np.zeros((B, H, Ck, P * ds), np.float32)
    lib().orc_pq_kbar(_ptr(k_codes), _ptr(k_cb), _ptr(pk), _ptr(ko), B, H, N, P, Cc, ds, Ck, _ptr(kbar))
    return kbar


def pq_tables(q_cb, kbar, scale):
    q_cb = _c(q_cb, np.float32)
    kbar = _c(kbar, np.float32)
    P, B, H, Cc, ds = q_cb.shape
    Ck = kbar.shape[2]
    t = np.zeros((B, H, P, Cc, Ck), np.float32)
    lib().orc_pq_tables(_ptr(q_cb), _ptr(kbar), B, H, P, Cc, ds, Ck, float(scale), _ptr(t))
    return t


def pq_votes(q_codes, tables, perm_q, q_offsets, k_offsets, exact_keys):
    q_codes = _c(q_codes, np.int32)
    tables = _c(tables, np.float32)
    pq_ = _c(perm_q, np.int32)
    qo = _c(q_offsets, np.int32)
    ko = _c(k_offsets, np.int32)
    P, B, H, N = q_codes.shape
    Cc = tables.shape[3]
    Cq, Ck = qo.shape[-1] - 1, ko.shape[-1] - 1
    v = np.zeros((B, H, Cq, Ck), np.int32)
    lib().orc_pq_votes(_ptr(q_codes), _ptr(tables), _ptr(pq_), _ptr(qo), _ptr(ko), B, H, N, P, Cc, Cq, Ck,
                       int(exact_keys), _ptr(v))
    return v
