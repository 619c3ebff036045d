"""Thin Python binding of libisg (include/isg.h): argument marshalling only.

Every step runs in the HIP library; torch provides device memory and the
stream.  There is no CPU path: without the built library, or with tensors that
are not on a GPU, every call raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

# ISG_LIBRARY names another build of the same sources (the host-sanitizer build)
LIB_PATH = os.environ.get("ISG_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libisg.so")

ISG_F32, ISG_BF16 = 0, 1
MODES = {"importance": 0, "uniform": 1, "votes": 2}
EXPORTS = ["isg_last_error", "isg_version", "isg_proposal_table", "isg_cluster_workspace_size",
           "isg_cluster", "isg_probs", "isg_select_sample", "isg_attention_workspace_size",
           "isg_attention", "isg_unpermute", "isg_pq_votes", "isg_select_sample_topp", "isg_cluster_noalloc",
           "isg_pq_codebooks_workspace_size", "isg_pq_codebooks"]

_lib = None


class IsgError(RuntimeError):
    pass


def lib():
    """Load the in-tree libisg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise IsgError(f"libisg.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


_p, _i, _u64, _f, _sz = C.c_void_p, C.c_int, C.c_uint64, C.c_float, C.c_size_t


def _declare(L):
    L.isg_last_error.restype = C.c_char_p
    L.isg_version.restype = _i
    L.isg_proposal_table.argtypes = [_p]
    L.isg_cluster_workspace_size.argtypes = [_i] * 5
    L.isg_cluster_workspace_size.restype = _sz
    L.isg_cluster.argtypes = [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                              _sz]
    L.isg_cluster_noalloc.argtypes = [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]
    L.isg_probs.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p]
    L.isg_select_sample.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _u64, _u64,
                                    _p, _p, _p, _p, _p]
    L.isg_attention_workspace_size.argtypes = [_i] * 6
    L.isg_attention_workspace_size.restype = _sz
    L.isg_attention.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p,
                                _i, _f, _p, _p, _p, _p, _p, _p, _sz]
    L.isg_unpermute.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p]
    L.isg_select_sample_topp.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _u64, _u64,
                                         _p, _p, _p, _p, _p]
    L.isg_pq_votes.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f,
                               _p, _p, _p]
    L.isg_pq_codebooks_workspace_size.argtypes = [_i] * 7
    L.isg_pq_codebooks_workspace_size.restype = _sz
    L.isg_pq_codebooks.argtypes = [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _sz]
    for name in ["isg_cluster", "isg_probs", "isg_select_sample", "isg_attention", "isg_unpermute",
                 "isg_pq_votes", "isg_select_sample_topp", "isg_cluster_noalloc", "isg_pq_codebooks"]:
        getattr(L, name).restype = _i


def _check(status, what):
    if status != 0:
        msg = lib().isg_last_error().decode(errors="replace")
        raise IsgError(f"{what} failed with status {status}: {msg}")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise IsgError(f"{name} must be a GPU tensor")
    return t


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return ISG_BF16
    if t.dtype == torch.float32:
        return ISG_F32
    raise IsgError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _i64x3(vals):
    return (C.c_int64 * 3)(*[int(v) for v in vals])


def version() -> int:
    return lib().isg_version()


def proposal_table():
    out = (C.c_uint32 * 256)()
    lib().isg_proposal_table(out)
    return list(out)


def cluster_workspace_size(B, H, N, d, C_):
    return int(lib().isg_cluster_workspace_size(B, H, N, d, C_))


def attention_workspace_size(B, H, N, Cq, Ck, m):
    return int(lib().isg_attention_workspace_size(B, H, N, Cq, Ck, m))


NOALLOC_SCRATCH_BYTES = 64 << 20  # ISG_CLUSTER_NOALLOC_SCRATCH_BYTES


def cluster_outputs(x, C_, *, companion=None, want_perm=True, want_max_sqnorm=False):
    """Output tensors of one isg_cluster call on x [B,H,N,d] (allocated here, once)."""
    B, H, N, d = x.shape
    dev = x.device
    labels = torch.empty((B, H, N), device=dev, dtype=torch.int32)
    return dict(centroids=torch.empty((B, H, C_, d), device=dev, dtype=torch.float32), labels=labels,
                perm=torch.empty_like(labels), offsets=torch.empty((B, H, C_ + 1), device=dev, dtype=torch.int32),
                x_perm=torch.empty((B, H, N, d), device=dev, dtype=x.dtype) if want_perm else None,
                companion_perm=(torch.empty((B, H, N, d), device=dev, dtype=x.dtype) if companion is not None
                                else None),
                max_sqnorm=torch.empty((B, H), device=dev, dtype=torch.float32) if want_max_sqnorm else None)


def _check_companion(x, companion):
    if companion is not None:
        _dev(companion, "companion")
        if companion.shape != x.shape or companion.stride() != x.stride() or companion.dtype != x.dtype:
            raise IsgError("companion must match x in shape, strides and dtype")


def isg_cluster(x, C_, iters, *, init=None, companion=None, want_perm=True, want_max_sqnorm=False,
                workspace=None, stream=None):
    """k-means + stable permutation per head of x [B,H,N,d] (d contiguous, any other strides).
    With want_max_sqnorm, also the per-head largest squared row norm [B,H] (fp32), which
    isg_attention takes as k_max_sqnorm when x is K."""
    _dev(x, "x")
    if x.stride(3) != 1:
        raise IsgError("x must have a contiguous last dimension")
    _check_companion(x, companion)
    B, H, N, d = x.shape
    o = cluster_outputs(x, C_, companion=companion, want_perm=want_perm, want_max_sqnorm=want_max_sqnorm)
    if init is not None:
        o["centroids"].copy_(init.to(device=x.device, dtype=torch.float32))
    need = cluster_workspace_size(B, H, N, d, C_)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    st = lib().isg_cluster(_stream(stream), _ptr(x), _dtype(x), _i64x3(x.stride()[:3]), B, H, N, d, C_, iters,
                           0 if init is None else 1, _ptr(companion), _ptr(o["centroids"]), _ptr(o["labels"]),
                           _ptr(o["perm"]), _ptr(o["offsets"]), _ptr(o["x_perm"]), _ptr(o["companion_perm"]),
                           _ptr(o["max_sqnorm"]), _ptr(ws), ws.numel())
    _check(st, "isg_cluster")
    return o


def isg_cluster_noalloc(x, C_, iters, out, *, init_given=False, companion=None, stream=None):
    """isg_cluster through isg_cluster_noalloc: no workspace (the library's static
    scratch) and no allocation here either -- every output goes into ``out``, a dict
    as returned by cluster_outputs (x_perm, companion_perm and max_sqnorm may be
    None).  With ``init_given`` the call starts from out["centroids"] as they are."""
    _dev(x, "x")
    if x.stride(3) != 1:
        raise IsgError("x must have a contiguous last dimension")
    _check_companion(x, companion)
    if (companion is None) != (out.get("companion_perm") is None):
        raise IsgError("out['companion_perm'] must be given exactly when companion is")
    B, H, N, d = x.shape
    st = lib().isg_cluster_noalloc(_stream(stream), _ptr(x), _dtype(x), _i64x3(x.stride()[:3]), B, H, N, d, C_,
                                   iters, 1 if init_given else 0, _ptr(companion), _ptr(out["centroids"]),
                                   _ptr(out["labels"]), _ptr(out["perm"]), _ptr(out["offsets"]),
                                   _ptr(out.get("x_perm")), _ptr(out.get("companion_perm")),
                                   _ptr(out.get("max_sqnorm")))
    _check(st, "isg_cluster_noalloc")
    return out


_side_streams = {}


def _side_stream(device):
    """A second stream of default priority per device (Q's clustering runs on it)."""
    key = torch.device(device).index
    if key is None:
        key = torch.cuda.current_device()
    s = _side_streams.get(key)
    if s is None:
        s = _side_streams[key] = torch.cuda.Stream(device=key)
    return s


def cluster_qk(q, k, v, Cq, Ck, iters, *, ws_q=None, ws_k=None, stream=None):
    """isg_cluster of Q and of K (companion V, and K's per-head largest squared norm
    for isg_attention), Q's on a second stream beside K's.

    Both start after the work already queued on ``stream`` (default: the current
    stream), and ``stream`` waits for both before this returns.  The calls share
    nothing but their inputs, so the results equal two calls in a row.  Every
    tensor Q's call returns is marked as used on ``stream``, so the caching
    allocator does not hand its memory to later side-stream work too early."""
    main = stream if stream is not None else torch.cuda.current_stream(q.device)
    side = _side_stream(q.device)
    ready = torch.cuda.Event()
    ready.record(main)
    side.wait_event(ready)
    with torch.cuda.stream(side):
        cq = isg_cluster(q, Cq, iters, workspace=ws_q, stream=side)
    q.record_stream(side)
    if ws_q is not None:
        ws_q.record_stream(side)
    with torch.cuda.stream(main):
        ck = isg_cluster(k, Ck, iters, companion=v, want_max_sqnorm=True, workspace=ws_k, stream=main)
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    for t in cq.values():
        if t is not None:
            t.record_stream(main)
    return cq, ck


def isg_probs(cq, ck, k_offsets, scale, *, want_pi=True, stream=None):
    _dev(cq, "cq"); _dev(ck, "ck"); _dev(k_offsets, "k_offsets")
    B, H, Cq, d = cq.shape
    Ck = ck.shape[2]
    scores = torch.empty((B, H, Cq, Ck), device=cq.device, dtype=torch.float32)
    pi = torch.empty_like(scores) if want_pi else None
    st = lib().isg_probs(_stream(stream), _ptr(cq.contiguous()), _ptr(ck.contiguous()),
                         _ptr(k_offsets.contiguous()), B, H, Cq, Ck, d, float(scale), _ptr(scores), _ptr(pi))
    _check(st, "isg_probs")
    return scores, pi


def _sel_outputs(scores, m):
    B, H, Cq, Ck = scores.shape
    dev = scores.device
    mm = max(int(m), 1)
    return dict(exact_groups=torch.empty((B, H, Cq, Ck), device=dev, dtype=torch.int32),
                n_exact=torch.empty((B, H, Cq), device=dev, dtype=torch.int32),
                sample_idx=torch.empty((B, H, Cq, mm), device=dev, dtype=torch.int32),
                sample_bias=torch.empty((B, H, Cq, mm), device=dev, dtype=torch.float32),
                n_sample=torch.empty((B, H, Cq), device=dev, dtype=torch.int32), m=int(m))


def isg_select_sample_topp(scores, pi, k_offsets, N, top_p, m, *, mode="importance", seed=0, call_id=0,
                           stream=None):
    """Exact set sized by the top-p rule on pi, then the shared sample."""
    _dev(scores, "scores"); _dev(pi, "pi"); _dev(k_offsets, "k_offsets")
    B, H, Cq, Ck = scores.shape
    out = _sel_outputs(scores, m)
    st = lib().isg_select_sample_topp(_stream(stream), _ptr(scores.contiguous()), _ptr(pi.contiguous()),
                                      _ptr(k_offsets.contiguous()), B, H, Cq, Ck, N, float(top_p), int(m),
                                      MODES[mode] if isinstance(mode, str) else int(mode), C.c_uint64(seed),
                                      C.c_uint64(call_id), _ptr(out["exact_groups"]), _ptr(out["n_exact"]),
                                      _ptr(out["sample_idx"]), _ptr(out["sample_bias"]), _ptr(out["n_sample"]))
    _check(st, "isg_select_sample_topp")
    return out


def isg_select_sample(scores, k_offsets, N, exact_keys, m, *, mode="importance", seed=0, call_id=0,
                      votes=None, stream=None):
    _dev(scores, "scores"); _dev(k_offsets, "k_offsets")
    B, H, Cq, Ck = scores.shape
    out = _sel_outputs(scores, m)
    st = lib().isg_select_sample(_stream(stream), _ptr(scores.contiguous()), _ptr(k_offsets.contiguous()),
                                 _ptr(None if votes is None else votes.contiguous()), B, H, Cq, Ck, N,
                                 int(exact_keys), int(m), MODES[mode] if isinstance(mode, str) else int(mode),
                                 C.c_uint64(seed), C.c_uint64(call_id), _ptr(out["exact_groups"]),
                                 _ptr(out["n_exact"]), _ptr(out["sample_idx"]), _ptr(out["sample_bias"]),
                                 _ptr(out["n_sample"]))
    _check(st, "isg_select_sample")
    return out


def isg_attention(q_p, k_p, v_p, q_offsets, k_offsets, sel, scale, *, k_max_sqnorm=None, perm_q=None,
                  want_lse=True, out=None, workspace=None, n_fallback_tiles=None, stream=None):
    """Attention over each query group's exact and sampled columns.  Rows come out
    in the permuted order of q_p, or in token order when ``perm_q`` (the query
    permutation from isg_cluster) is given, which fuses the un-permute step.
    ``n_fallback_tiles`` (a one-element int32 GPU tensor) receives the number of
    query tiles the rescaling fallback recomputed."""
    for n, t in (("q_p", q_p), ("k_p", k_p), ("v_p", v_p)):
        _dev(t, n)
        if not t.is_contiguous():
            raise IsgError(f"{n} must be contiguous [B,H,N,d]")
    B, H, N, d = q_p.shape
    Cq = q_offsets.shape[-1] - 1
    Ck = k_offsets.shape[-1] - 1
    o_p = out if out is not None else torch.empty_like(q_p)
    lse_p = torch.empty((B, H, N), device=q_p.device, dtype=torch.float32) if want_lse else None
    m = sel["sample_idx"].shape[-1] if sel.get("m") is None else sel["m"]
    need = attention_workspace_size(B, H, N, Cq, Ck, m)
    ws = workspace if workspace is not None else torch.empty(need, device=q_p.device, dtype=torch.uint8)
    st = lib().isg_attention(_stream(stream), _ptr(q_p), _ptr(k_p), _ptr(v_p), _dtype(q_p), B, H, N, d, Cq, Ck,
                             _ptr(q_offsets.contiguous()), _ptr(k_offsets.contiguous()),
                             _ptr(sel["exact_groups"]), _ptr(sel["n_exact"]), _ptr(sel["sample_idx"]),
                             _ptr(sel["sample_bias"]), _ptr(sel["n_sample"]), int(m), float(scale),
                             _ptr(k_max_sqnorm), _ptr(o_p), _ptr(lse_p),
                             _ptr(None if perm_q is None else perm_q.contiguous()), _ptr(n_fallback_tiles),
                             _ptr(ws), ws.numel())
    _check(st, "isg_attention")
    return o_p, lse_p


def isg_unpermute(o_p, lse_p, perm_q, *, out=None, lse_out=None, stream=None):
    _dev(o_p, "o_p"); _dev(perm_q, "perm_q")
    B, H, N, d = o_p.shape
    o = out if out is not None else torch.empty_like(o_p)
    if o.stride(3) != 1:
        raise IsgError("out must have a contiguous last dimension")
    lse = None
    if lse_p is not None:
        lse = lse_out if lse_out is not None else torch.empty_like(lse_p)
    st = lib().isg_unpermute(_stream(stream), _ptr(o_p), _ptr(lse_p), _ptr(perm_q.contiguous()), _dtype(o_p),
                             B, H, N, d, _ptr(o), _i64x3(o.stride()[:3]), _ptr(lse))
    _check(st, "isg_unpermute")
    return o, lse


def pq_codebooks_workspace_size(dtype, B, H, N, d, P, Cc) -> int:
    dt = ISG_BF16 if dtype == torch.bfloat16 else ISG_F32
    return int(lib().isg_pq_codebooks_workspace_size(dt, B, H, N, d, P, Cc))


def pq_codebooks(x, P, Cc, iters, *, workspace=None, stream=None):
    """Product-quantisation codes [P,B,H,N] and codebooks [P,B,H,Cc,d/P] of x [B,H,N,d]
    (isg_pq_codebooks: k-means of every d/P-dim subspace)."""
    _dev(x, "x")
    B, H, N, d = x.shape
    if P < 1 or d % P:
        raise IsgError(f"P={P} must divide d={d}")
    ds = d // P
    dev = x.device
    codes = torch.empty((P, B, H, N), device=dev, dtype=torch.int32)
    cbs = torch.empty((P, B, H, Cc, ds), device=dev, dtype=torch.float32)
    need = pq_codebooks_workspace_size(x.dtype, B, H, N, d, P, Cc)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    st = lib().isg_pq_codebooks(_stream(stream), _ptr(x), _dtype(x), _i64x3(x.stride()[:3]), B, H, N, d, P, Cc,
                                iters, _ptr(codes), _ptr(cbs), _ptr(ws), ws.numel())
    _check(st, "isg_pq_codebooks")
    return codes, cbs


def isg_pq_votes(q_codes, q_codebooks, k_codes, k_codebooks, perm_q, q_offsets, perm_k, k_offsets, exact_keys,
                 scale, *, stream=None):
    """Per-query PQ votes [B,H,Cq,Ck] (plus the Kbar and table intermediates)."""
    for n, t in (("q_codes", q_codes), ("q_codebooks", q_codebooks), ("k_codes", k_codes),
                 ("k_codebooks", k_codebooks), ("perm_q", perm_q), ("q_offsets", q_offsets),
                 ("perm_k", perm_k), ("k_offsets", k_offsets)):
        _dev(t, n)
    P, B, H, N = q_codes.shape
    Cc, ds = q_codebooks.shape[-2:]
    if k_codes.shape != q_codes.shape or k_codebooks.shape != q_codebooks.shape:
        raise IsgError("query and key codes/codebooks must have the same shapes")
    d = P * ds
    Cq, Ck = q_offsets.shape[-1] - 1, k_offsets.shape[-1] - 1
    dev = q_codes.device
    kbar = torch.empty((B, H, Ck, d), device=dev, dtype=torch.float32)
    tables = torch.empty((B, H, P, Cc, Ck), device=dev, dtype=torch.float32)
    votes = torch.empty((B, H, Cq, Ck), device=dev, dtype=torch.int32)
    st = lib().isg_pq_votes(_stream(stream), _ptr(q_codes.contiguous()), _ptr(q_codebooks.contiguous()),
                            _ptr(k_codes.contiguous()), _ptr(k_codebooks.contiguous()), _ptr(perm_q.contiguous()),
                            _ptr(q_offsets.contiguous()), _ptr(perm_k.contiguous()), _ptr(k_offsets.contiguous()),
                            B, H, N, d, P, Cc, Cq, Ck, int(exact_keys), float(scale), _ptr(kbar), _ptr(tables),
                            _ptr(votes))
    _check(st, "isg_pq_votes")
    return dict(kbar=kbar, tables=tables, votes=votes)


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to fp32 (the softmax scale of standard attention)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def pipeline(q, k, v, Cq, Ck, iters, exact_keys, m, *, mode="importance", seed=0, call_id=0, scale=None,
             pq=None, top_p=None, fuse_unpermute=True, stream=None):
    """All steps on one batch: cluster Q and K (+V) side by side on two streams,
    probs, [PQ votes], select/sample, attention, unpermute.  ``pq=(P, Cc)`` is required by
    mode "votes"; ``top_p`` sizes the exact set by mass instead of
    ``exact_keys``.  With ``fuse_unpermute`` the attention writes its rows in token
    order itself (o_p and lse_p are then None); otherwise isg_unpermute runs after
    it.  Returns every intermediate (all on the GPU), and the number of query tiles
    the attention's rescaling fallback recomputed (``n_fallback_tiles``)."""
    d = q.shape[-1]
    scale = default_scale(d) if scale is None else scale
    cq, ck = cluster_qk(q, k, v, Cq, Ck, iters, stream=stream)
    scores, pi = isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, stream=stream)
    pqr = None
    if (MODES[mode] if isinstance(mode, str) else int(mode)) == MODES["votes"]:
        if pq is None:
            raise IsgError('mode "votes" needs pq=(P, Cc)')
        P, Cc = pq
        qc, qcb = pq_codebooks(q, P, Cc, iters, stream=stream)
        kc, kcb = pq_codebooks(k, P, Cc, iters, stream=stream)
        pqr = isg_pq_votes(qc, qcb, kc, kcb, cq["perm"], cq["offsets"], ck["perm"], ck["offsets"], exact_keys,
                           scale, stream=stream)
        pqr.update(q_codes=qc, q_codebooks=qcb, k_codes=kc, k_codebooks=kcb)
    if top_p is not None:
        sel = isg_select_sample_topp(scores, pi, ck["offsets"], q.shape[2], top_p, m, mode=mode, seed=seed,
                                     call_id=call_id, stream=stream)
    else:
        sel = isg_select_sample(scores, ck["offsets"], q.shape[2], exact_keys, m, mode=mode, seed=seed,
                                call_id=call_id, votes=None if pqr is None else pqr["votes"], stream=stream)
    args = (cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"], sel, scale)
    nfb = torch.zeros(1, device=q.device, dtype=torch.int32)
    if fuse_unpermute:
        o_p = lse_p = None
        o, lse = isg_attention(*args, k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"], n_fallback_tiles=nfb,
                               stream=stream)
    else:
        o_p, lse_p = isg_attention(*args, k_max_sqnorm=ck["max_sqnorm"], n_fallback_tiles=nfb, stream=stream)
        o, lse = isg_unpermute(o_p, lse_p, cq["perm"], stream=stream)
    return dict(cq=cq, ck=ck, scores=scores, pi=pi, pq=pqr, sel=sel, o_p=o_p, lse_p=lse_p, o=o, lse=lse,
                scale=scale, n_fallback_tiles=nfb)
