"""Host-only checks of the C ABI: the library loads, exports every function that
include/isg.h declares, and rejects bad arguments before enqueuing anything.
None of these calls reaches a GPU (validation fails first)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from block_sparse_attention_means_amd import isg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "isg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(isg_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_exports():
    assert _declared() == sorted(isg.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = isg.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert isg.version() >= 1


def test_proposal_table_matches_oracle(orc):
    """Both sides build the table independently from its definition."""
    assert np.array_equal(np.array(isg.proposal_table(), np.uint32), orc.proposal_table())


def test_last_error_is_thread_local_string():
    L = isg.lib()
    assert isinstance(L.isg_last_error(), bytes)


FAKE = C.c_void_p(256)  # never dereferenced: validation fails before any launch


def _i64x3(a, b, c):
    return (C.c_int64 * 3)(a, b, c)


def _cluster(**kw):
    a = dict(stream=None, x=FAKE, dt=1, strides=_i64x3(8 * 64 * 128, 64 * 128, 128), B=1, H=8, N=64, d=128,
             C=8, iters=5, init=0, comp=None, cent=FAKE, lab=FAKE, perm=FAKE, off=FAKE, xp=FAKE, cp=None,
             mx=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return isg.lib().isg_cluster(a["stream"], a["x"], a["dt"], a["strides"], a["B"], a["H"], a["N"], a["d"],
                                 a["C"], a["iters"], a["init"], a["comp"], a["cent"], a["lab"], a["perm"],
                                 a["off"], a["xp"], a["cp"], a["mx"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(lab=None), 1), (dict(B=0), 1), (dict(N=0), 1),
    (dict(dt=7), 2), (dict(d=32), 3), (dict(C=0), 1), (dict(C=65), 1), (dict(iters=0), 1),
    (dict(init=2), 1), (dict(comp=FAKE), 1), (dict(strides=_i64x3(8 * 64 * 128, 64 * 128, 100)), 1),
    (dict(ws=None), 4), (dict(wsb=16), 4), (dict(x=C.c_void_p(258)), 1), (dict(B=2, H=40000), 1),
])
def test_cluster_rejects(kw, status):
    assert _cluster(**kw) == status
    assert len(isg.lib().isg_last_error()) > 0


def _cluster_noalloc(**kw):
    a = dict(stream=None, x=FAKE, dt=1, strides=_i64x3(8 * 64 * 128, 64 * 128, 128), B=1, H=8, N=64, d=128,
             C=8, iters=5, init=0, comp=None, cent=FAKE, lab=FAKE, perm=FAKE, off=FAKE, xp=FAKE, cp=None,
             mx=None)
    a.update(kw)
    return isg.lib().isg_cluster_noalloc(a["stream"], a["x"], a["dt"], a["strides"], a["B"], a["H"], a["N"],
                                         a["d"], a["C"], a["iters"], a["init"], a["comp"], a["cent"], a["lab"],
                                         a["perm"], a["off"], a["xp"], a["cp"], a["mx"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(perm=None), 1), (dict(B=0), 1), (dict(dt=3), 2), (dict(d=96), 3), (dict(C=65), 1),
    (dict(comp=FAKE), 1), (dict(x=C.c_void_p(258)), 1),
    # more scratch than the static array holds: K clustering of 40 heads at 84 latent frames
    (dict(H=40, N=302400, C=500, strides=_i64x3(40 * 302400 * 128, 302400 * 128, 128)), 4),
])
def test_cluster_noalloc_rejects(kw, status):
    """Host checks of the no-allocation variant, including a shape beyond its scratch."""
    assert _cluster_noalloc(**kw) == status
    assert len(isg.lib().isg_last_error()) > 0


def test_noalloc_scratch_covers_the_720p_workloads():
    from block_sparse_attention_means_amd.workloads import WORKLOADS
    for name in ("wan1.3b_480p", "wan1.3b_720p", "wan14b_720p", "wan14b_720p_stress_pq"):
        w = WORKLOADS[name]
        for C_ in (w["Cq"], w["Ck"]):
            assert isg.cluster_workspace_size(1, w["H"], w["N"], w["d"], C_) <= isg.NOALLOC_SCRATCH_BYTES, name
    assert isg.cluster_workspace_size(1, 40, 302400, 128, 500) > isg.NOALLOC_SCRATCH_BYTES


def _probs(**kw):
    a = dict(cq=FAKE, ck=FAKE, ko=FAKE, B=1, H=1, Cq=4, Ck=8, d=64, scale=0.125, s=FAKE, pi=None)
    a.update(kw)
    return isg.lib().isg_probs(None, a["cq"], a["ck"], a["ko"], a["B"], a["H"], a["Cq"], a["Ck"], a["d"],
                               a["scale"], a["s"], a["pi"])


@pytest.mark.parametrize("kw", [dict(cq=None), dict(s=None), dict(Cq=0), dict(Ck=2000), dict(d=0),
                                dict(scale=float("inf")), dict(scale=float("nan")), dict(scale=0.0),
                                dict(scale=-0.125)])
def test_probs_rejects(kw):
    assert _probs(**kw) == 1


def _sel(**kw):
    a = dict(S=FAKE, ko=FAKE, votes=None, B=1, H=1, Cq=4, Ck=8, N=100, E=10, m=10, mode=0, eg=FAKE, ne=FAKE,
             si=FAKE, sb=FAKE, ns=FAKE)
    a.update(kw)
    return isg.lib().isg_select_sample(None, a["S"], a["ko"], a["votes"], a["B"], a["H"], a["Cq"], a["Ck"],
                                       a["N"], a["E"], a["m"], a["mode"], C.c_uint64(0), C.c_uint64(0), a["eg"],
                                       a["ne"], a["si"], a["sb"], a["ns"])


@pytest.mark.parametrize("kw", [dict(S=None), dict(ns=None), dict(si=None), dict(E=-1), dict(m=-1),
                                dict(m=101), dict(mode=3), dict(mode=2), dict(votes=FAKE), dict(Ck=0),
                                dict(Ck=1025), dict(N=0)])
def test_select_rejects(kw):
    assert _sel(**kw) == 1


def _topp(**kw):
    a = dict(S=FAKE, pi=FAKE, ko=FAKE, B=1, H=1, Cq=4, Ck=8, N=100, p=0.9, m=10, mode=0, eg=FAKE, ne=FAKE,
             si=FAKE, sb=FAKE, ns=FAKE)
    a.update(kw)
    return isg.lib().isg_select_sample_topp(None, a["S"], a["pi"], a["ko"], a["B"], a["H"], a["Cq"], a["Ck"],
                                            a["N"], a["p"], a["m"], a["mode"], C.c_uint64(0), C.c_uint64(0),
                                            a["eg"], a["ne"], a["si"], a["sb"], a["ns"])


@pytest.mark.parametrize("kw", [dict(pi=None), dict(S=None), dict(ns=None), dict(p=0.0), dict(p=-1.0),
                                dict(p=float("nan")), dict(p=float("inf")), dict(m=101), dict(mode=2),
                                dict(mode=3), dict(Ck=1025), dict(si=None)])
def test_select_topp_rejects(kw):
    assert _topp(**kw) == 1


def test_select_allows_empty_sample_arrays_when_m_is_zero():
    # m = 0 with NULL sample arrays passes validation; a NULL stream with FAKE
    # pointers would launch, so only check that the NULL-array rule is m-dependent
    assert _sel(si=None, sb=None, m=5) == 1


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=1, B=1, H=1, N=256, d=128, Cq=4, Ck=8, qo=FAKE, ko=FAKE, eg=FAKE,
             ne=FAKE, si=FAKE, sb=FAKE, ns=FAKE, m=16, scale=0.088, kmx=None, o=FAKE, lse=None, pq=None,
             nfb=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return isg.lib().isg_attention(None, a["q"], a["k"], a["v"], a["dt"], a["B"], a["H"], a["N"], a["d"],
                                   a["Cq"], a["Ck"], a["qo"], a["ko"], a["eg"], a["ne"], a["si"], a["sb"],
                                   a["ns"], a["m"], a["scale"], a["kmx"], a["o"], a["lse"], a["pq"], a["nfb"],
                                   a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(si=None), 1), (dict(dt=5), 2), (dict(d=96), 3),
    (dict(d=16), 3), (dict(Cq=0), 1), (dict(Ck=4096), 1), (dict(m=257), 1), (dict(scale=float("nan")), 1),
    (dict(scale=0.0), 1), (dict(scale=-0.088), 1), (dict(scale=float("-inf")), 1),
    (dict(ws=None), 4), (dict(wsb=100), 4), (dict(v=C.c_void_p(264)), 1), (dict(B=2, H=40000), 1),
])
def test_attention_rejects(kw, status):
    assert _attn(**kw) == status


def test_workspace_sizes_grow_with_shape():
    a = isg.attention_workspace_size(1, 1, 1000, 8, 32, 100)
    b = isg.attention_workspace_size(1, 2, 1000, 8, 32, 100)
    assert 0 < a < b
    assert isg.cluster_workspace_size(1, 1, 5000, 128, 100) > isg.cluster_workspace_size(1, 1, 500, 128, 100) > 0
    assert isg.attention_workspace_size(0, 1, 10, 1, 1, 0) == 0
    assert isg.attention_workspace_size(1, 1, 10, 1, 1, 11) == 0  # m > N
    assert isg.attention_workspace_size(1, 1, 10, 1, 1, -1) == 0


def test_attention_workspace_follows_m():
    """The column map is sized for N exact rows plus the call's m samples per group:
    at the 14B 720p shape and m = 6,048 that is about half of what m = N needs."""
    H, N, Cq, Ck = 40, 75600, 100, 500
    small = isg.attention_workspace_size(1, H, N, Cq, Ck, 6048)
    full = isg.attention_workspace_size(1, H, N, Cq, Ck, N)
    assert small < 0.6 * full
    assert abs(small - H * Cq * (N + 6048) * 8) < 0.01 * small
    # a workspace sized for a smaller m is refused by a call with a larger m
    ws = isg.attention_workspace_size(1, 1, 256, 4, 8, 8)
    assert ws < isg.attention_workspace_size(1, 1, 256, 4, 8, 128)
    assert _attn(m=128, wsb=ws) == 4
    assert _attn(m=8, wsb=ws, scale=0.0) == 1


def _unperm(**kw):
    a = dict(op=FAKE, lp=None, perm=FAKE, dt=1, B=1, H=1, N=16, d=128, o=FAKE,
             os=_i64x3(16 * 128, 16 * 128, 128), lse=None)
    a.update(kw)
    return isg.lib().isg_unpermute(None, a["op"], a["lp"], a["perm"], a["dt"], a["B"], a["H"], a["N"], a["d"],
                                   a["o"], a["os"], a["lse"])


@pytest.mark.parametrize("kw,status", [
    (dict(op=None), 1), (dict(lp=FAKE), 1), (dict(dt=9), 2), (dict(d=48), 3),
    (dict(os=_i64x3(16 * 128, 16 * 128, 100)), 1), (dict(o=C.c_void_p(260)), 1),
])
def test_unpermute_rejects(kw, status):
    assert _unperm(**kw) == status


def _pq(**kw):
    a = dict(qc=FAKE, qcb=FAKE, kc=FAKE, kcb=FAKE, pq=FAKE, qo=FAKE, pk=FAKE, ko=FAKE, B=1, H=1, N=256, d=128,
             P=8, Cc=256, Cq=4, Ck=8, E=32, scale=0.088, kbar=FAKE, tab=FAKE, votes=FAKE)
    a.update(kw)
    return isg.lib().isg_pq_votes(None, a["qc"], a["qcb"], a["kc"], a["kcb"], a["pq"], a["qo"], a["pk"], a["ko"],
                                  a["B"], a["H"], a["N"], a["d"], a["P"], a["Cc"], a["Cq"], a["Ck"], a["E"],
                                  a["scale"], a["kbar"], a["tab"], a["votes"])


@pytest.mark.parametrize("kw", [dict(qc=None), dict(votes=None), dict(tab=None), dict(N=0), dict(d=512),
                                dict(P=3), dict(P=32, d=256), dict(Cc=0), dict(Cc=5000), dict(Cq=0),
                                dict(Ck=1025), dict(E=-1), dict(scale=float("inf")), dict(scale=0.0),
                                dict(scale=-1.0)])
def test_pq_votes_rejects(kw):
    assert _pq(**kw) == 1
    assert len(isg.lib().isg_last_error()) > 0


def _pqcb(**kw):
    a = dict(x=FAKE, dt=1, strides=_i64x3(8 * 256 * 128, 256 * 128, 128), B=1, H=8, N=256, d=128, P=8, Cc=64,
             iters=5, codes=FAKE, cbs=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return isg.lib().isg_pq_codebooks(None, a["x"], a["dt"], a["strides"], a["B"], a["H"], a["N"], a["d"], a["P"],
                                      a["Cc"], a["iters"], a["codes"], a["cbs"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(cbs=None), 1), (dict(N=0), 1), (dict(dt=7), 2),
    (dict(P=3), 1), (dict(P=4), 3), (dict(P=16), 3), (dict(Cc=0), 1), (dict(Cc=257), 1), (dict(iters=0), 1),
    (dict(H=8192), 1), (dict(strides=_i64x3(8 * 256 * 128, 256 * 128, 100)), 1),
    (dict(strides=_i64x3(8 * 256 * 128, 256 * 128, 120)), 1), (dict(x=C.c_void_p(264)), 1),
    (dict(ws=None), 4), (dict(wsb=1024), 4)])
def test_pq_codebooks_rejects(kw, status):
    assert _pqcb(**kw) == status
    assert len(isg.lib().isg_last_error()) > 0


def test_pq_codebooks_workspace_holds_every_region():
    L = isg.lib()
    B, H, N, d, P, Cc = 1, 40, 75600, 128, 8, 256
    bf = L.isg_pq_codebooks_workspace_size(1, B, H, N, d, P, Cc)
    f32 = L.isg_pq_codebooks_workspace_size(0, B, H, N, d, P, Cc)
    cl = L.isg_cluster_workspace_size(P * B, H, N, d // P, Cc)
    # bf16 16-dim subspaces: the copy, the clustering's own workspace and, per
    # (subspace, head) and chunk of 8192 tokens, Cc*16 int64 sums and Cc counts
    chunks = P * B * H * -(-N // 8192)
    assert bf >= cl + B * H * N * d * 2 + chunks * (Cc * 16 * 8 + Cc * 4)
    # fp32: the copy, the clustering's workspace, the permutation and offsets
    assert f32 >= cl + B * H * N * d * 4 + P * B * H * (N + Cc + 1) * 4
    # more than 256 codewords: the sorted update, as for fp32
    big = L.isg_pq_codebooks_workspace_size(1, B, H, N, d, P, 300)
    assert big >= L.isg_cluster_workspace_size(P * B, H, N, d // P, 300) + B * H * N * d * 2 + P * B * H * N * 4
    for bad in [(1, B, H, N, d, 3, Cc), (1, B, H, N, d, P, 0), (7, B, H, N, d, P, Cc), (1, 0, H, N, d, P, Cc)]:
        assert L.isg_pq_codebooks_workspace_size(*bad) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 16, 16)
    with pytest.raises(isg.IsgError):
        isg.isg_cluster(x, 2, 1)
