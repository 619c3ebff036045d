"""isg_cluster_noalloc (static scratch, no workspace, no allocation) against
isg_cluster (caller workspace), through the C ABI: every output bit for bit, on
two calls in a row, the second on a smaller input, so the second call runs on
scratch that still holds the first call's contents."""
import pytest
import torch

from block_sparse_attention_means_amd import isg
from block_sparse_attention_means_amd.synth import make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def _inputs(H, N, d, dtype, seed):
    q, k, v, _ = make_qkv(H, N, d, n_centers=12, dtype=dtype, seed=seed)
    return k.to(DEV), v.to(DEV)


def _compare(ref, got, keys):
    for key in keys:
        a, b = ref[key], got[key]
        if a is None:
            assert b is None, key
            continue
        assert torch.equal(a, b), key


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_noalloc_matches_workspace_call_twice(dtype, d):
    keys = ("centroids", "labels", "perm", "offsets", "x_perm", "companion_perm", "max_sqnorm")
    for (H, N, C, iters, seed) in ((4, 20000, 100, 3, 1), (2, 3001, 37, 2, 2)):
        say(f"noalloc dtype={dtype} d={d} H={H} N={N} C={C} iters={iters}")
        x, v = _inputs(H, N, d, dtype, seed)
        ref = isg.isg_cluster(x, C, iters, companion=v, want_max_sqnorm=True)
        out = isg.cluster_outputs(x, C, companion=v, want_max_sqnorm=True)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        isg.isg_cluster_noalloc(x, C, iters, out, companion=v)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        _compare(ref, out, keys)


def test_noalloc_given_centroids_and_strided_input():
    """init_mode 1 (start from the given centroids) and [B,N,H,d] input through
    strides, without the optional outputs; the second call is smaller."""
    for (H, N, C, seed) in ((3, 9000, 64, 4), (1, 700, 9, 5)):
        say(f"noalloc init given H={H} N={N} C={C}")
        x, _ = _inputs(H, N, 128, "bf16", seed)
        xs = x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        init = x[:, :, :C].float().contiguous() * 0.5
        ref = isg.isg_cluster(xs, C, 2, init=init, want_perm=False)
        out = isg.cluster_outputs(xs, C, want_perm=False)
        out["centroids"].copy_(init)
        isg.isg_cluster_noalloc(xs, C, 2, out, init_given=True)
        torch.cuda.synchronize()
        _compare(ref, out, ("centroids", "labels", "perm", "offsets"))


def test_noalloc_under_graph_capture():
    """A caller under graph capture: isg_cluster_noalloc recorded into a HIP graph
    (the call only launches kernels: no allocation, copy or memset), replayed three
    times.  Before each replay the outputs are overwritten and an eager call on
    another shape leaves other contents in the shared scratch; every replay equals
    the workspace call bit for bit."""
    keys = ("centroids", "labels", "perm", "offsets", "x_perm", "companion_perm", "max_sqnorm")
    H, N, C, iters = 2, 6000, 64, 3
    say(f"noalloc graph capture H={H} N={N} C={C} iters={iters}")
    x, v = _inputs(H, N, 128, "bf16", 7)
    ref = isg.isg_cluster(x, C, iters, companion=v, want_max_sqnorm=True)
    out = isg.cluster_outputs(x, C, companion=v, want_max_sqnorm=True)
    isg.isg_cluster_noalloc(x, C, iters, out, companion=v)  # eager first: the scratch address is looked up
    torch.cuda.synchronize()
    _compare(ref, out, keys)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        isg.isg_cluster_noalloc(x, C, iters, out, companion=v)
    torch.cuda.synchronize()
    x2, v2 = _inputs(1, 2500, 128, "bf16", 8)
    out2 = isg.cluster_outputs(x2, 20, companion=v2, want_max_sqnorm=True)
    for rep in range(3):
        for t in out.values():
            if t is not None:
                t.fill_(3)
        isg.isg_cluster_noalloc(x2, 20, 2, out2, companion=v2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        _compare(ref, out, keys)
