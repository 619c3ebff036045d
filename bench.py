"""Benchmark of the whole hot path on synthetic Wan2.1-shaped inputs.

One step = one pass of every stage over one batch already resident in HBM:
cluster Q, cluster K (+V), centroid scores and pi, exact set + shared sample,
fused exact+sampled attention, un-permute.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--exact 0.08] [--sample 0.08] [--no-cpu-baseline] [--no-sweep]

value = effective TFLOP/s of the step: algorithmic attention flops (4 d per
computed (query, column) pair over the exact and sampled columns, padding
excluded) divided by the whole step's time.  The roofline entry is for the
attention kernel alone, timed with HIP events on the stream it runs on.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
METRIC = "ms/call + effective TFLOP/s (% bf16 MFMA peak), 14B-shaped 720p attention"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--exact", type=float, default=0.08)
    ap.add_argument("--sample", type=float, default=0.08)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--mode", default=None, choices=["importance", "uniform", "votes"],
                    help="sampling mode (default: votes for a workload with product quantisation, else importance)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip timing the attention at every budget of the workload and, on the default workload, "
                         "the PQ stress step and the N sweep (all on by default)")
    ap.add_argument("--sweep", action="store_true", help=argparse.SUPPRESS)  # the default; kept for old commands
    ap.add_argument("--serial-cluster", action="store_true",
                    help="cluster Q, then K, on one stream (profiling aid: per-kernel durations do not overlap)")
    ap.add_argument("--top-p", type=float, default=None, metavar="P",
                    help="size the exact set by mass (groups by pi until the running pi reaches P) instead of --exact")
    ap.add_argument("--density-study", action="store_true",
                    help="also report the relative L2 error against dense attention of exact-only, importance and "
                         "uniform calls across the budget sweep (standard and high-entropy generators)")
    ap.add_argument("--study-heads", type=int, default=4, help="heads used by --density-study and --n-sweep")
    ap.add_argument("--n-sweep", action="store_true",
                    help="also time the step and the attention at N = 75600 x 1, 2, 4, 8 (more latent frames; "
                         "part of the default run on the default workload)")
    ap.add_argument("--attention-only", type=int, default=0, metavar="K",
                    help="profiling aid: after one full step, run only K attention calls and exit")
    ap.add_argument("--unpermute-calls", type=int, default=0, metavar="K",
                    help="profiling aid: after the timed steps, run K isg_unpermute calls on the step's permuted-order "
                         "attention output (the step itself fuses the un-permute into the attention)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="profiling aid: copy a GIB-sized buffer 3 times (a plain copy of known size) and exit")
    return ap.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "isg_attention_wan14b_720p_e8s8_traffic.md")
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_attention_means_amd", "csrc", "attention.hip")


def measured_traffic(workload, exact, sample):
    """HBM bytes per attention launch from the committed counter summary (FETCH_SIZE
    and WRITE_SIZE, each scaled by the plain-copy calibration), or None when that
    summary was taken on another workload or on a different attention source."""
    import hashlib
    if (workload, exact, sample) != ("wan14b_720p", 0.08, 0.08) or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    src = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
    if fields.get("source_sha256") != src:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_bytes(d, N, H, B, q_offsets, k_offsets, exact_groups, n_exact, n_sample):
    """Algorithmic HBM bytes of one attention launch: K and V rows (bf16) of every
    column of a query group read once per group, Q read and O written once (bf16),
    LSE written once (fp32)."""
    import numpy as np
    ko = k_offsets.cpu().numpy().astype(np.int64)
    eg = exact_groups.cpu().numpy()
    ne = n_exact.cpu().numpy()
    ns = n_sample.cpu().numpy().astype(np.int64)
    nk = np.diff(ko, axis=-1)
    Bq, Hq, Cq, Ck = eg.shape
    cols = ns.copy()
    for b in range(Bq):
        for h in range(Hq):
            valid = np.arange(Ck)[None, :] < ne[b, h][:, None]
            g = np.where(valid, eg[b, h], 0)
            cols[b, h] += (nk[b, h][g] * valid).sum(-1)
    return float(cols.sum() * 2 * d * 2 + 2 * B * H * N * d * 2 + B * H * N * 4)


def attention_flops(d, q_offsets, k_offsets, exact_groups, n_exact, n_sample):
    """4 d sum_i n^q_i (|E_i| + n_sample_i), from the lists the step produced."""
    import numpy as np
    qo = q_offsets.cpu().numpy().astype(np.int64)
    ko = k_offsets.cpu().numpy().astype(np.int64)
    eg = exact_groups.cpu().numpy()
    ne = n_exact.cpu().numpy()
    ns = n_sample.cpu().numpy().astype(np.int64)
    nq = np.diff(qo, axis=-1)
    nk = np.diff(ko, axis=-1)
    B, H, Cq, Ck = eg.shape
    exact_keys = np.zeros((B, H, Cq), np.int64)
    for b in range(B):
        for h in range(H):
            valid = np.arange(Ck)[None, :] < ne[b, h][:, None]
            g = np.where(valid, eg[b, h], 0)
            exact_keys[b, h] = (nk[b, h][g] * valid).sum(-1)
    cols = exact_keys + ns
    return float(4 * d * (nq * cols).sum()), float((nq * cols).sum())


def query_tiles(q_offsets):
    """128-row query tiles of one attention call (each query group in whole tiles)."""
    import numpy as np
    return int(((np.diff(q_offsets.cpu().numpy().astype(np.int64), axis=-1) + 127) // 128).sum())


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, q, k, v, E, m, seed, mode="importance", top_p=None):
    """The oracle as it stands on one head of the workload: every stage on the whole
    head except attention, which runs on a sample of query groups and is scaled to all
    groups of the head by its share of the head's attention flops."""
    import numpy as np
    import oracle
    d, N, Cq, Ck = w["d"], w["N"], w["Cq"], w["Ck"]
    scale = float(np.float32(1.0 / math.sqrt(d)))
    qh = q[:, :1].float().numpy()
    kh = k[:, :1].float().numpy()
    vh = v[:, :1].float().numpy()
    t0 = time.perf_counter()
    cq = oracle.cluster(qh, Cq, w["iters"])
    ck = oracle.cluster(kh, Ck, w["iters"], companion=vh)
    S, pi = oracle.probs(cq["centroids"], ck["centroids"], ck["offsets"], scale)
    votes = None
    if mode == "votes":
        P, Cc = w["pq"]
        qc, qcb = oracle.pq_codebooks(qh, P, Cc, w["iters"])
        kc, kcb = oracle.pq_codebooks(kh, P, Cc, w["iters"])
        kbar = oracle.pq_kbar(kc, kcb, ck["perm"], ck["offsets"])
        tables = oracle.pq_tables(qcb, kbar, scale)
        votes = oracle.pq_votes(qc, tables, cq["perm"], cq["offsets"], ck["offsets"], E)
    mcode = {"importance": 0, "uniform": 1, "votes": 2}[mode]
    if top_p is not None:
        sel = oracle.select_sample_topp(S, pi, ck["offsets"], N, top_p, m, mode=mcode, seed=seed)
    else:
        sel = oracle.select_sample(S, ck["offsets"], N, E, m, seed=seed, mode=mcode, votes=votes)
    t_pre = time.perf_counter() - t0
    nq = np.diff(cq["offsets"][0, 0])
    nk = np.diff(ck["offsets"][0, 0])
    cols = np.array([nk[sel["exact_groups"][0, 0, i, :sel["n_exact"][0, 0, i]]].sum() + sel["n_sample"][0, 0, i]
                     for i in range(Cq)], np.int64)
    work = nq * cols
    threads = oracle.num_threads()
    order = np.argsort(-work)
    # three query groups per host thread: about 10-20 s of oracle attention on the box
    pick = [i for i in order if work[i] > 0][:max(1, min(3 * threads, Cq))]
    gm = np.zeros((1, 1, Cq), np.uint8)
    gm[0, 0, pick] = 1
    t1 = time.perf_counter()
    o_p, lse_p = oracle.attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"],
                                  sel, m, scale, group_mask=gm)
    t_att = time.perf_counter() - t1
    t2 = time.perf_counter()
    oracle.unpermute(o_p, lse_p, cq["perm"])
    t_un = time.perf_counter() - t2
    frac = work[pick].sum() / work.sum()
    t_head = t_pre + t_att / frac + t_un
    flops_head = 4.0 * d * work.sum()
    return {"value": flops_head / t_head / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": (f"1 of {w['H']} heads of {w.get('name')}: clustering, scores, "
                       f"{'PQ votes, ' if mode == 'votes' else ''}selection and "
                       f"un-permute on the whole head ({t_pre + t_un:.1f} s); attention on the "
                       f"{len(pick)} heaviest query groups ({frac * 100:.1f} % of the head's attention flops, "
                       f"{t_att:.1f} s) scaled to the head; fp64 C with OpenMP"),
            "seconds_measured": round(t_pre + t_att + t_un, 2), "seconds_per_head_est": round(t_head, 2)}


def dense_rows(q, k, v, rows, scale):
    """Dense attention of the given query rows of every head, fp32 on the GPU (the
    reference of the density study; plain torch matmuls, not the product path)."""
    import torch
    B, H, N, d = q.shape
    out = torch.empty((B, H, len(rows), d), device=q.device, dtype=torch.float32)
    for b in range(B):
        for h in range(H):
            qs = q[b, h, rows].float()
            kk = k[b, h].float()
            s = torch.matmul(qs, kk.t().contiguous()) * scale
            pmat = torch.softmax(s, dim=-1)
            out[b, h] = torch.matmul(pmat, v[b, h].float())
    return out


def density_study(args, w, isg, make_workload, WORKLOADS, budget_keys, dev):
    """Relative L2 error of one call against dense attention, on a sample of query
    rows, for exact-only (E+S exact), exact+importance and exact+uniform calls across
    the workload's budget sweep; standard and high-entropy generators."""
    import numpy as np
    import torch
    from block_sparse_attention_means_amd.synth import structured_values
    out = {}
    gens = {"standard": dict(w), "high_entropy": dict(WORKLOADS["wan14b_720p_stress_pq"])}
    for (gname, wg), vkind in [(g, vk) for g in gens.items() for vk in ("v_iid", "v_clustered")]:
        H, N, d = args.study_heads, wg["N"], wg["d"]
        q, k, v, comp = make_workload(wg, seed=args.seed, H=H)
        if vkind == "v_clustered":
            v = structured_values(comp, d, n_centers=wg["n_centers"], seed=args.seed, dtype=wg["dtype"])
        qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
        scale = isg.default_scale(d)
        cq = isg.isg_cluster(qg, wg["Cq"], wg["iters"])
        ck = isg.isg_cluster(kg, wg["Ck"], wg["iters"], companion=vg)
        S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
        rows = torch.from_numpy(np.random.default_rng(1).choice(N, 512, replace=False)).to(dev)
        ref = dense_rows(qg, kg, vg, rows, scale)
        refn = float(torch.linalg.vector_norm(ref))
        table = {}
        for (es, ss) in w["sweep"]:
            E, m = budget_keys(es, N), budget_keys(ss, N)
            res = {}
            for name, e2, m2, mode in (("exact_only", budget_keys(es + ss, N), 0, "importance"),
                                       ("importance", E, m, "importance"), ("uniform", E, m, "uniform")):
                errs = []
                for seed in range(1 if m2 == 0 else 3):
                    sel = isg.isg_select_sample(S, ck["offsets"], N, e2, m2, mode=mode, seed=seed)
                    o_p, lse_p = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"],
                                                   cq["offsets"], ck["offsets"], sel, scale)
                    o, _ = isg.isg_unpermute(o_p, lse_p, cq["perm"])
                    errs.append(float(torch.linalg.vector_norm(o[:, :, rows].float() - ref)) / refn)
                res[name] = round(float(np.mean(errs)), 5)
            table[f"{int(es * 100)}+{int(ss * 100)}%"] = res
        out[f"{gname}/{vkind}"] = table
        del q, k, v, qg, kg, vg
    out["note"] = (f"relative L2 error of O over 512 query rows x {args.study_heads} heads against dense fp32 "
                   "attention; exact_only uses the whole E+S budget as exact keys; sampled modes average 3 seeds; "
                   "v_iid: values N(0, I) as in the benchmark inputs; v_clustered: values with per-component means")
    return out


def n_sweep(args, w, isg, make_workload, budget_keys, dev):
    """Attention and whole-step time as N grows (more latent frames of the same
    45 x 80 latent plane), 8+8 % budgets, study heads."""
    import torch
    out = []
    for mult in (1, 2, 4, 8):
        T = 21 * mult
        N = T * 45 * 80
        wn = dict(w, N=N, grid=(T, 45, 80))
        H = args.study_heads
        q, k, v, _ = make_workload(wn, seed=args.seed, H=H)
        qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
        del q, k, v
        scale = isg.default_scale(w["d"])
        E, m = budget_keys(args.exact, N), budget_keys(args.sample, N)
        stream = torch.cuda.current_stream()
        ws_a = torch.empty(isg.attention_workspace_size(1, H, N, w["Cq"], w["Ck"], m), device=dev,
                           dtype=torch.uint8)

        def run():
            cq, ck = isg.cluster_qk(qg, kg, vg, w["Cq"], w["Ck"], w["iters"], stream=stream)
            S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
            sel = isg.isg_select_sample(S, ck["offsets"], N, E, m, seed=args.seed)
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"], sel,
                              scale, k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"], workspace=ws_a)
            a1.record(stream)
            return cq, ck, sel, (a0, a1)

        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cq, ck, sel, (a0, a1) = run()
        e1.record(stream)
        torch.cuda.synchronize()
        flops, _ = attention_flops(w["d"], cq["offsets"], ck["offsets"], sel["exact_groups"], sel["n_exact"],
                                   sel["n_sample"])
        att_ms = a0.elapsed_time(a1)
        out.append({"N": N, "latent_frames": T, "H": H, "exact_keys": E, "m": m,
                    "step_ms": round(e0.elapsed_time(e1), 3), "attention_ms": round(att_ms, 3),
                    "attention_tflops": round(flops / (att_ms * 1e-3) / 1e12, 2)})
        del qg, kg, vg, ws_a
        torch.cuda.empty_cache()
    return out


def stress_pq_step(args, isg, make_workload, WORKLOADS, budget_keys, dev, steps=3):
    """The whole step of the PQ stress workload (high-entropy 14B-shaped 720p, votes
    mode: clustering, scores, PQ codes and votes, selection, attention), timed over
    `steps` steps after one warm-up, with per-stage HIP-event times."""
    import numpy as np
    import torch
    w = dict(WORKLOADS["wan14b_720p_stress_pq"])
    H, N, d = w["H"], w["N"], w["d"]
    E, m = budget_keys(args.exact, N), budget_keys(args.sample, N)
    q, k, v, _ = make_workload(w, seed=args.seed)
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    scale = isg.default_scale(d)
    P, Cc = w["pq"]
    stream = torch.cuda.current_stream()
    ws_q = torch.empty(isg.cluster_workspace_size(1, H, N, d, w["Cq"]), device=dev, dtype=torch.uint8)
    ws_k = torch.empty(isg.cluster_workspace_size(1, H, N, d, w["Ck"]), device=dev, dtype=torch.uint8)
    ws_p = torch.empty(isg.pq_codebooks_workspace_size(qg.dtype, 1, H, N, d, P, Cc), device=dev, dtype=torch.uint8)
    ws_a = torch.empty(isg.attention_workspace_size(1, H, N, w["Cq"], w["Ck"], m), device=dev, dtype=torch.uint8)
    # the PQ codes of Q and K run on a third stream beside the clustering (the
    # codebook assign is VALU-bound, K's assign matrix-core bound); pq_codes_exposed
    # is the main stream's wait for them after the scores
    stages = ["cluster_q_and_k", "probs", "pq_codes_exposed", "pq_votes", "select_sample", "attention_and_unpermute"]
    ev = {s: [] for s in stages}
    s_pq = torch.cuda.Stream()

    def step(record):
        mk = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
        mk[0].record(stream)
        s_pq.wait_stream(stream)
        with torch.cuda.stream(s_pq):
            qc, qcb = isg.pq_codebooks(qg, P, Cc, w["iters"], workspace=ws_p, stream=s_pq)
            kc, kcb = isg.pq_codebooks(kg, P, Cc, w["iters"], workspace=ws_p, stream=s_pq)
        cq, ck = isg.cluster_qk(qg, kg, vg, w["Cq"], w["Ck"], w["iters"], ws_q=ws_q, ws_k=ws_k, stream=stream)
        mk[1].record(stream)
        S, pi = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=True)
        mk[2].record(stream)
        stream.wait_stream(s_pq)
        mk[3].record(stream)
        votes = isg.isg_pq_votes(qc, qcb, kc, kcb, cq["perm"], cq["offsets"], ck["perm"], ck["offsets"], E,
                                 scale)["votes"]
        mk[4].record(stream)
        sel = isg.isg_select_sample(S, ck["offsets"], N, E, m, mode="votes", seed=args.seed, votes=votes)
        mk[5].record(stream)
        isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"], sel, scale,
                          k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"], workspace=ws_a)
        mk[6].record(stream)
        if record:
            for si, st in enumerate(stages):
                ev[st].append((mk[si], mk[si + 1]))
        return cq, ck, sel

    step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        cq, ck, sel = step(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    flops, _ = attention_flops(d, cq["offsets"], ck["offsets"], sel["exact_groups"], sel["n_exact"], sel["n_sample"])
    stage_ms = {st: round(float(np.mean([a.elapsed_time(b) for a, b in ev[st]])), 3) for st in stages}
    out = {"workload": "wan14b_720p_stress_pq", "mode": "votes", "pq": [P, Cc], "steps": steps,
           "ms_per_step": round(ms_step, 3), "value_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
           "attention_tflop_per_call": round(flops / 1e12, 4), "stage_ms": stage_ms}
    del qg, kg, vg, ws_q, ws_k, ws_p, ws_a
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from block_sparse_attention_means_amd import isg
    from block_sparse_attention_means_amd.synth import make_workload
    from block_sparse_attention_means_amd.workloads import WORKLOADS, budget_keys

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_call": n, "calls": 3,
                          "read_KiB_per_call": n / 1024, "write_KiB_per_call": n / 1024}), flush=True)
        return
    w = dict(WORKLOADS[args.workload])
    w["name"] = args.workload
    B, H, N, d = w.get("B", 1), w["H"], w["N"], w["d"]
    E, m = budget_keys(args.exact, N), budget_keys(args.sample, N)
    mode = args.mode or ("votes" if w.get("pq") else "importance")
    if args.top_p is not None and mode == "votes":
        print("bench.py: --top-p sizes the exact set by mass; it does not combine with votes mode", file=sys.stderr)
        sys.exit(2)
    if mode == "votes" and not w.get("pq"):
        print(f"bench.py: workload {args.workload} has no product-quantisation setting", file=sys.stderr)
        sys.exit(2)
    t0 = time.perf_counter()
    q, k, v, _ = make_workload(w, seed=args.seed)
    print(f"# inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    scale = isg.default_scale(d)
    stream = torch.cuda.current_stream()
    # Q's clustering runs on a second stream beside K's, each with its own workspace
    ws_q = torch.empty(isg.cluster_workspace_size(B, H, N, d, w["Cq"]), device=dev, dtype=torch.uint8)
    ws_k = torch.empty(isg.cluster_workspace_size(B, H, N, d, w["Ck"]), device=dev, dtype=torch.uint8)
    nfb = torch.zeros(1, device=dev, dtype=torch.int32)  # query tiles the rescaling fallback recomputed
    # sized for the largest sample of the workload's budgets (the sweep reuses it)
    m_max = max([m] + [budget_keys(ss, N) for (_, ss) in w.get("sweep", [])])
    ws_a = torch.empty(isg.attention_workspace_size(B, H, N, w["Cq"], w["Ck"], m_max), device=dev,
                       dtype=torch.uint8)
    # the attention writes O and LSE in token order itself (the un-permute step fused)
    # votes mode: the PQ codes of Q and K run on a third stream beside the
    # clustering (serially on the main stream with --serial-cluster); the stage then
    # records only the main stream's wait for them
    pq_side = mode == "votes" and not args.serial_cluster
    s_pq = torch.cuda.Stream() if pq_side else None
    stages = ["cluster_q_and_k", "probs"] + (
        ["pq_codes_exposed" if pq_side else "pq_codes", "pq_votes"] if mode == "votes" else []) + [
        "select_sample", "attention_and_unpermute"]
    ev = {s: [] for s in stages}

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] if record else None
        if record:
            marks[0].record(stream)
        if pq_side:
            P, Cc = w["pq"]
            s_pq.wait_stream(stream)
            with torch.cuda.stream(s_pq):
                qc, qcb = isg.pq_codebooks(qg, P, Cc, w["iters"], stream=s_pq)
                kc, kcb = isg.pq_codebooks(kg, P, Cc, w["iters"], stream=s_pq)
        if args.serial_cluster:
            cq = isg.isg_cluster(qg, w["Cq"], w["iters"], workspace=ws_q, stream=stream)
            ck = isg.isg_cluster(kg, w["Ck"], w["iters"], companion=vg, want_max_sqnorm=True, workspace=ws_k,
                                 stream=stream)
        else:
            cq, ck = isg.cluster_qk(qg, kg, vg, w["Cq"], w["Ck"], w["iters"], ws_q=ws_q, ws_k=ws_k, stream=stream)
        if record:
            marks[1].record(stream)
        # pi is written in every step (a row of the path), although only top-p sizing reads it
        S, pi = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=True)
        mi = 2
        if record:
            marks[mi].record(stream)
        votes = None
        if mode == "votes":
            P, Cc = w["pq"]
            if pq_side:
                stream.wait_stream(s_pq)
            else:
                qc, qcb = isg.pq_codebooks(qg, P, Cc, w["iters"])
                kc, kcb = isg.pq_codebooks(kg, P, Cc, w["iters"])
            mi += 1
            if record:
                marks[mi].record(stream)
            votes = isg.isg_pq_votes(qc, qcb, kc, kcb, cq["perm"], cq["offsets"], ck["perm"], ck["offsets"], E,
                                     scale)["votes"]
            mi += 1
            if record:
                marks[mi].record(stream)
        if args.top_p is not None:
            sel = isg.isg_select_sample_topp(S, pi, ck["offsets"], N, args.top_p, m, mode=mode, seed=args.seed)
        else:
            sel = isg.isg_select_sample(S, ck["offsets"], N, E, m, mode=mode, seed=args.seed, votes=votes)
        mi += 1
        if record:
            marks[mi].record(stream)
        o, lse = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"],
                                   sel, scale, k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"],
                                   workspace=ws_a, n_fallback_tiles=nfb)
        mi += 1
        if record:
            marks[mi].record(stream)
            for si, s in enumerate(stages):
                ev[s].append((marks[si], marks[si + 1]))
        return cq, ck, sel, o

    for _ in range(max(1, args.warmup) if args.attention_only else args.warmup):
        cq, ck, sel, o = step(False)
    torch.cuda.synchronize()
    if args.attention_only:
        for _ in range(args.attention_only):
            isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"], sel,
                              scale, k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"], workspace=ws_a)
        torch.cuda.synchronize()
        print(json.dumps({"attention_only_calls": args.attention_only}), flush=True)
        return
    print("# warmup done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        cq, ck, sel, o = step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # the work of the timed steps (every step computes the same lists)
    flops, pairs = attention_flops(d, cq["offsets"], ck["offsets"], sel["exact_groups"], sel["n_exact"],
                                   sel["n_sample"])
    abytes = attention_bytes(d, N, H, B, cq["offsets"], ck["offsets"], sel["exact_groups"], sel["n_exact"],
                             sel["n_sample"])
    print(f"# attention {flops / 1e12:.2f} TFLOP per call", file=sys.stderr, flush=True)
    ms_step = wall * 1e3 / args.steps
    stage_ms = {s: float(np.mean([a.elapsed_time(b) for a, b in ev[s]])) for s in stages}
    att_ms = stage_ms["attention_and_unpermute"]
    att_tflops = flops / (att_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w["dtype"] == "bf16" else PEAK_FP32_TFLOPS
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded Gaussian-mixture Q/K with 3-D locality bias, V ~ N(0,1); no model weights)",
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "Cq": w["Cq"], "Ck": w["Ck"],
                   "kmeans_iters": w["iters"], "exact_share": args.exact, "sample_share": args.sample,
                   "exact_keys": E, "m": m, "seed": args.seed, "mode": mode,
                   "pq": list(w["pq"]) if mode == "votes" else None, "top_p": args.top_p},
        "attention_ms": round(att_ms, 3),
        "attention_fallback_tiles": int(nfb.item()),
        "attention_query_tiles": query_tiles(cq["offsets"]),
        "attention_tflops": round(att_tflops, 2),
        "attention_tflop_per_call": round(flops / 1e12, 4),
        "stage_ms": {s: round(t, 3) for s, t in stage_ms.items()},
        "roofline": {"bound": "mfma" if w["dtype"] == "bf16" else "alu", "achieved": round(att_tflops, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(att_tflops / peak, 4),
                     "traffic": measured_traffic(args.workload, args.exact, args.sample),
                     "traffic_unit": "bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
                     "algorithmic_bytes": abytes,
                     "kernel": ("isg_attention: attn_pp_kernel with its column-list and tile-table prep, writing O and "
                                "LSE in token order (key norms come from K's clustering)")},
    }
    if not args.no_sweep:
        print("# budget sweep", file=sys.stderr, flush=True)
        sweep = {}
        for (es, ss) in w["sweep"]:
            E2, m2 = budget_keys(es, N), budget_keys(ss, N)
            S, _ = isg.isg_probs(cq["centroids"], ck["centroids"], ck["offsets"], scale, want_pi=False)
            sel2 = isg.isg_select_sample(S, ck["offsets"], N, E2, m2, seed=args.seed,
                                         mode="uniform" if mode == "uniform" else "importance")
            f2, _ = attention_flops(d, cq["offsets"], ck["offsets"], sel2["exact_groups"], sel2["n_exact"],
                                    sel2["n_sample"])
            for _ in range(2):
                isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"],
                                  sel2, scale, k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"], workspace=ws_a,
                                  n_fallback_tiles=nfb)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"],
                                  sel2, scale, k_max_sqnorm=ck["max_sqnorm"], perm_q=cq["perm"], workspace=ws_a)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 5
            sweep[f"{int(es * 100)}+{int(ss * 100)}%"] = {"attention_ms": round(ms, 3),
                                                           "tflop_per_call": round(f2 / 1e12, 4),
                                                           "tflops": round(f2 / ms / 1e9, 2),
                                                           "frac_peak": round(f2 / ms / 1e9 / peak, 4),
                                                           "fallback_tiles": int(nfb.item())}
        result["attention_sweep"] = sweep
    if args.unpermute_calls:
        o_p, lse_p = isg.isg_attention(cq["x_perm"], ck["x_perm"], ck["companion_perm"], cq["offsets"], ck["offsets"],
                                       sel, scale, k_max_sqnorm=ck["max_sqnorm"], workspace=ws_a)
        for _ in range(args.unpermute_calls):
            isg.isg_unpermute(o_p, lse_p, cq["perm"])
        torch.cuda.synchronize()
    if args.density_study:
        print("# density study", file=sys.stderr, flush=True)
        result["density_study"] = density_study(args, w, isg, make_workload, WORKLOADS, budget_keys, dev)
    extras = not args.no_sweep and args.workload == "wan14b_720p" and args.top_p is None and args.mode is None
    if extras:
        # the other headline numbers, measured by every default run: the PQ stress
        # step and the attention / step time as the sequence grows
        del qg, kg, vg, ws_q, ws_k, ws_a
        torch.cuda.empty_cache()
        print("# PQ stress step", file=sys.stderr, flush=True)
        result["stress_pq"] = stress_pq_step(args, isg, make_workload, WORKLOADS, budget_keys, dev)
    if args.n_sweep or extras:
        print("# N sweep", file=sys.stderr, flush=True)
        result["n_sweep"] = n_sweep(args, w, isg, make_workload, budget_keys, dev)
    if not args.no_cpu_baseline:
        print("# timing the oracle on the host (bounded sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, E, m, args.seed, mode, args.top_p)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
