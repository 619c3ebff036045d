/*
 * isg.h -- C ABI of libisg: group-shared importance-sampled permuted
 * block-sparse attention (InstaGen) on AMD Instinct MI355X (gfx950).
 *
 * The method (InstaGen, thelatestinai.com page, Figure 3; Paper Reading AI
 * Learner page, abstract), in this header's words: cluster the queries and keys
 * of each head, permute the tokens so every cluster is contiguous, turn
 * centroid scores into a probability pi per (query group, key group), compute
 * each query group's best key groups exactly, stand in for the other keys with
 * one sample per query group whose draw probabilities follow the estimated
 * attention (each sampled term divided by its draw probability), and run one
 * attention over the exact and sampled keys.  The entry points below are the steps of that path, in order:
 *
 *   isg_cluster (Q)  isg_cluster (K, companion V)  isg_probs
 *   isg_select_sample  isg_attention  isg_unpermute
 *
 * Conventions shared by every entry point
 *  - Pointers named as device pointers must be device memory (hipMalloc or a
 *    torch CUDA tensor) owned by the caller; the library never frees them and
 *    keeps no reference after the call returns.  Scratch comes from the
 *    caller's `workspace`, sized by the matching *_workspace_size().
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Every
 *    call only enqueues work on it and returns; nothing synchronises the host.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failed check returns a non-zero isg_status, launches nothing, and
 *    isg_last_error() (thread-local) describes it.  Nothing throws across the
 *    ABI.  Device-side contents (labels, offsets, lists) are trusted: they must
 *    come from the previous steps or satisfy the same invariants.
 *  - Tensors are row-major; "[B,H,N,d]" means d is contiguous.  Integer outputs
 *    (labels, permutations, offsets, exact lists, sample indices) are bitwise
 *    deterministic; float outputs are deterministic run to run (no float
 *    atomics).  Calls that overlap on one stream are ordered; the functions
 *    keep no global mutable state and are reentrant.
 *  - dtypes: ISG_F32 or ISG_BF16 for Q/K/V and the attention output; every
 *    accumulation is fp32 or wider.
 *  - Heads: isg_cluster, isg_attention and isg_pq_votes give each head a row
 *    of a launch grid, so they need B*H <= 65535 and reject more with
 *    ISG_E_ARG.
 */
#ifndef ISG_H
#define ISG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ISG_OK = 0,
    ISG_E_ARG = 1,          /* null pointer, bad shape, budget out of range */
    ISG_E_DTYPE = 2,        /* dtype not supported by this entry point */
    ISG_E_UNSUPPORTED = 3,  /* shape supported by the method but not built (e.g. d) */
    ISG_E_WORKSPACE = 4,    /* workspace missing or too small */
    ISG_E_HIP = 5           /* HIP runtime / launch error */
} isg_status;

/* dtypes.  A caller may pass any int here (unknown values return ISG_E_DTYPE); the
 * library is C++, where only a fixed underlying type makes every int a valid value. */
#ifdef __cplusplus
typedef enum isg_dtype_e : int { ISG_F32 = 0, ISG_BF16 = 1 } isg_dtype;
#else
typedef enum isg_dtype_e { ISG_F32 = 0, ISG_BF16 = 1 } isg_dtype;
#endif

typedef enum {
    ISG_SAMPLE_IMPORTANCE = 0,  /* proposal ~ n_j exp(S_ij) (quantised), the pages' main mode */
    ISG_SAMPLE_UNIFORM = 1,     /* every skipped key equally likely */
    ISG_SAMPLE_VOTES = 2        /* exact set ranked by per-query PQ votes, importance sample */
} isg_sample_mode;

/* Thread-local description of the last failure of an isg_* call on this thread. */
const char *isg_last_error(void);

/* ABI version (incremented on incompatible change). */
int isg_version(void);

/* The integer proposal weights used by isg_select_sample in importance mode:
 * out[k] = round(2^31 * 2^(-k/256)), k = 0..255 (host only, no GPU needed). */
void isg_proposal_table(uint32_t out[256]);

/* ------------------------------------------------------------------------ */
/* isg_cluster -- k-means (Lloyd) per head, then a stable permutation.
 * Pages: InstaGen, thelatestinai.com page, Figure 3(a) (Q and K partitioned by
 * clustering) and Figure 2 (Cq = 100, Ck = 500).  The pages do not
 * fix the algorithm; this is Euclidean Lloyd k-means on the raw vectors:
 *   init (init_mode 0): c_j = x_{floor(j*N/C)}; init_mode 1: centroids as given;
 *   `iters` rounds of: label_t = argmin_j |x_t - c_j|^2 (ties -> lowest j),
 *                      c_j = mean of its members (empty cluster keeps c_j);
 *   perm = tokens stably sorted by the last labels; offsets = prefix of counts;
 *   x_perm[r] = x[perm[r]], companion_perm[r] = companion[perm[r]].
 * The labels are the assignment of the last round and the centroids are the
 * means of those groups.  For bf16 x the argmin is screened on fp32 distances
 * (bf16 hi/lo centroid planes on the matrix cores) and the four best are kept
 * (three at d = 16); whenever other kept candidates lie within the screening
 * error bound of the best, it is re-decided on fp64 distances among them, or
 * over all C when all kept candidates are that close.  At d = 16 these fp64
 * distances are sequential unfused sums over k = 0..15, so the labels are the
 * fp64 argmin of the definition exactly; at larger d they sum per-lane pieces in
 * another order.  For fp32 x the argmin is taken on fp32 distances (sequential
 * fused sums) and stands unless the runner-up lies within 4e-5 relative of the
 * best; then every centroid is re-compared in fp64.  Outside bf16 at d = 16 a
 * label differs from the fp64 argmin only at fp64-level ties.
 *
 * x           device, dtype dt, element (b,h,t,k) at x[b*xs[0] + h*xs[1] + t*xs[2] + k]
 *             (xs = x_strides, in elements; k contiguous).  [B,N,H,d] and
 *             sub-vectors (product-quantisation subspaces) are expressible.
 * companion   device or NULL, same dtype and strides as x (V when x is K).
 * B,H,N,d,C   1 <= C <= min(N, 4096), d in {16, 64, 128}; iters >= 1.
 * centroids   device fp32 [B,H,C,d]; read when init_mode = 1, always written.
 * labels      device int32 [B,H,N] (written).
 * perm        device int32 [B,H,N] (written): perm[r] = token at sorted row r.
 * offsets     device int32 [B,H,C+1] (written): group j = rows [off[j], off[j+1]).
 * x_perm      device or NULL, dtype dt, contiguous [B,H,N,d] (written).
 * companion_perm  device or NULL (must be non-NULL iff companion is), [B,H,N,d].
 * max_sqnorm  device fp32 [B,H] or NULL: per head, the largest squared row norm
 *             of x (fp32 fma chain over each 8-element chunk, chunks of a row
 *             added by a butterfly), computed from the rows the last round's
 *             update reads; isg_attention accepts it as k_max_sqnorm.
 * workspace   device, >= isg_cluster_workspace_size(B,H,N,d,C) bytes. */
size_t isg_cluster_workspace_size(int B, int H, int N, int d, int C);
isg_status isg_cluster(void *stream, const void *x, isg_dtype dt, const int64_t x_strides[3],
                       int B, int H, int N, int d, int C, int iters, int init_mode,
                       const void *companion, float *centroids, int32_t *labels, int32_t *perm,
                       int32_t *offsets, void *x_perm, void *companion_perm, float *max_sqnorm,
                       void *workspace, size_t ws_bytes);

/* ------------------------------------------------------------------------ */
/* isg_cluster_noalloc -- isg_cluster without a workspace and without allocating.
 * For callers that cannot allocate device memory during a call: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, computation and results as isg_cluster (bit for bit), minus the
 * workspace: its scratch is a static device array of
 * ISG_CLUSTER_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per GPU, allocated with
 * the library's code object and held until the process ends.  A shape whose
 * isg_cluster_workspace_size() exceeds that returns ISG_E_WORKSPACE before
 * anything is enqueued (every 720p shape of this library's workloads fits: K of
 * 40 heads x 75,600 tokens at C = 500 needs about 50 MB; split the heads over
 * several calls otherwise).  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the first call on a device resolves that device's
 * copy of the array (hipGetSymbolAddress, with the device current) and keeps the
 * address.  The stream's device decides which copy is used (NULL: the current
 * device).  Calls on one GPU share the array: calls that may overlap on one GPU
 * (two streams, or two host threads) race and must be ordered by the caller. */
#define ISG_CLUSTER_NOALLOC_SCRATCH_BYTES (64u << 20)
isg_status isg_cluster_noalloc(void *stream, const void *x, isg_dtype dt, const int64_t x_strides[3],
                               int B, int H, int N, int d, int C, int iters, int init_mode,
                               const void *companion, float *centroids, int32_t *labels, int32_t *perm,
                               int32_t *offsets, void *x_perm, void *companion_perm, float *max_sqnorm);

/* ------------------------------------------------------------------------ */
/* isg_probs -- centroid scores and pi.
 * Pages: InstaGen, thelatestinai.com page, Figure 3(b) (centroid scores turned
 * into the probability pi that a query group uses a key group); Paper Reading
 * AI Learner page, abstract (draws follow the estimated attention).
 *   S_ij  = (fp32 fused multiply-add chain over k = 0..d-1 of cq_ik*ck_jk) * scale
 *           -- this exact fp32 order is part of the contract;
 *   pi_ij = n_j e^{S_ij} / sum_j' n_j' e^{S_ij'} over non-empty groups (0 if empty),
 *           with n_j = k_offsets[j+1] - k_offsets[j].
 * cq [B,H,Cq,d], ck [B,H,Ck,d] device fp32; k_offsets device int32 [B,H,Ck+1];
 * scores device fp32 [B,H,Cq,Ck] (written); pi device fp32 [B,H,Cq,Ck] or NULL.
 * Cq, Ck in [1, 1024]; d in [1, 1024]; scale finite and > 0. */
isg_status isg_probs(void *stream, const float *cq, const float *ck, const int32_t *k_offsets,
                     int B, int H, int Cq, int Ck, int d, float scale, float *scores, float *pi);

/* ------------------------------------------------------------------------ */
/* isg_select_sample -- exact set and the shared sample of each query group.
 * Pages: Paper Reading AI Learner page, abstract (high-scoring keys computed
 * exactly; the rest estimated from a sample drawn by estimated attention, each
 * term divided by its draw probability; one sample per query cluster, used by
 * all of its queries); thelatestinai.com page, Figure 3(c) (the best key group
 * is never dropped); acceptodds.com page, abstract (the number of sampled
 * tokens is the budget).
 *
 * Exact set of query group i: non-empty key groups ordered by (S_ij desc,
 * j asc) -- in ISG_SAMPLE_VOTES mode by (votes desc, S desc, j asc) -- the
 * first always, then the following ones while the running key count stays
 * <= exact_keys, stopping at the first that would exceed it.  Written as group
 * ids ascending, -1 padded: exact_groups [B,H,Cq,Ck], n_exact [B,H,Cq].
 *
 * Sample: the skipped region is every non-empty group not in the exact set
 * (M keys).  M = 0: no sample.  M <= m: every skipped key once (ascending
 * group, then row), offset 0.  Otherwise m i.i.d. draws with replacement: draw
 * t takes group j with probability n_j u_ij / T_i and a row uniformly inside
 * it; u_ij = max(1, tbl[a & 255] >> (a >> 8)) with a = clamp(rint((Smax_i - S_ij)
 * * 369.32993f), 0, 7936) in fp32 (importance) or u = 1 (uniform), tbl from
 * isg_proposal_table, Smax_i the largest score over the skipped groups.  The
 * offset is ln(T_i) - ln(u_ij) - ln(m) = ln(1 / (m p)), p the per-key draw
 * probability.  Randomness: Philox4x64-10, key (seed, call_id), counter
 * (floor(t/2) + 1, i, h, b); words 2(t%2), 2(t%2)+1 form a 128-bit r and the
 * draw position is floor(r T / 2^128).  sample_idx [B,H,Cq,m] holds rows of
 * the permuted K (absolute row within the head), sample_bias [B,H,Cq,m] the
 * offsets, n_sample [B,H,Cq] the count (entries past it are not written).
 *
 * scores device fp32 [B,H,Cq,Ck]; k_offsets device int32 [B,H,Ck+1];
 * votes device int32 [B,H,Cq,Ck], required iff mode = ISG_SAMPLE_VOTES;
 * 0 <= exact_keys; 0 <= m <= N; Ck in [1, 1024]. */
isg_status isg_select_sample(void *stream, const float *scores, const int32_t *k_offsets,
                             const int32_t *votes, int B, int H, int Cq, int Ck, int N,
                             int exact_keys, int m, int mode, uint64_t seed, uint64_t call_id,
                             int32_t *exact_groups, int32_t *n_exact, int32_t *sample_idx,
                             float *sample_bias, int32_t *n_sample);

/* ------------------------------------------------------------------------ */
/* isg_select_sample_topp -- isg_select_sample with the exact set sized by mass.
 * Pages: Paper Reading AI Learner page, abstract (the method wraps any
 * block-sparse selector); thelatestinai.com page, Figure 2 (SVG2, whose
 * selector keeps the smallest set of clusters reaching a probability mass).
 * Exact set of query group i: non-empty key groups ordered by (pi_ij desc,
 * j asc), taken one by one until the fp64 running sum of pi_ij, added in that
 * order, reaches top_p (so the first is always taken; top_p >= the total mass
 * takes every group).  The sample over the other groups is exactly that of
 * isg_select_sample in ISG_SAMPLE_IMPORTANCE or ISG_SAMPLE_UNIFORM mode.
 * pi device fp32 [B,H,Cq,Ck] as written by isg_probs; top_p finite, > 0;
 * every other argument and output as for isg_select_sample. */
isg_status isg_select_sample_topp(void *stream, const float *scores, const float *pi,
                                  const int32_t *k_offsets, int B, int H, int Cq, int Ck, int N,
                                  float top_p, int m, int mode, uint64_t seed, uint64_t call_id,
                                  int32_t *exact_groups, int32_t *n_exact, int32_t *sample_idx,
                                  float *sample_bias, int32_t *n_sample);

/* ------------------------------------------------------------------------ */
/* isg_attention -- one attention over the exact and sampled keys.
 * Pages: acceptodds.com page, abstract (exact blocks and sampled tokens go
 * through one attention kernel, the sampled scores adjusted to stand for every
 * skipped key); thelatestinai.com page, Figure 3(d) (one key set per query
 * group, so the work is dense blocks).
 * For query row r of group i the columns are every row of every exact group
 * (offset 0) followed by the n_sample samples (row sample_idx[t], offset
 * sample_bias[t]):
 *   l = scale <q_r, k> + offset,  O_r = sum e^l v / sum e^l,  LSE_r = ln sum e^l.
 * q_p, k_p, v_p device [B,H,N,d] in permuted order (from isg_cluster), dtype dt;
 * q_offsets [B,H,Cq+1], k_offsets [B,H,Ck+1] device int32; the list arguments
 * as written by isg_select_sample with the same m; d in {64, 128}; Cq, Ck in
 * [1, 1024]. k_max_sqnorm device fp32 [B,H] or NULL: the largest squared key
 * norm per head, as isg_cluster of K writes it (max_sqnorm); bf16 calls use it
 * for the fixed per-row reference and otherwise compute it with a pass over
 * k_p (fp32 calls do not use it). o_p device dtype dt [B,H,N,d] (written);
 * lse_p device fp32 [B,H,N] or NULL (natural log).  perm_q device int32
 * [B,H,N] or NULL: NULL writes row r of o_p and lse_p in the permuted order of
 * q_p; given (the query permutation from isg_cluster), row r goes to
 * o_p[perm_q[r]] and lse_p[perm_q[r]], i.e. token order, which is what
 * isg_unpermute would produce from the permuted rows (the un-permute fused).
 * n_fallback_tiles device int32 scalar or NULL: bf16 calls write the number of
 * 128-row query tiles whose weights fell so far below the fixed per-row
 * reference (row sum < 2^-80) that a second kernel recomputed them with a
 * running maximum (0 for fp32 calls, which always use a running maximum).
 * scale is the softmax scale (1/sqrt(d) in the method): finite and > 0, since the
 * fixed per-row reference of the bf16 kernels bounds the logits only for a
 * positive scale; anything else returns ISG_E_ARG.
 * workspace device, >= isg_attention_workspace_size(B,H,N,Cq,Ck,m) bytes (the
 * column map holds each query group's exact rows, at most N, plus its m samples:
 * about B*H*Cq*(N+m)*8 bytes).  Returns 0 for an invalid shape (m outside [0, N]). */
size_t isg_attention_workspace_size(int B, int H, int N, int Cq, int Ck, int m);
isg_status isg_attention(void *stream, const void *q_p, const void *k_p, const void *v_p,
                         isg_dtype dt, int B, int H, int N, int d, int Cq, int Ck,
                         const int32_t *q_offsets, const int32_t *k_offsets,
                         const int32_t *exact_groups, const int32_t *n_exact,
                         const int32_t *sample_idx, const float *sample_bias,
                         const int32_t *n_sample, int m, float scale, const float *k_max_sqnorm,
                         void *o_p, float *lse_p, const int32_t *perm_q, int32_t *n_fallback_tiles,
                         void *workspace, size_t ws_bytes);

/* ------------------------------------------------------------------------ */
/* isg_unpermute -- rows back to token order: o[perm_q[r]] = o_p[r] (and lse).
 * Implied by attention over a permuted matrix (Paper Reading AI Learner page,
 * abstract).  o_p device dtype dt [B,H,N,d]; lse_p device fp32 [B,H,N] or NULL;
 * perm_q device int32 [B,H,N] (a permutation per head); o device dtype dt with
 * element (b,h,t,k) at o[b*os[0] + h*os[1] + t*os[2] + k] (os = o_strides in
 * elements, so [B,N,H,d] works); lse device fp32 [B,H,N] or NULL (iff lse_p). */
isg_status isg_unpermute(void *stream, const void *o_p, const float *lse_p, const int32_t *perm_q,
                         isg_dtype dt, int B, int H, int N, int d, void *o,
                         const int64_t o_strides[3], float *lse);

/* ------------------------------------------------------------------------ */
/* isg_pq_codebooks -- product-quantisation codes and codebooks of x.
 * Pages: InstaGen, acceptodds.com page, abstract (queries and keys are product-
 * quantised).  The pages do not say how the codebooks are trained; the reading
 * taken: subspace s of x (dims [s*ds, (s+1)*ds), ds = d/P) is clustered by the
 * same k-means as isg_cluster (init_mode 0, iters rounds, Cc centroids), its
 * centroids are the subspace-s codebook and its labels the codes.  The call first
 * copies x into subspace-major order in the workspace, so every subspace's rows
 * are dense, then runs the rounds for all P*B*H (subspace, batch, head) triples at
 * once.  The labels of each round are isg_cluster's on that subspace alone.  The
 * means: for bf16 x with d/P = 16 and Cc <= 256 each codeword's rows are added as
 * exact integers: a fixed point of 2^-s per triple, s set by the triple's largest
 * exponent so that each value is below 2^lim and N of them below 2^62
 * (lim = min(62 - ceil(log2(N+1)), 51), 45 at N = 75,600); values whose exponent
 * lies more than lim - 8 below the largest are rounded to that grid.  The result
 * then does not depend on the order of the additions; the mean is that sum over
 * the count in fp64, rounded to fp32.  It equals isg_cluster's fp64 mean whenever
 * both sums are exact (a group's values spanning fewer than 45 - log2(N) binary
 * orders, 28 at N = 75,600, for isg_cluster's) and is otherwise within the grid's
 * rounding of the exact mean.  Other cases run isg_cluster's rounds and give its
 * result on each subspace alone.
 *
 * x          device, dt (ISG_BF16 or ISG_F32), element (b,h,t,k) at
 *            b*x_strides[0] + h*x_strides[1] + t*x_strides[2] + k (strides in
 *            elements, multiples of 8, x_strides[2] >= d; 16-byte aligned);
 * codes      device int32 [P,B,H,N] (written): the code of token t in subspace s;
 * codebooks  device fp32 [P,B,H,Cc,ds] (written);
 * workspace  device, >= isg_pq_codebooks_workspace_size(dt, B, H, N, d, P, Cc)
 *            bytes (the subspace-major copy, isg_cluster's own workspace, and
 *            either the integer sums per chunk of 8192 tokens or the sorted
 *            update's permutation and offsets); caller-owned, no state kept
 *            between calls.
 * Needs P | d, d/P in {16, 64, 128}, P*B*H <= 65535, 1 <= Cc <= min(N, 4096),
 * iters >= 1; else ISG_E_ARG / ISG_E_UNSUPPORTED / ISG_E_DTYPE / ISG_E_WORKSPACE
 * with nothing launched.  x is expected finite: with an infinity or NaN in it the
 * codes and codebooks are unspecified (every code still lies in [0, Cc) and every
 * access stays inside the buffers). */
size_t isg_pq_codebooks_workspace_size(isg_dtype dt, int B, int H, int N, int d, int P, int Cc);
isg_status isg_pq_codebooks(void *stream, const void *x, isg_dtype dt, const int64_t x_strides[3], int B, int H,
                            int N, int d, int P, int Cc, int iters, int32_t *codes, float *codebooks,
                            void *workspace, size_t ws_bytes);

/* ------------------------------------------------------------------------ */
/* isg_pq_votes -- product-quantised per-query votes for the exact set.
 * Pages: InstaGen, acceptodds.com page, abstract (product-quantised Q and K
 * make block scores affordable for every query; each query picks its own top
 * blocks; a query group's exact set is the blocks picked most often).  The pages give no formula; the reading taken:
 *   Kbar_{j,s} = mean over the rows of key group j of their subspace-s codeword
 *                (fp64 sum in permuted row order, one division, fp32 result;
 *                0 for an empty group);
 *   M_s[a][j]  = (fp32 fused multiply-add chain over the ds dims of
 *                cwq_{s,a} * Kbar_{j,s}) * scale;
 *   score(q,j) = fp32 sum over s ascending of M_s[code_s(q)][j];
 *   every query applies the exact-set rule of isg_select_sample to its own
 *   ranking (score desc, j asc) and votes for each group it takes;
 *   votes[i][j] = number of queries of group i that voted for j.
 * The votes feed isg_select_sample in ISG_SAMPLE_VOTES mode.
 *
 * q_codes, k_codes   device int32 [P,B,H,N], token order: the codes of
 *                    isg_pq_codebooks (subspace s = dims [s*ds, (s+1)*ds), ds = d/P);
 * q_codebooks, k_codebooks  device fp32 [P,B,H,Cc,ds]: its codebooks;
 * perm_q, q_offsets, perm_k, k_offsets  device int32, from isg_cluster on the
 *                    full vectors ([B,H,N] and [B,H,C+1]);
 * kbar    device fp32 [B,H,Ck,d] (written);
 * tables  device fp32 [B,H,P,Cc,Ck] (written);
 * votes   device int32 [B,H,Cq,Ck] (written).
 * d <= 256, 1 <= P <= 16, P | d; Cc in [1, 4096]; Cq, Ck in [1, 1024];
 * exact_keys >= 0; scale finite and > 0; codes must lie in [0, Cc) (not checked). */
isg_status isg_pq_votes(void *stream, const int32_t *q_codes, const float *q_codebooks,
                        const int32_t *k_codes, const float *k_codebooks, const int32_t *perm_q,
                        const int32_t *q_offsets, const int32_t *perm_k, const int32_t *k_offsets,
                        int B, int H, int N, int d, int P, int Cc, int Cq, int Ck, int exact_keys,
                        float scale, float *kbar, float *tables, int32_t *votes);

#ifdef __cplusplus
}
#endif
#endif /* ISG_H */
