/*
 * crisp.h -- C ABI of the CRISP sparse-prefill attention library (libcrisp.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes (per attention head, causal prefill, batch 1):
 *   1. proxy attention  A_hat = softmax(Q_lastblock K^T / sqrt(d)) over the
 *      last query block of b rows  [rcap.io CRISP summary, per-head
 *      pseudo-code; CRISP paper §2, "representative query subset"];
 *   2. routing  C_struct = (proxy mass on the first w_sink keys and the last
 *      w_local keys) / b; Vertical-Slash iff C_struct >= tau  [CRISP §3.2];
 *   3. selection -- Vertical-Slash heads: column means (vertical) and
 *      diagonal means (slash) of A_hat pooled into blocks, each direction keeps
 *      the first and last block and every block with p_j > alpha * mu,
 *      mu = max(1 - p_0 - p_last, 0) / (N_b - 2), the two unioned  [CRISP §4];
 *      Pooled-Estimation heads: softmax of block-mean-pooled Q K^T, flattened
 *      causal entries kept in descending order until their mass reaches
 *      gamma * total  [CRISP §2, FlexPrefill's PE path, kept by CRISP §4];
 *   4. block-sparse causal attention  O = softmax(Q K^T / sqrt(d) + M_S) V,
 *      M_S = 0 on selected (query-block, key-block) pairs with j <= i, -inf
 *      elsewhere  [CRISP §2, problem statement].
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates nothing, keeps no state between calls, never synchronises the
 *     host, and enqueues all work on `stream` (NULL = the default stream).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     negative status means nothing was launched.  CRISP_E_HIP reports a
 *     failed launch (hipGetLastError right after enqueueing).
 *   - Tensors are [heads, tokens, d] with the d axis contiguous; the head and
 *     token strides are given in ELEMENTS and must be multiples of 8; base
 *     pointers must be 16-byte aligned.  Q and O have hq heads, K and V have
 *     hkv heads; query head h reads KV head h / (hq / hkv).
 *   - Supported: d == 128, block == 128, n a positive multiple of 128 with
 *     n / 128 <= 32768, token strides <= 2^22 elements, hq a multiple of
 *     hkv.  dtype bf16 (compute: bf16 MFMA, fp32 softmax and accumulation) or
 *     fp32 (fp32 MFMA throughout).
 *   - Calls on different streams may overlap as long as their output and
 *     workspace buffers are distinct.
 */
#ifndef CRISP_H
#define CRISP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CRISP_OK = 0,
  CRISP_E_ARG = -1,          /* invalid argument: NULL pointer, bad shape, stride or parameter */
  CRISP_E_UNSUPPORTED = -2,  /* valid but not implemented: d != 128, block != 128, unknown dtype, n too long */
  CRISP_E_WORKSPACE = -3,    /* workspace or column capacity too small */
  CRISP_E_HIP = -4,          /* a kernel launch failed */
  CRISP_E_TOO_LARGE = -5     /* crisp_prefill_noalloc: the problem's workspace exceeds the fixed scratch */
} crisp_status;

typedef enum { CRISP_BF16 = 0, CRISP_FP32 = 1 } crisp_dtype;

/* Problem shape.  Strides are in elements; the d stride is 1. */
typedef struct {
  int64_t n;                 /* tokens (prefill length) */
  int32_t hq, hkv, d;        /* query heads, KV heads, head dim */
  int32_t dtype;             /* crisp_dtype of Q, K, V and O */
  int64_t sq_h, sq_n;        /* Q strides: head, token */
  int64_t sk_h, sk_n;        /* K strides */
  int64_t sv_h, sv_n;        /* V strides */
  int64_t so_h, so_n;        /* O strides */
} crisp_shape;

/* Selection parameters [CRISP §3.2, §4, §5 universal configuration]. */
typedef struct {
  int32_t block;             /* b: block size of pooling, selection and attention tiles; must be 128 */
  int32_t sink;              /* w_sink: keys [0, sink) count as sink mass in C_struct (0 <= sink <= n) */
  int32_t local;             /* w_local: keys [n - local, n) count as recency mass (0 <= local <= n) */
  float tau;                 /* routing threshold, >= 0: Vertical-Slash iff C_struct >= tau */
  float alpha;               /* noise-floor multiplier, >= 0: keep p_j > alpha * mu */
  float gamma;               /* Pooled-Estimation mass target, 0 < gamma <= 1 */
  int32_t min_blocks;        /* per-direction minimum budget for Vertical-Slash heads (0 = off):
                                a direction's set is topped up with its largest remaining scores,
                                ties to the lower index, until it holds min_blocks indices */
  int32_t dense_below_n;     /* length gate: n < dense_below_n takes the dense path (0 = off) */
  int32_t flags;             /* 0 = CRISP as published; otherwise an OR of the CRISP_FLAG_* variants
                                below (unknown bits, or MEDIAN together with COVERAGE: CRISP_E_ARG) */
} crisp_params;

/* Variants the pages compare CRISP against; each changes one decision rule and
 * keeps the proxy, the lists and the attention kernel. */
/* Route by the Jensen-Shannon divergence (natural log) between the pooled
 * estimate a_bar = softmax over key blocks of mean(Q_last) . mean_block(K) /
 * sqrt(d) and the per-query mean p^v: Vertical-Slash iff JSD >= tau, instead
 * of C_struct >= tau [CRISP §2, FlexPrefill's router]. */
#define CRISP_FLAG_ROUTE_JSD   1
/* Vertical-Slash noise floor = median of the non-anchor block scores of the
 * direction instead of their mean [CRISP appendix on the noise floor]. */
#define CRISP_FLAG_VS_MEDIAN   2
/* Vertical-Slash budget = per-direction coverage: blocks by descending score
 * (ties to the lower index) until gamma of the direction's mass, plus the first
 * and last blocks, instead of the noise floor [CRISP §2, FlexPrefill's
 * gamma-cumsum]. */
#define CRISP_FLAG_VS_COVERAGE 4

/* Selection results.  route, c_struct, row_ptr and col_idx are required; the
 * rest are optional diagnostics (NULL = not written).  Lists are one CSR over
 * the hq * N_b rows ordered head-major (row = h * N_b + qb): the key blocks of
 * row r are col_idx[row_ptr[r] .. row_ptr[r+1]), strictly ascending, all <= qb. */
typedef struct {
  int32_t *route;            /* [hq] 1 Vertical-Slash, 0 Pooled-Estimation, -1 dense path */
  float *c_struct;           /* [hq] structural mass (0 when the dense path is taken) */
  int32_t *row_ptr;          /* [hq * N_b + 1] */
  int32_t *col_idx;          /* [col_capacity] */
  int64_t col_capacity;      /* elements available in col_idx; >= crisp_col_capacity() */
  float *pv, *ps;            /* optional [hq * N_b]: block-pooled vertical and slash scores (fp32) */
  int32_t *sv, *nv;          /* optional: sv [hq * N_b] selected vertical indices (ascending), nv [hq] counts */
  int32_t *ss, *ns;          /* optional: the same for the slash direction */
  float *pe_prob;            /* optional [hq * N_b*(N_b+1)/2]: pooled-estimate probabilities of
                                Pooled-Estimation heads, causal triangle row-major
                                (row qb starts at qb*(qb+1)/2); rows of other heads untouched */
  double *jsd;               /* optional [hq]: JSD(a_bar, p^v) (written with CRISP_FLAG_ROUTE_JSD only) */
  float *abar;               /* optional [hq * N_b]: pooled estimate a_bar (CRISP_FLAG_ROUTE_JSD only) */
} crisp_selection;

/* Bytes of workspace needed by crisp_select / crisp_sparse_attn /
 * crisp_dense_attn / crisp_prefill for this shape (0 on invalid arguments).
 * The caller allocates it (256-byte aligned) and may reuse it across calls
 * that do not overlap in time. */
size_t crisp_select_workspace_bytes(const crisp_shape *shape, const crisp_params *params);
size_t crisp_attn_workspace_bytes(const crisp_shape *shape);
size_t crisp_workspace_bytes(const crisp_shape *shape, const crisp_params *params);

/* Worst-case number of list entries: hq * N_b * (N_b + 1) / 2 (0 on invalid shape). */
int64_t crisp_col_capacity(const crisp_shape *shape);

/* Stages 1-3: proxy attention, routing and index selection for every head
 * [CRISP §3.2, §4; rcap.io per-head pseudo-code].  Reads q and k; writes
 * `out`.  Takes the dense path (route -1, every list full) when N_b <= 2 (mu
 * undefined) or n < params->dense_below_n. */
int crisp_select(const crisp_shape *shape, const void *q, const void *k,
                 const crisp_params *params, crisp_selection *out,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Stage 4: causal block-sparse attention over the lists in `sel` (row_ptr and
 * col_idx are read; they may come from crisp_select or from the caller)
 * [CRISP §2, mask M_S].  Query i of block qb attends to keys j <= i whose
 * block is listed for (h, qb); a row with no allowed key yields zeros.
 * Writes o [hq, n, d]. */
int crisp_sparse_attn(const crisp_shape *shape, const void *q, const void *k, const void *v,
                      const crisp_selection *sel, void *o,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense causal attention on the same tile engine: every key block 0..qb for
 * every row, i.e. the problem statement's mask M_S with every causal block
 * selected [CRISP §2], and the exact dense attention the paper's latency
 * comparison measures speedups against [CRISP §5, attention-only latency].
 * Also the path the method falls back to (route -1).  Reads q, k, v; writes
 * o [hq, n, d].  Workspace and errors as for crisp_sparse_attn. */
int crisp_dense_attn(const crisp_shape *shape, const void *q, const void *k, const void *v,
                     void *o, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* All four stages: crisp_select then crisp_sparse_attn, enqueued back to back
 * on `stream` with no host round trip.  `sel` receives the selection.  When
 * the sequence is on the dense path (see crisp_select) the attention is
 * crisp_dense_attn's kernel: the same output as crisp_sparse_attn on the full
 * lists, bit for bit, without reading them. */
int crisp_prefill(const crisp_shape *shape, const void *q, const void *k, const void *v,
                  const crisp_params *params, crisp_selection *sel, void *o,
                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- allocation-free prefill -----------------------------------------------
 * For callers that cannot allocate device memory at call time: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * crisp_prefill_noalloc computes exactly what crisp_prefill computes, with the
 * same kernels, but takes no workspace argument: its workspace is a fixed
 * device array of CRISP_NOALLOC_SCRATCH_BYTES inside the library (one copy per
 * GPU, held until the process ends).  The caller still owns q, k, v, o and the
 * selection buffers.  It allocates nothing and calls no allocating routine.
 *   - A problem whose workspace (crisp_workspace_bytes) exceeds the scratch is
 *     rejected with CRISP_E_TOO_LARGE before anything is enqueued (128 MiB holds
 *     a bf16 Llama-shaped layer of 32 query / 8 KV heads up to 44,800 tokens).
 *   - The first call on a device looks up the array's device address on that
 *     device (hipGetSymbolAddress); CRISP_E_HIP if that fails.
 *   - Every call on one GPU uses the same array, so calls that overlap in time
 *     on one GPU (two streams, two host threads) race and give wrong results;
 *     calls on different GPUs do not interact.  No state is carried from one
 *     call to the next: every counter is cleared by the call's own kernels. */
#define CRISP_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
size_t crisp_noalloc_scratch_bytes(void);
int crisp_prefill_noalloc(const crisp_shape *shape, const void *q, const void *k, const void *v,
                          const crisp_params *params, crisp_selection *sel, void *o, hipStream_t stream);

/* ---- packed batches (varlen) ------------------------------------------------
 * nseq sequences (1 <= nseq <= 64) packed along the token axis of q, k, v, o:
 * sequence i holds tokens [cu_seqlens[i], cu_seqlens[i+1]) and attends only
 * within itself (causal).  cu_seqlens is a HOST array of nseq + 1 offsets with
 * cu_seqlens[0] = 0, cu_seqlens[nseq] = shape->n, every length a positive
 * multiple of 128.  Each sequence is routed and selected on its own, exactly as
 * crisp_prefill would on it alone [the pages leave batching open; CRISP §2
 * defines every step per head and per prompt]; the attention of all sequences
 * is one launch.  Selection outputs are sequence-major: route, c_struct, nv,
 * ns, jsd hold hq entries per sequence; pv, ps, sv, ss, abar hq * N_b(i) per
 * sequence; row_ptr holds hq * N_b(i) + 1 entries per sequence, relative to the
 * sequence's col_idx segment, which starts after hq * N_b(j)(N_b(j)+1)/2 entries
 * for every earlier sequence j (pe_prob is laid out the same way).  Errors as
 * for crisp_prefill; nseq > 64 is CRISP_E_UNSUPPORTED. */
int64_t crisp_varlen_col_capacity(const crisp_shape *shape, int32_t nseq, const int64_t *cu_seqlens);
size_t crisp_varlen_workspace_bytes(const crisp_shape *shape, int32_t nseq, const int64_t *cu_seqlens,
                                    const crisp_params *params);
int crisp_prefill_varlen(const crisp_shape *shape, int32_t nseq, const int64_t *cu_seqlens,
                         const void *q, const void *k, const void *v, const crisp_params *params,
                         crisp_selection *sel, void *o, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Static description of a status code. */
const char *crisp_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* CRISP_H */
