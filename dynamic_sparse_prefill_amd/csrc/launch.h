// Internal launchers (C++ linkage) called by the C-ABI layer in crisp.cpp.
// Every launcher only enqueues work on `s` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crisp {

struct Strides { int64_t q_h, q_n, k_h, k_n, v_h, v_n, o_h, o_n; };

// ---- attention (attn.hip)
// V [hkv][n][d] -> per-block transposed V^T; also zeroes *queue (may be NULL)
hipError_t launch_transpose_v(int fp32, const void* V, void* Vt, int nb, int hkv,
                              int64_t sv_h, int64_t sv_n, int* queue, hipStream_t s);
constexpr int ATTN_QUEUE_INTS = 16;   // work counters of the persistent attention kernel

// The bf16 V re-layout of a prefill, handed to the proxy launch so that it runs
// in the same grid as the proxy scores (extra work-groups) instead of as a
// launch of its own between selection and attention.  V == nullptr: none.
struct VtJob {
  const void* V = nullptr;
  void* Vt = nullptr;
  int64_t sv_h = 0, sv_n = 0;
  int nb = 0;                 // blocks of the whole packed V (V^T head stride)
  int* queue = nullptr;       // ATTN_QUEUE_INTS counters, zeroed with the re-layout
};

// Sequences of a packed batch (a single prefill is one sequence).  Passed by
// value to the attention kernel.  Sequence i owns tokens [tok[i], tok[i] + 128
// nb[i]) of Q, K, V^T and O, and its lists live at row_ptr + rp[i] (hq * nb[i]
// + 1 entries, offsets relative to col_idx + col[i]).
constexpr int MAX_SEQ = 64;
// Pooled-estimation logits are produced in segments of pe_seg(N_b) tiles of 32
// key blocks (one work item each); every row keeps one (max, sum) pair per
// segment.  Long sequences take longer segments (fewer item start-ups); the
// size depends on the sequence's own N_b only, so a sequence is cut the same
// way alone and in a packed batch.
__host__ __device__ inline int pe_seg(int nb) { return nb >= 4096 ? 16 : 8; }
__host__ __device__ inline int pe_segments(int nb) { return ((nb + 31) / 32 + pe_seg(nb) - 1) / pe_seg(nb); }
struct SeqTable {
  int nseq;
  int unit_off[MAX_SEQ + 1];   // work units (query-block pairs x KV heads) before sequence i
  int nb[MAX_SEQ];
  int64_t tok[MAX_SEQ];
  int64_t rp[MAX_SEQ];
  int64_t col[MAX_SEQ];
  int pair_major;              // set by the attention launcher: unit order (see queue_item in attn.hip)
};

// Sequences of a selection batch (a single prefill is one sequence), by
// value in the selection kernels: a kernel working on "virtual head"
// vh = s * hq + h finds where sequence s starts in the packed arrays with
// seq_pos.  Per-row arrays ([hq * N_b] per sequence) are sequence-major, the
// pooled matrices ([hq * N_b(N_b+1)/2]) and the row pointers ([hq * N_b + 1])
// likewise.
struct SeqList {
  int nseq;
  int nb[MAX_SEQ];
};
struct SeqPos {
  int nb;
  int64_t tok;     // first token
  int64_t rows;    // hq * N_b of the earlier sequences
  int64_t tri;     // hq * N_b(N_b+1)/2 of the earlier sequences
  int64_t rp;      // row pointers of the earlier sequences (hq * N_b + 1 each)
  int64_t kvrows;  // hkv * N_b of the earlier sequences (K-bar rows)
};
inline int pe_segments_max(const SeqList& L) {   // row stride of the per-segment partials
  int m = 1;
  for (int i = 0; i < L.nseq; ++i) m = pe_segments(L.nb[i]) > m ? pe_segments(L.nb[i]) : m;
  return m;
}
__host__ __device__ inline SeqPos seq_pos(const SeqList& L, int s, int hq, int hkv) {
  SeqPos p{L.nb[s], 0, 0, 0, 0, 0};
  for (int i = 0; i < s; ++i) {
    const int64_t b = L.nb[i];
    p.tok += b * 128;
    p.rows += hq * b;
    p.tri += hq * b * (b + 1) / 2;
    p.rp += hq * b + 1;
    p.kvrows += hkv * b;
  }
  return p;
}
// the dense path of a sequence: N_b <= 2 (mu undefined) or shorter than the length gate
__host__ __device__ inline bool seq_dense(int nb, int dense_below_n) {
  return nb <= 2 || (dense_below_n > 0 && (int64_t)nb * 128 < dense_below_n);
}

// queue: the persistent kernel's work counters, zero at launch (set by the V re-layout).
// nb_total: blocks of the whole packed V^T (its head stride).
hipError_t launch_attention(int fp32, bool dense, const void* Q, const void* K, const void* Vt, void* O,
                            const int32_t* row_ptr, const int32_t* col_idx, int* queue, const SeqTable& seqs,
                            int nb_total, int hq, int hkv, const Strides& st, hipStream_t s);

// ---- proxy (proxy.hip)
// row-partial chunks per virtual head that stats holds (the most any sequence
// of the list is cut into by the score pass)
int proxy_chunks(int fp32, const SeqList& seqs, int hq, int hkv);
hipError_t launch_proxy(int fp32, const void* Q, const void* K, const SeqList& seqs, int nb_max, int hq, int hkv,
                        const Strides& st, int w_sink, int w_local, int dense_below_n,
                        void* tstat /*[rows*128] float4*/, void* stats /*[nseq*hq*nchunk*128] float2*/,
                        void* rowstat /*[nseq*hq*128] float2*/, void* tiles /*[rows] float4*/,
                        float* kbar /*[kvrows*128]*/, const VtJob& vt, hipStream_t s);

// compute units of the current device (cached per device)
int device_cu_count();

// ---- selection (select.hip)
struct PeCut;                       // per-head radix-select state (select.hip)
size_t pe_cut_state_bytes();
constexpr int PE_BUCKETS = 2048;    // histogram size of one radix pass
int row_tiles(int64_t rows);        // tiles of the row-pointer scan
// entries per Pooled-Estimation head kept by the last radix pass (those that
// share the cut's top 22 bits); a head with more falls back to a full read
inline int pe_cand_cap(int64_t nb_max) {
  const int64_t c = nb_max * (nb_max + 1) / 2 / 256;
  return (int)(c < 1024 ? 1024 : (c > 65536 ? 65536 : c));
}
// the capacity used: pe_cand_cap, or less where CRISP_PE_CAND_CAP asks for it
// (both paths give the same counts; a smaller value sends heads to the full read)
int pe_cand_limit(int64_t nb_max);

struct SelectBufs {
  // inputs from the proxy
  const void* tiles;
  const float* kbar;
  // scratch
  float *pv, *ps, *qbar;
  float* P;                         // [hq * N_b (N_b + 1) / 2] pooled logits of the PE heads (causal triangles)
  void* pnorm;                      // [hq * N_b] float2: (max, 1/sum) of each pooled row
  float* pe_prob;                   // optional caller output: the pooled probabilities, same layout as P
  int32_t *sv, *nv, *ss, *ns;
  uint32_t* hcnt;  unsigned long long* hmass;  void* cut;
  int32_t *eqrow, *counts;
  void* cand;                       // [vh * pe_cand_cap(nb_max)] uint2: (packed row, value bits) of cut candidates
  void* pepart;                     // [hq * nb * nseg] float2: per-segment row max / sum of the pooled logits
  int* peq;                         // work counter of the pooled-logits kernel
  int32_t* rtsum;                   // [nseq * row_tiles(hq * nb_max)]: sums of tiles of row counts
  // caller outputs
  int32_t* route; float* c_struct; int32_t *row_ptr, *col_idx;
  float *pv_out, *ps_out; int32_t *sv_out, *nv_out, *ss_out, *ns_out;
  // variants: router 0 = C_struct, 1 = JSD; vs_budget 0 = mean floor, 1 = median floor, 2 = coverage
  double* jsd; float* abar;
  int router, vs_budget;
};

// nb_max: the longest sequence's N_b (grid extents, per-head scratch sizes).
// vt: the V re-layout of a bf16 prefill, done here when every sequence is on
// the dense path (the proxy launch, which does it otherwise, is then skipped).
hipError_t launch_select(int fp32, const void* Q, const SeqList& seqs, int nb_max, int hq, int hkv,
                         const Strides& st, int w_sink, int w_local, float tau, float alpha, float gamma,
                         int min_blocks, int dense_below_n, const SelectBufs& b, const VtJob& vt, hipStream_t s);

}  // namespace crisp
