// C ABI of libcrisp: argument validation, workspace planning and launch
// sequencing.  Everything here runs on the host; nothing allocates, nothing
// synchronises, and every check happens before the first launch.
#include "../../include/crisp.h"

#include <math.h>
#include <string.h>

#include <mutex>

#include "launch.h"

using namespace crisp;

// Workspace of crisp_prefill_noalloc: a fixed device array, one copy per GPU,
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host it names a stand-in, not device memory): it looks up the
// array's device address once per device and passes that.
static __device__ __align__(256) char scratch[CRISP_NOALLOC_SCRATCH_BYTES];

int crisp::device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

namespace {
constexpr int BLK = 128;   // block size b: pooling, selection and attention tile edge
constexpr int HD = 128;    // head dim d
}  // namespace

namespace {

constexpr int64_t MAX_NB = 32768;
// largest token stride (elements): a 128-row K tile then spans under 2^31 bytes, the range of
// the attention kernel's buffer resources and tile offsets
constexpr int64_t MAX_TOKEN_STRIDE = int64_t(1) << 22;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int check_shape(const crisp_shape* s) {
  if (!s) return CRISP_E_ARG;
  if (s->dtype != CRISP_BF16 && s->dtype != CRISP_FP32) return CRISP_E_UNSUPPORTED;
  if (s->d != HD) return CRISP_E_UNSUPPORTED;
  if (s->n <= 0 || s->n % BLK) return CRISP_E_ARG;
  if (s->n / BLK > MAX_NB) return CRISP_E_UNSUPPORTED;
  if (s->hq <= 0 || s->hkv <= 0 || s->hq % s->hkv) return CRISP_E_ARG;
  const int64_t st[8] = {s->sq_h, s->sq_n, s->sk_h, s->sk_n, s->sv_h, s->sv_n, s->so_h, s->so_n};
  for (int64_t x : st)
    if (x < 0 || x % 8) return CRISP_E_ARG;
  if (s->sq_n < HD || s->sk_n < HD || s->sv_n < HD || s->so_n < HD) return CRISP_E_ARG;
  if (s->sq_n > MAX_TOKEN_STRIDE || s->sk_n > MAX_TOKEN_STRIDE || s->sv_n > MAX_TOKEN_STRIDE ||
      s->so_n > MAX_TOKEN_STRIDE)
    return CRISP_E_UNSUPPORTED;
  // worst-case list size must fit int32 row pointers
  const int64_t nb = s->n / BLK;
  if ((int64_t)s->hq * nb * (nb + 1) / 2 > 0x7fffffffLL) return CRISP_E_UNSUPPORTED;
  return CRISP_OK;
}

int check_params(const crisp_shape* s, const crisp_params* p) {
  if (!p) return CRISP_E_ARG;
  if (p->block != BLK) return CRISP_E_UNSUPPORTED;
  if (p->sink < 0 || p->local < 0 || p->sink > s->n || p->local > s->n) return CRISP_E_ARG;
  if (!(p->tau >= 0.f) || !(p->alpha >= 0.f) || !isfinite(p->tau) || !isfinite(p->alpha)) return CRISP_E_ARG;
  if (!(p->gamma > 0.f) || !(p->gamma <= 1.f)) return CRISP_E_ARG;
  if (p->min_blocks < 0 || p->dense_below_n < 0) return CRISP_E_ARG;
  const int known = CRISP_FLAG_ROUTE_JSD | CRISP_FLAG_VS_MEDIAN | CRISP_FLAG_VS_COVERAGE;
  if (p->flags & ~known) return CRISP_E_ARG;
  if ((p->flags & CRISP_FLAG_VS_MEDIAN) && (p->flags & CRISP_FLAG_VS_COVERAGE)) return CRISP_E_ARG;
  return CRISP_OK;
}

Strides strides(const crisp_shape* s) {
  return Strides{s->sq_h, s->sq_n, s->sk_h, s->sk_n, s->sv_h, s->sv_n, s->so_h, s->so_n};
}

int64_t tri(int64_t nb) { return nb * (nb + 1) / 2; }

// Selection workspace layout (every region 256-byte aligned).
struct SelectLayout {
  size_t tstat, stats, rowstat, tiles, pv, ps, sv, ss, nv, ns, kbar, qbar, P, hcnt, hmass, cut, eqrow, counts, jsd, abar,
      cand, pnorm, pepart, peq, rtsum, total;
};

SeqList one_sequence(const crisp_shape* s) {
  SeqList L;
  L.nseq = 1;
  L.nb[0] = (int)(s->n / BLK);
  return L;
}

// Packed per-row arrays hold every sequence's hq * N_b rows; per-head scratch
// of fixed size is indexed by virtual head (sequence, query head) and sized
// for the longest sequence.
SelectLayout select_layout(const crisp_shape* s, const SeqList& seqs) {
  const int64_t hq = s->hq, hkv = s->hkv, vh = seqs.nseq * hq;
  int64_t rows = 0, kvrows = 0, tris = 0, nb_max = 0;
  for (int i = 0; i < seqs.nseq; ++i) {
    const int64_t nb = seqs.nb[i];
    rows += hq * nb;
    kvrows += hkv * nb;
    tris += hq * tri(nb);
    if (nb > nb_max) nb_max = nb;
  }
  const int64_t nch = proxy_chunks(s->dtype == CRISP_FP32, seqs, (int)hq, (int)hkv);
  const int64_t nseg = pe_segments_max(seqs);
  SelectLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.tstat = take(rows * BLK * 16);
  L.stats = take(vh * nch * BLK * 8);
  L.rowstat = take(vh * BLK * 8);
  L.tiles = take(rows * 16);
  L.pv = take(rows * 4);
  L.ps = take(rows * 4);
  L.sv = take(rows * 4);
  L.ss = take(rows * 4);
  L.nv = take(vh * 4);
  L.ns = take(vh * 4);
  L.kbar = take(kvrows * HD * 4);
  L.qbar = take(rows * HD * 4);
  L.P = take(tris * 4);
  L.hcnt = take(vh * 3 * PE_BUCKETS * 4);
  L.hmass = take(vh * 3 * PE_BUCKETS * 8);
  L.cut = take(vh * pe_cut_state_bytes());
  L.eqrow = take(rows * 4);
  L.counts = take(rows * 4);
  L.cand = take((size_t)vh * pe_cand_cap(nb_max) * 8);
  L.pnorm = take(rows * 8);
  L.jsd = take(vh * 8);
  L.abar = take(rows * 4);
  L.pepart = take(rows * nseg * 8);
  L.peq = take(sizeof(int));
  L.rtsum = take((size_t)seqs.nseq * row_tiles(hq * nb_max) * 4);
  L.total = o;
  return L;
}
SelectLayout select_layout(const crisp_shape* s) { return select_layout(s, one_sequence(s)); }

// Attention workspace: re-laid-out V^T, then the work-queue counter.
size_t vt_bytes(const crisp_shape* s) {
  const size_t esz = s->dtype == CRISP_FP32 ? 4 : 2;
  return align256((size_t)s->hkv * (size_t)s->n * HD * esz);
}
size_t attn_ws(const crisp_shape* s) { return vt_bytes(s) + 256; }


int status_of(hipError_t e) { return e == hipSuccess ? CRISP_OK : CRISP_E_HIP; }

int check_qkv(const crisp_shape* s, const void* q, const void* k, const void* v, const void* o) {
  if (!q || !k || !aligned16(q) || !aligned16(k)) return CRISP_E_ARG;
  if (v && !aligned16(v)) return CRISP_E_ARG;
  if (o && !aligned16(o)) return CRISP_E_ARG;
  (void)s;
  return CRISP_OK;
}

int validate_select(const crisp_shape* s, const void* q, const void* k, const crisp_params* p,
                    const crisp_selection* out, const void* ws, size_t ws_bytes) {
  int st = check_shape(s);
  if (st) return st;
  if ((st = check_params(s, p))) return st;
  if ((st = check_qkv(s, q, k, nullptr, nullptr))) return st;
  if (!out || !out->route || !out->c_struct || !out->row_ptr || !out->col_idx) return CRISP_E_ARG;
  if (out->col_capacity < crisp_col_capacity(s)) return CRISP_E_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255)) return CRISP_E_ARG;
  if (ws_bytes < select_layout(s).total) return CRISP_E_WORKSPACE;
  return CRISP_OK;
}

int validate_attn(const crisp_shape* s, const void* q, const void* k, const void* v, void* o, const void* ws,
                  size_t ws_bytes) {
  int st = check_shape(s);
  if (st) return st;
  if (!v || !o) return CRISP_E_ARG;
  if ((st = check_qkv(s, q, k, v, o))) return st;
  if (!ws || ((uintptr_t)ws & 255)) return CRISP_E_ARG;
  if (ws_bytes < attn_ws(s)) return CRISP_E_WORKSPACE;
  return CRISP_OK;
}

// Selection of every sequence in `seqs` (one prefill: one sequence), all at once.
int run_select(const crisp_shape* s, const void* q, const void* k, const crisp_params* p, crisp_selection* out,
               void* ws, hipStream_t stream, const SeqList& seqs, const VtJob& vt = VtJob{}) {
  const SelectLayout L = select_layout(s, seqs);
  char* w = (char*)ws;
  int nb_max = 0;
  for (int i = 0; i < seqs.nseq; ++i) nb_max = seqs.nb[i] > nb_max ? seqs.nb[i] : nb_max;
  const int fp32 = s->dtype == CRISP_FP32;
  const Strides st = strides(s);
  hipError_t e = launch_proxy(fp32, q, k, seqs, nb_max, s->hq, s->hkv, st, p->sink, p->local, p->dense_below_n,
                              w + L.tstat, w + L.stats, w + L.rowstat, w + L.tiles, (float*)(w + L.kbar), vt, stream);
  if (e != hipSuccess) return CRISP_E_HIP;
  SelectBufs b;
  b.tiles = w + L.tiles;
  b.kbar = (const float*)(w + L.kbar);
  b.pv = (float*)(w + L.pv);
  b.ps = (float*)(w + L.ps);
  b.qbar = (float*)(w + L.qbar);
  b.P = (float*)(w + L.P);
  b.pnorm = w + L.pnorm;
  b.pe_prob = out->pe_prob;
  b.sv = (int32_t*)(w + L.sv);
  b.nv = (int32_t*)(w + L.nv);
  b.ss = (int32_t*)(w + L.ss);
  b.ns = (int32_t*)(w + L.ns);
  b.hcnt = (uint32_t*)(w + L.hcnt);
  b.hmass = (unsigned long long*)(w + L.hmass);
  b.cut = w + L.cut;
  b.eqrow = (int32_t*)(w + L.eqrow);
  b.counts = (int32_t*)(w + L.counts);
  b.cand = w + L.cand;
  b.pepart = w + L.pepart;
  b.peq = (int*)(w + L.peq);
  b.rtsum = (int32_t*)(w + L.rtsum);
  b.route = out->route;
  b.c_struct = out->c_struct;
  b.row_ptr = out->row_ptr;
  b.col_idx = out->col_idx;
  b.pv_out = out->pv;
  b.ps_out = out->ps;
  b.sv_out = out->sv;
  b.nv_out = out->nv;
  b.ss_out = out->ss;
  b.ns_out = out->ns;
  b.jsd = out->jsd ? out->jsd : (double*)(w + L.jsd);
  b.abar = out->abar ? out->abar : (float*)(w + L.abar);
  b.router = (p->flags & CRISP_FLAG_ROUTE_JSD) ? 1 : 0;
  b.vs_budget = (p->flags & CRISP_FLAG_VS_MEDIAN) ? 1 : ((p->flags & CRISP_FLAG_VS_COVERAGE) ? 2 : 0);
  return status_of(launch_select(fp32, q, seqs, nb_max, s->hq, s->hkv, st, p->sink, p->local, p->tau, p->alpha,
                                 p->gamma, p->min_blocks, p->dense_below_n, b, vt, stream));
}
int run_select(const crisp_shape* s, const void* q, const void* k, const crisp_params* p, crisp_selection* out,
               void* ws, hipStream_t stream, const VtJob& vt = VtJob{}) {
  return run_select(s, q, k, p, out, ws, stream, one_sequence(s), vt);
}

// The V re-layout of a bf16 prefill, done by the proxy launch (the fp32 path
// keeps its own re-layout launch): V^T at the start of the attention
// workspace, the attention's work counters right after it.
VtJob prefill_vt_job(const crisp_shape* s, const void* v, void* attn_ws) {
  VtJob j;
  if (s->dtype != CRISP_BF16) return j;
  j.V = v;
  j.Vt = attn_ws;
  j.sv_h = s->sv_h;
  j.sv_n = s->sv_n;
  j.nb = (int)(s->n / BLK);
  j.queue = (int*)((char*)attn_ws + vt_bytes(s));
  return j;
}

SeqTable single_sequence(int nb, int hkv) {
  SeqTable t;
  t.nseq = 1;
  t.pair_major = 0;
  t.unit_off[0] = 0;
  t.unit_off[1] = ((nb + 1) / 2) * hkv;
  t.nb[0] = nb;
  t.tok[0] = 0;
  t.rp[0] = 0;
  t.col[0] = 0;
  return t;
}

// A single sequence on the dense path (below the length gate, or N_b <= 2):
// its selection is every causal block, so the prefill runs the dense kernel,
// which gives the same output as the sparse kernel on those lists without
// reading them.
bool gated_dense(const crisp_shape* s, const crisp_params* p) { return seq_dense((int)(s->n / BLK), p->dense_below_n); }

// vt_ready: the proxy launch of the same prefill has already re-laid out V
// (prefill_vt_job) and cleared the work counters.
int run_attn(const crisp_shape* s, const void* q, const void* k, const void* v, const int32_t* row_ptr,
             const int32_t* col_idx, bool dense, void* o, void* ws, hipStream_t stream, const SeqTable* seqs = nullptr,
             bool vt_ready = false) {
  const int nb = (int)(s->n / BLK);
  const int fp32 = s->dtype == CRISP_FP32;
  int* queue = (int*)((char*)ws + vt_bytes(s));
  if (!vt_ready) {
    const hipError_t e = launch_transpose_v(fp32, v, ws, nb, s->hkv, s->sv_h, s->sv_n, queue, stream);
    if (e != hipSuccess) return CRISP_E_HIP;
  }
  const SeqTable one = single_sequence(nb, s->hkv);
  return status_of(launch_attention(fp32, dense, q, k, ws, o, row_ptr, col_idx, queue, seqs ? *seqs : one, nb,
                                    s->hq, s->hkv, strides(s), stream));
}

// ---- allocation-free prefill

std::mutex scratch_mu;
void* scratch_dev[64];   // device address of `scratch` per device, looked up on first use

// Device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CRISP_E_HIP;
  if (dev < 0 || dev >= 64) return CRISP_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CRISP_E_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return CRISP_OK;
}

// ---- packed batches (varlen)

struct VarlenPlan {
  int nseq;
  int64_t len[MAX_SEQ], tok[MAX_SEQ];
  int64_t rows_before[MAX_SEQ];   // hq * nb of the earlier sequences (diagnostic arrays)
  int64_t rp_before[MAX_SEQ];     // row_ptr entries of the earlier sequences (hq * nb + 1 each)
  int64_t col_before[MAX_SEQ];    // list capacity of the earlier sequences (hq * nb(nb+1)/2 each)
  int64_t col_total;
  SeqList seqs;
  size_t sel_ws;                  // selection workspace of the whole batch
};

crisp_shape sub_shape(const crisp_shape* s, int64_t len) {
  crisp_shape t = *s;
  t.n = len;
  return t;
}

int plan_varlen(const crisp_shape* s, int32_t nseq, const int64_t* cu, const crisp_params* p, VarlenPlan* P) {
  int st = check_shape(s);
  if (st) return st;
  if (nseq < 1 || !cu) return CRISP_E_ARG;
  if (nseq > MAX_SEQ) return CRISP_E_UNSUPPORTED;
  if (cu[0] != 0 || cu[nseq] != s->n) return CRISP_E_ARG;
  P->nseq = nseq;
  int64_t rows = 0, rp = 0, col = 0;
  for (int i = 0; i < nseq; ++i) {
    const int64_t len = cu[i + 1] - cu[i];
    if (len <= 0 || len % BLK) return CRISP_E_ARG;
    const crisp_shape t = sub_shape(s, len);
    if ((st = check_shape(&t))) return st;
    if (p && (st = check_params(&t, p))) return st;
    const int64_t nb = len / BLK;
    P->len[i] = len;
    P->tok[i] = cu[i];
    P->rows_before[i] = rows;
    P->rp_before[i] = rp;
    P->col_before[i] = col;
    rows += s->hq * nb;
    rp += s->hq * nb + 1;
    col += s->hq * tri(nb);
    P->seqs.nb[i] = (int)nb;
  }
  P->col_total = col;
  P->seqs.nseq = nseq;
  P->sel_ws = select_layout(s, P->seqs).total;
  return CRISP_OK;
}

}  // namespace

extern "C" {

size_t crisp_select_workspace_bytes(const crisp_shape* shape, const crisp_params* params) {
  if (check_shape(shape) || check_params(shape, params)) return 0;
  return select_layout(shape).total;
}

size_t crisp_attn_workspace_bytes(const crisp_shape* shape) {
  if (check_shape(shape)) return 0;
  return attn_ws(shape);
}

size_t crisp_workspace_bytes(const crisp_shape* shape, const crisp_params* params) {
  if (check_shape(shape) || check_params(shape, params)) return 0;
  return select_layout(shape).total + attn_ws(shape);
}

int64_t crisp_col_capacity(const crisp_shape* shape) {
  if (check_shape(shape)) return 0;
  return (int64_t)shape->hq * tri(shape->n / BLK);
}

int crisp_select(const crisp_shape* shape, const void* q, const void* k, const crisp_params* params,
                 crisp_selection* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = validate_select(shape, q, k, params, out, workspace, workspace_bytes);
  if (st) return st;
  return run_select(shape, q, k, params, out, workspace, stream);
}

int crisp_sparse_attn(const crisp_shape* shape, const void* q, const void* k, const void* v,
                      const crisp_selection* sel, void* o, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  const int st = validate_attn(shape, q, k, v, o, workspace, workspace_bytes);
  if (st) return st;
  if (!sel || !sel->row_ptr || !sel->col_idx) return CRISP_E_ARG;
  return run_attn(shape, q, k, v, sel->row_ptr, sel->col_idx, false, o, workspace, stream);
}

int crisp_dense_attn(const crisp_shape* shape, const void* q, const void* k, const void* v, void* o,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = validate_attn(shape, q, k, v, o, workspace, workspace_bytes);
  if (st) return st;
  return run_attn(shape, q, k, v, nullptr, nullptr, true, o, workspace, stream);
}

int crisp_prefill(const crisp_shape* shape, const void* q, const void* k, const void* v,
                  const crisp_params* params, crisp_selection* sel, void* o, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const size_t sel_bytes = crisp_select_workspace_bytes(shape, params);
  if (!sel_bytes) return check_params(shape, params) ? check_params(shape, params) : CRISP_E_ARG;
  if (workspace_bytes < sel_bytes + attn_ws(shape)) return CRISP_E_WORKSPACE;
  st = validate_select(shape, q, k, params, sel, workspace, sel_bytes);
  if (st) return st;
  char* attn_ws_ptr = (char*)workspace + sel_bytes;
  st = validate_attn(shape, q, k, v, o, attn_ws_ptr, workspace_bytes - sel_bytes);
  if (st) return st;
  const VtJob vt = prefill_vt_job(shape, v, attn_ws_ptr);
  st = run_select(shape, q, k, params, sel, workspace, stream, vt);
  if (st) return st;
  return run_attn(shape, q, k, v, sel->row_ptr, sel->col_idx, gated_dense(shape, params), o, attn_ws_ptr, stream,
                  nullptr, vt.V != nullptr);
}

size_t crisp_noalloc_scratch_bytes(void) { return CRISP_NOALLOC_SCRATCH_BYTES; }

int crisp_prefill_noalloc(const crisp_shape* shape, const void* q, const void* k, const void* v,
                          const crisp_params* params, crisp_selection* sel, void* o, hipStream_t stream) {
  // every check before the first HIP call
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_params(shape, params))) return st;
  const size_t sel_bytes = select_layout(shape).total;
  if (sel_bytes + attn_ws(shape) > CRISP_NOALLOC_SCRATCH_BYTES) return CRISP_E_TOO_LARGE;
  if (!v || !o) return CRISP_E_ARG;
  if ((st = check_qkv(shape, q, k, v, o))) return st;
  if (!sel || !sel->route || !sel->c_struct || !sel->row_ptr || !sel->col_idx) return CRISP_E_ARG;
  if (sel->col_capacity < crisp_col_capacity(shape)) return CRISP_E_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  const VtJob vt = prefill_vt_job(shape, v, (char*)ws + sel_bytes);
  st = run_select(shape, q, k, params, sel, ws, stream, vt);
  if (st) return st;
  return run_attn(shape, q, k, v, sel->row_ptr, sel->col_idx, gated_dense(shape, params), o, (char*)ws + sel_bytes,
                  stream, nullptr, vt.V != nullptr);
}

int64_t crisp_varlen_col_capacity(const crisp_shape* shape, int32_t nseq, const int64_t* cu_seqlens) {
  VarlenPlan P;
  if (plan_varlen(shape, nseq, cu_seqlens, nullptr, &P)) return 0;
  return P.col_total;
}

size_t crisp_varlen_workspace_bytes(const crisp_shape* shape, int32_t nseq, const int64_t* cu_seqlens,
                                    const crisp_params* params) {
  VarlenPlan P;
  if (!params || plan_varlen(shape, nseq, cu_seqlens, params, &P)) return 0;
  return align256(P.sel_ws) + attn_ws(shape);
}

int crisp_prefill_varlen(const crisp_shape* shape, int32_t nseq, const int64_t* cu_seqlens, const void* q,
                         const void* k, const void* v, const crisp_params* params, crisp_selection* sel, void* o,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  VarlenPlan P;
  if (!params) return CRISP_E_ARG;
  int st = plan_varlen(shape, nseq, cu_seqlens, params, &P);
  if (st) return st;
  if (!sel || !sel->route || !sel->c_struct || !sel->row_ptr || !sel->col_idx) return CRISP_E_ARG;
  if (sel->col_capacity < P.col_total) return CRISP_E_WORKSPACE;
  if ((st = check_qkv(shape, q, k, v, o))) return st;
  if (!v || !o || !workspace || ((uintptr_t)workspace & 255)) return CRISP_E_ARG;
  const size_t sel_bytes = align256(P.sel_ws);
  if (workspace_bytes < sel_bytes + attn_ws(shape)) return CRISP_E_WORKSPACE;
  // selection of every sequence at once (virtual heads = sequence x query head)
  const VtJob vt = prefill_vt_job(shape, v, (char*)workspace + sel_bytes);
  st = run_select(shape, q, k, params, sel, workspace, stream, P.seqs, vt);
  if (st) return st;
  SeqTable seqs;
  seqs.nseq = nseq;
  seqs.pair_major = 0;
  seqs.unit_off[0] = 0;
  for (int i = 0; i < nseq; ++i) {
    const int64_t nb = P.len[i] / BLK;
    seqs.nb[i] = (int)nb;
    seqs.tok[i] = P.tok[i];
    seqs.rp[i] = P.rp_before[i];
    seqs.col[i] = P.col_before[i];
    seqs.unit_off[i + 1] = seqs.unit_off[i] + (int)((nb + 1) / 2) * shape->hkv;
  }
  return run_attn(shape, q, k, v, sel->row_ptr, sel->col_idx, false, o, (char*)workspace + sel_bytes, stream,
                  &seqs, vt.V != nullptr);
}

const char* crisp_status_string(int status) {
  switch (status) {
    case CRISP_OK: return "ok";
    case CRISP_E_ARG: return "invalid argument";
    case CRISP_E_UNSUPPORTED: return "unsupported shape or dtype";
    case CRISP_E_WORKSPACE: return "workspace or list capacity too small";
    case CRISP_E_HIP: return "kernel launch failed";
    case CRISP_E_TOO_LARGE: return "problem needs more workspace than the allocation-free entry point's fixed scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
