// Routing and index selection (gfx950).
//
//  vs_select   per head: p^v, p^s from the proxy tile sums, C_struct, route
//              (VS iff C_struct >= tau) [CRISP §3.2]; for VS heads the noise
//              floor mu_d = max(1 - p_0 - p_last, 0)/(N_b - 2) and the sets
//              S_d = {k : p_k > alpha mu_d} U {0, N_b - 1} per direction
//              [CRISP §4], compacted in ascending order; optional min budget.
//  pool_q      block means of Q for Pooled-Estimation heads.
//  pe_logits   pooled logits Qbar[qb] . Kbar[kb] / sqrt(d), kb <= qb (fp32
//              MFMA), with per-segment row max / sum;
//  pe_norm     the causal row softmax in one pass [CRISP §2, PE path].
//  pe_hist/    global gamma-cut over the flattened causal matrix: a radix
//  pe_scan     select on the float32 bit pattern (11+11+10 bits, three
//              passes) with per-bucket mass in 2^-46 fixed point, so the sums
//              are exact integers and order-independent.  Entries are taken in
//              descending value, ties by ascending row-major flat index,
//              until the mass reaches gamma * total.
//  list_*      per (head, query block) ascending key-block lists in one CSR:
//              VS rows = {S_v <= qb} U {qb - S_s} U {0, qb}, PE rows = the
//              selected entries of the row plus (qb, 0) and (qb, qb), dense
//              rows = 0..qb.
//
// Variants the pages compare against (selected by flags):
//  jsd_route   FlexPrefill's router [CRISP §2]: pooled estimate a_bar =
//              softmax over key blocks of mean(Q_last) . Kbar / sqrt(d), and
//              JSD(a_bar, p^v) in float64; Vertical-Slash iff JSD >= tau.
//  vs_rank     per (head, direction) of a Vertical-Slash head: the median
//              noise floor [CRISP appendix on the floor] or FlexPrefill's
//              coverage budget (descending scores until gamma of the mass)
//              [CRISP §2], both by radix selection on the float32 bits.
//
// The decision arithmetic (route, mu, threshold) is written with explicit
// round-to-nearest float32 operations in a fixed order so that it can be
// reproduced exactly on the host from the same float32 scores.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "lanes.h"
#include "launch.h"

namespace crisp {

struct PeCut {
  unsigned long long total, target, need, above_mass, take, eq_cnt;
  uint32_t prefix, vstar;
  int32_t active;
  int32_t pad;
};
size_t pe_cut_state_bytes() { return sizeof(PeCut); }

constexpr double FX_SCALE = 70368744177664.0;  // 2^46
__device__ __forceinline__ unsigned long long fx_mass(uint32_t bits) {
  return (unsigned long long)((double)__uint_as_float(bits) * FX_SCALE);
}

// ------------------------------------------------------------------ block helpers (256 threads)

__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int x = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

// ------------------------------------------------------------------ VS selection

__device__ void compact_flags(const uint8_t* flag, int nb, int32_t* out, int* count, int* sh) {
  const int tid = threadIdx.x;
  const int per = (nb + 255) / 256;
  const int a = min(nb, tid * per), b = min(nb, a + per);
  int c = 0;
  for (int k = a; k < b; ++k) c += flag[k];
  int tot;
  int pos = block_excl_scan(c, sh, &tot);
  for (int k = a; k < b; ++k)
    if (flag[k]) out[pos++] = k;
  if (tid == 0) *count = tot;
  __syncthreads();
}

// top up the set to `want` members with the largest remaining scores, ties to the lower index
__device__ void top_up(uint8_t* flag, const float* p, int nb, int want, float* shv, int* shi) {
  const int tid = threadIdx.x;
  int have = 0;
  for (int k = tid; k < nb; k += 256) have += flag[k];
  shi[tid] = have;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) shi[tid] += shi[tid + o];
    __syncthreads();
  }
  have = shi[0];
  __syncthreads();
  for (; have < want; ++have) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int k = tid; k < nb; k += 256)
      if (!flag[k] && (p[k] > bv || (p[k] == bv && k < bi))) { bv = p[k]; bi = k; }
    shv[tid] = bv;
    shi[tid] = bi;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) {
        const float v2 = shv[tid + o];
        const int i2 = shi[tid + o];
        if (v2 > shv[tid] || (v2 == shv[tid] && i2 < shi[tid])) { shv[tid] = v2; shi[tid] = i2; }
      }
      __syncthreads();
    }
    if (tid == 0 && shi[0] < nb) flag[shi[0]] = 1;
    __syncthreads();
  }
}

// One work-group per virtual head (sequence, query head).
__global__ __launch_bounds__(256) void vs_select_kernel(
    const float4* __restrict__ tiles, const SeqList seqs, int hq, int hkv, int w_sink, int w_local, float tau,
    float alpha, int min_blocks, int dense_below_n, const double* __restrict__ jsd, int vs_budget,
    int32_t* __restrict__ route, float* __restrict__ c_struct, float* __restrict__ pv, float* __restrict__ ps,
    int32_t* __restrict__ sv, int32_t* __restrict__ nv, int32_t* __restrict__ ss, int32_t* __restrict__ ns,
    float* pv_out, float* ps_out) {
  extern __shared__ uint8_t flag[];  // nb bytes
  __shared__ int shi[256];
  __shared__ float shv[256];
  __shared__ int s_route;
  const int h = blockIdx.x, tid = threadIdx.x;   // h: virtual head
  const SeqPos sp = seq_pos(seqs, h / hq, hq, hkv);
  const int nb = sp.nb;
  const int64_t n = (int64_t)nb * BLK, rowb = sp.rows + (int64_t)(h % hq) * nb;
  if (seq_dense(nb, dense_below_n)) {
    if (tid == 0) { route[h] = -1; c_struct[h] = 0.f; nv[h] = 0; ns[h] = 0; }
    return;
  }
  const float4* T = tiles + rowb;
  float* PV = pv + rowb;
  float* PS = ps + rowb;
  const float inv_b = 1.f / BLK;  // exact power of two
  for (int k = tid; k < nb; k += 256) {
    const float4 t = T[k];
    const float v = __fmul_rn(__fadd_rn(t.x, t.y), inv_b);
    const float lo = T[nb - 1 - k].x;
    const float up = (k <= nb - 2) ? T[nb - 2 - k].y : 0.f;
    const float sl = __fmul_rn(__fadd_rn(lo, up), inv_b);
    PV[k] = v;
    PS[k] = sl;
    if (pv_out) pv_out[rowb + k] = v;
    if (ps_out) ps_out[rowb + k] = sl;
  }
  if (tid == 0) {
    // tiles touching [0, w_sink) or [n - w_local, n), ascending: the sink tiles,
    // then the recency tiles not already counted
    float c = 0.f;
    const int sink_end = (int)min<int64_t>(nb, (w_sink + BLK - 1) / BLK);
    const int rec_begin = (int)max<int64_t>(sink_end, (n - w_local) / BLK);
    for (int kb = 0; kb < sink_end; ++kb) c = __fadd_rn(c, T[kb].z);
    for (int kb = rec_begin; kb < nb; ++kb) {
      const int64_t j0 = (int64_t)kb * BLK;
      if (j0 + BLK > n - w_local) c = __fadd_rn(c, T[kb].z);
    }
    c = __fmul_rn(c, inv_b);
    c_struct[h] = c;
    // jsd != NULL: FlexPrefill's router on the float64 divergence
    const int r = (jsd ? (jsd[h] >= (double)tau) : (c >= tau)) ? 1 : 0;
    route[h] = r;
    s_route = r;
  }
  __syncthreads();
  if (s_route != 1 || vs_budget != 0) {   // other budgets: vs_rank_kernel writes the sets
    if (tid == 0) { nv[h] = 0; ns[h] = 0; }
    return;
  }
  const float denom = (float)(nb - 2);
  for (int dir = 0; dir < 2; ++dir) {
    const float* p = dir == 0 ? PV : PS;
    float t = __fsub_rn(1.f, p[0]);
    t = __fsub_rn(t, p[nb - 1]);
    t = fmaxf(t, 0.f);
    const float mu = __fdiv_rn(t, denom);
    const float thr = __fmul_rn(alpha, mu);
    for (int k = tid; k < nb; k += 256) flag[k] = (p[k] > thr) || k == 0 || k == nb - 1;
    __syncthreads();
    if (min_blocks > 0) top_up(flag, p, nb, min(min_blocks, nb), shv, shi);
    compact_flags(flag, nb, (dir == 0 ? sv : ss) + rowb, (dir == 0 ? nv : ns) + h, shi);
  }
}

// ------------------------------------------------------------------ variant: JSD router

__device__ float block256_max(float v, float* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) sh[tid] = fmaxf(sh[tid], sh[tid + o]);
    __syncthreads();
  }
  const float r = sh[0];
  __syncthreads();
  return r;
}

template <typename V>
__device__ V block256_sum(V v, V* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) sh[tid] += sh[tid + o];
    __syncthreads();
  }
  const V r = sh[0];
  __syncthreads();
  return r;
}

// One work-group per query head.  a_bar[kb] = softmax_kb(scale * qm . Kbar[kb]),
// qm = mean of the head's last 128 query rows; p^v[kb] = (lower + upper)/b from
// the proxy tile sums, exactly as vs_select forms it; then
// JSD = (KL(a_bar || m) + KL(p^v || m)) / 2, m = (a_bar + p^v)/2, in float64
// with natural logarithms, terms of zero weight dropped.
template <typename T>
__global__ __launch_bounds__(256) void jsd_route_kernel(const T* __restrict__ Q, const float4* __restrict__ tiles,
                                                        const float* __restrict__ kbar, float* __restrict__ abar,
                                                        double* __restrict__ jsd, const SeqList seqs, int hq,
                                                        int hkv, int64_t sq_h, int64_t sq_n, int dense_below_n,
                                                        float scale) {
  __shared__ float qm[HD];
  __shared__ float red[2][HD];
  __shared__ float shf[256];
  __shared__ double shd[256];
  const int vh = blockIdx.x, tid = threadIdx.x;
  const int h = vh % hq;
  const int kvh = h / (hq / hkv);
  const SeqPos sp = seq_pos(seqs, vh / hq, hq, hkv);
  const int nb = sp.nb;
  if (seq_dense(nb, dense_below_n)) {
    if (tid == 0) jsd[vh] = 0.0;
    return;
  }
  Q += sp.tok * sq_n;
  tiles += sp.rows;
  kbar += sp.kvrows * HD;
  abar += sp.rows;
  {
    const int d = tid & (HD - 1), half = tid >> 7;
    const T* base = Q + (int64_t)h * sq_h + ((int64_t)(nb - 1) * BLK + 64 * half) * sq_n + d;
    float sum = 0.f;
    for (int r = 0; r < 64; ++r) sum += to_f32(base[(int64_t)r * sq_n]);
    red[half][d] = sum;
    __syncthreads();
    if (half == 0) qm[d] = (red[0][d] + red[1][d]) * (1.f / BLK);
    __syncthreads();
  }
  float* A = abar + (int64_t)h * nb;
  const float* Kb = kbar + (int64_t)kvh * nb * HD;
  float mx = -INFINITY;
  for (int kb = tid; kb < nb; kb += 256) {
    const float* kr = Kb + (int64_t)kb * HD;
    float acc = 0.f;
    for (int d = 0; d < HD; ++d) acc = fmaf(qm[d], kr[d], acc);
    const float L = acc * scale;
    A[kb] = L;
    mx = fmaxf(mx, L);
  }
  mx = block256_max(mx, shf);
  float se = 0.f;
  for (int kb = tid; kb < nb; kb += 256) {
    const float e = expf(A[kb] - mx);
    A[kb] = e;
    se += e;
  }
  se = block256_sum(se, shf);
  const float4* Th = tiles + (int64_t)h * nb;
  double acc = 0.0;
  for (int kb = tid; kb < nb; kb += 256) {
    const float a = __fdiv_rn(A[kb], se);
    A[kb] = a;
    const float4 t = Th[kb];
    const float b = __fmul_rn(__fadd_rn(t.x, t.y), 1.f / BLK);
    const double m = 0.5 * ((double)a + (double)b);
    if (a > 0.f) acc += (double)a * log((double)a / m);
    if (b > 0.f) acc += (double)b * log((double)b / m);
  }
  acc = block256_sum(acc, shd);
  if (tid == 0) jsd[vh] = 0.5 * acc;
}

// ------------------------------------------------------------------ variant: median floor / coverage budget

// 1024-thread helpers
__device__ int block1k_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    for (int i = 0; i < 16; ++i) { const int x = sh[i]; sh[i] = a; a += x; }
    sh[16] = a;
  }
  __syncthreads();
  const int r = sh[w] + incl - v;
  *total = sh[16];
  __syncthreads();
  return r;
}

__device__ unsigned long long block1k_sum_u64(unsigned long long v, unsigned long long* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (tid < o) sh[tid] += sh[tid + o];
    __syncthreads();
  }
  const unsigned long long r = sh[0];
  __syncthreads();
  return r;
}

// Radix selection over the float32 bit patterns of p[lo, hi) (values >= 0, so
// bit order is value order), three passes of 11 / 11 / 10 bits from the top.
// BY_MASS = false: bits of the r-th largest value (r counted from 0).
// BY_MASS = true:  bits of the value at which the descending 2^-46 fixed-point
// prefix mass first reaches `need`; on return *above = mass of the larger
// values, *eq_cnt = number of entries equal to the result.
template <bool BY_MASS>
__device__ uint32_t radix_pick(const float* __restrict__ p, int lo, int hi, unsigned long long need,
                               uint32_t* cnt, unsigned long long* mass, unsigned long long* above,
                               uint32_t* eq_cnt) {
  __shared__ uint32_t s_prefix;
  __shared__ unsigned long long s_need, s_above;
  __shared__ uint32_t s_eq;
  const int tid = threadIdx.x;
  if (tid == 0) { s_prefix = 0; s_need = need; s_above = 0; }
  __syncthreads();
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int width = pass == 2 ? 10 : 11;
    const uint32_t mask = (1u << width) - 1;
    const int top = shift + width;
    for (int i = tid; i < PE_BUCKETS; i += 1024) { cnt[i] = 0; if (BY_MASS) mass[i] = 0; }
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int k = lo + tid; k < hi; k += 1024) {
      const uint32_t x = __float_as_uint(p[k]);
      if (pass > 0 && (x >> top) != (prefix >> top)) continue;
      const uint32_t b = (x >> shift) & mask;
      atomicAdd(&cnt[b], 1u);
      if (BY_MASS) atomicAdd(&mass[b], fx_mass(x));
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long acc = 0, nd = s_need;
      int sel = 0;
      for (int b = (int)mask; b >= 0; --b) {
        const unsigned long long v = BY_MASS ? mass[b] : (unsigned long long)cnt[b];
        if (BY_MASS ? (acc + v >= nd) : (acc + v > nd)) { sel = b; break; }
        acc += v;
        sel = b;
      }
      s_need = nd - acc;
      s_above += acc;
      s_prefix = prefix | ((uint32_t)sel << shift);
      s_eq = cnt[sel];
    }
    __syncthreads();
  }
  const uint32_t r = s_prefix;
  if (above) *above = s_above;
  if (eq_cnt) *eq_cnt = s_eq;
  __syncthreads();
  return r;
}

// One work-group (1024 threads) per (Vertical-Slash head, direction).
//   MEDIAN:   thr = alpha * median(p_1 .. p_{N_b-2}) (the mean of the two middle
//             values for an even count, (a + b) * 0.5 in float32); keep p_k > thr.
//   COVERAGE: keep the entries in descending order (ties to the lower index)
//             until their 2^-46 fixed-point mass reaches ceil(gamma * total),
//             the same arithmetic as the Pooled-Estimation cut; gamma >= 1 keeps all.
// Then the anchors 0 and N_b - 1, the optional min budget, ascending compaction.
template <bool MEDIAN>
__global__ __launch_bounds__(1024) void vs_rank_kernel(const int32_t* __restrict__ route, const float* __restrict__ pv,
                                                       const float* __restrict__ ps, const SeqList seqs, int hq,
                                                       int hkv, float alpha, float gamma, int min_blocks,
                                                       int32_t* __restrict__ sv, int32_t* __restrict__ nv,
                                                       int32_t* __restrict__ ss, int32_t* __restrict__ ns) {
  extern __shared__ uint8_t flag[];  // nb bytes
  // radix histograms; outside the radix passes the same memory serves the
  // block reductions (shi: 1024 ints over cnt, shv: 1024 floats over mass)
  __shared__ uint32_t cnt[PE_BUCKETS];
  __shared__ unsigned long long mass[PE_BUCKETS];
  int* shi = (int*)cnt;
  float* shv = (float*)mass;
  const int h = blockIdx.x, dir = blockIdx.y, tid = threadIdx.x;   // h: virtual head
  if (route[h] != 1) return;
  const SeqPos sp = seq_pos(seqs, h / hq, hq, hkv);
  const int nb = sp.nb;
  const int64_t rowb = sp.rows + (int64_t)(h % hq) * nb;
  const float* p = (dir == 0 ? pv : ps) + rowb;
  if (MEDIAN) {
    const int m = nb - 2;
    float med;
    if (m & 1) {
      med = __uint_as_float(radix_pick<false>(p, 1, nb - 1, (unsigned long long)((m - 1) / 2), cnt, mass,
                                              nullptr, nullptr));
    } else {
      const float a = __uint_as_float(radix_pick<false>(p, 1, nb - 1, (unsigned long long)(m / 2 - 1), cnt, mass,
                                                        nullptr, nullptr));
      const float b = __uint_as_float(radix_pick<false>(p, 1, nb - 1, (unsigned long long)(m / 2), cnt, mass,
                                                        nullptr, nullptr));
      med = __fmul_rn(__fadd_rn(a, b), 0.5f);
    }
    const float thr = __fmul_rn(alpha, med);
    for (int k = tid; k < nb; k += 1024) flag[k] = (p[k] > thr) || k == 0 || k == nb - 1;
    __syncthreads();
  } else if (gamma >= 1.f) {
    for (int k = tid; k < nb; k += 1024) flag[k] = 1;
    __syncthreads();
  } else {
    unsigned long long t = 0;
    for (int k = tid; k < nb; k += 1024) t += fx_mass(__float_as_uint(p[k]));
    t = block1k_sum_u64(t, mass);
    unsigned long long target = (unsigned long long)ceil((double)gamma * (double)t);
    if (target == 0) target = 1;
    unsigned long long above = 0;
    uint32_t eq_cnt = 0;
    const uint32_t vstar = radix_pick<true>(p, 0, nb, target, cnt, mass, &above, &eq_cnt);
    const unsigned long long need = target - above;
    const unsigned long long fv = fx_mass(vstar);
    unsigned long long take = fv ? (need + fv - 1) / fv : eq_cnt;
    if (take > eq_cnt) take = eq_cnt;
    // entries equal to the cut value are taken in index order: rank them with a scan
    const int per = (nb + 1023) / 1024;
    const int a = min(nb, tid * per), b = min(nb, a + per);
    int e = 0;
    for (int k = a; k < b; ++k) e += (__float_as_uint(p[k]) == vstar);
    int tot;
    int rank = block1k_excl_scan(e, shi, &tot);
    for (int k = a; k < b; ++k) {
      const uint32_t x = __float_as_uint(p[k]);
      bool sel = x > vstar || k == 0 || k == nb - 1;
      if (x == vstar) { if ((unsigned long long)rank < take) sel = true; ++rank; }
      flag[k] = sel;
    }
    __syncthreads();
  }
  if (min_blocks > 0) {  // top up with the largest remaining scores, ties to the lower index
    const int want = min(min_blocks, nb);
    int have = 0;
    for (int k = tid; k < nb; k += 1024) have += flag[k];
    int tot;
    block1k_excl_scan(have, shi, &tot);
    for (have = tot; have < want; ++have) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int k = tid; k < nb; k += 1024)
        if (!flag[k] && (p[k] > bv || (p[k] == bv && k < bi))) { bv = p[k]; bi = k; }
      shv[tid] = bv;
      shi[tid] = bi;
      __syncthreads();
      for (int o = 512; o > 0; o >>= 1) {
        if (tid < o) {
          const float v2 = shv[tid + o];
          const int i2 = shi[tid + o];
          if (v2 > shv[tid] || (v2 == shv[tid] && i2 < shi[tid])) { shv[tid] = v2; shi[tid] = i2; }
        }
        __syncthreads();
      }
      if (tid == 0 && shi[0] < nb) flag[shi[0]] = 1;
      __syncthreads();
    }
  }
  // ascending compaction
  const int per = (nb + 1023) / 1024;
  const int a = min(nb, tid * per), b = min(nb, a + per);
  int c = 0;
  for (int k = a; k < b; ++k) c += flag[k];
  int tot;
  int pos = block1k_excl_scan(c, shi, &tot);
  int32_t* out = (dir == 0 ? sv : ss) + rowb;
  for (int k = a; k < b; ++k)
    if (flag[k]) out[pos++] = k;
  if (tid == 0) (dir == 0 ? nv : ns)[h] = tot;
}

// ------------------------------------------------------------------ PE: pooled Q

template <typename T>
__global__ __launch_bounds__(256) void pool_q_kernel(const T* __restrict__ Q, const int32_t* __restrict__ route,
                                                     float* __restrict__ qbar, const SeqList seqs, int hq, int hkv,
                                                     int64_t sq_h, int64_t sq_n, int* __restrict__ queue) {
  constexpr int E = 16 / sizeof(T);         // elements per 16-byte load
  constexpr int CPR = HD / E;               // 16-byte chunks per row
  constexpr int RG = 256 / CPR;             // row groups
  __shared__ float red[RG][HD];
  const int qb = blockIdx.x, vh = blockIdx.y, tid = threadIdx.x;
  if (queue && qb == 0 && vh == 0 && tid == 0) *queue = 0;   // the logits kernel's work counter
  if (route[vh] != 0) return;
  const int h = vh % hq;
  const SeqPos sp = seq_pos(seqs, vh / hq, hq, hkv);
  const int nb = sp.nb;
  if (qb >= nb) return;
  const int ch = tid % CPR, rg = tid / CPR;
  const T* base = Q + (int64_t)h * sq_h + (sp.tok + (int64_t)qb * BLK) * sq_n + ch * E;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int r = rg; r < BLK; r += RG) {
    const T* p = base + (int64_t)r * sq_n;
    const uint4 raw = *(const uint4*)p;
    const T* v = (const T*)&raw;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += to_f32(v[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[rg][ch * E + e] = acc[e];
  __syncthreads();
  if (tid < HD) {
    float s = 0.f;
    for (int q = 0; q < RG; ++q) s += red[q][tid];
    qbar[(sp.rows + (int64_t)h * nb + qb) * HD + tid] = s * (1.f / BLK);
  }
}

// ------------------------------------------------------------------ PE: pooled probabilities

__device__ __forceinline__ int64_t tri(int64_t qb) { return qb * (qb + 1) / 2; }


constexpr int PE_RB = 4;     // 32-query-block row blocks (one wave each) per logits work-group

// e^x of the pooled softmax as v_exp_f32 (2^x) of x log2(e): relative error
// about |x| 2^-24 beyond the instruction's own, far below the probabilities'
// use (they are compared to 1e-5 and cut on their own float32 values).
__device__ __forceinline__ float pe_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
constexpr int KT_PITCH = 132; // LDS pitch (floats) of a key-block-mean row: conflict-free 16-byte reads

// Logits: one item per (PE_RB row blocks of 32 query blocks, segment cs of
// PE_SEG key tiles, Pooled-Estimation head); wave w owns row block rb0 + w.
// L[qb][kb] = scale * Qbar[qb] . Kbar[kb] for kb <= qb is formed 32 key blocks
// at a time with v_mfma_f32_32x32x2f32 in the transposed form L^T = Kbar Qbar^T
// (lane l owns query block 32 rb + l%32 and 16 of the 32 key blocks; the d
// index of MFMA step s, lane half g is 64 g + s).  The 32 key-block means of a
// tile are staged once in LDS (double-buffered, the next tile's copy in flight
// during the MFMAs) and shared by the work-group's waves.  Each tile is turned
// row-major through LDS and stored with whole 128-byte row segments; the
// segment's row max and sum of exp(L - max) go to `part` for the softmax.
// One item: row group rg_from_end counted from the bottom of the sequence's
// triangle (0 = the longest rows), segment cs, virtual head vh.
__device__ __forceinline__ void pe_logits_item(float (&kt)[2][32 * KT_PITCH], float (&tileT)[PE_RB][32][33],
                                               const float* __restrict__ qbar, const float* __restrict__ kbar,
                                               float* __restrict__ P, float2* __restrict__ part, const SeqList& seqs,
                                               int hq, int hkv, int nseg, float scale, int vh, int rg_from_end, int cs) {
  const int h = vh % hq;
  const SeqPos sp = seq_pos(seqs, vh / hq, hq, hkv);
  const int nb = sp.nb;
  const int nrb = (nb + 31) / 32, nrg = (nrb + PE_RB - 1) / PE_RB;
  const int rg = nrg - 1 - rg_from_end;
  if (rg < 0) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int rb = rg * PE_RB + w;
  // tiles this wave needs: key tiles 0 .. ntile - 1 of its row block (none past nb)
  const int ntile = rb < nrb ? min(nb - 1, rb * 32 + 31) / 32 + 1 : 0;
  const int rb_top = min(nrb - 1, rg * PE_RB + PE_RB - 1);
  const int ntile_top = min(nb - 1, rb_top * 32 + 31) / 32 + 1;
  const int ct0 = cs * PE_SEG, ct1 = min(ntile_top, ct0 + PE_SEG);
  if (ct0 >= ct1) return;
  qbar += sp.rows * HD;
  kbar += sp.kvrows * HD;
  P += sp.tri;
  part += sp.rows * nseg;
  const int kvh = h / (hq / hkv);
  const int qb = rb * 32 + l32;
  const bool row_ok = qb < nb;
  float qv[64];
  {
    const float4* src = (const float4*)(qbar + ((int64_t)h * nb + (row_ok ? qb : 0)) * HD + 64 * g);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 x = row_ok ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[4 * i] = x.x; qv[4 * i + 1] = x.y; qv[4 * i + 2] = x.z; qv[4 * i + 3] = x.w;
    }
  }
  float* Ph = P + (int64_t)h * tri(nb);
  const float* kh = kbar + (int64_t)kvh * nb * HD;
  // 256 threads copy a tile's 32 x 128 floats: thread t holds row t / 8, floats 16 (t % 8) .. + 15
  const int cr = tid >> 3, cc = (tid & 7) * 16;
  f32x4 stg[4];   // a register vector type: float4 struct copies would go through scratch
  auto kfetch = [&](int ct) {
    const int krow = ct * 32 + cr;
    const f32x4* src = (const f32x4*)(kh + (int64_t)(krow < nb ? krow : 0) * HD + cc);
#pragma unroll
    for (int i = 0; i < 4; ++i) stg[i] = src[i];
  };
  auto kstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(f32x4*)&kt[buf][cr * KT_PITCH + cc + 4 * i] = stg[i];
  };
  kfetch(ct0);
  kstore(0);
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  for (int ct = ct0; ct < ct1; ++ct) {
    const int buf = (ct - ct0) & 1;
    if (ct + 1 < ct1) kfetch(ct + 1);
    if (ct < ntile) {
      // two independent chains (d slices 4i..4i+1 and 4i+2..4i+3) keep the
      // matrix unit fed from one wave, summed at the end; the operands are
      // read one step ahead of the four MFMAs that use them (the order is
      // pinned: left to itself the compiler waits on each read just before
      // its use)
      f32x16 acc = {}, acc2 = {};
      const float* ka = &kt[buf][l32 * KT_PITCH + 64 * g];
      __builtin_amdgcn_sched_barrier(0);
      float4 a = *(const float4*)ka;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float4 an = a;
        if (i < 15) an = *(const float4*)(ka + 4 * (i + 1));
        acc = mfma_f32(a.x, qv[4 * i], acc);
        acc2 = mfma_f32(a.z, qv[4 * i + 2], acc2);
        acc = mfma_f32(a.y, qv[4 * i + 1], acc);
        acc2 = mfma_f32(a.w, qv[4 * i + 3], acc2);
        a = an;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
#pragma unroll
      for (int i = 0; i < 15; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0); // four MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // the next read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
      acc += acc2;
      // an interior tile (below the diagonal tile, rows inside the sequence)
      // needs no causal mask, no -inf test and no per-row store predicate: the
      // same values by a shorter path (a scalar branch: rb and ct are
      // wave-uniform)
      auto epilogue = [&](auto interior) {
        constexpr bool IN = decltype(interior)::value;
        float tmx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kb = ct * 32 + mfma32_row(r, g);
          const float x = acc[r] * scale;
          acc[r] = (IN || (row_ok && kb <= qb)) ? x : -INFINITY;
          tmx = fmaxf(tmx, acc[r]);
          tileT[w][l32][mfma32_row(r, g)] = x;
        }
        tmx = pair_max(tmx);
        const float mn = fmaxf(m, tmx);
        float se = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) se += (!IN && acc[r] == -INFINITY) ? 0.f : pe_exp(acc[r] - mn);
        se = pair_sum(se);
        l = (m == -INFINITY ? 0.f : l * pe_exp(m - mn)) + se;
        m = mn;
        __builtin_amdgcn_wave_barrier();
        // rows 2j + g of the tile, key block ct*32 + l32: 128 contiguous bytes per row;
        // all 16 reads first (one wait), then the stores
        float vals[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) vals[j] = tileT[w][2 * j + g][l32];
        const int kb = ct * 32 + l32;
        int q = rb * 32 + g;
        int64_t tq = tri(q);                 // tri(q + 2) = tri(q) + 2q + 3
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (IN || (q < nb && kb <= q)) Ph[tq + kb] = vals[j];
          tq += 2 * q + 3;
          q += 2;
        }
      };
      if (ct < rb && rb * 32 + 31 < nb) epilogue(std::true_type{});
      else epilogue(std::false_type{});
      __builtin_amdgcn_wave_barrier();
    }
    if (ct + 1 < ct1) {
      kstore(buf ^ 1);   // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  }
  if (row_ok && g == 0 && ct0 < ntile) part[((int64_t)h * nb + qb) * nseg + cs] = make_float2(m, l);
}

// Persistent: gridDim.x work-groups (two per CU) take items from *queue
// (zeroed by pool_q) until none is left.  Item it: virtual head it % nvh
// fastest, then segment, then row group from the top of the triangle (the
// longest rows first); items of other routes or past a triangle are skipped.
// The row groups of one head differ in work up to 8x, so a fixed grid left
// whole XCDs idle at the end.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void pe_logits_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, const int32_t* __restrict__ route,
    float* __restrict__ P, float2* __restrict__ part, const SeqList seqs, int hq, int hkv, int nseg, float scale,
    int* __restrict__ queue, int nvh, int nitems) {
  __shared__ __attribute__((aligned(16))) float kt[2][32 * KT_PITCH];
  __shared__ float tileT[PE_RB][32][33];
  __shared__ int s_item;
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(queue, 1);
    __syncthreads();
    const int it = __builtin_amdgcn_readfirstlane(s_item);   // uniform: the item's indices stay scalar
    __syncthreads();   // read by every thread before the next item is fetched
    if (it >= nitems) break;
    const int vh = it % nvh, rest = it / nvh;
    if (route[vh] != 0) continue;
    pe_logits_item(kt, tileT, qbar, kbar, P, part, seqs, hq, hkv, nseg, scale, vh, rest / nseg, rest % nseg);
  }
}

// Row softmax in place: one work-group per (query block, Pooled-Estimation
// head) merges the row's segment maxima and sums, then P = exp(L - M) / S.
__global__ __launch_bounds__(256) void pe_norm_kernel(const int32_t* __restrict__ route, const float2* __restrict__ part,
                                                      float* __restrict__ P, const SeqList seqs, int hq, int hkv,
                                                      int nseg) {
  const int qb = blockIdx.x, vh = blockIdx.y, tid = threadIdx.x;
  if (route[vh] != 0) return;
  const int h = vh % hq;
  const SeqPos sp = seq_pos(seqs, vh / hq, hq, hkv);
  const int nb = sp.nb;
  if (qb >= nb) return;
  P += sp.tri;
  const int ns = ((qb / 32) + 1 + PE_SEG - 1) / PE_SEG;   // segments this row block produced
  const float2* pp = part + (sp.rows + (int64_t)h * nb + qb) * nseg;
  float M = -INFINITY;
  for (int c = 0; c < ns; ++c) M = fmaxf(M, pp[c].x);
  float S = 0.f;
  for (int c = 0; c < ns; ++c) S += pp[c].x == -INFINITY ? 0.f : pp[c].y * pe_exp(pp[c].x - M);
  const float inv = 1.f / S;
  float* row = P + (int64_t)h * tri(nb) + tri(qb);
  for (int k0 = 0; k0 <= qb; k0 += 2048) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kb = k0 + 256 * j + tid;
      x[j] = kb <= qb ? row[kb] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kb = k0 + 256 * j + tid;
      if (kb <= qb) row[kb] = pe_exp(x[j] - M) * inv;
    }
  }
}

// ------------------------------------------------------------------ PE: radix select of the gamma cut

constexpr int PE_SLICE = 32768;  // entries per histogram work-group

__global__ void pe_cut_init_kernel(const int32_t* __restrict__ route, PeCut* __restrict__ cut,
                                   uint32_t* __restrict__ hcnt, unsigned long long* __restrict__ hmass,
                                   float gamma) {
  const int h = blockIdx.x, tid = threadIdx.x;
  uint32_t* c = hcnt + (int64_t)h * 3 * PE_BUCKETS;
  unsigned long long* m = hmass + (int64_t)h * 3 * PE_BUCKETS;
  for (int i = tid; i < 3 * PE_BUCKETS; i += blockDim.x) { c[i] = 0; m[i] = 0; }
  if (tid == 0) {
    PeCut z = {};
    z.active = (route[h] == 0 && gamma < 1.f) ? 1 : 0;
    cut[h] = z;
  }
}

__host__ __device__ constexpr int pe_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ constexpr int pe_width(int pass) { return pass == 2 ? 10 : 11; }

template <int PASS>
__global__ __launch_bounds__(256) void pe_hist_kernel(const float* __restrict__ P, const PeCut* __restrict__ cut,
                                                      uint32_t* __restrict__ hcnt,
                                                      unsigned long long* __restrict__ hmass, const SeqList seqs,
                                                      int hq, int hkv) {
  __shared__ uint32_t sc[PE_BUCKETS];
  __shared__ unsigned long long sm[PE_BUCKETS];
  const int h = blockIdx.y, tid = threadIdx.x;   // h: virtual head
  if (!cut[h].active) return;
  const SeqPos sp = seq_pos(seqs, h / hq, hq, hkv);
  const int64_t total = tri(sp.nb);
  if ((int64_t)blockIdx.x * PE_SLICE >= total) return;
  P += sp.tri + (int64_t)(h % hq) * total;
  constexpr int shift = pe_shift(PASS), width = pe_width(PASS);
  constexpr uint32_t mask = (1u << width) - 1;
  constexpr int hi = shift + width;
  const uint32_t prefix = cut[h].prefix;
  for (int i = tid; i < PE_BUCKETS; i += 256) { sc[i] = 0; sm[i] = 0; }
  __syncthreads();
  const uint32_t* bits = (const uint32_t*)P;
  const int64_t a = (int64_t)blockIdx.x * PE_SLICE, b = min(total, a + PE_SLICE);
  // neighbouring entries of a softmax row mostly fall into the same bucket:
  // each thread merges runs of equal buckets in registers (over its strided
  // entries) and commits a run with one pair of LDS atomics
  uint32_t run_b = 0xffffffffu, run_c = 0;
  unsigned long long run_m = 0;
  auto take = [&](uint32_t x) {
    if (PASS > 0 && (x >> hi) != (prefix >> hi)) return;
    const uint32_t bk = (x >> shift) & mask;
    if (bk != run_b) {
      if (run_c) { atomicAdd(&sc[run_b], run_c); atomicAdd(&sm[run_b], run_m); }
      run_b = bk;
      run_c = 0;
      run_m = 0;
    }
    ++run_c;
    run_m += fx_mass(x);
  };
  constexpr int U = 4;
  if (((uintptr_t)bits & 15) == 0) {
    // 16-byte loads of four consecutive entries, four loads in flight per
    // thread; a ragged end of the slice is read entry by entry
    for (int64_t e0 = a + 4 * tid; e0 < b; e0 += 4 * 256 * U) {
      uint4 xs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = e0 + 1024 * u;
        if (e + 4 <= b) xs[u] = *(const uint4*)(bits + e);
        else xs[u] = make_uint4(e < b ? bits[e] : 0u, e + 1 < b ? bits[e + 1] : 0u, e + 2 < b ? bits[e + 2] : 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = e0 + 1024 * u;
        if (e >= b) break;
        take(xs[u].x);
        if (e + 1 < b) take(xs[u].y);
        if (e + 2 < b) take(xs[u].z);
        if (e + 3 < b) take(xs[u].w);
      }
    }
  } else {
    // four strided entries are loaded before any is used (memory-level
    // parallelism); they are then taken in the same order as one at a time
    for (int64_t e0 = a + tid; e0 < b; e0 += U * 256) {
      uint32_t xs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) xs[u] = e0 + 256 * u < b ? bits[e0 + 256 * u] : 0u;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (e0 + 256 * u >= b) break;
        take(xs[u]);
      }
    }
  }
  if (run_c) { atomicAdd(&sc[run_b], run_c); atomicAdd(&sm[run_b], run_m); }
  __syncthreads();
  uint32_t* gc = hcnt + ((int64_t)h * 3 + PASS) * PE_BUCKETS;
  unsigned long long* gm = hmass + ((int64_t)h * 3 + PASS) * PE_BUCKETS;
  for (int i = tid; i < PE_BUCKETS; i += 256)
    if (sc[i]) { atomicAdd(&gc[i], sc[i]); atomicAdd(&gm[i], sm[i]); }
}

// One wave per head: lane L owns the buckets nbk-1-32L down to nbk-32-32L (from
// the top); the lane sums are scanned across the wave and the lane in which the
// running mass first reaches `need` walks its own buckets.  Integer sums, so
// the result equals a sequential walk from the top bucket.
template <int PASS>
__global__ __launch_bounds__(64) void pe_scan_kernel(PeCut* __restrict__ cut, const uint32_t* __restrict__ hcnt,
                                                     const unsigned long long* __restrict__ hmass, float gamma) {
  const int h = blockIdx.x, lane = threadIdx.x;
  PeCut c = cut[h];
  if (!c.active) return;
  constexpr int shift = pe_shift(PASS), width = pe_width(PASS);
  const uint32_t* hc = hcnt + ((int64_t)h * 3 + PASS) * PE_BUCKETS;
  const unsigned long long* hm = hmass + ((int64_t)h * 3 + PASS) * PE_BUCKETS;
  constexpr int nbk = 1 << width;
  constexpr int per = nbk / 64;
  const int top = nbk - 1 - per * lane;
  unsigned long long mine = 0;
  for (int i = 0; i < per; ++i) mine += hm[top - i];
  unsigned long long incl = mine;
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (PASS == 0) {
    const unsigned long long t = __shfl(incl, 63, 64);
    c.total = t;
    c.target = (unsigned long long)ceil((double)gamma * (double)t);
    if (c.target == 0) c.target = 1;
    c.need = c.target;
  }
  // first lane whose inclusive mass reaches need (the last lane if none does)
  const unsigned long long hit = __ballot(incl >= c.need);
  const int L = hit ? __builtin_ctzll(hit) : 63;
  if (lane != L) return;
  unsigned long long acc = incl - mine;
  int sel = top - per + 1;
  for (int i = top; i > top - per; --i) {
    if (acc + hm[i] >= c.need) { sel = i; break; }
    acc += hm[i];
    sel = i;
  }
  c.need -= acc;
  c.above_mass += acc;
  c.prefix |= (uint32_t)sel << shift;
  if (PASS == 2) {
    c.vstar = c.prefix;
    c.eq_cnt = hc[sel];
    const unsigned long long fv = fx_mass(c.vstar);
    unsigned long long take = fv ? (c.need + fv - 1) / fv : c.eq_cnt;
    c.take = take < c.eq_cnt ? take : c.eq_cnt;
  }
  cut[h] = c;
}

// count of entries equal to the cut value per row, then an exclusive scan per head (only when the cut
// splits a run of equal values)
__global__ __launch_bounds__(256) void pe_eq_count_kernel(const float* __restrict__ P, const PeCut* __restrict__ cut,
                                                          int32_t* __restrict__ eqrow, const SeqList seqs, int hq,
                                                          int hkv) {
  const int h = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;   // h: virtual head
  const int qb = blockIdx.x * 4 + w;
  const PeCut c = cut[h];
  if (!c.active || c.take >= c.eq_cnt) return;
  const SeqPos sp = seq_pos(seqs, h / hq, hq, hkv);
  const int nb = sp.nb;
  if (qb >= nb) return;
  const uint32_t* row = (const uint32_t*)(P + sp.tri + (int64_t)(h % hq) * tri(nb) + tri(qb));
  int cnt = 0;
  for (int k0 = lane; k0 <= qb; k0 += 256) {   // four loads in flight per lane
    uint32_t xs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) xs[u] = k0 + 64 * u <= qb ? row[k0 + 64 * u] : ~c.vstar;
#pragma unroll
    for (int u = 0; u < 4; ++u) cnt += (xs[u] == c.vstar);
  }
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) eqrow[sp.rows + (int64_t)(h % hq) * nb + qb] = cnt;
}

__global__ __launch_bounds__(256) void pe_eq_scan_kernel(const PeCut* __restrict__ cut, int32_t* __restrict__ eqrow,
                                                         const SeqList seqs, int hq, int hkv) {
  __shared__ int sh[256];
  const int h = blockIdx.x;   // virtual head
  const PeCut c = cut[h];
  if (!c.active || c.take >= c.eq_cnt) return;
  const SeqPos sp = seq_pos(seqs, h / hq, hq, hkv);
  const int nb = sp.nb;
  int32_t* e = eqrow + sp.rows + (int64_t)(h % hq) * nb;
  const int per = (nb + 255) / 256;
  const int a = min(nb, (int)threadIdx.x * per), b = min(nb, a + per);
  int s = 0;
  for (int k = a; k < b; ++k) s += e[k];
  int tot;
  int base = block_excl_scan(s, sh, &tot);
  for (int k = a; k < b; ++k) { const int v = e[k]; e[k] = base; base += v; }
}

// ------------------------------------------------------------------ lists

__device__ __forceinline__ int lane_prefix(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// One wave per (head, query block).  FILL = false writes the row's count,
// FILL = true writes its ascending key blocks at row_ptr[row].
template <bool FILL>
__global__ __launch_bounds__(256) void list_kernel(const int32_t* __restrict__ route,
                                                   const int32_t* __restrict__ sv, const int32_t* __restrict__ nv,
                                                   const int32_t* __restrict__ ss, const int32_t* __restrict__ ns,
                                                   const float* __restrict__ P, const PeCut* __restrict__ cut,
                                                   const int32_t* __restrict__ eqrow, int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col,
                                                   const SeqList seqs, int hq, int hkv, int nb_max, int pe_all) {
  extern __shared__ uint32_t bitmap[];  // 4 waves x ceil(nb_max/32) words
  const int h = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;   // h: virtual head
  const int qb = blockIdx.x * 4 + w;
  const SeqPos sp = seq_pos(seqs, h / hq, hq, hkv);
  const int nb = sp.nb;
  if (qb >= nb) return;
  const int hl = h % hq;                                     // query head within the sequence
  const int64_t row = sp.rows + (int64_t)hl * nb + qb;       // packed per-row arrays
  const int r = route[h];
  // the sequence's own CSR: row pointers at rp, relative to its column segment at tri
  int32_t* out = FILL ? col + sp.tri + row_ptr[sp.rp + (int64_t)hl * nb + qb] : nullptr;
  if (r == -1 || (r == 0 && pe_all)) {
    if (!FILL) { if (lane == 0) counts[row] = qb + 1; }
    else for (int k = lane; k <= qb; k += 64) out[k] = k;
    return;
  }
  if (r == 0) {
    const PeCut c = cut[h];
    const uint32_t* bits = (const uint32_t*)(P + sp.tri + (int64_t)hl * tri(nb) + tri(qb));
    const bool split = c.take < c.eq_cnt;
    int base = 0;
    long long eqb = split ? eqrow[row] : 0;
    // eight 64-entry pieces are loaded before any is used, then taken in order
    for (int k00 = 0; k00 <= qb; k00 += 512) {
      uint32_t xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k00 + 64 * u + lane;
        xs[u] = k <= qb ? bits[k] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k0 = k00 + 64 * u;
        if (k0 > qb) break;
        const int k = k0 + lane;
        const bool valid = k <= qb;
        const uint32_t x = xs[u];
        bool sel = valid && ((x > c.vstar) || k == 0 || k == qb || (!split && x == c.vstar));
        if (split) {  // the cut splits a run of equal values: take them in flat order
          const bool eq = valid && x == c.vstar;
          const unsigned long long em = __ballot(eq);
          if (eq && (unsigned long long)(eqb + lane_prefix(em)) < c.take) sel = true;
          eqb += __popcll(em);
        }
        const unsigned long long m = __ballot(sel);
        if (FILL && sel) out[base + lane_prefix(m)] = k;
        base += __popcll(m);
      }
    }
    if (!FILL && lane == 0) counts[row] = base;
    return;
  }
  // Vertical-Slash: set bits in a per-wave bitmap, then read them out in order
  const int nw = (nb + 31) / 32;
  uint32_t* bm = bitmap + w * nw;
  const int words = qb / 32 + 1;
  for (int i = lane; i < words; i += 64) bm[i] = 0;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const int32_t* svh = sv + sp.rows + (int64_t)hl * nb;
  const int32_t* ssh = ss + sp.rows + (int64_t)hl * nb;
  const int cv = nv[h], cs = ns[h];
  for (int i = lane; i < cv; i += 64) {
    const int k = svh[i];
    if (k <= qb) atomicOr(&bm[k >> 5], 1u << (k & 31));
  }
  for (int i = lane; i < cs; i += 64) {
    const int k = ssh[i];
    if (k <= qb) { const int kb = qb - k; atomicOr(&bm[kb >> 5], 1u << (kb & 31)); }
  }
  if (lane == 0) {
    atomicOr(&bm[0], 1u);
    atomicOr(&bm[qb >> 5], 1u << (qb & 31));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  int base = 0;
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int wi = w0 + lane;
    uint32_t word = wi < words ? bm[wi] : 0u;
    if (wi == qb >> 5) word &= (qb & 31) == 31 ? 0xffffffffu : ((2u << (qb & 31)) - 1u);
    const int pc = __popc(word);
    int incl = pc;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (FILL) {
      int pos = base + incl - pc;
      while (word) {
        const int b = __ffs(word) - 1;
        out[pos++] = wi * 32 + b;
        word &= word - 1;
      }
    }
    base += __shfl(incl, 63, 64);
  }
  if (!FILL && lane == 0) counts[row] = base;
}

// Exclusive scan of each sequence's row counts into its row pointers (a
// sequence's total fits int32, checked on the host), over tiles of ROW_TILE
// counts in two launches: the sum of every tile, then every tile scanned on
// top of the sum of the tiles before it (integer sums: the result equals a
// sequential scan).
constexpr int ROW_TILE = 4096;
int row_tiles(int64_t rows) { return (int)((rows + ROW_TILE - 1) / ROW_TILE); }

__device__ __forceinline__ int block_sum_1024(int v, int* wsum) {   // 1024 threads; wsum[16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) wsum[w] = v;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < 16; ++i) t += wsum[i];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(1024) void row_tile_sum_kernel(const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ tsum, const SeqList seqs, int hq,
                                                            int hkv, int ntile_max) {
  __shared__ int wsum[16];
  const SeqPos sp = seq_pos(seqs, blockIdx.y, hq, hkv);
  const int64_t rows = (int64_t)hq * sp.nb, i0 = (int64_t)blockIdx.x * ROW_TILE + 4 * threadIdx.x;
  if ((int64_t)blockIdx.x * ROW_TILE >= rows) return;
  counts += sp.rows;
  int own = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) own += i0 + e < rows ? counts[i0 + e] : 0;
  const int t = block_sum_1024(own, wsum);
  if (threadIdx.x == 0) tsum[(int64_t)blockIdx.y * ntile_max + blockIdx.x] = t;
}

__global__ __launch_bounds__(1024) void scan_rows_kernel(const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ tsum,
                                                         int32_t* __restrict__ row_ptr, const SeqList seqs, int hq,
                                                         int hkv, int ntile_max) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const SeqPos sp = seq_pos(seqs, blockIdx.y, hq, hkv);
  const int64_t rows = (int64_t)hq * sp.nb, base = (int64_t)blockIdx.x * ROW_TILE;
  if (base >= rows) return;
  counts += sp.rows;
  row_ptr += sp.rp;
  // sum of the tiles before this one
  int pre = 0;
  for (int i = tid; i < (int)blockIdx.x; i += 1024) pre += tsum[(int64_t)blockIdx.y * ntile_max + i];
  const int carry = block_sum_1024(pre, wsum);
  const int64_t i0 = base + 4 * tid;
  int v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = i0 + e < rows ? counts[i0 + e] : 0;
  const int own = v[0] + v[1] + v[2] + v[3];
  int incl = own;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = carry;
  for (int i = 0; i < w; ++i) before += wsum[i];
  int run = before + incl - own;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (i0 + e < rows) row_ptr[i0 + e] = run;
    run += v[e];
  }
  if (tid == 1023 && base + ROW_TILE >= rows) row_ptr[rows] = run;   // the sequence's total
}

__global__ void copy_sets_kernel(const int32_t* __restrict__ sv, const int32_t* __restrict__ nv,
                                 const int32_t* __restrict__ ss, const int32_t* __restrict__ ns, int32_t* sv_out,
                                 int32_t* nv_out, int32_t* ss_out, int32_t* ns_out, const SeqList seqs, int hq,
                                 int hkv) {
  const int h = blockIdx.x;   // virtual head
  const SeqPos sp = seq_pos(seqs, h / hq, hq, hkv);
  const int64_t rowb = sp.rows + (int64_t)(h % hq) * sp.nb;
  const int a = nv[h], b = ns[h];
  if (threadIdx.x == 0) { if (nv_out) nv_out[h] = a; if (ns_out) ns_out[h] = b; }
  for (int i = threadIdx.x; i < a; i += blockDim.x) if (sv_out) sv_out[rowb + i] = sv[rowb + i];
  for (int i = threadIdx.x; i < b; i += blockDim.x) if (ss_out) ss_out[rowb + i] = ss[rowb + i];
}

// ------------------------------------------------------------------ launcher

hipError_t launch_select(int fp32, const void* Q, const SeqList& seqs, int nb_max, int hq, int hkv,
                         const Strides& st, int w_sink, int w_local, float tau, float alpha, float gamma,
                         int min_blocks, int dense_below_n, const SelectBufs& b, hipStream_t s) {
  const unsigned vh = (unsigned)(seqs.nseq * hq);   // virtual heads: (sequence, query head)
  const bool jsd_on = b.router == 1;
  if (jsd_on) {
    const float scale = 1.f / sqrtf((float)HD);
    if (fp32)
      jsd_route_kernel<float><<<vh, 256, 0, s>>>((const float*)Q, (const float4*)b.tiles, b.kbar, b.abar, b.jsd,
                                                 seqs, hq, hkv, st.q_h, st.q_n, dense_below_n, scale);
    else
      jsd_route_kernel<bf16><<<vh, 256, 0, s>>>((const bf16*)Q, (const float4*)b.tiles, b.kbar, b.abar, b.jsd, seqs,
                                                hq, hkv, st.q_h, st.q_n, dense_below_n, scale);
  }
  vs_select_kernel<<<vh, 256, nb_max, s>>>((const float4*)b.tiles, seqs, hq, hkv, w_sink, w_local, tau, alpha,
                                           min_blocks, dense_below_n, jsd_on ? b.jsd : nullptr, b.vs_budget,
                                           b.route, b.c_struct, b.pv, b.ps, b.sv, b.nv, b.ss, b.ns, b.pv_out,
                                           b.ps_out);
  if (b.vs_budget != 0) {
    if (b.vs_budget == 1)
      vs_rank_kernel<true><<<dim3(vh, 2), 1024, nb_max, s>>>(b.route, b.pv, b.ps, seqs, hq, hkv, alpha, gamma,
                                                             min_blocks, b.sv, b.nv, b.ss, b.ns);
    else
      vs_rank_kernel<false><<<dim3(vh, 2), 1024, nb_max, s>>>(b.route, b.pv, b.ps, seqs, hq, hkv, alpha, gamma,
                                                              min_blocks, b.sv, b.nv, b.ss, b.ns);
  }
  PeCut* cut = (PeCut*)b.cut;
  const int64_t total_max = (int64_t)nb_max * (nb_max + 1) / 2;
  const int pe_all = gamma >= 1.f ? 1 : 0;
  const dim3 gq(nb_max, vh);
  if (fp32)
    pool_q_kernel<float><<<gq, 256, 0, s>>>((const float*)Q, b.route, b.qbar, seqs, hq, hkv, st.q_h, st.q_n, b.peq);
  else
    pool_q_kernel<bf16><<<gq, 256, 0, s>>>((const bf16*)Q, b.route, b.qbar, seqs, hq, hkv, st.q_h, st.q_n, b.peq);
  const int nrb = (nb_max + 31) / 32, nseg = pe_segments(nb_max);
  const int pe_items = ((nrb + PE_RB - 1) / PE_RB) * nseg * vh;
  pe_logits_kernel<<<std::min(pe_items, 2 * device_cu_count()), 256, 0, s>>>(
      b.qbar, b.kbar, b.route, b.P, (float2*)b.pepart, seqs, hq, hkv, nseg, 1.f / sqrtf((float)HD), b.peq, vh,
      pe_items);
  pe_norm_kernel<<<dim3(nb_max, vh), 256, 0, s>>>(b.route, (const float2*)b.pepart, b.P, seqs, hq, hkv, nseg);
  pe_cut_init_kernel<<<vh, 256, 0, s>>>(b.route, cut, b.hcnt, b.hmass, gamma);
  const dim3 gh((unsigned)((total_max + PE_SLICE - 1) / PE_SLICE), vh);
  pe_hist_kernel<0><<<gh, 256, 0, s>>>(b.P, cut, b.hcnt, b.hmass, seqs, hq, hkv);
  pe_scan_kernel<0><<<vh, 64, 0, s>>>(cut, b.hcnt, b.hmass, gamma);
  pe_hist_kernel<1><<<gh, 256, 0, s>>>(b.P, cut, b.hcnt, b.hmass, seqs, hq, hkv);
  pe_scan_kernel<1><<<vh, 64, 0, s>>>(cut, b.hcnt, b.hmass, gamma);
  pe_hist_kernel<2><<<gh, 256, 0, s>>>(b.P, cut, b.hcnt, b.hmass, seqs, hq, hkv);
  pe_scan_kernel<2><<<vh, 64, 0, s>>>(cut, b.hcnt, b.hmass, gamma);
  pe_eq_count_kernel<<<dim3((nb_max + 3) / 4, vh), 256, 0, s>>>(b.P, cut, b.eqrow, seqs, hq, hkv);
  pe_eq_scan_kernel<<<vh, 256, 0, s>>>(cut, b.eqrow, seqs, hq, hkv);
  const dim3 gl((nb_max + 3) / 4, vh);
  const size_t bm_bytes = 4 * ((nb_max + 31) / 32) * sizeof(uint32_t);
  list_kernel<false><<<gl, 256, bm_bytes, s>>>(b.route, b.sv, b.nv, b.ss, b.ns, b.P, cut, b.eqrow, b.counts,
                                               b.row_ptr, b.col_idx, seqs, hq, hkv, nb_max, pe_all);
  const int ntile = row_tiles((int64_t)hq * nb_max);
  row_tile_sum_kernel<<<dim3(ntile, seqs.nseq), 1024, 0, s>>>(b.counts, b.rtsum, seqs, hq, hkv, ntile);
  scan_rows_kernel<<<dim3(ntile, seqs.nseq), 1024, 0, s>>>(b.counts, b.rtsum, b.row_ptr, seqs, hq, hkv, ntile);
  list_kernel<true><<<gl, 256, bm_bytes, s>>>(b.route, b.sv, b.nv, b.ss, b.ns, b.P, cut, b.eqrow, b.counts,
                                              b.row_ptr, b.col_idx, seqs, hq, hkv, nb_max, pe_all);
  if (b.sv_out || b.nv_out || b.ss_out || b.ns_out)
    copy_sets_kernel<<<vh, 256, 0, s>>>(b.sv, b.nv, b.ss, b.ns, b.sv_out, b.nv_out, b.ss_out, b.ns_out, seqs, hq,
                                        hkv);
  return hipGetLastError();
}

}  // namespace crisp
