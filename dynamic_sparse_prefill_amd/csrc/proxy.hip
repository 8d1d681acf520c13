// Proxy attention for routing and Vertical-Slash scores (gfx950).
//
// For every query head h, A_hat = causal softmax(Q_last K^T / sqrt(d)) over the
// last query block (rows at positions n-128 .. n-1)  [rcap.io CRISP summary,
// per-head pseudo-code; CRISP paper §2, representative query subset].  A_hat is
// never stored: it is reduced on the fly, per 128-key tile kb, into three sums
// over the tile's entries (r = query row, c = key column within the tile):
//   lower[kb]  = sum over c <= r of A_hat   -> slash bin N_b-1-kb
//   upper[kb]  = sum over c >  r of A_hat   -> slash bin N_b-2-kb
//   anchor[kb] = sum over keys in [0, w_sink) U [n - w_local, n)
// because the diagonal offset o = q_r - j of tile kb is (N_b-1-kb)*128 + (r-c).
// From these the selection stage forms p^v[kb] = (lower+upper)/b,
// p^s[k] = (lower[N_b-1-k] + upper[N_b-2-k])/b and C_struct = sum(anchor)/b
// [CRISP §3.2, §4].
//
// Two passes over K: pass A computes per-(head, key chunk) row max / sum,
// a tiny combine yields the exact row normaliser, pass B recomputes the
// scores and accumulates the normalised tile sums.  Every reduction has a
// fixed order (no float atomics), so the scores are bit-reproducible.
// Pass A also writes the block means of K (K-bar) used by Pooled Estimation.
// Grid: blockIdx -> (key chunk, head-in-group, KV head) so the G query heads
// sharing a K chunk run on one XCD and share its L2.
#include "common.h"
#include "launch.h"
#include "tile.h"

namespace crisp {

constexpr int PCH = 8;  // key blocks per proxy work-group

int proxy_chunks(int nb) { return (nb + PCH - 1) / PCH; }

template <typename T>
__global__ __launch_bounds__(256) void proxy_stats_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          float2* __restrict__ stats, float* __restrict__ kbar,
                                                          int nb, int hq, int hkv, int nchunk, int64_t sq_h,
                                                          int64_t sq_n, int64_t sk_h, int64_t sk_n, float sl2) {
  __shared__ __attribute__((aligned(16))) T sK[BLK * Tile<T>::KP];
  __shared__ float red[2][HD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int G = hq / hkv;
  const int chunk = blockIdx.x / hq, rem = blockIdx.x % hq;
  const int kvh = rem % hkv, hig = rem / hkv, h = kvh * G + hig;
  const int qrow = 32 * w + l32;
  typename Tile<T>::QFrag qf;
  Tile<T>::load_q(qf, Q + (int64_t)h * sq_h + (int64_t)((nb - 1) * BLK + qrow) * sq_n, g);
  const int kb0 = chunk * PCH, kb1 = min(nb, kb0 + PCH);
  float m = -1e30f, l = 0.f;
  for (int kb = kb0; kb < kb1; ++kb) {
    __syncthreads();
    Tile<T>::load_k(sK, K + (int64_t)kvh * sk_h + (int64_t)kb * BLK * sk_n, sk_n, tid);
    __syncthreads();
    if (hig == 0) {  // block mean of K for Pooled Estimation, once per KV head
      const int d = tid & 127, half = tid >> 7;
      float sum = 0.f;
      for (int r = 0; r < 64; ++r) sum += to_f32(sK[(64 * half + r) * Tile<T>::KP + d]);
      red[half][d] = sum;
      __syncthreads();
      if (half == 0) kbar[((int64_t)kvh * nb + kb) * HD + d] = (red[0][d] + red[1][d]) * (1.f / BLK);
    }
    f32x16 s[4];
    Tile<T>::st(s, sK, qf, l32, g);
    if (kb == nb - 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * t + mfma32_row(i, g) > qrow) s[t][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
    const float mn = fmaxf(m, mx);
    const float mb = mn * sl2;
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) rs += fast_exp2(fmaf(s[t][i], sl2, -mb));
    l = l * fast_exp2((m - mn) * sl2) + rs;
    m = mn;
  }
  const float m2 = __shfl_xor(m, 32, 64), l2 = __shfl_xor(l, 32, 64);
  const float M = fmaxf(m, m2);
  const float L = l * fast_exp2((m - M) * sl2) + l2 * fast_exp2((m2 - M) * sl2);
  if (g == 0) stats[((int64_t)h * nchunk + chunk) * BLK + qrow] = make_float2(M, L);
}

// Row normaliser of the proxy rows: M = max over chunks, 1/L with L rescaled to
// M.  Eight groups of 128 threads take every eighth chunk; their partial
// (max, sum) pairs are merged in group order, so the result is reproducible.
constexpr int CMB_GROUPS = 8;
__global__ __launch_bounds__(BLK * CMB_GROUPS) void proxy_combine_kernel(const float2* __restrict__ stats,
                                                                         float2* __restrict__ rowstat, int nchunk,
                                                                         float sl2) {
  __shared__ float2 part[CMB_GROUPS][BLK];
  const int h = blockIdx.x, r = threadIdx.x % BLK, grp = threadIdx.x / BLK;
  const float2* p = stats + (int64_t)h * nchunk * BLK + r;
  float M = -1e30f;
  for (int c = grp; c < nchunk; c += CMB_GROUPS) M = fmaxf(M, p[(int64_t)c * BLK].x);
  float L = 0.f;
  for (int c = grp; c < nchunk; c += CMB_GROUPS) {
    const float2 v = p[(int64_t)c * BLK];
    L += v.y * fast_exp2((v.x - M) * sl2);
  }
  part[grp][r] = make_float2(M, L);
  __syncthreads();
  if (grp == 0) {
    float Mt = -1e30f;
    for (int q = 0; q < CMB_GROUPS; ++q) Mt = fmaxf(Mt, part[q][r].x);
    float Lt = 0.f;
    for (int q = 0; q < CMB_GROUPS; ++q) Lt += part[q][r].y * fast_exp2((part[q][r].x - Mt) * sl2);
    rowstat[h * BLK + r] = make_float2(Mt, 1.f / Lt);
  }
}

// Lower / upper sums of one interior tile for wave W (rows 32W .. 32W+31).
template <int W>
__device__ __forceinline__ void interior_sums(const f32x16 (&s)[4], float sl2, float mbl, int qrow, int g,
                                              float& lo, float& up) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[t][i], sl2, -mbl));
      if (t < W) lo += p;
      else if (t > W) up += p;
      else if (32 * t + mfma32_row(i, g) <= qrow) lo += p;
      else up += p;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void proxy_pool_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                         const float2* __restrict__ rowstat,
                                                         float4* __restrict__ tiles, int64_t n, int nb, int hq,
                                                         int hkv, int64_t sq_h, int64_t sq_n, int64_t sk_h,
                                                         int64_t sk_n, int w_sink, int w_local, float sl2) {
  __shared__ __attribute__((aligned(16))) T sK[BLK * Tile<T>::KP];
  __shared__ float red[4][3];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: the t-vs-w branches are scalar
  const int G = hq / hkv;
  const int chunk = blockIdx.x / hq, rem = blockIdx.x % hq;
  const int kvh = rem % hkv, h = kvh * G + rem / hkv;
  const int qrow = 32 * w + l32;
  typename Tile<T>::QFrag qf;
  Tile<T>::load_q(qf, Q + (int64_t)h * sq_h + (int64_t)((nb - 1) * BLK + qrow) * sq_n, g);
  const float2 rsx = rowstat[h * BLK + qrow];
  // p = exp2(s sl2 - M sl2) / L = exp2(s sl2 - (M sl2 + log2 L)): one fma and one exp per score
  const float mbl = rsx.x * sl2 - __log2f(rsx.y);
  const int kb0 = chunk * PCH, kb1 = min(nb, kb0 + PCH);
  for (int kb = kb0; kb < kb1; ++kb) {
    __syncthreads();
    Tile<T>::load_k(sK, K + (int64_t)kvh * sk_h + (int64_t)kb * BLK * sk_n, sk_n, tid);
    __syncthreads();
    f32x16 s[4];
    Tile<T>::st(s, sK, qf, l32, g);
    const bool last = (kb == nb - 1);
    const int64_t j0 = (int64_t)kb * BLK;
    const bool touches_anchor = (j0 < w_sink) || (j0 + BLK > n - w_local);
    float lo = 0.f, up = 0.f, an = 0.f;
    // key c = 32t + .. of this tile against this wave's rows 32w .. 32w+31:
    // t < w all lower (c <= qrow), t > w all upper, t = w split per score; on the
    // last tile the upper part is masked (keys after the query).  Interior
    // tiles take a path specialised on w (no per-score selects off the diagonal
    // block); the last tile and the anchor tiles take the general one.
    if (!last && !touches_anchor) {
      switch (w) {
        case 0: interior_sums<0>(s, sl2, mbl, qrow, g, lo, up); break;
        case 1: interior_sums<1>(s, sl2, mbl, qrow, g, lo, up); break;
        case 2: interior_sums<2>(s, sl2, mbl, qrow, g, lo, up); break;
        default: interior_sums<3>(s, sl2, mbl, qrow, g, lo, up); break;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t > w && last) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * t + mfma32_row(i, g);
          const float p = fast_exp2(fmaf(s[t][i], sl2, -mbl));
          bool lower = t < w;
          if (t == w) lower = c <= qrow;
          if (lower) lo += p;
          else if (!last) up += p;
          if (touches_anchor && (lower || !last)) {
            const int64_t j = j0 + c;
            if (j < w_sink || j >= n - w_local) an += p;
          }
        }
      }
    }
    lo = wave_sum(lo);
    up = wave_sum(up);
    an = wave_sum(an);
    if (lane == 0) { red[w][0] = lo; red[w][1] = up; red[w][2] = an; }
    __syncthreads();
    if (tid == 0) {
      float a = 0.f, b = 0.f, c = 0.f;
      for (int q = 0; q < 4; ++q) { a += red[q][0]; b += red[q][1]; c += red[q][2]; }
      tiles[(int64_t)h * nb + kb] = make_float4(a, b, c, 0.f);
    }
  }
}

hipError_t launch_proxy(int fp32, const void* Q, const void* K, int64_t n, int nb, int hq, int hkv,
                        const Strides& st, int w_sink, int w_local, void* stats, void* rowstat, void* tiles,
                        float* kbar, hipStream_t s) {
  const float sl2 = LOG2E / sqrtf((float)HD);
  const int nchunk = proxy_chunks(nb);
  const dim3 grid((unsigned)(nchunk * hq));
  if (fp32) {
    proxy_stats_kernel<float><<<grid, 256, 0, s>>>((const float*)Q, (const float*)K, (float2*)stats, kbar, nb, hq,
                                                   hkv, nchunk, st.q_h, st.q_n, st.k_h, st.k_n, sl2);
  } else {
    proxy_stats_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)Q, (const bf16*)K, (float2*)stats, kbar, nb, hq,
                                                  hkv, nchunk, st.q_h, st.q_n, st.k_h, st.k_n, sl2);
  }
  proxy_combine_kernel<<<hq, BLK * CMB_GROUPS, 0, s>>>((const float2*)stats, (float2*)rowstat, nchunk, sl2);
  if (fp32) {
    proxy_pool_kernel<float><<<grid, 256, 0, s>>>((const float*)Q, (const float*)K, (const float2*)rowstat,
                                                  (float4*)tiles, n, nb, hq, hkv, st.q_h, st.q_n, st.k_h, st.k_n,
                                                  w_sink, w_local, sl2);
  } else {
    proxy_pool_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)Q, (const bf16*)K, (const float2*)rowstat,
                                                 (float4*)tiles, n, nb, hq, hkv, st.q_h, st.q_n, st.k_h, st.k_n,
                                                 w_sink, w_local, sl2);
  }
  return hipGetLastError();
}

}  // namespace crisp
