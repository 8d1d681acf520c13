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
// One pass over K: for every (tile, row) the row's tile max m and the three
// sums of exp(s - m) are stored (16 bytes); a row pass merges the tile maxima
// and sums into the exact row normaliser (max M, 1/L), and a tile pass
// rescales the stored sums by exp(m - M) / L and adds them over the rows.
// Every reduction has a fixed order (no float atomics), so the scores are
// bit-reproducible.  The score pass also writes the block means of K (K-bar)
// used by Pooled Estimation.  Grid: blockIdx -> (key chunk, group of query
// heads of a KV group, KV head) so the work-groups sharing a K chunk run on
// one XCD and share its L2; the heads of a group share each K tile in LDS.
#include <algorithm>

#include "common.h"
#include "lanes.h"
#include "launch.h"
#include "tile.h"

namespace crisp {

constexpr int PCH = 16;       // most key blocks per score work-group (fewer when the grid would be small)
// query heads of a KV group per score work-group: they share each K tile the
// group loads (bf16; the fp32 path's query fragments are twice as large)
template <typename T> constexpr int proxy_heads() { return sizeof(T) == 2 ? 2 : 1; }
constexpr int RS_TILES = 64;  // key blocks per row-statistics work-group

int proxy_chunks(int nb) { return (nb + RS_TILES - 1) / RS_TILES; }
__device__ __forceinline__ int rs_chunks(int nb) { return (nb + RS_TILES - 1) / RS_TILES; }

// Lower / upper sums of one interior tile for the wave owning rows 32w ..
// 32w+31, p = exp2(s sl2 - mb): key sub-tile t < w lies wholly below the
// diagonal of every row of the wave, t > w wholly above it (w is wave-uniform,
// so those are scalar branches), and only the diagonal sub-tile t = w is split
// per score.  Each sub-tile is summed on its own, then added in t order.
__device__ __forceinline__ void interior_sums(const f32x16 (&s)[4], float sl2, float mb, int w, int l32, int g,
                                              float& lo, float& up) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float a = 0.f, b = 0.f;
    if (t == w) {
      int lim = l32 - 4 * g;               // key 32t + 8(i/4) + 4g + i%4 <= row 32w + l32
      asm volatile("" : "+v"(lim));        // the 16 compares stay here (not hoisted into SGPR masks)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[t][i], sl2, -mb));
        if (8 * (i >> 2) + (i & 3) <= lim) a += p;
        else b += p;
      }
      lo += a;
      up += b;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) a += fast_exp2(fmaf(s[t][i], sl2, -mb));
      const bool below = t < w;             // value selects (a pointer select would go to scratch)
      lo += below ? a : 0.f;
      up += below ? 0.f : a;
    }
  }
}

// K-bar partials of a staged bf16 tile for wave w: column sums over the
// wave's 32 rows (4w + k + 16i), the lanes that share columns added pairwise
// (lane ^ 16, then lane ^ 32), written by lanes 0..15 to dst[w][0..127].
__device__ __forceinline__ void kbar_partials(float (*dst)[HD], const Tile<bf16>::KStage& stg, int w, int lane) {
  float cs[8];
  Tile<bf16>::col_sums(cs, stg);
#pragma unroll
  for (int j = 0; j < 8; ++j) cs[j] = pair_sum(row_pair_sum(cs[j]));
  if (lane < 16) {
    *(f32x4*)&dst[w][8 * lane] = f32x4{cs[0], cs[1], cs[2], cs[3]};
    *(f32x4*)&dst[w][8 * lane + 4] = f32x4{cs[4], cs[5], cs[6], cs[7]};
  }
}

// Scores of the last query block against kpc <= PCH key blocks; per (tile, row):
// tile max m of the row and the sums of exp(s - m) over the lower part (key
// column <= row: slash bin N_b-1-kb), the upper part (bin N_b-2-kb) and the
// anchor windows.
template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void proxy_tiles_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          float4* __restrict__ tstat, float* __restrict__ kbar,
                                                          const SeqList seqs, int hq, int hkv, int64_t sq_h,
                                                          int64_t sq_n, int64_t sk_h, int64_t sk_n, int w_sink,
                                                          int w_local, int dense_below_n, float sl2, int kpc) {
  // bf16: two K tiles (the next one is written while the current one is read);
  // fp32 keeps one (its staging would not fit in registers)
  constexpr bool PIPE = sizeof(T) == 2;
  constexpr int TILE = BLK * Tile<T>::KP;
  __shared__ __attribute__((aligned(16))) T sK[(PIPE ? 2 : 1) * TILE];
  // K-bar partial column sums: bf16 per (tile parity, wave), fp32 per half tile
  __shared__ __attribute__((aligned(16))) float red[2][4][HD];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: the t-vs-w branches are scalar
  constexpr int HPW = proxy_heads<T>();
  const int G = hq / hkv, npg = (G + HPW - 1) / HPW;   // head groups per KV head
  const int chunk = blockIdx.x / (hkv * npg), rem = blockIdx.x % (hkv * npg);
  const int kvh = rem % hkv, hp = rem / hkv;
  const int h0 = kvh * G + HPW * hp, nh = min(HPW, G - HPW * hp);   // heads h0 .. h0 + nh - 1
  const bool kbar_wg = hp == 0;   // block means of K, once per KV head
  const SeqPos sp = seq_pos(seqs, blockIdx.y, hq, hkv);
  const int nb = sp.nb;
  const int64_t n = (int64_t)nb * BLK;
  if (chunk * kpc >= nb || seq_dense(nb, dense_below_n)) return;
  Q += sp.tok * sq_n;
  K += sp.tok * sk_n;
  tstat += (sp.rows + (int64_t)h0 * nb) * BLK;   // head h0 + hh at tstat + hh * nb * BLK
  kbar += sp.kvrows * HD;
  const int qrow = 32 * w + l32;
  typename Tile<T>::QFrag qf[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j)
    if (j < nh) Tile<T>::load_q(qf[j], Q + (int64_t)(h0 + j) * sq_h + (int64_t)((nb - 1) * BLK + qrow) * sq_n, g);
  const int kb0 = chunk * kpc, kb1 = min(nb, kb0 + kpc);
  const T* Kh = K + (int64_t)kvh * sk_h;
  typename Tile<bf16>::KStage stg;
  if constexpr (PIPE) {
    Tile<bf16>::fetch_k(stg, (const bf16*)Kh + (int64_t)kb0 * BLK * sk_n, sk_n, tid);
    Tile<bf16>::store_k((bf16*)sK, stg, tid);
    if (kbar_wg) kbar_partials(red[0], stg, w, lane);
    __syncthreads();
  }
  for (int kb = kb0; kb < kb1; ++kb) {
    const int par = (kb - kb0) & 1;
    T* cur = sK + (PIPE ? par * TILE : 0);
    if constexpr (PIPE) {
      if (kb + 1 < kb1) Tile<bf16>::fetch_k(stg, (const bf16*)Kh + (int64_t)(kb + 1) * BLK * sk_n, sk_n, tid);
    } else {
      __syncthreads();
      Tile<T>::load_k(cur, Kh + (int64_t)kb * BLK * sk_n, sk_n, tid);
      __syncthreads();
    }
    if (kbar_wg) {  // block mean of K for Pooled Estimation
      if constexpr (PIPE) {
        // the partials of this tile were written before the last barrier
        if (tid < HD)
          kbar[((int64_t)kvh * nb + kb) * HD + tid] =
              (((red[par][0][tid] + red[par][1][tid]) + red[par][2][tid]) + red[par][3][tid]) * (1.f / BLK);
      } else {
        const int d = tid & 127, half = tid >> 7;
        float sum = 0.f;
        for (int r = 0; r < 64; ++r) sum += to_f32(cur[(64 * half + r) * Tile<T>::KP + d]);
        red[0][half][d] = sum;
        __syncthreads();
        if (half == 0) kbar[((int64_t)kvh * nb + kb) * HD + d] = (red[0][0][d] + red[0][1][d]) * (1.f / BLK);
      }
    }
    // every head of the group against the same K tile
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (hh >= nh) break;
      f32x16 s[4];
      Tile<T>::st(s, cur, qf[hh], l32, g);
      const bool last = (kb == nb - 1);
      if (last) {
        int lim = qrow;
        asm volatile("" : "+v"(lim));   // compares stay in this once-per-row branch (no hoisted SGPR masks)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * t + mfma32_row(i, g) > lim) s[t][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
      mx = pair_max(mx);   // every row keeps at least its diagonal key: finite
      const float mb = mx * sl2;
      const int64_t j0 = (int64_t)kb * BLK;
      const bool touches_anchor = (j0 < w_sink) || (j0 + BLK > n - w_local);
      float lo = 0.f, up = 0.f, an = 0.f;
      // key c = 32t + .. against this wave's rows 32w .. 32w+31: t < w all lower,
      // t > w all upper, t = w split per score; interior tiles take the short
      // path, the last tile and the anchor tiles the general one
      if (!last && !touches_anchor) {
        interior_sums(s, sl2, mb, w, l32, g, lo, up);
      } else {
        int lim = qrow;
        asm volatile("" : "+v"(lim));   // as above: the per-score compares stay in this branch
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t > w && last) continue;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = 32 * t + mfma32_row(i, g);
            const float p = fast_exp2(fmaf(s[t][i], sl2, -mb));
            bool lower = t < w;
            if (t == w) lower = c <= lim;
            if (lower) lo += p;
            else if (!last) up += p;
            if (touches_anchor && (lower || !last)) {
              const int64_t j = j0 + c;
              if (j < w_sink || j >= n - w_local) an += p;
            }
          }
        }
      }
      lo = pair_sum(lo);
      up = pair_sum(up);
      an = pair_sum(an);
      if (g == 0) tstat[((int64_t)hh * nb + kb) * BLK + qrow] = make_float4(mx, lo, up, an);
    }
    if constexpr (PIPE) {
      // the other buffer and the other partials were last read before the
      // previous barrier
      if (kb + 1 < kb1) {
        Tile<bf16>::store_k((bf16*)sK + (par ^ 1) * TILE, stg, tid);
        if (kbar_wg) kbar_partials(red[par ^ 1], stg, w, lane);
        __syncthreads();
      }
    }
  }
}

// Row statistics over RS_TILES tiles: M = max of the tile maxima, L = sum of
// the tile sums rescaled to M (online, in tile order).
__global__ __launch_bounds__(BLK) void proxy_rowstat_kernel(const float4* __restrict__ tstat,
                                                            float2* __restrict__ stats, const SeqList seqs, int hq,
                                                            int hkv, int nchunk, int dense_below_n, float sl2) {
  const int chunk = blockIdx.x, vh = blockIdx.y, r = threadIdx.x;
  const int h = vh % hq;
  const SeqPos sp = seq_pos(seqs, vh / hq, hq, hkv);
  const int nb = sp.nb;
  if (seq_dense(nb, dense_below_n)) return;
  const int t0 = chunk * RS_TILES, t1 = min(nb, t0 + RS_TILES);
  tstat += (sp.rows + (int64_t)h * nb) * BLK;
  float M = -1e30f, L = 0.f;
  for (int t = t0; t < t1; ++t) {
    const float4 v = tstat[(int64_t)t * BLK + r];
    const float tot = v.y + v.z;
    if (v.x > M) {
      L = L * fast_exp2((M - v.x) * sl2) + tot;
      M = v.x;
    } else {
      L += tot * fast_exp2((v.x - M) * sl2);
    }
  }
  stats[((int64_t)vh * nchunk + chunk) * BLK + r] = make_float2(M, L);
}

// Row normaliser of the proxy rows: M = max over chunks, 1/L with L rescaled to
// M.  Eight groups of 128 threads take every eighth chunk; their partial
// (max, sum) pairs are merged in group order, so the result is reproducible.
constexpr int CMB_GROUPS = 8;
__global__ __launch_bounds__(BLK * CMB_GROUPS) void proxy_combine_kernel(const float2* __restrict__ stats,
                                                                         float2* __restrict__ rowstat,
                                                                         const SeqList seqs, int hq, int nchunk,
                                                                         int dense_below_n, float sl2) {
  __shared__ float2 part[CMB_GROUPS][BLK];
  const int h = blockIdx.x, r = threadIdx.x % BLK, grp = threadIdx.x / BLK;   // h: virtual head
  const int nb = seqs.nb[h / hq];
  if (seq_dense(nb, dense_below_n)) return;
  const int nc = rs_chunks(nb);
  const float2* p = stats + (int64_t)h * nchunk * BLK + r;
  float M = -1e30f;
  for (int c = grp; c < nc; c += CMB_GROUPS) M = fmaxf(M, p[(int64_t)c * BLK].x);
  float L = 0.f;
  for (int c = grp; c < nc; c += CMB_GROUPS) {
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

// Tile sums: one wave per (head, tile); lane l takes rows l and l + 64 and
// rescales the stored sums by exp(m - M) / L of the row.
__global__ __launch_bounds__(256) void proxy_tilesum_kernel(const float4* __restrict__ tstat,
                                                            const float2* __restrict__ rowstat,
                                                            float4* __restrict__ tiles, const SeqList seqs, int hq,
                                                            int hkv, int dense_below_n, float sl2) {
  const int vh = blockIdx.y, lane = threadIdx.x & 63, h = vh % hq;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const SeqPos sp = seq_pos(seqs, vh / hq, hq, hkv);
  const int nb = sp.nb;
  if (t >= nb || seq_dense(nb, dense_below_n)) return;
  const int64_t rowb = sp.rows + (int64_t)h * nb;
  float lo = 0.f, up = 0.f, an = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = lane + 64 * k;
    const float4 v = tstat[(rowb + t) * BLK + r];
    const float2 rs = rowstat[(int64_t)vh * BLK + r];
    const float wgt = fast_exp2((v.x - rs.x) * sl2) * rs.y;
    lo += v.y * wgt;
    up += v.z * wgt;
    an += v.w * wgt;
  }
  lo = wave_sum(lo);
  up = wave_sum(up);
  an = wave_sum(an);
  if (lane == 0) tiles[rowb + t] = make_float4(lo, up, an, 0.f);
}

hipError_t launch_proxy(int fp32, const void* Q, const void* K, const SeqList& seqs, int nb_max, int hq, int hkv,
                        const Strides& st, int w_sink, int w_local, int dense_below_n, void* tstat, void* stats,
                        void* rowstat, void* tiles, float* kbar, hipStream_t s) {
  const float sl2 = LOG2E / sqrtf((float)HD);
  const int nseq = seqs.nseq;
  const int G = hq / hkv;
  const int groups = hkv * ((G + (fp32 ? proxy_heads<float>() : proxy_heads<bf16>()) - 1) /
                            (fp32 ? proxy_heads<float>() : proxy_heads<bf16>()));
  // key blocks per work-group: PCH, or fewer so that about two work-groups per
  // CU exist (short sequences would otherwise run a few long serial chains)
  const int64_t want = 2 * (int64_t)device_cu_count();
  const int64_t per_chunk = (int64_t)groups * nseq;
  const int64_t chunks = (want + per_chunk - 1) / per_chunk;
  const int kpc = (int)std::max<int64_t>(1, std::min<int64_t>(PCH, (nb_max + chunks - 1) / chunks));
  const dim3 grid((unsigned)(((nb_max + kpc - 1) / kpc) * groups), (unsigned)nseq);
  if (fp32) {
    proxy_tiles_kernel<float><<<grid, 256, 0, s>>>((const float*)Q, (const float*)K, (float4*)tstat, kbar, seqs, hq,
                                                   hkv, st.q_h, st.q_n, st.k_h, st.k_n, w_sink, w_local,
                                                   dense_below_n, sl2, kpc);
  } else {
    proxy_tiles_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)Q, (const bf16*)K, (float4*)tstat, kbar, seqs, hq,
                                                  hkv, st.q_h, st.q_n, st.k_h, st.k_n, w_sink, w_local,
                                                  dense_below_n, sl2, kpc);
  }
  const int nchunk = proxy_chunks(nb_max);
  const unsigned vheads = (unsigned)(nseq * hq);
  proxy_rowstat_kernel<<<dim3(nchunk, vheads), BLK, 0, s>>>((const float4*)tstat, (float2*)stats, seqs, hq, hkv,
                                                             nchunk, dense_below_n, sl2);
  proxy_combine_kernel<<<vheads, BLK * CMB_GROUPS, 0, s>>>((const float2*)stats, (float2*)rowstat, seqs, hq, nchunk,
                                                           dense_below_n, sl2);
  proxy_tilesum_kernel<<<dim3((nb_max + 3) / 4, vheads), 256, 0, s>>>((const float4*)tstat, (const float2*)rowstat,
                                                                      (float4*)tiles, seqs, hq, hkv, dense_below_n,
                                                                      sl2);
  return hipGetLastError();
}

}  // namespace crisp
