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
// used by Pooled Estimation, and in a bf16 prefill extra work-groups of the
// same launch re-lay V out for the attention that follows (vt.h), beside the
// selection instead of in a launch of their own.  Grid: blockIdx -> (key
// chunk, group of query heads of a KV group, KV head) so the work-groups
// sharing a K chunk run on one XCD and share its L2; the heads of a group
// share each K tile in LDS.
#include <algorithm>

#include "common.h"
#include "lanes.h"
#include "launch.h"
#include "tile.h"
#include "vt.h"

namespace crisp {

constexpr int PCH = 16;       // most key blocks per score work-group (fewer when the grid would be small)

// Key blocks per score work-group: PCH, or fewer so that a sequence alone
// would give about two work-groups per CU (short sequences would otherwise run
// a few long serial chains).  It depends on the sequence's own N_b only, so a
// sequence is chunked the same way alone and in a packed batch; the score pass
// writes one (max, sum) row partial per chunk, merged in chunk order.
// chunks1: target chunk count of a sequence, ceil(2 * CUs / work-groups per chunk).
__host__ __device__ inline int seq_kpc(int nb, int chunks1) {
  const int k = (nb + chunks1 - 1) / chunks1;
  return k < 1 ? 1 : (k > PCH ? PCH : k);
}
int proxy_chunks1(int fp32, int hq, int hkv) {
  const int G = hq / hkv;
  const int hpw = fp32 ? 1 : 2;   // query heads per score work-group (PX_HEADS for bf16)
  const int groups = hkv * ((G + hpw - 1) / hpw);
  const int want = 2 * device_cu_count();
  return (want + groups - 1) / groups;
}
int proxy_chunks(int fp32, const SeqList& seqs, int hq, int hkv) {
  const int c1 = proxy_chunks1(fp32, hq, hkv);
  int nch = 1;
  for (int i = 0; i < seqs.nseq; ++i) {
    const int nb = seqs.nb[i], kpc = seq_kpc(nb, c1);
    nch = std::max(nch, (nb + kpc - 1) / kpc);
  }
  return nch;
}

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

// Online merge of a tile's (max m, sum of exp(s - m)) into a row's running
// (M, L), in tile order.
__device__ __forceinline__ void merge_row(float& M, float& L, float m, float tot, float sl2) {
  if (m > M) {
    L = L * fast_exp2((M - m) * sl2) + tot;
    M = m;
  } else {
    L += tot * fast_exp2((m - M) * sl2);
  }
}

// ---- bf16 score pass: 8 waves per work-group, one query head per 4 waves
//
// Two query heads of a KV group share each K tile, which is
// copied into LDS by the tile loads themselves (buffer_load ... lds, no
// register staging), two stages deep.  Wave w serves head h0 + w/4 and query
// rows 32(w%4) .. +31; it takes S^T of a tile in two halves of 64 keys, so a
// wave needs about half the registers of a whole tile and four waves fit on
// each SIMD (two work-groups per CU, 72 KiB of LDS each, which keeps the two
// out of step with each other).  The row's tile max is the max of the two half
// maxima: the sums of the first half, taken relative to its own max, are
// rescaled once when the second half raises it.
constexpr int PX_HEADS = 2, PX_WAVES = 4 * PX_HEADS, PX_ROWS = BLK / PX_WAVES;   // PX_ROWS: K rows copied per wave
static_assert(PX_HEADS == 2, "proxy_kpc counts two query heads per bf16 score work-group");

typedef __attribute__((address_space(3))) void px_lds_void;
constexpr int PX_WAIT_VM0 = 0x0F70;   // s_waitcnt: vector-memory count 0 only

__device__ __forceinline__ void px_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16-byte chunk c of K row r sits at chunk c ^ (r & 15) of the row's 256 bytes:
// the 32 lanes reading one chunk of 32 consecutive rows hit 16 bank groups
// twice, every pair conflict-free.  Wave w copies rows PX_ROWS w .. + PX_ROWS-1
// with 1 KB loads (lane L of load i: row PX_ROWS w + 4i + L/16, physical chunk
// L % 16).
struct PxCopy {   // the offsets are formed at each issue: a few ALU ops per tile, no registers held
  uint32_t row_bytes;
  int w, lane;
  __device__ void issue(const bf16* tile, int bytes, char* dst) const {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)tile, 0, bytes, 0x00020000);
    const int pc = lane & 15;
#pragma unroll
    for (int i = 0; i < PX_ROWS / 4; ++i) {
      const int r = PX_ROWS * w + 4 * i + (lane >> 4);
      const uint32_t off = (uint32_t)r * row_bytes + ((uint32_t)(pc ^ (r & 15)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (px_lds_void*)(dst + (PX_ROWS * w + 4 * i) * 256), 16, off, 0,
                                               0, 0);
    }
  }
};

__global__ __launch_bounds__(PX_WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) void proxy_scores_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, float4* __restrict__ tstat, float* __restrict__ kbar,
    float2* __restrict__ stats, const SeqList seqs, int hq, int hkv, int64_t sq_h, int64_t sq_n, int64_t sk_h,
    int64_t sk_n, int w_sink, int w_local, int dense_below_n, float sl2, int chunks1, int nchunk, int nscore,
    VtJob vt) {
  if ((int)blockIdx.x >= nscore) {   // the V re-layout of a prefill: two tiles per work-group
    const int tid = threadIdx.x;
    // the re-layout work-groups of every grid row (sequence), numbered row after row
    const int64_t wg = (int64_t)blockIdx.y * (gridDim.x - nscore) + (blockIdx.x - nscore);
    const int64_t tile = 2 * wg + (tid >> 8);   // tile = g * nb + kb
    if (wg == 0 && tid < ATTN_QUEUE_INTS) vt.queue[tid] = 0;
    if (tile < (int64_t)hkv * vt.nb)
      vt_tile_bf16((const bf16*)vt.V, (bf16*)vt.Vt, vt.sv_h, vt.sv_n, vt.nb, (int)(tile % vt.nb), (int)(tile / vt.nb),
                   tid & 255);
    return;
  }
  __shared__ __attribute__((aligned(1024))) char sK0[BLK * 256];
  __shared__ __attribute__((aligned(1024))) char sK1[BLK * 256];
  __shared__ __attribute__((aligned(16))) float red[2][PX_WAVES][HD];   // K-bar partials per (tile parity, 16-row group)
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = w >> 2, wq = w & 3;   // head of the group, row group (wave-uniform)
  const int G = hq / hkv, npg = (G + PX_HEADS - 1) / PX_HEADS;
  const int chunk = blockIdx.x / (hkv * npg), rem = blockIdx.x % (hkv * npg);
  const int kvh = rem % hkv, hp = rem / hkv;
  const int h0 = kvh * G + PX_HEADS * hp, nh = min(PX_HEADS, G - PX_HEADS * hp);
  // block means of K, once per KV head: with two or more work-groups per KV
  // head the first two take alternate tiles (tile kb by work-group kb % 2), so
  // that the pair reading each K tile does equal work, stays in step and the
  // second read of a tile finds it in L2
  const int kbar_ways = npg > 1 ? 2 : 1;
  auto kbar_owner = [&](int kb) __attribute__((always_inline)) { return hp == kb % kbar_ways; };
  const bool scores = hg < nh;         // this wave has a head
  const SeqPos sp = seq_pos(seqs, blockIdx.y, hq, hkv);
  const int nb = sp.nb;
  const int64_t n = (int64_t)nb * BLK;
  const int kpc = seq_kpc(nb, chunks1);
  if (chunk * kpc >= nb || seq_dense(nb, dense_below_n)) return;
  Q += sp.tok * sq_n;
  K += sp.tok * sk_n;
  float4* ts = tstat + (sp.rows + (int64_t)(h0 + hg) * nb) * BLK;
  kbar += sp.kvrows * HD;
  const int qrow = 32 * wq + l32;
  Tile<bf16>::QFrag qf;
  if (scores) Tile<bf16>::load_q(qf, Q + (int64_t)(h0 + hg) * sq_h + (int64_t)((nb - 1) * BLK + qrow) * sq_n, g);
  const int kb0 = chunk * kpc, kb1 = min(nb, kb0 + kpc);
  const bf16* Kh = K + (int64_t)kvh * sk_h;
  float rM = -1e30f, rL = 0.f;   // the row's max and sum over this chunk's key blocks
  const uint32_t krow = (uint32_t)(sk_n * 2);
  const int kspan = (int)((BLK - 1) * krow + 256);
  const PxCopy kc{krow, w, lane};
  uint32_t kx[8];   // S^T A operand: key row 32t + l32, d chunk 2c + g (t adds 8192 bytes)
#pragma unroll
  for (int c = 0; c < 8; ++c) kx[c] = l32 * 256 + (((2 * c + g) ^ (l32 & 15)) << 4);
  // K-bar partials, taken by the second head's four waves only (each for two
  // row groups vw = 2 wq, 2 wq + 1), so that the first head's waves sharing
  // their SIMDs start on the scores while they sum: lane L of row group vw sums
  // rows PX_ROWS vw + 4i + L/16 of columns 8(L%16) .. +7
  const int kb_c = lane & 15;
  const bf16x2 px_ones = {(bf16)1.f, (bf16)1.f};
  auto kbar_partials = [&](const char* cur, int par, int vw) __attribute__((always_inline)) {
    const int kb_r0 = PX_ROWS * vw + (lane >> 4);
    float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // rows r and r + 4 at a time: the same column of both side by side
    // (v_perm), then both added with one v_dot2 against (1, 1), two
    // instructions per pair of elements
#pragma unroll
    for (int i = 0; i < PX_ROWS / 4; i += 2) {
      const int r = kb_r0 + 4 * i;
      const uint4 u0 = *(const uint4*)(cur + r * 256 + ((kb_c ^ (r & 15)) << 4));
      const uint4 u1 = *(const uint4*)(cur + (r + 4) * 256 + ((kb_c ^ ((r + 4) & 15)) << 4));
      const unsigned a[4] = {u0.x, u0.y, u0.z, u0.w}, b[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const unsigned lo = __builtin_amdgcn_perm(b[p], a[p], 0x05040100u);   // column 2p of both rows
        const unsigned hi = __builtin_amdgcn_perm(b[p], a[p], 0x07060302u);   // column 2p + 1
        cs[2 * p] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lo), px_ones, cs[2 * p], false);
        cs[2 * p + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hi), px_ones, cs[2 * p + 1], false);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cs[j] += __shfl_xor(cs[j], 16, 64);
      cs[j] += __shfl_xor(cs[j], 32, 64);
    }
    if (lane < 16) {
      *(f32x4*)&red[par][vw][8 * lane] = f32x4{cs[0], cs[1], cs[2], cs[3]};
      *(f32x4*)&red[par][vw][8 * lane + 4] = f32x4{cs[4], cs[5], cs[6], cs[7]};
    }
  };
  auto kbar_final = [&](int kb, int par) __attribute__((always_inline)) {
    if (tid < HD) {
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < PX_WAVES; ++v) sum += red[par][v][tid];
      kbar[((int64_t)kvh * nb + kb) * HD + tid] = sum * (1.f / BLK);
    }
  };

  float4 pend = make_float4(0.f, 0.f, 0.f, 0.f);   // the last tile's row statistics, not yet stored
  int pend_kb = -1;
  auto tile = [&](int kb, const char* cur, char* nxt, int par) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(PX_WAIT_VM0);   // this wave's share of tile kb has landed
    px_barrier();                              // all of it has; every wave left the other stage
    if (kb + 1 < kb1) kc.issue(Kh + (int64_t)(kb + 1) * BLK * sk_n, kspan, nxt);
    // the previous tile's row statistics are stored only now, after this
    // tile's copy is issued: the wait at the start of the next tile (which
    // counts stores too) then finds the store long completed
    if (pend_kb >= 0 && g == 0) ts[(int64_t)pend_kb * BLK + qrow] = pend;
    // the last tile's partials were written before the barrier
    if (kb > kb0 && kbar_owner(kb - 1)) kbar_final(kb - 1, par ^ 1);
    if (hg == 1 && kbar_owner(kb)) {
      kbar_partials(cur, par, 2 * wq);
      kbar_partials(cur, par, 2 * wq + 1);
    }
    if (!scores) return;
    const bool last = kb == nb - 1;
    const int64_t j0 = (int64_t)kb * BLK;
    const bool touches_anchor = (j0 < w_sink) || (j0 + BLK > n - w_local);
    // anchor windows relative to the tile, clamped to [-1, BLK]: key c of the
    // tile is in the sink window iff c < ws_lim, in the local one iff c >= wl_lim
    const int ws_lim = (int)min<int64_t>(BLK, max<int64_t>(-1, (int64_t)w_sink - j0));
    const int wl_lim = (int)min<int64_t>(BLK + 1, max<int64_t>(-1, n - w_local - j0));
    float m = -INFINITY, lo = 0.f, up = 0.f, an = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 s[2] = {f32x16{}, f32x16{}};
      // fragments double-buffered in source order (the reads for step c + 1 go
      // out before the MFMAs of step c), which bounds the registers in flight
      bf16x8 fk[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) fk[0][t] = *(const bf16x8*)(cur + kx[0] + 8192 * (2 * hf + t));
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c + 1 < 8) {
#pragma unroll
          for (int t = 0; t < 2; ++t) fk[(c + 1) & 1][t] = *(const bf16x8*)(cur + kx[c + 1] + 8192 * (2 * hf + t));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 2; ++t) s[t] = mfma_bf16(fk[c & 1][t], qf.v[c], s[t]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (last) {   // keys after the query row are masked
        int lim = qrow;
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * (2 * hf + t) + mfma32_row(i, g) > lim) s[t][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
      mx = pair_max(mx);   // half 0 holds key 0 of every row: finite after it
      if (hf == 1 && mx > m) {
        const float r = fast_exp2((m - mx) * sl2);
        lo *= r;
        up *= r;
        an *= r;
      }
      m = fmaxf(m, mx);
      const float mb = m * sl2;
      // key c = 32t' + .. (t' = 2hf + t) against rows 32wq .. 32wq+31: t' < wq
      // all lower, t' > wq all upper, t' = wq split per score
      if (!last && !touches_anchor) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int tt = 2 * hf + t;
          float a = 0.f, b = 0.f;
          if (tt == wq) {
            int lim = l32 - 4 * g;   // key 32tt + 8(i/4) + 4g + i%4 <= row 32wq + l32
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = fast_exp2(fmaf(s[t][i], sl2, -mb));
              if (8 * (i >> 2) + (i & 3) <= lim) a += p;
              else b += p;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) a += fast_exp2(fmaf(s[t][i], sl2, -mb));
            if (tt > wq) { b = a; a = 0.f; }
          }
          lo += a;
          up += b;
        }
      } else {
        // score i of sub-tile tt is key 32tt + 4g + ci, ci = 8(i/4) + i%4: the
        // tests against the row and the anchor windows become tests of the
        // compile-time ci against three per-lane limits
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int tt = 2 * hf + t;
          if (tt > wq && last) continue;
          int dl = qrow - 32 * tt - 4 * g;   // lower part: ci <= dl
          int ds = ws_lim - 32 * tt - 4 * g; // sink window: ci < ds
          int dw = wl_lim - 32 * tt - 4 * g; // local window: ci >= dw
          asm volatile("" : "+v"(dl), "+v"(ds), "+v"(dw));
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ci = 8 * (i >> 2) + (i & 3);
            const float p = fast_exp2(fmaf(s[t][i], sl2, -mb));
            const bool lower = tt < wq || (tt == wq && ci <= dl);
            if (lower) lo += p;
            else if (!last) up += p;
            if (touches_anchor && (lower || !last) && (ci < ds || ci >= dw)) an += p;
          }
        }
      }
    }
    lo = pair_sum(lo);
    up = pair_sum(up);
    an = pair_sum(an);
    pend = make_float4(m, lo, up, an);
    pend_kb = kb;
    merge_row(rM, rL, m, lo + up, sl2);
  };

  kc.issue(Kh + (int64_t)kb0 * BLK * sk_n, kspan, sK0);
  for (int kb = kb0; kb < kb1; kb += 2) {
    tile(kb, sK0, sK1, 0);
    if (kb + 1 < kb1) tile(kb + 1, sK1, sK0, 1);
  }
  if (pend_kb >= 0 && g == 0) ts[(int64_t)pend_kb * BLK + qrow] = pend;
  if (scores && g == 0)
    stats[(((int64_t)blockIdx.y * hq + h0 + hg) * nchunk + chunk) * BLK + qrow] = make_float2(rM, rL);
  if (kbar_owner(kb1 - 1)) {
    __builtin_amdgcn_s_waitcnt(0);
    px_barrier();
    kbar_final(kb1 - 1, (kb1 - 1 - kb0) & 1);
  }
}

// fp32 score pass: scores of the last query block against kpc <= PCH key
// blocks, one query head per work-group of 4 waves, one K tile in LDS at a
// time; per (tile, row): tile max m of the row and the sums of exp(s - m)
// over the lower part (key column <= row: slash bin N_b-1-kb), the upper part
// (bin N_b-2-kb) and the anchor windows.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void proxy_tiles_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, float4* __restrict__ tstat, float* __restrict__ kbar,
    float2* __restrict__ stats, const SeqList seqs, int hq, int hkv, int64_t sq_h, int64_t sq_n, int64_t sk_h,
    int64_t sk_n, int w_sink, int w_local, int dense_below_n, float sl2, int chunks1, int nchunk) {
  __shared__ __attribute__((aligned(16))) float sK[BLK * Tile<float>::KP];
  __shared__ __attribute__((aligned(16))) float red[2][HD];   // K-bar column sums per half tile
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: the t-vs-w branches are scalar
  const int G = hq / hkv;
  const int chunk = blockIdx.x / (hkv * G), rem = blockIdx.x % (hkv * G);
  const int kvh = rem % hkv, hp = rem / hkv;
  const int h = kvh * G + hp;
  const bool kbar_wg = hp == 0;   // block means of K, once per KV head
  const SeqPos sp = seq_pos(seqs, blockIdx.y, hq, hkv);
  const int nb = sp.nb;
  const int64_t n = (int64_t)nb * BLK;
  const int kpc = seq_kpc(nb, chunks1);
  if (chunk * kpc >= nb || seq_dense(nb, dense_below_n)) return;
  Q += sp.tok * sq_n;
  K += sp.tok * sk_n;
  tstat += (sp.rows + (int64_t)h * nb) * BLK;
  kbar += sp.kvrows * HD;
  const int qrow = 32 * w + l32;
  Tile<float>::QFrag qf;
  Tile<float>::load_q(qf, Q + (int64_t)h * sq_h + (int64_t)((nb - 1) * BLK + qrow) * sq_n, g);
  const int kb0 = chunk * kpc, kb1 = min(nb, kb0 + kpc);
  const float* Kh = K + (int64_t)kvh * sk_h;
  float rM = -1e30f, rL = 0.f;   // the row's max and sum over this chunk's key blocks
  for (int kb = kb0; kb < kb1; ++kb) {
    __syncthreads();
    Tile<float>::load_k(sK, Kh + (int64_t)kb * BLK * sk_n, sk_n, tid);
    __syncthreads();
    if (kbar_wg) {  // block mean of K for Pooled Estimation
      const int d = tid & 127, half = tid >> 7;
      float sum = 0.f;
      for (int r = 0; r < 64; ++r) sum += sK[(64 * half + r) * Tile<float>::KP + d];
      red[half][d] = sum;
      __syncthreads();
      if (half == 0) kbar[((int64_t)kvh * nb + kb) * HD + d] = (red[0][d] + red[1][d]) * (1.f / BLK);
    }
    f32x16 s[4];
    Tile<float>::st(s, sK, qf, l32, g);
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
    if (g == 0) tstat[(int64_t)kb * BLK + qrow] = make_float4(mx, lo, up, an);
    merge_row(rM, rL, mx, lo + up, sl2);
  }
  if (g == 0) stats[(((int64_t)blockIdx.y * hq + h) * nchunk + chunk) * BLK + qrow] = make_float2(rM, rL);
}

// Row normaliser of the proxy rows from the score pass's chunk partials: M =
// max over chunks, 1/L with L rescaled to M.  Eight groups of 128 threads take every eighth chunk; their partial
// (max, sum) pairs are merged in group order, so the result is reproducible.
constexpr int CMB_GROUPS = 8;
__global__ __launch_bounds__(BLK * CMB_GROUPS) void proxy_combine_kernel(const float2* __restrict__ stats,
                                                                         float2* __restrict__ rowstat,
                                                                         const SeqList seqs, int hq, int nchunk,
                                                                         int chunks1, int dense_below_n, float sl2) {
  __shared__ float2 part[CMB_GROUPS][BLK];
  const int h = blockIdx.x, r = threadIdx.x % BLK, grp = threadIdx.x / BLK;   // h: virtual head
  const int nb = seqs.nb[h / hq];
  if (seq_dense(nb, dense_below_n)) return;
  const int kpc = seq_kpc(nb, chunks1);
  const int nc = (nb + kpc - 1) / kpc;   // the score pass's chunks of this sequence
  const float2* p = stats + (int64_t)h * nchunk * BLK + r;
  float M = -1e30f, L = 0.f;
  for (int c0 = grp; c0 < nc; c0 += 4 * CMB_GROUPS) {   // four chunks' loads in flight, then merged in chunk order
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[(int64_t)min(c0 + CMB_GROUPS * u, nc - 1) * BLK];
    float m4 = M;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + CMB_GROUPS * u < nc) m4 = fmaxf(m4, v[u].x);
    L *= fast_exp2((M - m4) * sl2);
    M = m4;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + CMB_GROUPS * u < nc) L += v[u].y * fast_exp2((v[u].x - M) * sl2);
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
                        void* rowstat, void* tiles, float* kbar, const VtJob& vt, hipStream_t s) {
  const float sl2 = LOG2E / sqrtf((float)HD);
  const int nseq = seqs.nseq;
  const int G = hq / hkv;
  const int hpw = fp32 ? 1 : PX_HEADS;   // query heads per score work-group
  const int groups = hkv * ((G + hpw - 1) / hpw);
  const int chunks1 = proxy_chunks1(fp32, hq, hkv);
  const int nchunk = proxy_chunks(fp32, seqs, hq, hkv);
  // every sequence on the dense path (below the length gate, or N_b <= 2): no
  // scores are needed, and the selection launch does the V re-layout of a
  // bf16 prefill beside writing the full lists
  bool all_dense = true;
  for (int i = 0; i < nseq; ++i) all_dense = all_dense && seq_dense(seqs.nb[i], dense_below_n);
  if (all_dense) return hipSuccess;
  const int nscore = nchunk * groups;
  const dim3 grid((unsigned)nscore, (unsigned)nseq);
  if (fp32) {
    proxy_tiles_f32_kernel<<<grid, 256, 0, s>>>((const float*)Q, (const float*)K, (float4*)tstat, kbar,
                                                 (float2*)stats, seqs, hq, hkv, st.q_h, st.q_n, st.k_h, st.k_n, w_sink,
                                                 w_local, dense_below_n, sl2, chunks1, nchunk);
  } else {
    static_assert(PX_WAVES * 64 == 512, "the fused V re-layout takes two 256-thread tiles per work-group");
    // the V re-layout's work-groups (two tiles each) spread over the grid's rows
    const int64_t vt_wgs = vt.V ? ((int64_t)vt.nb * hkv + 1) / 2 : 0;
    const dim3 g2((unsigned)(nscore + (vt_wgs + nseq - 1) / nseq), (unsigned)nseq);
    proxy_scores_bf16_kernel<<<g2, PX_WAVES * 64, 0, s>>>((const bf16*)Q, (const bf16*)K, (float4*)tstat, kbar,
                                                          (float2*)stats, seqs, hq, hkv, st.q_h, st.q_n, st.k_h,
                                                          st.k_n, w_sink, w_local, dense_below_n, sl2, chunks1,
                                                          nchunk, nscore, vt);
  }
  const unsigned vheads = (unsigned)(nseq * hq);
  proxy_combine_kernel<<<vheads, BLK * CMB_GROUPS, 0, s>>>((const float2*)stats, (float2*)rowstat, seqs, hq, nchunk,
                                                           chunks1, dense_below_n, sl2);
  proxy_tilesum_kernel<<<dim3((nb_max + 3) / 4, vheads), 256, 0, s>>>((const float4*)tstat, (const float2*)rowstat,
                                                                      (float4*)tiles, seqs, hq, hkv, dense_below_n,
                                                                      sl2);
  return hipGetLastError();
}

}  // namespace crisp
