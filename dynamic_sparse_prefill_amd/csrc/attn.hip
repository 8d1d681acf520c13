// Causal block-sparse flash attention forward for gfx950, and its dense form.
//
// Computes, for every query head h and query block qb, the rows
//   O_i = sum_{j in J_i} softmax_j(q_i . k_j / sqrt(d)) v_j,
//   J_i = { j <= i : block(j) is listed for (h, qb) }
// which is exact softmax attention under the block mask M_S of the CRISP paper
// (§2, problem statement; the sparse kernel computes exact attention on the
// blocks it selects).  Dense attention is the same loop over every block
// 0..qb.
//
// Design:
//  * Scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so
//    each lane owns one query row and 64 of its 128 scores per key tile; the
//    online-softmax max / sum are in-lane plus one lane^32 exchange.
//  * The output is accumulated transposed, O^T += V^T P^T: P (rounded to bf16)
//    is already in the B-operand layout, and V^T comes from LDS.  V is
//    re-laid out once per call as per-block transposed tiles [d][key] so that
//    the tile copy to LDS is a plain coalesced 32 KB copy.
//  * One work-group = one head x two adjacent query blocks (256 rows, 8
//    waves).  K and V^T tiles go straight from global memory to LDS (buffer
//    loads with the LDS bit, no staging registers), XOR-swizzled for
//    conflict-free 16-byte reads, double-buffered so the next block streams
//    in during a whole iteration; one barrier per key block.
//  * Operand fragments are read from LDS one MFMA step ahead (the reads of
//    step c + 1 are in flight while the MFMAs of step c run), and every MFMA
//    waits only for its own fragment.  The compiler can count the LDS reads
//    that precisely only while the copy in flight is a buffer (MUBUF) load:
//    a global (FLAT) copy into LDS makes it wait for every outstanding LDS
//    read at each use.
//  * Scheduling: a persistent grid (one work-group per CU) pulls (pair, head)
//    items from 8 per-XCD queues, two KV groups at a time, longest rows
//    first, stealing from other queues at the end: every CU stays busy
//    whatever the list lengths, and K/V is shared through L2 and the
//    last-level cache.
#include <algorithm>

#include "common.h"
#include "lanes.h"
#include "launch.h"
#include "tile.h"
#include "vt.h"

namespace crisp {

constexpr int NQUEUE = 8;  // work queues of the persistent attention kernel (one per XCD)
// Sparse attention of long sequences walks the item order twice, each pass
// with its own NQUEUE counters: first it takes only the items whose lists
// cover more than a quarter of their causal key blocks, then the rest.  Long
// items then start in waves of about equal length, as in dense attention, and
// the work-groups of an XCD walk the same K / V tiles of their KV group at
// about the same time, sharing them through L2; with short items interleaved,
// long ones would start at scattered times and walk unrelated tiles.  The
// short items fill the end of the launch.  The second walk costs every
// work-group a pull from each queue; with a few items per CU (sequences under
// TWO_PASS_NB blocks) that outweighs the locality, and sparse attention makes
// one pass over all items, as dense attention always does.
constexpr int NPHASE = 2;
constexpr int TWO_PASS_NB = 256;
static_assert(NQUEUE * NPHASE == ATTN_QUEUE_INTS, "the V re-layout clears ATTN_QUEUE_INTS counters");

// ------------------------------------------------------------------ V re-layout

// V [hkv][n][d] (token stride sv_n) -> Vt [hkv][nb][d][128] (the layout of
// vt.h).  Also clears the attention kernels' work-queue counters (they run
// right after).  fp32: one tile per work-group through LDS; bf16: two tiles per
// 512-thread work-group in registers (vt_tile_bf16).
__global__ __launch_bounds__(256) void transpose_v_f32_kernel(const float* __restrict__ V, float* __restrict__ Vt,
                                                              int nb, int64_t sv_h, int64_t sv_n, int* queue) {
  __shared__ float tile[BLK][HD + 2];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  if (kb == 0 && g == 0 && tid < ATTN_QUEUE_INTS && queue) queue[tid] = 0;
  const float* src = V + (int64_t)g * sv_h + (int64_t)kb * BLK * sv_n;
  for (int e = tid; e < BLK * HD; e += 256) {
    const int r = e / HD, d = e % HD;
    tile[r][d] = src[(int64_t)r * sv_n + d];
  }
  __syncthreads();
  float* dst = Vt + ((int64_t)g * nb + kb) * (BLK * HD);
  for (int e = tid; e < BLK * HD; e += 256) {
    const int d = e / BLK, r = e % BLK;
    dst[d * BLK + r] = tile[r][d];
  }
}

__global__ __launch_bounds__(512) void transpose_v_bf16_kernel(const bf16* __restrict__ V, bf16* __restrict__ Vt,
                                                               int nb, int hkv, int64_t sv_h, int64_t sv_n,
                                                               int* queue) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid < ATTN_QUEUE_INTS && queue) queue[tid] = 0;
  const int64_t tile = 2 * (int64_t)blockIdx.x + (tid >> 8);   // tile = g * nb + kb
  if (tile >= (int64_t)hkv * nb) return;
  vt_tile_bf16(V, Vt, sv_h, sv_n, nb, (int)(tile % nb), (int)(tile / nb), tid & 255);
}

// ------------------------------------------------------------------ bf16 MFMA kernel

typedef __attribute__((address_space(3))) void lds_void;

// gfx9 s_waitcnt immediates: wait for vector-memory count <= N only.
constexpr int WAIT_VM0 = 0x0F70;

__device__ __forceinline__ void block_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A 128-row x 256-byte tile goes to LDS as 16-byte chunks, chunk c of row r at
// physical chunk c ^ (r & 15): 16 lanes reading the same logical chunk of 16
// consecutive rows hit 16 different bank groups.  With 8 waves, wave w copies
// rows 16w..16w+15 with 4 buffer loads of 1 KB (4 rows) each that write LDS
// directly; lane L of load i fills row 16w + 4i + L/16, physical chunk L%16.
// The buffer resource is based at the tile and spans exactly its bytes, so an
// offset outside the tile would read zeros rather than other memory.
struct TileCopy {
  uint32_t off[4];
  __device__ void init(int wu, int lane, uint32_t row_bytes) {
    const int pc = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wu + 4 * i + (lane >> 4);
      off[i] = (uint32_t)r * row_bytes + ((uint32_t)(pc ^ (r & 15)) << 4);
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, char* dst, int wu) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (16 * wu + 4 * i) * 256), 16, off[i], 0, 0, 0);
  }
};

// buffer resource over `bytes` bytes at p (raw: no stride, no swizzle)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, bytes, 0x00020000);
}

constexpr int TILE_BYTES = BLK * 256;  // one K or V^T tile in LDS

// Offset operand of the V^T reads of one key chunk.  A DS read adds only a
// 16-bit constant to its address register.  The K stages take the first 64 KiB
// of LDS, so every K read folds stage, tile and chunk into that constant; the
// V^T stages lie above, so the register has to carry the stage-0 V^T address.
// The empty asm stops the compiler from folding that address back into a new
// constant per read (one VALU op per read); the reads still index the stage
// arrays, which is how the compiler tells them from the copy into the other
// stage and issues no wait for it.
__device__ __forceinline__ uint32_t vt_operand(uint32_t lane_off, uint32_t vbase) {
  uint32_t r = lane_off + vbase;
  __asm__ volatile("" : "+v"(r));
  return r - vbase;
}

// Work queues.  The kernel is persistent (one work-group per CU).  A unit of
// work is one (query-block pair, KV head) with its G query heads, whose items
// are consecutive in a queue so they run side by side and share each K/V tile
// through L2.  Units are numbered two KV groups at a time (see queue_item),
// longest rows first, and unit u belongs to queue u % 8: every XCD works on
// the same two groups at once, keeping the K/V working set small.  Work-group
// b starts on queue b % 8 (dispatch places it on XCD b % 8), takes items from
// it, then steals from the other queues until all are empty.  Only locality
// depends on the placement; every item is taken exactly once.

// t-th item of queue x -> (sequence, pair, kvh, h); false once the queue is
// exhausted.  Units are numbered sequence after sequence.  Within a sequence
// whose K and V are larger than the last-level cache, KV groups go two at a
// time (2j, 2j+1 alternating unit by unit, longest rows first; a last odd
// group alone), so all queues stream the K/V of the same two groups at any
// moment: a working set that stays in that cache.  When K and V fit in it
// (sq.pair_major), units go pair by pair over all KV groups, longest rows
// first: plain longest-first packing, which evens out the end of a short
// launch (8k-64k tokens: 5-12% faster; at 512k it costs 8%).
// Rank rho (0 = longest) of a group's np pairs, dealt to S queues in turn
// (queue rho % S takes its (rho / S)-th pair), mapped to the pair rank that
// queue gets: chunks of PAIR_CHUNK consecutive ranks, the S queues taking
// chunks in turn, so the items an XCD runs at one time are of neighbouring
// pairs (about equal lengths, nearly the same key blocks) rather than of every
// S-th pair; the ranks past the last whole round of chunks keep their order.
// A bijection on [0, np).
constexpr int PAIR_CHUNK = 16;
__device__ __forceinline__ int chunked_rank(int rho, int np, int S) {
  const int round = S * PAIR_CHUNK, whole = (np / round) * round;
  if (rho >= whole) return rho;
  const int q = rho % S, k = rho / S;
  return PAIR_CHUNK * (S * (k / PAIR_CHUNK) + q) + k % PAIR_CHUNK;
}

__device__ inline bool queue_item(int x, int t, const SeqTable& sq, int hq, int hkv, int& seq, int& pair, int& kvh,
                                  int& h) {
  const int G = hq / hkv;
  const int u = NQUEUE * (t / G) + x;                       // the queue's (t/G)-th unit
  if (u >= sq.unit_off[sq.nseq]) return false;
  int i = 0;
  while (u >= sq.unit_off[i + 1]) ++i;
  const int v = u - sq.unit_off[i];
  const int np = (sq.nb[i] + 1) >> 1;
  seq = i;
  if (sq.pair_major) {
    kvh = v % hkv;
    pair = np - 1 - v / hkv;
    h = kvh * G + t % G;
    return true;
  }
  const int gp = v / (2 * np), r = v % (2 * np);
  if (2 * gp + 1 < hkv) {
    kvh = 2 * gp + (r & 1);
    pair = np - 1 - chunked_rank(r >> 1, np, NQUEUE / 2);
  } else {                                                  // odd group count: the last group alone
    kvh = 2 * gp;
    pair = np - 1 - chunked_rank(r, np, NQUEUE);
  }
  h = kvh * G + t % G;
  return true;
}

// An ascending key-block list read through a window of 64 entries, one per
// lane of a VGPR, with the next window already loaded: an entry costs one
// v_readlane instead of a dependent scalar load per key block, and a window's
// load is consumed only 64 entries later.  Loads use a clamped index (no
// select on the loaded value, which would wait for it at once).
struct ListWindow {
  const int32_t* l;
  int n, base, cur, nxt;
  __device__ void init(const int32_t* list, int len, int lane) {
    l = list;
    n = len;
    base = 0;
    cur = nxt = 0;
    if (n > 0) {
      cur = l[min(lane, n - 1)];
      nxt = l[min(64 + lane, n - 1)];
    }
  }
  // entry i, 0 <= i < n, i never below a previous call's (the walk is forward)
  __device__ int at(int i, int lane) {
    while (i - base >= 64) {                 // wave-uniform
      base += 64;
      cur = nxt;
      nxt = l[min(base + 64 + lane, n - 1)];
    }
    return __builtin_amdgcn_readlane(cur, i - base);
  }
};

// Walks the union of the ascending key-block lists of the two query blocks of
// a work-group.  Entries outside [0, qb] of their own block are skipped.
struct PairCursor {
  ListWindow a, b;
  int ia, ib, qa, qb;
  __device__ int head(ListWindow& l, int& i, int q, int lane) {
    while (i < l.n) {
      const int k = l.at(i, lane);
      if ((unsigned)k <= (unsigned)q) return k;
      ++i;
    }
    return 0x7fffffff;
  }
  // next block of the union (-1 when done) and which halves list it
  __device__ int next(bool& in_a, bool& in_b, int lane) {
    const int x = head(a, ia, qa, lane), y = head(b, ib, qb, lane);
    const int k = min(x, y);
    in_a = (x == k) && k != 0x7fffffff;
    in_b = (y == k) && k != 0x7fffffff;
    if (in_a) ++ia;
    if (in_b) ++ib;
    return k == 0x7fffffff ? -1 : k;
  }
};

// One work-group = one query head x two adjacent query blocks (2p, 2p+1):
// waves 0-3 own block 2p, waves 4-7 block 2p+1, 32 rows per wave.  The K and
// V^T tiles of a key block are loaded once into LDS and used by both halves;
// tiles are double-buffered so the next block's copy runs during a whole
// iteration, with one barrier per key block.
template <bool DENSE>
__device__ __forceinline__ void fa_bf16_item(
    char* sK0, char* sV0, char* sK1, char* sV1, int pair, int kvh, int h,
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ Vt, bf16* __restrict__ O,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int nb, int hq, int hkv,
    int64_t sq_h, int64_t sq_n, int64_t sk_h, int64_t sk_n, int64_t so_h, int64_t so_n, int64_t vt_h, float sl2) {
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = w >> 2, wq = w & 3;
  const int G = hq / hkv;
  const int qlo = 2 * pair, qhi = 2 * pair + 1;
  const bool hi_ok = qhi < nb;
  const int qmine = half ? qhi : qlo;
  const bool rows_ok = half == 0 || hi_ok;

  PairCursor cur;
  cur.qa = qlo;
  cur.qb = hi_ok ? qhi : -1;
  cur.ia = cur.ib = 0;
  if (!DENSE) {
    const int64_t ra = (int64_t)h * nb + qlo;
    const int32_t p0 = row_ptr[ra], p1 = row_ptr[ra + 1];
    cur.a.init(col_idx + p0, p1 - p0, lane);
    if (hi_ok)
      cur.b.init(col_idx + p1, row_ptr[ra + 2] - p1, lane);
    else
      cur.b.init(col_idx + p0, 0, lane);
  }
  int dense_next = 0;
  auto next_block = [&](bool& ia, bool& ib) -> int {
    if (DENSE) {
      const int k = dense_next++;
      const int top = hi_ok ? qhi : qlo;
      ia = k <= qlo;
      ib = hi_ok && k <= qhi;
      return k <= top ? k : -1;
    }
    return cur.next(ia, ib, lane);
  };

  const int qrow = 32 * wq + l32;
  bf16* orow = O + (int64_t)h * so_h + (int64_t)(qmine * BLK + qrow) * so_n;

  const uint32_t krow = (uint32_t)(sk_n * 2);
  const char* Kh = (const char*)(K + (int64_t)kvh * sk_h);
  const char* Vh = (const char*)(Vt + (int64_t)kvh * vt_h);
  TileCopy kc, vc;
  kc.init(w, lane, krow);
  vc.init(w, lane, 256);
  const int kspan = (int)((BLK - 1) * krow + 256);
  auto issue = [&](int kb, char* dK, char* dV) {
    kc.issue(tile_rsrc(Kh + (int64_t)kb * BLK * krow, kspan), dK, w);
    vc.issue(tile_rsrc(Vh + (int64_t)kb * (BLK * HD * 2), BLK * HD * 2), dV, w);
  };

  bool a0, b0;
  int kb = next_block(a0, b0);
  if (kb >= 0) issue(kb, sK0, sV0);
  bool a1 = false, b1 = false;
  int kb1 = kb >= 0 ? next_block(a1, b1) : -1;

  Tile<bf16>::QFrag qf;
  if (rows_ok) Tile<bf16>::load_q(qf, Q + (int64_t)h * sq_h + (int64_t)(qmine * BLK + qrow) * sq_n, g);
  const uint32_t vbase = (uint32_t)(uintptr_t)(lds_void*)sV0;
  uint32_t kx[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) kx[c] = l32 * 256 + (((2 * c + g) ^ (l32 & 15)) << 4);

  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{};
  float m = -1e30f, l = 0.f;
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

  // One key block with its tiles in (cK, cV) while the next block's are copied
  // into (nK, nV).  The stages are separate LDS arrays named at compile time
  // (the loop below alternates two inlined copies of the step), so the
  // compiler can tell the reads of one stage from the copy into the other.
  auto step = [&](const char* cK, const char* cV, char* nK, char* nV) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);       // this wave's share of the tiles of kb has landed
    block_barrier();                            // all of them have; every wave left the other stage
    // the list lookup comes before the copy is issued: a window refill then has
    // nothing in flight to wait for (all loads completed at the wait above)
    bool a2 = false, b2 = false;
    const int kb2 = kb1 >= 0 ? next_block(a2, b2) : -1;
    if (kb1 >= 0) issue(kb1, nK, nV);
    const bool active = half ? b0 : a0;
    if (active) {
      f32x16 s[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = f32x16{};
      // Operand fragments are double-buffered in source order: the reads of
      // step c + 1 are issued before the MFMAs of step c (the scheduling
      // barriers keep that order), so each MFMA waits only for a read issued
      // four MFMAs earlier.  The last step reads the first V^T fragments.
      bf16x8 fk[2][4], fv[2][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) fk[0][t] = *(const bf16x8*)(cK + kx[0] + 8192 * t);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c + 1 < 8) {
#pragma unroll
          for (int t = 0; t < 4; ++t) fk[(c + 1) & 1][t] = *(const bf16x8*)(cK + kx[c + 1] + 8192 * t);
        } else {
          const uint32_t kv = vt_operand(kx[0], vbase);
#pragma unroll
          for (int u = 0; u < 4; ++u) fv[0][u] = *(const bf16x8*)(cV + kv + 8192 * u);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) s[t] = mfma_bf16(fk[c & 1][t], qf.v[c], s[t]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kb == qmine) {  // diagonal tile: keys after the query are masked
        // key 32t + 8(i/4) + 4g + i%4 > qrow  <=>  32t + 8(i/4) + i%4 > lim; lim is
        // formed from kb so the 64 compares are not hoisted out of the loop
        const int lim = qrow - 4 * g + (kb - qmine) * BLK;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * t + 8 * (i >> 2) + (i & 3) > lim) s[t][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
      mx = pair_max(mx);
      // Lazy running max: m is raised only when a row's tile max exceeds it by
      // more than 2^8 in probability, so most tiles skip rescaling O and l.
      // Exact softmax either way: p = exp2((s - m) sl2) <= 2^8 in fp32 / bf16.
      if (__ballot((mx - m) * sl2 > 8.f)) {
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2((m - mn) * sl2);
        l *= alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] *= alpha;
        m = mn;
      }
      const float mb = m * sl2;
      // P in bf16, already in the B-operand order of the O^T MFMAs; the row sum
      // is taken over the same rounded values (v_dot2 with (1, 1)).  P for key
      // chunk mm + 2 is formed while the MFMAs of chunk mm run.
      bf16x8 pb[8];
      auto form_p = [&](int mm) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          bf16x2 pr;
          pr[0] = (bf16)fast_exp2(fmaf(s[mm >> 1][8 * (mm & 1) + j], sl2, -mb));
          pr[1] = (bf16)fast_exp2(fmaf(s[mm >> 1][8 * (mm & 1) + j + 1], sl2, -mb));
          l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
          pb[mm][j] = pr[0];
          pb[mm][j + 1] = pr[1];
        }
      };
      form_p(0);
      form_p(1);
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) {
        if (mm + 1 < 8) {
          const uint32_t kv = vt_operand(kx[mm + 1], vbase);
#pragma unroll
          for (int u = 0; u < 4; ++u) fv[(mm + 1) & 1][u] = *(const bf16x8*)(cV + kv + 8192 * u);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma_bf16(fv[mm & 1][u], pb[mm], acc[u]);
        if (mm + 2 < 8) form_p(mm + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    kb = kb1; a0 = a1; b0 = b1;
    kb1 = kb2; a1 = a2; b1 = b2;
  };
  while (kb >= 0) {
    step(sK0, sV0, sK1, sV1);
    if (kb < 0) break;
    step(sK1, sV1, sK0, sV0);
  }
  if (!rows_ok) return;
  l += __shfl_xor(l, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (bf16)(acc[u][4 * j + e] * inv);
      *(bf16x4*)(orow + 32 * u + 8 * j + 4 * g) = o4;
    }
}

// Persistent loop: one work-group per CU takes items from the queues until
// all are empty.  `queue` holds NQUEUE counters per pass, zero at launch.
// passes == 1: one pass over every item.  passes == 2 (sparse only): the
// first pass takes only the items whose two lists hold more than a quarter of
// the pair's causal key blocks, the second the others.
template <bool DENSE>
__global__ __launch_bounds__(512, 2) void fa_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ Vt, bf16* __restrict__ O,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int* __restrict__ queue,
    const SeqTable sq, int nb_total, int hq, int hkv, int64_t sq_h, int64_t sq_n, int64_t sk_h, int64_t sk_n,
    int64_t so_h, int64_t so_n, float sl2, int passes) {
  // two stages of (K, V^T) tiles, each stage tile its own array; K first (see vt_operand)
  __shared__ __attribute__((aligned(1024))) char sK0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE_BYTES];
  __shared__ int s_item;
  const int home = blockIdx.x % NQUEUE;
  const int64_t vt_h = (int64_t)nb_total * (BLK * HD);
  for (int pass = 0; pass < passes; ++pass) {
    int* qs = queue + NQUEUE * pass;
    for (int k = 0; k < NQUEUE; ++k) {
      const int x = (home + k) % NQUEUE;
      while (true) {
        __builtin_amdgcn_s_waitcnt(0);              // nothing of the last item is still in flight
        __syncthreads();                            // every wave is done with the last item's LDS
        if (threadIdx.x == 0) s_item = atomicAdd(qs + x, 1);
        __syncthreads();
        int seq, pair, kvh, h;
        if (!queue_item(x, s_item, sq, hq, hkv, seq, pair, kvh, h)) break;
        if (!DENSE && passes > 1) {                 // long items in pass 0, short ones in pass 1
          const int nbs = sq.nb[seq], qlo = 2 * pair;
          const int32_t* rp = row_ptr + sq.rp[seq] + (int64_t)h * nbs + qlo;
          const bool two = qlo + 1 < nbs;
          const int len = (two ? rp[2] : rp[1]) - rp[0];
          const int causal = qlo + 1 + (two ? qlo + 2 : 0);
          if ((4 * len > causal) != (pass == 0)) continue;
        }
        const int64_t t0 = sq.tok[seq];
        fa_bf16_item<DENSE>(sK0, sV0, sK1, sV1, pair, kvh, h, Q + t0 * sq_n, K + t0 * sk_n, Vt + t0 * HD,
                            O + t0 * so_n, row_ptr + sq.rp[seq], col_idx + sq.col[seq], sq.nb[seq], hq, hkv, sq_h,
                            sq_n, sk_h, sk_n, so_h, so_n, vt_h, sl2);
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 MFMA kernel

template <bool DENSE>
__global__ __launch_bounds__(256, 1) void fa_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ Vt, float* __restrict__ O,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int nb, int hq, int hkv,
    int64_t sq_h, int64_t sq_n, int64_t sk_h, int64_t sk_n, int64_t so_h, int64_t so_n, int64_t vt_h, float sl2) {
  constexpr int KP = Tile<float>::KP, VP = 132;
  __shared__ __attribute__((aligned(16))) float sK[BLK * KP];
  __shared__ __attribute__((aligned(16))) float sV[HD * VP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int G = hq / hkv;
  const int bid = blockIdx.x;
  const int qb = nb - 1 - bid / hq;
  const int rem = bid % hq;
  const int kvh = rem % hkv, h = kvh * G + rem / hkv;
  int beg = 0, cnt = qb + 1;
  if (!DENSE) {
    const int64_t r = (int64_t)h * nb + qb;
    beg = row_ptr[r];
    cnt = row_ptr[r + 1] - beg;
  }
  const int qrow = 32 * w + l32;
  float* orow = O + (int64_t)h * so_h + (int64_t)(qb * BLK + qrow) * so_n;
  Tile<float>::QFrag qf;
  Tile<float>::load_q(qf, Q + (int64_t)h * sq_h + (int64_t)(qb * BLK + qrow) * sq_n, g);
  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{};
  float m = -1e30f, l = 0.f;
  for (int it = 0; it < cnt; ++it) {
    const int kb = DENSE ? it : col_idx[beg + it];
    if ((unsigned)kb > (unsigned)qb) continue;  // no key j <= i in a later block
    __syncthreads();
    Tile<float>::load_k(sK, K + (int64_t)kvh * sk_h + (int64_t)kb * BLK * sk_n, sk_n, tid);
    Tile<float>::load_k(sV, Vt + (int64_t)kvh * vt_h + (int64_t)kb * (BLK * HD), BLK, tid);
    __syncthreads();
    f32x16 s[4];
    Tile<float>::st(s, sK, qf, l32, g);
    if (kb == qb) {
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
    mx = pair_max(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2((m - mn) * sl2);
    const float mb = mn * sl2;
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[t][i], sl2, -mb));
        s[t][i] = p;
        rs += p;
      }
    l = fmaf(l, alpha, rs);
    m = mn;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] *= alpha;
    // O^T += V^T P^T, one key pair (lane halves) per v_mfma_f32_32x32x2f32
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * t + mfma32_row(i, g);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma_f32(sV[(32 * u + l32) * VP + key], s[t][i], acc[u]);
      }
  }
  l += __shfl_xor(l, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 o4 = make_float4(acc[u][4 * j] * inv, acc[u][4 * j + 1] * inv, acc[u][4 * j + 2] * inv,
                              acc[u][4 * j + 3] * inv);
      *(float4*)(orow + 32 * u + 8 * j + 4 * g) = o4;
    }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_transpose_v(int fp32, const void* V, void* Vt, int nb, int hkv, int64_t sv_h, int64_t sv_n,
                              int* queue, hipStream_t s) {
  if (fp32) {
    transpose_v_f32_kernel<<<dim3(nb, hkv), 256, 0, s>>>((const float*)V, (float*)Vt, nb, sv_h, sv_n, queue);
  } else {
    const int64_t tiles = (int64_t)nb * hkv;
    transpose_v_bf16_kernel<<<(unsigned)((tiles + 1) / 2), 512, 0, s>>>((const bf16*)V, (bf16*)Vt, nb, hkv, sv_h,
                                                                          sv_n, queue);
  }
  return hipGetLastError();
}

hipError_t launch_attention(int fp32, bool dense, const void* Q, const void* K, const void* Vt, void* O,
                            const int32_t* row_ptr, const int32_t* col_idx, int* queue, const SeqTable& seqs,
                            int nb_total, int hq, int hkv, const Strides& st, hipStream_t s) {
  const float sl2 = LOG2E / sqrtf((float)HD);
  const int64_t vt_h = (int64_t)nb_total * (BLK * HD);
  if (fp32) {  // one launch per sequence (the fp32 path serves small checking layers)
    auto k = dense ? fa_f32_kernel<true> : fa_f32_kernel<false>;
    for (int i = 0; i < seqs.nseq; ++i) {
      const int64_t t0 = seqs.tok[i];
      const dim3 grid((unsigned)((int64_t)seqs.nb[i] * hq));
      k<<<grid, 256, 0, s>>>((const float*)Q + t0 * st.q_n, (const float*)K + t0 * st.k_n,
                             (const float*)Vt + t0 * HD, (float*)O + t0 * st.o_n,
                             row_ptr ? row_ptr + seqs.rp[i] : nullptr, col_idx ? col_idx + seqs.col[i] : nullptr,
                             seqs.nb[i], hq, hkv, st.q_h, st.q_n, st.k_h, st.k_n, st.o_h, st.o_n, vt_h, sl2);
    }
  } else {
    const int64_t items = (int64_t)seqs.unit_off[seqs.nseq] * (hq / hkv);
    const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(items, device_cu_count())));
    // unit order: longest-first packing when every sequence's K and V fit in
    // the 256 MB last-level cache, two KV groups at a time otherwise
    SeqTable t = seqs;
    int64_t nb_max = 0;
    for (int i = 0; i < t.nseq; ++i) nb_max = std::max<int64_t>(nb_max, t.nb[i]);
    t.pair_major = 2 * (int64_t)hkv * nb_max * BLK * HD * 2 <= (int64_t(256) << 20);
    const int passes = (!dense && nb_max >= TWO_PASS_NB) ? NPHASE : 1;
    auto k = dense ? fa_bf16_kernel<true> : fa_bf16_kernel<false>;
    k<<<grid, 512, 0, s>>>((const bf16*)Q, (const bf16*)K, (const bf16*)Vt, (bf16*)O, row_ptr, col_idx, queue, t,
                           nb_total, hq, hkv, st.q_h, st.q_n, st.k_h, st.k_n, st.o_h, st.o_n, sl2, passes);
  }
  return hipGetLastError();
}

}  // namespace crisp
