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
// Design (one work-group = one (head, query block) = 128 query rows, 4 waves):
//  * Scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so
//    each lane owns one query row and 64 of its 128 scores per key tile; the
//    online-softmax max / sum are in-lane plus one lane^32 exchange.
//  * The output is accumulated transposed, O^T += V^T P^T: P (rounded to bf16)
//    is already in the B-operand layout, and V^T comes from LDS.  V is
//    re-laid out once per call as per-block transposed tiles [d][key] so that
//    the tile copy to LDS is a plain coalesced 32 KB copy.
//  * K and V^T tiles are staged in padded LDS (67 KB per work-group, two
//    work-groups per CU); the next tile's global loads are issued into
//    registers before the current tile is computed.
//  * Work order: blockIdx -> (qb descending, head-in-group, KV head).  With 8
//    KV heads the 8 XCDs each see one KV head (blockIdx mod 8), so a KV head's
//    K/V stream stays in one XCD's L2; long (late) rows start first.
#include "common.h"
#include "launch.h"
#include "tile.h"

namespace crisp {

// ------------------------------------------------------------------ V re-layout

// V [hkv][n][d] (token stride sv_n) -> Vt [hkv][nb][d][128]
template <typename T>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T* __restrict__ V, T* __restrict__ Vt,
                                                          int nb, int64_t sv_h, int64_t sv_n) {
  __shared__ T tile[BLK][HD + 2];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const T* src = V + (int64_t)g * sv_h + (int64_t)kb * BLK * sv_n;
  for (int e = tid; e < BLK * HD; e += 256) {
    const int r = e / HD, d = e % HD;
    tile[r][d] = src[(int64_t)r * sv_n + d];
  }
  __syncthreads();
  T* dst = Vt + ((int64_t)g * nb + kb) * (BLK * HD);
  for (int e = tid; e < BLK * HD; e += 256) {
    const int d = e / BLK, r = e % BLK;
    dst[e] = tile[r][d];
  }
}

// ------------------------------------------------------------------ bf16 MFMA kernel

template <bool DENSE>
__global__ __launch_bounds__(256, 2) void fa_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ Vt, bf16* __restrict__ O,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int nb, int hq, int hkv,
    int64_t sq_h, int64_t sq_n, int64_t sk_h, int64_t sk_n, int64_t so_h, int64_t so_n, float sl2) {
  constexpr int KP = Tile<bf16>::KP;  // K tile pitch (elements)
  constexpr int VP = 132;             // V^T tile pitch: 264 B, conflict-free 8-B reads
  __shared__ __attribute__((aligned(16))) bf16 sK[BLK * KP];
  __shared__ __attribute__((aligned(16))) bf16 sV[HD * VP];

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
  bf16* orow = O + (int64_t)h * so_h + (int64_t)(qb * BLK + qrow) * so_n;
  if (cnt <= 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) *(bf16x4*)(orow + 32 * u + 8 * j + 4 * g) = bf16x4{};
    return;
  }

  Tile<bf16>::QFrag qf;
  Tile<bf16>::load_q(qf, Q + (int64_t)h * sq_h + (int64_t)(qb * BLK + qrow) * sq_n, g);

  const bf16* Kh = K + (int64_t)kvh * sk_h;
  const bf16* Vh = Vt + (int64_t)kvh * nb * (BLK * HD);
  uint4 kr[8], vr[8];
  auto gload = [&](int kb) {
    const bf16* kbase = Kh + (int64_t)kb * BLK * sk_n;
    const bf16* vbase = Vh + (int64_t)kb * (BLK * HD);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, r = c >> 4, gr = c & 15;
      kr[i] = *(const uint4*)(kbase + (int64_t)r * sk_n + gr * 8);
      vr[i] = *(const uint4*)(vbase + r * BLK + gr * 8);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, r = c >> 4, gr = c & 15;
      *(uint4*)(sK + r * KP + gr * 8) = kr[i];
      uint2* vd = (uint2*)(sV + r * VP + gr * 8);
      vd[0] = make_uint2(vr[i].x, vr[i].y);
      vd[1] = make_uint2(vr[i].z, vr[i].w);
    }
  };

  // Listed blocks outside [0, qb] hold no key j <= i: they are skipped (never loaded).
  auto valid = [&](int kb) { return (unsigned)kb <= (unsigned)qb; };
  int kb_next = DENSE ? 0 : col_idx[beg];
  if (valid(kb_next)) gload(kb_next);
  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{};
  float m = -1e30f, l = 0.f;

  for (int it = 0; it < cnt; ++it) {
    const int kb = kb_next;
    const bool ok = valid(kb);
    __syncthreads();
    if (ok) lstore();
    __syncthreads();
    if (it + 1 < cnt) {
      kb_next = DENSE ? it + 1 : col_idx[beg + it + 1];
      if (valid(kb_next)) gload(kb_next);
    }
    if (!ok) continue;
    f32x16 s[4];
    Tile<bf16>::st(s, sK, qf, l32, g);
    if (kb == qb) {  // diagonal tile: keys after the query are masked
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
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      bf16x8 b;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = (bf16)s[mm >> 1][8 * (mm & 1) + j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16* vp = sV + (32 * u + l32) * VP + 16 * mm + 4 * g;
        const bf16x4 lo = *(const bf16x4*)vp, hi = *(const bf16x4*)(vp + 8);
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[u] = mfma_bf16(a, b, acc[u]);
      }
    }
  }
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

// ------------------------------------------------------------------ fp32 MFMA kernel

template <bool DENSE>
__global__ __launch_bounds__(256, 1) void fa_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ Vt, float* __restrict__ O,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int nb, int hq, int hkv,
    int64_t sq_h, int64_t sq_n, int64_t sk_h, int64_t sk_n, int64_t so_h, int64_t so_n, float sl2) {
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
    Tile<float>::load_k(sV, Vt + ((int64_t)kvh * nb + kb) * (BLK * HD), BLK, tid);
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
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
                              hipStream_t s) {
  dim3 grid(nb, hkv);
  if (fp32)
    transpose_v_kernel<float><<<grid, 256, 0, s>>>((const float*)V, (float*)Vt, nb, sv_h, sv_n);
  else
    transpose_v_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)V, (bf16*)Vt, nb, sv_h, sv_n);
  return hipGetLastError();
}

hipError_t launch_attention(int fp32, bool dense, const void* Q, const void* K, const void* Vt, void* O,
                            const int32_t* row_ptr, const int32_t* col_idx, int nb, int hq, int hkv,
                            const Strides& st, hipStream_t s) {
  const float sl2 = LOG2E / sqrtf((float)HD);
  const dim3 grid((unsigned)((int64_t)nb * hq));
  if (fp32) {
    auto k = dense ? fa_f32_kernel<true> : fa_f32_kernel<false>;
    k<<<grid, 256, 0, s>>>((const float*)Q, (const float*)K, (const float*)Vt, (float*)O, row_ptr, col_idx, nb,
                           hq, hkv, st.q_h, st.q_n, st.k_h, st.k_n, st.o_h, st.o_n, sl2);
  } else {
    auto k = dense ? fa_bf16_kernel<true> : fa_bf16_kernel<false>;
    k<<<grid, 256, 0, s>>>((const bf16*)Q, (const bf16*)K, (const bf16*)Vt, (bf16*)O, row_ptr, col_idx, nb, hq,
                           hkv, st.q_h, st.q_n, st.k_h, st.k_n, st.o_h, st.o_n, sl2);
  }
  return hipGetLastError();
}

}  // namespace crisp
