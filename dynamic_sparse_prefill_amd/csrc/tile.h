// S^T = K_tile * Q_rows^T on one 128-key tile, for the proxy and attention kernels.
//
// A work-group of 4 waves covers 128 query rows; wave w owns rows 32w..32w+31
// and lane l owns row 32w + l%32.  The product is taken with K as the MFMA A
// operand (rows = keys) and Q as the B operand (columns = queries), so after
// the 4 x (d/16) MFMAs lane l holds 64 scores of ITS OWN query row:
//   st[t][i] = s(query 32w + l%32, key 32t + 8(i/4) + 4(l/32) + i%4).
// Row-wise max and sum are then in-lane plus one exchange with lane l^32.
#pragma once
#include "common.h"

namespace crisp {

template <typename T> struct Tile;

template <> struct Tile<bf16> {
  struct QFrag { bf16x8 v[8]; };
  // lane's query row, d-slices 16c + 8g .. +8 (B operand of v_mfma_f32_32x32x16_bf16)
  __device__ static void load_q(QFrag& f, const bf16* row, int g) {
#pragma unroll
    for (int c = 0; c < 8; ++c) f.v[c] = *(const bf16x8*)(row + 16 * c + 8 * g);
  }
};

template <> struct Tile<float> {
  static constexpr int KP = 132;            // 528 B pitch
  struct QFrag { float v[64]; };
  // lane's query row, element 2c + g (B operand of v_mfma_f32_32x32x2f32)
  __device__ static void load_q(QFrag& f, const float* row, int g) {
#pragma unroll
    for (int c = 0; c < 64; ++c) f.v[c] = row[2 * c + g];
  }
  __device__ static void load_k(float* sK, const float* kbase, int64_t ld, int tid) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = tid + 256 * i, r = c >> 5, gr = c & 31;
      *(float4*)(sK + r * KP + gr * 4) = *(const float4*)(kbase + (int64_t)r * ld + gr * 4);
    }
  }
  __device__ static void st(f32x16 (&s)[4], const float* sK, const QFrag& f, int l32, int g) {
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = f32x16{};
#pragma unroll 8
    for (int c = 0; c < 64; ++c) {
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = mfma_f32(sK[(32 * t + l32) * KP + 2 * c + g], f.v[c], s[t]);
    }
  }
};

}  // namespace crisp
