// Re-layout of V into per-block transposed tiles for the attention kernels'
// O^T += V^T P^T products (bf16 and fp32), shared by the stand-alone re-layout
// kernel, the proxy launch of a prefill (which does it beside the selection)
// and the dense selection launch (a prefill with every sequence below the
// length gate).
//
// V [hkv][n][d] (token stride sv_n, head stride sv_h) -> Vt [hkv][N_b][d][128]:
// row d of tile (g, kb) holds V[g][128 kb + key][d] for the block's 128 keys.
// bf16 rows are in vt_pos order: within each group of 16 keys, positions
// 8a .. 8a + 7 hold keys {4a .. 4a + 3, 8 + 4a .. 8 + 4a + 3} -- exactly the
// eight keys that lane half a contributes to one 32x32x16 MFMA of the
// product, so each A operand is a single 16-byte LDS read.
#pragma once
#include "common.h"

namespace crisp {

// Position of key e (0..127) inside a re-laid-out bf16 V^T row.
__host__ __device__ __forceinline__ int vt_pos(int e) {
  const int grp = e >> 4, k = e & 15, h = k >> 3, g = (k >> 2) & 1, j = k & 3;
  return 16 * grp + 8 * g + 4 * h + j;
}

// One bf16 tile (g, kb) by 256 threads, t = 0..255, in registers: thread t
// takes dims 8c .. 8c + 7 (c = t % 16) of the eight keys that fill output
// positions 8o .. 8o + 7 (o = t / 16), with eight 16-byte loads (the 16
// threads of one key row read its 256 bytes) and eight 16-byte stores.
__device__ __forceinline__ void vt_tile_bf16(const bf16* __restrict__ V, bf16* __restrict__ Vt, int64_t sv_h,
                                             int64_t sv_n, int nb, int kb, int g, int t) {
  const int c = t & 15, o = t >> 4;
  // output position 8o + p holds key 16(o/2) + 8(p/4) + 4(o%2) + p%4
  const int key0 = 16 * (o >> 1) + 4 * (o & 1);
  const bf16* src = V + (int64_t)g * sv_h + ((int64_t)kb * BLK + key0) * sv_n + 8 * c;
  bf16x8 r[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) r[p] = *(const bf16x8*)(src + (int64_t)(8 * (p >> 2) + (p & 3)) * sv_n);
  bf16* dst = Vt + (((int64_t)g * nb + kb) * HD + 8 * c) * BLK + 8 * o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16x8 w;
#pragma unroll
    for (int p = 0; p < 8; ++p) w[p] = r[p][e];
    *(bf16x8*)(dst + e * BLK) = w;
  }
}

}  // namespace crisp
