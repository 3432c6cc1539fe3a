// The MLP scorer's arithmetic on one 16-row tile (KVpop section 3.3
// "Stateless scorers", Appendix E.1-E.2, Eq. 35-36: score = w2 . act(W1
// [k; v] + b1) + b2, key first), shared by the scorer kernel and the fused
// eviction kernel so that both produce the same bits for the same row.
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with 8 consecutive
// contraction indices starting at 8 * (l / 16); the accumulator holds
// C[4 * (l / 16) + i][l % 16], i = 0..3.
#pragma once

#include "kve_internal.h"

namespace kve {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4*)p);
}

__device__ __forceinline__ float mlp_activate(float a, int act) {
  if (act == 0) return fmaxf(a, 0.f);
  return a / (1.f + __expf(-a));  // SiLU
}

// The A operand of a tile: this lane's 8 contraction indices of every
// 32-wide step of [k; v] for row `slot` of the slice (k then v).
template <int D>
__device__ __forceinline__ void mlp_load_row(bf16x8_t (&a)[2 * D / 32],
                                             const uint16_t* krow,
                                             const uint16_t* vrow, int kq) {
  constexpr int KSTEPS = 2 * D / 32, KHALF = D / 32;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    a[ks] = ks < KHALF ? load_bf16x8(krow + ks * 32 + kq)
                       : load_bf16x8(vrow + (ks - KHALF) * 32 + kq);
}

// Scores of the tile's rows 4 * (lane / 16) + i, i = 0..3 (every lane of a
// 16-lane group ends with the same four values). w1s holds the head's W1
// rows in LDS with a row stride of lstr bf16; bias and w2v hold hidden unit
// nb * 16 + lane % 16.
template <int D, int NB>
__device__ __forceinline__ void mlp_tile_scores(
    const bf16x8_t (&a)[2 * D / 32], const uint16_t* w1s, int lstr,
    const float (&bias)[NB], const float (&w2v)[NB], float b2, int act,
    float (&out)[4]) {
  constexpr int KSTEPS = 2 * D / 32;
  const int lane = threadIdx.x & 63;
  const int ncol = lane & 15;
  const int kq = (lane >> 4) * 8;
  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t B = __builtin_bit_cast(
          bf16x8_t,
          *(const u32x4*)(w1s + (nb * 16 + ncol) * lstr + ks * 32 + kq));
      acc[nb] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], B, acc[nb], 0, 0, 0);
    }
  }
  // Second layer over the 16 hidden units of this lane's columns, then
  // summed over the 16 columns.
  float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      part[i] += mlp_activate(acc[nb][i] + bias[nb], act) * w2v[nb];
#pragma unroll
  for (int off = 1; off < 16; off <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] += __shfl_xor(part[i], off);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = part[i] + b2;
}

// Stage head h's W1 ([HID][IN] bf16) into w1s with row stride lstr, using
// `threads` threads.
template <int HID, int IN>
__device__ __forceinline__ void mlp_stage_w1(uint16_t* w1s, int lstr,
                                             const uint16_t* w1, int threads) {
  for (int c = threadIdx.x; c < HID * IN / 8; c += threads) {
    const int n = c / (IN / 8);
    const int k8 = c % (IN / 8);
    *(u32x4*)(w1s + n * lstr + k8 * 8) =
        *(const u32x4*)(w1 + (size_t)n * IN + k8 * 8);
  }
}

}  // namespace kve
