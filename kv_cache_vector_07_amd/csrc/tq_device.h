// Device helpers shared by the TurboQuant kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
__device__ constexpr float rsqrt_dim() {
  return D == 128 ? 0.08838834764831845f : (D == 256 ? 0.0625f : 0.0f);
}

// sqrt(pi/2) / m with m = D rows in the QJL matrix.
template <int D>
__device__ constexpr float qjl_kappa() {
  return 1.2533141373155003f / (float)D;
}

template <int DT>
__device__ inline float load_elem(const void *p, size_t i) {
  if constexpr (DT == TQ_F32) {
    return reinterpret_cast<const float *>(p)[i];
  } else {
    uint32_t b = reinterpret_cast<const uint16_t *>(p)[i];
    return __uint_as_float(b << 16);
  }
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Unnormalised Walsh-Hadamard butterflies over D = 64*R values held by one
// wave, coordinate i = lane + 64*r in v[r]. Pair distance h < 64 crosses lanes,
// h >= 64 stays inside a lane's registers.
template <int R>
__device__ inline void fwht_wave(float (&v)[R]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const bool upper = lane & h;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float o = __shfl_xor(v[r], h, 64);
      v[r] = upper ? (o - v[r]) : (v[r] + o);
    }
  }
#pragma unroll
  for (int hh = 1; hh < R; hh <<= 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!(r & hh)) {
        float x = v[r], y = v[r | hh];
        v[r] = x + y;
        v[r | hh] = x - y;
      }
    }
  }
}

// c[idx] by a select tree (idx in 0..7) over the levels held in SGPRs.
__device__ inline float level_of(const Codebook &cb, int idx) {
  const bool b0 = idx & 1, b1 = idx & 2, b2 = idx & 4;
  float l01 = b0 ? cb.levels[1] : cb.levels[0];
  float l23 = b0 ? cb.levels[3] : cb.levels[2];
  float l45 = b0 ? cb.levels[5] : cb.levels[4];
  float l67 = b0 ? cb.levels[7] : cb.levels[6];
  float l03 = b1 ? l23 : l01;
  float l47 = b1 ? l67 : l45;
  return b2 ? l47 : l03;
}

// Code = number of thresholds t_k <= y (a tie goes to the upper cell).
__device__ inline int quantize_code(const Codebook &cb, float y) {
  int idx = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) idx += (y >= cb.thresholds[k]) ? 1 : 0;
  return idx;
}

// Page offsets are split as t = 64 b + 16 tau + 4 k + r (b: 64-token block;
// tau, k, r = 0..3). The per-page N / G arrays hold token t at entry
// 64 b + 16 k + 4 r + tau, so the 16 tokens with one (b, k) are adjacent.
__host__ __device__ inline int side_entry(int t) {
  return (t & ~63) | ((t & 12) << 2) | ((t & 3) << 2) | ((t >> 4) & 3);
}

// V code bits: bit j of the code of coordinate i = 16 (2 kp + h) + n of token
// t is bit 8 r + 4 h + tau of u32 word b*6D + j*2D + (16 k + n)*(D/32) + kp.
// One lane of the decode kernel (k, n) reads its D/32 words of a plane as one
// contiguous run, and the words of one plane and block are contiguous.
template <int D>
__device__ inline int v_word(int t, int i, int j) {
  return (t >> 6) * 6 * D + j * 2 * D + (16 * ((t >> 2) & 3) + (i & 15)) * (D / 32) + (i >> 5);
}
__device__ inline int v_bit(int t, int i) { return 8 * (t & 3) + 4 * ((i >> 4) & 1) + ((t >> 4) & 3); }

// Weights of the odd-codebook bit planes: c[idx] = sum_j 2 a_j plane_j - c7 with
// planes (b0, b1, b2, b0^b1^b2).
__device__ inline void plane_weights(const Codebook &cb, float (&w)[4]) {
  const float c4 = cb.levels[4], c5 = cb.levels[5], c6 = cb.levels[6], c7 = cb.levels[7];
  const float a2 = 0.25f * (c4 + c5 + c6 + c7);
  w[0] = 2.f * (0.5f * (c5 + c7) - a2);
  w[1] = 2.f * (0.5f * (c6 + c7) - a2);
  w[2] = 2.f * a2;
  w[3] = 2.f * (0.5f * (c4 + c7) - a2);
}

__device__ inline uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even, overflow to inf
  return __builtin_bit_cast(uint16_t, h);
}

__device__ inline float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

}  // namespace tq
