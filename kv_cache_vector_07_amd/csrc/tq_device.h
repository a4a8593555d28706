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

// Value of lane (lane ^ H) of the wave. H = 1, 2: one DPP quad permutation;
// H = 4, 8: two DPP moves (a mirror inside 8 or 16 lanes composed with a
// smaller xor); H = 16: ds_swizzle inside 32 lanes; H = 32: ds_bpermute.
template <int H>
__device__ inline float xor_lane(float v) {
  const int x = __builtin_bit_cast(int, v);
  int y;
  if constexpr (H == 1) {
    y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);        // quad_perm [1,0,3,2]
  } else if constexpr (H == 2) {
    y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);        // quad_perm [2,3,0,1]
  } else if constexpr (H == 4) {
    const int m = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);   // lane ^ 7 (half-row mirror)
    y = __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true);        // then lane ^ 3 (quad_perm [3,2,1,0])
  } else if constexpr (H == 8) {
    const int m = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);   // lane ^ 15 (row mirror)
    y = __builtin_amdgcn_mov_dpp(m, 0x141, 0xF, 0xF, true);       // then lane ^ 7
  } else if constexpr (H == 16) {
    y = __builtin_amdgcn_ds_swizzle(x, 0x401F);                    // and 0x1f, xor 0x10
  } else {
    static_assert(H == 32, "lane xor distance");
    y = __builtin_bit_cast(int, __shfl_xor(v, 32, 64));
  }
  return __builtin_bit_cast(float, y);
}

__device__ inline float wave_sum(float x) {
  x += xor_lane<32>(x);
  x += xor_lane<16>(x);
  x += xor_lane<8>(x);
  x += xor_lane<4>(x);
  x += xor_lane<2>(x);
  return x + xor_lane<1>(x);
}

__device__ inline float wave_max(float x) {
  x = fmaxf(x, xor_lane<32>(x));
  x = fmaxf(x, xor_lane<16>(x));
  x = fmaxf(x, xor_lane<8>(x));
  x = fmaxf(x, xor_lane<4>(x));
  x = fmaxf(x, xor_lane<2>(x));
  return fmaxf(x, xor_lane<1>(x));
}

template <int H, int R>
__device__ inline void fwht_stage(float (&v)[R], int lane) {
  const bool upper = lane & H;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float o = xor_lane<H>(v[r]);
    v[r] = upper ? (o - v[r]) : (v[r] + o);
  }
}

// Unnormalised Walsh-Hadamard butterflies over D = 64*R values held by one
// wave, coordinate i = lane + 64*r in v[r]. Pair distance h < 64 crosses lanes,
// h >= 64 stays inside a lane's registers.
template <int R>
__device__ inline void fwht_wave(float (&v)[R]) {
  const int lane = threadIdx.x & 63;
  fwht_stage<1>(v, lane);
  fwht_stage<2>(v, lane);
  fwht_stage<4>(v, lane);
  fwht_stage<8>(v, lane);
  fwht_stage<16>(v, lane);
  fwht_stage<32>(v, lane);
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

// Code = number of thresholds t_k <= y (a tie goes to the upper cell); NT
// thresholds (7 for 3-bit codes).
template <int NT = 7>
__device__ inline int quantize_code(const Codebook &cb, float y) {
  int idx = 0;
#pragma unroll
  for (int k = 0; k < NT; ++k) idx += (y >= cb.thresholds[k]) ? 1 : 0;
  return idx;
}

// c[idx] for a code of up to 4 bits (not on a hot path).
__device__ inline float level_any(const Codebook &cb, int idx) {
  float r = cb.levels[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) r = idx == k ? cb.levels[k] : r;
  return r;
}

// Page offsets are split as t = 64 b + 16 tau + 4 k + r (b: 64-token block;
// tau, k, r = 0..3). The per-page N / G arrays hold token t at entry
// 64 b + 16 k + 4 r + tau = 64 b + 4 n + tau (n = 4 k + r), so the four tokens
// 16 tau + n of one (b, n) are adjacent.
__host__ __device__ inline int side_entry(int t) {
  return (t & ~63) | ((t & 12) << 2) | ((t & 3) << 2) | ((t >> 4) & 3);
}

// V code bits (VB-bit codes): bit j of the code of coordinate i = 16 (2 kp + h)
// + n of token t is bit 8 r + 4 h + tau of u32 word
// b*2*VB*D + j*2D + (16 k + n)*(D/32) + kp. One lane of the decode kernel
// (k, n) reads its D/32 words of a plane as one contiguous run, and the words
// of one plane and block are contiguous.
template <int D, int VB = 3>
__device__ inline int v_word(int t, int i, int j) {
  return (t >> 6) * 2 * VB * D + j * 2 * D + (16 * ((t >> 2) & 3) + (i & 15)) * (D / 32) + (i >> 5);
}
__device__ inline int v_word_rt(int t, int i, int j, int d, int vb) {
  return (t >> 6) * 2 * vb * d + j * 2 * d + (16 * ((t >> 2) & 3) + (i & 15)) * (d / 32) + (i >> 5);
}
__device__ inline int v_bit(int t, int i) { return 8 * (t & 3) + 4 * ((i >> 4) & 1) + ((t >> 4) & 3); }

// Bit planes of VB-bit codes for an odd codebook (c[n-1-k] = -c[k]): the odd
// Walsh functions of the code bits, i.e. the parities of the bit subsets of odd
// size, as masks. c[idx] = sum_p w_p parity(idx & mask_p) - c[n-1], with
// w_p = -2 a_p and a_p the Walsh coefficient 2^-VB sum_idx c[idx] (-1)^popc(idx & mask_p).
template <int VB> struct VPlanes;
template <> struct VPlanes<2> {
  static constexpr int n = 2;
  static constexpr int mask[2] = {1, 2};
};
template <> struct VPlanes<3> {
  static constexpr int n = 4;
  static constexpr int mask[4] = {1, 2, 4, 7};
};
template <> struct VPlanes<4> {
  static constexpr int n = 8;
  static constexpr int mask[8] = {1, 2, 4, 8, 7, 11, 13, 14};
};

template <int VB>
__device__ inline void plane_weights_walsh(const Codebook &cb, float (&w)[VPlanes<VB>::n]) {
#pragma unroll
  for (int p = 0; p < VPlanes<VB>::n; ++p) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < (1 << VB); ++i)
      a += (__builtin_popcount(i & VPlanes<VB>::mask[p]) & 1) ? -cb.levels[i] : cb.levels[i];
    w[p] = -2.f * a / (float)(1 << VB);
  }
}

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

// fp6 e2m3 (OCP MX format: sign, 2 exponent bits with bias 1, 3 mantissa
// bits; no infinities or NaN, largest magnitude 7.5) rounding of |x| < 8:
// round to nearest even, 7.75 and above saturating to 7.5. Returns the rounded
// value; `code` gets its 6-bit code. The step is 1/8 below 2, 1/4 in [2, 4) and
// 1/2 in [4, 8): adding 1.5 * 2^(20 + e) rounds to a multiple of 2^(e - 3) in
// fp32, and subtracting it back is exact.
__device__ inline float fp6_e2m3_round(float x, uint32_t &code) {
  const float a = fabsf(x);
  const int e = min(2, max(0, __builtin_amdgcn_frexp_expf(a) - 1));
  const float k = __builtin_ldexpf(1.5f, 20 + e);
  const float q = fminf((a + k) - k, 7.5f);
  // codes: 8 q below 2 (subnormals and the first binade alike), then 4 q + 8,
  // 2 q + 16, i.e. q 2^(3 - e) + 8 e. The three agree where the binades meet,
  // so e taken before rounding gives the code of q, without branches.
  const float cf = fmaf(q, __builtin_ldexpf(1.f, 3 - e), (float)(8 * e));
  code = (uint32_t)cf | (x < 0.f ? 0x20u : 0u);
  return x < 0.f ? -q : q;
}

__device__ inline uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even, overflow to inf
  return __builtin_bit_cast(uint16_t, h);
}

__device__ inline float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

}  // namespace tq
