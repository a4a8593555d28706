// Encode (K and V) and dequantise kernels.
//
// Method: AI Heartland news "Apple Silicon向けSwiftLM、TurboQuant KVキャッシュ圧縮と
// SSD Expert Streamingを実装", section 技術的な詳細, "K-Cache圧縮" flow steps 1-5 and
// "V-Cache圧縮" (steps 1-3 only). One wave handles whole head vectors: lane l holds
// coordinates l + 64 r, so loads and stores are coalesced and the rotation's
// butterflies are lane shuffles (distance < 64) or register pairs (distance >= 64).
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kWaves = 4;      // waves per workgroup

// Steps 1-3 for one vector: norm, rotation, codes. Returns y (rotated, unit
// norm) in y[], the codes in idx[] and the norm.
template <int D, int DT>
__device__ inline float encode_front(const void *x, size_t base, const Codebook &cb,
                                     float (&y)[D / 64], int (&idx)[D / 64]) {
  constexpr int R = D / 64;
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    y[r] = load_elem<DT>(x, base + lane + 64 * r);
    ss += y[r] * y[r];
  }
  ss = wave_sum(ss);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) y[r] *= inv;
  fwht_wave<R>(y);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    y[r] *= rsqrt_dim<D>();
    idx[r] = quantize_code(cb, y[r]);
  }
  return n;
}

// VPW K vectors per wave share each load of S in the S r product: 4 for bulk
// encodes, 1 for short appends (where latency, not S traffic, dominates).
template <int D, int DT, int kKVecPerWave>
__global__ __launch_bounds__(256) void encode_k_kernel(EncodeArgs a) {
  constexpr int R = D / 64;
  constexpr int NWORD = D / 8;              // u32 words per K record
  constexpr size_t KSEC = (size_t)kPage * D / 2 + 4 * kPage;
  constexpr size_t KCODES = (size_t)kPage * D / 2;
  __shared__ float4 rbuf[kWaves][kKVecPerWave][D / 4];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long total = (long)a.n_tokens * a.n_heads;
  const long v0 = ((long)blockIdx.x * kWaves + wave) * kKVecPerWave;

  float nrm[kKVecPerWave], gam[kKVecPerWave];
  uint64_t code[kKVecPerWave][R][3];

#pragma unroll
  for (int v = 0; v < kKVecPerWave; ++v) {
    const long vec = v0 + v;
    float r[R];
    if (vec < total) {
      int idx[R];
      nrm[v] = encode_front<D, DT>(a.x, (size_t)vec * D, a.cb, r, idx);
      float rr = 0.f;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        r[k] -= level_of(a.cb, idx[k]);
        rr += r[k] * r[k];
#pragma unroll
        for (int j = 0; j < 3; ++j) code[v][k][j] = __ballot((idx[k] >> j) & 1);
      }
      gam[v] = sqrtf(wave_sum(rr));
    } else {
      nrm[v] = gam[v] = 0.f;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        r[k] = 0.f;
#pragma unroll
        for (int j = 0; j < 3; ++j) code[v][k][j] = 0;
      }
    }
    float *rb = reinterpret_cast<float *>(rbuf[wave][v]);
#pragma unroll
    for (int k = 0; k < R; ++k) rb[lane + 64 * k] = r[k];
  }
  __syncthreads();

  // z_l = sum_i S[l][i] r_i for rows l = lane + 64 k of each of the wave's vectors.
  float z[kKVecPerWave][R];
#pragma unroll
  for (int v = 0; v < kKVecPerWave; ++v)
#pragma unroll
    for (int k = 0; k < R; ++k) z[v][k] = 0.f;
  const float4 *S4 = reinterpret_cast<const float4 *>(a.qjl);
#pragma unroll 8
  for (int i4 = 0; i4 < D / 4; ++i4) {
    float4 s[R];
#pragma unroll
    for (int k = 0; k < R; ++k) s[k] = S4[(size_t)(lane + 64 * k) * (D / 4) + i4];
#pragma unroll
    for (int v = 0; v < kKVecPerWave; ++v) {
      const float4 rv = rbuf[wave][v][i4];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        z[v][k] = fmaf(s[k].x, rv.x, z[v][k]);
        z[v][k] = fmaf(s[k].y, rv.y, z[v][k]);
        z[v][k] = fmaf(s[k].z, rv.z, z[v][k]);
        z[v][k] = fmaf(s[k].w, rv.w, z[v][k]);
      }
    }
  }

#pragma unroll
  for (int v = 0; v < kKVecPerWave; ++v) {
    const long vec = v0 + v;
    uint64_t sgn[R];
#pragma unroll
    for (int k = 0; k < R; ++k) sgn[k] = __ballot(z[v][k] >= 0.f);
    if (vec >= total) continue;
    const long tok = vec / a.n_heads;
    const int head = (int)(vec % a.n_heads);
    const int slot = a.slots[tok];
    uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * KSEC;
    const int off = slot % kPage;
    uint32_t w = 0;
#pragma unroll
    for (int kk = 0; kk < NWORD; ++kk) {
      const int s = kk >> 2, j = kk & 3;
      const uint64_t m = j < 3 ? code[v][s >> 1][j] : sgn[s >> 1];
      const uint32_t word = (s & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
      if (lane == kk) w = word;
    }
    if (lane < NWORD) reinterpret_cast<uint32_t *>(sec + (size_t)off * (D / 2))[lane] = w;
    if (lane == 0) {
      reinterpret_cast<uint16_t *>(sec + KCODES)[side_entry(off)] = f32_to_f16_bits(nrm[v]);
      reinterpret_cast<uint16_t *>(sec + KCODES + 2 * kPage)[side_entry(off)] = f32_to_f16_bits(gam[v]);
    }
  }
}

template <int D, int DT>
__global__ __launch_bounds__(256) void encode_v_kernel(EncodeArgs a) {
  constexpr int R = D / 64;
  constexpr size_t VSEC = (size_t)3 * D * kPage / 8 + 2 * kPage;
  constexpr size_t VCODES = (size_t)3 * D * kPage / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long vec = (long)blockIdx.x * kWaves + wave;
  if (vec >= (long)a.n_tokens * a.n_heads) return;
  float y[R];
  int idx[R];
  const float n = encode_front<D, DT>(a.x, (size_t)vec * D, a.cb, y, idx);
  const long tok = vec / a.n_heads;
  const int head = (int)(vec % a.n_heads);
  const int slot = a.slots[tok];
  uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * VSEC;
  const int off = slot % kPage;
  uint32_t *rows = reinterpret_cast<uint32_t *>(sec);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = lane + 64 * r;
    const uint32_t bit = 1u << v_bit(off, i);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      uint32_t *w = rows + v_word<D>(off, i, j);
      if ((idx[r] >> j) & 1)
        atomicOr(w, bit);
      else
        atomicAnd(w, ~bit);
    }
  }
  if (lane == 0) reinterpret_cast<uint16_t *>(sec + VCODES)[side_entry(off)] = f32_to_f16_bits(n);
}

template <int D>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a, int which) {
  constexpr int R = D / 64;
  constexpr size_t KSEC = (size_t)kPage * D / 2 + 4 * kPage;
  constexpr size_t KCODES = (size_t)kPage * D / 2;
  constexpr size_t VSEC = (size_t)3 * D * kPage / 8 + 2 * kPage;
  constexpr size_t VCODES = (size_t)3 * D * kPage / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long vec = (long)blockIdx.x * kWaves + wave;
  if (vec >= (long)a.n_tokens * a.n_heads) return;
  const long tok = vec / a.n_heads;
  const int head = (int)(vec % a.n_heads);
  const int slot = a.slots[tok];
  const int off = slot % kPage;
  float v[R];
  float scale;
  if (which == 0) {
    const uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * KSEC;
    const uint32_t *rec = reinterpret_cast<const uint32_t *>(sec + (size_t)off * (D / 2));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = lane + 64 * r, s = i >> 5, e = i & 31;
      const int idx = ((rec[4 * s] >> e) & 1) | (((rec[4 * s + 1] >> e) & 1) << 1) |
                      (((rec[4 * s + 2] >> e) & 1) << 2);
      v[r] = level_of(a.cb, idx);
    }
    scale = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(sec + KCODES)[side_entry(off)]);
    if (a.with_qjl) {
      const float G = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(sec + KCODES + 2 * kPage)[side_entry(off)]);
      float t[R];
#pragma unroll
      for (int r = 0; r < R; ++r) t[r] = 0.f;
      for (int l = 0; l < D; ++l) {
        const bool pos = (rec[4 * (l >> 5) + 3] >> (l & 31)) & 1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float s = a.qjl[(size_t)l * D + lane + 64 * r];
          t[r] += pos ? s : -s;
        }
      }
      const float k = qjl_kappa<D>() * G;
#pragma unroll
      for (int r = 0; r < R; ++r) v[r] = fmaf(k, t[r], v[r]);
    }
  } else {
    const uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * VSEC;
    const uint32_t *rows = reinterpret_cast<const uint32_t *>(sec);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = lane + 64 * r, bit = v_bit(off, i);
      int idx = 0;
#pragma unroll
      for (int j = 0; j < 3; ++j) idx |= ((rows[v_word<D>(off, i, j)] >> bit) & 1) << j;
      v[r] = level_of(a.cb, idx);
    }
    scale = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(sec + VCODES)[side_entry(off)]);
  }
  fwht_wave<R>(v);
  scale *= rsqrt_dim<D>();
  float *o = a.out + (size_t)vec * D;
#pragma unroll
  for (int r = 0; r < R; ++r) o[lane + 64 * r] = v[r] * scale;
}

template <typename F>
hipError_t by_dim_dtype(int d, int dtype, F &&f) {
  if (d == 128) {
    if (dtype == TQ_F32) return f(std::integral_constant<int, 128>{}, std::integral_constant<int, TQ_F32>{});
    return f(std::integral_constant<int, 128>{}, std::integral_constant<int, TQ_BF16>{});
  }
  if (dtype == TQ_F32) return f(std::integral_constant<int, 256>{}, std::integral_constant<int, TQ_F32>{});
  return f(std::integral_constant<int, 256>{}, std::integral_constant<int, TQ_BF16>{});
}

}  // namespace

hipError_t launch_encode_k(const EncodeArgs &a, int d, hipStream_t s) {
  const long total = (long)a.n_tokens * a.n_heads;
  return by_dim_dtype(d, a.dtype, [&](auto D, auto DT) {
    if (total < 4096) {
      const dim3 grid((unsigned)((total + kWaves - 1) / kWaves));
      hipLaunchKernelGGL((encode_k_kernel<D.value, DT.value, 1>), grid, dim3(256), 0, s, a);
    } else {
      const long per_block = kWaves * 4;
      const dim3 grid((unsigned)((total + per_block - 1) / per_block));
      hipLaunchKernelGGL((encode_k_kernel<D.value, DT.value, 4>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  });
}

hipError_t launch_encode_v(const EncodeArgs &a, int d, hipStream_t s) {
  const long total = (long)a.n_tokens * a.n_heads;
  const dim3 grid((unsigned)((total + kWaves - 1) / kWaves));
  return by_dim_dtype(d, a.dtype, [&](auto D, auto DT) {
    hipLaunchKernelGGL((encode_v_kernel<D.value, DT.value>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_dequant(const DequantArgs &a, int d, int which, hipStream_t s) {
  const long total = (long)a.n_tokens * a.n_heads;
  const dim3 grid((unsigned)((total + kWaves - 1) / kWaves));
  if (d == 128)
    hipLaunchKernelGGL((dequant_kernel<128>), grid, dim3(256), 0, s, a, which);
  else
    hipLaunchKernelGGL((dequant_kernel<256>), grid, dim3(256), 0, s, a, which);
  return hipGetLastError();
}

}  // namespace tq
