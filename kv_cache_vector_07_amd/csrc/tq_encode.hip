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

// Steps 1-3 for one vector: norm, rotation, codes (NT thresholds). Returns y
// (rotated, unit norm) in y[], the codes in idx[] and the norm.
template <int D, int DT>
__device__ inline void load_vector(const void *x, size_t base, float (&y)[D / 64]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < D / 64; ++r) y[r] = load_elem<DT>(x, base + lane + 64 * r);
}

// The same steps on a vector already loaded into y[].
template <int D, int NT = 7>
__device__ inline float encode_front_loaded(const Codebook &cb, float (&y)[D / 64], int (&idx)[D / 64]) {
  constexpr int R = D / 64;
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) ss += y[r] * y[r];
  ss = wave_sum(ss);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) y[r] *= inv;
  fwht_wave<R>(y);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    y[r] *= rsqrt_dim<D>();
    idx[r] = quantize_code<NT>(cb, y[r]);
  }
  return n;
}

template <int D, int DT, int NT = 7>
__device__ inline float encode_front(const void *x, size_t base, const Codebook &cb,
                                     float (&y)[D / 64], int (&idx)[D / 64]) {
  load_vector<D, DT>(x, base, y);
  return encode_front_loaded<D, NT>(cb, y, idx);
}

// K encode of short appends: one vector per workgroup. Wave 0 runs steps 1-4
// (codes by ballot, residual into LDS); then wave w computes rows
// 16 (RT w + t) + l16 of z = S r with lane FMAs: lane (l16, kq) holds
// S[row][16 c + 4 kq + m] (read from L2 before the encode starts at d = 128),
// the four lane groups' partial sums are added across lanes, and the signs come
// back by ballot. Few vectors leave most of a 16-wide MFMA tile as padding, and
// one vector per workgroup spreads a step's appends over more SIMDs.
template <int D, int DT, int KB>
__device__ void encode_k_block(const EncodeArgs &a, long vec) {
  constexpr int R = D / 64;
  constexpr int NWORD = (KB + 1) * D / 32;  // u32 words per K record: KB code planes + signs per 32
  constexpr int RT = D / 16 / kWaves;       // 16-row tiles of S per wave: 2 or 4
  constexpr size_t KREC = (size_t)(KB + 1) * D / 8;
  constexpr size_t KCODES = (size_t)kPage * KREC;
  constexpr size_t KSEC = KCODES + 4 * kPage;
  __shared__ float4 s_r[D / 4];             // residual
  __shared__ uint64_t s_code[KB][R];        // code bit planes
  __shared__ uint16_t s_sign[D / 16];       // sign bits, 16 rows of S per entry
  __shared__ float s_ng[2];                 // N, G

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;

  // the vector is loaded before S: loads complete in order
  float y[R];
  if (wave == 0) load_vector<D, DT>(a.x, (size_t)vec * D, y);
  // S rows of this wave's tiles: the loads do not depend on the data, so for
  // d = 128 they are all issued before the encode starts
  const float4 *S4 = reinterpret_cast<const float4 *>(a.qjl);
  const bool qjl = a.qjl != nullptr;   // MSE-only keys (no S) skip z = S r
  constexpr bool kHoist = D == 128;
  float4 sreg[kHoist ? RT * (D / 16) : 1];
  if (kHoist && qjl) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        sreg[t * (D / 16) + c] = S4[(size_t)(16 * (wave * RT + t) + l16) * (D / 4) + 4 * c + kq];
  }

  if (wave == 0) {
    int idx[R];
    const float n = encode_front_loaded<D, (1 << KB) - 1>(a.cb, y, idx);
    float rr = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      y[k] -= KB == 3 ? level_of(a.cb, idx[k]) : level_any(a.cb, idx[k]);
      rr += y[k] * y[k];
      reinterpret_cast<float *>(s_r)[lane + 64 * k] = y[k];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const uint64_t m = __ballot((idx[k] >> j) & 1);
        if (lane == 0) s_code[j][k] = m;
      }
    }
    const float gm = sqrtf(wave_sum(rr));
    if (lane == 0) {
      s_ng[0] = n;
      s_ng[1] = gm;
    }
  }
  __syncthreads();

  // z[t]: row 16 (RT wave + t) + l16 of S times the residual, this lane group's
  // coordinates 16 c + 4 kq + m, then summed over the four lane groups
  if (qjl) {
    float z[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) z[t] = 0.f;
    auto step = [&](int c) {
      const float4 rv = s_r[4 * c + kq];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float4 bv = kHoist ? sreg[t * (D / 16) + c]
                                 : S4[(size_t)(16 * (wave * RT + t) + l16) * (D / 4) + 4 * c + kq];
        z[t] = fmaf(bv.x, rv.x, z[t]);
        z[t] = fmaf(bv.y, rv.y, z[t]);
        z[t] = fmaf(bv.z, rv.z, z[t]);
        z[t] = fmaf(bv.w, rv.w, z[t]);
      }
    };
    if constexpr (kHoist) {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) step(c);
    } else {
      // at d = 256 the S loads go out four steps at a time (registers)
#pragma unroll 4
      for (int c = 0; c < D / 16; ++c) step(c);
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float v = z[t];
      v += xor_lane<16>(v);
      v += xor_lane<32>(v);
      const uint64_t m = __ballot(v >= 0.f);   // the four lane groups agree
      if (lane == 0) s_sign[wave * RT + t] = (uint16_t)m;
    }
  }
  __syncthreads();

  // the record, by wave 0
  if (wave == 0) {
    const long tok = vec / a.n_heads;
    const int head = (int)(vec % a.n_heads);
    const int slot = a.slots[tok];
    uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * KSEC;
    const int off = slot % kPage;
    if (lane < NWORD) {
      const int s = lane / (KB + 1), j = lane % (KB + 1);   // coordinate group, word in it
      uint32_t w;
      if (j < KB) {
        const uint64_t m = s_code[j][s >> 1];
        w = (s & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
      } else {
        w = qjl ? (uint32_t)s_sign[2 * s] | ((uint32_t)s_sign[2 * s + 1] << 16) : 0u;
      }
      reinterpret_cast<uint32_t *>(sec + (size_t)off * KREC)[lane] = w;
    }
    if (lane == 0) {
      reinterpret_cast<uint16_t *>(sec + KCODES)[side_entry(off)] = f32_to_f16_bits(s_ng[0]);
      reinterpret_cast<uint16_t *>(sec + KCODES + 2 * kPage)[side_entry(off)] = f32_to_f16_bits(s_ng[1]);
    }
  }
}

// V encode: 64 tokens of one KV head per workgroup. Codes go to LDS by ballot;
// when the 64 slots are one whole aligned 64-token block of a page, the block's
// words are assembled and stored whole (coalesced, no atomics). Otherwise each
// token's bits are set one by one with atomics, which leaves the neighbours in
// the same words intact.
template <int D, int DT, int VPW, int VBITS>
__device__ void encode_v_block(const EncodeArgs &a, int bx, int head) {
  constexpr int R = D / 64;
  constexpr int VB = kWaves * VPW;   // tokens per workgroup: 64 (whole blocks possible) or 4
  constexpr size_t VCODES = (size_t)VBITS * D * kPage / 8;
  constexpr size_t VSEC = VCODES + 2 * kPage;
  __shared__ uint64_t s_code[VB][VBITS][R];
  __shared__ float s_n[VB];
  __shared__ int s_whole;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = bx * VB;
  const int nt = min(VB, a.n_tokens - t0);
  if (threadIdx.x == 0) {
    const int s0 = a.slots[t0];
    s_whole = (VB == 64 && nt == VB && (s0 & 63) == 0);
  }
  __syncthreads();
  if (threadIdx.x < VB && threadIdx.x < nt && a.slots[t0 + threadIdx.x] != a.slots[t0] + threadIdx.x)
    s_whole = 0;   // benign race: every writer stores 0

  for (int u = wave; u < nt; u += kWaves) {
    float y[R];
    int idx[R];
    const float n = encode_front<D, DT, (1 << VBITS) - 1>(a.x, ((size_t)(t0 + u) * a.n_heads + head) * D,
                                                          a.cb, y, idx);
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int j = 0; j < VBITS; ++j) {
        const uint64_t m = __ballot((idx[k] >> j) & 1);
        if (lane == 0) s_code[u][j][k] = m;
      }
    if (lane == 0) s_n[u] = n;
  }
  __syncthreads();

  if (VB == 64 && s_whole) {
    const int s0 = a.slots[t0];
    uint8_t *sec = a.pool + ((size_t)(s0 / kPage) * a.n_heads + head) * VSEC;
    const int bofs = s0 % kPage;   // offset of the block in the page (a multiple of 64)
    uint32_t *words = reinterpret_cast<uint32_t *>(sec) + (bofs >> 6) * 2 * VBITS * D;
    // word e = j*2D + (16 k + n)*(D/32) + kp; bit 8 r + 4 h + tau <- token 16 tau + 4 k + r,
    // coordinate 32 kp + 16 h + n (both coordinates in the same 64-bit ballot)
    for (int e = threadIdx.x; e < 2 * VBITS * D; e += 256) {
      const int j = e / (2 * D), rem = e % (2 * D);
      const int c = rem / (D / 32), kp = rem % (D / 32);
      const int k = c >> 4, n = c & 15;
      const int i0 = 32 * kp + n;
      const int sh = i0 & 63;
      uint32_t w = 0;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint64_t m = s_code[16 * tau + 4 * k + r][j][i0 >> 6];
          w |= (uint32_t)((m >> sh) & 1) << (8 * r + tau);
          w |= (uint32_t)((m >> (sh + 16)) & 1) << (8 * r + 4 + tau);
        }
      words[e] = w;
    }
    if (threadIdx.x < VB)
      reinterpret_cast<uint16_t *>(sec + VCODES)[side_entry(bofs + threadIdx.x)] = f32_to_f16_bits(s_n[threadIdx.x]);
    return;
  }

  for (int u = wave; u < nt; u += kWaves) {
    const int slot = a.slots[t0 + u];
    uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * VSEC;
    const int off = slot % kPage;
    uint32_t *rows = reinterpret_cast<uint32_t *>(sec);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = lane + 64 * k;
      const uint32_t bit = 1u << v_bit(off, i);
#pragma unroll
      for (int j = 0; j < VBITS; ++j) {
        uint32_t *w = rows + v_word<D, VBITS>(off, i, j);
        if ((s_code[u][j][k] >> lane) & 1)
          atomicOr(w, bit);
        else
          atomicAnd(w, ~bit);
      }
    }
    if (lane == 0) reinterpret_cast<uint16_t *>(sec + VCODES)[side_entry(off)] = f32_to_f16_bits(s_n[u]);
  }
}

// ------------------------------------------------------------------ bulk encode
// Four lanes per vector: lane 4 v + p of a wave holds coordinates C p + e
// (e = 0 .. C - 1, C = D / 4) of the wave's v-th vector, so the norm and all
// but two rotation stages run in registers (the butterflies at distance C and
// 2 C are the quad swaps lane ^ 1 and lane ^ 2), and the lane's code bits of
// each 32-coordinate group are that group's plane words. A workgroup encodes 64
// vectors, 16 per wave.

// Loads the C coordinates of one vector this lane holds.
template <int D, int DT>
__device__ inline void load_quarter(const void *x, size_t base, int p, float (&y)[D / 4]) {
  constexpr int C = D / 4;
  if constexpr (DT == TQ_F32) {
    const float4 *src = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + base + C * p);
#pragma unroll
    for (int q = 0; q < C / 4; ++q) {
      const float4 f = src[q];
      y[4 * q] = f.x;
      y[4 * q + 1] = f.y;
      y[4 * q + 2] = f.z;
      y[4 * q + 3] = f.w;
    }
  } else {
    const uint4 *src = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + base + C * p);
#pragma unroll
    for (int q = 0; q < C / 8; ++q) {
      const uint4 u = src[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[8 * q + 2 * k] = __uint_as_float(w[k] << 16);
        y[8 * q + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  }
}

// Unnormalised Walsh-Hadamard butterflies over a vector spread over a quad of
// lanes (coordinate C p + e in y[e] of lane p), distances 1, 2, ..., 2 C in
// increasing order, each pair (a, b) -> (a + b, a - b).
template <int D>
__device__ inline void fwht_quad(float (&y)[D / 4], int p) {
  constexpr int C = D / 4;
#pragma unroll
  for (int h = 1; h < C; h <<= 1)
#pragma unroll
    for (int e = 0; e < C; ++e)
      if (!(e & h)) {
        const float a = y[e], b = y[e | h];
        y[e] = a + b;
        y[e | h] = a - b;
      }
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const float o = xor_lane<1>(y[e]);
    y[e] = (p & 1) ? o - y[e] : y[e] + o;
  }
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const float o = xor_lane<2>(y[e]);
    y[e] = (p & 2) ? o - y[e] : y[e] + o;
  }
}

// Steps 1-3 on a quad: norm (returned), y = Pi x / ||x|| (0 for a zero vector).
template <int D>
__device__ inline float front_quad(float (&y)[D / 4], int p) {
  constexpr int C = D / 4;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < C; ++e) ss = fmaf(y[e], y[e], ss);
  ss += xor_lane<1>(ss);
  ss += xor_lane<2>(ss);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;
#pragma unroll
  for (int e = 0; e < C; ++e) y[e] *= inv;
  fwht_quad<D>(y, p);
#pragma unroll
  for (int e = 0; e < C; ++e) y[e] *= rsqrt_dim<D>();
  return n;
}

// Bitwise select: a where the mask m is all ones, b where it is zero (one
// v_bfi_b32; written this way so that no select becomes a branch).
__device__ inline uint32_t bsel(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }
__device__ inline uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline uint32_t ge_mask(float y, uint32_t t) {
  return y >= __builtin_bit_cast(float, t) ? 0xFFFFFFFFu : 0u;
}

// Code = #{k : t_k <= y} (a tie goes to the upper cell) by binary search over
// the ascending thresholds, NB-bit codes; m[j] is the all-ones mask of code bit
// j (the bit planes), the code is returned.
template <int NB>
__device__ inline int code_bsearch(const Codebook &cb, float y, uint32_t (&m)[NB]) {
  uint32_t T[(1 << NB) - 1];
#pragma unroll
  for (int k = 0; k < (1 << NB) - 1; ++k) T[k] = fbits(cb.thresholds[k]);
  if constexpr (NB == 2) {
    m[1] = ge_mask(y, T[1]);
    m[0] = ge_mask(y, bsel(m[1], T[2], T[0]));
  } else if constexpr (NB == 3) {
    m[2] = ge_mask(y, T[3]);
    m[1] = ge_mask(y, bsel(m[2], T[5], T[1]));
    m[0] = ge_mask(y, bsel(m[2], bsel(m[1], T[6], T[4]), bsel(m[1], T[2], T[0])));
  } else {
    static_assert(NB == 4, "code width");
    m[3] = ge_mask(y, T[7]);
    m[2] = ge_mask(y, bsel(m[3], T[11], T[3]));
    m[1] = ge_mask(y, bsel(m[3], bsel(m[2], T[13], T[9]), bsel(m[2], T[5], T[1])));
    const uint32_t t0 = bsel(m[3], bsel(m[2], bsel(m[1], T[14], T[12]), bsel(m[1], T[10], T[8])),
                             bsel(m[2], bsel(m[1], T[6], T[4]), bsel(m[1], T[2], T[0])));
    m[0] = ge_mask(y, t0);
  }
  int idx = 0;
#pragma unroll
  for (int j = 0; j < NB; ++j) idx |= (int)(m[j] & (1u << j));
  return idx;
}

// c[code] from the bit-plane masks, by bitwise selects over the levels.
template <int NB, int BASE = 0>
__device__ inline uint32_t level_bits(const Codebook &cb, const uint32_t (&m)[NB]) {
  if constexpr (NB == 0) {
    return fbits(cb.levels[BASE]);
  } else {
    // the top remaining bit is m[NB - 1]
    uint32_t mm[NB - 1 > 0 ? NB - 1 : 1];
#pragma unroll
    for (int j = 0; j + 1 < NB; ++j) mm[j] = m[j];
    if constexpr (NB == 1) {
      return bsel(m[0], fbits(cb.levels[BASE + 1]), fbits(cb.levels[BASE]));
    } else {
      const uint32_t lo = level_bits<NB - 1, BASE>(cb, reinterpret_cast<const uint32_t (&)[NB - 1]>(mm));
      const uint32_t hi = level_bits<NB - 1, BASE + (1 << (NB - 1))>(cb, reinterpret_cast<const uint32_t (&)[NB - 1]>(mm));
      return bsel(m[NB - 1], hi, lo);
    }
  }
}

typedef float v4f __attribute__((ext_vector_type(4)));

// K encode of 64 vectors: codes, residual and G on quads; the residuals go to
// LDS, where Z = R S^T runs on fp32 MFMA (16x16x4 tiles: 16 vectors by 16 rows
// of S, with S read from L2 once per workgroup), and the signs come back by
// ballot; each lane then stores its groups' record words.
template <int D, int DT, int KB>
__device__ void encode_k_bulk(const EncodeArgs &a, long blk) {
  constexpr int C = D / 4;                  // coordinates per lane
  constexpr int NGL = C / 32;               // 32-coordinate groups per lane: 1 or 2
  constexpr int VB = 64, VT = 4;            // vectors per workgroup, 16-vector MFMA tiles
  constexpr int RT = D / 16 / kWaves;       // 16-row tiles of S per wave: 2 or 4
  constexpr size_t KREC = (size_t)(KB + 1) * D / 8;
  constexpr size_t KCODES = (size_t)kPage * KREC;
  constexpr size_t KSEC = KCODES + 4 * kPage;
  __shared__ float4 s_r[VB][D / 4 + 1];     // residuals (rows padded: no bank conflicts)
  __shared__ uint16_t s_sign[VB][D / 16];   // sign bits, 16 rows of S per entry

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int v = lane >> 2, p = lane & 3;
  const int u = 16 * wave + v;              // this lane's vector in the workgroup
  const long total = (long)a.n_tokens * a.n_heads;
  const long v0 = blk * VB;
  const int nv = (int)min((long)VB, total - v0);
  const bool live = u < nv;

  const float4 *S4 = reinterpret_cast<const float4 *>(a.qjl);
  const bool qjl = a.qjl != nullptr;        // MSE-only keys skip z = S r
  constexpr bool kHoist = D == 128;
  float4 sreg[kHoist ? RT * (D / 16) : 1];
  if (kHoist && qjl) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        sreg[t * (D / 16) + c] = S4[(size_t)(16 * (wave * RT + t) + l16) * (D / 4) + 4 * c + kq];
  }

  float y[C];
  if (live) {
    load_quarter<D, DT>(a.x, (size_t)(v0 + u) * D, p, y);
  } else {
#pragma unroll
    for (int e = 0; e < C; ++e) y[e] = 0.f;
  }
  const float n = front_quad<D>(y, p);
  uint32_t w[NGL][KB];
#pragma unroll
  for (int g = 0; g < NGL; ++g)
#pragma unroll
    for (int j = 0; j < KB; ++j) w[g][j] = 0u;
  float rr = 0.f;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    uint32_t m[KB];
    code_bsearch<KB>(a.cb, y[e], m);
    y[e] -= __builtin_bit_cast(float, level_bits<KB>(a.cb, m));
    rr = fmaf(y[e], y[e], rr);
#pragma unroll
    for (int j = 0; j < KB; ++j) w[e / 32][j] |= m[j] & (1u << (e % 32));
  }
  rr += xor_lane<1>(rr);
  rr += xor_lane<2>(rr);
  const float gm = sqrtf(rr);
  // residuals of dead vectors are zero (their Z rows are not used)
#pragma unroll
  for (int q = 0; q < C / 4; ++q)
    s_r[u][(C / 4) * p + q] = live ? make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3])
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();

  // Z tile (vector tile vt, row tile rt) = sum over i of R[16 vt + .][i] S[16 rt + .][i]
  if (qjl) {
    v4f acc[VT][RT];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[vt][t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      float4 bv[RT], av[VT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if constexpr (kHoist)
          bv[t] = sreg[t * (D / 16) + c];
        else
          bv[t] = S4[(size_t)(16 * (wave * RT + t) + l16) * (D / 4) + 4 * c + kq];
      }
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) av[vt] = s_r[16 * vt + l16][4 * c + kq];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
#pragma unroll
          for (int t = 0; t < RT; ++t)
            acc[vt][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[vt][m], bv[t][m], acc[vt][t], 0, 0, 0);
    }
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint64_t m = __ballot(acc[vt][t][r] >= 0.f);
          const int uu = 16 * vt + 4 * kq + r;
          if (l16 == 0) s_sign[uu][wave * RT + t] = (uint16_t)(m >> (16 * kq));
        }
  }
  __syncthreads();

  if (!live) return;
  const long vec = v0 + u;
  const long tok = vec / a.n_heads;
  const int head = (int)(vec % a.n_heads);
  const int slot = a.slots[tok];
  uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * KSEC;
  const int off = slot % kPage;
  uint32_t *rec = reinterpret_cast<uint32_t *>(sec + (size_t)off * KREC);
#pragma unroll
  for (int g = 0; g < NGL; ++g) {
    const int sg = NGL * p + g;             // coordinate group of these words
    const uint32_t sw = qjl ? (uint32_t)s_sign[u][2 * sg] | ((uint32_t)s_sign[u][2 * sg + 1] << 16) : 0u;
    if constexpr (KB == 3) {
      reinterpret_cast<uint4 *>(rec)[sg] = make_uint4(w[g][0], w[g][1], w[g][2], sw);
    } else {
#pragma unroll
      for (int j = 0; j < KB; ++j) rec[(KB + 1) * sg + j] = w[g][j];
      rec[(KB + 1) * sg + KB] = sw;
    }
  }
  if (p == 0) {
    reinterpret_cast<uint16_t *>(sec + KCODES)[side_entry(off)] = f32_to_f16_bits(n);
    reinterpret_cast<uint16_t *>(sec + KCODES + 2 * kPage)[side_entry(off)] = f32_to_f16_bits(gm);
  }
}

// V encode of 64 tokens of one KV head: codes on quads; each lane's plane
// words go to LDS as [plane][group][token]. When the 64 slots are one whole
// aligned 64-token block of a page, the block's words are assembled from there
// and stored whole; otherwise each token's bits are set one by one with
// atomics, leaving the neighbours in the same words intact.
template <int D, int DT, int VBITS>
__device__ void encode_v_bulk(const EncodeArgs &a, int bx, int head) {
  constexpr int C = D / 4;
  constexpr int NGL = C / 32;
  constexpr int NGR = D / 32;               // 32-coordinate groups per vector
  constexpr int TP = 64 + 4;                // token stride of a group row (padded)
  constexpr size_t VCODES = (size_t)VBITS * D * kPage / 8;
  constexpr size_t VSEC = VCODES + 2 * kPage;
  __shared__ __attribute__((aligned(16))) uint32_t s_pl[VBITS][NGR][TP];
  __shared__ int s_whole;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int v = lane >> 2, p = lane & 3;
  const int ut = 16 * wave + v;             // this lane's token in the workgroup
  const int t0 = bx * 64;
  const int nt = min(64, a.n_tokens - t0);
  const bool live = ut < nt;
  if (threadIdx.x == 0) {
    const int s0 = a.slots[t0];
    s_whole = (nt == 64 && (s0 & 63) == 0);
  }
  __syncthreads();
  if (threadIdx.x < nt && a.slots[t0 + threadIdx.x] != a.slots[t0] + (int)threadIdx.x)
    s_whole = 0;   // benign race: every writer stores 0

  float y[C];
  if (live) {
    load_quarter<D, DT>(a.x, ((size_t)(t0 + ut) * a.n_heads + head) * D, p, y);
  } else {
#pragma unroll
    for (int e = 0; e < C; ++e) y[e] = 0.f;
  }
  const float n = front_quad<D>(y, p);
  uint32_t w[NGL][VBITS];
#pragma unroll
  for (int g = 0; g < NGL; ++g)
#pragma unroll
    for (int j = 0; j < VBITS; ++j) w[g][j] = 0u;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    uint32_t m[VBITS];
    code_bsearch<VBITS>(a.cb, y[e], m);
#pragma unroll
    for (int j = 0; j < VBITS; ++j) w[e / 32][j] |= m[j] & (1u << (e % 32));
  }
#pragma unroll
  for (int g = 0; g < NGL; ++g)
#pragma unroll
    for (int j = 0; j < VBITS; ++j) s_pl[j][NGL * p + g][ut] = w[g][j];
  __syncthreads();

  if (s_whole) {
    const int s0 = a.slots[t0];
    uint8_t *sec = a.pool + ((size_t)(s0 / kPage) * a.n_heads + head) * VSEC;
    const int bofs = s0 % kPage;   // offset of the block in the page (a multiple of 64)
    uint32_t *words = reinterpret_cast<uint32_t *>(sec) + (bofs >> 6) * 2 * VBITS * D;
    // word e = j*2D + (16 k + nn)*(D/32) + kp; bit 8 r + 4 h + tau <- token
    // 16 tau + 4 k + r, coordinate 32 kp + 16 h + nn: bit nn + 16 h of the
    // token's group-kp word
    for (int e = threadIdx.x; e < 2 * VBITS * D; e += 256) {
      const int j = e / (2 * D), rem = e % (2 * D);
      const int c = rem / NGR, kp = rem % NGR;
      const int k = c >> 4, nn = c & 15;
      const uint32_t *row = &s_pl[j][kp][4 * k];
      uint32_t word = 0u;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        const uint4 q = *reinterpret_cast<const uint4 *>(row + 16 * tau);   // tokens 16 tau + 4 k + r
        const uint32_t qs[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          word |= ((qs[r] >> nn) & 1u) << (8 * r + tau);
          word |= ((qs[r] >> (nn + 16)) & 1u) << (8 * r + 4 + tau);
        }
      }
      words[e] = word;
    }
    if (live && p == 0)
      reinterpret_cast<uint16_t *>(sec + VCODES)[side_entry(bofs + ut)] = f32_to_f16_bits(n);
    return;
  }

  if (!live) return;
  const int slot = a.slots[t0 + ut];
  uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * VSEC;
  const int off = slot % kPage;
  uint32_t *rows = reinterpret_cast<uint32_t *>(sec);
  // coordinates i = 32 kp + 16 h + nn and i + 16 share a word: set and clear
  // both bits with one atomic each
#pragma unroll
  for (int g = 0; g < NGL; ++g) {
    const int kp = NGL * p + g;
#pragma unroll
    for (int j = 0; j < VBITS; ++j)
#pragma unroll
      for (int nn = 0; nn < 16; ++nn) {
        const int i = 32 * kp + nn;
        uint32_t *wd = rows + v_word<D, VBITS>(off, i, j);
        const uint32_t b0 = 1u << v_bit(off, i), b1 = 1u << v_bit(off, i + 16);
        const uint32_t set = ((w[g][j] >> nn) & 1u ? b0 : 0u) | ((w[g][j] >> (nn + 16)) & 1u ? b1 : 0u);
        const uint32_t clr = (b0 | b1) & ~set;
        if (set) atomicOr(wd, set);
        if (clr) atomicAnd(wd, ~clr);
      }
  }
  if (p == 0) reinterpret_cast<uint16_t *>(sec + VCODES)[side_entry(off)] = f32_to_f16_bits(n);
}

template <int D, int DT, int KB>
__global__ __launch_bounds__(256) void encode_k_bulk_kernel(EncodeArgs a) {
  encode_k_bulk<D, DT, KB>(a, blockIdx.x);
}

template <int D, int DT, int VBITS>
__global__ __launch_bounds__(256) void encode_v_bulk_kernel(EncodeArgs a) {
  encode_v_bulk<D, DT, VBITS>(a, blockIdx.x, blockIdx.y);
}

template <int D, int DT, int KB>
__global__ __launch_bounds__(256) void encode_k_kernel(EncodeArgs a) {
  encode_k_block<D, DT, KB>(a, blockIdx.x);
}

template <int D, int DT, int VPW, int VBITS>
__global__ __launch_bounds__(256) void encode_v_kernel(EncodeArgs a) {
  encode_v_block<D, DT, VPW, VBITS>(a, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------ prepare
// One or kPrepPieces workgroups per query row qq of a (sequence, KV head)
// group (a.pieces): each rotates the row and projects it with S (the four
// waves split the m rows of S, and every S load of a chunk is issued before the
// row is rotated), then packs its share of the kPrepPieces shares of the row's
// fp6 scoring operand; piece 0 also writes q~, p and the row constants. Packing
// is a long chain of dependent steps per lane, so with few rows it is spread
// over more SIMDs; with many rows a workgroup takes kPrepRows rows and reads S
// once for them.
constexpr int kPrepPieces = 4;
constexpr int kPrepRows = 4;

// Rotation and projection of NRW consecutive rows qq0 .. qq0 + NRW - 1 of a
// (sequence, KV head) group, of which the first nr exist (the same for every key
// code width): q~ of row i into s_q[i], p = S q~ into s_p[i]; piece 0 writes both
// to the query region. The S loads are shared by the NRW rows.
template <int D, int DT, int NRW>
__device__ void prepare_front(const PrepArgs &a, int qq0, int nr, int kvh, int b, int piece, float (*s_q)[D],
                              float (*s_p)[D]) {
  constexpr int R = D / 64;
  constexpr int RPW = D / 4;         // rows of S per wave
  constexpr int LPR = 64 / RPW;      // lanes per row of S: 2 (d = 128) or 1 (d = 256)
  constexpr int EPL = D / LPR;       // elements of a row per lane
  constexpr int CH = 16;             // float4 loads in flight per lane
  constexpr int NCH = EPL / 4 / CH;  // chunks: 1 (d = 128) or 4 (d = 256)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = a.n_q_heads / a.n_kv_heads;
  size_t row[NRW];
#pragma unroll
  for (int i = 0; i < NRW; ++i) {
    const int qq = qq0 + min(i, nr - 1);   // rows past the group repeat the last one (not written)
    const int t = qq / g, hh = qq % g;
    row[i] = ((size_t)b * a.n_q + t) * a.n_q_heads + kvh * g + hh;
  }
  const int srow = wave * RPW + lane / LPR, part = lane % LPR;
  const float4 *S4 = reinterpret_cast<const float4 *>(a.qjl);
  const size_t s_off = (size_t)srow * (D / 4) + part * (EPL / 4);   // this lane's part of its S row
  const bool qjl = a.qjl != nullptr;   // MSE-only keys: p = 0, S is not read
  // the rows are loaded first: loads complete in order, and the rotation, which
  // needs the rows, runs while the S loads are in flight
  float v[NRW][R];
#pragma unroll
  for (int i = 0; i < NRW; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) v[i][r] = load_elem<DT>(a.q, row[i] * D + lane + 64 * r);
  float4 sv[CH];
  if (qjl) {
#pragma unroll
    for (int k = 0; k < CH; ++k) sv[k] = S4[s_off + k];
  }
#pragma unroll
  for (int i = 0; i < NRW; ++i) {
    fwht_wave<R>(v[i]);
#pragma unroll
    for (int r = 0; r < R; ++r) v[i][r] *= rsqrt_dim<D>();
  }
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < NRW; ++i) {
      float *dst = a.prep + row[i] * 2 * D;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s_q[i][lane + 64 * r] = v[i][r];
        if (piece == 0 && i < nr) dst[lane + 64 * r] = v[i][r];
      }
    }
  }
  __syncthreads();

  // p_l = sum_i S[l][i] q~_i
  float acc[NRW];
#pragma unroll
  for (int i = 0; i < NRW; ++i) acc[i] = 0.f;
  if (qjl) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c > 0) {
#pragma unroll
        for (int k = 0; k < CH; ++k) sv[k] = S4[s_off + c * CH + k];
      }
#pragma unroll
      for (int i = 0; i < NRW; ++i) {
        const float4 *q4 = reinterpret_cast<const float4 *>(s_q[i]) + part * (EPL / 4);
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const float4 qv = q4[c * CH + k];
          acc[i] = fmaf(sv[k].x, qv.x, acc[i]);
          acc[i] = fmaf(sv[k].y, qv.y, acc[i]);
          acc[i] = fmaf(sv[k].z, qv.z, acc[i]);
          acc[i] = fmaf(sv[k].w, qv.w, acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NRW; ++i) {
    if (LPR == 2) acc[i] += __shfl_xor(acc[i], 1, 64);
    if (part == 0) {
      s_p[i][srow] = acc[i];
      if (piece == 0 && i < nr) a.prep[row[i] * 2 * D + D + srow] = acc[i];
    }
  }
}

// This piece's share of the row's scoring operand (KB-bit key codes), from
// s_q and s_p. In a 4-row group the operand of MFMA mu holds the row's four
// limbs on rows 4 qloc + limb; in a 16-row (wide) group limb l of every row
// has an operand of its own, (mu, l), with the row on row qloc.
template <int D, int KB, bool WIDE>
__device__ void prepare_pack(const PrepArgs &a, int qq, int kvh, int b, int piece, const float *s_q,
                             const float *s_p) {
  constexpr int R = D / 64;
  constexpr int NPK = k_planes(KB);    // key code planes (KB-bit codes), then the sign plane
  constexpr int NMU = mfma_per_tile(D, KB);   // scoring MFMAs per 16-token tile
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.n_q_heads / a.n_kv_heads * a.n_q;

  // Scoring operand of this row for the fp6 x fp4 block-scaled MFMA
  // (16x16x128): MFMA mu = 5 c + pl scores coordinate chunk c (coordinates
  // 128 c .. 128 c + 127) against key plane pl (code bits 0..2, their xor, then
  // the QJL sign). Both operands hold K = 32 kq + f in lane group kq, slot f (a
  // nibble of the key side, a 6-bit field of the query side, fields packed
  // contiguously from bit 0). Key side (B, fp4): slot f = 8 v + m of lane group
  // kq holds bit 4 m + v of the plane word of coordinate group s = kq + 4 c,
  // i.e. coordinate 32 s + 4 m + v, with value 0.5, 1, 2, 2 for v = 0..3 (v = 3
  // is shifted down one bit). Query side (A, fp6 e2m3): the paired slot holds
  // y / value, y = w_pl * q~_i (code planes; c[idx] = sum_pl w_pl b_pl - c7) or
  // 2 kappa p_i (sign plane, sigma = 2 b - 1), as four limbs on the rows
  // 4 q + limb, each limb with an E8M0 scale per 32-slot block (in lane
  // 16 kq + row), so the MFMA sums of the four limb rows add up to the product.
  float w[NPK];
  if constexpr (KB == 3)
    plane_weights(a.cb, w);
  else
    plane_weights_walsh<KB>(a.cb, w);
  float sq = 0.f, sp = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    sq += s_q[lane + 64 * r];
    sp += s_p[lane + 64 * r];
  }
  sq = wave_sum(sq);
  sp = wave_sum(sp);
  // query group rho = qq / RG has its own operand; this row is its row qloc
  constexpr int RG = WIDE ? kWideRows : kMfmaMaxGroup;   // rows per query group
  constexpr int NOP = WIDE ? 4 * NMU : NMU;              // MFMA operands per group
  static_assert(!WIDE || KB == 3, "wide groups take 3-bit keys");
  const int QG = (G + RG - 1) / RG, rho = qq / RG, qloc = qq % RG;
  const int Gr = min(RG, G - RG * rho);   // rows of the group
  const size_t gbytes = WIDE ? packed_group_bytes_wide(D) : packed_group_bytes(D, KB);
  uint8_t *grp = a.packed + (((size_t)b * a.n_kv_heads + kvh) * QG + rho) * gbytes;
  uint8_t *opb = grp;                                                  // [operand][lane][32] bytes
  uint32_t *scl = reinterpret_cast<uint32_t *>(grp + (size_t)NOP * 2048);   // [operand][lane]
  // where limb `limb` of this row's k-block kb sits: operand and lane
  auto op_lane = [&](int mu, int kb, int limb) {
    return WIDE ? (mu * 4 + limb) * 64 + 16 * kb + qloc : mu * 64 + 16 * kb + 4 * qloc + limb;
  };
  const float kap2 = 2.f * qjl_kappa<D>();
  // Piece p takes the (MFMA, block pair) tasks p TP .. p TP + TP - 1 and its
  // wave w the tasks w, w + 4, ... of them: two 32-slot blocks at a time, one
  // per half-wave, as one branch-free block, so their limb chains interleave. Lane e of a half holds
  // field e; the fields (field f at bits 6 f .. 6 f + 5 of the 192) are packed
  // in registers: field pairs, then quads, are merged across lanes (a quad's 24
  // bits in its first lane), and lane 4 j of each 16-lane row (j = 0, 1, 2)
  // builds dword j of the row's 96 bits from its quad and the next, or (j = 3)
  // a zero for dword 6 or 7. Every lane of a quad stores its first lane's dword
  // and every lane of a half the block's scale: same address, same value.
  constexpr int NTASK = NMU * 2;   // (mu, block pair) tasks
  const int e = threadIdx.x & 31, hb = lane >> 5;
  const int fv = e >> 3, fm = e & 7;   // field e: bit 4 fm + fv of its plane word
  const float ival = fv == 0 ? 2.f : fv == 1 ? 1.f : 0.5f;   // 1 / the key slot's value
  const int prow = e >> 4, pj = (e & 15) >> 2;   // the lane's row and quad in it
  const int pdw = pj < 3 ? 3 * prow + pj : 6 + prow;   // the dword quad pj of row prow writes
  auto pack_task = [&](int task) {
    const int mu = task >> 1, kb = 2 * (task & 1) + hb;
    const int c = mu / (NPK + 1), pl = mu % (NPK + 1);
    const int i = 32 * (kb + 4 * c) + 4 * fm + fv;
    const float sqi = s_q[i], spi = s_p[i];   // both read: no branch on the plane
    float r = (pl < NPK ? w[min(pl, NPK - 1)] * sqi : kap2 * spi) * ival;
    // limb 0: the block scale 2^ex puts the block's largest value in [4, 8).
    // Later limbs take their scale from the rounding bound of the previous one
    // (no reduction): limb 0 leaves |r| <= 0.5 * 2^ex (0.25 from rounding in
    // [4, 8), 0.5 where 7.75 .. 8 saturates to 7.5), so limb 1 uses ex - 3;
    // a limb whose values stay below 4 leaves |r| <= 0.125 * 2^ex, so limbs 2
    // and 3 use ex - 5. Every later limb value is then at most 4, no later limb
    // saturates, and after four limbs |r| <= 2^(ex0 - 16), under 2^-18 of the
    // block's largest value.
    float mx = fabsf(r);
    mx = fmaxf(mx, xor_lane<1>(mx));
    mx = fmaxf(mx, xor_lane<2>(mx));
    mx = fmaxf(mx, xor_lane<4>(mx));
    mx = fmaxf(mx, xor_lane<8>(mx));
    mx = fmaxf(mx, xor_lane<16>(mx));
    const int ex0 = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) - 3 : 0;
#pragma unroll
    for (int limb = 0; limb < 4; ++limb) {
      const int ex = max(-127, min(127, ex0 - (limb == 0 ? 0 : limb == 1 ? 3 : 3 + 5 * (limb - 1))));
      uint32_t code;
      const float qv = fp6_e2m3_round(__builtin_ldexpf(r, -ex), code);
      r = fmaf(-qv, __builtin_ldexpf(1.f, ex), r);
      // pairs (lane 2 k), then quads (lane 4 k): fields 4 k .. 4 k + 3 in 24 bits
      uint32_t pk = code | ((uint32_t)__builtin_amdgcn_mov_dpp((int)code, 0xB1, 0xF, 0xF, true) << 6);
      pk |= (uint32_t)__builtin_amdgcn_mov_dpp((int)pk, 0x4E, 0xF, 0xF, true) << 12;
      const uint32_t nx = (uint32_t)__shfl_down((int)pk, 4, 16);   // the next quad of the row
      uint32_t word = pj < 3 ? (pk >> (8 * pj)) | (nx << (24 - 8 * pj)) : 0u;
      word = (uint32_t)__builtin_amdgcn_mov_dpp((int)word, 0x00, 0xF, 0xF, true);   // quad_perm [0,0,0,0]
      reinterpret_cast<uint32_t *>(opb)[(size_t)op_lane(mu, kb, limb) * 8 + pdw] = word;
      scl[op_lane(mu, kb, limb)] = (uint32_t)(ex + 127);
    }
  };
  // every wave runs the same number of rounds; a task index past the piece's
  // last is clamped to it, so that task is computed twice and stored twice with
  // the same values, and all rounds stay one branch-free block
  constexpr int TP = (NTASK + kPrepPieces - 1) / kPrepPieces, NT = (TP + 3) / 4;
  const int per = kPrepPieces / a.pieces;   // shares of this workgroup
  for (int sh = piece * per; sh < piece * per + per; ++sh) {
    const int tlast = min(NTASK, TP * (sh + 1)) - 1;
    if (TP * sh <= tlast) {
#pragma unroll
      for (int t = 0; t < NT; ++t) pack_task(min(TP * sh + wave + 4 * t, tlast));
    }
  }
  if (piece != 0) return;
  // MFMA rows of the group's rows Gr .. RG - 1 (no query): zero fields, unit
  // scales (operand rows 4 r + limb of a 4-row group, row r of a wide one)
  constexpr int RPR = WIDE ? 1 : 4;   // MFMA rows per query row in one operand
  if (qloc == 0 && Gr < RG) {
    const int nrow = RPR * (RG - Gr);
    for (int t = threadIdx.x; t < NOP * 4 * nrow * 32; t += 256) {
      const int byte = t & 31, rest = t >> 5;
      const int row = RPR * Gr + rest % nrow, lg = (rest / nrow) & 3, op = rest / nrow / 4;
      opb[((size_t)op * 64 + 16 * lg + row) * 32 + byte] = 0;
      if (byte == 0) scl[op * 64 + 16 * lg + row] = 127u;
    }
  }
  // row constants: {0, 0, sum q~, sum p} per row of a 4-row group, {sum q~, sum p} of a wide one
  constexpr int RCW = WIDE ? 2 : 4;
  float *rc = reinterpret_cast<float *>(grp + (size_t)NOP * (2048 + 256));
  if (threadIdx.x < RCW) {
    const float cv[4] = {0.f, 0.f, sq, sp};
    rc[RCW * qloc + threadIdx.x] = cv[4 - RCW + threadIdx.x];
  } else if (qloc == 0 && threadIdx.x < RCW * RG && threadIdx.x >= RCW * Gr) {
    rc[threadIdx.x] = 0.f;
  }
}

// Rows qq0 .. qq0 + nr - 1 (nr <= NRW) of one (sequence, KV head) group.
template <int D, int DT, int NRW>
__device__ void prepare_rows(const PrepArgs &a, int qq0, int nr, int kvh, int b, int piece) {
  __shared__ float s_q[NRW][D], s_p[NRW][D];
  prepare_front<D, DT, NRW>(a, qq0, nr, kvh, b, piece, s_q, s_p);
  if (a.packed == nullptr) return;
  __syncthreads();
  for (int i = 0; i < nr; ++i) {
    // the K code width and the group width are uniform over the launch
    if (a.wide)
      prepare_pack<D, 3, true>(a, qq0 + i, kvh, b, piece, s_q[i], s_p[i]);
    else if (a.k_bits == 2)
      prepare_pack<D, 2, false>(a, qq0 + i, kvh, b, piece, s_q[i], s_p[i]);
    else if (a.k_bits == 4)
      prepare_pack<D, 4, false>(a, qq0 + i, kvh, b, piece, s_q[i], s_p[i]);
    else
      prepare_pack<D, 3, false>(a, qq0 + i, kvh, b, piece, s_q[i], s_p[i]);
  }
}

template <int D, int DT>
__device__ void prepare_row(const PrepArgs &a, int qq, int kvh, int b, int piece) {
  prepare_rows<D, DT, 1>(a, qq, 1, kvh, b, piece);
}

// Workgroup x of a (sequence, KV head): with pieces > 1, piece x % pieces of
// row x / pieces; else rows kPrepRows x .. kPrepRows x + kPrepRows - 1.
template <int D, int DT>
__global__ __launch_bounds__(256) void prepare_kernel(PrepArgs a) {
  if (a.pieces > 1) {
    prepare_row<D, DT>(a, blockIdx.x / a.pieces, blockIdx.y, blockIdx.z, blockIdx.x % a.pieces);
  } else {
    const int G = a.n_q * (a.n_q_heads / a.n_kv_heads);
    const int qq0 = kPrepRows * blockIdx.x;
    prepare_rows<D, DT, kPrepRows>(a, qq0, min(kPrepRows, G - qq0), blockIdx.y, blockIdx.z, 0);
  }
}

// One launch for the work of a decode step that precedes the split-K decode:
// workgroups [0, nk) encode the appended K vectors (one each), the next nv
// encode the appended V vectors (one token per wave and KV head) and the rest
// prepare the query rows (kPrepPieces workgroups each). The three parts touch
// disjoint memory.
// The workgroup counts come first and the query arguments next, so the role
// test and the start of a query row read one or two kernel-argument lines.
struct StepArgs {
  int nk, nvx, nv, pad;   // K workgroups; V workgroups per KV head and in total
  PrepArgs p;
  EncodeArgs k, v;
};

template <int D, int DT>
__global__ __launch_bounds__(256) void step_prologue_kernel(StepArgs s) {
  // both counts in one load, before the first branch
  const int nk = s.nk, nv = s.nv;
  asm volatile("" ::"s"(nk), "s"(nv));
  int id = blockIdx.x;
  if (id < nk) {
    // the K code width is uniform over the launch
    if (s.k.bits == 2)
      encode_k_block<D, DT, 2>(s.k, id);
    else if (s.k.bits == 4)
      encode_k_block<D, DT, 4>(s.k, id);
    else
      encode_k_block<D, DT, 3>(s.k, id);
    return;
  }
  id -= nk;
  if (id < nv) {
    // the V code width is uniform over the launch
    if (s.v.bits == 2)
      encode_v_block<D, DT, 1, 2>(s.v, id % s.nvx, id / s.nvx);
    else if (s.v.bits == 4)
      encode_v_block<D, DT, 1, 4>(s.v, id % s.nvx, id / s.nvx);
    else
      encode_v_block<D, DT, 1, 3>(s.v, id % s.nvx, id / s.nvx);
    return;
  }
  id -= nv;
  const int piece = id % s.p.pieces;
  id /= s.p.pieces;
  const int G = s.p.n_q * (s.p.n_q_heads / s.p.n_kv_heads);
  const int qq = id % G, kvh = (id / G) % s.p.n_kv_heads, b = id / (G * s.p.n_kv_heads);
  prepare_row<D, DT>(s.p, qq, kvh, b, piece);
}

template <int D>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a, int which) {
  constexpr int R = D / 64;
  const int kw = a.bits + 1;                          // K: words per 32 coordinates
  const size_t KREC = (size_t)kw * D / 8;
  const size_t KCODES = (size_t)kPage * KREC;
  const size_t KSEC = KCODES + 4 * kPage;
  const size_t VCODES = (size_t)a.bits * D * kPage / 8;   // V: a.bits-bit codes
  const size_t VSEC = VCODES + 2 * kPage;
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
    const uint32_t *rec = reinterpret_cast<const uint32_t *>(sec + (size_t)off * KREC);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = lane + 64 * r, s = i >> 5, e = i & 31;
      int idx = 0;
      for (int j = 0; j < a.bits; ++j) idx |= ((rec[kw * s + j] >> e) & 1) << j;
      v[r] = level_any(a.cb, idx);
    }
    scale = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(sec + KCODES)[side_entry(off)]);
    if (a.with_qjl) {
      const float G = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(sec + KCODES + 2 * kPage)[side_entry(off)]);
      float t[R];
#pragma unroll
      for (int r = 0; r < R; ++r) t[r] = 0.f;
      for (int l = 0; l < D; ++l) {
        const bool pos = (rec[kw * (l >> 5) + a.bits] >> (l & 31)) & 1;
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
      for (int j = 0; j < a.bits; ++j) idx |= ((rows[v_word_rt(off, i, j, D, a.bits)] >> bit) & 1) << j;
      v[r] = level_any(a.cb, idx);
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

// Bulk calls (4096 vectors or more) use the quad kernels, 64 vectors per
// workgroup; short appends use one vector per wave, so that the work spreads
// over more workgroups and each vector's latency chain is short.
hipError_t launch_encode_k(const EncodeArgs &a, int d, hipStream_t s) {
  const long total = (long)a.n_tokens * a.n_heads;
  return by_dim_dtype(d, a.dtype, [&](auto D, auto DT) {
    auto go = [&](auto KB) {
      if (total < 4096) {
        const dim3 grid((unsigned)total);   // one vector per workgroup
        hipLaunchKernelGGL((encode_k_kernel<D.value, DT.value, KB.value>), grid, dim3(256), 0, s, a);
      } else {
        const dim3 grid((unsigned)((total + 63) / 64));
        hipLaunchKernelGGL((encode_k_bulk_kernel<D.value, DT.value, KB.value>), grid, dim3(256), 0, s, a);
      }
    };
    if (a.bits == 2)
      go(std::integral_constant<int, 2>{});
    else if (a.bits == 4)
      go(std::integral_constant<int, 4>{});
    else
      go(std::integral_constant<int, 3>{});
    return hipGetLastError();
  });
}

hipError_t launch_encode_v(const EncodeArgs &a, int d, hipStream_t s) {
  const long total = (long)a.n_tokens * a.n_heads;
  return by_dim_dtype(d, a.dtype, [&](auto D, auto DT) {
    auto go = [&](auto VBITS) {
      if (total < 4096) {
        const dim3 grid((unsigned)((a.n_tokens + kWaves - 1) / kWaves), (unsigned)a.n_heads);
        hipLaunchKernelGGL((encode_v_kernel<D.value, DT.value, 1, VBITS.value>), grid, dim3(256), 0, s, a);
      } else {
        const dim3 grid((unsigned)((a.n_tokens + 63) / 64), (unsigned)a.n_heads);
        hipLaunchKernelGGL((encode_v_bulk_kernel<D.value, DT.value, VBITS.value>), grid, dim3(256), 0, s, a);
      }
    };
    if (a.bits == 2)
      go(std::integral_constant<int, 2>{});
    else if (a.bits == 4)
      go(std::integral_constant<int, 4>{});
    else
      go(std::integral_constant<int, 3>{});
    return hipGetLastError();
  });
}

// Workgroups per query row: kPrepPieces while the rows are few (the launch is
// latency-bound), else one (each workgroup reads S).
static int prep_pieces(const PrepArgs &a) {
  const long rows = (long)a.n_q * a.n_q_heads * a.batch;
  return rows <= 256 ? kPrepPieces : 1;
}

hipError_t launch_prepare(const PrepArgs &a, int d, hipStream_t s) {
  PrepArgs pa = a;
  pa.pieces = prep_pieces(a);
  const int G = a.n_q * (a.n_q_heads / a.n_kv_heads);   // rows per (sequence, KV head)
  const dim3 grid(pa.pieces > 1 ? G * pa.pieces : (G + kPrepRows - 1) / kPrepRows, a.n_kv_heads, a.batch);
  if (d == 128) {
    if (a.dtype == TQ_F32)
      hipLaunchKernelGGL((prepare_kernel<128, TQ_F32>), grid, dim3(256), 0, s, pa);
    else
      hipLaunchKernelGGL((prepare_kernel<128, TQ_BF16>), grid, dim3(256), 0, s, pa);
  } else {
    if (a.dtype == TQ_F32)
      hipLaunchKernelGGL((prepare_kernel<256, TQ_F32>), grid, dim3(256), 0, s, pa);
    else
      hipLaunchKernelGGL((prepare_kernel<256, TQ_BF16>), grid, dim3(256), 0, s, pa);
  }
  return hipGetLastError();
}

bool step_prologue_fits(const EncodeArgs &k, const PrepArgs &p) {
  return (long)k.n_tokens * k.n_heads < 4096 && k.dtype == p.dtype;
}

hipError_t launch_step_prologue(const EncodeArgs &k, const EncodeArgs &v, const PrepArgs &p, int d,
                                hipStream_t s) {
  StepArgs sa;
  sa.pad = 0;
  sa.k = k;
  sa.v = v;
  sa.p = p;
  sa.p.pieces = prep_pieces(p);
  sa.nk = (int)((long)k.n_tokens * k.n_heads);   // one K vector per workgroup
  sa.nvx = (v.n_tokens + kWaves - 1) / kWaves;
  sa.nv = sa.nvx * v.n_heads;
  const long np = (long)p.n_q * p.n_q_heads * p.batch;   // query rows
  const dim3 grid((unsigned)(sa.nk + sa.nv + np * sa.p.pieces));
  return by_dim_dtype(d, k.dtype, [&](auto D, auto DT) {
    hipLaunchKernelGGL((step_prologue_kernel<D.value, DT.value>), grid, dim3(256), 0, s, sa);
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
