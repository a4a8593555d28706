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
template <int D, int DT, int NT = 7>
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
    idx[r] = quantize_code<NT>(cb, y[r]);
  }
  return n;
}

// K encode: VPW vectors per wave (16 for bulk encodes, 1 for short appends
// where latency rules). Each wave runs steps 1-4 on its vectors (codes by
// ballot, residual into LDS); the QJL product Z = R S^T over the workgroup's
// residuals then runs on fp32 MFMA (16x16x4), with S read from L2 once per
// workgroup; signs come back by ballot. Rows of R past the last vector are
// zero and their records are not written.
typedef float v4f __attribute__((ext_vector_type(4)));

template <int D, int DT, int VPW, int KB>
__device__ void encode_k_block(const EncodeArgs &a, long blk) {
  constexpr int R = D / 64;
  constexpr int NWORD = (KB + 1) * D / 32;  // u32 words per K record: KB code planes + signs per 32
  constexpr int VB = kWaves * VPW;          // vectors per workgroup
  constexpr int VT = (VB + 15) / 16;        // 16-vector MFMA tiles
  constexpr int RT = D / 16 / kWaves;       // 16-row tiles of S per wave: 2 or 4
  constexpr size_t KREC = (size_t)(KB + 1) * D / 8;
  constexpr size_t KCODES = (size_t)kPage * KREC;
  constexpr size_t KSEC = KCODES + 4 * kPage;
  __shared__ float4 s_r[16 * VT][D / 4];    // residuals
  __shared__ uint64_t s_code[VB][KB][R];    // code bit planes
  __shared__ uint16_t s_sign[VB][D / 16];   // sign bits, 16 rows of S per entry
  __shared__ float s_ng[VB][2];             // N, G

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const long total = (long)a.n_tokens * a.n_heads;
  const long v0 = blk * VB;
  const int nv = (int)min((long)VB, total - v0);

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

  for (int u = wave; u < 16 * VT; u += kWaves) {
    float4 *rrow = s_r[u];
    if (u >= nv) {
      for (int e = lane; e < D / 4; e += 64) rrow[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
    float y[R];
    int idx[R];
    const float n = encode_front<D, DT, (1 << KB) - 1>(a.x, (size_t)(v0 + u) * D, a.cb, y, idx);
    float rr = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      y[k] -= KB == 3 ? level_of(a.cb, idx[k]) : level_any(a.cb, idx[k]);
      rr += y[k] * y[k];
      reinterpret_cast<float *>(rrow)[lane + 64 * k] = y[k];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const uint64_t m = __ballot((idx[k] >> j) & 1);
        if (lane == 0) s_code[u][j][k] = m;
      }
    }
    const float gm = sqrtf(wave_sum(rr));
    if (lane == 0) {
      s_ng[u][0] = n;
      s_ng[u][1] = gm;
    }
  }
  __syncthreads();

  // Z tile (vector tile vt, row tile rt) = sum over i of R[16 vt + .][i] S[16 rt + .][i].
  // MFMA m of a 16-wide i step uses i = i0 + 4 kq + m in lane group kq, for A and B alike.
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
      // independent tiles between the dependent steps of one accumulator
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
#pragma unroll
          for (int t = 0; t < RT; ++t)
            acc[vt][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[vt][m], bv[t][m], acc[vt][t], 0, 0, 0);
    }
    // lane (l16, kq), register r of a tile: vector 16 vt + 4 kq + r, row 16 rt + l16
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint64_t m = __ballot(acc[vt][t][r] >= 0.f);
          const int u = 16 * vt + 4 * kq + r;
          if (l16 == 0 && u < VB) s_sign[u][wave * RT + t] = (uint16_t)(m >> (16 * kq));
        }
  }
  __syncthreads();

  // records: wave w writes vectors w, w + 4, ...
  for (int u = wave; u < nv; u += kWaves) {
    const long vec = v0 + u;
    const long tok = vec / a.n_heads;
    const int head = (int)(vec % a.n_heads);
    const int slot = a.slots[tok];
    uint8_t *sec = a.pool + ((size_t)(slot / kPage) * a.n_heads + head) * KSEC;
    const int off = slot % kPage;
    if (lane < NWORD) {
      const int s = lane / (KB + 1), j = lane % (KB + 1);   // coordinate group, word in it
      uint32_t w;
      if (j < KB) {
        const uint64_t m = s_code[u][j][s >> 1];
        w = (s & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
      } else {
        w = qjl ? (uint32_t)s_sign[u][2 * s] | ((uint32_t)s_sign[u][2 * s + 1] << 16) : 0u;
      }
      reinterpret_cast<uint32_t *>(sec + (size_t)off * KREC)[lane] = w;
    }
    if (lane == 0) {
      reinterpret_cast<uint16_t *>(sec + KCODES)[side_entry(off)] = f32_to_f16_bits(s_ng[u][0]);
      reinterpret_cast<uint16_t *>(sec + KCODES + 2 * kPage)[side_entry(off)] = f32_to_f16_bits(s_ng[u][1]);
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

template <int D, int DT, int VPW, int KB>
__global__ __launch_bounds__(256) void encode_k_kernel(EncodeArgs a) {
  encode_k_block<D, DT, VPW, KB>(a, blockIdx.x);
}

template <int D, int DT, int VPW, int VBITS>
__global__ __launch_bounds__(256) void encode_v_kernel(EncodeArgs a) {
  encode_v_block<D, DT, VPW, VBITS>(a, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------ prepare
// One workgroup per query row qq of a (sequence, KV head) group: rotate the
// row, project it with S, write q~ and p, and on the MFMA path pack this row's
// four limb rows of the fp6 scoring operand. The four waves split the m rows
// of S, and every S load of a chunk is issued before the row is rotated.
template <int D, int DT, int KB>
__device__ void prepare_row(const PrepArgs &a, int qq, int kvh, int b) {
  constexpr int R = D / 64;
  constexpr int NPK = k_planes(KB);    // key code planes (KB-bit codes), then the sign plane
  constexpr int NMU = mfma_per_tile(D, KB);   // scoring MFMAs per 16-token tile
  constexpr int RPW = D / 4;         // rows of S per wave
  constexpr int LPR = 64 / RPW;      // lanes per row of S: 2 (d = 128) or 1 (d = 256)
  constexpr int EPL = D / LPR;       // elements of a row per lane
  constexpr int CH = 16;             // float4 loads in flight per lane
  constexpr int NCH = EPL / 4 / CH;  // chunks: 1 (d = 128) or 4 (d = 256)
  __shared__ float s_q[D], s_p[D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = a.n_q_heads / a.n_kv_heads, G = g * a.n_q;
  const int t = qq / g, hh = qq % g;
  const size_t row = ((size_t)b * a.n_q + t) * a.n_q_heads + kvh * g + hh;
  const int srow = wave * RPW + lane / LPR, part = lane % LPR;
  const float4 *S4 = reinterpret_cast<const float4 *>(a.qjl);
  const size_t s_off = (size_t)srow * (D / 4) + part * (EPL / 4);   // this lane's part of its S row
  const bool qjl = a.qjl != nullptr;   // MSE-only keys: p = 0, S is not read
  float4 sv[CH];
  if (qjl) {
#pragma unroll
    for (int k = 0; k < CH; ++k) sv[k] = S4[s_off + k];
  }

  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = load_elem<DT>(a.q, row * D + lane + 64 * r);
  fwht_wave<R>(v);
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] *= rsqrt_dim<D>();
  float *dst = a.prep + row * 2 * D;
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s_q[lane + 64 * r] = v[r];
      dst[lane + 64 * r] = v[r];
    }
  }
  __syncthreads();

  // p_l = sum_i S[l][i] q~_i
  const float4 *q4 = reinterpret_cast<const float4 *>(s_q) + part * (EPL / 4);
  float acc = 0.f;
  if (qjl) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c > 0) {
#pragma unroll
        for (int k = 0; k < CH; ++k) sv[k] = S4[s_off + c * CH + k];
      }
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const float4 qv = q4[c * CH + k];
        acc = fmaf(sv[k].x, qv.x, acc);
        acc = fmaf(sv[k].y, qv.y, acc);
        acc = fmaf(sv[k].z, qv.z, acc);
        acc = fmaf(sv[k].w, qv.w, acc);
      }
    }
  }
  if (LPR == 2) acc += __shfl_xor(acc, 1, 64);
  if (part == 0) {
    s_p[srow] = acc;
    dst[D + srow] = acc;
  }
  if (a.packed == nullptr) return;
  __syncthreads();

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
  // query group rho = qq / 4 has its own operand; this row is its row group qloc
  const int QG = query_groups(G), rho = qq / kMfmaMaxGroup, qloc = qq % kMfmaMaxGroup;
  const int Gr = min(kMfmaMaxGroup, G - kMfmaMaxGroup * rho);   // rows of the group
  uint8_t *grp = a.packed + (((size_t)b * a.n_kv_heads + kvh) * QG + rho) * packed_group_bytes(D, KB);
  uint8_t *opb = grp;                                                  // [mu][lane][32] bytes
  uint32_t *scl = reinterpret_cast<uint32_t *>(grp + (size_t)NMU * 2048);   // [mu][lane]
  const float kap2 = 2.f * qjl_kappa<D>();
  // Half-wave h takes the (mu, block) tasks h, h + 8, ...: all of them in one
  // pass, so their limb chains interleave. Fields are ORed into LDS dwords
  // (field f of a lane's 32 sits at bits 6 f .. 6 f + 5 of its 192), then each
  // packed dword is stored once.
  constexpr int NTASK = NMU * 4, NT = (NTASK + 7) / 8;
  __shared__ uint32_t s_pk[8][NT][4][6];                      // per half-wave: task, limb, dword
  const int half = threadIdx.x >> 5, e = threadIdx.x & 31;
  for (int z = e; z < NT * 4 * 6; z += 32) (&s_pk[half][0][0][0])[z] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int fv = e >> 3, fm = e & 7;   // field e: bit 4 fm + fv of its plane word
  const float val = fv == 0 ? 0.5f : fv == 1 ? 1.f : 2.f;
  const int sh0 = (6 * e) & 31, dw0 = (6 * e) >> 5;   // where field e starts
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int blkid = half + 8 * t;   // the same for both halves of a wave
    if (blkid < NTASK) {
      const int mu = blkid >> 2, kb = blkid & 3;
      const int c = mu / (NPK + 1), pl = mu % (NPK + 1);
      const int i = 32 * (kb + 4 * c) + 4 * fm + fv;
      float r = (pl < NPK ? w[pl] * s_q[i] : kap2 * s_p[i]) / val;
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
        atomicOr(&s_pk[half][t][limb][dw0], code << sh0);
        if (sh0 > 26) atomicOr(&s_pk[half][t][limb][dw0 + 1], code >> (32 - sh0));
        if (e == 0) scl[mu * 64 + 16 * kb + 4 * qloc + limb] = (uint32_t)(ex + 127);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // lane e < 24 stores dword e % 6 of limb e / 6; lanes 24..31 clear dwords 6 and 7
  const int plimb = e < 24 ? e / 6 : (e - 24) >> 1;
  const int pdw = e < 24 ? e % 6 : 6 + ((e - 24) & 1);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int blkid = half + 8 * t;
    if (blkid < NTASK) {
      const int mu = blkid >> 2, kb = blkid & 3;
      const uint32_t word = e < 24 ? s_pk[half][t][plimb][pdw] : 0u;
      reinterpret_cast<uint32_t *>(opb)[((size_t)mu * 64 + 16 * kb + 4 * qloc + plimb) * 8 + pdw] = word;
    }
  }
  // limb rows of rows Gr .. 3 of the group (no query): zero fields, unit scales
  if (qloc == 0 && Gr < kMfmaMaxGroup) {
    const int nrow = 4 * (kMfmaMaxGroup - Gr);
    for (int t = threadIdx.x; t < NMU * 4 * nrow * 32; t += 256) {
      const int byte = t & 31, rest = t >> 5;
      const int row = 4 * Gr + rest % nrow, lg = (rest / nrow) & 3, mu = rest / nrow / 4;
      opb[((size_t)mu * 64 + 16 * lg + row) * 32 + byte] = 0;
      if (byte == 0) scl[mu * 64 + 16 * lg + row] = 127u;
    }
  }
  float *rc = reinterpret_cast<float *>(grp + (size_t)NMU * (2048 + 256));
  if (threadIdx.x < 4) {
    const float cv[4] = {0.f, 0.f, sq, sp};
    rc[4 * qloc + threadIdx.x] = cv[threadIdx.x];
  } else if (qloc == 0 && threadIdx.x < 4 * kMfmaMaxGroup && threadIdx.x >= 4 * Gr) {
    rc[threadIdx.x] = 0.f;
  }
}

template <int D, int DT>
__global__ __launch_bounds__(256) void prepare_kernel(PrepArgs a) {
  // the K code width is uniform over the launch
  if (a.k_bits == 2)
    prepare_row<D, DT, 2>(a, blockIdx.x, blockIdx.y, blockIdx.z);
  else if (a.k_bits == 4)
    prepare_row<D, DT, 4>(a, blockIdx.x, blockIdx.y, blockIdx.z);
  else
    prepare_row<D, DT, 3>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// One launch for the work of a decode step that precedes the split-K decode:
// workgroups [0, nk) encode the appended K vectors (one per wave), the next nv
// encode the appended V vectors (one token per wave and KV head) and the rest
// prepare one query row each. The three parts touch disjoint memory.
struct StepArgs {
  EncodeArgs k, v;
  PrepArgs p;
  int nk, nvx, nv;   // K workgroups; V workgroups per KV head and in total
};

template <int D, int DT>
__global__ __launch_bounds__(256) void step_prologue_kernel(StepArgs s) {
  int id = blockIdx.x;
  if (id < s.nk) {
    // the K code width is uniform over the launch
    if (s.k.bits == 2)
      encode_k_block<D, DT, 1, 2>(s.k, id);
    else if (s.k.bits == 4)
      encode_k_block<D, DT, 1, 4>(s.k, id);
    else
      encode_k_block<D, DT, 1, 3>(s.k, id);
    return;
  }
  id -= s.nk;
  if (id < s.nv) {
    // the V code width is uniform over the launch
    if (s.v.bits == 2)
      encode_v_block<D, DT, 1, 2>(s.v, id % s.nvx, id / s.nvx);
    else if (s.v.bits == 4)
      encode_v_block<D, DT, 1, 4>(s.v, id % s.nvx, id / s.nvx);
    else
      encode_v_block<D, DT, 1, 3>(s.v, id % s.nvx, id / s.nvx);
    return;
  }
  id -= s.nv;
  const int G = s.p.n_q * (s.p.n_q_heads / s.p.n_kv_heads);
  const int qq = id % G, kvh = (id / G) % s.p.n_kv_heads, b = id / (G * s.p.n_kv_heads);
  if (s.p.k_bits == 2)
    prepare_row<D, DT, 2>(s.p, qq, kvh, b);
  else if (s.p.k_bits == 4)
    prepare_row<D, DT, 4>(s.p, qq, kvh, b);
  else
    prepare_row<D, DT, 3>(s.p, qq, kvh, b);
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

// Bulk calls use 16 vectors per wave; short appends (below 4096 vectors) one,
// so that the work spreads over more workgroups.
hipError_t launch_encode_k(const EncodeArgs &a, int d, hipStream_t s) {
  const long total = (long)a.n_tokens * a.n_heads;
  return by_dim_dtype(d, a.dtype, [&](auto D, auto DT) {
    auto go = [&](auto KB) {
      if (total < 4096) {
        const dim3 grid((unsigned)((total + kWaves - 1) / kWaves));
        hipLaunchKernelGGL((encode_k_kernel<D.value, DT.value, 1, KB.value>), grid, dim3(256), 0, s, a);
      } else {
        const dim3 grid((unsigned)((total + 63) / 64));
        hipLaunchKernelGGL((encode_k_kernel<D.value, DT.value, 16, KB.value>), grid, dim3(256), 0, s, a);
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
        hipLaunchKernelGGL((encode_v_kernel<D.value, DT.value, 16, VBITS.value>), grid, dim3(256), 0, s, a);
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

hipError_t launch_prepare(const PrepArgs &a, int d, hipStream_t s) {
  const dim3 grid(a.n_q * (a.n_q_heads / a.n_kv_heads), a.n_kv_heads, a.batch);
  if (d == 128) {
    if (a.dtype == TQ_F32)
      hipLaunchKernelGGL((prepare_kernel<128, TQ_F32>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prepare_kernel<128, TQ_BF16>), grid, dim3(256), 0, s, a);
  } else {
    if (a.dtype == TQ_F32)
      hipLaunchKernelGGL((prepare_kernel<256, TQ_F32>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prepare_kernel<256, TQ_BF16>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool step_prologue_fits(const EncodeArgs &k, const PrepArgs &p) {
  return (long)k.n_tokens * k.n_heads < 4096 && k.dtype == p.dtype;
}

hipError_t launch_step_prologue(const EncodeArgs &k, const EncodeArgs &v, const PrepArgs &p, int d,
                                hipStream_t s) {
  StepArgs sa;
  sa.k = k;
  sa.v = v;
  sa.p = p;
  sa.nk = (int)(((long)k.n_tokens * k.n_heads + kWaves - 1) / kWaves);
  sa.nvx = (v.n_tokens + kWaves - 1) / kWaves;
  sa.nv = sa.nvx * v.n_heads;
  const long np = (long)p.n_q * p.n_q_heads * p.batch;   // query rows
  const dim3 grid((unsigned)(sa.nk + sa.nv + np));
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
