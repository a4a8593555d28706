// Uncompressed bf16 decode attention: the baseline the compressed path is
// measured against on the long-context workload. Same split-K grid and the same
// partial format as the compressed kernel (merged by the same merge kernel,
// without the inverse rotation): softmax(q K^T * scale) V over dense bf16 K and
// V laid out [batch][Hkv][max_len][d], so each (sequence, KV head) streams
// one contiguous run, as each (page, KV head) section of the compressed cache does.
//
// Each wave owns 64-token blocks of its workgroup's token range. Scores: lane =
// token, its K row read as 16-byte chunks (the next loads of the same lane use
// the rest of each cache line), q from LDS as broadcasts. V: lane (s, c) takes
// tokens 16 s .. 16 s + 15 of the block and coordinates 8 c .. 8 c + 7 (16 at
// d = 256), so 16 lanes read one V row as a contiguous run; the four token
// subsets are summed once at the end. At d = 128 the loads are pipelined: a
// block's V rows are requested before its scores are computed, and the next
// block's K rows before this block's V is accumulated.
#include "tq_device.h"

namespace tq {
namespace {

constexpr float kFltMaxD = 3.402823466e38f;
constexpr int kPartHeadD = 4;   // m, l, m, pad, then acc[d] (the merge's record)

__device__ inline void bf16x8_to_f32(const uint4 &u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <int D, int DT, int NQ>
__global__ __launch_bounds__(256) void dense_decode_kernel(DenseArgs a) {
  constexpr int CPL = D / 16;          // coordinates per lane (V) and per K chunk run
  constexpr int KCH = D / 128;         // 16-byte K chunks per lane and token
  __shared__ float4 s_q[NQ][D / 4];
  __shared__ float s_p[4][NQ][64];
  __shared__ float s_st[4][2][NQ];
  __shared__ float s_acc[4][NQ][D];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.n_kv_heads, g = a.n_q_heads / H, G = g * a.n_q;
  const int L = min(a.seq_lens[b], a.max_len);
  const int t0 = split * a.tokens_per_split;
  const int t1 = min(L, t0 + a.tokens_per_split);
  const float scale2 = a.scale * 1.4426950408889634f;   // log2 units

  for (int e = tid; e < NQ * D; e += 256) {
    const int qq = e / D, i = e % D;
    float v = 0.f;
    if (qq < G) {
      const size_t row = ((size_t)b * a.n_q + qq / g) * a.n_q_heads + kvh * g + qq % g;
      v = load_elem<DT>(a.q, row * D + i) * scale2;
    }
    reinterpret_cast<float *>(s_q[qq])[i] = v;
  }
  __syncthreads();

  float m[NQ], l[NQ], acc[NQ][CPL];
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    m[qq] = -kFltMaxD;
    l[qq] = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[qq][e] = 0.f;
  }
  const int ts = lane >> 4, dc = lane & 15;
  const size_t tok_stride = D;   // bf16 elements between tokens
  const uint16_t *kbase = a.k + ((size_t)b * H + kvh) * a.max_len * D;
  const uint16_t *vbase = a.v + ((size_t)b * H + kvh) * a.max_len * D;
  constexpr bool kPipe = D == 128;
  constexpr int VPL = CPL / 8;                     // 16-byte V chunks per lane and token
  uint4 kb[D / 8], vb[kPipe ? 16 * VPL : 1];

  auto load_k = [&](int blk) {
    const int t = blk + lane;
    if (t < t1) {
      const uint4 *kr = reinterpret_cast<const uint4 *>(kbase + (size_t)t * tok_stride);
#pragma unroll
      for (int c = 0; c < D / 8; ++c) kb[c] = kr[c];
    }
  };
  auto v_row = [&](int blk, int j) {
    return reinterpret_cast<const uint4 *>(vbase + (size_t)(blk + 16 * ts + j) * tok_stride) + dc * VPL;
  };

  int blk = t0 + 64 * wave;
  if (blk < t1) load_k(blk);
  for (; blk < t1; blk += 256) {
    if constexpr (kPipe) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (blk + 16 * ts + j < t1) vb[j] = v_row(blk, j)[0];
    }
    // ---- scores, lane = token
    const int t = blk + lane;
    const bool live = t < t1;
    float s[NQ];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) s[qq] = 0.f;
    if (live) {
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        float k8[8];
        bf16x8_to_f32(kb[c], k8);
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
          const float4 q0 = s_q[qq][2 * c], q1 = s_q[qq][2 * c + 1];
          s[qq] = fmaf(k8[0], q0.x, s[qq]);
          s[qq] = fmaf(k8[1], q0.y, s[qq]);
          s[qq] = fmaf(k8[2], q0.z, s[qq]);
          s[qq] = fmaf(k8[3], q0.w, s[qq]);
          s[qq] = fmaf(k8[4], q1.x, s[qq]);
          s[qq] = fmaf(k8[5], q1.y, s[qq]);
          s[qq] = fmaf(k8[6], q1.z, s[qq]);
          s[qq] = fmaf(k8[7], q1.w, s[qq]);
        }
      }
    }
    // ---- online softmax per row over the block's 64 tokens
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const float sq = (live && qq < G) ? s[qq] : kNegInf;
      const float m_new = fmaxf(m[qq], wave_max(sq));
      const float alpha = __builtin_amdgcn_exp2f(m[qq] - m_new);
      const float p = __builtin_amdgcn_exp2f(sq - m_new);
      l[qq] = l[qq] * alpha + wave_sum(p);
      m[qq] = m_new;
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[qq][e] *= alpha;
      s_p[wave][qq][lane] = p;
    }
    if constexpr (kPipe) {
      if (blk + 256 < t1) load_k(blk + 256);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- V, lane (ts, dc): tokens 16 ts + j, coordinates CPL * dc ..
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int tt = 16 * ts + j;
      if (blk + tt >= t1) break;
#pragma unroll
      for (int h = 0; h < VPL; ++h) {
        float v8[8];
        if constexpr (kPipe)
          bf16x8_to_f32(vb[j], v8);
        else
          bf16x8_to_f32(v_row(blk, j)[h], v8);
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
          const float p = s_p[wave][qq][tt];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[qq][8 * h + e] = fmaf(p, v8[e], acc[qq][8 * h + e]);
        }
      }
    }
    if constexpr (!kPipe) {
      if (blk + 256 < t1) load_k(blk + 256);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  // the four token subsets of a coordinate chunk: lanes dc, dc + 16, dc + 32, dc + 48
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      acc[qq][e] += xor_lane<16>(acc[qq][e]);
      acc[qq][e] += xor_lane<32>(acc[qq][e]);
    }
  if (lane < 16) {
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
      for (int e = 0; e < CPL; ++e) s_acc[wave][qq][CPL * dc + e] = acc[qq][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      s_st[wave][0][qq] = m[qq];
      s_st[wave][1][qq] = l[qq];
    }
  }
  __syncthreads();
  // ---- combine the four waves: one partial per query row
  const size_t pbase = (((size_t)b * H + kvh) * a.n_split + split) * G;
  for (int qq = wave; qq < G; qq += 4) {
    float M = -kFltMaxD;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (s_st[w][1][qq] > 0.f) M = fmaxf(M, s_st[w][0][qq]);
    float lsum = 0.f, fw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      fw[w] = s_st[w][1][qq] > 0.f ? __builtin_amdgcn_exp2f(s_st[w][0][qq] - M) : 0.f;
      lsum += fw[w] * s_st[w][1][qq];
    }
    float *pr = a.partials + (pbase + qq) * (D + kPartHeadD);
    if (lane == 0) {
      pr[0] = M;
      pr[1] = lsum;
      pr[2] = M;   // the V numerator shares the score reference
      pr[3] = 0.f;
    }
    for (int i = lane; i < D; i += 64) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) x = fmaf(fw[w], s_acc[w][qq][i], x);
      pr[kPartHeadD + i] = x;
    }
  }
}

}  // namespace

template <int D, int DT>
hipError_t launch_dense_nq(const DenseArgs &a, int G, hipStream_t s) {
  const dim3 grid(a.n_split, a.n_kv_heads, a.batch);
  if (G <= 1)
    hipLaunchKernelGGL((dense_decode_kernel<D, DT, 1>), grid, dim3(256), 0, s, a);
  else if (G <= 2)
    hipLaunchKernelGGL((dense_decode_kernel<D, DT, 2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dense_decode_kernel<D, DT, 4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_split(const DenseArgs &a, int d, hipStream_t s) {
  const int G = a.n_q_heads / a.n_kv_heads * a.n_q;
  if (d == 128)
    return a.q_dtype == TQ_F32 ? launch_dense_nq<128, TQ_F32>(a, G, s) : launch_dense_nq<128, TQ_BF16>(a, G, s);
  return a.q_dtype == TQ_F32 ? launch_dense_nq<256, TQ_F32>(a, G, s) : launch_dense_nq<256, TQ_BF16>(a, G, s);
}

}  // namespace tq
