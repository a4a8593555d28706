// Split-K decode attention over the packed TurboQuant cache.
//
// Method: AI Heartland news "Apple Silicon向けSwiftLM、TurboQuant KVキャッシュ圧縮と
// SSD Expert Streamingを実装", section 技術的な詳細: "K-Cache圧縮" (QJL signs keep the
// inner-product score accurate), "V-Cache圧縮" (V is only accumulated), and
// "TurboQuant KVキャッシュ圧縮アーキテクチャ" item 2 (dequantisation fused into the
// attention kernel: no dequantised K/V ever reaches memory).
//
// Grid (split, kv_head, sequence); a workgroup streams whole 256-token pages of
// one (sequence, KV head), scores every token against all query rows of that KV
// head (Hq/Hkv heads x n_q tokens) in the rotated domain, keeps an online softmax
// and accumulates V in the rotated domain. The last workgroup of a (sequence, KV
// head) to finish merges the split partials by log-sum-exp, applies the single
// inverse rotation and writes float32 outputs.
#include "tq_device.h"

namespace tq {
namespace {

template <int D, int GT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int R = D / 64;
  constexpr int KREC = D / 2;
  constexpr size_t KCODES = (size_t)kPage * KREC;
  constexpr size_t KSEC = KCODES + 4 * kPage;
  constexpr size_t VCODES = (size_t)3 * D * kPage / 8;
  constexpr size_t VSEC = VCODES + 2 * kPage;
  constexpr int NS = 256 / D;               // query sets in the V phase
  constexpr int QPS = (GT + NS - 1) / NS;   // query rows per thread in the V phase

  __shared__ float s_qt[D][GT];             // rotated queries, [coordinate][row]
  __shared__ float s_pp[D][GT];             // S * rotated queries
  __shared__ float s_w[kPage][GT];          // scores, then softmax numerators
  __shared__ float s_nv[kPage];
  __shared__ float s_m[GT], s_l[GT], s_alpha[GT];
  __shared__ int s_last;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.n_kv_heads, Hq = a.n_q_heads, g = Hq / H, G = a.plan.group;
  const int nsplit = a.plan.n_split;
  const int L = a.seq_lens[b];

  for (int e = tid; e < GT * D; e += 256) {
    const int qq = e / D, i = e % D;
    float qv = 0.f, pv = 0.f;
    if (qq < G) {
      const int t = qq / g, hh = qq % g;
      const size_t row = ((size_t)b * a.n_q + t) * Hq + kvh * g + hh;
      qv = a.prep[row * 2 * D + i];
      pv = a.prep[row * 2 * D + D + i];
    }
    s_qt[i][qq] = qv;
    s_pp[i][qq] = pv;
  }
  if (tid < GT) {
    s_m[tid] = kNegInf;
    s_l[tid] = 0.f;
  }
  int vis[GT];
#pragma unroll
  for (int qq = 0; qq < GT; ++qq) {
    const int t = qq / g;
    vis[qq] = qq < G ? (a.causal_tail ? L - (a.n_q - 1 - t) : L) : 0;
  }
  const float kappa = qjl_kappa<D>();
  float acc[QPS];
#pragma unroll
  for (int k = 0; k < QPS; ++k) acc[k] = 0.f;

  // pages beyond the block table's width are never read
  const int n_pages_seq = min((L + kPage - 1) / kPage, a.max_pages);
  const int pg0 = split * a.plan.pages_per_split;
  const int pg1 = min(pg0 + a.plan.pages_per_split, n_pages_seq);
  __syncthreads();

  for (int pg = pg0; pg < pg1; ++pg) {
    const int phys = a.block_table[(size_t)b * a.max_pages + pg];
    const uint8_t *ksec = a.k_pool + ((size_t)phys * H + kvh) * KSEC;
    const uint8_t *vsec = a.v_pool + ((size_t)phys * H + kvh) * VSEC;
    const int tok0 = pg * kPage;
    const int ntok = min(kPage, L - tok0);

    // ---- scores: one thread per token of the page
    {
      const int t = tid;
      float s1[GT], s2[GT];
#pragma unroll
      for (int qq = 0; qq < GT; ++qq) s1[qq] = s2[qq] = 0.f;
      if (t < ntok) {
        const uint4 *rec = reinterpret_cast<const uint4 *>(ksec + (size_t)t * KREC);
        for (int s = 0; s < D / 32; ++s) {
          const uint4 w = rec[s];
#pragma unroll 8
          for (int e = 0; e < 32; ++e) {
            const int i = 32 * s + e;
            const int idx = ((w.x >> e) & 1) | (((w.y >> e) & 1) << 1) | (((w.z >> e) & 1) << 2);
            const float cv = level_of(a.cb, idx);
            const float sg = ((w.w >> e) & 1) ? 1.f : -1.f;
#pragma unroll
            for (int qq = 0; qq < GT; ++qq) {
              s1[qq] = fmaf(s_qt[i][qq], cv, s1[qq]);
              s2[qq] = fmaf(s_pp[i][qq], sg, s2[qq]);
            }
          }
        }
        const float N = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(ksec + KCODES)[t]);
        const float Gm = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(ksec + KCODES + 2 * kPage)[t]);
#pragma unroll
        for (int qq = 0; qq < GT; ++qq) {
          const float sc = a.scale * N * fmaf(kappa * Gm, s2[qq], s1[qq]);
          s_w[t][qq] = (tok0 + t < vis[qq]) ? sc : kNegInf;
        }
        s_nv[t] = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(vsec + VCODES)[t]);
      } else {
#pragma unroll
        for (int qq = 0; qq < GT; ++qq) s_w[t][qq] = kNegInf;
        s_nv[t] = 0.f;
      }
    }
    __syncthreads();

    // ---- online softmax update: wave w owns rows w, w+4, ...
    for (int qq = wave; qq < GT; qq += 4) {
      float mx = kNegInf;
#pragma unroll
      for (int k = 0; k < kPage / 64; ++k) mx = fmaxf(mx, s_w[lane + 64 * k][qq]);
      mx = wave_max(mx);
      const float m_old = s_m[qq];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < kPage / 64; ++k) {
        const int t = lane + 64 * k;
        const float e = m_new == kNegInf ? 0.f : __expf(s_w[t][qq] - m_new);
        s_w[t][qq] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        const float alpha = m_old == kNegInf ? 0.f : __expf(m_old - m_new);
        s_alpha[qq] = alpha;
        s_l[qq] = s_l[qq] * alpha + sum;
        s_m[qq] = m_new;
      }
    }
    __syncthreads();

    // ---- V accumulation: thread (coordinate i, query set) walks the page's tokens
    {
      const int i = tid % D, set = tid / D;
#pragma unroll
      for (int k = 0; k < QPS; ++k) {
        const int qq = set + NS * k;
        if (qq < GT) acc[k] *= s_alpha[qq];
      }
      const uint4 *r0 = reinterpret_cast<const uint4 *>(vsec + (size_t)(0 * D + i) * (kPage / 8));
      const uint4 *r1 = reinterpret_cast<const uint4 *>(vsec + (size_t)(1 * D + i) * (kPage / 8));
      const uint4 *r2 = reinterpret_cast<const uint4 *>(vsec + (size_t)(2 * D + i) * (kPage / 8));
      const uint4 p0[2] = {r0[0], r0[1]}, p1[2] = {r1[0], r1[1]}, p2[2] = {r2[0], r2[1]};
#pragma unroll
      for (int wi = 0; wi < kPage / 32; ++wi) {
        const int tb = wi * 32;
        if (tb >= ntok) break;
        const uint4 &q0 = p0[wi >> 2], &q1 = p1[wi >> 2], &q2 = p2[wi >> 2];
        const int c = wi & 3;
        const uint32_t w0 = c == 0 ? q0.x : c == 1 ? q0.y : c == 2 ? q0.z : q0.w;
        const uint32_t w1 = c == 0 ? q1.x : c == 1 ? q1.y : c == 2 ? q1.z : q1.w;
        const uint32_t w2 = c == 0 ? q2.x : c == 1 ? q2.y : c == 2 ? q2.z : q2.w;
#pragma unroll 4
        for (int e = 0; e < 32; ++e) {
          const int t = tb + e;
          const int idx = ((w0 >> e) & 1) | (((w1 >> e) & 1) << 1) | (((w2 >> e) & 1) << 2);
          const float val = s_nv[t] * level_of(a.cb, idx);
#pragma unroll
          for (int k = 0; k < QPS; ++k) {
            const int qq = set + NS * k;
            if (qq < GT) acc[k] = fmaf(s_w[t][qq], val, acc[k]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- partials: [B*Hkv][n_split][GT... group rows] x (m, l, acc[D])
  const size_t pbase = (((size_t)b * H + kvh) * nsplit + split) * G;
  {
    const int i = tid % D, set = tid / D;
#pragma unroll
    for (int k = 0; k < QPS; ++k) {
      const int qq = set + NS * k;
      if (qq < G) a.partials[(pbase + qq) * (D + 2) + 2 + i] = acc[k];
    }
    if (tid < G) {
      a.partials[(pbase + tid) * (D + 2) + 0] = s_m[tid];
      a.partials[(pbase + tid) * (D + 2) + 1] = s_l[tid];
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&a.counters[b * H + kvh], 1u);
    s_last = prev == (uint32_t)(nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- merge (last workgroup): one wave per query row
  const size_t mbase = ((size_t)b * H + kvh) * nsplit * G;
  for (int qq = wave; qq < G; qq += 4) {
    float M = kNegInf;
    for (int sp = lane; sp < nsplit; sp += 64) {
      const float *pr = a.partials + (mbase + (size_t)sp * G + qq) * (D + 2);
      if (pr[1] > 0.f) M = fmaxf(M, pr[0]);
    }
    M = wave_max(M);
    float x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = 0.f;
    float lsum = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float *pr = a.partials + (mbase + (size_t)sp * G + qq) * (D + 2);
      const float l = pr[1];
      if (l > 0.f) {
        const float f = __expf(pr[0] - M);
        lsum += l * f;
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = fmaf(f, pr[2 + lane + 64 * r], x[r]);
      }
    }
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] *= inv;
    fwht_wave<R>(x);
    const int t = qq / g, hh = qq % g;
    float *o = a.out + (((size_t)b * a.n_q + t) * Hq + kvh * g + hh) * D;
#pragma unroll
    for (int r = 0; r < R; ++r) o[lane + 64 * r] = x[r] * rsqrt_dim<D>();
  }
  if (tid == 0) a.counters[b * H + kvh] = 0u;
}

template <int D>
hipError_t launch_dim(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid(a.plan.n_split, a.n_kv_heads, a.batch);
  const int G = a.plan.group;
  if (G <= 1)
    hipLaunchKernelGGL((decode_kernel<D, 1>), grid, dim3(256), 0, s, a);
  else if (G <= 2)
    hipLaunchKernelGGL((decode_kernel<D, 2>), grid, dim3(256), 0, s, a);
  else if (G <= 4)
    hipLaunchKernelGGL((decode_kernel<D, 4>), grid, dim3(256), 0, s, a);
  else if (G <= 8)
    hipLaunchKernelGGL((decode_kernel<D, 8>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, 16>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t s) {
  return d == 128 ? launch_dim<128>(a, s) : launch_dim<256>(a, s);
}

}  // namespace tq
