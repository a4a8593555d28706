// Query preparation and split-K decode attention over the packed TurboQuant cache.
//
// Method: AI Heartland news "Apple Silicon向けSwiftLM、TurboQuant KVキャッシュ圧縮と
// SSD Expert Streamingを実装", section 技術的な詳細: "K-Cache圧縮" (QJL signs keep the
// inner-product score accurate), "V-Cache圧縮" (V is only accumulated) and
// "TurboQuant KVキャッシュ圧縮アーキテクチャ" item 2 (dequantisation fused into the
// attention kernel: no dequantised K/V ever reaches memory). The query is rotated
// and projected once per step; scores and the V sum live in the rotated domain
// and one inverse rotation is applied per output row.
//
// Grid (split, KV head, sequence x query-group workgroup). A workgroup streams
// whole 256-token pages of one (sequence, KV head) for the query rows of one or
// two query groups (4 rows each), keeps an online softmax, and writes (max, sum,
// V numerator) partials; a second, small kernel merges the partials of each
// query row by log-sum-exp and writes float32 rows. (Merging in the
// last-arriving workgroup would need a device-scope release per workgroup, which
// on this GPU writes back and invalidates the whole L2 of the XCD every time.)
//
// Scores are a block-scaled fp6 x fp4 MFMA contraction. The codebook is odd
// (c[7-k] = -c[k]), so the 3-bit code splits over four binary planes,
// c[idx] = 2 (a0 b0 + a1 b1 + a2 b2 + a3 (b0^b1^b2)) - c7, and each key bit plane
// becomes an fp4 operand (one AND per eight coordinates, the bit's position
// folded into the fp4 value); the query side is four fp6 (e2m3) limbs with a
// power-of-two scale per 32 coordinates on the MFMA rows (4 query rows x 4 limbs
// per query group), exact to under 2^-18 of the largest term of each block. V is
// accumulated with the same planes on int8 MFMA: the softmax weight times each
// plane weight, as four int8 limbs, against the V bit planes; every product there
// is exact in int32. V codes may also have 2 or 4 bits (a bit-width variant):
// their planes are the odd Walsh functions of the code bits (b0, b1; or the four
// bits and their four 3-bit parities), taken one plane at a time.
#include "tq_device.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kFltMax = 3.402823466e38f;
// Headroom of a running softmax reference (log2 units): weights relative to it
// stay below 2^0.8 = 1.74, so weight * 2^30 plus the limb offset 0x80808080
// stays inside 32 bits.
constexpr float kSlack = 0.8f;
constexpr int kPartHead = 4;   // partial record: m, l, mU (log2 units), pad, then acc[d]


// ------------------------------------------------------------------ MFMA kernel
__device__ inline int dpp_swap1(int x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true); }
__device__ inline int dpp_swap2(int x) { return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); }
template <int CTRL>
__device__ inline float dppf(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Reductions over the 16 lanes of one DPP row (one query row of the score
// layout): row mirror (i <-> 15 - i), half-row mirror (i <-> 7 - i), then the
// quad swaps i ^ 2 and i ^ 1 leave every lane with all 16 values combined.
__device__ inline float rowmax16(float x) {
  x = fmaxf(x, dppf<0x140>(x));
  x = fmaxf(x, dppf<0x141>(x));
  x = fmaxf(x, dppf<0x4E>(x));
  return fmaxf(x, dppf<0xB1>(x));
}
__device__ inline float rowsum16(float x) {
  x += dppf<0x140>(x);
  x += dppf<0x141>(x);
  x += dppf<0x4E>(x);
  return x + dppf<0xB1>(x);
}

// 4x4 byte transpose inside a quad: lane L holds the four bytes of token L; on
// return lane L holds byte L of tokens 0..3.
__device__ inline uint32_t quad_byte_transpose(uint32_t d, int lam) {
  const uint32_t p1 = (uint32_t)dpp_swap1((int)d);
  const uint32_t e = __builtin_amdgcn_perm(p1, d, (lam & 1) ? 0x03070105u : 0x06020400u);
  const uint32_t p2 = (uint32_t)dpp_swap2((int)e);
  return __builtin_amdgcn_perm(p2, e, (lam & 2) ? 0x03020706u : 0x05040100u);
}

// Each wave owns 64-token blocks (block w of every page of the split) from the
// loads to the V accumulation, with its own online softmax; the four waves of
// the workgroup combine once at the end into one partial per query row.
//
// Scores: scaled MFMA with the query limbs as A (16 rows = 4 query rows x 4
// limbs, fp6) and the key bit planes as B (16 token columns x 128 coordinates,
// fp4). Lane (n, kg) receives rows 4 kg .. 4 kg + 3 of column n: the four limbs
// of query row kg for token 16 tau + n, summed in the lane, so each score, its
// sidecars and its softmax step live in exactly one lane, and the 16 lanes of a
// DPP row hold one query row. The softmax weights then move to the V operand
// layout with one ds_bpermute per 16-token tile.
// V: int8 MFMA with the softmax weight (times each plane weight) as 4 int8 limbs
// on the 16 rows and the V bit planes on the columns: lane (n, k) reads its 16
// tokens x 2 coordinates per u32 word, and a shift plus one AND per 4 tokens
// makes the B operand. The int32 sums are folded into a float accumulator
// after every block, or (one query group at d = 256) only when the softmax
// reference moves, and once at the end. (Folding only at a rescale also fits at
// d = 128 but measured slower there.)
//
// Up to TQ_MAX_GROUP query rows per KV head (a few for decode and verify, a
// whole chunk's for chunked prefill) run as query groups of 4 rows (4 rows x 4
// limbs fill the 16 MFMA rows). At d = 128 two groups share a workgroup; the
// workgroups of one split sit in blockIdx.z, n_split * Hkv apart, so with
// n_split * Hkv a multiple of 8 they land on the same XCD and share its L2.
// With a causal tail a workgroup stops at the last token its rows can see.
//
// With TWO_SETS (d = 128, one group, more than two pages per split),
// everything one block needs (key records, sidecars, V words) is loaded one
// block ahead; two register sets alternate between even and odd pages so that
// no copy is needed. Otherwise the block's loads are issued at its start: at
// d = 256 to keep two waves per SIMD, and at d = 128 with two pages or fewer
// per split, where a wave sees at most two blocks and the one-set kernel
// (about 115 VGPRs against 180) finishes sooner.

// Copies the packed scoring operand of a query group (NMU x 64 lanes x 32 bytes,
// then NMU x 64 scale words) into LDS.
template <int NMU>
__device__ inline void stage_query(const uint8_t *grp, v8i *s_qop, int *s_qsc, int tid) {
  const uint4 *src = reinterpret_cast<const uint4 *>(grp);
  uint4 *dst = reinterpret_cast<uint4 *>(s_qop);
  for (int e = tid; e < NMU * 128; e += 256) dst[e] = src[e];
  const int *ssrc = reinterpret_cast<const int *>(grp + (size_t)NMU * 2048);
  for (int e = tid; e < NMU * 64; e += 256) s_qsc[e] = ssrc[e];
}

template <int D, int VBITS, int KBITS>
struct MfmaBlock {
  static constexpr bool kPrefetchV = D == 128;
  // key record words (KBITS code planes, then the signs) of coordinate groups
  // kg + 4 c of tokens 16 tau + n
  uint32_t kw[4][D / 128][KBITS + 1];
  uint2 g, nk, nv;                 // G, N^K, N^V of side entries 4 n + tau (tokens 16 tau + n)
  uint4 v[kPrefetchV ? VBITS : 1][D / 128];   // V words of plane j: coordinate pairs kp
};

// NG query groups (4 rows each) share a workgroup: the key and V operands of a
// block are built once and each MFMA operand of the keys or V bits meets the NG
// query operands in turn. NG = 1 gives each group its own workgroup.
template <int D, int NG, int VBITS, int KBITS, bool TWO_SETS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NG == 1 ? 2 : 1))) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(!TWO_SETS || (D == 128 && NG == 1), "two register sets only at d = 128 with one group");
  constexpr int NPK = k_planes(KBITS);      // key code planes (then the sign plane)
  constexpr int NMU = mfma_per_tile(D, KBITS);   // scaled MFMAs per 16-token scoring tile
  constexpr int NCH = D / 128;              // 128-coordinate chunks per token
  constexpr int KREC = (KBITS + 1) * D / 8; // K record bytes
  constexpr size_t KCODES = (size_t)kPage * KREC;
  constexpr size_t KSEC = KCODES + 4 * kPage;
  constexpr size_t VCODES = (size_t)VBITS * D * kPage / 8;   // VBITS-bit V codes
  constexpr size_t VSEC = VCODES + 2 * kPage;
  constexpr int NP = VPlanes<VBITS>::n;     // V bit planes (odd Walsh functions of the code bits)
  constexpr int NB = D / 16;                // 16-coordinate V column blocks
  constexpr int NR = NG * kMfmaMaxGroup;    // query rows of the workgroup

  // the query operands live in LDS during the page loop; the same bytes then
  // hold the per-wave V numerators for the final combine
  constexpr size_t QOP_BYTES = (size_t)NG * NMU * 64 * 32, QSC_BYTES = (size_t)NG * NMU * 64 * 4;
  constexpr size_t WACC_BYTES = (size_t)4 * NR * D * 4;
  constexpr size_t RAW = QOP_BYTES + QSC_BYTES > WACC_BYTES ? QOP_BYTES + QSC_BYTES : WACC_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[RAW];
  __shared__ float s_wm[4][4][NR];                  // per wave: m, l, mU, sum U of each row
  v8i *s_qop = reinterpret_cast<v8i *>(s_raw);      // [group][mfma][lane]
  int *s_qsc = reinterpret_cast<int *>(s_raw + QOP_BYTES);
  auto s_wacc = reinterpret_cast<float (*)[NR][D]>(s_raw);   // [wave][row][d]

  const int QG = a.plan.qgroups, WZ = a.plan.wg_per_seq;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z / WZ;
  const int rho0 = (blockIdx.z % WZ) * NG;           // first query group of the workgroup
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, kg = lane >> 4;   // scores: token 16 tau + n of query row kg
  const int lam = n & 3;                     // V weight operand: limb row / token of the quad
  const int H = a.n_kv_heads, g = a.n_q_heads / H;
  const int L = a.seq_lens[b];

  const uint8_t *grp0 = a.packed + (((size_t)b * H + kvh) * QG + rho0) * packed_group_bytes(D, KBITS);
  float off1[NG], off2[NG];
  int vis[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int row = kMfmaMaxGroup * (rho0 + gi) + kg;   // query row of this lane in group gi
    off1[gi] = off2[gi] = 0.f;
    vis[gi] = 0;
    if (row < a.plan.group) {
      const float4 rc = reinterpret_cast<const float4 *>(grp0 + (size_t)gi * packed_group_bytes(D, KBITS) +
                                                         (size_t)NMU * (2048 + 256))[kg];
      off1[gi] = a.cb.levels[(1 << KBITS) - 1] * rc.z;
      off2[gi] = rc.w * qjl_kappa<D>();
      vis[gi] = a.causal_tail ? L - (a.n_q - 1 - row / g) : L;
    }
  }
  // V weight operand: lane 16 kg + 4 q + lam takes the weight of query q, token
  // 16 tau + 4 kg + lam, which the score layout holds in lane 16 q + 4 kg + lam
  const int perm_addr = 4 * (16 * (n >> 2) + 4 * kg + lam);
  const float scale2 = a.scale * 1.4426950408889634f;   // scores in log2 units
  float wpl[NP];
  if constexpr (VBITS == 3)
    plane_weights(a.vcb, wpl);
  else
    plane_weights_walsh<VBITS>(a.vcb, wpl);
  float wmax = 0.f;
#pragma unroll
  for (int j = 0; j < NP; ++j) wmax = fmaxf(wmax, fabsf(wpl[j]));
  // weight limbs: X = U * 2^-tau * (w_j / wmax) * 2^30, where 2^tau is the value
  // the V bit of token 16 tau + 4 k + r takes in byte r of the B operand
  float cx[NP], half[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    half[j] = wpl[j] < 0.f ? -0.5f : 0.5f;   // round to nearest with a truncating convert
    cx[j] = wpl[j] / wmax * 1073741824.f;
  }
  const float delta_u = wmax * 0x1p-30f;

  // running maxima start finite, so exp2 of a masked (-inf) score is 0 and no
  // per-token guard is needed; a row with no visible token keeps l = 0
  float m_run[NG], mu_run[NG], l_lane[NG], us_lane[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    m_run[gi] = mu_run[gi] = -kFltMax;
    l_lane[gi] = us_lane[gi] = 0.f;
  }
  // V sums: int32 MFMA accumulators folded into a float accumulator. With one
  // group at d = 256 they are folded only when the softmax reference moves and
  // at the end (per 64-token block a limb row gains at most NP <= 8 planes x 64
  // tokens x 128 x 8 = 2^19, so up to 2^12 blocks, far more than the 256 blocks
  // a wave sees in one split, fit in int32); otherwise they are folded after
  // every block.
  constexpr bool kLazyV = D == 256 && NG == 1;
  float facc[NG][NB];
  v4i vacc[NG][NB];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      facc[gi][k] = 0.f;
      vacc[gi][k] = v4i{0, 0, 0, 0};
    }
  // rows 4 kg + r of a V accumulator are (query kg, limb r): limb r weighs 256^r
  auto fold_one = [&](int gi, int k) {
    const float v = (float)vacc[gi][k][0] + 256.f * (float)vacc[gi][k][1] + 65536.f * (float)vacc[gi][k][2] +
                    16777216.f * (float)vacc[gi][k][3];
    facc[gi][k] = fmaf(delta_u, v, facc[gi][k]);
    vacc[gi][k] = v4i{0, 0, 0, 0};
  };
  auto fold_v = [&](int gi) {
#pragma unroll
    for (int k = 0; k < NB; ++k) fold_one(gi, k);
  };

  // Lv: one past the last token any row of the workgroup sees (with a causal
  // tail the last row sees the most); pages from Lv on are not read
  const int row_last = min(kMfmaMaxGroup * (rho0 + NG), a.plan.group) - 1;
  const int Lv = a.causal_tail ? L - (a.n_q - 1 - row_last / g) : L;
  const int n_pages_seq = min((Lv + kPage - 1) / kPage, a.max_pages);
  // tokens before S0 are not visible (a window); pages wholly before it are
  // never read, so their block-table entries may point at recycled pages
  const int S0 = a.seq_starts ? max(0, a.seq_starts[b]) : 0;
  const int pg0 = max(split * a.plan.pages_per_split, S0 / kPage);
  int pg1 = min(split * a.plan.pages_per_split + a.plan.pages_per_split, n_pages_seq);
  const int blk0 = 64 * wave;
  // pages whose block of this wave holds no visible token are skipped (only the last can)
  if (pg1 > pg0 && blk0 >= Lv - (pg1 - 1) * kPage) --pg1;

  // the query operands of the workgroup's groups (a group past the last one
  // gets zero operands; its rows are masked)
  auto stage = [&]() {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (rho0 + gi < QG) {
        stage_query<NMU>(grp0 + (size_t)gi * packed_group_bytes(D, KBITS), s_qop + gi * NMU * 64,
                         s_qsc + gi * NMU * 64, tid);
      } else {
        uint4 *dst = reinterpret_cast<uint4 *>(s_qop + gi * NMU * 64);
        for (int e = tid; e < NMU * 128; e += 256) dst[e] = make_uint4(0u, 0u, 0u, 0u);
        for (int e = tid; e < NMU * 64; e += 256) s_qsc[gi * NMU * 64 + e] = 127;
      }
    }
  };

  auto load_block = [&](MfmaBlock<D, VBITS, KBITS> &d, int pg) {
    const int phys = a.block_table[(size_t)b * a.max_pages + pg];
    const uint8_t *ks = a.k_pool + ((size_t)phys * H + kvh) * KSEC;
    const uint8_t *vs = a.v_pool + ((size_t)phys * H + kvh) * VSEC;
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint8_t *rec = ks + (size_t)(blk0 + 16 * tau + n) * KREC;
        if constexpr (KBITS == 3) {   // four words: one 16-byte load
          const uint4 u = reinterpret_cast<const uint4 *>(rec)[kg + 4 * c];
          d.kw[tau][c][0] = u.x;
          d.kw[tau][c][1] = u.y;
          d.kw[tau][c][2] = u.z;
          d.kw[tau][c][3] = u.w;
        } else {
          const uint32_t *r32 = reinterpret_cast<const uint32_t *>(rec) + (KBITS + 1) * (kg + 4 * c);
#pragma unroll
          for (int j = 0; j <= KBITS; ++j) d.kw[tau][c][j] = r32[j];
        }
      }
    const int se = blk0 + 4 * n;   // side entries of tokens 16 tau + n, tau = 0..3
    d.g = *reinterpret_cast<const uint2 *>(ks + KCODES + 2 * kPage + 2 * se);
    d.nk = *reinterpret_cast<const uint2 *>(ks + KCODES + 2 * se);
    d.nv = *reinterpret_cast<const uint2 *>(vs + VCODES + 2 * se);
    if constexpr (MfmaBlock<D, VBITS, KBITS>::kPrefetchV) {
      const uint4 *vw = reinterpret_cast<const uint4 *>(vs + (size_t)4 * (wave * 2 * VBITS * D) + 4 * (D / 32) * lane);
#pragma unroll
      for (int j = 0; j < VBITS; ++j)
#pragma unroll
        for (int c = 0; c < NCH; ++c) d.v[j][c] = vw[j * 2 * D * 4 / 16 + c];
    }
  };

  auto process = [&](const MfmaBlock<D, VBITS, KBITS> &d, int pg) {
    // at d = 256 the query operand (20 MFMA operands, 80 registers) is read from
    // LDS where it is used: an opaque lane offset keeps it from being hoisted
    int qo = lane;
    if constexpr (D == 256 || NG > 1) asm volatile("" : "+v"(qo));
    uint4 vcur[VBITS][NCH];
    if constexpr (MfmaBlock<D, VBITS, KBITS>::kPrefetchV) {
#pragma unroll
      for (int j = 0; j < VBITS; ++j)
#pragma unroll
        for (int c = 0; c < NCH; ++c) vcur[j][c] = d.v[j][c];
    } else {
      const int phys = a.block_table[(size_t)b * a.max_pages + pg];
      const uint8_t *vs = a.v_pool + ((size_t)phys * H + kvh) * VSEC;
      const uint4 *vw = reinterpret_cast<const uint4 *>(vs + (size_t)4 * (wave * 2 * VBITS * D) + 4 * (D / 32) * lane);
#pragma unroll
      for (int j = 0; j < VBITS; ++j)
#pragma unroll
        for (int c = 0; c < NCH; ++c) vcur[j][c] = vw[j * 2 * D * 4 / 16 + c];
    }
    const int tok0 = pg * kPage;
    const int ntok = min(kPage, L - tok0);
    // ---- scores: lane (n, kg) ends with query row kg of each group, token blk0 + 16 tau + n
    float sc[NG][4], sv[NG][4];
    // the four 16-token tiles' MFMAs are interleaved (consecutive MFMAs are
    // independent); the query operand of each step is shared by the four, and
    // each tile's key operand by the NG groups.
    // Key operand (B, fp4 e2m1): nibble m of dword v holds plane bit 4 m + v, as
    // 0.5, 1, 2, 2 (bit 3 shifted down one place); the query side (A, fp6)
    // carries 1 / value.
    v4f c1[NG][4], c2[NG][4];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) c1[gi][tau] = c2[gi][tau] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int j = 0; j <= NPK; ++j) {   // code planes (b0, b1, b2, b0^b1^b2 at 3 bits), then the signs
        v8i op[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const uint32_t *w = d.kw[tau][c];
          uint32_t pl;
          if constexpr (KBITS == 3) {
            pl = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : j == 3 ? (w[0] ^ w[1] ^ w[2]) : w[3];
          } else if (j == NPK) {
            pl = w[KBITS];
          } else {
            pl = 0u;
#pragma unroll
            for (int b2 = 0; b2 < KBITS; ++b2)
              if ((VPlanes<KBITS>::mask[j] >> b2) & 1) pl ^= w[b2];
          }
          op[tau] = v8i{(int)(pl & 0x11111111u), (int)(pl & 0x22222222u), (int)(pl & 0x44444444u),
                        (int)((pl >> 1) & 0x44444444u), 0, 0, 0, 0};
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const v8i qop = s_qop[(gi * NMU + (NPK + 1) * c + j) * 64 + qo];
          const int qsc = s_qsc[(gi * NMU + (NPK + 1) * c + j) * 64 + qo];
#pragma unroll
          for (int tau = 0; tau < 4; ++tau) {
            if (j < NPK)
              c1[gi][tau] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qop, op[tau], c1[gi][tau], 2, 4, 0, qsc, 0, 127);
            else
              c2[gi][tau] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qop, op[tau], c2[gi][tau], 2, 4, 0, qsc, 0, 127);
          }
        }
      }
    }
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const int sh = 16 * (tau & 1);
      const float Gt = f16_bits_to_f32((uint16_t)(((tau >> 1) ? d.g.y : d.g.x) >> sh));
      const float N = f16_bits_to_f32((uint16_t)(((tau >> 1) ? d.nk.y : d.nk.x) >> sh));
      const float lnv = __builtin_amdgcn_logf(f16_bits_to_f32((uint16_t)(((tau >> 1) ? d.nv.y : d.nv.x) >> sh)));
      const int tok = blk0 + 16 * tau + n;
      const bool in_page = tok < ntok && tok0 + tok >= S0;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        // the four limbs of (S1, S2) for query row kg, token 16 tau + n
        const float T1 = (c1[gi][tau][0] + c1[gi][tau][1]) + (c1[gi][tau][2] + c1[gi][tau][3]);
        const float T2 = (c2[gi][tau][0] + c2[gi][tau][1]) + (c2[gi][tau][2] + c2[gi][tau][3]);
        const bool valid = in_page && tok0 + tok < vis[gi];   // vis = 0 for rows past the group
        const float sco = scale2 * N * fmaf(Gt, T2 - off2[gi], T1 - off1[gi]);
        sc[gi][tau] = valid ? sco : kNegInf;
        sv[gi][tau] = valid ? sco + lnv : kNegInf;   // + log2 N^V
      }
    }

    // ---- online softmax of this wave (log2 units; scores, and scores + log2 N^V for V).
    // m_run / mu_run are references, not exact maxima: they move only when a
    // score exceeds them by more than kSlack (log2 units), so every V weight
    // stays below 2^kSlack (its int32 limbs cannot overflow) and most blocks
    // skip the cross-lane maximum and the rescale.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float smax = fmaxf(fmaxf(sc[gi][0], sc[gi][1]), fmaxf(sc[gi][2], sc[gi][3]));
      const float vmax = fmaxf(fmaxf(sv[gi][0], sv[gi][1]), fmaxf(sv[gi][2], sv[gi][3]));
      if (__any(smax > m_run[gi] + kSlack || vmax > mu_run[gi] + kSlack)) {
        const float m_new = fmaxf(m_run[gi], rowmax16(smax));
        const float mu_new = fmaxf(mu_run[gi], rowmax16(vmax));
        const float alpha = __builtin_amdgcn_exp2f(m_run[gi] - m_new);
        const float alphaU = __builtin_amdgcn_exp2f(mu_run[gi] - mu_new);
        // the V accumulator rows of this lane are query row kg, as its scores
        if constexpr (kLazyV) fold_v(gi);
#pragma unroll
        for (int k = 0; k < NB; ++k) facc[gi][k] *= alphaU;
        l_lane[gi] *= alpha;
        us_lane[gi] *= alphaU;
        m_run[gi] = m_new;
        mu_run[gi] = mu_new;
      }
    }
    // the weights go to the V operand layout first, so the ds_bpermutes are in
    // flight together
    float Uv[NG][4];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float ps = 0.f, us = 0.f;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        ps += __builtin_amdgcn_exp2f(sc[gi][tau] - m_run[gi]);
        const float U = __builtin_amdgcn_exp2f(sv[gi][tau] - mu_run[gi]);
        us += U;
        Uv[gi][tau] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(perm_addr, __builtin_bit_cast(int, U)));
      }
      l_lane[gi] += ps;
      us_lane[gi] += us;
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (VBITS == 3) {
    v4i A[NG][4];   // per group and plane: weight limbs, VGPR tau, byte r = token 16 tau + 4 kg + r
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        const float Ut = __builtin_amdgcn_ldexpf(Uv[gi][tau], -tau);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int X = (int)fmaf(Ut, cx[j], half[j]);
          const uint32_t t4 = quad_byte_transpose((uint32_t)X + 0x80808080u, lam) ^ 0x80808080u;
          A[gi][j][tau] = (int)t4;
        }
      }

    // ---- V: one 64-token K block, D/16 column blocks x 4 planes
    auto vword = [&](int j, int kp) -> uint32_t {
      const uint4 &u = vcur[j][kp >> 2];
      const int e = kp & 3;
      return e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
    };
    uint32_t xw[D / 32];
#pragma unroll
    for (int kp = 0; kp < D / 32; ++kp) xw[kp] = vword(0, kp) ^ vword(1, kp) ^ vword(2, kp);
    // column blocks 2 kp and 2 kp + 1 come from the low and high nibbles of the
    // same words; their accumulation chains (and those of the groups) are
    // interleaved
#pragma unroll
    for (int kp = 0; kp < D / 32; ++kp) {
      const uint32_t wj[4] = {vword(0, kp), vword(1, kp), vword(2, kp), xw[kp]};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w = wj[j] >> (4 * h);
          v4i bop;   // VGPR tau, byte r: token 16 tau + 4 kg + r, bit value 2^tau
          bop.x = (int)(w & 0x01010101u);
          bop.y = (int)(w & 0x02020202u);
          bop.z = (int)(w & 0x04040404u);
          bop.w = (int)(w & 0x08080808u);
#pragma unroll
          for (int gi = 0; gi < NG; ++gi)
            vacc[gi][2 * kp + h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[gi][j], bop, vacc[gi][2 * kp + h], 0, 0, 0);
        }
      if constexpr (!kLazyV) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          fold_one(gi, 2 * kp);
          fold_one(gi, 2 * kp + 1);
        }
      }
    }
    } else {
    // other code widths: the NP planes in turn, each with its own weight limbs
    float Ut[NG][4];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) Ut[gi][tau] = __builtin_amdgcn_ldexpf(Uv[gi][tau], -tau);
    auto vword = [&](int j, int kp) -> uint32_t {
      const uint4 &u = vcur[j][kp >> 2];
      const int e = kp & 3;
      return e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
    };
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      v4i Ap[NG];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const int X = (int)fmaf(Ut[gi][tau], cx[p], half[p]);
          Ap[gi][tau] = (int)(quad_byte_transpose((uint32_t)X + 0x80808080u, lam) ^ 0x80808080u);
        }
#pragma unroll
      for (int kp = 0; kp < D / 32; ++kp) {
        // the plane word: parity of the code bits in the plane's mask
        uint32_t wp = 0u;
#pragma unroll
        for (int j = 0; j < VBITS; ++j)
          if ((VPlanes<VBITS>::mask[p] >> j) & 1) wp ^= vword(j, kp);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w = wp >> (4 * h);
          v4i bop;   // VGPR tau, byte r: token 16 tau + 4 kg + r, bit value 2^tau
          bop.x = (int)(w & 0x01010101u);
          bop.y = (int)(w & 0x02020202u);
          bop.z = (int)(w & 0x04040404u);
          bop.w = (int)(w & 0x08080808u);
#pragma unroll
          for (int gi = 0; gi < NG; ++gi)
            vacc[gi][2 * kp + h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ap[gi], bop, vacc[gi][2 * kp + h], 0, 0, 0);
        }
      }
    }
    if constexpr (!kLazyV) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) fold_v(gi);
    }
    }
  };

  // the first block's loads go out before the query operand is staged, so the
  // two fetches overlap
  if constexpr (TWO_SETS) {
    MfmaBlock<D, VBITS, KBITS> d0, d1;
    if (pg0 < pg1) load_block(d0, pg0);
    // the packed query operand is shared by the four waves: keep it in LDS
    stage();
    __syncthreads();
    for (int pg = pg0; pg < pg1; pg += 2) {
      if (pg + 1 < pg1) load_block(d1, pg + 1);
      process(d0, pg);
      if (pg + 1 >= pg1) break;
      if (pg + 2 < pg1) load_block(d0, pg + 2);
      process(d1, pg + 1);
    }
  } else {
    // one register set
    stage();
    __syncthreads();
    for (int pg = pg0; pg < pg1; ++pg) {
      MfmaBlock<D, VBITS, KBITS> d0;
      load_block(d0, pg);
      process(d0, pg);
    }
  }

  if constexpr (kLazyV) fold_v(0);
  // ---- combine the four waves into one partial per query row
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float l_row = rowsum16(l_lane[gi]), us_row = rowsum16(us_lane[gi]);
    if (n == 0) {
      s_wm[wave][0][4 * gi + kg] = m_run[gi];
      s_wm[wave][1][4 * gi + kg] = l_row;
      s_wm[wave][2][4 * gi + kg] = mu_run[gi];
      s_wm[wave][3][4 * gi + kg] = us_row;
    }
  }
  __syncthreads();   // every wave is past the page loop: the query operands are dead
  {
    const float c7 = a.vcb.levels[(1 << VBITS) - 1];   // the V codebook's largest level
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float usq = s_wm[wave][3][4 * gi + kg];
#pragma unroll
      for (int k = 0; k < NB; ++k) s_wacc[wave][4 * gi + kg][16 * k + n] = facc[gi][k] - c7 * usq;
    }
  }
  __syncthreads();
  const int nsplit = a.plan.n_split;
  const int rbase = kMfmaMaxGroup * rho0;   // first query row of the workgroup
  const int nrow = min(NR, a.plan.group - rbase);
  const size_t pbase = (((size_t)b * H + kvh) * nsplit + split) * a.plan.group + rbase;
  for (int qq = wave; qq < nrow; qq += 4) {
    float M = kNegInf, MU = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (s_wm[w][1][qq] > 0.f) {
        M = fmaxf(M, s_wm[w][0][qq]);
        MU = fmaxf(MU, s_wm[w][2][qq]);
      }
    float lsum = 0.f, fw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bool live = s_wm[w][1][qq] > 0.f;
      lsum += live ? s_wm[w][1][qq] * __builtin_amdgcn_exp2f(s_wm[w][0][qq] - M) : 0.f;
      fw[w] = live ? __builtin_amdgcn_exp2f(s_wm[w][2][qq] - MU) : 0.f;
    }
    float *pr = a.partials + (pbase + qq) * (D + kPartHead);
    if (lane == 0) {
      pr[0] = M;
      pr[1] = lsum;
      pr[2] = MU;
      pr[3] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < D / 64; ++r) {
      const int i = lane + 64 * r;
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) x = fmaf(fw[w], s_wacc[w][qq][i], x);
      pr[kPartHead + i] = x;
    }
  }
}

// One workgroup per (query row, KV head, sequence). Wave w takes splits
// w, w + 4, ...: it issues the loads of up to 16 of them at once (the headers are
// wave-uniform) and folds them with a running log-sum-exp; the four waves then
// combine in LDS, and wave 0 applies the inverse rotation and writes the row.
template <int D, bool kRotate>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  constexpr int R = D / 64;
  constexpr int CH = 16;   // splits per wave in flight
  __shared__ float s_st[4][3];
  __shared__ float s_x[4][D];
  const int qq = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int H = a.n_kv_heads, Hq = a.n_q_heads, g = Hq / H, G = a.plan.group;
  const int nsplit = a.plan.n_split;
  const size_t stride = (size_t)G * (D + kPartHead);
  const float *part = a.partials + (((size_t)b * H + kvh) * nsplit * G + qq) * (D + kPartHead);

  float M = -kFltMax, MU = -kFltMax, l = 0.f, x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = 0.f;
  for (int base = wv; base < nsplit; base += 4 * CH) {
    float4 hd[CH];
    float v[CH][R];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int sp = base + 4 * c;
      if (sp < nsplit) {
        const float *pr = part + (size_t)sp * stride;
        hd[c] = *reinterpret_cast<const float4 *>(pr);
#pragma unroll
        for (int r = 0; r < R; ++r) v[c][r] = pr[kPartHead + lane + 64 * r];
      } else {
        hd[c] = make_float4(-kFltMax, 0.f, -kFltMax, 0.f);
#pragma unroll
        for (int r = 0; r < R; ++r) v[c][r] = 0.f;
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (hd[c].y > 0.f) {   // a split with no visible token has l = 0
        const float mn = fmaxf(M, hd[c].x), mun = fmaxf(MU, hd[c].z);
        l = l * __builtin_amdgcn_exp2f(M - mn) + hd[c].y * __builtin_amdgcn_exp2f(hd[c].x - mn);
        const float f0 = __builtin_amdgcn_exp2f(MU - mun), f1 = __builtin_amdgcn_exp2f(hd[c].z - mun);
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = fmaf(x[r], f0, v[c][r] * f1);
        M = mn;
        MU = mun;
      }
    }
  }
  if (lane == 0) {
    s_st[wv][0] = M;
    s_st[wv][1] = MU;
    s_st[wv][2] = l;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) s_x[wv][lane + 64 * r] = x[r];
  __syncthreads();
  if (wv != 0) return;
  float Mg = -kFltMax, MUg = -kFltMax;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (s_st[w][2] > 0.f) {
      Mg = fmaxf(Mg, s_st[w][0]);
      MUg = fmaxf(MUg, s_st[w][1]);
    }
  float lsum = 0.f, fw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const bool live = s_st[w][2] > 0.f;
    lsum += live ? s_st[w][2] * __builtin_amdgcn_exp2f(s_st[w][0] - Mg) : 0.f;
    fw[w] = live ? __builtin_amdgcn_exp2f(s_st[w][1] - MUg) : 0.f;
  }
  const float inv = lsum > 0.f ? __builtin_amdgcn_exp2f(MUg - Mg) / lsum : 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = lane + 64 * r;
    x[r] = (fw[0] * s_x[0][i] + fw[1] * s_x[1][i] + fw[2] * s_x[2][i] + fw[3] * s_x[3][i]) * inv;
  }
  if constexpr (kRotate) {
    fwht_wave<R>(x);
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] *= rsqrt_dim<D>();
  }
  const int t = qq / g, hh = qq % g;
  float *o = a.out + (((size_t)b * a.n_q + t) * Hq + kvh * g + hh) * D;
#pragma unroll
  for (int r = 0; r < R; ++r) o[lane + 64 * r] = x[r];
}

template <int D, int VBITS, int KBITS>
hipError_t launch_split_bits(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid(a.plan.n_split, a.n_kv_heads, a.batch * a.plan.wg_per_seq);
  switch (a.plan.groups_per_wg) {
    case 1:
      // loads one block ahead pay off once a wave sees more than two blocks
      if (D == 128 && a.plan.pages_per_split > 2)
        hipLaunchKernelGGL((decode_mfma_kernel<D, 1, VBITS, KBITS, D == 128>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((decode_mfma_kernel<D, 1, VBITS, KBITS, false>), grid, dim3(256), 0, s, a);
      break;
    case 2:
      if constexpr (D == 128) {
        hipLaunchKernelGGL((decode_mfma_kernel<D, 2, VBITS, KBITS, false>), grid, dim3(256), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_dim(const DecodeArgs &a, hipStream_t s) {
  const int G = a.plan.group;
  if (!a.plan.mfma || G > TQ_MAX_GROUP) return hipErrorInvalidValue;
  auto by_k = [&](auto VB) -> hipError_t {
    switch (a.k_bits) {
      case 2: return launch_split_bits<D, VB.value, 2>(a, s);
      case 3: return launch_split_bits<D, VB.value, 3>(a, s);
      case 4: return launch_split_bits<D, VB.value, 4>(a, s);
      default: return hipErrorInvalidValue;
    }
  };
  switch (a.v_bits) {
    case 2: return by_k(std::integral_constant<int, 2>{});
    case 3: return by_k(std::integral_constant<int, 3>{});
    case 4: return by_k(std::integral_constant<int, 4>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t prep_region_bytes(int d, int batch, int n_q, int n_q_heads, int n_kv_heads, int kb) {
  size_t bytes = prep_float_bytes(d, batch, n_q, n_q_heads);
  const int group = n_q_heads / n_kv_heads * n_q;
  if (mfma_path(d, group))
    bytes += ((size_t)batch * n_kv_heads * query_groups(group) * packed_group_bytes(d, kb) + 255) / 256 * 256;
  return bytes;
}


hipError_t launch_decode_split(const DecodeArgs &a, int d, hipStream_t s) {
  return d == 128 ? launch_split_dim<128>(a, s) : launch_split_dim<256>(a, s);
}

hipError_t launch_decode_merge(const DecodeArgs &a, int d, hipStream_t s, bool rotate) {
  const dim3 grid(a.plan.group, a.n_kv_heads, a.batch);
  if (d == 128) {
    if (rotate)
      hipLaunchKernelGGL((merge_kernel<128, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((merge_kernel<128, false>), grid, dim3(256), 0, s, a);
  } else {
    if (rotate)
      hipLaunchKernelGGL((merge_kernel<256, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((merge_kernel<256, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tq
