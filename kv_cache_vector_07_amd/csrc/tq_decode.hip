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
// Query rows per KV head run as query groups of 4 rows (4 rows x 4 limbs fill
// the 16 MFMA rows); with 16 rows or more and 3-bit codes decode_wide_kernel
// below takes them instead. At d = 128 two groups share a workgroup; the
// workgroups of one split sit in blockIdx.z, n_split * Hkv apart, so with
// n_split * Hkv a multiple of 8 they land on the same XCD and share its L2.
// With a causal tail a workgroup stops at the last token its rows can see.
//
// One register set holds a block's loads (the first block's go out before the
// query operand is staged): at d = 128 with one group that leaves three waves
// per SIMD (under 170 VGPRs). There the next block's key words are loaded as
// soon as the score MFMAs have read the current ones, and its sidecars and V
// words after the V MFMAs; at d = 256 a block's loads go out at its start, and
// one set keeps two waves per SIMD.

// The packed scoring operand of the workgroup's query groups (per group NMU x
// 64 lanes x 32 bytes, then NMU x 64 scale words), held in registers between
// its loads and its copy into LDS. Every load is issued at once and none sits
// under a branch (indices past the end are clamped and the values replaced), so
// the block loads issued after them do not hold up the copy: loads complete in
// order. A group past the last one gets zero operands and unit scales.
template <int NMU, int NG>
struct QueryStage {
  static constexpr int NV = (NMU * 128 + 255) / 256, NS = (NMU * 64 + 255) / 256;
  uint4 v[NG][NV];
  int sc[NG][NS];

  // seq: the (sequence, KV head)'s first group; groups rho0 .. rho0 + NG - 1 of QG
  __device__ inline void load(const uint8_t *seq, size_t gbytes, int rho0, int QG, int tid) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const uint8_t *grp = seq + (size_t)min(rho0 + gi, QG - 1) * gbytes;
      const uint4 *src = reinterpret_cast<const uint4 *>(grp);
      const int *ssrc = reinterpret_cast<const int *>(grp + (size_t)NMU * 2048);
#pragma unroll
      for (int i = 0; i < NV; ++i) v[gi][i] = src[min(tid + 256 * i, NMU * 128 - 1)];
#pragma unroll
      for (int i = 0; i < NS; ++i) sc[gi][i] = ssrc[min(tid + 256 * i, NMU * 64 - 1)];
    }
  }

  // groups from QG - rho0 on are past the last one
  __device__ inline void store(v8i *s_qop, int *s_qsc, int rho0, int QG, int tid) const {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const bool live = rho0 + gi < QG;
      uint4 *dst = reinterpret_cast<uint4 *>(s_qop + gi * NMU * 64);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = tid + 256 * i;
        if (e < NMU * 128) dst[e] = live ? v[gi][i] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = tid + 256 * i;
        if (e < NMU * 64) s_qsc[gi * NMU * 64 + e] = live ? sc[gi][i] : 127;
      }
    }
  }
};

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
template <int D, int NG, int VBITS, int KBITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NG == 1 ? (D == 128 ? 3 : 2) : 1))) void decode_mfma_kernel(DecodeArgs a) {
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

  // the query operands live in LDS during the page loop; the per-wave V
  // numerators of the final combine have their own region, so a wave can write
  // them while others still read query operands
  constexpr size_t QOP_BYTES = (size_t)NG * NMU * 64 * 32, QSC_BYTES = (size_t)NG * NMU * 64 * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[QOP_BYTES + QSC_BYTES];
  __shared__ float s_wacc[4][NR][D];                // per wave: V numerator of each row
  __shared__ float s_wm[4][4][NR];                  // per wave: m, l, mU, sum U of each row
  v8i *s_qop = reinterpret_cast<v8i *>(s_raw);      // [group][mfma][lane]
  int *s_qsc = reinterpret_cast<int *>(s_raw + QOP_BYTES);

  const int QG = a.plan.qgroups, WZ = a.plan.wg_per_seq;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z / WZ;
  const int rho0 = (blockIdx.z % WZ) * NG;           // first query group of the workgroup
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 15, kg = lane >> 4;   // scores: token 16 tau + n of query row kg
  const int lam = n & 3;                     // V weight operand: limb row / token of the quad
  const int H = a.n_kv_heads, g = a.n_q_heads / H;

  // The start is a chain of latencies (arguments, then the packed query operand
  // and the sequence's length and block table, then the first block), so the
  // loads go out in that order, none under a branch, before anything waits.
  const size_t gbytes = packed_group_bytes(D, KBITS);
  const uint8_t *seq_grp = a.packed + ((size_t)b * H + kvh) * QG * gbytes;
  QueryStage<NMU, NG> qs;
  qs.load(seq_grp, gbytes, rho0, QG, tid);
  float4 rc[NG];   // row constants {0, 0, sum q~, sum p} of this lane's query row
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
    rc[gi] = reinterpret_cast<const float4 *>(seq_grp + (size_t)min(rho0 + gi, QG - 1) * gbytes +
                                              (size_t)NMU * (2048 + 256))[kg];
  // The sequence's length and first visible token and the block-table entries
  // of the split's first two pages are loaded together (an entry past the
  // sequence is read but not used; without a window the start is read from the
  // lengths and dropped), and the empty asm keeps the compiler from sinking
  // them past the branches below, one after another.
  const int L = a.seq_lens[b];
  const int s0raw = (a.seq_starts ? a.seq_starts : a.seq_lens)[b];
  const int pgs = split * a.plan.pages_per_split;
  const int32_t *brow = a.block_table + (size_t)b * a.max_pages;
  const int physA = brow[min(pgs, a.max_pages - 1)];
  const int physB = brow[min(pgs + 1, a.max_pages - 1)];
  asm volatile("" ::"s"(L), "s"(s0raw), "s"(physA), "s"(physB));
  auto phys_of = [&](int pg) { return pg == pgs ? physA : pg == pgs + 1 ? physB : brow[pg]; };
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
  const int S0 = a.seq_starts ? max(0, s0raw) : 0;
  const int pg0 = max(split * a.plan.pages_per_split, S0 / kPage);
  int pg1 = min(split * a.plan.pages_per_split + a.plan.pages_per_split, n_pages_seq);
  const int blk0 = 64 * wave;
  // pages whose block of this wave holds no visible token are skipped (only the last can)
  if (pg1 > pg0 && blk0 >= Lv - (pg1 - 1) * kPage) --pg1;


  // a block's key words (read by the score MFMAs) and the rest (sidecars and V
  // words, read after them) load separately
  auto load_keys_at = [&](MfmaBlock<D, VBITS, KBITS> &d, int phys) {
    const uint8_t *ks = a.k_pool + ((size_t)phys * H + kvh) * KSEC;
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
  };
  auto load_rest_at = [&](MfmaBlock<D, VBITS, KBITS> &d, int phys) {
    const uint8_t *ks = a.k_pool + ((size_t)phys * H + kvh) * KSEC;
    const uint8_t *vs = a.v_pool + ((size_t)phys * H + kvh) * VSEC;
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
  auto load_block_at = [&](MfmaBlock<D, VBITS, KBITS> &d, int phys) {
    load_keys_at(d, phys);
    load_rest_at(d, phys);
  };
  auto load_block = [&](MfmaBlock<D, VBITS, KBITS> &d, int pg) { load_block_at(d, phys_of(pg)); };

  // the first block's loads go out before anything waits for the query operand
  // (at d = 128: at d = 256 its registers would be live across the copy). An
  // empty split loads a block of page 0, which always exists, and never uses it.
  constexpr bool kEarly = D == 128;
  MfmaBlock<D, VBITS, KBITS> d0;
  if constexpr (kEarly) load_block_at(d0, pg0 < pg1 ? phys_of(pg0) : 0);

  float off1[NG], off2[NG];
  int vis[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int row = kMfmaMaxGroup * (rho0 + gi) + kg;   // query row of this lane in group gi
    const bool live = row < a.plan.group;
    off1[gi] = live ? a.cb.levels[(1 << KBITS) - 1] * rc[gi].z : 0.f;
    off2[gi] = live ? rc[gi].w * qjl_kappa<D>() : 0.f;
    vis[gi] = !live ? 0 : a.causal_tail ? L - (a.n_q - 1 - row / g) : L;
  }

  // At d = 128 block pg + 1 loads while block pg is processed, into the same
  // registers: its key words once the score MFMAs have been issued, the rest at
  // the end (the last block loads itself again, so the loop has no branch).
  constexpr bool kRot = D == 128 && KBITS + VBITS <= 7;
  auto process = [&](MfmaBlock<D, VBITS, KBITS> &d, int pg, int phys_next) {
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
      const int phys = phys_of(pg);
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
    if constexpr (kRot) load_keys_at(d, phys_next);
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
    if constexpr (kRot) load_rest_at(d, phys_next);
  };

  // the packed query operand is shared by the four waves: keep it in LDS
  qs.store(s_qop, s_qsc, rho0, QG, tid);
  __syncthreads();
  for (int pg = pg0; pg < pg1; ++pg) {
    if (!kEarly || (!kRot && pg > pg0)) load_block(d0, pg);
    process(d0, pg, kRot ? phys_of(min(pg + 1, pg1 - 1)) : 0);
  }

  if constexpr (kLazyV) fold_v(0);
  // ---- combine the four waves into one partial per query row
  {
    const float c7 = a.vcb.levels[(1 << VBITS) - 1];   // the V codebook's largest level
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      // every lane of a DPP row (one query row) holds the row sums
      const float l_row = rowsum16(l_lane[gi]), us_row = rowsum16(us_lane[gi]);
      if (n == 0) {
        s_wm[wave][0][4 * gi + kg] = m_run[gi];
        s_wm[wave][1][4 * gi + kg] = l_row;
        s_wm[wave][2][4 * gi + kg] = mu_run[gi];
        s_wm[wave][3][4 * gi + kg] = us_row;
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) s_wacc[wave][4 * gi + kg][16 * k + n] = facc[gi][k] - c7 * us_row;
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

// Everything one 64-token block of a wave needs (key record words, sidecars,
// V words), loaded before the block is processed.
template <int D>
struct WideBlock {
  uint32_t kw[4][D / 128][4];   // key words of coordinate groups kg + 4 c of tokens 16 tau + n
  uint2 g, nk, nv;              // G, N^K, N^V of side entries 4 n + tau
  uint4 v[3][D / 128];          // V words of plane j: coordinate pairs kp
};

// ------------------------------------------------------------- wide groups
// Sixteen distinct query rows per workgroup (3-bit K and V codes). Each wave
// owns 64-token blocks as in decode_mfma_kernel, but every operand built from
// the keys and the V bits serves all 16 rows:
//
// Scores: the A operand of scaled MFMA (mu, l) holds limb l of the 16 rows
// (fp6, E8M0 block scales per row), so the four limb MFMAs of a key operand
// accumulate into one result and the sum over limbs comes out of the MFMA.
// Output lane (n, kg) holds rows 4 kg + r (r = 0..3) of token 16 tau + n: one
// DPP row of 16 lanes holds four query rows, each with its own online softmax.
//
// V: per block and row the weights are scaled by a power of two that puts their
// largest in [0.5, 1), then (times each plane weight) taken in fixed point
// below 2^23 as three balanced int8 limbs, each with its own int32 sums; the
// block's sums are folded into fp32 with the scale undone (per block, as the
// scales differ). The weight operand of lane (m, kgA) is row m at tokens
// 16 tau + 4 kgA + r: a 4x4 transpose inside each quad of the score layout
// and a lane permutation (kg <-> kgA, one ds_bpermute per weight) bring the
// weights there, and byte permutes pack the limbs.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_wide_kernel(DecodeArgs a) {
  constexpr int VBITS = 3, KBITS = 3;
  constexpr int NPK = 4;                       // key code planes (then the sign plane)
  constexpr int NMU = mfma_per_tile(D, KBITS);
  constexpr int NOP = 4 * NMU;                 // (mu, limb) query operands
  constexpr int NCH = D / 128;
  constexpr int KREC = (KBITS + 1) * D / 8;
  constexpr size_t KCODES = (size_t)kPage * KREC;
  constexpr size_t KSEC = KCODES + 4 * kPage;
  constexpr size_t VCODES = (size_t)VBITS * D * kPage / 8;
  constexpr size_t VSEC = VCODES + 2 * kPage;
  constexpr int NB = D / 16;
  constexpr int RW = kWideRows;
  // the query operands live in LDS during the page loop, without the two zero
  // dwords of each lane's 32 bytes (fp6 fields fill six): dwords 0-3 and 4-5 in
  // planes of their own (conflict-free 16- and 8-byte reads), then the scale
  // words. The same bytes then hold the per-wave V numerators for the final
  // combine. At d = 256 that keeps two workgroups per CU.
  constexpr size_t Q16_BYTES = (size_t)NOP * 64 * 16, Q8_BYTES = (size_t)NOP * 64 * 8;
  constexpr size_t QSC_BYTES = (size_t)NOP * 64 * 4;
  constexpr size_t QALL = Q16_BYTES + Q8_BYTES + QSC_BYTES;
  constexpr size_t WACC_BYTES = (size_t)4 * RW * D * 4;
  constexpr size_t RAW = QALL > WACC_BYTES ? QALL : WACC_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[RAW];
  __shared__ float s_wm[4][4][RW];                  // per wave: m, l, mU, sum U of each row
  __shared__ float4 s_rc[RW];                       // per row: code and sign offsets, visible length
  uint4 *s_q16 = reinterpret_cast<uint4 *>(s_raw);  // [operand][lane]
  uint2 *s_q8 = reinterpret_cast<uint2 *>(s_raw + Q16_BYTES);
  int *s_qsc = reinterpret_cast<int *>(s_raw + Q16_BYTES + Q8_BYTES);
  auto s_wacc = reinterpret_cast<float (*)[RW][D]>(s_raw);   // [wave][row][d], after the loop

  const int QG = a.plan.qgroups;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z / QG, rho = blockIdx.z % QG;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 15, kg = lane >> 4;
  const int H = a.n_kv_heads, g = a.n_q_heads / H, G = a.plan.group;
  const int row0 = RW * rho;   // first query row of the workgroup

  // loads first, none under a branch: the group's packed operand and row
  // constants, then the sequence's length and start and the split's first
  // block-table entries
  const size_t gbytes = packed_group_bytes_wide(D);
  const uint8_t *grp = a.packed + (((size_t)b * H + kvh) * QG + rho) * gbytes;
  QueryStage<NOP, 1> qs;
  qs.load(grp, gbytes, 0, 1, tid);
  const float4 *rcp = reinterpret_cast<const float4 *>(grp + (size_t)NOP * (2048 + 256));
  const float4 rcA = rcp[2 * kg], rcB = rcp[2 * kg + 1];   // {sum q~, sum p} of rows 4 kg .. 4 kg + 3
  const int L = a.seq_lens[b];
  const int s0raw = (a.seq_starts ? a.seq_starts : a.seq_lens)[b];
  const int pgs = split * a.plan.pages_per_split;
  const int32_t *brow = a.block_table + (size_t)b * a.max_pages;
  const int physA = brow[min(pgs, a.max_pages - 1)];
  asm volatile("" ::"s"(L), "s"(s0raw), "s"(physA));
  auto phys_of = [&](int pg) { return pg == pgs ? physA : brow[pg]; };

  // Lv: one past the last token any row of the workgroup sees
  const int row_last = min(row0 + RW, G) - 1;
  const int Lv = a.causal_tail ? L - (a.n_q - 1 - row_last / g) : L;
  // one past the last token the workgroup's first row (the one that sees least) sees
  const int vis_first = a.causal_tail ? L - (a.n_q - 1 - row0 / g) : L;
  const int n_pages_seq = min((Lv + kPage - 1) / kPage, a.max_pages);
  const int S0 = a.seq_starts ? max(0, s0raw) : 0;
  const int pg0 = max(pgs, S0 / kPage);
  int pg1 = min(pgs + a.plan.pages_per_split, n_pages_seq);
  const int blk0 = 64 * wave;
  if (pg1 > pg0 && blk0 >= Lv - (pg1 - 1) * kPage) --pg1;

  // this lane's rows 4 kg + r
  const float c7k = a.cb.levels[(1 << KBITS) - 1];
  float off1[4], off2[4];
  int vis[4];
  {
    const float sqv[4] = {rcA.x, rcA.z, rcB.x, rcB.z}, spv[4] = {rcA.y, rcA.w, rcB.y, rcB.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * kg + r;
      const bool live = row < G;
      off1[r] = live ? c7k * sqv[r] : 0.f;
      off2[r] = live ? spv[r] * qjl_kappa<D>() : 0.f;
      vis[r] = !live ? 0 : a.causal_tail ? L - (a.n_q - 1 - row / g) : L;
    }
  }
  // the row constants are read from LDS where they are used, which keeps them
  // out of the registers of the page loop
  if (wave == 0 && n == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_rc[4 * kg + r] = make_float4(off1[r], off2[r], __int_as_float(vis[r]), 0.f);
  }
  const float scale2 = a.scale * 1.4426950408889634f;   // scores in log2 units
  float wpl[4];
  plane_weights(a.vcb, wpl);
  float wmax = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) wmax = fmaxf(wmax, fabsf(wpl[j]));
  // weight X = U' * 2^-tau * (|w_j| / wmax) * kFix with U' < 1 the block-scaled
  // weight, 2^tau being the value the V bit of token 16 tau + 4 k + r takes in
  // byte r of the B operand. A plane with a negative weight is taken as its
  // complement, w p = |w| (1 - p) + w, so X >= 0 and the constant w joins the
  // offset: the levels are sum_j |w_j| p'_j - c_eff with c_eff = c7 - sum of the
  // negative w_j. With 0 <= X <= kFix, X + 0x8080 < 2^23: it is exact in the
  // mantissa of 2^23 + 0x8080 + X (round to nearest), and its top byte is int8.
  constexpr float kFix = 8355000.f;
  constexpr float kMagic = 8421504.f;   // 2^23 + 0x8080
  float cx[4], c_eff = a.vcb.levels[(1 << VBITS) - 1];
  uint32_t flip[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cx[j] = fabsf(wpl[j]) / wmax * kFix;
    flip[j] = wpl[j] < 0.f ? 0xFFFFFFFFu : 0u;
    c_eff -= wpl[j] < 0.f ? wpl[j] : 0.f;
  }
  float delta_u = wmax / kFix;
  if constexpr (D == 256) {
    // these are the same in every lane: scalar registers free vector ones
    // (at d = 256 that takes the kernel's register spills out of the page loop)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cx[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, cx[j])));
      flip[j] = (uint32_t)__builtin_amdgcn_readfirstlane((int)flip[j]);
    }
    c_eff = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, c_eff)));
    delta_u = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, delta_u)));
  }
  // source lane of the weight transpose (kg <-> kgA): lane 16 a + 4 b + c reads lane 16 b + 4 a + c
  const int tr_addr = 4 * (16 * ((lane >> 2) & 3) + 4 * (lane >> 4) + (lane & 3));
  const int rq = lane & 3;   // the lane's place in its quad

  float m_run[4], mu_run[4], l_lane[4], us_lane[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = mu_run[r] = -kFltMax;
    l_lane[r] = us_lane[r] = 0.f;
  }
  v4f facc[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) facc[k] = v4f{0.f, 0.f, 0.f, 0.f};

  auto load_block_at = [&](WideBlock<D> &d, int phys) {
    const uint8_t *ks = a.k_pool + ((size_t)phys * H + kvh) * KSEC;
    const uint8_t *vs = a.v_pool + ((size_t)phys * H + kvh) * VSEC;
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint8_t *rec = ks + (size_t)(blk0 + 16 * tau + n) * KREC;
        const uint4 u = reinterpret_cast<const uint4 *>(rec)[kg + 4 * c];
        d.kw[tau][c][0] = u.x;
        d.kw[tau][c][1] = u.y;
        d.kw[tau][c][2] = u.z;
        d.kw[tau][c][3] = u.w;
      }
    const int se = blk0 + 4 * n;   // side entries of tokens 16 tau + n, tau = 0..3
    d.g = *reinterpret_cast<const uint2 *>(ks + KCODES + 2 * kPage + 2 * se);
    d.nk = *reinterpret_cast<const uint2 *>(ks + KCODES + 2 * se);
    d.nv = *reinterpret_cast<const uint2 *>(vs + VCODES + 2 * se);
    const uint4 *vw = reinterpret_cast<const uint4 *>(vs + (size_t)4 * (wave * 2 * VBITS * D) + 4 * (D / 32) * lane);
#pragma unroll
    for (int j = 0; j < VBITS; ++j)
#pragma unroll
      for (int c = 0; c < NCH; ++c) d.v[j][c] = vw[j * 2 * D * 4 / 16 + c];
  };

  // ---- scores of the 16 rows: c1 (code planes) and c2 (signs) per tile
  auto score_mfma = [&](const WideBlock<D> &d, v4f (&c1)[4], v4f (&c2)[4]) {
    // the query operands are read from LDS where they are used (an opaque lane
    // offset keeps them from being hoisted out of the page loop)
    int qo = lane;
    asm volatile("" : "+v"(qo));
    // the accumulators start at minus the rows' code and sign offsets, so the
    // MFMAs leave the offset-corrected sums
    {
      int ro = 4 * kg;
      asm volatile("" : "+v"(ro));
      float4 rcr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rcr[r] = s_rc[ro + r];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        c1[tau] = v4f{-rcr[0].x, -rcr[1].x, -rcr[2].x, -rcr[3].x};
        c2[tau] = v4f{-rcr[0].y, -rcr[1].y, -rcr[2].y, -rcr[3].y};
      }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int j = 0; j <= NPK; ++j) {
        v8i op[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const uint32_t *w = d.kw[tau][c];
          const uint32_t pl = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : j == 3 ? (w[0] ^ w[1] ^ w[2]) : w[3];
          op[tau] = v8i{(int)(pl & 0x11111111u), (int)(pl & 0x22222222u), (int)(pl & 0x44444444u),
                        (int)((pl >> 1) & 0x44444444u), 0, 0, 0, 0};
        }
#pragma unroll
        for (int limb = 0; limb < 4; ++limb) {
          const int o = ((NPK + 1) * c + j) * 4 + limb;
          const uint4 q16 = s_q16[o * 64 + qo];
          const uint2 q8 = s_q8[o * 64 + qo];
          const v8i qop = v8i{(int)q16.x, (int)q16.y, (int)q16.z, (int)q16.w, (int)q8.x, (int)q8.y, 0, 0};
          const int qsc = s_qsc[o * 64 + qo];
#pragma unroll
          for (int tau = 0; tau < 4; ++tau) {
            if (j < NPK)
              c1[tau] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qop, op[tau], c1[tau], 2, 4, 0, qsc, 0, 127);
            else
              c2[tau] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qop, op[tau], c2[tau], 2, 4, 0, qsc, 0, 127);
          }
        }
      }
    }
  };

  // the rest of a block: scores, softmax, weights, V
  auto finish = [&](const WideBlock<D> &d, int pg, const v4f (&c1)[4], const v4f (&c2)[4]) {
    const uint4 (&vcur)[VBITS][NCH] = d.v;
    const int tok0 = pg * kPage;
    const int ntok = min(kPage, L - tok0);
    float sc[4][4], sv[4][4];   // [tau][row r]
    float sN[4], lnv[4];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const int sh = 16 * (tau & 1);
      const float Gt = f16_bits_to_f32((uint16_t)(((tau >> 1) ? d.g.y : d.g.x) >> sh));
      const float N = f16_bits_to_f32((uint16_t)(((tau >> 1) ? d.nk.y : d.nk.x) >> sh));
      lnv[tau] = __builtin_amdgcn_logf(f16_bits_to_f32((uint16_t)(((tau >> 1) ? d.nv.y : d.nv.x) >> sh)));
      sN[tau] = scale2 * N;
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[tau][r] = sN[tau] * fmaf(Gt, c2[tau][r], c1[tau][r]);
    }
    // a block that every row of the workgroup sees whole (inside the page and
    // the window, before the first row's causal end) needs no mask
    if (tok0 + blk0 >= S0 && tok0 + blk0 + 64 <= vis_first) {
#pragma unroll
      for (int tau = 0; tau < 4; ++tau)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[tau][r] = sc[tau][r] + lnv[tau];   // + log2 N^V
    } else {
      int ro = 4 * kg;
      asm volatile("" : "+v"(ro));
      int visr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) visr[r] = __float_as_int(s_rc[ro + r].z);
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        const int tok = blk0 + 16 * tau + n;
        const bool in_page = tok < ntok && tok0 + tok >= S0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool valid = in_page && tok0 + tok < visr[r];   // 0 for rows past the group
          sv[tau][r] = valid ? sc[tau][r] + lnv[tau] : kNegInf;
          sc[tau][r] = valid ? sc[tau][r] : kNegInf;
        }
      }
    }

    // ---- online softmax of this wave, per row (lazy references, as in decode_mfma_kernel)
    {
      float smax[4], vmax[4];
      bool move = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        smax[r] = fmaxf(fmaxf(sc[0][r], sc[1][r]), fmaxf(sc[2][r], sc[3][r]));
        vmax[r] = fmaxf(fmaxf(sv[0][r], sv[1][r]), fmaxf(sv[2][r], sv[3][r]));
        move |= smax[r] > m_run[r] + kSlack || vmax[r] > mu_run[r] + kSlack;
      }
      if (__any(move)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float m_new = fmaxf(m_run[r], rowmax16(smax[r]));
          const float mu_new = fmaxf(mu_run[r], rowmax16(vmax[r]));
          const float alpha = __builtin_amdgcn_exp2f(m_run[r] - m_new);
          const float alphaU = __builtin_amdgcn_exp2f(mu_run[r] - mu_new);
#pragma unroll
          for (int k = 0; k < NB; ++k) facc[k][r] *= alphaU;
          l_lane[r] *= alpha;
          us_lane[r] *= alphaU;
          m_run[r] = m_new;
          mu_run[r] = mu_new;
        }
      }
    }
    float U[4][4];   // [tau][row r]
    float dsc[4];    // per row: delta_u * 2^E, 2^-E the block's weight scale
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float ps = 0.f, us = 0.f, um = 0.f;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        ps += __builtin_amdgcn_exp2f(sc[tau][r] - m_run[r]);
        U[tau][r] = __builtin_amdgcn_exp2f(sv[tau][r] - mu_run[r]);
        us += U[tau][r];
        um = fmaxf(um, U[tau][r]);
      }
      l_lane[r] += ps;
      us_lane[r] += us;
      // the block's largest weight of the row, as m 2^E with m in [0.5, 1) (E = 0 if none)
      const float bm = rowmax16(um);
      const int E = bm > 0.f ? __builtin_amdgcn_frexp_expf(bm) : 0;
      dsc[r] = __builtin_amdgcn_ldexpf(delta_u, E);
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) U[tau][r] = __builtin_amdgcn_ldexpf(U[tau][r], -E);
    }

    // ---- weights to the V operand layout. Transpose inside each quad (lane q
    // of the quad gets slot q of lanes 0..3: rows 4 kg + q, tokens 16 tau + 4 (n >> 2) + r),
    // then lane 16 a + 4 b + c takes lane 16 b + 4 a + c.
    float T[4][4];   // [tau][r]: row (lane & 15), token 16 tau + 4 (lane >> 4) + r
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      float s1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float o = dppf<0x4E>(U[tau][r ^ 2]);   // quad_perm [2,3,0,1]
        s1[r] = ((r ^ rq) & 2) ? o : U[tau][r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float o = dppf<0xB1>(s1[r ^ 1]);       // quad_perm [1,0,3,2]
        const float t = ((r ^ rq) & 1) ? o : s1[r];
        T[tau][r] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(tr_addr, __builtin_bit_cast(int, t)));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
      for (int r = 0; r < 4; ++r) T[tau][r] = __builtin_amdgcn_ldexpf(T[tau][r], -tau);

    // ---- V: chunks of column blocks; per chunk the four planes in turn, each
    // with three limbs. A chunk's int32 sums start at zero and are folded with
    // the row's scale.
    auto vword = [&](int j, int kp) -> uint32_t {
      const uint4 &u = vcur[j][kp >> 2];
      const int e = kp & 3;
      return e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
    };
    // weight limbs of plane j: bytes r = limb l of the weight of token
    // 16 tau + 4 kgA + r. Y = X + 0x8080 (low three bytes of the float
    // 2^23 + 0x8080 + X); limbs: bytes 0 and 1 of Y with their top bit flipped,
    // then byte 2 (in [0, 127]): X = b0 + 256 b1 + 65536 b2.
    auto build_a = [&](int j, v4i (&Aj)[3]) {
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          uint32_t Y[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) Y[r] = __float_as_uint(fmaf(T[tau][r], cx[j], kMagic));
          const uint32_t t01 = __builtin_amdgcn_perm(Y[1], Y[0], 0x05010400u);   // Y0.b0 Y1.b0 Y0.b1 Y1.b1
          const uint32_t t23 = __builtin_amdgcn_perm(Y[3], Y[2], 0x05010400u);
          const uint32_t u01 = __builtin_amdgcn_perm(Y[1], Y[0], 0x06020602u);   // Y0.b2 Y1.b2 (twice)
          const uint32_t u23 = __builtin_amdgcn_perm(Y[3], Y[2], 0x06020602u);
          Aj[0][tau] = (int)(__builtin_amdgcn_perm(t23, t01, 0x05040100u) ^ 0x80808080u);
          Aj[1][tau] = (int)(__builtin_amdgcn_perm(t23, t01, 0x07060302u) ^ 0x80808080u);
          Aj[2][tau] = (int)__builtin_amdgcn_perm(u23, u01, 0x05040100u);
        }
    };
    // the four planes' limbs, built once for all column chunks
    v4i Aall[4][3];
#pragma unroll
    for (int j = 0; j < 4; ++j) build_a(j, Aall[j]);
    // column blocks per chunk: 4 at d = 128, 2 at d = 256 (two waves per SIMD
    // need at most 256 registers)
    constexpr int CBK = D == 128 ? 4 : 2;
#pragma unroll
    for (int ch = 0; ch < NB / CBK; ++ch) {
      v4i vacc[3][CBK];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        const v4i (&Aj)[3] = Aall[j];
#pragma unroll
        for (int kq = 0; kq < CBK / 2; ++kq) {
          const int kp = (CBK / 2) * ch + kq;
          const uint32_t wj = (j < 3 ? vword(j, kp) : vword(0, kp) ^ vword(1, kp) ^ vword(2, kp)) ^ flip[j];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t w = wj >> (4 * h);
            v4i bop;   // VGPR tau, byte r: token 16 tau + 4 k + r, bit value 2^tau
            bop.x = (int)(w & 0x01010101u);
            bop.y = (int)(w & 0x02020202u);
            bop.z = (int)(w & 0x04040404u);
            bop.w = (int)(w & 0x08080808u);
#pragma unroll
            for (int l = 0; l < 3; ++l)
              vacc[l][2 * kq + h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                  Aj[l], bop, j == 0 ? v4i{0, 0, 0, 0} : vacc[l][2 * kq + h], 0, 0, 0);
          }
        }
      }
      // a limb row gains at most 64 tokens x 4 planes x 128 x 8 = 2^18 per block,
      // so b0 + 256 b1 stays exact in int32
#pragma unroll
      for (int k = 0; k < CBK; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float lo = (float)(vacc[0][k][r] + (vacc[1][k][r] << 8));
          facc[CBK * ch + k][r] = fmaf(dsc[r], fmaf(65536.f, (float)vacc[2][k][r], lo), facc[CBK * ch + k][r]);
        }
    }
  };

  // the query operand (shared by the four waves, kept in LDS) is loaded first,
  // then the first block, then the operand is copied into LDS
  WideBlock<D> d0;
  load_block_at(d0, pg0 < pg1 ? phys_of(pg0) : 0);
  {
    // uint4 e of the operands: operand e >> 7, lane (e >> 1) & 63, half e & 1
#pragma unroll
    for (int i = 0; i < QueryStage<NOP, 1>::NV; ++i) {
      const int e = tid + 256 * i;
      if (e < NOP * 128) {
        const int o64 = (e >> 7) * 64 + ((e >> 1) & 63);
        if (e & 1)
          s_q8[o64] = make_uint2(qs.v[0][i].x, qs.v[0][i].y);
        else
          s_q16[o64] = qs.v[0][i];
      }
    }
#pragma unroll
    for (int i = 0; i < QueryStage<NOP, 1>::NS; ++i) {
      const int e = tid + 256 * i;
      if (e < NOP * 64) s_qsc[e] = qs.sc[0][i];
    }
  }
  __syncthreads();
  for (int pg = pg0; pg < pg1; ++pg) {
    if (pg > pg0) load_block_at(d0, phys_of(pg));
    v4f a1[4], a2[4];
    score_mfma(d0, a1, a2);
    finish(d0, pg, a1, a2);
  }

  // ---- combine the four waves into one partial per query row
  __syncthreads();   // every wave is past the page loop: the query operands are dead
  {
    const float c7 = c_eff;   // the V levels' offset (the largest level, less the flipped planes' weights)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float l_row = rowsum16(l_lane[r]), us_row = rowsum16(us_lane[r]);
      if (n == 0) {
        s_wm[wave][0][4 * kg + r] = m_run[r];
        s_wm[wave][1][4 * kg + r] = l_row;
        s_wm[wave][2][4 * kg + r] = mu_run[r];
        s_wm[wave][3][4 * kg + r] = us_row;
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) s_wacc[wave][4 * kg + r][16 * k + n] = facc[k][r] - c7 * us_row;
    }
  }
  __syncthreads();
  const int nsplit = a.plan.n_split;
  const int nrow = min(RW, G - row0);
  const size_t pbase = (((size_t)b * H + kvh) * nsplit + split) * G + row0;
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
// w, w + 4, ..., 16 at a time: lane c loads the header (m, l, mU) of the c-th,
// every lane loads its coordinates of all 16 (split indices past the last are
// clamped, so every load is in bounds and none is branched around), and the
// splits are folded in order with a running log-sum-exp, each header read from
// its lane; the four waves then combine in LDS, and wave 0 applies the inverse
// rotation and writes the row.
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
    float4 hl = make_float4(-kFltMax, 0.f, -kFltMax, 0.f);
    if (lane < CH && base + 4 * lane < nsplit)
      hl = *reinterpret_cast<const float4 *>(part + (size_t)(base + 4 * lane) * stride);
    float v[CH][R];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float *pr = part + (size_t)min(base + 4 * c, nsplit - 1) * stride;
#pragma unroll
      for (int r = 0; r < R; ++r) v[c][r] = pr[kPartHead + lane + 64 * r];
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float hy = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hl.y), c));
      if (hy > 0.f) {   // a split with no visible token has l = 0 (as has one past the last)
        const float hx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hl.x), c));
        const float hz = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hl.z), c));
        const float mn = fmaxf(M, hx), mun = fmaxf(MU, hz);
        l = l * __builtin_amdgcn_exp2f(M - mn) + hy * __builtin_amdgcn_exp2f(hx - mn);
        const float f0 = __builtin_amdgcn_exp2f(MU - mun), f1 = __builtin_amdgcn_exp2f(hz - mun);
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
      hipLaunchKernelGGL((decode_mfma_kernel<D, 1, VBITS, KBITS>), grid, dim3(256), 0, s, a);
      break;
    case 2:
      if constexpr (D == 128) {
        hipLaunchKernelGGL((decode_mfma_kernel<D, 2, VBITS, KBITS>), grid, dim3(256), 0, s, a);
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
  if (a.plan.wide) {
    if (a.k_bits != 3 || a.v_bits != 3 || a.plan.wg_per_seq != a.plan.qgroups) return hipErrorInvalidValue;
    const dim3 grid(a.plan.n_split, a.n_kv_heads, a.batch * a.plan.qgroups);
    hipLaunchKernelGGL((decode_wide_kernel<D>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
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

size_t prep_region_bytes(int d, int batch, int n_q, int n_q_heads, int n_kv_heads, int kb, int vb) {
  size_t bytes = prep_float_bytes(d, batch, n_q, n_q_heads);
  const int group = n_q_heads / n_kv_heads * n_q;
  if (wide_path(d, group, kb, vb))
    bytes += ((size_t)batch * n_kv_heads * ((group + kWideRows - 1) / kWideRows) * packed_group_bytes_wide(d) +
              255) / 256 * 256;
  else if (mfma_path(d, group))
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
