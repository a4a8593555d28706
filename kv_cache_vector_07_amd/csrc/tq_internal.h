// Internal interface between the C-ABI layer (tq_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

constexpr int kPage = TQ_PAGE_SIZE;

// Levels and thresholds of one codebook: 2^bits and 2^bits - 1 entries used
// (K: 3 bits; V: 2, 3 or 4).
struct Codebook {
  float levels[16];
  float thresholds[15];
};

inline size_t k_section_bytes(int d, int kbits = 3) {
  return (size_t)kPage * (kbits + 1) * d / 8 + 4u * kPage;
}
inline size_t v_section_bytes(int d, int vbits = 3) {
  return (size_t)vbits * d * kPage / 8 + 2u * kPage;
}

struct EncodeArgs {
  const void *x;          // [n_tokens][H][d], float32 or bfloat16
  int dtype;
  const int32_t *slots;   // [n_tokens]
  int n_tokens;
  int n_heads;
  uint8_t *pool;          // K or V pool
  const float *qjl;       // S [d][d] (K only)
  Codebook cb;            // the codebook of what is encoded
  int bits;               // code width (2, 3 or 4) of what is encoded
};

struct DequantArgs {
  const uint8_t *pool;
  const int32_t *slots;
  int n_tokens;
  int n_heads;
  int with_qjl;
  const float *qjl;
  float *out;             // [n_tokens][H][d]
  Codebook cb;            // K or V codebook
  int bits;               // code width of the records (K or V)
};

// Query preparation for one decode call: rotation, QJL projection and, for
// the MFMA decode path, the packed scoring operand (fp6 query limbs with block
// scales) of each (sequence, KV head, query group).
struct PrepArgs {
  const void *q;          // [batch][n_q][Hq][d]
  int dtype;
  int k_bits;             // K code width: the number of key bit planes follows
  int batch, n_q, n_q_heads, n_kv_heads;
  const float *qjl;
  float *prep;            // [rows][2][d]: Pi q, then S Pi q
  uint8_t *packed;        // per (sequence, KV head, query group): operand + row constants (or null)
  int wide;               // the packed operand is in 16-row groups (else 4-row groups)
  int pieces;             // workgroups per query row (set at launch)
  Codebook cb;            // K
};

// Bytes of the packed scoring operand of one query group of a (sequence, KV
// head): per 16-token tile a wave issues mfma_per_tile scaled fp6 x fp4 MFMAs
// whose query operand (32 B per lane) is stored lane-major, then their scale
// words (4 B per lane), then 4 rows x {0, 0, sum q~, sum p}.
// Key bit planes of kb-bit codes (the odd Walsh functions of the code bits):
// 2, 4 or 8; one more MFMA per 128 coordinates scores the QJL signs.
__host__ __device__ constexpr int k_planes(int kb) { return kb == 2 ? 2 : kb == 3 ? 4 : 8; }
__host__ __device__ constexpr int mfma_per_tile(int d, int kb = 3) { return (k_planes(kb) + 1) * (d / 128); }
__host__ __device__ inline size_t packed_group_bytes(int d, int kb = 3) {
  return (size_t)mfma_per_tile(d, kb) * (64 * 32 + 64 * 4) + 64;
}
constexpr int kMfmaMaxGroup = 4;   // query rows per MFMA query group (4 rows x 4 limbs)
__host__ __device__ inline int query_groups(int group) { return (group + kMfmaMaxGroup - 1) / kMfmaMaxGroup; }
// Most query groups one decode workgroup serves (1 or 2), by head_dim. At
// d = 128 two groups per workgroup keep two waves per SIMD (242 VGPRs) and
// share the key and V operands; at d = 256 two groups need more than 256
// registers (one wave per SIMD) and are slower than one group per workgroup.
__host__ __device__ inline int max_groups_per_wg(int d) { return d == 128 ? 2 : 1; }
// The MFMA decode kernel covers head_dim 128 and 256 with up to TQ_MAX_GROUP
// query rows per KV head, as query groups of 4 rows.
__host__ __device__ inline bool mfma_path(int d, int group) {
  return (d == 128 || d == 256) && group <= TQ_MAX_GROUP;
}
// Wide query groups: 16 distinct query rows per scoring MFMA (one fp6 limb of
// each row per MFMA, the four limbs accumulating in one result) and per V
// MFMA (weights as two int8 limbs, each with its own int32 sums), for 16 or
// more rows per KV head with 3-bit K and V codes. Packed operand of a wide
// group: per scoring MFMA mu and limb, 64 lanes x 32 bytes, then the scale
// words of the same operands (64 per operand), then 16 rows x {sum q~, sum p}.
constexpr int kWideRows = 16;
__host__ __device__ inline bool wide_path(int d, int group, int kb, int vb) {
  return mfma_path(d, group) && group >= kWideRows && kb == 3 && vb == 3;
}
__host__ __device__ inline size_t packed_group_bytes_wide(int d) {
  return (size_t)mfma_per_tile(d, 3) * 4 * (64 * 32 + 64 * 4) + kWideRows * 8;
}

// Split-K plan of one decode call.
struct DecodePlan {
  int group;              // query rows per (sequence, KV head) = Hq/Hkv * n_q
  bool wide;              // query groups of 16 rows (wide_path), else of 4
  int qgroups;            // MFMA query groups of 4 (or 16) rows (MFMA path)
  int groups_per_wg;      // query groups one decode workgroup serves: 1 or 2
  int wg_per_seq;         // decode workgroups per (split, KV head, sequence)
  int pages_per_split;
  int n_split;
  size_t partial_bytes;   // [B*Hkv][n_split][group] x (d + 4) float32
  size_t prep_bytes;      // query region (tq_attn_decode only)
  bool mfma;              // the shape is one the MFMA decode kernel covers
};

// Query region of a decode call: [rows][2][d] float32, then (MFMA path) the
// packed operands of the B*Hkv groups.
size_t prep_region_bytes(int d, int batch, int n_q, int n_q_heads, int n_kv_heads, int kb, int vb);
inline size_t prep_float_bytes(int d, int batch, int n_q, int n_q_heads) {
  return ((size_t)batch * n_q * n_q_heads * 2 * d * sizeof(float) + 255) / 256 * 256;
}

struct DecodeArgs {
  const uint8_t *k_pool;
  const uint8_t *v_pool;
  const float *prep;      // [B][n_q][Hq][2][d]
  const uint8_t *packed;  // packed scoring operands (MFMA path)
  const int32_t *block_table;
  int max_pages;
  const int32_t *seq_lens;
  const int32_t *seq_starts;  // first visible token per sequence (or null: 0)
  float *out;             // [B][n_q][Hq][d]
  float *partials;
  int batch, n_q, n_q_heads, n_kv_heads;
  int causal_tail;
  float scale;
  DecodePlan plan;
  Codebook cb;            // K, k_bits wide
  Codebook vcb;           // V, v_bits wide
  int k_bits, v_bits;
};

DecodePlan plan_decode(int d, int batch, int n_q, int n_q_heads, int n_kv_heads, int max_pages,
                       int kb, int vb);

hipError_t launch_encode_k(const EncodeArgs &a, int d, hipStream_t s);
hipError_t launch_encode_v(const EncodeArgs &a, int d, hipStream_t s);
hipError_t launch_dequant(const DequantArgs &a, int d, int which, hipStream_t s);
hipError_t launch_prepare(const PrepArgs &a, int d, hipStream_t s);
// Encode of a short append (k, v: same tokens and dtype) and the query prepare in
// one launch; false when the shapes need the separate kernels (long appends, or
// query and K/V in different dtypes).
bool step_prologue_fits(const EncodeArgs &k, const PrepArgs &p);
hipError_t launch_step_prologue(const EncodeArgs &k, const EncodeArgs &v, const PrepArgs &p, int d,
                                hipStream_t s);
hipError_t launch_decode_split(const DecodeArgs &a, int d, hipStream_t s);
// Merge of split partials; rotate = apply the inverse rotation (the compressed
// path accumulates in the rotated domain, the dense baseline does not).
hipError_t launch_decode_merge(const DecodeArgs &a, int d, hipStream_t s, bool rotate = true);

// Uncompressed bf16 baseline: K and V dense as [batch][Hkv][max_len][d].
struct DenseArgs {
  const uint16_t *k, *v;
  int max_len;
  const void *q;
  int q_dtype;
  const int32_t *seq_lens;
  int batch, n_q, n_q_heads, n_kv_heads;
  int tokens_per_split, n_split;
  float scale;
  float *partials;
};
hipError_t launch_dense_split(const DenseArgs &a, int d, hipStream_t s);

// The whole of tq_append_decode (checks, workspace sizing, launches), shared by
// the entry point with a caller workspace and the one with the static scratch.
int append_decode(const tq_cache *c, const void *k_new, const void *v_new, int32_t kv_dtype,
                  const int32_t *slots, int32_t n_new, const void *q, int32_t q_dtype,
                  int32_t batch, int32_t n_q, int32_t n_q_heads, const int32_t *block_table,
                  int32_t max_pages, const int32_t *seq_lens, int32_t causal_tail, float scale,
                  float *out, void *workspace, size_t *workspace_bytes, void *stream);

}  // namespace tq
