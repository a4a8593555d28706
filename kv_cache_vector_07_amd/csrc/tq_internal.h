// Internal interface between the C-ABI layer (tq_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

constexpr int kPage = TQ_PAGE_SIZE;

struct Codebook {
  float levels[8];
  float thresholds[7];
};

inline size_t k_section_bytes(int d) { return (size_t)kPage * d / 2 + 4u * kPage; }
inline size_t v_section_bytes(int d) { return (size_t)3 * d * kPage / 8 + 2u * kPage; }

struct EncodeArgs {
  const void *x;          // [n_tokens][H][d], float32 or bfloat16
  int dtype;
  const int32_t *slots;   // [n_tokens]
  int n_tokens;
  int n_heads;
  uint8_t *pool;          // K or V pool
  const float *qjl;       // S [d][d] (K only)
  Codebook cb;
};

struct DequantArgs {
  const uint8_t *pool;
  const int32_t *slots;
  int n_tokens;
  int n_heads;
  int with_qjl;
  const float *qjl;
  float *out;             // [n_tokens][H][d]
  Codebook cb;
};

struct PrepArgs {
  const void *q;          // [rows][d]
  int dtype;
  int rows;
  const float *qjl;
  float *prep;            // [rows][2][d]
};

// Split-K plan of one decode call.
struct DecodePlan {
  int group;              // query rows per (sequence, KV head) = Hq/Hkv * n_q
  int pages_per_split;
  int n_split;
  size_t counter_bytes;   // [B*Hkv] u32, padded
  size_t partial_bytes;   // [B*Hkv][n_split][group] x (d + 2) float32
  size_t prep_bytes;      // [B*n_q*Hq][2][d] float32 (tq_attn_decode only)
};

struct DecodeArgs {
  const uint8_t *k_pool;
  const uint8_t *v_pool;
  const float *prep;      // [B][n_q][Hq][2][d]
  const int32_t *block_table;
  int max_pages;
  const int32_t *seq_lens;
  float *out;             // [B][n_q][Hq][d]
  float *partials;
  uint32_t *counters;
  int batch, n_q, n_q_heads, n_kv_heads;
  int causal_tail;
  float scale;
  DecodePlan plan;
  Codebook cb;
};

DecodePlan plan_decode(int d, int batch, int n_q, int n_q_heads, int n_kv_heads, int max_pages);

hipError_t launch_encode_k(const EncodeArgs &a, int d, hipStream_t s);
hipError_t launch_encode_v(const EncodeArgs &a, int d, hipStream_t s);
hipError_t launch_dequant(const DequantArgs &a, int d, int which, hipStream_t s);
hipError_t launch_prepare(const PrepArgs &a, int d, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t s);

}  // namespace tq
