// tq_append_decode_static: the decode step of tq_append_decode with its
// workspace (split partials, prepared queries) in a static device buffer, for
// callers that cannot allocate. The kernels are those of tq_append_decode; they
// receive the buffer's device address like any caller workspace.
#include <mutex>

#include "tq_internal.h"

namespace {

// One copy per GPU the library runs on, held until the process ends. From host
// code only its looked-up device address is used, never this name.
static __device__ __align__(256) unsigned char scratch[TQ_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device

// The device address of the current device's scratch, looked up on the first
// call on that device (with it current) and kept.
int scratch_of_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_EHIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return TQ_OK;
}

}  // namespace

extern "C" int tq_append_decode_static(const tq_cache *c, const void *k_new, const void *v_new,
                                       int32_t kv_dtype, const int32_t *slots, int32_t n_new,
                                       const void *q, int32_t q_dtype, int32_t batch, int32_t n_q,
                                       int32_t n_q_heads, const int32_t *block_table,
                                       int32_t max_pages, const int32_t *seq_lens,
                                       int32_t causal_tail, float scale, float *out, void *stream) {
  // the size first: a request the buffer cannot hold launches nothing
  size_t need = 0;
  int st = tq::append_decode(c, k_new, v_new, kv_dtype, slots, n_new, q, q_dtype, batch, n_q,
                             n_q_heads, block_table, max_pages, seq_lens, causal_tail, scale, out,
                             nullptr, &need, stream);
  if (st) return st;
  if (need > TQ_STATIC_SCRATCH_BYTES) return TQ_ESCRATCH;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st) return st;
  size_t have = TQ_STATIC_SCRATCH_BYTES;
  return tq::append_decode(c, k_new, v_new, kv_dtype, slots, n_new, q, q_dtype, batch, n_q,
                           n_q_heads, block_table, max_pages, seq_lens, causal_tail, scale, out, ws,
                           &have, stream);
}
