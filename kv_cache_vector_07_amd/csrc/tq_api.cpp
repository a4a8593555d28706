// C-ABI entry points: argument checks, the host-side codebook / QJL matrix,
// the decode split plan and workspace sizing. Device work lives in *.hip.
#include <math.h>

#include <algorithm>
#include <string.h>

#include "tq_internal.h"

using tq::Codebook;

namespace {

bool supported_dim(int d) { return d == 128 || d == 256; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_codebooks(const tq_cache *c);

int check_cache(const tq_cache *c) {
  if (!c) return TQ_EINVAL;
  if (c->head_dim <= 0 || c->n_kv_heads <= 0 || c->page_size <= 0 || c->n_pages <= 0)
    return TQ_EINVAL;
  if (!supported_dim(c->head_dim) || c->page_size != TQ_PAGE_SIZE) return TQ_EUNSUPPORTED;
  if (!c->k_pool || !c->v_pool) return TQ_EINVAL;
  if (!aligned(c->k_pool, 256) || !aligned(c->v_pool, 256)) return TQ_EALIGN;
  return check_codebooks(c);
}

// Code widths, key mode and codebooks of a descriptor (everything but the pools)
int check_codebooks(const tq_cache *c) {
  if (c->k_mse_only != 0 && c->k_mse_only != 1) return TQ_EINVAL;
  // the decode kernels split each level into odd bit-plane weights: the
  // codebooks must be strictly increasing and odd (c[n-1-k] = -c[k])
  auto odd_increasing = [](const float *lv, int n) {
    for (int k = 0; k < n; ++k) {
      if (!isfinite(lv[k]) || lv[n - 1 - k] != -lv[k]) return false;
      if (k > 0 && !(lv[k] > lv[k - 1])) return false;
    }
    return true;
  };
  // thresholds strictly increasing (the encoders locate a code by binary search)
  auto increasing = [](const float *t, int n) {
    for (int k = 0; k < n; ++k)
      if (!isfinite(t[k]) || (k > 0 && !(t[k] > t[k - 1]))) return false;
    return true;
  };
  if (!odd_increasing(c->levels, 8) || !increasing(c->thresholds, 7)) return TQ_EINVAL;
  if (c->v_bits != 0 && c->v_bits != 2 && c->v_bits != 3 && c->v_bits != 4) return TQ_EINVAL;
  if ((c->v_bits == 2 || c->v_bits == 4) &&
      (!odd_increasing(c->v_levels, 1 << c->v_bits) || !increasing(c->v_thresholds, (1 << c->v_bits) - 1)))
    return TQ_EINVAL;
  if (c->k_bits != 0 && c->k_bits != 2 && c->k_bits != 3 && c->k_bits != 4) return TQ_EINVAL;
  if ((c->k_bits == 2 || c->k_bits == 4) &&
      (!odd_increasing(c->k_levels, 1 << c->k_bits) || !increasing(c->k_thresholds, (1 << c->k_bits) - 1)))
    return TQ_EINVAL;
  return TQ_OK;
}

// K code width and codebook: 3-bit K uses levels / thresholds
int k_bits_of(const tq_cache *c) { return (c->k_bits == 2 || c->k_bits == 4) ? c->k_bits : 3; }
Codebook codebook_of(const tq_cache *c) {
  Codebook cb = {};
  if (k_bits_of(c) == 3) {
    memcpy(cb.levels, c->levels, sizeof c->levels);
    memcpy(cb.thresholds, c->thresholds, sizeof c->thresholds);
  } else {
    const int n = 1 << c->k_bits;
    memcpy(cb.levels, c->k_levels, sizeof(float) * n);
    memcpy(cb.thresholds, c->k_thresholds, sizeof(float) * (n - 1));
  }
  return cb;
}

// The 3-bit codebook in levels / thresholds (V at 3 bits uses it)
Codebook codebook3_of(const tq_cache *c) {
  Codebook cb = {};
  memcpy(cb.levels, c->levels, sizeof c->levels);
  memcpy(cb.thresholds, c->thresholds, sizeof c->thresholds);
  return cb;
}

// V code width and codebook: 3-bit V shares the K codebook
int v_bits_of(const tq_cache *c) { return (c->v_bits == 2 || c->v_bits == 4) ? c->v_bits : 3; }
Codebook v_codebook_of(const tq_cache *c) {
  if (v_bits_of(c) == 3) return codebook3_of(c);
  Codebook cb = {};
  const int n = 1 << c->v_bits;
  memcpy(cb.levels, c->v_levels, sizeof(float) * n);
  memcpy(cb.thresholds, c->v_thresholds, sizeof(float) * (n - 1));
  return cb;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_EHIP; }

// The QJL matrix as the key-side kernels see it: NULL for MSE-only keys, which
// makes the encoder skip z = S r and the query prologue write p = 0.
const float *qjl_of(const tq_cache *c) { return c->k_mse_only ? nullptr : c->qjl; }
bool qjl_missing(const tq_cache *c) { return !c->k_mse_only && !c->qjl; }

// ---- Lloyd-Max for N(0, sigma^2), float64 -------------------------------------
double std_pdf(double u) { return isinf(u) ? 0.0 : exp(-0.5 * u * u) / sqrt(2.0 * M_PI); }

// P(a < Z <= b), Z ~ N(0,1); upper-tail form when a >= 0 to avoid cancellation.
double std_mass(double a, double b) {
  auto upper = [](double x) { return 0.5 * erfc(x / M_SQRT2); };  // P(Z > x)
  if (a >= 0) return upper(a) - upper(b);
  return upper(-b) - upper(-a);
}

// Phi^-1(p) by bisection on erfc (only used for the starting levels).
double std_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    double cdf = 0.5 * erfc(-mid / M_SQRT2);
    (cdf < p ? lo : hi) = mid;
  }
  return 0.5 * (lo + hi);
}

// n levels (n <= 16) of N(0, sigma^2); c[n], t[n - 1]
void lloyd_max(double sigma, int n, double *c, double *t) {
  for (int k = 0; k < n; ++k) c[k] = sigma * std_quantile((k + 0.5) / n);
  for (int it = 0; it < 10000; ++it) {
    for (int k = 0; k + 1 < n; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    double delta = 0.0;
    for (int k = 0; k < n; ++k) {
      double a = k == 0 ? -INFINITY : t[k - 1] / sigma;
      double b = k == n - 1 ? INFINITY : t[k] / sigma;
      double nc = sigma * (std_pdf(a) - std_pdf(b)) / std_mass(a, b);
      delta = fmax(delta, fabs(nc - c[k]));
      c[k] = nc;
    }
    if (delta < 1e-14 * sigma) break;
  }
  double s[16];
  for (int k = 0; k < n; ++k) s[k] = 0.5 * (c[k] - c[n - 1 - k]);
  for (int k = 0; k < n; ++k) c[k] = s[k];
  for (int k = 0; k + 1 < n; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  t[n / 2 - 1] = 0.0;
}

// ---- Lloyd-Max for one coordinate of a uniform unit vector in R^d, float64 ----
// The density is proportional to (1 - x^2)^((d-3)/2) on (-1, 1). With x = sin u
// the mass of a cell (a, b) is proportional to the integral of cos^(d-2) u over
// (asin a, asin b), a smooth integrand, taken here by composite 8-point
// Gauss-Legendre; the first moment has the closed form
// ((1 - a^2)^((d-1)/2) - (1 - b^2)^((d-1)/2)) / (d - 1) in the same units, so
// the normalising constant cancels in the centroid.
double sphere_mass(int d, double a, double b) {
  static const double xg[4] = {0.1834346424956498, 0.5255324099163290, 0.7966664774136267,
                               0.9602898564975363};
  static const double wg[4] = {0.3626837833783620, 0.3137066458778873, 0.2223810344533745,
                               0.1012285362903763};
  const int panels = 128;
  const double u0 = asin(fmax(-1.0, fmin(1.0, a))), u1 = asin(fmax(-1.0, fmin(1.0, b)));
  const double h = (u1 - u0) / panels;
  double sum = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double mid = u0 + (p + 0.5) * h;
    for (int k = 0; k < 4; ++k) {
      sum += wg[k] * pow(cos(mid - 0.5 * h * xg[k]), d - 2);
      sum += wg[k] * pow(cos(mid + 0.5 * h * xg[k]), d - 2);
    }
  }
  return 0.5 * h * sum;
}

double sphere_moment(int d, double a, double b) {
  auto F = [d](double x) {
    x = fmax(-1.0, fmin(1.0, x));
    return pow(1.0 - x * x, 0.5 * (d - 1)) / (d - 1);
  };
  return F(a) - F(b);
}

void lloyd_max_sphere(int d, int n, double *c, double *t) {
  lloyd_max(1.0 / sqrt((double)d), n, c, t);
  for (int k = 0; k < n; ++k) c[k] = fmax(-0.999, fmin(0.999, c[k]));
  double scale = 0.0;
  for (int k = 0; k < n; ++k) scale = fmax(scale, fabs(c[k]));
  for (int it = 0; it < 20000; ++it) {
    for (int k = 0; k + 1 < n; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    double delta = 0.0;
    for (int k = 0; k < n; ++k) {
      const double a = k == 0 ? -1.0 : t[k - 1];
      const double b = k == n - 1 ? 1.0 : t[k];
      const double nc = sphere_moment(d, a, b) / sphere_mass(d, a, b);
      delta = fmax(delta, fabs(nc - c[k]));
      c[k] = nc;
    }
    if (delta < 1e-14 * scale) break;
  }
  double s[16];
  for (int k = 0; k < n; ++k) s[k] = 0.5 * (c[k] - c[n - 1 - k]);
  for (int k = 0; k < n; ++k) c[k] = s[k];
  for (int k = 0; k + 1 < n; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  t[n / 2 - 1] = 0.0;
}

uint64_t splitmix64_next(uint64_t &state) {
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

namespace tq {

DecodePlan plan_decode(int d, int batch, int n_q, int n_q_heads, int n_kv_heads, int max_pages,
                       int kb, int vb) {
  DecodePlan p;
  p.group = n_q_heads / n_kv_heads * n_q;
  p.mfma = mfma_path(d, p.group);
  p.wide = wide_path(d, p.group, kb, vb);
  p.qgroups = !p.mfma ? 1 : p.wide ? (p.group + kWideRows - 1) / kWideRows : query_groups(p.group);
  // Several 4-row query groups of a (sequence, KV head) share a workgroup, so
  // the key and V operands of a block are built once for all of them; a wide
  // group has a workgroup of its own.
  p.groups_per_wg = p.qgroups > 1 && !p.wide ? max_groups_per_wg(d) : 1;
  p.wg_per_seq = (p.qgroups + p.groups_per_wg - 1) / p.groups_per_wg;
  // About 512 workgroups (two per CU, one occupancy round), or 768 for the
  // one-group kernel at d = 128 (three per CU), so that every workgroup streams
  // several pages with its loads overlapped; whole pages per split; at most 256
  // pages (65536 tokens) per split.
  const long target = d == 128 && !p.wide && p.groups_per_wg == 1 ? 768 : 512;
  long work = (long)batch * n_kv_heads * max_pages * p.wg_per_seq;
  int pps = (int)((work + target - 1) / target);
  if (pps < 1) pps = 1;
  if (pps > 256) pps = 256;
  p.pages_per_split = pps;
  p.n_split = (max_pages + pps - 1) / pps;
  p.partial_bytes =
      round_up((size_t)batch * n_kv_heads * p.n_split * p.group * (d + 4) * sizeof(float), 256);
  p.prep_bytes = prep_region_bytes(d, batch, n_q, n_q_heads, n_kv_heads, kb, vb);
  return p;
}

}  // namespace tq

extern "C" {

size_t tq_k_page_bytes(int32_t head_dim, int32_t page_size) {
  return tq_k_page_bytes_bits(head_dim, page_size, 3);
}

size_t tq_k_page_bytes_bits(int32_t head_dim, int32_t page_size, int32_t bits) {
  if (head_dim <= 0 || head_dim % 32 || page_size <= 0 || page_size % 32) return 0;
  if (bits < 2 || bits > 4) return 0;
  return (size_t)page_size * (bits + 1) * head_dim / 8 + 4u * page_size;
}

size_t tq_v_page_bytes(int32_t head_dim, int32_t page_size) {
  return tq_v_page_bytes_bits(head_dim, page_size, 3);
}

size_t tq_v_page_bytes_bits(int32_t head_dim, int32_t page_size, int32_t bits) {
  if (head_dim <= 0 || head_dim % 32 || page_size <= 0 || page_size % 32) return 0;
  if (bits < 2 || bits > 4) return 0;
  return (size_t)bits * head_dim * page_size / 8 + 2u * page_size;
}

const char *tq_status_string(int32_t s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_EALIGN: return "misaligned buffer";
    case TQ_EWORKSPACE: return "workspace too small";
    case TQ_EHIP: return "HIP runtime error";
    case TQ_ESCRATCH: return "needs more than the static scratch (TQ_STATIC_SCRATCH_BYTES) holds";
    default: return "unknown status";
  }
}

static void build_qjl(int32_t head_dim, uint64_t qjl_seed, float *qjl_host) {
  uint64_t state = qjl_seed;
  const size_t n = (size_t)head_dim * head_dim;
  for (size_t i = 0; i < n; i += 2) {
    uint64_t x1 = splitmix64_next(state), x2 = splitmix64_next(state);
    double u1 = (double)((x1 >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)((x2 >> 11) + 1) * 0x1.0p-53;
    double rad = sqrt(-2.0 * log(u1));
    double ang = 2.0 * M_PI * u2;
    qjl_host[i] = (float)(rad * cos(ang));
    if (i + 1 < n) qjl_host[i + 1] = (float)(rad * sin(ang));
  }
}

int tq_build_codebook(int32_t head_dim, int32_t bits, uint64_t qjl_seed, float *levels,
                      float *thresholds, float *qjl_host) {
  if (!levels || !thresholds) return TQ_EINVAL;
  if (head_dim < 2 || (head_dim & (head_dim - 1))) return TQ_EINVAL;
  if (bits < 2 || bits > 4) return TQ_EUNSUPPORTED;
  const int n = 1 << bits;
  double c[16], t[15];
  lloyd_max(1.0 / sqrt((double)head_dim), n, c, t);
  for (int k = 0; k < n; ++k) levels[k] = (float)c[k];
  for (int k = 0; k + 1 < n; ++k) thresholds[k] = (float)t[k];
  if (qjl_host) build_qjl(head_dim, qjl_seed, qjl_host);
  return TQ_OK;
}

int tq_build_codebook_sphere(int32_t head_dim, int32_t bits, uint64_t qjl_seed, float *levels,
                             float *thresholds, float *qjl_host) {
  if (!levels || !thresholds) return TQ_EINVAL;
  if (head_dim < 4 || (head_dim & (head_dim - 1))) return TQ_EINVAL;
  if (bits < 2 || bits > 4) return TQ_EUNSUPPORTED;
  const int n = 1 << bits;
  double c[16], t[15];
  lloyd_max_sphere(head_dim, n, c, t);
  for (int k = 0; k < n; ++k) levels[k] = (float)c[k];
  for (int k = 0; k + 1 < n; ++k) thresholds[k] = (float)t[k];
  if (qjl_host) build_qjl(head_dim, qjl_seed, qjl_host);
  return TQ_OK;
}

static int encode_common(const tq_cache *c, const void *x, int32_t dtype, const int32_t *slots,
                         int32_t n_tokens, void *stream, bool is_k) {
  int st = check_cache(c);
  if (st) return st;
  if (n_tokens < 0) return TQ_EINVAL;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_EUNSUPPORTED;
  if (n_tokens == 0) return TQ_OK;
  if (!x || !slots || (is_k && qjl_missing(c))) return TQ_EINVAL;
  if (!aligned(x, 16) || !aligned(slots, 4) || (is_k && !aligned(qjl_of(c), 16))) return TQ_EALIGN;
  tq::EncodeArgs a;
  a.x = x;
  a.dtype = dtype;
  a.slots = slots;
  a.n_tokens = n_tokens;
  a.n_heads = c->n_kv_heads;
  a.pool = (uint8_t *)(is_k ? c->k_pool : c->v_pool);
  a.qjl = qjl_of(c);
  a.cb = is_k ? codebook_of(c) : v_codebook_of(c);
  a.bits = is_k ? k_bits_of(c) : v_bits_of(c);
  hipStream_t s = (hipStream_t)stream;
  return hip_status(is_k ? tq::launch_encode_k(a, c->head_dim, s)
                         : tq::launch_encode_v(a, c->head_dim, s));
}

int tq_encode_k(const tq_cache *c, const void *k, int32_t dtype, const int32_t *slots,
                int32_t n_tokens, void *stream) {
  return encode_common(c, k, dtype, slots, n_tokens, stream, true);
}

int tq_encode_v(const tq_cache *c, const void *v, int32_t dtype, const int32_t *slots,
                int32_t n_tokens, void *stream) {
  return encode_common(c, v, dtype, slots, n_tokens, stream, false);
}

// The decode grids are (splits, Hkv, batch x workgroups per sequence) and the
// merge grid (rows, Hkv, batch); the second and third dimensions stay within
// 65535.
static bool grid_fits(const tq_cache *c, int32_t batch, int32_t n_q, int32_t n_q_heads) {
  const tq::DecodePlan p = tq::plan_decode(c->head_dim, batch, n_q, n_q_heads, c->n_kv_heads, 1,
                                           k_bits_of(c), v_bits_of(c));
  return c->n_kv_heads <= 65535 && (long)batch * p.wg_per_seq <= 65535;
}

static int prepare_checks(const tq_cache *c, int32_t dtype, int32_t batch, int32_t n_q,
                          int32_t n_q_heads) {
  if (!c) return TQ_EINVAL;
  if (c->head_dim <= 0 || c->n_kv_heads <= 0) return TQ_EINVAL;
  if (int st = check_codebooks(c)) return st;
  if (!supported_dim(c->head_dim)) return TQ_EUNSUPPORTED;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_EUNSUPPORTED;
  if (batch <= 0 || n_q <= 0 || n_q_heads <= 0 || n_q_heads % c->n_kv_heads) return TQ_EINVAL;
  if (n_q_heads / c->n_kv_heads * n_q > TQ_MAX_GROUP) return TQ_EUNSUPPORTED;
  if (!grid_fits(c, batch, n_q, n_q_heads)) return TQ_EUNSUPPORTED;
  return TQ_OK;
}

static hipError_t run_prepare(const tq_cache *c, const void *q, int32_t dtype, int32_t batch,
                              int32_t n_q, int32_t n_q_heads, uint8_t *prep, hipStream_t s) {
  tq::PrepArgs a;
  a.q = q;
  a.dtype = dtype;
  a.batch = batch;
  a.n_q = n_q;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = c->n_kv_heads;
  a.qjl = qjl_of(c);
  a.prep = (float *)prep;
  const int group = n_q_heads / c->n_kv_heads * n_q;
  const bool mfma = tq::mfma_path(c->head_dim, group);
  a.packed = mfma ? prep + tq::prep_float_bytes(c->head_dim, batch, n_q, n_q_heads) : nullptr;
  a.wide = tq::wide_path(c->head_dim, group, k_bits_of(c), v_bits_of(c));
  a.cb = codebook_of(c);
  a.k_bits = k_bits_of(c);
  return tq::launch_prepare(a, c->head_dim, s);
}

int tq_query_prepare(const tq_cache *c, const void *q, int32_t dtype, int32_t batch, int32_t n_q,
                     int32_t n_q_heads, void *prep, size_t *prep_bytes, void *stream) {
  int st = prepare_checks(c, dtype, batch, n_q, n_q_heads);
  if (st) return st;
  if (!prep_bytes) return TQ_EINVAL;
  const size_t need =
      tq::prep_region_bytes(c->head_dim, batch, n_q, n_q_heads, c->n_kv_heads, k_bits_of(c),
                            v_bits_of(c));
  if (!prep) {
    *prep_bytes = need;
    return TQ_OK;
  }
  if (*prep_bytes < need) {
    *prep_bytes = need;
    return TQ_EWORKSPACE;
  }
  if (!q || qjl_missing(c)) return TQ_EINVAL;
  if (!aligned(q, 16) || !aligned(prep, 256) || !aligned(qjl_of(c), 16)) return TQ_EALIGN;
  return hip_status(run_prepare(c, q, dtype, batch, n_q, n_q_heads, (uint8_t *)prep,
                                (hipStream_t)stream));
}

static int decode_checks(const tq_cache *c, int32_t batch, int32_t n_q, int32_t n_q_heads,
                         const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens,
                         int32_t causal_tail, float *out, size_t *workspace_bytes) {
  int st = check_cache(c);
  if (st) return st;
  if (!workspace_bytes) return TQ_EINVAL;
  if (batch <= 0 || n_q <= 0 || n_q_heads <= 0 || max_pages <= 0) return TQ_EINVAL;
  if (n_q_heads % c->n_kv_heads) return TQ_EINVAL;
  if (causal_tail != 0 && causal_tail != 1) return TQ_EINVAL;
  if (n_q_heads / c->n_kv_heads * n_q > TQ_MAX_GROUP) return TQ_EUNSUPPORTED;
  if (!grid_fits(c, batch, n_q, n_q_heads)) return TQ_EUNSUPPORTED;
  if (!block_table || !seq_lens || !out || qjl_missing(c)) return TQ_EINVAL;
  if (!aligned(out, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4)) return TQ_EALIGN;
  return TQ_OK;
}

static tq::DecodeArgs decode_args(const tq_cache *c, const uint8_t *prep, int32_t batch,
                                  int32_t n_q, int32_t n_q_heads, const int32_t *block_table,
                                  int32_t max_pages, const int32_t *seq_lens, int32_t causal_tail,
                                  float scale, float *out, uint8_t *ws,
                                  const tq::DecodePlan &plan) {
  tq::DecodeArgs a;
  a.k_pool = (const uint8_t *)c->k_pool;
  a.v_pool = (const uint8_t *)c->v_pool;
  a.prep = (const float *)prep;
  a.packed = prep ? prep + tq::prep_float_bytes(c->head_dim, batch, n_q, n_q_heads) : nullptr;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.seq_starts = nullptr;
  a.out = out;
  a.partials = (float *)ws;
  a.batch = batch;
  a.n_q = n_q;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = c->n_kv_heads;
  a.causal_tail = causal_tail;
  a.scale = scale;
  a.plan = plan;
  a.cb = codebook_of(c);
  a.vcb = v_codebook_of(c);
  a.k_bits = k_bits_of(c);
  a.v_bits = v_bits_of(c);
  return a;
}

static int decode_run(const tq_cache *c, const uint8_t *prep, int32_t batch, int32_t n_q,
                      int32_t n_q_heads, const int32_t *block_table, int32_t max_pages,
                      const int32_t *seq_lens, int32_t causal_tail, float scale, float *out,
                      uint8_t *ws, const tq::DecodePlan &plan, hipStream_t s,
                      const int32_t *seq_starts = nullptr) {
  tq::DecodeArgs a = decode_args(c, prep, batch, n_q, n_q_heads, block_table, max_pages,
                                 seq_lens, causal_tail, scale, out, ws, plan);
  a.seq_starts = seq_starts;
  if (tq::launch_decode_split(a, c->head_dim, s) != hipSuccess) return TQ_EHIP;
  return hip_status(tq::launch_decode_merge(a, c->head_dim, s));
}

static int attn_decode_impl(const tq_cache *c, const void *q, int32_t dtype, int32_t batch,
                            int32_t n_q, int32_t n_q_heads, const int32_t *block_table,
                            int32_t max_pages, const int32_t *seq_lens, const int32_t *seq_starts,
                            int32_t causal_tail, float scale, float *out, void *workspace,
                            size_t *workspace_bytes, void *stream) {
  int st = decode_checks(c, batch, n_q, n_q_heads, block_table, max_pages, seq_lens, causal_tail,
                         out, workspace_bytes);
  if (st) return st;
  if (seq_starts && !aligned(seq_starts, 4)) return TQ_EALIGN;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_EUNSUPPORTED;
  tq::DecodePlan plan =
      tq::plan_decode(c->head_dim, batch, n_q, n_q_heads, c->n_kv_heads, max_pages,
                      k_bits_of(c), v_bits_of(c));
  size_t need = plan.partial_bytes + plan.prep_bytes;
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return TQ_EWORKSPACE;
  }
  if (!q) return TQ_EINVAL;
  if (!aligned(q, 16) || !aligned(workspace, 256)) return TQ_EALIGN;
  uint8_t *ws = (uint8_t *)workspace;
  uint8_t *prep = ws + plan.partial_bytes;
  hipStream_t s = (hipStream_t)stream;
  if (run_prepare(c, q, dtype, batch, n_q, n_q_heads, prep, s) != hipSuccess) return TQ_EHIP;
  return decode_run(c, prep, batch, n_q, n_q_heads, block_table, max_pages, seq_lens, causal_tail,
                    scale, out, ws, plan, s, seq_starts);
}

int tq_attn_decode(const tq_cache *c, const void *q, int32_t dtype, int32_t batch, int32_t n_q,
                   int32_t n_q_heads, const int32_t *block_table, int32_t max_pages,
                   const int32_t *seq_lens, int32_t causal_tail, float scale, float *out,
                   void *workspace, size_t *workspace_bytes, void *stream) {
  return attn_decode_impl(c, q, dtype, batch, n_q, n_q_heads, block_table, max_pages, seq_lens,
                          nullptr, causal_tail, scale, out, workspace, workspace_bytes, stream);
}

int tq_attn_decode_window(const tq_cache *c, const void *q, int32_t dtype, int32_t batch,
                          int32_t n_q, int32_t n_q_heads, const int32_t *block_table,
                          int32_t max_pages, const int32_t *seq_lens, const int32_t *seq_starts,
                          int32_t causal_tail, float scale, float *out, void *workspace,
                          size_t *workspace_bytes, void *stream) {
  if (!seq_starts) return TQ_EINVAL;
  return attn_decode_impl(c, q, dtype, batch, n_q, n_q_heads, block_table, max_pages, seq_lens,
                          seq_starts, causal_tail, scale, out, workspace, workspace_bytes, stream);
}

int tq_append_decode(const tq_cache *c, const void *k_new, const void *v_new, int32_t kv_dtype,
                     const int32_t *slots, int32_t n_new, const void *q, int32_t q_dtype,
                     int32_t batch, int32_t n_q, int32_t n_q_heads, const int32_t *block_table,
                     int32_t max_pages, const int32_t *seq_lens, int32_t causal_tail, float scale,
                     float *out, void *workspace, size_t *workspace_bytes, void *stream) {
  return tq::append_decode(c, k_new, v_new, kv_dtype, slots, n_new, q, q_dtype, batch, n_q,
                           n_q_heads, block_table, max_pages, seq_lens, causal_tail, scale, out,
                           workspace, workspace_bytes, stream);
}

}  // extern "C"

int tq::append_decode(const tq_cache *c, const void *k_new, const void *v_new, int32_t kv_dtype,
                      const int32_t *slots, int32_t n_new, const void *q, int32_t q_dtype,
                      int32_t batch, int32_t n_q, int32_t n_q_heads, const int32_t *block_table,
                      int32_t max_pages, const int32_t *seq_lens, int32_t causal_tail, float scale,
                      float *out, void *workspace, size_t *workspace_bytes, void *stream) {
  int st = decode_checks(c, batch, n_q, n_q_heads, block_table, max_pages, seq_lens, causal_tail,
                         out, workspace_bytes);
  if (st) return st;
  if (kv_dtype != TQ_F32 && kv_dtype != TQ_BF16) return TQ_EUNSUPPORTED;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_EUNSUPPORTED;
  if (n_new < 0) return TQ_EINVAL;
  tq::DecodePlan plan =
      tq::plan_decode(c->head_dim, batch, n_q, n_q_heads, c->n_kv_heads, max_pages,
                      k_bits_of(c), v_bits_of(c));
  size_t need = plan.partial_bytes + plan.prep_bytes;
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return TQ_EWORKSPACE;
  }
  if (!q || qjl_missing(c)) return TQ_EINVAL;
  if (n_new > 0 && (!k_new || !v_new || !slots)) return TQ_EINVAL;
  if (!aligned(q, 16) || !aligned(workspace, 256) || !aligned(qjl_of(c), 16)) return TQ_EALIGN;
  if (n_new > 0 && (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slots, 4)))
    return TQ_EALIGN;
  uint8_t *ws = (uint8_t *)workspace;
  uint8_t *prep = ws + plan.partial_bytes;
  hipStream_t s = (hipStream_t)stream;

  tq::EncodeArgs ek, ev;
  ek.x = k_new;
  ek.dtype = kv_dtype;
  ek.slots = slots;
  ek.n_tokens = n_new;
  ek.n_heads = c->n_kv_heads;
  ek.pool = (uint8_t *)c->k_pool;
  ek.qjl = qjl_of(c);
  ek.cb = codebook_of(c);
  ek.bits = k_bits_of(c);
  ev = ek;
  ev.x = v_new;
  ev.pool = (uint8_t *)c->v_pool;
  ev.cb = v_codebook_of(c);
  ev.bits = v_bits_of(c);
  tq::PrepArgs pa;
  pa.q = q;
  pa.dtype = q_dtype;
  pa.batch = batch;
  pa.n_q = n_q;
  pa.n_q_heads = n_q_heads;
  pa.n_kv_heads = c->n_kv_heads;
  pa.qjl = qjl_of(c);
  pa.prep = (float *)prep;
  pa.packed = prep + tq::prep_float_bytes(c->head_dim, batch, n_q, n_q_heads);
  pa.wide = plan.wide;
  pa.cb = codebook_of(c);
  pa.k_bits = k_bits_of(c);
  if (n_new > 0 && tq::step_prologue_fits(ek, pa)) {
    if (tq::launch_step_prologue(ek, ev, pa, c->head_dim, s) != hipSuccess) return TQ_EHIP;
  } else {
    if (n_new > 0 && (tq::launch_encode_k(ek, c->head_dim, s) != hipSuccess ||
                      tq::launch_encode_v(ev, c->head_dim, s) != hipSuccess))
      return TQ_EHIP;
    if (tq::launch_prepare(pa, c->head_dim, s) != hipSuccess) return TQ_EHIP;
  }
  return decode_run(c, prep, batch, n_q, n_q_heads, block_table, max_pages, seq_lens, causal_tail,
                    scale, out, ws, plan, s);
}

extern "C" {

int tq_attn_decode_prepared(const tq_cache *c, const void *prep, int32_t batch, int32_t n_q,
                            int32_t n_q_heads, const int32_t *block_table, int32_t max_pages,
                            const int32_t *seq_lens, int32_t causal_tail, float scale, float *out,
                            void *workspace, size_t *workspace_bytes, void *stream) {
  int st = decode_checks(c, batch, n_q, n_q_heads, block_table, max_pages, seq_lens, causal_tail,
                         out, workspace_bytes);
  if (st) return st;
  tq::DecodePlan plan =
      tq::plan_decode(c->head_dim, batch, n_q, n_q_heads, c->n_kv_heads, max_pages,
                      k_bits_of(c), v_bits_of(c));
  size_t need = plan.partial_bytes;
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return TQ_EWORKSPACE;
  }
  if (!prep) return TQ_EINVAL;
  if (!aligned(prep, 256) || !aligned(workspace, 256)) return TQ_EALIGN;
  return decode_run(c, (const uint8_t *)prep, batch, n_q, n_q_heads, block_table, max_pages, seq_lens, causal_tail,
                    scale, out, (uint8_t *)workspace, plan, (hipStream_t)stream);
}

int tq_attn_decode_split(const tq_cache *c, const void *prep, int32_t batch, int32_t n_q,
                         int32_t n_q_heads, const int32_t *block_table, int32_t max_pages,
                         const int32_t *seq_lens, int32_t causal_tail, float scale,
                         void *workspace, size_t *workspace_bytes, void *stream) {
  float dummy_out[4] __attribute__((aligned(16)));
  int st = decode_checks(c, batch, n_q, n_q_heads, block_table, max_pages, seq_lens, causal_tail,
                         dummy_out, workspace_bytes);
  if (st) return st;
  tq::DecodePlan plan =
      tq::plan_decode(c->head_dim, batch, n_q, n_q_heads, c->n_kv_heads, max_pages,
                      k_bits_of(c), v_bits_of(c));
  size_t need = plan.partial_bytes;
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return TQ_EWORKSPACE;
  }
  if (!prep) return TQ_EINVAL;
  if (!aligned(prep, 256) || !aligned(workspace, 256)) return TQ_EALIGN;
  tq::DecodeArgs a = decode_args(c, (const uint8_t *)prep, batch, n_q, n_q_heads, block_table,
                                 max_pages, seq_lens, causal_tail, scale, nullptr,
                                 (uint8_t *)workspace, plan);
  return hip_status(tq::launch_decode_split(a, c->head_dim, (hipStream_t)stream));
}

int tq_attn_decode_merge(const tq_cache *c, int32_t batch, int32_t n_q, int32_t n_q_heads,
                         int32_t max_pages, float *out, const void *workspace,
                         size_t workspace_bytes, void *stream) {
  int st = check_cache(c);
  if (st) return st;
  if (batch <= 0 || n_q <= 0 || n_q_heads <= 0 || max_pages <= 0) return TQ_EINVAL;
  if (n_q_heads % c->n_kv_heads) return TQ_EINVAL;
  if (n_q_heads / c->n_kv_heads * n_q > TQ_MAX_GROUP) return TQ_EUNSUPPORTED;
  if (!grid_fits(c, batch, n_q, n_q_heads)) return TQ_EUNSUPPORTED;
  if (!out || !workspace) return TQ_EINVAL;
  if (!aligned(out, 16) || !aligned(workspace, 256)) return TQ_EALIGN;
  tq::DecodePlan plan =
      tq::plan_decode(c->head_dim, batch, n_q, n_q_heads, c->n_kv_heads, max_pages,
                      k_bits_of(c), v_bits_of(c));
  if (workspace_bytes < plan.partial_bytes) return TQ_EWORKSPACE;
  tq::DecodeArgs a = decode_args(c, nullptr, batch, n_q, n_q_heads, nullptr, max_pages, nullptr, 0,
                                 0.f, out, (uint8_t *)workspace, plan);
  return hip_status(tq::launch_decode_merge(a, c->head_dim, (hipStream_t)stream));
}

int tq_dense_attn_decode(const void *k, const void *v, int32_t head_dim, int32_t n_kv_heads,
                         int32_t max_len, const void *q, int32_t q_dtype, int32_t batch,
                         int32_t n_q, int32_t n_q_heads, const int32_t *seq_lens, float scale,
                         float *out, void *workspace, size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes) return TQ_EINVAL;
  if (head_dim <= 0 || n_kv_heads <= 0 || max_len <= 0 || batch <= 0 || n_q <= 0 ||
      n_q_heads <= 0 || n_q_heads % n_kv_heads)
    return TQ_EINVAL;
  if (!supported_dim(head_dim) || (q_dtype != TQ_F32 && q_dtype != TQ_BF16)) return TQ_EUNSUPPORTED;
  const int group = n_q_heads / n_kv_heads * n_q;
  if (group > tq::kMfmaMaxGroup) return TQ_EUNSUPPORTED;
  // about 512 workgroups, whole 256-token ranges per split
  const long work = (long)batch * n_kv_heads * ((max_len + 255) / 256);
  const int tps = (int)std::max(1L, (work + 511) / 512) * 256;
  const int n_split = (max_len + tps - 1) / tps;
  const size_t need =
      round_up((size_t)batch * n_kv_heads * n_split * group * (head_dim + 4) * sizeof(float), 256);
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return TQ_EWORKSPACE;
  }
  if (!k || !v || !q || !seq_lens || !out) return TQ_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(q, 16) || !aligned(out, 16) ||
      !aligned(workspace, 256))
    return TQ_EALIGN;
  tq::DenseArgs da;
  da.k = (const uint16_t *)k;
  da.v = (const uint16_t *)v;
  da.max_len = max_len;
  da.q = q;
  da.q_dtype = q_dtype;
  da.seq_lens = seq_lens;
  da.batch = batch;
  da.n_q = n_q;
  da.n_q_heads = n_q_heads;
  da.n_kv_heads = n_kv_heads;
  da.tokens_per_split = tps;
  da.n_split = n_split;
  da.scale = scale;
  da.partials = (float *)workspace;
  hipStream_t s = (hipStream_t)stream;
  if (tq::launch_dense_split(da, head_dim, s) != hipSuccess) return TQ_EHIP;
  tq::DecodeArgs ma = {};
  ma.partials = (float *)workspace;
  ma.out = out;
  ma.batch = batch;
  ma.n_q = n_q;
  ma.n_q_heads = n_q_heads;
  ma.n_kv_heads = n_kv_heads;
  ma.plan.group = group;
  ma.plan.n_split = n_split;
  ma.plan.qgroups = 1;
  ma.plan.groups_per_wg = 1;
  ma.plan.wg_per_seq = 1;
  return hip_status(tq::launch_decode_merge(ma, head_dim, s, false));
}

int tq_dequant(const tq_cache *c, int32_t which, int32_t with_qjl, const int32_t *slots,
               int32_t n_tokens, float *out, void *stream) {
  int st = check_cache(c);
  if (st) return st;
  if ((which != 0 && which != 1) || (with_qjl != 0 && with_qjl != 1) || n_tokens < 0)
    return TQ_EINVAL;
  if (n_tokens == 0) return TQ_OK;
  if (!slots || !out || (which == 0 && with_qjl && (c->k_mse_only || !c->qjl))) return TQ_EINVAL;
  if (!aligned(out, 16) || !aligned(slots, 4)) return TQ_EALIGN;
  tq::DequantArgs a;
  a.pool = (const uint8_t *)(which == 0 ? c->k_pool : c->v_pool);
  a.slots = slots;
  a.n_tokens = n_tokens;
  a.n_heads = c->n_kv_heads;
  a.with_qjl = which == 0 ? with_qjl : 0;
  a.qjl = c->qjl;
  a.out = out;
  a.cb = which == 0 ? codebook_of(c) : v_codebook_of(c);
  a.bits = which == 0 ? k_bits_of(c) : v_bits_of(c);
  return hip_status(tq::launch_dequant(a, c->head_dim, which, (hipStream_t)stream));
}

}  // extern "C"
