// Host side of the TurboQuant packed-page KV library: the C ABI declared in
// include/tq.h, argument validation, the context (rotation signs and
// Lloyd-Max codebooks computed on the host), and work-split selection for
// the decode kernels.
//
// Sources: TurboQuant documentation pages "vLLM Usage" (sections "TQ Byte
// Layout", "Slot Mapping", "TQ Packed Page Contract"), "vLLM Reference
// Audit" (Feature Checklist: Lloyd-Max codebooks with the exact Beta law,
// RHT transforms, 1..5-bit packing) and "Architecture" ("Cache Storage
// Objects", "Diagnostic vs Serving Paths").

#include "tq.h"
#include "tq_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

using tq::kHeadDim;

struct tq_ctx {
  int head_dim;
  uint64_t seed;
  int8_t signs[kHeadDim];
  uint32_t sign_bits[kHeadDim / 32];
  float cent[6][32];     // [bits][j], bits 1..5
  float bound[6][31];
  float tab_scale[6];    // fp16-friendly scale of the centroid tables per bits
};

namespace {

thread_local int g_last_hip_error = 0;

tq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return TQ_OK;
  g_last_hip_error = static_cast<int>(e);
  return TQ_ERR_HIP;
}

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): the rotation's sign source.
uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// ---------------------------------------------------------------------------
// Lloyd-Max codebook of the coordinate law of a uniform unit vector in R^d:
// f(x) = K (1 - x^2)^m on [-1, 1], m = (d - 3) / 2, in long double.
//
// Cell masses use the antiderivative J_m(x) = int_0^x (1 - t^2)^m dt from the
// recursion (2m + 1) J_m = x (1 - x^2)^m + 2m J_{m-1}, started at
// J_0 = x (integer m) or J_{-1/2} = asin(x) (half-integer m).  First moments
// are closed form: int x (1 - x^2)^m = -(1 - x^2)^(m+1) / (2(m + 1)).
class CoordinateLaw {
 public:
  explicit CoordinateLaw(int d) : d_(d), m_((d - 3) / 2.0L) {
    logK_ = lgammal(d / 2.0L) - 0.5L * logl(3.14159265358979323846264338327950288L) -
            lgammal((d - 1) / 2.0L);
    half_integer_ = (d % 2) == 0;  // m = (d-3)/2 is half-integer for even d
  }

  long double J(long double x) const {
    long double w = 1.0L - x * x;
    if (w < 0) w = 0;
    long double mm, val, pw;
    if (half_integer_) {
      mm = -0.5L;
      val = asinl(x);
      pw = sqrtl(w);  // w^(mm + 1)
    } else {
      mm = 0.0L;
      val = x;
      pw = w;
    }
    while (mm < m_ - 0.25L) {
      mm += 1.0L;
      val = (x * pw + 2.0L * mm * val) / (2.0L * mm + 1.0L);
      pw *= w;
    }
    return val;
  }

  long double K() const { return expl(logK_); }
  long double W(long double x) const {  // (1 - x^2)^(m + 1)
    long double w = 1.0L - x * x;
    return w <= 0 ? 0.0L : powl(w, m_ + 1);
  }
  long double m() const { return m_; }

  long double mass(long double a, long double b) const { return expl(logK_) * (J(b) - J(a)); }

  long double moment(long double a, long double b) const {
    long double wa = 1.0L - a * a, wb = 1.0L - b * b;
    if (wa < 0) wa = 0;
    if (wb < 0) wb = 0;
    return expl(logK_) * (powl(wa, m_ + 1) - powl(wb, m_ + 1)) / (2.0L * (m_ + 1));
  }

 private:
  int d_;
  long double m_;
  long double logK_;
  bool half_integer_;
};

void solve_codebook(int d, int bits, float* cent32, float* bound32) {
  const int n = 1 << bits;
  CoordinateLaw law(d);
  long double c[32], cn[32], e[33];
  // start: evenly spaced over +-3 standard deviations of the law (1/sqrt(d))
  const long double spread = fminl(0.95L, 3.0L / sqrtl((long double)d));
  for (int j = 0; j < n; ++j) c[j] = spread * ((2.0L * j + 1) / n - 1.0L);
  long double Jv[33], Wv[33];
  const long double K = law.K();
  int tail = -1;  // iterations left once the steps reach the rounding noise
  for (int it = 0; it < 100000; ++it) {
    e[0] = -1.0L;
    e[n] = 1.0L;
    for (int j = 1; j < n; ++j) e[j] = 0.5L * (c[j - 1] + c[j]);
    for (int k = 0; k <= n; ++k) {
      Jv[k] = law.J(e[k]);
      Wv[k] = law.W(e[k]);
    }
    long double step = 0;
    for (int j = 0; j < n; ++j) {
      const long double mass = K * (Jv[j + 1] - Jv[j]);
      const long double mom = K * (Wv[j] - Wv[j + 1]) / (2.0L * (law.m() + 1));
      cn[j] = mom / mass;
      step = fmaxl(step, fabsl(cn[j] - c[j]));
    }
    for (int j = 0; j < n; ++j) c[j] = cn[j];
    if (step < 1e-18L) break;
    // long double rounding noise keeps the steps near 1e-17..1e-16; run a
    // few hundred more iterations once below 1e-16, then stop
    if (tail < 0 && step < 1e-16L) tail = 400;
    if (tail >= 0 && tail-- == 0) break;
  }
  for (int j = 0; j < n; ++j) cent32[j] = (float)(0.5L * (c[j] - c[n - 1 - j]));
  if (bound32)
    for (int j = 0; j + 1 < n; ++j)
      bound32[j] = (float)(0.5 * ((double)cent32[j] + (double)cent32[j + 1]));
}

// fp32 -> fp16 bits, round to nearest even (normal and subnormal range).
uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x47800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax < 0x33000000u) return (uint16_t)sign;  // below half the smallest subnormal
  int exp = (int)(ax >> 23) - 127;
  uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
  int shift = (exp < -14) ? (13 + (-14 - exp)) : 13;
  uint32_t r = mant >> shift;
  uint32_t rem = mant & ((1u << shift) - 1);
  uint32_t halfway = 1u << (shift - 1);
  if (rem > halfway || (rem == halfway && (r & 1))) ++r;
  uint32_t out = (exp < -14) ? r : ((uint32_t)(exp + 15) << 10) + (r - 0x400u);
  return (uint16_t)(sign | out);
}

float f16_bits_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v;
  if (e == 0)
    v = std::ldexp((float)m, -24);
  else
    v = std::ldexp((float)(m | 0x400), (int)e - 25);
  uint32_t bitsv;
  std::memcpy(&bitsv, &v, 4);
  bitsv |= sign;
  std::memcpy(&v, &bitsv, 4);
  return v;
}

// Scale s in [1, 2) for which the fp16 roundings of s*c_j have the smallest
// worst relative error; the value tables of the decode hold fp16(s * c_j)
// and the output is divided by s at the end.
float best_fp16_scale(const float* c, int n) {
  float best_s = 1.0f;
  double best_err = 1e30;
  for (int k = 0; k < (1 << 18); ++k) {
    float s = 1.0f + (float)k / (float)(1 << 18);
    double worst = 0;
    for (int j = n / 2; j < n; ++j) {  // magnitudes (the codebook is symmetric)
      float v = s * c[j];
      double err = std::fabs((double)f16_bits_to_f32(f32_to_f16_bits(v)) - (double)v) / (double)v;
      if (err > worst) worst = err;
      if (worst >= best_err) break;
    }
    if (worst < best_err) {
      best_err = worst;
      best_s = s;
    }
  }
  return best_s;
}

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// Decode work split.  A workgroup covers kv_per_wg KV heads of one sequence
// and pages_per_split of its pages; its waves are kv_per_wg * q_groups
// (ceil(group / 8) query groups per KV head) times streams.  A stage is
// `streams` pages of the workgroup's heads, staged as 16-byte chunk windows
// over each token's slice; two stage slots, the lookup tables and the block
// ids share the CU's LDS, which bounds kv_per_wg and streams.  The split
// count aims at one workgroup per CU (a workgroup fills a CU's LDS), keeps at
// least 4 splits for the longest sequence (so ragged batches balance; more,
// smaller splits cost more in per-workgroup set-up than they gain) and at
// most 64 (the merge holds one split weight per lane).
struct SplitPlan {
  int q_groups;
  int kv_per_wg;
  int head_groups;
  int streams;
  int pages_per_split;
  int num_splits;
  int tok_chunks[2];  // K, V
  int slice_chunks[2];
  int chunks[2];
  int loads[2];
  int page_slot;
  int bt_base;
};

#ifndef TQ_WG_WAVES
#define TQ_WG_WAVES 16
#endif
constexpr int kMaxWavesPerWg = TQ_WG_WAVES;
constexpr int kMaxLoadsPerWave = 4;
constexpr int kLdsBytes = tq::kDecodeLdsBytes;

bool plan_split(int batch, int num_kv_heads, int group, int max_seq_len, int k_bits, int v_bits, int num_cus,
                SplitPlan* out) {
  SplitPlan p;
  p.q_groups = (group + 7) / 8;
  const int rb[2] = {(int)tq_row_bytes(kHeadDim, k_bits), (int)tq_row_bytes(kHeadDim, v_bits)};
  const int tables = tq::decode_table_bytes(k_bits, v_bits);
  const int max_pages = (max_seq_len + tq::kBlockSize - 1) / tq::kBlockSize;
  const int bt_cap = std::max(1, std::min((max_pages + 3) / 4, std::max(2048, (max_pages + 63) / 64)));
  const int bt_bytes = 4 * bt_cap;
  bool found = false;
  for (int kv = num_kv_heads; kv >= 1 && !found; --kv) {
    if (num_kv_heads % kv || kv * p.q_groups > kMaxWavesPerWg) continue;
    for (int i = 0; i < 2; ++i) {
      if (kv == num_kv_heads) {  // whole pages: rows in 16-byte slices, an odd number of chunks per token
        p.slice_chunks[i] = (rb[i] + 15) / 16;
        p.tok_chunks[i] = num_kv_heads * p.slice_chunks[i] | 1;
        p.chunks[i] = tq::kBlockSize * p.tok_chunks[i];
      } else {
        p.slice_chunks[i] = 0;                   // window start at most 31 bytes before the slice
        p.tok_chunks[i] = (kv * rb[i] + 16 + 15) / 16;
        p.chunks[i] = tq::kBlockSize * p.tok_chunks[i];
      }
      p.loads[i] = (p.chunks[i] + 63) / 64;
    }
    p.page_slot = 16 * (p.chunks[0] + p.chunks[1]);
    const int hpw = kv * p.q_groups;
    for (int strm = kMaxWavesPerWg / hpw; strm >= 1; strm /= 2) {
      const int waves = hpw * strm;
      const int lds = tables + 2 * strm * p.page_slot + bt_bytes;
      const int per_wave = (strm * (p.loads[0] + p.loads[1]) + waves - 1) / waves;
      if (lds <= kLdsBytes && per_wave <= kMaxLoadsPerWave) {
        p.kv_per_wg = kv;
        p.streams = strm;
        p.bt_base = tables + 2 * strm * p.page_slot;
        found = true;
        break;
      }
    }
  }
  if (!found) return false;
  p.head_groups = num_kv_heads / p.kv_per_wg;
  if (max_pages <= 0) {
    p.pages_per_split = 1;
    p.num_splits = 1;
    *out = p;
    return true;
  }
  const long long units = (long long)batch * p.head_groups;
  const long long target = num_cus;
  long long s0 = (target + units - 1) / units;
  if (s0 < 1) s0 = 1;
  long long pps = (max_pages + s0 - 1) / s0;
  const long long cap = (max_pages + 3) / 4;
  if (pps > cap) pps = cap;
  if (pps > bt_cap) pps = bt_cap;
  const long long floor_pps = (max_pages + 63) / 64;
  if (pps < floor_pps) pps = floor_pps;
  if (pps < 1) pps = 1;
  p.pages_per_split = (int)pps;
  p.num_splits = (int)((max_pages + pps - 1) / pps);
  *out = p;
  return true;
}

// Wave-private decode plan (tq_decode_wave.hip): each wave owns every KV head
// of the page (num_kv_heads 1, 2 or 4, group <= 8) and loads whole pages
// itself; the pages are split evenly over num_wg workgroups, one per CU (a
// workgroup holds the CU's registers).  It beats the staged kernel where few
// heads share a page (measured on the pages' geometry and the ragged batch);
// with 8 heads a wave would hold 8 query groups and the staged kernel wins.
// A small batch (at most kDirectPages pages in all, at most 64 sequences)
// runs as one workgroup, which finishes every sequence itself: no merge
// kernel, whose launch and dependent loads cost more than a few pages.
// Returns false when the shape is outside this kernel's reach.
constexpr long long kDirectPages = 32;  // four pages per wave of the one workgroup

struct WavePlan {
  int nh;      // KV heads per wave (all of the page's)
  int num_wg;
};

// TQ_DECODE_KERNEL overrides the choice: "staged" (tq_decode.hip) or "wave"
// (tq_decode_wave.hip, where the shape allows it); unset or "auto": the
// planner's choice.
int decode_kernel_choice() {
  static const int choice = [] {
    const char* e = std::getenv("TQ_DECODE_KERNEL");
    if (!e || !*e || std::strcmp(e, "auto") == 0) return 0;
    if (std::strcmp(e, "staged") == 0) return 1;
    if (std::strcmp(e, "wave") == 0) return 2;
    return 0;
  }();
  return choice;
}

bool plan_wave(int batch, int num_kv_heads, int group, int max_seq_len, int k_bits, int v_bits, int num_cus,
               WavePlan* out) {
  if (decode_kernel_choice() == 1 || group < 1 || group > 8) return false;
  const long long max_pages = (max_seq_len + tq::kBlockSize - 1) / tq::kBlockSize;
  if ((long long)batch * max_pages > (1LL << 40)) return false;
  const int hkv = num_kv_heads;
  if (hkv != 1 && hkv != 2 && hkv != 4) return false;
  const int waves = tq::wave_waves(hkv);
  if (waves == 0 || !tq::wave_fits(k_bits, v_bits, hkv, hkv)) return false;
  WavePlan p;
  p.nh = hkv;
  const long long units = std::max<long long>(1, (long long)batch * max_pages);
  p.num_wg = (units <= kDirectPages && batch <= 64) ? 1 : (int)std::min<long long>(num_cus, units);
  *out = p;
  return true;
}

// The current device must be a gfx950; checked once per device.
bool device_is_gfx950() {
  static std::mutex mu;
  static signed char cache[64] = {0};  // 0 unknown, 1 yes, -1 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev >= 64) {
    hipDeviceProp_t prop;
    return hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    const bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    cache[dev] = ok ? 1 : -1;
  }
  return cache[dev] > 0;
}

bool bits_ok(int b) { return b >= 2 && b <= 5; }

}  // namespace

extern "C" {

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_ALIGNMENT: return "misaligned pointer";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_HIP: return "HIP runtime error";
    case TQ_ERR_NO_DEVICE: return "no gfx950 device";
  }
  return "unknown status";
}

int tq_last_hip_error(void) { return g_last_hip_error; }

size_t tq_row_bytes(int head_dim, int bits) {
  if (head_dim <= 0 || bits < 1 || bits > 8) return 0;
  return ((size_t)head_dim * bits + 7) / 8 + 4;
}

tq_status tq_codebook(int head_dim, int bits, float* centroids, float* boundaries) {
  if (!centroids || head_dim < 3 || head_dim > 4096 || bits < 1 || bits > 5) return TQ_ERR_INVALID_ARG;
  solve_codebook(head_dim, bits, centroids, boundaries);
  return TQ_OK;
}

tq_status tq_rht_signs(uint64_t seed, int head_dim, int8_t* signs) {
  if (!signs || head_dim <= 0) return TQ_ERR_INVALID_ARG;
  uint64_t st = seed;
  for (int i = 0; i < head_dim; ++i) signs[i] = (splitmix64_next(st) >> 63) ? -1 : 1;
  return TQ_OK;
}

tq_status tq_ctx_create(int head_dim, uint64_t rht_seed, tq_ctx** out) {
  if (!out) return TQ_ERR_INVALID_ARG;
  *out = nullptr;
  if (head_dim != kHeadDim) return TQ_ERR_UNSUPPORTED;
  tq_ctx* c = new (std::nothrow) tq_ctx;
  if (!c) return TQ_ERR_INVALID_ARG;
  std::memset(c, 0, sizeof(*c));
  c->head_dim = head_dim;
  c->seed = rht_seed;
  tq_rht_signs(rht_seed, head_dim, c->signs);
  for (int i = 0; i < head_dim; ++i)
    if (c->signs[i] < 0) c->sign_bits[i >> 5] |= 1u << (i & 31);
  for (int b = 1; b <= 5; ++b) {
    solve_codebook(head_dim, b, c->cent[b], c->bound[b]);
    c->tab_scale[b] = best_fp16_scale(c->cent[b], 1 << b);
  }
  *out = c;
  return TQ_OK;
}

tq_status tq_ctx_destroy(tq_ctx* ctx) {
  delete ctx;
  return TQ_OK;
}

}  // extern "C"

namespace {

// Validate one component's write and fill its kernel arguments.
tq_status make_write_args(const tq_ctx* ctx, const void* raw, tq_dtype raw_dtype, int64_t num_tokens,
                          int num_kv_heads, uint8_t* pages, int64_t num_blocks, int block_size,
                          const int64_t* slots, int bits, int32_t* err_count, tq::WriteArgs* out) {
  if (!ctx || num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0)
    return TQ_ERR_INVALID_ARG;
  if (raw_dtype != TQ_F32 && raw_dtype != TQ_F16 && raw_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!bits_ok(bits)) return TQ_ERR_UNSUPPORTED;
  tq::WriteArgs& a = *out;
  std::memset(&a, 0, sizeof(a));
  if (num_tokens == 0) return TQ_OK;  // nothing to write (pointers unused)
  if (!raw || !pages || !slots) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(raw) & 3) || (reinterpret_cast<uintptr_t>(pages) & 3) ||
      (reinterpret_cast<uintptr_t>(slots) & 7))
    return TQ_ERR_ALIGNMENT;
  a.raw = raw;
  a.pages = pages;
  a.slots = slots;
  a.err_count = err_count;
  a.num_rows = num_tokens * num_kv_heads;
  a.num_slots = num_blocks * block_size;
  a.row_bytes = (int)tq_row_bytes(kHeadDim, bits);
  a.page_bytes = (int64_t)block_size * num_kv_heads * a.row_bytes;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  std::memcpy(a.sign_bits, ctx->sign_bits, sizeof(a.sign_bits));
  const int n = 1 << bits;
  for (int j = 0; j < n / 2 - 1; ++j) a.pos_bounds[j] = ctx->bound[bits][n / 2 + j];
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_write_kv(const tq_ctx* ctx, const void* raw, tq_dtype raw_dtype, int64_t num_tokens,
                      int num_kv_heads, uint8_t* pages, int64_t num_blocks, int block_size,
                      const int64_t* slots, int bits, int32_t* err_count, void* stream) {
  tq::WriteArgs a;
  const tq_status st = make_write_args(ctx, raw, raw_dtype, num_tokens, num_kv_heads, pages, num_blocks,
                                       block_size, slots, bits, err_count, &a);
  if (st != TQ_OK || num_tokens == 0) return st;
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
  return hip_status(tq::launch_write(a, (int)raw_dtype, bits, (hipStream_t)stream));
}

tq_status tq_write_kv_pair(const tq_ctx* ctx, const void* raw_k, const void* raw_v, tq_dtype raw_dtype,
                           int64_t num_tokens, int num_kv_heads, uint8_t* k_pages, int k_bits,
                           uint8_t* v_pages, int v_bits, int64_t num_blocks, int block_size,
                           const int64_t* slots, int32_t* err_count, void* stream) {
  tq::WriteArgs k, v;
  tq_status st = make_write_args(ctx, raw_k, raw_dtype, num_tokens, num_kv_heads, k_pages, num_blocks,
                                 block_size, slots, k_bits, err_count, &k);
  if (st != TQ_OK) return st;
  // an out-of-range slot is counted once (by the K rows); both components skip it
  st = make_write_args(ctx, raw_v, raw_dtype, num_tokens, num_kv_heads, v_pages, num_blocks, block_size,
                       slots, v_bits, nullptr, &v);
  if (st != TQ_OK || num_tokens == 0) return st;
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
  return hip_status(tq::launch_write_pair(k, v, (int)raw_dtype, k_bits, v_bits, (hipStream_t)stream));
}

tq_status tq_decompress_kv(const tq_ctx* ctx, const uint8_t* pages, int64_t num_blocks, int block_size,
                           int num_kv_heads, int bits, const int64_t* slots, int64_t num_tokens, void* out,
                           tq_dtype out_dtype, int32_t* err_count, void* stream) {
  if (!ctx || num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0)
    return TQ_ERR_INVALID_ARG;
  if (out_dtype != TQ_F32 && out_dtype != TQ_F16 && out_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!bits_ok(bits)) return TQ_ERR_UNSUPPORTED;
  if (num_tokens == 0) return TQ_OK;  // nothing to read (pointers unused)
  if (!pages || !slots || !out) return TQ_ERR_INVALID_ARG;
  if (num_tokens > (INT64_C(1) << 31) / num_kv_heads - 1) return TQ_ERR_UNSUPPORTED;  // rows < 2^31
  if ((reinterpret_cast<uintptr_t>(pages) & 3) || (reinterpret_cast<uintptr_t>(slots) & 7) ||
      (reinterpret_cast<uintptr_t>(out) & 15))
    return TQ_ERR_ALIGNMENT;
  tq::ReadArgs a;
  std::memset(&a, 0, sizeof(a));
  a.pages = pages;
  a.slots = slots;
  a.out = out;
  a.err_count = err_count;
  a.num_rows = (uint32_t)(num_tokens * num_kv_heads);
  a.num_slots = num_blocks * block_size;
  a.row_bytes = (int)tq_row_bytes(kHeadDim, bits);
  a.page_bytes = (int64_t)block_size * num_kv_heads * a.row_bytes;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  if (a.page_bytes >= (INT64_C(1) << 31)) return TQ_ERR_UNSUPPORTED;
  a.hkv_shift = (num_kv_heads & (num_kv_heads - 1)) ? -1 : __builtin_ctz((unsigned)num_kv_heads);
  a.bs_shift = (block_size & (block_size - 1)) ? -1 : __builtin_ctz((unsigned)block_size);
  std::memcpy(a.cent, ctx->cent[bits], sizeof(float) << bits);
  for (int q = 0; q < 4; ++q) {
    const bool odd = ((q ^ (q >> 1)) & 1) != 0;  // popcount(q) odd
    for (int j = 0; j < 32; ++j)
      if ((ctx->signs[32 * q + j] < 0) != odd) a.neg_bits[q] |= 1u << j;
  }
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
  return hip_status(tq::launch_decompress(a, bits, (int)out_dtype, device_cu_count(), (hipStream_t)stream));
}

size_t tq_prod_row_bytes(int head_dim, int bits) {
  if (head_dim <= 0 || head_dim % 8 || bits < 2 || bits > 8) return 0;
  return ((size_t)head_dim * (bits - 1) + 7) / 8 + 4 + (size_t)head_dim / 8 + 4;
}

tq_status tq_write_kv_prod(const tq_ctx* ctx, const void* raw, tq_dtype raw_dtype, int64_t num_tokens,
                           int num_kv_heads, uint8_t* pages, int64_t num_blocks, int block_size,
                           const int64_t* slots, int bits, const float* sketch, int32_t* err_count, void* stream) {
  if (!bits_ok(bits)) return TQ_ERR_UNSUPPORTED;
  tq::ProdWriteArgs a;
  std::memset(&a, 0, sizeof(a));
  // the MSE part: the (bits - 1)-bit codec's boundaries; 1-bit indices are
  // the sign of each coordinate
  const tq_status st = make_write_args(ctx, raw, raw_dtype, num_tokens, num_kv_heads, pages, num_blocks, block_size,
                                       slots, bits == 2 ? 2 : bits - 1, err_count, &a.w);
  if (st != TQ_OK || num_tokens == 0) return st;
  if (!sketch) return TQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(sketch) & 15) return TQ_ERR_ALIGNMENT;
  const int mb = bits - 1, n = 1 << mb;
  a.w.row_bytes = (int)tq_prod_row_bytes(kHeadDim, bits);
  a.w.page_bytes = (int64_t)block_size * num_kv_heads * a.w.row_bytes;
  std::memset(a.w.pos_bounds, 0, sizeof(a.w.pos_bounds));
  for (int j = 0; j < n / 2 - 1; ++j) a.w.pos_bounds[j] = ctx->bound[mb][n / 2 + j];
  for (int j = 0; j < n / 2; ++j) a.cpos[j] = ctx->cent[mb][n / 2 + j];
  a.sketch = sketch;
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
  return hip_status(tq::launch_write_prod(a, (int)raw_dtype, bits, device_cu_count(), (hipStream_t)stream));
}

size_t tq_prod_scores_workspace_bytes(int batch, int num_q_heads) {
  if (batch <= 0 || num_q_heads <= 0) return 0;
  return 2 * (size_t)batch * num_q_heads * kHeadDim * sizeof(float);
}

tq_status tq_prod_scores(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch, int num_q_heads,
                         int num_kv_heads, const uint8_t* pages, int bits, int64_t num_blocks, int block_size,
                         const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                         int max_seq_len, const float* sketch, float* scores, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!ctx || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_seq_len < 0)
    return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_F16 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return TQ_ERR_INVALID_ARG;
  if (!bits_ok(bits) || block_size != tq::kBlockSize) return TQ_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size < max_seq_len) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  if (!q || !pages || !block_table || !seq_lens || !sketch || !scores) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(pages) & 3) || (reinterpret_cast<uintptr_t>(sketch) & 15) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15) || (reinterpret_cast<uintptr_t>(q) & 3) ||
      (reinterpret_cast<uintptr_t>(scores) & 3))
    return TQ_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < tq_prod_scores_workspace_bytes(batch, num_q_heads)) return TQ_ERR_WORKSPACE;
  const int row_bytes = (int)tq_prod_row_bytes(kHeadDim, bits);
  if ((long long)block_size * num_kv_heads * row_bytes > (1 << 30)) return TQ_ERR_UNSUPPORTED;
  if ((long long)max_seq_len * 8 * sizeof(float) >= (1LL << 31)) return TQ_ERR_UNSUPPORTED;  // 8 score rows per buffer
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
  tq::ProdScoreArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.pages = pages;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.sketch = sketch;
  a.qr = static_cast<float*>(workspace);
  a.sq = a.qr + (size_t)batch * num_q_heads * kHeadDim;
  a.scores = scores;
  a.page_bytes = (int64_t)block_size * num_kv_heads * row_bytes;
  a.num_blocks = num_blocks;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.max_len = (int)std::min<long long>((long long)max_blocks_per_seq * block_size, 0x7fffffffLL);
  a.row_bytes = row_bytes;
  a.q_dtype = (int)q_dtype;
  std::memcpy(a.sign_bits, ctx->sign_bits, sizeof(a.sign_bits));
  for (int i = 0; i < (1 << (bits - 1)); ++i) a.cent[i] = 16.0f * ctx->cent[bits - 1][i];  // exact
  // pages per workgroup: enough workgroups for the device (about 4 per CU),
  // at most 128 pages each, a multiple of the 4 waves
  const int npages = (max_seq_len + block_size - 1) / block_size;
  // with 8 or more KV heads a workgroup takes four neighbouring heads, one per
  // wave, so that its waves read whole cache lines of a page together (7 %
  // faster at 8 heads); with fewer heads, one head per workgroup is faster
  a.head_group = (num_kv_heads >= 8 && num_kv_heads % 4 == 0) ? 4 : 1;
  a.phases = 4 / a.head_group;
  const long long units = (long long)batch * (num_kv_heads / a.head_group) * ((num_q_heads / num_kv_heads + 7) / 8);
  const long long per_seq = std::max(1LL, (4LL * device_cu_count() + units - 1) / units);
  int cp = (int)std::min<long long>(128, (npages + per_seq - 1) / per_seq);
  cp = std::max(4, (cp + 3) / 4 * 4);
  a.chunk_pages = cp;
  a.chunks = (npages + cp - 1) / cp;
  a.vec_store = (max_seq_len % 4 == 0) && !(reinterpret_cast<uintptr_t>(scores) & 15);
  return hip_status(tq::launch_prod_scores(a, bits, (hipStream_t)stream));
}

size_t tq_decode_workspace_bytes(const tq_ctx* ctx, int batch, int num_q_heads, int num_kv_heads,
                                 int max_seq_len, int block_size) {
  (void)ctx;
  (void)block_size;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return 0;
  // the split count depends on the bit widths through the LDS budget: size
  // for the largest over every supported pair
  int splits = 1;
  for (int kb = 2; kb <= 5; ++kb)
    for (int vb = 2; vb <= 5; ++vb) {
      SplitPlan p;
      if (plan_split(batch, num_kv_heads, num_q_heads / num_kv_heads, max_seq_len, kb, vb, device_cu_count(), &p) &&
          p.num_splits > splits)
        splits = p.num_splits;
    }
  size_t per = (size_t)batch * num_q_heads * splits;
  // the wave-private kernel: one partial per (sequence, workgroup) pair it touches
  const size_t wave_slots = (size_t)batch + (size_t)device_cu_count();
  per = std::max(per, wave_slots * (size_t)num_q_heads);
  return per * (kHeadDim + 1) * sizeof(float) + 256;
}

const char* tq_decode_kernel(int batch, int num_q_heads, int num_kv_heads, int max_seq_len, int k_bits,
                             int v_bits) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 || num_q_heads % num_kv_heads ||
      !bits_ok(k_bits) || !bits_ok(v_bits))
    return nullptr;
  const int group = num_q_heads / num_kv_heads;
  if (group > tq::kMaxGroup) return nullptr;
  WavePlan wp;
  if (plan_wave(batch, num_kv_heads, group, max_seq_len, k_bits, v_bits, device_cu_count(), &wp))
    return wp.num_wg == 1 ? "wave1" : "wave";
  SplitPlan p;
  if (plan_split(batch, num_kv_heads, group, max_seq_len, k_bits, v_bits, device_cu_count(), &p)) return "staged";
  return nullptr;
}

}  // extern "C"

namespace {

// The decode of tq_paged_decode; lse_out (device [batch, num_q_heads] or
// null) receives each query head's log2-sum-exp2 of its scores times log2(e)
// (-inf for an empty sequence) where the output is finished.
tq_status decode_impl(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch, int num_q_heads,
                      int num_kv_heads, const uint8_t* k_pages, int k_bits, const uint8_t* v_pages, int v_bits,
                      int64_t num_blocks, int block_size, const int32_t* block_table, int max_blocks_per_seq,
                      const int32_t* seq_lens, int max_seq_len, float scale, float* out, float* lse_out,
                      void* workspace, size_t workspace_bytes, void* stream,
                      const tq::AppendArgs* app = nullptr) {
  if (!ctx || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_seq_len < 0)
    return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_F16 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return TQ_ERR_INVALID_ARG;
  const int group = num_q_heads / num_kv_heads;
  if (block_size != tq::kBlockSize || group > tq::kMaxGroup || !bits_ok(k_bits) || !bits_ok(v_bits))
    return TQ_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size < max_seq_len) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_pages) & 15) || (reinterpret_cast<uintptr_t>(v_pages) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15) || (reinterpret_cast<uintptr_t>(workspace) & 15) ||
      (reinterpret_cast<uintptr_t>(q) & 3))
    return TQ_ERR_ALIGNMENT;
  const size_t need =
      tq_decode_workspace_bytes(ctx, batch, num_q_heads, num_kv_heads, max_seq_len, block_size);
  if (!workspace || workspace_bytes < need) return TQ_ERR_WORKSPACE;

  const float sm_scale = scale > 0 ? scale : 1.0f / std::sqrt((float)kHeadDim);
  const float k_scale = ctx->tab_scale[k_bits];
  const float v_scale = ctx->tab_scale[v_bits];
  const int k_row_bytes = (int)tq_row_bytes(kHeadDim, k_bits);
  const int v_row_bytes = (int)tq_row_bytes(kHeadDim, v_bits);
  const long long max_len_cap = std::min<long long>((long long)max_blocks_per_seq * block_size, 0x7fffffffLL);
  if ((long long)block_size * num_kv_heads * std::max(k_row_bytes, v_row_bytes) > (1 << 30)) return TQ_ERR_UNSUPPORTED;

  WavePlan wp;
  if (plan_wave(batch, num_kv_heads, group, max_seq_len, k_bits, v_bits, device_cu_count(), &wp)) {
    if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
    tq::WaveArgs w;
    std::memset(&w, 0, sizeof(w));
    w.q = q;
    w.k_pages = k_pages;
    w.v_pages = v_pages;
    w.block_table = block_table;
    w.seq_lens = seq_lens;
    w.part_acc = static_cast<float*>(workspace);
    w.part_lse = w.part_acc + ((size_t)batch + wp.num_wg) * num_q_heads * kHeadDim;
    w.out = out;
    w.lse_out = lse_out;
    w.direct = wp.num_wg == 1 ? 1 : 0;  // then every sequence is finished by the decode kernel
    w.k_page_bytes = (int64_t)block_size * num_kv_heads * k_row_bytes;
    w.v_page_bytes = (int64_t)block_size * num_kv_heads * v_row_bytes;
    w.num_blocks = num_blocks;
    w.max_len = (int)max_len_cap;
    w.batch = batch;
    w.num_q_heads = num_q_heads;
    w.num_kv_heads = num_kv_heads;
    w.group = group;
    w.max_blocks_per_seq = max_blocks_per_seq;
    w.num_wg = wp.num_wg;
    w.q_dtype = (int)q_dtype;
    w.q_scale = (float)((double)sm_scale * 1.4426950408889634 / (std::sqrt((double)kHeadDim) * k_scale));
    w.out_scale = (float)(1.0 / ((double)v_scale * std::sqrt((double)kHeadDim)));
    std::memcpy(w.sign_bits, ctx->sign_bits, sizeof(w.sign_bits));
    for (int j = 0; j < (1 << k_bits); ++j) w.k_cent[j] = ctx->cent[k_bits][j] * k_scale;
    for (int j = 0; j < (1 << v_bits); ++j) w.v_cent[j] = ctx->cent[v_bits][j] * v_scale;
    if (app) {
      // the wave-private decode does not append: the appending row writer
      // runs first (a workgroup that also encoded would hold every later
      // page load of its sequences' ends behind the encode)
      tq::AppendWriteArgs aw;
      std::memset(&aw, 0, sizeof(aw));
      aw.app = *app;
      aw.k_pages = const_cast<uint8_t*>(k_pages);
      aw.v_pages = const_cast<uint8_t*>(v_pages);
      aw.block_table = block_table;
      aw.seq_lens = seq_lens;
      aw.k_page_bytes = w.k_page_bytes;
      aw.v_page_bytes = w.v_page_bytes;
      aw.num_blocks = num_blocks;
      aw.batch = batch;
      aw.num_kv_heads = num_kv_heads;
      aw.max_blocks_per_seq = max_blocks_per_seq;
      aw.max_len = w.max_len;
      aw.k_row_bytes = k_row_bytes;
      aw.v_row_bytes = v_row_bytes;
      std::memcpy(aw.sign_bits, ctx->sign_bits, sizeof(aw.sign_bits));
      const tq_status sa = hip_status(tq::launch_write_append(aw, k_bits, v_bits, (hipStream_t)stream));
      if (sa != TQ_OK) return sa;
    }
    tq_status st = hip_status(tq::launch_decode_wave(w, k_bits, v_bits, wp.nh, (hipStream_t)stream));
    if (st != TQ_OK || w.direct) return st;
    tq::WaveMergeArgs m;
    std::memset(&m, 0, sizeof(m));
    m.part_acc = w.part_acc;
    m.part_lse = w.part_lse;
    m.seq_lens = seq_lens;
    m.out = out;
    m.lse_out = lse_out;
    m.batch = batch;
    m.num_q_heads = num_q_heads;
    m.num_wg = wp.num_wg;
    m.max_len = w.max_len;
    m.inv_v_scale_over_sqrt_d = w.out_scale;
    std::memcpy(m.sign_bits, ctx->sign_bits, sizeof(m.sign_bits));
    return hip_status(tq::launch_merge_wave(m, (hipStream_t)stream));
  }

  SplitPlan p;
  if (!plan_split(batch, num_kv_heads, group, max_seq_len, k_bits, v_bits, device_cu_count(), &p))
    return TQ_ERR_UNSUPPORTED;
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;

  tq::DecodeArgs d;
  std::memset(&d, 0, sizeof(d));
  d.q = q;
  d.k_pages = k_pages;
  d.v_pages = v_pages;
  d.block_table = block_table;
  d.seq_lens = seq_lens;
  d.part_acc = static_cast<float*>(workspace);
  d.part_lse = d.part_acc + (size_t)batch * num_q_heads * p.num_splits * kHeadDim;
  d.k_row_bytes = k_row_bytes;
  d.v_row_bytes = v_row_bytes;
  d.k_page_bytes = (int64_t)block_size * num_kv_heads * d.k_row_bytes;
  d.v_page_bytes = (int64_t)block_size * num_kv_heads * d.v_row_bytes;
  d.batch = batch;
  d.num_q_heads = num_q_heads;
  d.num_kv_heads = num_kv_heads;
  d.group = group;
  d.q_groups = p.q_groups;
  d.max_blocks_per_seq = max_blocks_per_seq;
  d.num_blocks = num_blocks;
  {
    // a device-side length beyond the block table or the planned splits is
    // clamped, so no page past them is ever read
    const long long cap_pages = std::min<long long>(max_blocks_per_seq, (long long)p.num_splits * p.pages_per_split);
    d.max_len = (int)std::min<long long>(cap_pages * block_size, 0x7fffffffLL);
  }
  d.kv_per_wg = p.kv_per_wg;
  d.head_groups = p.head_groups;
  d.streams = p.streams;
  d.waves = p.kv_per_wg * p.q_groups * p.streams;
  d.pages_per_split = p.pages_per_split;
  d.num_splits = p.num_splits;
  d.q_dtype = (int)q_dtype;
  d.k_tok_chunks = p.tok_chunks[0];
  d.v_tok_chunks = p.tok_chunks[1];
  d.k_slice_chunks = p.slice_chunks[0];
  d.v_slice_chunks = p.slice_chunks[1];
  d.k_chunks = p.chunks[0];
  d.v_chunks = p.chunks[1];
  d.k_loads = p.loads[0];
  d.v_loads = p.loads[1];
  d.k_region = 16 * p.chunks[0];
  d.page_slot_bytes = p.page_slot;
  d.stage_bytes = p.streams * p.page_slot;
  d.bt_base = p.bt_base;
  d.q_scale = (float)((double)sm_scale * 1.4426950408889634 / (std::sqrt((double)kHeadDim) * k_scale));
  std::memcpy(d.sign_bits, ctx->sign_bits, sizeof(d.sign_bits));
  for (int j = 0; j < (1 << k_bits); ++j) d.k_cent[j] = ctx->cent[k_bits][j] * k_scale;
  for (int j = 0; j < (1 << v_bits); ++j) d.v_cent[j] = ctx->cent[v_bits][j] * v_scale;
  if (app) d.app = *app;
  // per-page byte offsets are 32-bit inside a page
  if (d.k_page_bytes > (1 << 30) || d.v_page_bytes > (1 << 30)) return TQ_ERR_UNSUPPORTED;

  tq_status st = hip_status(tq::launch_decode(d, k_bits, v_bits, (hipStream_t)stream));
  if (st != TQ_OK) return st;

  tq::MergeArgs m;
  std::memset(&m, 0, sizeof(m));
  m.part_acc = d.part_acc;
  m.part_lse = d.part_lse;
  m.seq_lens = seq_lens;
  m.out = out;
  m.lse_out = lse_out;
  m.batch = batch;
  m.num_q_heads = num_q_heads;
  m.pages_per_split = p.pages_per_split;
  m.num_splits = p.num_splits;
  m.max_len = d.max_len;
  m.inv_v_scale_over_sqrt_d = (float)(1.0 / ((double)v_scale * std::sqrt((double)kHeadDim)));
  std::memcpy(m.sign_bits, ctx->sign_bits, sizeof(m.sign_bits));
  return hip_status(tq::launch_merge(m, (hipStream_t)stream));
}

}  // namespace

extern "C" {

tq_status tq_paged_decode(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch,
                          int num_q_heads, int num_kv_heads, const uint8_t* k_pages, int k_bits,
                          const uint8_t* v_pages, int v_bits, int64_t num_blocks, int block_size,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* seq_lens, int max_seq_len, float scale, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(ctx, q, q_dtype, batch, num_q_heads, num_kv_heads, k_pages, k_bits, v_pages, v_bits,
                     num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len, scale, out,
                     nullptr, workspace, workspace_bytes, stream);
}

tq_status tq_paged_decode_append(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch,
                                 int num_q_heads, int num_kv_heads, const void* k_new, const void* v_new,
                                 tq_dtype new_dtype, uint8_t* k_pages, int k_bits, uint8_t* v_pages, int v_bits,
                                 int64_t num_blocks, int block_size, const int32_t* block_table,
                                 int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, float scale,
                                 float* out, void* workspace, size_t workspace_bytes, int32_t* err_count,
                                 void* stream) {
  if (new_dtype != TQ_F32 && new_dtype != TQ_F16 && new_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!ctx || !bits_ok(k_bits) || !bits_ok(v_bits)) return ctx ? TQ_ERR_UNSUPPORTED : TQ_ERR_INVALID_ARG;
  if (batch > 0 && (!k_new || !v_new)) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_new) & 3) || (reinterpret_cast<uintptr_t>(v_new) & 3)) return TQ_ERR_ALIGNMENT;
  tq::AppendArgs app;
  std::memset(&app, 0, sizeof(app));
  app.k_new = k_new;
  app.v_new = v_new;
  app.err_count = err_count;
  app.on = 1;
  app.new_dtype = (int)new_dtype;
  const int nk = 1 << k_bits, nv = 1 << v_bits;
  for (int j = 0; j < nk / 2 - 1; ++j) app.k_bounds[j] = ctx->bound[k_bits][nk / 2 + j];
  for (int j = 0; j < nv / 2 - 1; ++j) app.v_bounds[j] = ctx->bound[v_bits][nv / 2 + j];
  return decode_impl(ctx, q, q_dtype, batch, num_q_heads, num_kv_heads, k_pages, k_bits, v_pages, v_bits,
                     num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len, scale, out,
                     nullptr, workspace, workspace_bytes, stream, &app);
}

size_t tq_hybrid_workspace_bytes(const tq_ctx* ctx, int batch, int num_q_heads, int num_kv_heads,
                                 int max_seq_len, int block_size) {
  const size_t dec = tq_decode_workspace_bytes(ctx, batch, num_q_heads, num_kv_heads, max_seq_len, block_size);
  if (dec == 0) return 0;
  return ((dec + 255) & ~(size_t)255) + (size_t)batch * num_q_heads * sizeof(float);
}

tq_status tq_paged_decode_hybrid(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch,
                                 int num_q_heads, int num_kv_heads, const uint8_t* k_pages, int k_bits,
                                 const uint8_t* v_pages, int v_bits, int64_t num_blocks, int block_size,
                                 const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                                 int max_seq_len, const void* recent_k, const void* recent_v,
                                 tq_dtype recent_dtype, int recent_cap, const int32_t* recent_lens, float scale,
                                 float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || recent_cap < 0) return TQ_ERR_INVALID_ARG;
  if (recent_dtype != TQ_F32 && recent_dtype != TQ_F16 && recent_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  if (recent_cap > 0 && (!recent_k || !recent_v || !recent_lens)) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(recent_k) | reinterpret_cast<uintptr_t>(recent_v)) & 15) return TQ_ERR_ALIGNMENT;
  const size_t need = tq_hybrid_workspace_bytes(ctx, batch, num_q_heads, num_kv_heads, max_seq_len, block_size);
  if (!workspace || need == 0 || workspace_bytes < need) return TQ_ERR_WORKSPACE;
  const size_t dec = (tq_decode_workspace_bytes(ctx, batch, num_q_heads, num_kv_heads, max_seq_len, block_size) +
                      255) & ~(size_t)255;
  float* lse = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + dec);
  tq_status st = decode_impl(ctx, q, q_dtype, batch, num_q_heads, num_kv_heads, k_pages, k_bits, v_pages, v_bits,
                             num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len, scale,
                             out, lse, workspace, dec, stream);
  if (st != TQ_OK || recent_cap == 0) return st;
  tq::HybridArgs h;
  std::memset(&h, 0, sizeof(h));
  h.q = q;
  h.recent_k = recent_k;
  h.recent_v = recent_v;
  h.recent_lens = recent_lens;
  h.lse = lse;
  h.out = out;
  h.batch = batch;
  h.num_q_heads = num_q_heads;
  h.num_kv_heads = num_kv_heads;
  h.group = num_q_heads / num_kv_heads;
  h.cap = recent_cap;
  h.q_dtype = (int)q_dtype;
  h.r_dtype = (int)recent_dtype;
  const float sm_scale = scale > 0 ? scale : 1.0f / std::sqrt((float)kHeadDim);
  h.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  return hip_status(tq::launch_hybrid(h, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Workspace of tq_paged_prefill, in 256-byte aligned pieces: the decode-order
// queries, the decode-order outputs, prefix and tail lengths, tail slots,
// the dense tail K and V, then the hybrid decode's workspace for Lq * Hq
// query heads.
struct PrefillLayout {
  size_t vq, vout, plen, tlen, slots, tk, tv, hyb, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool prefill_layout(const tq_ctx* ctx, int batch, int q_len, int num_q_heads, int num_kv_heads, int max_seq_len,
                    int block_size, size_t q_elem, PrefillLayout* l) {
  const size_t rows = (size_t)batch * q_len * num_q_heads;
  const size_t tail = (size_t)batch * (q_len - 1);
  const size_t hyb = tq_hybrid_workspace_bytes(ctx, batch, num_q_heads * q_len, num_kv_heads, max_seq_len, block_size);
  if (hyb == 0) return false;
  size_t off = 0;
  l->vq = off;
  off += align256(rows * kHeadDim * q_elem);
  l->vout = off;
  off += align256(rows * kHeadDim * sizeof(float));
  l->plen = off;
  off += align256((size_t)batch * 4);
  l->tlen = off;
  off += align256((size_t)batch * 4);
  l->slots = off;
  off += align256(tail * 8);
  l->tk = off;
  off += align256(tail * num_kv_heads * kHeadDim * sizeof(float));
  l->tv = off;
  off += align256(tail * num_kv_heads * kHeadDim * sizeof(float));
  l->hyb = off;
  off += hyb;
  l->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t tq_prefill_workspace_bytes(const tq_ctx* ctx, int batch, int q_len, int num_q_heads, int num_kv_heads,
                                  int max_seq_len, int block_size) {
  if (batch <= 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return 0;
  PrefillLayout l;
  if (!prefill_layout(ctx, batch, q_len, num_q_heads, num_kv_heads, max_seq_len, block_size, 4, &l)) return 0;
  return l.total;  // sized for fp32 queries, which covers fp16 / bf16
}

tq_status tq_paged_prefill(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch, int q_len,
                           const int32_t* q_lens, int num_q_heads, int num_kv_heads, const uint8_t* k_pages,
                           int k_bits, const uint8_t* v_pages, int v_bits, int64_t num_blocks, int block_size,
                           const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                           int max_seq_len, float scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!ctx || batch < 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_seq_len < 0 || block_size <= 0)
    return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_F16 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return TQ_ERR_INVALID_ARG;
  if ((long long)(num_q_heads / num_kv_heads) * q_len > tq::kMaxGroup) return TQ_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size < max_seq_len) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  if (!q || !q_lens || !seq_lens || !block_table || !out) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(out) & 15) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return TQ_ERR_ALIGNMENT;
  PrefillLayout l;
  if (!prefill_layout(ctx, batch, q_len, num_q_heads, num_kv_heads, max_seq_len, block_size, 4, &l))
    return TQ_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < l.total) return TQ_ERR_WORKSPACE;
  if (!bits_ok(k_bits) || !bits_ok(v_bits) || block_size != tq::kBlockSize) return TQ_ERR_UNSUPPORTED;
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const hipStream_t st = (hipStream_t)stream;
  tq::PrefillArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.q_lens = q_lens;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.vq = ws + l.vq;
  a.prefix_lens = reinterpret_cast<int32_t*>(ws + l.plen);
  a.tail_lens = reinterpret_cast<int32_t*>(ws + l.tlen);
  a.tail_slots = reinterpret_cast<int64_t*>(ws + l.slots);
  a.vout = reinterpret_cast<float*>(ws + l.vout);
  a.out = out;
  a.batch = batch;
  a.q_len = q_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_size;
  a.max_len = (int)std::min<long long>((long long)max_blocks_per_seq * block_size, 0x7fffffffLL);
  a.q_dtype = (int)q_dtype;
  tq_status s = hip_status(tq::launch_prefill_prep(a, st));
  if (s != TQ_OK) return s;
  const int tail = q_len - 1;
  if (tail > 0) {  // the chunk's tokens after the shared prefix, read back densely
    s = tq_decompress_kv(ctx, k_pages, num_blocks, block_size, num_kv_heads, k_bits, a.tail_slots,
                         (int64_t)batch * tail, ws + l.tk, TQ_F32, nullptr, stream);
    if (s != TQ_OK) return s;
    s = tq_decompress_kv(ctx, v_pages, num_blocks, block_size, num_kv_heads, v_bits, a.tail_slots,
                         (int64_t)batch * tail, ws + l.tv, TQ_F32, nullptr, stream);
    if (s != TQ_OK) return s;
  }
  const int vheads = num_q_heads * q_len;
  float* lse = reinterpret_cast<float*>(
      ws + l.hyb + align256(tq_decode_workspace_bytes(ctx, batch, vheads, num_kv_heads, max_seq_len, block_size)));
  s = decode_impl(ctx, a.vq, q_dtype, batch, vheads, num_kv_heads, k_pages, k_bits, v_pages, v_bits, num_blocks,
                  block_size, block_table, max_blocks_per_seq, a.prefix_lens, max_seq_len, scale,
                  const_cast<float*>(a.vout), lse, ws + l.hyb, l.total - l.hyb, stream);
  if (s != TQ_OK) return s;
  if (tail > 0) {
    tq::HybridArgs h;
    std::memset(&h, 0, sizeof(h));
    h.q = a.vq;
    h.recent_k = ws + l.tk;
    h.recent_v = ws + l.tv;
    h.recent_lens = a.tail_lens;
    h.lse = lse;
    h.out = const_cast<float*>(a.vout);
    h.batch = batch;
    h.num_q_heads = vheads;
    h.num_kv_heads = num_kv_heads;
    h.group = vheads / num_kv_heads;
    h.cap = tail;
    h.q_dtype = (int)q_dtype;
    h.r_dtype = (int)TQ_F32;
    h.causal_group = num_q_heads / num_kv_heads;
    const float sm_scale = scale > 0 ? scale : 1.0f / std::sqrt((float)kHeadDim);
    h.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
    s = hip_status(tq::launch_hybrid(h, st));
    if (s != TQ_OK) return s;
  }
  return hip_status(tq::launch_prefill_out(a, st));
}

tq_status tq_paged_decode_noalloc(const tq_ctx* ctx, const void* q, tq_dtype q_dtype, int batch,
                                  int num_q_heads, int num_kv_heads, const uint8_t* k_pages, int k_bits,
                                  const uint8_t* v_pages, int v_bits, int64_t num_blocks, int block_size,
                                  const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                                  int max_seq_len, float scale, float* out, void* stream) {
  if (!ctx || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  const size_t need = tq_decode_workspace_bytes(ctx, batch, num_q_heads, num_kv_heads, max_seq_len, block_size);
  if (need > tq::scratch_bytes()) return TQ_ERR_WORKSPACE;  // beyond the static scratch
  if (!device_is_gfx950()) return TQ_ERR_NO_DEVICE;
  hipError_t e = hipSuccess;
  void* ws = tq::scratch_device_ptr(&e);
  if (!ws) return hip_status(e);
  return tq_paged_decode(ctx, q, q_dtype, batch, num_q_heads, num_kv_heads, k_pages, k_bits, v_pages, v_bits,
                         num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len, scale, out,
                         ws, tq::scratch_bytes(), stream);
}

}  // extern "C"
