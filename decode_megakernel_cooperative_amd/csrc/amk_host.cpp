// Host side of the decode library: validation, weight packing and W8A16 quantization, upload,
// RoPE tables, scratch, cooperative launch and error mapping behind the C ABI in amk.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "amk.h"
#include "amk_kparams.h"

extern "C" __attribute__((visibility("hidden"))) const void* amk_kernel_handle(int head_dim, int fmt, int gmax, int cg);
extern "C" __attribute__((visibility("hidden"))) const void* amk_clear_kernel_handle();
extern "C" __attribute__((visibility("hidden"))) hipError_t amk_static_scratch(void** ptr, size_t* bytes);

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& what) {
  g_last_error = what;
  return code;
}

#define HIP_TRY(call)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail(e_ == hipErrorOutOfMemory ? AMK_ERR_OOM : AMK_ERR_HIP,                    \
                  std::string(#call) + ": " + hipGetErrorString(e_));                       \
  } while (0)

constexpr uint64_t kDefaultSpinLimit = 100000000ull;  // 1 s at the 100 MHz wall clock

inline float bf16_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Quantizes rows [r0, r1) of a bf16 matrix: s = amax / 127 (IEEE fp32 division), q =
// clamp(nearbyint(w / s), -127, 127) with the default round-to-nearest-even mode.
// Symmetric per-row quantizer with codes in [-qmax, qmax] (127: int8, 7: int4).
void quantize_rows(const uint16_t* w, int64_t cols, int64_t r0, int64_t r1, int8_t* codes, float* scales,
                   float qmax) {
  for (int64_t r = r0; r < r1; ++r) {
    const uint16_t* row = w + r * cols;
    float amax = 0.f;
    for (int64_t c = 0; c < cols; ++c) amax = std::max(amax, std::fabs(bf16_to_float(row[c])));
    int8_t* out = codes + r * cols;
    if (amax == 0.f) {
      scales[r] = 0.f;
      std::memset(out, 0, static_cast<size_t>(cols));
      continue;
    }
    volatile float denom = qmax;  // keep a true division (never a reciprocal multiply)
    const float s = amax / denom;
    scales[r] = s;
    for (int64_t c = 0; c < cols; ++c) {
      float q = std::nearbyint(bf16_to_float(row[c]) / s);
      q = std::min(qmax, std::max(-qmax, q));
      out[c] = static_cast<int8_t>(q);
    }
  }
}

// fp32 -> IEEE half, round to nearest even, for finite |f| <= 65504 (the group-scale range).
uint16_t f32_to_f16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
  if (a < 0x38800000u) {  // below 2^-14: a multiple of 2^-24 (the exact scaling rounds once)
    const float m = std::nearbyint(std::fabs(f) * 16777216.0f);
    return static_cast<uint16_t>(sign | static_cast<uint32_t>(m));  // 1024 encodes 2^-14 itself
  }
  const uint32_t r = a + 0xfffu + ((a >> 13) & 1u);  // round the 13 dropped bits to nearest even
  return static_cast<uint16_t>(sign | ((r - (112u << 23)) >> 13));
}
float f16_to_f32(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  const float v = e == 0 ? std::ldexp(static_cast<float>(m), -24) : std::ldexp(static_cast<float>(1024 + m), e - 25);
  return (h & 0x8000u) ? -v : v;
}

constexpr int64_t kGroup = 128;  // columns per int4 group scale

// Group-wise int4 quantizer for rows [r0, r1): per 128-column group, s = fp16(amax / 7) (IEEE
// fp32 division, then nearest-even half; saturating at 65504), q = clamp(nearbyint(w / s), -7,
// 7); s == 0 gives q = 0. scales: fp32 [rows][ceil(cols / 128)] holding the half values.
void quantize_groups(const uint16_t* w, int64_t cols, int64_t r0, int64_t r1, int8_t* codes, float* scales) {
  const int64_t ng = (cols + kGroup - 1) / kGroup;
  for (int64_t r = r0; r < r1; ++r) {
    const uint16_t* row = w + r * cols;
    int8_t* out = codes + r * cols;
    for (int64_t g = 0; g < ng; ++g) {
      const int64_t c0 = g * kGroup, c1 = std::min(cols, c0 + kGroup);
      float amax = 0.f;
      for (int64_t c = c0; c < c1; ++c) amax = std::max(amax, std::fabs(bf16_to_float(row[c])));
      volatile float denom = 7.0f;  // a true division
      const float s = f16_to_f32(f32_to_f16(std::min(amax / denom, 65504.0f)));
      scales[r * ng + g] = s;
      for (int64_t c = c0; c < c1; ++c) {
        float q = 0.f;
        if (s != 0.f) q = std::min(7.0f, std::max(-7.0f, std::nearbyint(bf16_to_float(row[c]) / s)));
        out[c] = static_cast<int8_t>(q);
      }
    }
  }
}

// Bytes of a format-3 (group-scaled int4) matrix's packed scales: 64 per row pair and 2048-column
// chunk.
inline int64_t gscale_bytes(int64_t rows, int64_t cols) { return rows / 2 * ((cols + 2047) / 2048) * 64; }

template <typename F>
void parallel_rows(int64_t rows, F&& f) {
  const unsigned hw = std::max(1u, std::min(32u, std::thread::hardware_concurrency()));
  const int64_t nt = std::min<int64_t>(hw, std::max<int64_t>(1, rows / 64));
  if (nt <= 1) {
    f(0, rows);
    return;
  }
  std::vector<std::thread> th;
  for (int64_t t = 0; t < nt; ++t) {
    const int64_t a = rows * t / nt, b = rows * (t + 1) / nt;
    th.emplace_back([&f, a, b] { f(a, b); });
  }
  for (auto& t : th) t.join();
}

}  // namespace

struct amk_model {
  amk_config cfg{};
  int device = 0;
  int grid = 0;
  int lds_bytes = 0;
  int gmax = 4;
  int cg = 2;               // chunk slots per GEMV item of the kernel variant
  int s_cap = 1;
  uint32_t tag0 = 1;        // tag base of the next launch
  const void* kernel = nullptr;
  uint64_t spin_limit = kDefaultSpinLimit;
  uint64_t* trace = nullptr;
  int32_t trace_stride = 0;
  // device memory
  uint8_t* weights = nullptr;
  size_t weight_bytes = 0;
  uint8_t* scratch = nullptr;
  size_t scratch_bytes = 0;
  unsigned* herr = nullptr;  // pinned host word the first failing block of a launch writes its code to
  uint8_t* static_scratch = nullptr;  // this device's static exchange array (amk_decode_step_noalloc)
  size_t static_bytes = 0;
  float* dump = nullptr;     // per-stage dump (amk_set_dump), or null
  int64_t dump_layer = 0;    // floats per layer of the dump
  amk::KParams kp{};  // pointers and dims filled at load; step fields filled per call
  // packing metadata for export
  size_t off_qkv = 0, off_o = 0, off_gu = 0, off_d = 0, off_lm = 0;
  size_t off_sqkv = 0, off_so = 0, off_sgu = 0, off_sd = 0, off_slm = 0;
};

namespace {

int validate_config(const amk_config* c) {
  if (!c) return fail(AMK_ERR_INVALID_ARG, "null config");
  if (c->hidden <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->ffn <= 0 || c->vocab <= 0 || c->max_ctx <= 0)
    return fail(AMK_ERR_UNSUPPORTED, "non-positive dimension");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(AMK_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->n_q_heads % c->n_kv_heads != 0) return fail(AMK_ERR_UNSUPPORTED, "n_q_heads % n_kv_heads != 0");
  if (c->n_q_heads / c->n_kv_heads > 8) return fail(AMK_ERR_UNSUPPORTED, "more than 8 query heads per kv head");
  if (c->hidden % 16 || c->ffn % 16 || (c->n_q_heads * c->head_dim) % 16)
    return fail(AMK_ERR_UNSUPPORTED, "hidden, ffn and n_q_heads*head_dim must be multiples of 16");
  if (c->hidden > 8192) return fail(AMK_ERR_UNSUPPORTED, "hidden > 8192");
  if (c->ffn > 32768 || c->n_q_heads * c->head_dim > 32768) return fail(AMK_ERR_UNSUPPORTED, "ffn or q dim > 32768");
  if (c->vocab % 2) return fail(AMK_ERR_UNSUPPORTED, "vocab must be even");
  if (c->weight_format != AMK_BF16 && c->weight_format != AMK_W8A16 && c->weight_format != AMK_W8A16_BF16_HEAD &&
      c->weight_format != AMK_W4A16 && c->weight_format != AMK_W4A16_G128)
    return fail(AMK_ERR_UNSUPPORTED, "weight_format");
  const bool int4 = c->weight_format == AMK_W4A16 || c->weight_format == AMK_W4A16_G128;
  if (int4 && (c->hidden % 32 || c->ffn % 32 || (c->n_q_heads * c->head_dim) % 32))
    return fail(AMK_ERR_UNSUPPORTED, "int4 weights need hidden, ffn and n_q_heads*head_dim multiples of 32");
  if (c->rope_scale_factor > 1.0f &&
      !(c->rope_low_freq_factor > 0.0f && c->rope_high_freq_factor > c->rope_low_freq_factor &&
        c->rope_original_ctx > 0))
    return fail(AMK_ERR_UNSUPPORTED, "rope scaling parameters");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(AMK_ERR_UNSUPPORTED, "rms_eps / rope_theta");
  // the kernel addresses every packed matrix, the embedding and each (layer, K/V, kv head) block
  // of the cache through buffer resources with 32-bit byte offsets
  const int64_t H = c->hidden, F = c->ffn, V = c->vocab, hd = c->head_dim;
  const int64_t QD = c->n_q_heads * hd, QKV = QD + 2 * c->n_kv_heads * hd;
  const int64_t pbits = c->weight_format == AMK_BF16 ? 16 : (int4 ? 4 : 8);
  const int64_t lm_bits = c->weight_format == AMK_W8A16 ? 8 : 16;
  const int64_t lim = int64_t(1) << 31;
  if (QKV * H * pbits / 8 >= lim || H * QD * pbits / 8 >= lim || 2 * F * H * pbits / 8 >= lim ||
      H * F * pbits / 8 >= lim || V * H * lm_bits / 8 >= lim || V * H * 2 >= lim ||
      static_cast<int64_t>(c->max_ctx) * hd * 2 >= lim)
    return fail(AMK_ERR_UNSUPPORTED, "a weight matrix, the embedding or a KV-cache block reaches 2^31 bytes");
  return AMK_OK;
}

// Conditions on the grid (one persistent block per compute unit) that the tagged hand-offs rely
// on. An exchange word is overwritten by the next stage of the same kind, one layer later; every
// block that polls it must have finished before that. A block's stages run in order, so it holds
// up the overwriting stage if it produces some value on the way to it: with the strided row map
// block b owns row pair b of every GEMV stage, so fewer pairs than blocks in the gate/up stage
// (between the x-after-O poll and the down stage that rewrites x) or, with two or more layers, in
// the QKV stage (between the x-after-down poll and the next O stage) would let a block without
// rows fall behind. Attention units are one per block, so nkv cannot exceed the grid.
int validate_grid(const amk_config& c, int grid) {
  const int64_t qkv_pairs = static_cast<int64_t>(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim / 2;
  if (c.n_kv_heads > grid) return fail(AMK_ERR_UNSUPPORTED, "n_kv_heads exceeds the number of compute units");
  if (c.ffn < grid) return fail(AMK_ERR_UNSUPPORTED, "ffn below the number of compute units");
  if (c.n_layers >= 2 && qkv_pairs < grid)
    return fail(AMK_ERR_UNSUPPORTED, "(n_q_heads + 2 n_kv_heads) * head_dim / 2 below the number of compute units");
  return AMK_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Eight int4 codes (q in [-7, 7], columns c .. c + 7) as one 32-bit word for the kernel's fp8
// decode. Byte k holds |q_k| in bits 0..2 and the sign of q_k in bit 7, |q_(k+4)| in bits 4..6,
// and the sign of q_((k+3) mod 4 + 4) in bit 3. Masking the word, and the word rotated right by 4,
// with 0x87878787 then yields four e4m3 codes each whose values are q * 2^-9 in column order.
uint32_t pack_int4_word(const int8_t* q) {
  uint32_t w = 0;
  for (int k = 0; k < 4; ++k) {
    const int a = q[k], b = q[k + 4];
    w |= static_cast<uint32_t>(a < 0 ? -a : a) << (8 * k);
    w |= static_cast<uint32_t>(a < 0) << (8 * k + 7);
    w |= static_cast<uint32_t>(b < 0 ? -b : b) << (8 * k + 4);
    w |= static_cast<uint32_t>(b < 0) << ((8 * k + 11) % 32);
  }
  return w;
}
void unpack_int4_word(uint32_t w, int8_t* q) {
  for (int k = 0; k < 4; ++k) {
    const int a = static_cast<int>((w >> (8 * k)) & 7u), b = static_cast<int>((w >> (8 * k + 4)) & 7u);
    q[k] = static_cast<int8_t>((w >> (8 * k + 7)) & 1u ? -a : a);
    q[k + 4] = static_cast<int8_t>((w >> ((8 * k + 11) % 32)) & 1u ? -b : b);
  }
}

// Row order of the packed QKV matrix: pair p = (head block hb, i) occupies rows 2p, 2p+1 and
// holds source rows hb*hd + i and hb*hd + i + hd/2 (head blocks: nq query, nkv key, nkv value).
// Returns the source (tensor offset 0 = q, 1 = k, 2 = v) and row for packed row r.
inline void qkv_source(const amk_config& c, int64_t r, int* which, int64_t* src_row) {
  const int hd = c.head_dim, half = hd / 2;
  const int64_t pr = r / 2;
  const int64_t hb = pr / half, i = pr % half;
  const int64_t row_in_head = (r & 1) ? i + half : i;
  if (hb < c.n_q_heads) {
    *which = 0;
    *src_row = hb * hd + row_in_head;
  } else if (hb < c.n_q_heads + c.n_kv_heads) {
    *which = 1;
    *src_row = (hb - c.n_q_heads) * hd + row_in_head;
  } else {
    *which = 2;
    *src_row = (hb - c.n_q_heads - c.n_kv_heads) * hd + row_in_head;
  }
}

}  // namespace

extern "C" {

const char* amk_status_string(int status) {
  static thread_local std::string s;
  const char* base = "unknown status";
  switch (status) {
    case AMK_OK: base = "ok"; break;
    case AMK_ERR_INVALID_ARG: base = "invalid argument"; break;
    case AMK_ERR_UNSUPPORTED: base = "unsupported model or format"; break;
    case AMK_ERR_HIP: base = "HIP runtime error"; break;
    case AMK_ERR_COOPERATIVE: base = "persistent grid cannot be co-resident"; break;
    case AMK_ERR_SYNC_TIMEOUT: base = "a grid-level wait (hand-off poll or barrier) timed out on the device"; break;
    case AMK_ERR_OOM: base = "out of memory"; break;
  }
  s = base;
  if (status != AMK_OK && !g_last_error.empty()) s += ": " + g_last_error;
  return s.c_str();
}

int amk_validate_config(const amk_config* cfg, int32_t compute_units) {
  const int st = validate_config(cfg);
  if (st) return st;
  if (compute_units <= 0) return fail(AMK_ERR_INVALID_ARG, "compute_units must be positive");
  return validate_grid(*cfg, compute_units);
}

int amk_quantize_int8(const uint16_t* w, int64_t rows, int64_t cols, int8_t* codes, float* scales) {
  if (!w || !codes || !scales) return fail(AMK_ERR_INVALID_ARG, "null pointer");
  if (rows <= 0 || cols <= 0) return fail(AMK_ERR_INVALID_ARG, "non-positive size");
  parallel_rows(rows, [&](int64_t a, int64_t b) { quantize_rows(w, cols, a, b, codes, scales, 127.0f); });
  return AMK_OK;
}

int amk_quantize_int4(const uint16_t* w, int64_t rows, int64_t cols, int8_t* codes, float* scales) {
  if (!w || !codes || !scales) return fail(AMK_ERR_INVALID_ARG, "null pointer");
  if (rows <= 0 || cols <= 0) return fail(AMK_ERR_INVALID_ARG, "non-positive size");
  parallel_rows(rows, [&](int64_t a, int64_t b) { quantize_rows(w, cols, a, b, codes, scales, 7.0f); });
  return AMK_OK;
}

int amk_quantize_int4_g128(const uint16_t* w, int64_t rows, int64_t cols, int8_t* codes, float* scales) {
  if (!w || !codes || !scales) return fail(AMK_ERR_INVALID_ARG, "null pointer");
  if (rows <= 0 || cols <= 0) return fail(AMK_ERR_INVALID_ARG, "non-positive size");
  parallel_rows(rows, [&](int64_t a, int64_t b) { quantize_groups(w, cols, a, b, codes, scales); });
  return AMK_OK;
}

int amk_load_weights(const amk_config* cfg, const uint16_t* const* t, int32_t n_tensors, amk_model** out) {
  if (!out) return fail(AMK_ERR_INVALID_ARG, "null out");
  *out = nullptr;
  int st = validate_config(cfg);
  if (st) return st;
  const amk_config c = *cfg;
  const int L = c.n_layers;
  const int expected = 2 + 9 * L + (c.tied_embeddings ? 0 : 1);
  if (!t || n_tensors != expected) return fail(AMK_ERR_INVALID_ARG, "expected " + std::to_string(expected) + " tensors");
  for (int i = 0; i < n_tensors; ++i)
    if (!t[i]) return fail(AMK_ERR_INVALID_ARG, "null tensor " + std::to_string(i));

  const int64_t H = c.hidden, F = c.ffn, V = c.vocab, hd = c.head_dim;
  const int64_t QD = c.n_q_heads * hd, KD = c.n_kv_heads * hd;
  const int64_t QKV = QD + 2 * KD;
  const bool q8 = c.weight_format != AMK_BF16;         // quantized projections (int8 or int4)
  const bool lm_q8 = c.weight_format == AMK_W8A16;     // int8 lm_head
  const bool grp = c.weight_format == AMK_W4A16_G128;  // int4 with group scales
  const int pbits = c.weight_format == AMK_BF16 ? 16 : (c.weight_format == AMK_W4A16 || grp ? 4 : 8);  // projections
  const int kfmt = pbits == 16 ? 0 : (pbits == 8 ? 1 : (grp ? 3 : 2));  // kernel weight format

  auto m = new amk_model();
  m->cfg = c;
  hipError_t he = hipGetDevice(&m->device);
  if (he != hipSuccess) { delete m; return fail(AMK_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he)); }
  hipDeviceProp_t prop;
  he = hipGetDeviceProperties(&prop, m->device);
  if (he != hipSuccess) { delete m; return fail(AMK_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(he)); }
  int coop = 0;
  hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, m->device);
  if (!coop) { delete m; return fail(AMK_ERR_COOPERATIVE, "device does not support cooperative launch"); }

  // ---------------- layout ----------------
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t l_qkv = static_cast<size_t>(QKV * H * pbits / 8), l_o = static_cast<size_t>(H * QD * pbits / 8);
  const size_t l_gu = static_cast<size_t>(2 * F * H * pbits / 8), l_d = static_cast<size_t>(H * F * pbits / 8);
  const size_t off_embed = take(static_cast<size_t>(V * H * 2));
  m->off_qkv = take(l_qkv * L);
  m->off_o = take(l_o * L);
  m->off_gu = take(l_gu * L);
  m->off_d = take(l_d * L);
  const bool lm_shares_embed = !lm_q8 && c.tied_embeddings;
  m->off_lm = lm_shares_embed ? off_embed : take(static_cast<size_t>(V * H * (lm_q8 ? 1 : 2)));
  // per-layer scale bytes: fp32 row scales, or the packed group scales of format 3
  const size_t sl_qkv = static_cast<size_t>(grp ? gscale_bytes(QKV, H) : 4 * QKV);
  const size_t sl_o = static_cast<size_t>(grp ? gscale_bytes(H, QD) : 4 * H);
  const size_t sl_gu = static_cast<size_t>(grp ? gscale_bytes(2 * F, H) : 4 * 2 * F);
  const size_t sl_d = static_cast<size_t>(grp ? gscale_bytes(H, F) : 4 * H);
  if (q8) {
    m->off_sqkv = take(sl_qkv * L);
    m->off_so = take(sl_o * L);
    m->off_sgu = take(sl_gu * L);
    m->off_sd = take(sl_d * L);
  }
  if (lm_q8) m->off_slm = take(4 * V);
  const size_t off_nin = take(4 * H * L), off_npost = take(4 * H * L), off_nfin = take(4 * H);
  const size_t off_cos = take(4 * static_cast<size_t>(c.max_ctx) * (hd / 2));
  const size_t off_sin = take(4 * static_cast<size_t>(c.max_ctx) * (hd / 2));
  m->weight_bytes = off;

  // grid / LDS / splits
  m->grid = prop.multiProcessorCount;
  st = validate_grid(c, m->grid);
  if (st) { delete m; return st; }
  const int G = c.n_q_heads / c.n_kv_heads;
  m->gmax = G <= 4 ? 4 : 8;
  // split cap: one attention unit per block, and the split merge puts the splits of one output
  // on the lanes of a wave, so at most 64
  m->s_cap = std::min(64, std::max(1, m->grid / c.n_kv_heads));
  const int cw = 8192 / pbits;  // columns per 1 KB weight chunk
  auto pad = [&](int64_t k) { return (k + cw - 1) / cw * cw; };
  const int64_t xs_f = std::max({pad(H), pad(QD), pad(F)});
  {
    // the GEMV input vector, or the attention stage's tiles, results, q and K/V(pos)
    const int64_t attn_b = amk::attn_lds_bytes(static_cast<int>(hd), m->gmax, G);
    m->lds_bytes = static_cast<int>(std::max(4 * xs_f, attn_b));
    // one-slot items (half the reads in flight at each hand-off) for hidden sizes up to 2048,
    // two-slot items (the deeper stream) above
    m->cg = c.hidden <= 2048 ? 1 : 2;
    m->kernel = amk_kernel_handle(static_cast<int>(hd), kfmt, m->gmax, m->cg);
  }
  if (m->lds_bytes > 160 * 1024) { delete m; return fail(AMK_ERR_UNSUPPORTED, "LDS need exceeds 160 KB"); }
  if (!m->kernel) { delete m; return fail(AMK_ERR_UNSUPPORTED, "no kernel variant"); }
  he = hipFuncSetAttribute(m->kernel, hipFuncAttributeMaxDynamicSharedMemorySize, m->lds_bytes);
  if (he != hipSuccess) { delete m; return fail(AMK_ERR_HIP, std::string("hipFuncSetAttribute: ") + hipGetErrorString(he)); }
  int per_cu = 0;
  he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, m->kernel, amk::kThreads, m->lds_bytes);
  if (he != hipSuccess || per_cu < 1) {
    delete m;
    return fail(AMK_ERR_COOPERATIVE, "persistent block does not fit on a compute unit");
  }

  // ---------------- scratch ----------------
  size_t so = 0;
  auto stake = [&](size_t bytes) { size_t o = so; so = align_up(so + bytes, 256); return o; };
  const size_t s_err = stake(4 * amk::kCtrStride);
  // tagged exchange words (8 bytes each; the SwiGLU output uses 4-byte words), one contiguous
  // region so a single buffer resource covers every poll
  const size_t s_tag = so;
  const size_t t_x = stake(8 * H), t_q = stake(8 * QD), t_kv = stake(8 * KD), t_o = stake(8 * QD / 2),
               t_m = stake(8 * F / 2);
  const size_t t_part = stake(8 * static_cast<size_t>(c.n_q_heads) * m->s_cap * (hd + 2));
  const size_t t_arg = stake(16 * static_cast<size_t>(m->grid));
  const size_t s_tag_end = so;
  m->scratch_bytes = so;

  he = hipMalloc(&m->weights, m->weight_bytes);
  if (he != hipSuccess) { delete m; return fail(AMK_ERR_OOM, std::string("hipMalloc(weights): ") + hipGetErrorString(he)); }
  he = hipMalloc(&m->scratch, m->scratch_bytes);
  if (he != hipSuccess) { amk_free(m); return fail(AMK_ERR_OOM, std::string("hipMalloc(scratch): ") + hipGetErrorString(he)); }
  he = hipMemset(m->scratch, 0, m->scratch_bytes);
  if (he != hipSuccess) { amk_free(m); return fail(AMK_ERR_HIP, std::string("hipMemset: ") + hipGetErrorString(he)); }
  // coherent pinned host memory: a system-scope store from the kernel is visible to the host
  // without a synchronisation
  he = hipHostMalloc(reinterpret_cast<void**>(&m->herr), 64, hipHostMallocMapped | hipHostMallocCoherent);
  if (he != hipSuccess) { amk_free(m); return fail(AMK_ERR_OOM, std::string("hipHostMalloc: ") + hipGetErrorString(he)); }
  __atomic_store_n(m->herr, 0u, __ATOMIC_RELEASE);
  unsigned* herr_dev = nullptr;
  he = hipHostGetDevicePointer(reinterpret_cast<void**>(&herr_dev), m->herr, 0);
  if (he != hipSuccess) { amk_free(m); return fail(AMK_ERR_HIP, std::string("hipHostGetDevicePointer: ") + hipGetErrorString(he)); }
  m->dump_layer = 6 * H + QKV + 2 * QD + 3 * F;  // the slots of one layer in the dump
  {  // set-up of the allocation-free step: this device's static exchange array (looked up once)
    void* sp = nullptr;
    size_t sb = 0;
    he = amk_static_scratch(&sp, &sb);
    if (he != hipSuccess) { amk_free(m); return fail(AMK_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(he)); }
    m->static_scratch = static_cast<uint8_t*>(sp);
    m->static_bytes = sb;
  }

  // ---------------- packing + upload ----------------
  std::vector<uint8_t> stage;
  std::vector<int8_t> codes;
  std::vector<float> scales, fbuf;
  int rc = AMK_OK;
  auto upload = [&](size_t dst, const void* src, size_t bytes) -> int {
    hipError_t e = hipMemcpy(m->weights + dst, src, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(AMK_ERR_HIP, std::string("hipMemcpy: ") + hipGetErrorString(e));
    return AMK_OK;
  };
  // Packs rows of one layer's matrix given a row map (packed row -> source pointer).
  // bits: 16 (bf16 rows copied), 8 (int8 codes) or 4 (int4 codes, eight per 32-bit word in the
  // sign-magnitude layout of pack_int4_word); gs: group scales (format 3) instead of row scales
  auto pack_matrix = [&](int bits, bool gs, int64_t rows, int64_t cols, size_t dst_w, size_t dst_s,
                         const std::vector<const uint16_t*>& src_tensors,
                         auto&& row_source) -> int {
    if (bits != 16) {
      // quantize each source tensor in canonical order, then permute rows
      const int64_t ns = gs ? (cols + kGroup - 1) / kGroup : 1;  // scales per row
      std::vector<std::vector<int8_t>> qc(src_tensors.size());
      std::vector<std::vector<float>> qs(src_tensors.size());
      for (size_t k = 0; k < src_tensors.size(); ++k) {
        int64_t r_k = 0;
        for (int64_t r = 0; r < rows; ++r) { int w; int64_t sr; row_source(r, &w, &sr); if (w == static_cast<int>(k)) ++r_k; }
        qc[k].resize(static_cast<size_t>(r_k * cols));
        qs[k].resize(static_cast<size_t>(r_k * ns));
        int e = bits == 8 ? amk_quantize_int8(src_tensors[k], r_k, cols, qc[k].data(), qs[k].data())
                : gs      ? amk_quantize_int4_g128(src_tensors[k], r_k, cols, qc[k].data(), qs[k].data())
                          : amk_quantize_int4(src_tensors[k], r_k, cols, qc[k].data(), qs[k].data());
        if (e) return e;
      }
      codes.resize(static_cast<size_t>(rows * cols));
      scales.resize(static_cast<size_t>(rows * ns));
      for (int64_t r = 0; r < rows; ++r) {
        int w; int64_t sr; row_source(r, &w, &sr);
        std::memcpy(codes.data() + r * cols, qc[w].data() + sr * cols, static_cast<size_t>(cols));
        std::memcpy(scales.data() + r * ns, qs[w].data() + sr * ns, static_cast<size_t>(ns) * 4);
      }
      std::vector<uint16_t> gpk;
      if (gs) {  // pair pr, chunk ch: 16 dwords (row 0 scale | row 1 scale << 16) of groups 16 ch ..
        const int64_t nch = (cols + 2047) / 2048;
        gpk.assign(static_cast<size_t>(gscale_bytes(rows, cols) / 2), 0);
        for (int64_t r = 0; r < rows; ++r)
          for (int64_t g = 0; g < ns; ++g)
            gpk[static_cast<size_t>((((r / 2) * nch + g / 16) * 16 + g % 16) * 2 + (r & 1))] =
                f32_to_f16(scales[static_cast<size_t>(r * ns + g)]);
      }
      if (bits == 4) {  // eight codes per word, in place (word i is written after codes 8i .. 8i + 7 are read)
        const int64_t n = rows * cols / 8;
        for (int64_t i = 0; i < n; ++i) {
          const uint32_t w = pack_int4_word(codes.data() + 8 * i);
          std::memcpy(codes.data() + 4 * i, &w, 4);
        }
      }
      int e = upload(dst_w, codes.data(), static_cast<size_t>(rows * cols * bits / 8));
      if (e) return e;
      if (gs) return upload(dst_s, gpk.data(), gpk.size() * 2);
      return upload(dst_s, scales.data(), static_cast<size_t>(rows) * 4);
    }
    stage.resize(static_cast<size_t>(rows * cols * 2));
    for (int64_t r = 0; r < rows; ++r) {
      int w; int64_t sr; row_source(r, &w, &sr);
      std::memcpy(stage.data() + r * cols * 2, src_tensors[w] + sr * cols, static_cast<size_t>(cols * 2));
    }
    return upload(dst_w, stage.data(), stage.size());
  };

  rc = upload(off_embed, t[0], static_cast<size_t>(V * H * 2));
  std::vector<float> nin(static_cast<size_t>(H * L)), npost(static_cast<size_t>(H * L)), nfin(static_cast<size_t>(H));
  for (int l = 0; l < L && rc == AMK_OK; ++l) {
    const uint16_t* const* lt = t + 1 + 9 * l;
    for (int64_t i = 0; i < H; ++i) {
      nin[static_cast<size_t>(l * H + i)] = bf16_to_float(lt[0][i]);
      npost[static_cast<size_t>(l * H + i)] = bf16_to_float(lt[5][i]);
    }
    rc = pack_matrix(pbits, grp, QKV, H, m->off_qkv + l * l_qkv, m->off_sqkv + sl_qkv * l, {lt[1], lt[2], lt[3]},
                     [&](int64_t r, int* w, int64_t* sr) { qkv_source(c, r, w, sr); });
    if (rc) break;
    rc = pack_matrix(pbits, grp, H, QD, m->off_o + l * l_o, m->off_so + sl_o * l, {lt[4]},
                     [&](int64_t r, int* w, int64_t* sr) { *w = 0; *sr = r; });
    if (rc) break;
    rc = pack_matrix(pbits, grp, 2 * F, H, m->off_gu + l * l_gu, m->off_sgu + sl_gu * l, {lt[6], lt[7]},
                     [&](int64_t r, int* w, int64_t* sr) { *w = static_cast<int>(r & 1); *sr = r >> 1; });
    if (rc) break;
    rc = pack_matrix(pbits, grp, H, F, m->off_d + l * l_d, m->off_sd + sl_d * l, {lt[8]},
                     [&](int64_t r, int* w, int64_t* sr) { *w = 0; *sr = r; });
  }
  if (rc == AMK_OK) {
    for (int64_t i = 0; i < H; ++i) nfin[static_cast<size_t>(i)] = bf16_to_float(t[1 + 9 * L][i]);
    const uint16_t* lm = c.tied_embeddings ? t[0] : t[2 + 9 * L];
    if (!lm_shares_embed)
      rc = pack_matrix(lm_q8 ? 8 : 16, false, V, H, m->off_lm, m->off_slm, {lm},
                       [&](int64_t r, int* w, int64_t* sr) { *w = 0; *sr = r; });
  }
  if (rc == AMK_OK) rc = upload(off_nin, nin.data(), nin.size() * 4);
  if (rc == AMK_OK) rc = upload(off_npost, npost.data(), npost.size() * 4);
  if (rc == AMK_OK) rc = upload(off_nfin, nfin.data(), nfin.size() * 4);
  if (rc == AMK_OK) {
    // RoPE: inv_freq_i = theta^(-2i/hd) (then the Llama-3 frequency scaling, if configured) and
    // angle = pos * inv_freq_i in double, rounded once
    const int64_t half = hd / 2;
    std::vector<double> inv_freq(static_cast<size_t>(half));
    const double kPi = 3.14159265358979323846;
    for (int64_t i = 0; i < half; ++i) {
      double f = std::pow(static_cast<double>(c.rope_theta), -2.0 * static_cast<double>(i) / static_cast<double>(hd));
      if (c.rope_scale_factor > 1.0f) {
        const double factor = c.rope_scale_factor, lo = c.rope_low_freq_factor, hi = c.rope_high_freq_factor;
        const double orig = c.rope_original_ctx, wavelen = 2.0 * kPi / f;
        if (wavelen > orig / lo) {
          f = f / factor;
        } else if (wavelen >= orig / hi) {
          const double t = (orig / wavelen - lo) / (hi - lo);
          f = (1.0 - t) * f / factor + t * f;
        }
      }
      inv_freq[static_cast<size_t>(i)] = f;
    }
    std::vector<float> cs(static_cast<size_t>(c.max_ctx * half)), sn(cs.size());
    for (int64_t pos = 0; pos < c.max_ctx; ++pos)
      for (int64_t i = 0; i < half; ++i) {
        const double a = static_cast<double>(pos) * inv_freq[static_cast<size_t>(i)];
        cs[static_cast<size_t>(pos * half + i)] = static_cast<float>(std::cos(a));
        sn[static_cast<size_t>(pos * half + i)] = static_cast<float>(std::sin(a));
      }
    rc = upload(off_cos, cs.data(), cs.size() * 4);
    if (rc == AMK_OK) rc = upload(off_sin, sn.data(), sn.size() * 4);
  }
  if (rc != AMK_OK) {
    std::string keep = g_last_error;
    amk_free(m);
    g_last_error = keep;
    return rc;
  }

  // ---------------- kernel parameters ----------------
  amk::KParams& k = m->kp;
  k.H = static_cast<int32_t>(H); k.L = L; k.nq = c.n_q_heads; k.nkv = c.n_kv_heads; k.hd = static_cast<int32_t>(hd);
  k.F = static_cast<int32_t>(F); k.V = static_cast<int32_t>(V); k.max_ctx = c.max_ctx;
  k.eps = c.rms_eps;
  k.attn_scale = 1.0f / std::sqrt(static_cast<float>(hd));
  uint8_t* W = m->weights;
  k.w_qkv = W + m->off_qkv; k.w_qkv_ls = static_cast<int64_t>(l_qkv);
  k.w_o = W + m->off_o; k.w_o_ls = static_cast<int64_t>(l_o);
  k.w_gu = W + m->off_gu; k.w_gu_ls = static_cast<int64_t>(l_gu);
  k.w_d = W + m->off_d; k.w_d_ls = static_cast<int64_t>(l_d);
  k.w_lm = W + m->off_lm;
  if (q8) {
    // layer strides in floats (the packed group scales are whole dwords too)
    k.s_qkv = reinterpret_cast<const float*>(W + m->off_sqkv); k.s_qkv_ls = static_cast<int64_t>(sl_qkv / 4);
    k.s_o = reinterpret_cast<const float*>(W + m->off_so); k.s_o_ls = static_cast<int64_t>(sl_o / 4);
    k.s_gu = reinterpret_cast<const float*>(W + m->off_sgu); k.s_gu_ls = static_cast<int64_t>(sl_gu / 4);
    k.s_d = reinterpret_cast<const float*>(W + m->off_sd); k.s_d_ls = static_cast<int64_t>(sl_d / 4);
  }
  if (lm_q8) k.s_lm = reinterpret_cast<const float*>(W + m->off_slm);
  k.lm_fmt = lm_q8 ? 1 : 0;
  k.embed = reinterpret_cast<const uint16_t*>(W + off_embed);
  k.norm_in = reinterpret_cast<const float*>(W + off_nin);
  k.norm_post = reinterpret_cast<const float*>(W + off_npost);
  k.norm_final = reinterpret_cast<const float*>(W + off_nfin);
  k.rope_cos = reinterpret_cast<const float*>(W + off_cos);
  k.rope_sin = reinterpret_cast<const float*>(W + off_sin);
  uint8_t* S = m->scratch;
  k.s_cap = m->s_cap;
  k.err = reinterpret_cast<unsigned*>(S + s_err);
  k.herr = herr_dev;
  k.spin_limit = m->spin_limit;
  k.tagged = reinterpret_cast<uint64_t*>(S + s_tag);
  k.tagged_bytes = static_cast<uint32_t>(s_tag_end - s_tag);
  k.tx = reinterpret_cast<uint64_t*>(S + t_x);
  k.tq = reinterpret_cast<uint64_t*>(S + t_q);
  k.tkv = reinterpret_cast<uint64_t*>(S + t_kv);
  k.to = reinterpret_cast<uint64_t*>(S + t_o);
  k.tm = reinterpret_cast<uint64_t*>(S + t_m);
  k.tpart = reinterpret_cast<uint64_t*>(S + t_part);
    k.targ = reinterpret_cast<uint64_t*>(S + t_arg);
  *out = m;
  return AMK_OK;
}

namespace {
// Enqueues on `stream` the reset of the model's device state after a failed step: the error flag
// and every exchange word go back to zero (after every launch already enqueued), and the tags
// restart at 1, above the zero of a cleared word.
int enqueue_clear(uint8_t* base, size_t bytes, void* stream) {
  uint32_t* p = reinterpret_cast<uint32_t*>(base);
  size_t n = bytes / 4;
  void* args[] = {&p, &n};
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>(1024, (n + 255) / 256));
  HIP_TRY(hipLaunchKernel(amk_clear_kernel_handle(), dim3(blocks), dim3(256), args, 0, static_cast<hipStream_t>(stream)));
  return AMK_OK;
}
int enqueue_reset(amk_model* m, void* stream) {
  const int rc = enqueue_clear(m->scratch, m->scratch_bytes, stream);
  if (rc) return rc;
  m->tag0 = 1;
  return AMK_OK;
}

// Error code of a device failure as an ABI status (with its description).
int device_error_status(unsigned code) {
  if (code == amk::kErrBadToken) return fail(AMK_ERR_INVALID_ARG, "a greedy step read a device token outside [0, vocab)");
  return fail(AMK_ERR_SYNC_TIMEOUT, "a decode step abandoned a hand-off wait (bounded poll timed out)");
}

// A failure of an earlier step that the device has already reported through the pinned host word
// (read without synchronising): clears the word, enqueues the reset, and returns the error;
// AMK_OK when there is none. Exactly one block of a failed launch writes the word.
int take_pending_error(amk_model* m, void* stream) {
  const unsigned code = __atomic_load_n(m->herr, __ATOMIC_ACQUIRE);
  if (code == 0u) return AMK_OK;
  __atomic_store_n(m->herr, 0u, __ATOMIC_RELEASE);
  const int rc = enqueue_reset(m, stream);
  if (rc) return rc;
  return device_error_status(code);
}

// One decode step: a single cooperative launch. token_dev / next_token are null for a
// host-token step. A pending failure of an earlier step is reported instead of launching.
// With use_static, the launch keeps its exchange words and error flag in the device's static
// array instead of the model's scratch: the used part is cleared first (a kernel, on the stream),
// and the tags start at 1.
int launch_step(amk_model* m, int32_t token, const int32_t* token_dev, int32_t pos, void* kv_cache,
                float* logits_out, int32_t* next_token, void* stream, bool use_static = false) {
  const int pending = take_pending_error(m, stream);
  if (pending) return pending;
  amk::KParams k = m->kp;
  if (use_static) {
    const int rc = enqueue_clear(m->static_scratch, m->scratch_bytes, stream);
    if (rc) return rc;
    auto rebase = [&](auto* p) { return reinterpret_cast<decltype(p)>(m->static_scratch + (reinterpret_cast<uint8_t*>(p) - m->scratch)); };
    k.err = rebase(k.err);
    k.tagged = rebase(k.tagged);
    k.tx = rebase(k.tx);
    k.tq = rebase(k.tq);
    k.tkv = rebase(k.tkv);
    k.tpart = rebase(k.tpart);
    k.to = rebase(k.to);
    k.targ = rebase(k.targ);
    k.tm = rebase(k.tm);
  }
  k.token = token;
  k.token_dev = token_dev;
  k.next_token = next_token;
  k.pos = pos;
  const int ctx = pos + 1;
  // split-KV plan: at most s_cap splits per kv head (one attention unit per block), at least
  // 16 positions per split. A context of at most tstep positions (128 at head_dim 128, 256 at
  // head_dim 64, half that with more than 4 query heads per kv head: one or two 16-position tiles
  // per wave) runs as one split per kv head, which writes the attention output itself, with no
  // merge hand-off.
  const int tstep = amk::kWaves * (m->gmax > 4 ? 2 : 4) * (512 / m->cfg.head_dim);
  int T = std::max(16, (ctx + m->s_cap - 1) / m->s_cap);
  if (ctx <= tstep) T = tstep;
  k.T = T;
  k.S = (ctx + T - 1) / T;
  k.kv = static_cast<uint16_t*>(kv_cache);
  k.logits = logits_out;
  k.spin_limit = m->spin_limit;
  k.trace = m->trace;
  k.trace_stride = m->trace_stride;
  k.dump = m->dump;
  k.dump_stride = m->dump_layer;
  if (use_static) {
    k.tag0 = 1;
  } else {
    // tags are compared for equality, so a wrap of the 32-bit counter would only matter where a
    // launch's tag reached 0, the tag of a cleared word; restart from a cleared state well before
    const uint32_t per_launch = static_cast<uint32_t>(amk::kTagsPerLayer * m->cfg.n_layers + 1);
    if (m->tag0 > UINT32_MAX - 2 * per_launch) {
      const int rc = enqueue_reset(m, stream);
      if (rc) return rc;
    }
    k.tag0 = m->tag0;
    m->tag0 += per_launch;
  }
  void* args[] = {&k};
  HIP_TRY(hipLaunchCooperativeKernel(m->kernel, dim3(m->grid), dim3(amk::kThreads), args,
                                     static_cast<unsigned>(m->lds_bytes), static_cast<hipStream_t>(stream)));
  return AMK_OK;
}
}  // namespace

int amk_decode_step(amk_model* m, int32_t token, int32_t pos, void* kv_cache, float* logits_out, void* stream) {
  if (!m || !kv_cache || !logits_out) return fail(AMK_ERR_INVALID_ARG, "null handle or buffer");
  if (token < 0 || token >= m->cfg.vocab) return fail(AMK_ERR_INVALID_ARG, "token out of range");
  if (pos < 0 || pos >= m->cfg.max_ctx) return fail(AMK_ERR_INVALID_ARG, "pos out of range");
  return launch_step(m, token, nullptr, pos, kv_cache, logits_out, nullptr, stream);
}

int amk_decode_step_noalloc(amk_model* m, int32_t token, int32_t pos, void* kv_cache, float* logits_out,
                            void* stream) {
  if (!m || !kv_cache || !logits_out) return fail(AMK_ERR_INVALID_ARG, "null handle or buffer");
  if (token < 0 || token >= m->cfg.vocab) return fail(AMK_ERR_INVALID_ARG, "token out of range");
  if (pos < 0 || pos >= m->cfg.max_ctx) return fail(AMK_ERR_INVALID_ARG, "pos out of range");
  if (!m->static_scratch) return fail(AMK_ERR_HIP, "the static exchange array was not found at load");
  if (m->scratch_bytes > m->static_bytes)
    return fail(AMK_ERR_UNSUPPORTED, "the model needs " + std::to_string(m->scratch_bytes) +
                                         " bytes of exchange words; the static array holds " +
                                         std::to_string(m->static_bytes));
  return launch_step(m, token, nullptr, pos, kv_cache, logits_out, nullptr, stream, true);
}

int amk_decode_step_greedy(amk_model* m, const int32_t* token_in, int32_t pos, void* kv_cache, float* logits_out,
                           int32_t* next_token_out, void* stream) {
  if (!m || !token_in || !kv_cache || !next_token_out) return fail(AMK_ERR_INVALID_ARG, "null handle or buffer");
  if (pos < 0 || pos >= m->cfg.max_ctx) return fail(AMK_ERR_INVALID_ARG, "pos out of range");
  return launch_step(m, 0, token_in, pos, kv_cache, logits_out, next_token_out, stream);
}

int amk_sync(amk_model* m, void* stream) {
  if (!m) return fail(AMK_ERR_INVALID_ARG, "null handle");
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  int rc = take_pending_error(m, stream);
  if (rc == AMK_OK) {
    // the device flag is the authority; the host word only saves the call a synchronisation
    unsigned err = 0;
    HIP_TRY(hipMemcpy(&err, m->kp.err, 4, hipMemcpyDeviceToHost));
    if (err != 0u) {
      const int r = enqueue_reset(m, stream);
      rc = r ? r : device_error_status(err);
    }
  }
  if (rc != AMK_OK) {
    const std::string keep = g_last_error;
    HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));  // the reset has run
    g_last_error = keep;
  }
  return rc;
}

size_t amk_kv_cache_bytes(const amk_model* m) {
  if (!m) return 0;
  const amk_config& c = m->cfg;
  return static_cast<size_t>(c.n_layers) * 2 * c.n_kv_heads * static_cast<size_t>(c.max_ctx) * c.head_dim * 2;
}

int amk_get_info(const amk_model* m, amk_info* info) {
  if (!m || !info) return fail(AMK_ERR_INVALID_ARG, "null pointer");
  info->grid_blocks = m->grid;
  info->block_threads = amk::kThreads;
  info->lds_bytes = m->lds_bytes;
  // grid-wide tagged vector exchanges per step
  // (streaming kernel: RMSNorm input, q, split partials, attention output, RMSNorm input, SwiGLU
  // output per layer, then the final RMSNorm input)
  info->handoffs_per_step = amk::kTagsPerLayer * m->cfg.n_layers + 1;
  info->weight_bytes = static_cast<int64_t>(m->weight_bytes);
  info->scratch_bytes = static_cast<int64_t>(m->scratch_bytes);
  info->max_splits = m->s_cap;
  info->device = m->device;
  info->dump_layer_floats = m->dump_layer;
  info->dump_floats = m->dump_layer * m->cfg.n_layers + m->cfg.hidden;
  info->gemv_item_slots = m->cg;
  return AMK_OK;
}

int amk_export_quantized(const amk_model* m, int32_t idx, int8_t* codes_out, float* scales_out) {
  if (!m || !codes_out || !scales_out) return fail(AMK_ERR_INVALID_ARG, "null pointer");
  const amk_config& c = m->cfg;
  if (c.weight_format == AMK_BF16) return fail(AMK_ERR_UNSUPPORTED, "model has no quantized weights");
  const int L = c.n_layers;
  const int64_t H = c.hidden, F = c.ffn, V = c.vocab, hd = c.head_dim;
  const int64_t QD = c.n_q_heads * hd, KD = c.n_kv_heads * hd, QKV = QD + 2 * KD;
  const bool grp = c.weight_format == AMK_W4A16_G128;
  const int pbits = c.weight_format == AMK_W4A16 || grp ? 4 : 8;  // projection code width
  auto lb = [&](int64_t n) { return static_cast<size_t>(n * pbits / 8); };  // bytes of n codes
  // bytes of one layer's scales of a matrix
  auto sb = [&](int64_t r, int64_t k) { return static_cast<size_t>(grp ? gscale_bytes(r, k) : 4 * r); };
  const int lm_idx = c.tied_embeddings ? 0 : 2 + 9 * L;
  int64_t rows = 0, cols = 0, mrows = 0;
  size_t wsrc = 0, ssrc = 0;
  int which = -1;           // which source tensor of a fused matrix we export
  int kind = -1;            // 0 qkv, 1 o, 2 gu, 3 d, 4 lm
  if (idx == lm_idx) {
    if (c.weight_format != AMK_W8A16) return fail(AMK_ERR_INVALID_ARG, "the lm_head of this model is not quantized");
    kind = 4; rows = mrows = V; cols = H; wsrc = m->off_lm; ssrc = m->off_slm;
  } else if (idx >= 1 && idx < 1 + 9 * L) {
    const int l = (idx - 1) / 9, o = (idx - 1) % 9;
    switch (o) {
      case 1: case 2: case 3:
        kind = 0; which = o - 1; rows = (o == 1) ? QD : KD; cols = H; mrows = QKV;
        wsrc = m->off_qkv + l * lb(QKV * H); ssrc = m->off_sqkv + sb(QKV, H) * l; break;
      case 4: kind = 1; rows = mrows = H; cols = QD; wsrc = m->off_o + l * lb(H * QD); ssrc = m->off_so + sb(H, QD) * l; break;
      case 6: case 7:
        kind = 2; which = o - 6; rows = F; cols = H; mrows = 2 * F;
        wsrc = m->off_gu + l * lb(2 * F * H); ssrc = m->off_sgu + sb(2 * F, H) * l; break;
      case 8: kind = 3; rows = mrows = H; cols = F; wsrc = m->off_d + l * lb(H * F); ssrc = m->off_sd + sb(H, F) * l; break;
      default: break;
    }
  }
  if (kind < 0) return fail(AMK_ERR_INVALID_ARG, "tensor index is not a quantized matrix");
  const int bits = kind == 4 ? 8 : pbits;
  const bool gs = grp && kind != 4;
  const int64_t ns = gs ? (cols + kGroup - 1) / kGroup : 1;  // scales per row
  std::vector<int8_t> allc(static_cast<size_t>(mrows * cols));
  std::vector<float> alls(static_cast<size_t>(mrows * ns));
  HIP_TRY(hipMemcpy(allc.data(), m->weights + wsrc, static_cast<size_t>(mrows * cols * bits / 8), hipMemcpyDeviceToHost));
  if (gs) {  // unpack the pair-chunk layout of the group scales
    const int64_t nch = (cols + 2047) / 2048;
    std::vector<uint16_t> gpk(static_cast<size_t>(gscale_bytes(mrows, cols) / 2));
    HIP_TRY(hipMemcpy(gpk.data(), m->weights + ssrc, gpk.size() * 2, hipMemcpyDeviceToHost));
    for (int64_t r = 0; r < mrows; ++r)
      for (int64_t g = 0; g < ns; ++g)
        alls[static_cast<size_t>(r * ns + g)] =
            f16_to_f32(gpk[static_cast<size_t>((((r / 2) * nch + g / 16) * 16 + g % 16) * 2 + (r & 1))]);
  } else {
    HIP_TRY(hipMemcpy(alls.data(), m->weights + ssrc, alls.size() * 4, hipMemcpyDeviceToHost));
  }
  if (bits == 4)  // unpack in place from the back: word i holds codes 8i .. 8i + 7
    for (int64_t i = mrows * cols / 8 - 1; i >= 0; --i) {
      uint32_t w;
      std::memcpy(&w, allc.data() + 4 * i, 4);
      unpack_int4_word(w, allc.data() + 8 * i);
    }
  for (int64_t r = 0; r < mrows; ++r) {
    int w = 0;
    int64_t sr = r;
    if (kind == 0) qkv_source(c, r, &w, &sr);
    else if (kind == 2) { w = static_cast<int>(r & 1); sr = r >> 1; }
    if (which >= 0 && w != which) continue;
    std::memcpy(codes_out + sr * cols, allc.data() + r * cols, static_cast<size_t>(cols));
    std::memcpy(scales_out + sr * ns, alls.data() + r * ns, static_cast<size_t>(ns) * 4);
  }
  (void)rows;
  return AMK_OK;
}

int amk_set_spin_limit(amk_model* m, uint64_t ticks) {
  if (!m) return fail(AMK_ERR_INVALID_ARG, "null handle");
  m->spin_limit = ticks ? ticks : kDefaultSpinLimit;
  return AMK_OK;
}

int amk_set_trace(amk_model* m, uint64_t* trace, int32_t events_per_block) {
  if (!m) return fail(AMK_ERR_INVALID_ARG, "null handle");
  const int need = 3 + 11 * m->cfg.n_layers;
  if (trace && events_per_block < need) return fail(AMK_ERR_INVALID_ARG, "events_per_block too small");
  m->trace = trace;
  m->trace_stride = trace ? events_per_block : 0;
  return AMK_OK;
}

int amk_set_dump(amk_model* m, float* dump, int64_t floats) {
  if (!m) return fail(AMK_ERR_INVALID_ARG, "null handle");
  if (dump && floats < m->dump_layer * m->cfg.n_layers + m->cfg.hidden)
    return fail(AMK_ERR_INVALID_ARG, "dump buffer too small");
  m->dump = dump;
  return AMK_OK;
}

int amk_free(amk_model* m) {
  if (!m) return AMK_OK;
  int rc = AMK_OK;
  if (m->herr && hipHostFree(m->herr) != hipSuccess) rc = fail(AMK_ERR_HIP, "hipHostFree(error word)");
  if (m->weights && hipFree(m->weights) != hipSuccess) rc = fail(AMK_ERR_HIP, "hipFree(weights)");
  if (m->scratch && hipFree(m->scratch) != hipSuccess) rc = fail(AMK_ERR_HIP, "hipFree(scratch)");
  delete m;
  return rc;
}

}  // extern "C"
