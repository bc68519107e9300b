// Streaming persistent decode kernel for gfx950 (MI355X): one cooperative launch per token runs
// the whole batch-1 Llama forward pass (RMSNorm, QKV GEMV + RoPE + KV append, split-KV GQA
// attention, O-projection + residual, RMSNorm + SwiGLU gate/up, down + residual, final RMSNorm
// + lm_head).
//
// Method: the decode-megakernel pages (AutoMegaKernel paper index, Abstract; gist.science
// explainer, Technical Summary > Problem Statement and Methodology) fuse the forward pass into
// one persistent kernel whose blocks synchronise through memory flags instead of kernel
// boundaries and prefetch the next weights while computing. On MI355X the step time is decided
// by the chain of cross-block hand-offs (one per GEMV input vector) and by how much of the
// weight stream overlaps it. Two measured facts shape this file:
//
//  * A compute unit returns vector-memory loads in issue order. A load issued behind the unit's
//    in-flight weight loads waits for all of them (about 1 us at full HBM rate), while the same
//    load from an idle unit takes about 0.1 us, however busy the rest of the chip is.
//  * A grid barrier built from store acknowledgements and counters costs four such round trips.
//
// Design:
//  * Tagged hand-offs. Every value that crosses blocks is a 64-bit word: a 32-bit payload (one
//    fp32, or two bf16) and a 32-bit tag naming the launch and stage that wrote it. Producers
//    store and move on; consumers read the vector and re-read words whose tag is not the
//    expected one. An aligned 64-bit store is single-copy atomic, so a payload is never seen
//    with a wrong tag, and every word of a buffer is rewritten each launch, so a stale tag never
//    matches. A hand-off costs one round trip instead of four.
//  * Register ring with deferred refills. Each wave streams its share of the program — per layer
//    QKV rows, K/V positions of the block's attention unit, O rows, gate/up rows, down rows;
//    then lm_head rows — through a ring of RING slots (two 1 KB loads each). A slot is refilled
//    as soon as it is consumed, so the next RING items stay in flight, across stage boundaries
//    too. The last round of a stage is consumed without refilling: the block first issues the
//    poll for the next stage's input (an empty queue, so it returns fast) and then the deferred
//    refills, which stream while the hand-off completes. A wave's item count per stage is padded
//    to whole rounds (padding items read nothing), so every stage starts at ring slot 0 and
//    the compiler's vmcnt bookkeeping stays exact.
//  * All eight waves of a block stream and all share the hand-off work between stages:
//    epilogues (scales, RoPE, residual, SwiGLU, KV append), the tagged polls, the RMSNorm
//    (block-wide sum of squares) and the attention merges.
//  * GEMV: a stage's row pairs are split evenly over the blocks and each block's (pair, chunk)
//    items evenly over its waves; a wave accumulates a pair's chunks and writes its partial sums
//    to LDS, which the epilogue adds in a fixed order. Rows are packed at load so a RoPE pair
//    (i, i + hd/2) and a SwiGLU pair (gate n, up n) share an item. int8 codes convert with one
//    v_cvt_f32_i32 (SDWA byte select) per weight into an fp32 FMA; the input vector sits in LDS
//    in a swizzled layout (conflict-free 16-byte lane reads).
//  * Attention: split-KV over (kv head, position range) units, one per block; the G query heads
//    of the kv head share every K/V load and each 16-lane (hd 128) or 8-lane (hd 64) row runs an
//    online softmax. The block merges its waves into a partial (max, sum, weighted values); the
//    blocks of a kv head then each merge one slice of its outputs over all splits.
//  * No MFMA: batch-1 decode is a matrix-vector product, far below the MFMA ridge point.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "amk_kparams.h"

namespace amk {
namespace sk {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kOOB = static_cast<int>(0x80000000u);
constexpr int kNT = 2;    // buffer load cache policy: non-temporal (weights, K/V)
constexpr int kSC1 = 16;  // buffer load cache policy: agent coherent (tagged words)
#ifndef AMK_RING
#define AMK_RING 2        // ring slots per wave (2 x 1 KB loads each)
#endif
#ifndef AMK_DEFER
#define AMK_DEFER 0       // 1: a stage's last ring round defers its refills to the next hand-off
#endif
#ifndef AMK_ATT_PF
#define AMK_ATT_PF 0      // attention items per wave prefetched into registers during QKV
#endif
#ifndef AMK_DBG
#define AMK_DBG 0         // 1: per-stage debug stamps after the stage stamps (compute end, B exit)
#endif

// stage types of the per-layer program, in program order
enum { ST_QKV = 0, ST_ATT = 1, ST_O = 2, ST_GU = 3, ST_D = 4, ST_LM = 5, ST_END = 6 };
constexpr int kProgStages = 5;  // per layer

// ------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------
// f(integral_constant<int, I>) for I = B .. E-1, as separate inlined copies: register arrays
// indexed by the constant stay in registers whatever the unroller decides.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
__device__ __forceinline__ unsigned ldc(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t payload, uint32_t tag) {
  __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// An empty asm that hides a value from the optimizer (keeps per-thread address math inside the
// loops that use it instead of hoisting and spilling it).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(opaque(threadIdx.x) >> 6); }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ i32x4 ldnt(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kNT);
}
__device__ __forceinline__ i32x4 ldsc1(__amdgpu_buffer_rsrc_t rs, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kSC1);
}

__device__ __forceinline__ float bf_lo(int v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ float bf_hi(int v) { return __uint_as_float(static_cast<uint32_t>(v) & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float((b & 0xffffu) << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {  // round to nearest, ties to even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }
__device__ __forceinline__ float i8_to_f32(int v, int k) {
  return static_cast<float>(static_cast<signed char>(static_cast<uint32_t>(v) >> (8 * k)));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  // every lane of the row patterns used here reads a lane of its own row; written as an update
  // with a zero fill so the compiler folds the move into the consuming add / max (one DPP op)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum over each aligned group of LANES (8 or 16) lanes, in every lane of the group
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  if (LANES == 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}
// v of lane (lane ^ OFF), OFF in {8, 16, 32}: DPP row rotate by 8, or the gfx950 permlane swaps
template <int OFF>
__device__ __forceinline__ float xor_lane(float v) {
  if (OFF == 8) return dpp<0x128>(v);  // row_ror:8
  const unsigned u = __float_as_uint(v);
  if (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  v += xor_lane<16>(v);
  v += xor_lane<32>(v);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  v = fmaxf(v, xor_lane<16>(v));
  v = fmaxf(v, xor_lane<32>(v));
  return v;
}

// ------------------------------------------------------------------------------------------
// weight formats and the swizzled LDS layout of a GEMV input vector
// ------------------------------------------------------------------------------------------
template <int FMT> struct Fmt;
template <> struct Fmt<0> { static constexpr int WB = 2, CW = 512, LC = 8; };   // bf16
template <> struct Fmt<1> { static constexpr int WB = 1, CW = 1024, LC = 16; };  // int8
// A 1 KB weight chunk covers CW columns; lane L owns LC consecutive columns (16 bytes). Column
// e sits at chunk*CW + (k/4)*256 + L*4 + k%4 with k = e's index inside the lane, so the k/4-th
// float4 of every lane is at a 16-byte lane stride.
template <int FMT>
__device__ __forceinline__ int swz(int e) {
  constexpr int CW = Fmt<FMT>::CW, LC = Fmt<FMT>::LC;
  const int ch = e / CW, r = e - ch * CW, ln = r / LC, k = r - ln * LC;
  return ch * CW + (k >> 2) * 256 + ln * 4 + (k & 3);
}
template <int FMT>
__device__ __forceinline__ int padded(int K) {
  constexpr int CW = Fmt<FMT>::CW;
  return (K + CW - 1) / CW * CW;
}

// max / sum over each aligned group of SP lanes (SP a power of two <= 64), in every lane of the
// group; SP is wave-uniform
__device__ __forceinline__ float seg_sum(float v, int SP) {
  if (SP >= 2) v += dpp<0xB1>(v);
  if (SP >= 4) v += dpp<0x4E>(v);
  if (SP >= 8) v += dpp<0x141>(v);
  if (SP >= 16) v += dpp<0x140>(v);
  if (SP >= 32) v += xor_lane<16>(v);
  if (SP >= 64) v += xor_lane<32>(v);
  return v;
}
__device__ __forceinline__ float seg_max(float v, int SP) {
  if (SP >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if (SP >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if (SP >= 8) v = fmaxf(v, dpp<0x141>(v));
  if (SP >= 16) v = fmaxf(v, dpp<0x140>(v));
  if (SP >= 32) v = fmaxf(v, xor_lane<16>(v));
  if (SP >= 64) v = fmaxf(v, xor_lane<32>(v));
  return v;
}

// ------------------------------------------------------------------------------------------
// LDS layout (offsets in floats, computed by the host)
// ------------------------------------------------------------------------------------------
struct Lds {
  float* vec;    // GEMV input vector (swizzled); attention: q [G][hd] fp32, then K/V(pos) bf16
  float* part;   // wave partials: GEMV [pair][wave][2]; attention [wave][G][hd + 2]
  float* xres;   // residual rows owned by this block [2 * pairs]
  float* rope;   // cos [hd/2], sin [hd/2] at pos
  float* red;    // [kWaves] block reductions
  int* flag;     // [0] abort
  int4* stab;    // per stage type: GEMV {first pair, pairs, chunks per row, row bytes};
                 // attention {t0, t1, kv head, items}
  int4* wtab;    // per stage type and wave: {first item, end item, pair << 16 | chunk, rounds}
};

// ------------------------------------------------------------------------------------------
// the program: stage k = layer * 5 + type for k < 5L, then lm_head, then the end
// ------------------------------------------------------------------------------------------
struct Stage {
  int k;         // program stage index
  int type, layer;
  int c0, c1;    // this wave's items (block relative)
  int pl0, ch0;  // pair and chunk of item c0
  int rounds;    // ring rounds: ceil((c1 - c0) / RING); items past c1 are padding
  int C;         // the block's item count
  int nch, rb, pb0, np;  // GEMV
  int t0, t1, g;         // attention
  int pf0;               // attention: first item (items pf0 .. c0 - 1 come from the prefetch registers)
};

// Fills the per-block stage tables (threads 0..47: type = tid / 8, wave = tid % 8).
template <int HD, int FMT, int RING>
__device__ __forceinline__ void build_tables(const KParams& p, int4* stab, int4* wtab) {
  constexpr int PPC = 64 / (HD / 8);  // positions per attention item
  const int tid = threadIdx.x;
  if (tid >= 6 * kWaves) return;
  const int type = tid / kWaves, w = tid % kWaves;
  const int nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  int4 st{0, 0, 1, 0};
  int C = 0, nch = 1;
  if (type == ST_ATT) {
    const int S = p.S;
    const bool active = b < p.nkv * S;
    const int g = active ? b / S : 0;
    const int j = active ? b - g * S : 0;
    const int t0 = j * p.T, t1 = min(t0 + p.T, p.pos + 1);
    C = active ? (t1 - t0 + PPC - 1) / PPC : 0;
    st = int4{t0, t1, g, C};
  } else {
    int K = 0, P = 0, unit = 1;
    switch (type) {
      case ST_QKV: K = p.H; P = (p.nq + 2 * p.nkv) * (HD / 2); break;
      case ST_O: K = p.nq * HD; P = p.H / 2; break;
      case ST_GU: K = p.H; P = p.F; unit = 2; break;
      case ST_D: K = p.F; P = p.H / 2; break;
      default: K = p.H; P = p.V / 2; break;  // ST_LM
    }
    const int nu = P / unit;
    const int u0 = nu * b / nb, u1 = nu * (b + 1) / nb;  // nu * nb < 2^31 (checked by the host)
    const int rb = K * Fmt<FMT>::WB;
    nch = (rb + 1023) / 1024;
    const int np = (u1 - u0) * unit;
    C = np * nch;
    st = int4{u0 * unit, np, nch, rb};
  }
  if (w == 0) stab[type] = st;
  const int c0 = C * w / kWaves, c1 = C * (w + 1) / kWaves;
  if (type == ST_ATT) {  // the first AMK_ATT_PF items come from the prefetch registers
    const int r0 = min(c1, c0 + AMK_ATT_PF);
    wtab[type * kWaves + w] = int4{r0, c1, c0, (c1 - r0 + RING - 1) / RING};
  } else {
    const int pl = c0 / nch;
    wtab[type * kWaves + w] = int4{c0, c1, (pl << 16) | (c0 - pl * nch), (c1 - c0 + RING - 1) / RING};
  }
}

// Stage k of the program as seen by wave w.
__device__ __forceinline__ Stage stage_at(const KParams& p, const Lds& L, int k, int w) {
  Stage s;
  s.k = k;
  const int nst = kProgStages * p.L;
  s.layer = k < nst ? k / kProgStages : p.L;
  s.type = k < nst ? k - s.layer * kProgStages : (k == nst ? ST_LM : ST_END);
  s.nch = 1; s.rb = 0; s.pb0 = 0; s.np = 0; s.C = 0; s.t0 = 0; s.t1 = 0; s.g = 0;
  s.c0 = s.c1 = s.pl0 = s.ch0 = s.rounds = s.pf0 = 0;
  if (s.type == ST_END) return s;
  const int4 a = L.stab[s.type];
  const int4 x = L.wtab[s.type * kWaves + w];
  if (s.type == ST_ATT) {
    s.t0 = uni(a.x); s.t1 = uni(a.y); s.g = uni(a.z); s.C = uni(a.w);
  } else {
    s.pb0 = uni(a.x); s.np = uni(a.y); s.nch = uni(a.z); s.rb = uni(a.w);
    s.C = s.np * s.nch;
  }
  s.c0 = uni(x.x); s.c1 = uni(x.y);
  const int pc = uni(x.z);
  s.pf0 = pc;
  s.pl0 = s.type == ST_ATT ? 0 : pc >> 16;
  s.ch0 = s.type == ST_ATT ? 0 : pc & 0xffff;
  s.rounds = uni(x.w);
  return s;
}

// weight matrix of a GEMV stage (bytes) and its scales
__device__ __forceinline__ const uint8_t* stage_w(const KParams& p, int type, int l) {
  switch (type) {
    case ST_QKV: return p.w_qkv + l * p.w_qkv_ls;
    case ST_O: return p.w_o + l * p.w_o_ls;
    case ST_GU: return p.w_gu + l * p.w_gu_ls;
    case ST_D: return p.w_d + l * p.w_d_ls;
    default: return p.w_lm;
  }
}
__device__ __forceinline__ const float* stage_s(const KParams& p, int type, int l) {
  switch (type) {
    case ST_QKV: return p.s_qkv + l * p.s_qkv_ls;
    case ST_O: return p.s_o + l * p.s_o_ls;
    case ST_GU: return p.s_gu + l * p.s_gu_ls;
    case ST_D: return p.s_d + l * p.s_d_ls;
    default: return p.s_lm;
  }
}

// ------------------------------------------------------------------------------------------
// ring: issue side
// ------------------------------------------------------------------------------------------
template <int HD, int RING>
struct IssueCursor {
  Stage s;
  int c, pl, ch, cend;  // item (padding past c1), pair (block relative), chunk, end of the rounds
  // GEMV: both loads from the block's rows of the matrix; attention: the K and V blocks. Kept as
  // pointer + size; the buffer resources are rebuilt at each load (a few scalar instructions).
  const void* b0;
  const void* b1;
  uint32_t n0, n1;

  __device__ __forceinline__ void enter(const KParams& p, const Lds& L, int k, int w) {
    for (;;) {
      s = stage_at(p, L, k, w);
      if (s.type == ST_END || s.rounds > 0) break;
      ++k;
    }
    c = s.c0;
    pl = s.pl0;
    ch = s.ch0;
    cend = s.c0 + s.rounds * RING;
    if (s.type == ST_ATT) {
      const size_t blk = static_cast<size_t>(p.max_ctx) * HD;  // elements of one (layer, kv, head) block
      b0 = p.kv + (static_cast<size_t>(s.layer * 2) * p.nkv + s.g) * blk;
      b1 = p.kv + (static_cast<size_t>(s.layer * 2 + 1) * p.nkv + s.g) * blk;
      n0 = n1 = static_cast<uint32_t>(blk * 2);
    } else if (s.type != ST_END) {
      b0 = b1 = stage_w(p, s.type, s.layer) + static_cast<size_t>(2 * s.pb0) * s.rb;
      n0 = n1 = static_cast<uint32_t>(2 * s.np) * static_cast<uint32_t>(s.rb);
    } else {
      b0 = b1 = p.w_lm;  // past the program: every load reads zeros
      n0 = n1 = 0u;
    }
  }

  // the two loads of the current item (zeros for padding and past the program), then advance
  __device__ __forceinline__ void issue(const KParams& p, const Lds& L, int w, i32x4& a, i32x4& b) {
    constexpr int LPP = HD / 8, PPC = 64 / LPP;
    const int lane = __lane_id();
    int voff = kOOB, soff0 = 0, soff1 = 0;
    if (c < s.c1) {
      if (s.type == ST_ATT) {
        const int tb = s.t0 + c * PPC;
        const int t = tb + lane / LPP;
        voff = t < s.t1 ? (lane / LPP) * (HD * 2) + (lane % LPP) * 16 : kOOB;
        soff0 = soff1 = tb * (HD * 2);
      } else {
        const int off = ch * 1024 + lane * 16;
        voff = off < s.rb ? lane * 16 : kOOB;
        soff0 = 2 * pl * s.rb + ch * 1024;
        soff1 = soff0 + s.rb;
      }
    }
    a = ldnt(make_rsrc(b0, n0), voff, uni(soff0));
    b = ldnt(make_rsrc(b1, n1), voff, uni(soff1));
    if (s.type == ST_END) return;
    ++c;
    if (++ch == s.nch) { ch = 0; ++pl; }
    if (c == cend) enter(p, L, s.k + 1, w);
  }
};

// Issues wave w's first AMK_ATT_PF attention items of layer `layer` (K and V of PPC positions
// each) into dedicated registers; they stream in during the QKV stage.
template <int HD, int NA, int NR>
__device__ __forceinline__ void att_prefetch(const KParams& p, const Lds& L, int layer, int w, i32x4 (&pk)[NR],
                                             i32x4 (&pv)[NR]) {
  constexpr int LPP = HD / 8, PPC = 64 / LPP;
  const Stage s = stage_at(p, L, layer * kProgStages + ST_ATT, w);
  const int lane = __lane_id();
  const size_t blk = static_cast<size_t>(p.max_ctx) * HD;
  const uint16_t* kb = p.kv + (static_cast<size_t>(layer * 2) * p.nkv + s.g) * blk;
  const uint16_t* vb = p.kv + (static_cast<size_t>(layer * 2 + 1) * p.nkv + s.g) * blk;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, static_cast<uint32_t>(blk * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, static_cast<uint32_t>(blk * 2));
  static_for<0, NA>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    const int c = s.pf0 + i;
    const int tb = s.t0 + c * PPC;
    const int t = tb + lane / LPP;
    const int voff = (c < s.c0 && t < s.t1) ? (lane / LPP) * (HD * 2) + (lane % LPP) * 16 : kOOB;
    const int soff = uni(c < s.c0 ? tb * (HD * 2) : 0);
    pk[i] = ldnt(rk, voff, soff);
    pv[i] = ldnt(rv, voff, soff);
  });
}

// ------------------------------------------------------------------------------------------
// ring: consume side
// ------------------------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ void chunk_fma(const i32x4 w0, const i32x4 w1, const float* __restrict__ xl,
                                          float& a0, float& a1) {
  if (FMT == 1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(xl + d * 256);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a0 = __builtin_fmaf(i8_to_f32(w0[d], k), x[k], a0);
        a1 = __builtin_fmaf(i8_to_f32(w1[d], k), x[k], a1);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(xl + h * 256);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int u0 = w0[2 * h + d], u1 = w1[2 * h + d];
        a0 = __builtin_fmaf(bf_lo(u0), x[2 * d], a0);
        a0 = __builtin_fmaf(bf_hi(u0), x[2 * d + 1], a0);
        a1 = __builtin_fmaf(bf_lo(u1), x[2 * d], a1);
        a1 = __builtin_fmaf(bf_hi(u1), x[2 * d + 1], a1);
      }
    }
  }
}

// online-softmax state of one attention row (the lanes of a row hold the same m, l)
template <int GMAX>
struct AttnState {
  float m[GMAX], l[GMAX], acc[GMAX][8];
};

template <int GMAX>
__device__ __forceinline__ void att_reset(AttnState<GMAX>& st) {
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    st.m[h] = -__builtin_inff();
    st.l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[h][i] = 0.f;
  }
}

// Scores one item (PPC positions, one per row) against the G query heads in LDS and updates the
// online softmax. The current position's K/V come from LDS (this step wrote them).
template <int HD, int GMAX>
__device__ __forceinline__ void att_consume(const KParams& p, const Lds& L, int t0, int t1, int c, i32x4 kr,
                                            i32x4 vr, AttnState<GMAX>& st) {
  constexpr int LPP = HD / 8, PPC = 64 / LPP;
  const int lane = __lane_id(), ri = lane / LPP, li = lane % LPP;
  const int tb = t0 + c * PPC;
  const int t = tb + ri;
  const int G = p.nq / p.nkv;
  if (tb <= p.pos && p.pos < tb + PPC) {  // uniform: this item holds the current position
    const uint16_t* kvp = reinterpret_cast<const uint16_t*>(L.vec + G * HD);
    const i32x4 kl = *reinterpret_cast<const i32x4*>(kvp + li * 8);
    const i32x4 vl = *reinterpret_cast<const i32x4*>(kvp + HD + li * 8);
    if (t == p.pos) { kr = kl; vr = vl; }
  }
  const bool valid = t < t1;
  float kf[8], vf[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    kf[2 * d] = bf_lo(kr[d]);
    kf[2 * d + 1] = bf_hi(kr[d]);
    vf[2 * d] = bf_lo(vr[d]);
    vf[2 * d + 1] = bf_hi(vr[d]);
  }
  const float NEG_INF = -__builtin_inff();
  float sc[GMAX], mn[GMAX];
  bool moved = false;
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    sc[h] = NEG_INF;
    mn[h] = st.m[h];
    if (h < G) {
      const float* qp = L.vec + h * HD + li * 8;
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(qp);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(qp + 4);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) dot = __builtin_fmaf(q0[i], kf[i], dot);
#pragma unroll
      for (int i = 0; i < 4; ++i) dot = __builtin_fmaf(q1[i], kf[4 + i], dot);
      dot = group_sum<LPP>(dot);
      sc[h] = valid ? dot * p.attn_scale : NEG_INF;
      mn[h] = fmaxf(st.m[h], sc[h]);
      moved |= mn[h] != st.m[h];
    }
  }
  if (__builtin_amdgcn_ballot_w64(moved) == 0) {
    // no running maximum of the wave moved: no rescale
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < G) {
        const float pe = (sc[h] == NEG_INF) ? 0.f : __expf(sc[h] - st.m[h]);
        st.l[h] += pe;
#pragma unroll
        for (int i = 0; i < 8; ++i) st.acc[h][i] = __builtin_fmaf(pe, vf[i], st.acc[h][i]);
      }
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      const float corr = (st.m[h] == NEG_INF) ? 0.f : __expf(st.m[h] - mn[h]);
      const float pe = (sc[h] == NEG_INF) ? 0.f : __expf(sc[h] - mn[h]);
      st.l[h] = st.l[h] * corr + pe;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.acc[h][i] = __builtin_fmaf(pe, vf[i], st.acc[h][i] * corr);
      st.m[h] = mn[h];
    }
  }
}

// merges the rows of the wave and writes the wave's state to LDS part[w][h][hd + 2]
template <int HD, int GMAX>
__device__ __forceinline__ void att_finish(const KParams& p, const Lds& L, int w, AttnState<GMAX>& st) {
  constexpr int LPP = HD / 8;
  const float NEG_INF = -__builtin_inff();
  const int G = p.nq / p.nkv;
  const int lane = __lane_id(), ri = lane / LPP, li = lane % LPP;
  auto merge = [&](auto off_tag) {
    constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      const float mo = xor_lane<OFF>(st.m[h]), lo = xor_lane<OFF>(st.l[h]);
      const float M = fmaxf(st.m[h], mo);
      const float ea = (st.m[h] == NEG_INF) ? 0.f : __expf(st.m[h] - M);
      const float eb = (mo == NEG_INF) ? 0.f : __expf(mo - M);
      st.l[h] = st.l[h] * ea + lo * eb;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.acc[h][i] = st.acc[h][i] * ea + xor_lane<OFF>(st.acc[h][i]) * eb;
      st.m[h] = M;
    }
  };
  if (LPP == 8) merge(std::integral_constant<int, 8>{});
  merge(std::integral_constant<int, 16>{});
  merge(std::integral_constant<int, 32>{});
  if (ri == 0) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < G) {
        float* dst = L.part + (w * G + h) * (HD + 2);
        *reinterpret_cast<f32x4*>(dst + li * 8) = f32x4{st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]};
        *reinterpret_cast<f32x4*>(dst + li * 8 + 4) = f32x4{st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]};
        if (li == 0) {
          dst[HD] = st.m[h];
          dst[HD + 1] = st.l[h];
        }
      }
    }
  }
}

// Runs wave w's items of stage st through the ring. Every round but the last refills each slot
// right after consuming it; the last round only consumes (its refills are issued by the next
// hand-off, behind that hand-off's poll).
template <int HD, int FMT, int GMAX, int RING, bool ATT>
__device__ __forceinline__ void run_stage(const KParams& p, const Lds& L, const Stage& st, int w,
                                          i32x4 (&ra)[RING], i32x4 (&rb)[RING], IssueCursor<HD, RING>& ic,
                                          AttnState<GMAX>& as, bool& ring_free) {
  constexpr int CW = Fmt<FMT>::CW;
  if (st.rounds == 0) return;
  const int lane = __lane_id();
  int c = st.c0, pl = st.pl0, ch = st.ch0;
  float acc0 = 0.f, acc1 = 0.f;
  auto consume = [&](const i32x4 wa, const i32x4 wb) {
    if (c < st.c1) {
      if constexpr (ATT) {
        att_consume<HD, GMAX>(p, L, st.t0, st.t1, c, wa, wb, as);
      } else {
        chunk_fma<FMT>(wa, wb, L.vec + ch * CW + lane * 4, acc0, acc1);
        if (ch == st.nch - 1 || c == st.c1 - 1) {
          const float y0 = wave_sum(acc0), y1 = wave_sum(acc1);
          acc0 = acc1 = 0.f;
          if (lane == 0) *reinterpret_cast<float2*>(L.part + (pl * kWaves + w) * 2) = float2{y0, y1};
        }
        if (++ch == st.nch) { ch = 0; ++pl; }
      }
    }
    ++c;
  };
  for (int r = 0; r + 1 < st.rounds; ++r) {
    static_for<0, RING>([&](auto si) {
      constexpr int s = decltype(si)::value;
      __builtin_amdgcn_sched_barrier(0);
      consume(ra[s], rb[s]);
      __builtin_amdgcn_sched_barrier(0);
      ic.issue(p, L, w, ra[s], rb[s]);
    });
  }
  static_for<0, RING>([&](auto si) {
    constexpr int s = decltype(si)::value;
    __builtin_amdgcn_sched_barrier(0);
    consume(ra[s], rb[s]);
    if (!AMK_DEFER) {
      __builtin_amdgcn_sched_barrier(0);
      ic.issue(p, L, w, ra[s], rb[s]);
    }
  });
  ring_free = AMK_DEFER != 0;
}

// ------------------------------------------------------------------------------------------
// block-wide hand-off work
// ------------------------------------------------------------------------------------------
// Workgroup barrier for the stage hand-offs inside a block. It waits only for this wave's LDS
// traffic (lgkmcnt 0): weight loads stay in flight across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t tag_of(const KParams& p, int layer, int which) {
  return p.tag0 + static_cast<uint32_t>(layer * kTagsPerLayer + which);
}
// byte offset of a tagged buffer inside the tagged region
__device__ __forceinline__ int toff(const KParams& p, const uint64_t* buf) {
  return static_cast<int>(reinterpret_cast<const uint8_t*>(buf) - reinterpret_cast<const uint8_t*>(p.tagged));
}

// Block-wide poll of nquads 16-byte quads (two tagged words each) of the tagged region: thread t
// owns quads t + 512 b, b < VB (then further batches of 512 VB). After the first batch's loads are
// issued, mid() runs (the deferred ring refills go there, behind the poll). When every tag of a
// thread's quads equals `tag` on the first read (the common case) visit(b, qi, payload0,
// payload1) runs straight away, so the compiler waits only for the poll's own loads; otherwise
// the thread re-reads its pending quads until they are fresh. off(qi) is the quad's byte offset,
// or kOOB for a quad to skip. Returns false if the step must be abandoned (timeout, or an error
// raised elsewhere).
template <int VB, class Off, class Visit, class Mid>
__device__ __forceinline__ bool poll_block(const KParams& p, int nquads, uint32_t tag, Off off, Visit visit, Mid mid,
                                           uint64_t* dbg = nullptr) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.tagged, p.tagged_bytes);
  const int tid = opaque(threadIdx.x);
  if (AMK_DBG && dbg != nullptr && threadIdx.x == 0) dbg[0] = wall_clock64();
  if (nquads <= 0) mid();
  for (int q0 = 0; q0 < nquads; q0 += kThreads * VB) {
    i32x4 v[VB];
    uint32_t skip = 0;
    static_for<0, VB>([&](auto bi) {
      constexpr int b = decltype(bi)::value;
      const int qi = q0 + b * kThreads + tid;
      const int o = qi < nquads ? off(qi) : kOOB;
      skip |= (o == kOOB) ? (1u << b) : 0u;
      v[b] = ldsc1(rs, o);
    });
    if (q0 == 0) mid();
    auto pending = [&]() {
      uint32_t pend = 0;
      static_for<0, VB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        const bool good = ((skip >> b) & 1u) ||
                          (static_cast<uint32_t>(v[b].y) == tag && static_cast<uint32_t>(v[b].w) == tag);
        pend |= good ? 0u : (1u << b);
      });
      return pend;
    };
    auto visit_all = [&]() {
      static_for<0, VB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        if (!((skip >> b) & 1u))
          visit(bi, q0 + b * kThreads + tid, static_cast<uint32_t>(v[b].x), static_cast<uint32_t>(v[b].z));
      });
    };
    uint32_t pend = pending();
    if (AMK_DBG && dbg != nullptr && q0 == 0) {
      if (threadIdx.x == 0) dbg[1] = wall_clock64();
      if (pend != 0u) atomicAdd(reinterpret_cast<unsigned long long*>(dbg + 3), 1ull);
    }
    if (pend == 0u) {
      visit_all();
      continue;
    }
    const uint64_t t_start = wall_clock64();
    unsigned it = 0;
    while (pend != 0u) {
      if (((++it) & 15u) == 0) {
        if (ldc(p.err) != 0u) return false;  // raised elsewhere: keep its code
        if (wall_clock64() - t_start > p.spin_limit) {
          stc(p.err, kErrTimeout);
          return false;
        }
      }
      __builtin_amdgcn_s_sleep(2);
      static_for<0, VB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        if (pend & (1u << b)) v[b] = ldsc1(rs, off(q0 + b * kThreads + tid));
      });
      pend = pending();
    }
    visit_all();
  }
  if (AMK_DBG && dbg != nullptr && threadIdx.x == 0) dbg[2] = wall_clock64();
  return true;
}

// sum over the block, in every thread (two workgroup barriers)
__device__ __forceinline__ float block_sum(const Lds& L, float v) {
  v = wave_sum(v);
  if (__lane_id() == 0) L.red[wave_id()] = v;
  wg_barrier();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += L.red[i];
  wg_barrier();
  return t;
}

// W8A16 scales of the pairs a thread finishes in the next epilogue: pair t (x, y), or pairs 2t
// and 2t + 1 for gate/up (x, y, z, w). Loaded one hand-off ahead and carried in registers.
__device__ __forceinline__ float4 load_scales(const float* __restrict__ src, int np, bool two) {
  const int tid = opaque(threadIdx.x);
  float4 r{1.f, 1.f, 1.f, 1.f};
  if (two) {
    if (2 * tid < np) r = *reinterpret_cast<const float4*>(src + 4 * tid);
  } else if (tid < np) {
    const float2 v = *reinterpret_cast<const float2*>(src + 2 * tid);
    r.x = v.x;
    r.y = v.y;
  }
  return r;
}

// the waves that wrote partial sums for pair pl (their item ranges meet the pair's chunks)
__device__ __forceinline__ float pair_sum(const Lds& L, int C, int nch, int pl, int row) {
  float y = 0.f;
  const int a = pl * nch, e = a + nch;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c0 = C * w / kWaves, c1 = C * (w + 1) / kWaves;
    if (c0 < c1 && c0 < e && c1 > a) y += L.part[(pl * kWaves + w) * 2 + row];
  }
  return y;
}

constexpr int kNormVB = 8;  // H <= 8192: thread t owns elements 2 (t + 512 b), b < 8

// The RMSNorm weights of the elements a thread owns in norm_from_x, loaded one hand-off ahead
// and carried in registers (so no load sits in front of a hand-off's poll).
__device__ __forceinline__ void load_norm_weight(const float* __restrict__ w, int H, float2 (&wv)[kNormVB]) {
  const int tid = opaque(threadIdx.x);
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) {
    const int e = 2 * (b * kThreads + tid);
    wv[b] = e < H ? *reinterpret_cast<const float2*>(w + e) : float2{0.f, 0.f};
  }
}

// RMSNorm of x (polled, tag `tag`) into the GEMV input vector: h = bf16((x * r) * w), zero padded.
// Thread t owns quads t + 512 b (elements 2 qi, 2 qi + 1). mid() runs behind the poll's loads.
template <int FMT, class Mid>
__device__ __forceinline__ bool norm_from_x(const KParams& p, const Lds& L, uint32_t tag, const float2 (&wv)[kNormVB],
                                            Mid mid, uint64_t* dbg = nullptr) {
#pragma clang fp contract(off)
  constexpr int VB = kNormVB;
  const int H = p.H, tid = opaque(threadIdx.x);
  float2 xv[VB];
#pragma unroll
  for (int b = 0; b < VB; ++b) xv[b] = float2{0.f, 0.f};
  const int ob = toff(p, p.tx);
  const bool ok = poll_block<VB>(
      p, H / 2, tag, [&](int qi) { return ob + 16 * qi; },
      [&](auto bi, int, uint32_t a, uint32_t c) { xv[decltype(bi)::value] = float2{__uint_as_float(a), __uint_as_float(c)}; },
      mid, dbg);
  float ss = 0.f;
#pragma unroll
  for (int b = 0; b < VB; ++b) ss += xv[b].x * xv[b].x + xv[b].y * xv[b].y;
  ss = block_sum(L, ss);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + p.eps);
#pragma unroll
  for (int b = 0; b < VB; ++b) {
    const int e = 2 * (b * kThreads + tid);
    if (e < H) {
      L.vec[swz<FMT>(e)] = round_bf16((xv[b].x * r) * wv[b].x);
      L.vec[swz<FMT>(e + 1)] = round_bf16((xv[b].y * r) * wv[b].y);
    }
  }
  for (int e = H + tid; e < padded<FMT>(H); e += kThreads) L.vec[swz<FMT>(e)] = 0.f;
  return ok;
}

// bf16 vector of K elements (2 per tagged word) into the GEMV input vector, zero padded
template <int FMT, class Mid>
__device__ __forceinline__ bool vector_from_words(const KParams& p, const Lds& L, const uint64_t* src, int K,
                                                  uint32_t tag, Mid mid, uint64_t* dbg = nullptr) {
  const int ob = toff(p, src);
  const bool ok = poll_block<8>(
      p, K / 4, tag, [&](int qi) { return ob + 16 * qi; },
      [&](auto, int qi, uint32_t a, uint32_t c) {
        *reinterpret_cast<f32x4*>(L.vec + swz<FMT>(4 * qi)) =
            f32x4{bf16_to_f32(a), bf16_to_f32(a >> 16), bf16_to_f32(c), bf16_to_f32(c >> 16)};
      },
      mid, dbg);
  for (int e = K + opaque(threadIdx.x); e < padded<FMT>(K); e += kThreads) L.vec[swz<FMT>(e)] = 0.f;
  return ok;
}

// ------------------------------------------------------------------------------------------
// the kernel
// ------------------------------------------------------------------------------------------
template <int HD, int FMT, int GMAX, int RING>
__global__ void __launch_bounds__(kThreads, 1) amk_stream_kernel(const KParams p) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int flags[4];
  __shared__ float red[kWaves];
  __shared__ int4 stab[6], wtab[6 * kWaves];
  if (threadIdx.x == 0) flags[0] = 0;
  build_tables<HD, FMT, RING>(p, stab, wtab);
  const unsigned err0 = ldc(p.err);
  __syncthreads();
  if (err0 != 0u) return;
  Lds L;
  L.vec = smem;
  L.part = smem + p.lds_part;
  L.xres = smem + p.lds_xres;
  L.rope = smem + p.lds_rope;
  L.red = red;
  L.flag = flags;
  L.stab = stab;
  L.wtab = wtab;

  const int w = wave_id();
  const int nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  const int G = p.nq / p.nkv, half = HD / 2, H = p.H;
  const float NEG_INF = -__builtin_inff();
  uint64_t* trace = p.trace ? p.trace + static_cast<size_t>(b) * p.trace_stride : nullptr;
  int ev = 0;
  auto stamp = [&]() {
    if (trace != nullptr && threadIdx.x == 0) trace[ev] = wall_clock64();
    ++ev;
  };
  stamp();

  // Launch constants, issued before the ring so they do not queue behind it: RoPE at pos, the
  // residual rows of this block (from the embedding row), the first stage's scales, and the
  // embedding row with the first RMSNorm weight.
  float4 scn{1.f, 1.f, 1.f, 1.f};  // W8A16 scales for the next epilogue (carried across the stage)
  float2 nwv[kNormVB];              // RMSNorm weights of the next norm (carried across stages)
  {
    const int tid = opaque(threadIdx.x);
    const uint16_t* emb = p.embed + static_cast<size_t>(p.token) * H;
    const int ho_pb0 = (H / 2) * b / nb, ho_np = (H / 2) * (b + 1) / nb - ho_pb0;
    float rope_v = 0.f, xres_v = 0.f;
    if (tid < HD)
      rope_v = tid < half ? p.rope_cos[static_cast<size_t>(p.pos) * half + tid]
                          : p.rope_sin[static_cast<size_t>(p.pos) * half + tid - half];
    if (tid < 2 * ho_np) xres_v = bf16_to_f32(emb[2 * ho_pb0 + tid]);
    const Stage s0 = stage_at(p, L, 0, w);
    if (FMT == 1) scn = load_scales(stage_s(p, ST_QKV, 0) + 2 * s0.pb0, s0.np, false);
    constexpr int VB = 8;  // H <= 8192
    float2 xv[VB], wv[VB];
#pragma unroll
    for (int bb = 0; bb < VB; ++bb) {
      const int e = 2 * (bb * kThreads + tid);
      xv[bb] = float2{0.f, 0.f};
      wv[bb] = float2{0.f, 0.f};
      if (e < H) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(emb + e);
        xv[bb] = float2{bf_lo(static_cast<int>(u)), bf_hi(static_cast<int>(u))};
        wv[bb] = *reinterpret_cast<const float2*>(p.norm_in + e);
      }
    }
    if (tid < HD) L.rope[tid] = rope_v;
    if (tid < 2 * ho_np) L.xres[tid] = xres_v;
    float ss = 0.f;
#pragma unroll
    for (int bb = 0; bb < VB; ++bb) ss += xv[bb].x * xv[bb].x + xv[bb].y * xv[bb].y;
    ss = block_sum(L, ss);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + p.eps);
#pragma unroll
    for (int bb = 0; bb < VB; ++bb) {
      const int e = 2 * (bb * kThreads + tid);
      if (e < H) {
        L.vec[swz<FMT>(e)] = round_bf16((xv[bb].x * r) * wv[bb].x);
        L.vec[swz<FMT>(e + 1)] = round_bf16((xv[bb].y * r) * wv[bb].y);
      }
    }
    for (int e = H + tid; e < padded<FMT>(H); e += kThreads) L.vec[swz<FMT>(e)] = 0.f;
  }
  // ring prologue
  i32x4 ra[RING], rb[RING];
  IssueCursor<HD, RING> ic;
  ic.enter(p, L, 0, w);
  static_for<0, RING>([&](auto si) { ic.issue(p, L, w, ra[si.value], rb[si.value]); });
  i32x4 pk[AMK_ATT_PF > 0 ? AMK_ATT_PF : 1], pv[AMK_ATT_PF > 0 ? AMK_ATT_PF : 1];  // next attention items
  if (AMK_ATT_PF > 0) att_prefetch<HD, AMK_ATT_PF>(p, L, 0, w, pk, pv);
  bool ring_free = false;
  // Deferred refills, issued behind a hand-off's poll: the workgroup barrier makes every wave's
  // poll loads enter the unit's (in-order) memory queue before any refill does.
  auto refill = [&]() {
    wg_barrier();
    if (ring_free) static_for<0, RING>([&](auto si) { ic.issue(p, L, w, ra[si.value], rb[si.value]); });
    ring_free = false;
  };
  stamp();
  wg_barrier();  // A of stage 0

  const int S = p.S;
  for (int k = 0;; ++k) {
    const Stage st = stage_at(p, L, k, w);
    if (st.type == ST_ATT) {
      AttnState<GMAX> as;
      att_reset<GMAX>(as);
      static_for<0, AMK_ATT_PF>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        if (st.pf0 + i < st.c0) att_consume<HD, GMAX>(p, L, st.t0, st.t1, st.pf0 + i, pk[i], pv[i], as);
      });
      run_stage<HD, FMT, GMAX, RING, true>(p, L, st, w, ra, rb, ic, as, ring_free);
      att_finish<HD, GMAX>(p, L, w, as);
    } else {
      AttnState<GMAX> unused;
      run_stage<HD, FMT, GMAX, RING, false>(p, L, st, w, ra, rb, ic, unused, ring_free);
    }
    if (AMK_DBG && trace != nullptr && threadIdx.x == 0) trace[3 + 11 * p.L + 2 * k] = wall_clock64();
    wg_barrier();  // B: this stage's partials are in LDS
    if (AMK_DBG && trace != nullptr && threadIdx.x == 0) trace[3 + 11 * p.L + 2 * k + 1] = wall_clock64();

    // ---- epilogue of stage k and the input of the next stage ----
    uint64_t* pdbg = (AMK_DBG && trace != nullptr) ? trace + 3 + 11 * p.L + 2 * (5 * p.L + 1) + 8 * k : nullptr;
    const int l = st.layer;
    const int tid = opaque(threadIdx.x);
    const float4 sc = scn;  // this stage's scales (pair tid, or pairs 2 tid, 2 tid + 1 for gate/up)
    bool ok = true;
    if (st.type == ST_QKV) {
      const uint32_t tg = tag_of(p, l, kTagQKV);
      if (tid < st.np) {
        float y0 = pair_sum(L, st.C, st.nch, tid, 0) * sc.x, y1 = pair_sum(L, st.C, st.nch, tid, 1) * sc.y;
        const int pr = st.pb0 + tid;
        const int hb = pr / half, i = pr - hb * half;
        float a = y0, c2 = y1;
        if (hb < p.nq + p.nkv) {  // RoPE (rotate-half pairs i, i + hd/2)
          const float cs = L.rope[i], sn = L.rope[half + i];
          a = y0 * cs - y1 * sn;
          c2 = y1 * cs + y0 * sn;
        }
        if (hb < p.nq) {
          st_tag(p.tq + hb * HD + i, __float_as_uint(a), tg);
          st_tag(p.tq + hb * HD + i + half, __float_as_uint(c2), tg);
        } else {
          const int kvs = hb < p.nq + p.nkv ? 0 : 1;
          const int g = hb - p.nq - kvs * p.nkv;
          const uint32_t ba = f32_to_bf16(a), bc = f32_to_bf16(c2);
          uint16_t* dst = p.kv + ((static_cast<size_t>(l * 2 + kvs) * p.nkv + g) * p.max_ctx + p.pos) * HD;
          dst[i] = static_cast<uint16_t>(ba);
          dst[i + half] = static_cast<uint16_t>(bc);
          st_tag(p.tkv + (kvs * p.nkv + g) * half + i, ba | (bc << 16), tg);
        }
      }
      stamp();
      // input of attention: q of the G heads of kv head g, and K/V(pos) when the unit holds pos
      const Stage sa = stage_at(p, L, k + 1, w);
      if (sa.C > 0) {
        const bool has_pos = sa.t1 == p.pos + 1;
        const int nq4 = G * HD / 2, nkv4 = has_pos ? half / 2 : 0;
        const int oq = toff(p, p.tq) + sa.g * G * HD * 8, okk = toff(p, p.tkv) + sa.g * half * 8,
                  ov = toff(p, p.tkv) + (p.nkv + sa.g) * half * 8;
        uint16_t* kvp = reinterpret_cast<uint16_t*>(L.vec + G * HD);
        ok = poll_block<2>(
            p, nq4 + 2 * nkv4, tg,
            [&](int qi) {
              return qi < nq4 ? oq + 16 * qi : (qi < nq4 + nkv4 ? okk + 16 * (qi - nq4) : ov + 16 * (qi - nq4 - nkv4));
            },
            [&](auto, int qi, uint32_t a, uint32_t c2) {
              if (qi < nq4) {
                L.vec[2 * qi] = __uint_as_float(a);
                L.vec[2 * qi + 1] = __uint_as_float(c2);
              } else {
                const int r = qi - nq4;
                const int kvs = r < nkv4 ? 0 : 1;
                const int i = 2 * (r - kvs * nkv4);
                uint16_t* d = kvp + kvs * HD;
                d[i] = static_cast<uint16_t>(a & 0xffffu);
                d[i + half] = static_cast<uint16_t>(a >> 16);
                d[i + 1] = static_cast<uint16_t>(c2 & 0xffffu);
                d[i + 1 + half] = static_cast<uint16_t>(c2 >> 16);
              }
            },
            refill, pdbg);
      } else {
        refill();
      }
      load_norm_weight(p.norm_post + static_cast<size_t>(l) * H, H, nwv);  // for the norm after O
      stamp();
    } else if (st.type == ST_ATT) {
      const bool active = st.C > 0;
      const int j = active ? b - st.g * S : 0;
      const uint32_t tpart = tag_of(p, l, kTagPart);
      // merge the waves' states into this unit's partial (max, sum, weighted values)
      if (active) {
        for (int it = tid; it < G * HD; it += kThreads) {
          const int h = it / HD, d = it - h * HD;
          float M = NEG_INF;
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, L.part[(ww * G + h) * (HD + 2) + HD]);
          float A = 0.f, Ls = 0.f;
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) {
            const float* src = L.part + (ww * G + h) * (HD + 2);
            const float mw = src[HD];
            const float e = (mw == NEG_INF) ? 0.f : __expf(mw - M);
            A += src[d] * e;
            Ls += src[HD + 1] * e;
          }
          uint64_t* dst = p.tpart + ((static_cast<size_t>(st.g * G + h) * p.s_cap + j) * (HD + 2));
          st_tag(dst + d, __float_as_uint(A), tpart);
          if (d == 0) {
            st_tag(dst + HD, __float_as_uint(M), tpart);
            st_tag(dst + HD + 1, __float_as_uint(Ls), tpart);
          }
        }
      }
      stamp();
      // this block's slice of the kv head's outputs, merged over the S splits: thread t holds
      // split t % SP of output word w0 + t / SP (+ 512 / SP in the second round)
      const uint32_t to_tag = tag_of(p, l, kTagO);
      if (active) {
        const int nw = G * HD / 2;  // output words of the kv head (2 bf16 each)
        const int w0 = nw * j / S, w1 = nw * (j + 1) / S;
        int SP = 1;
        while (SP < S) SP *= 2;
        const int wpr = kThreads / SP;  // words per round
        const int obase = toff(p, p.tpart);
        float av[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
        float mv[2] = {NEG_INF, NEG_INF}, lv[2] = {0.f, 0.f};
        ok = poll_block<4>(
            p, 4 * kThreads, tpart,
            [&](int qi) {
              const int bq = qi / kThreads, t = qi - bq * kThreads;
              const int r = bq >> 1, which = bq & 1;
              const int wd = w0 + r * wpr + t / SP, sp = t % SP;
              if (wd >= w1 || sp >= S) return kOOB;
              const int h = wd / (HD / 2), d = 2 * (wd - h * (HD / 2));
              const int rec = (st.g * G + h) * p.s_cap + sp;
              return obase + (rec * (HD + 2) + (which ? HD : d)) * 8;
            },
            [&](auto bi, int, uint32_t a, uint32_t c2) {
              constexpr int bq = decltype(bi)::value;
              if (bq & 1) {
                mv[bq >> 1] = __uint_as_float(a);
                lv[bq >> 1] = __uint_as_float(c2);
              } else {
                av[bq >> 1][0] = __uint_as_float(a);
                av[bq >> 1][1] = __uint_as_float(c2);
              }
            },
            refill, pdbg);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int wd = w0 + r * wpr + tid / SP, sp = tid % SP;
          const bool v = wd < w1 && sp < S;
          const float mj = v ? mv[r] : NEG_INF;
          const float M = seg_max(mj, SP);
          const float e = (mj == NEG_INF) ? 0.f : __expf(mj - M);
          const float Ls = seg_sum(v ? lv[r] * e : 0.f, SP);
          const float wgt = e * (1.0f / Ls);
          const float o0 = seg_sum(v ? av[r][0] * wgt : 0.f, SP);
          const float o1 = seg_sum(v ? av[r][1] * wgt : 0.f, SP);
          if (ok && v && sp == 0) {
            const int h = wd / (HD / 2), d = 2 * (wd - h * (HD / 2));
            st_tag(p.to + ((st.g * G + h) * HD + d) / 2, f32_to_bf16(o0) | (f32_to_bf16(o1) << 16), to_tag);
          }
        }
      } else {
        refill();
      }
      stamp();
      if (ok) ok = vector_from_words<FMT>(p, L, p.to, p.nq * HD, to_tag, [] {}, pdbg ? pdbg + 4 : nullptr);
      const Stage so = stage_at(p, L, k + 1, w);  // the O-projection's scales, for the next hand-off
      if (FMT == 1) scn = load_scales(stage_s(p, ST_O, l) + 2 * so.pb0, so.np, false);
      stamp();
    } else if (st.type == ST_O || st.type == ST_D) {
      const bool is_o = st.type == ST_O;
      const uint32_t tg = tag_of(p, l, is_o ? kTagXO : kTagXD);
      if (tid < st.np) {
        const float y0 = pair_sum(L, st.C, st.nch, tid, 0) * sc.x, y1 = pair_sum(L, st.C, st.nch, tid, 1) * sc.y;
        const float x0 = L.xres[2 * tid] + y0, x1 = L.xres[2 * tid + 1] + y1;
        L.xres[2 * tid] = x0;
        L.xres[2 * tid + 1] = x1;
        st_tag(p.tx + 2 * (st.pb0 + tid), __float_as_uint(x0), tg);
        st_tag(p.tx + 2 * (st.pb0 + tid) + 1, __float_as_uint(x1), tg);
      }
      stamp();
      // input of the next GEMV: RMSNorm of the new residual (gate/up, next layer's QKV, lm_head)
      ok = norm_from_x<FMT>(p, L, tg, nwv, refill, pdbg);
      if (AMK_ATT_PF > 0 && !is_o && l + 1 < p.L) att_prefetch<HD, AMK_ATT_PF>(p, L, l + 1, w, pk, pv);
      const Stage sn = stage_at(p, L, k + 1, w);
      if (FMT == 1) scn = load_scales(stage_s(p, sn.type, sn.layer) + 2 * sn.pb0, sn.np, sn.type == ST_GU);
      stamp();
    } else if (st.type == ST_GU) {
      const uint32_t tg = tag_of(p, l, kTagM);
      if (2 * tid < st.np) {  // two pairs (two outputs) per word
        float g0 = pair_sum(L, st.C, st.nch, 2 * tid, 0) * sc.x, u0 = pair_sum(L, st.C, st.nch, 2 * tid, 1) * sc.y;
        float g1 = pair_sum(L, st.C, st.nch, 2 * tid + 1, 0) * sc.z, u1 = pair_sum(L, st.C, st.nch, 2 * tid + 1, 1) * sc.w;
        const float m0 = (g0 / (1.0f + expf(-g0))) * u0, m1 = (g1 / (1.0f + expf(-g1))) * u1;
        st_tag(p.tm + (st.pb0 / 2 + tid), f32_to_bf16(m0) | (f32_to_bf16(m1) << 16), tg);
      }
      stamp();
      ok = vector_from_words<FMT>(p, L, p.tm, p.F, tg, refill, pdbg);
      const Stage sd = stage_at(p, L, k + 1, w);
      if (FMT == 1) scn = load_scales(stage_s(p, ST_D, l) + 2 * sd.pb0, sd.np, false);
      load_norm_weight(l + 1 < p.L ? p.norm_in + static_cast<size_t>(l + 1) * H : p.norm_final, H, nwv);
      stamp();
    } else {  // ST_LM
      if (tid < st.np) {
        p.logits[2 * (st.pb0 + tid)] = pair_sum(L, st.C, st.nch, tid, 0) * sc.x;
        p.logits[2 * (st.pb0 + tid) + 1] = pair_sum(L, st.C, st.nch, tid, 1) * sc.y;
      }
      stamp();
      break;
    }
    // A: the next stage's input is in LDS (or the step is abandoned)
    if (!ok) L.flag[0] = 1;
    wg_barrier();
    if (L.flag[0] != 0) break;
  }
  __builtin_amdgcn_s_waitcnt(0);
}

template __global__ void amk_stream_kernel<64, 0, 4, AMK_RING>(const KParams);
template __global__ void amk_stream_kernel<64, 1, 4, AMK_RING>(const KParams);
template __global__ void amk_stream_kernel<128, 0, 4, AMK_RING>(const KParams);
template __global__ void amk_stream_kernel<128, 1, 4, AMK_RING>(const KParams);

}  // namespace sk
}  // namespace amk

extern "C" __attribute__((visibility("hidden"))) const void* amk_stream_kernel_handle(int head_dim, int fmt, int gmax) {
  using namespace amk::sk;
  if (gmax != 4) return nullptr;
  if (head_dim == 64)
    return fmt ? (const void*)&amk_stream_kernel<64, 1, 4, AMK_RING> : (const void*)&amk_stream_kernel<64, 0, 4, AMK_RING>;
  if (head_dim == 128)
    return fmt ? (const void*)&amk_stream_kernel<128, 1, 4, AMK_RING> : (const void*)&amk_stream_kernel<128, 0, 4, AMK_RING>;
  return nullptr;
}
