// Persistent cooperative decode kernel for gfx950 (MI355X): one launch per token runs the
// whole Llama forward pass — RMSNorm, QKV GEMV + RoPE + KV append, split-KV GQA attention,
// O-projection + residual, RMSNorm + SwiGLU gate/up, down + residual, final RMSNorm + lm_head.
//
// Method: the decode-megakernel pages (AutoMegaKernel paper index, Abstract; gist.science
// explainer, Technical Summary > Problem Statement and Methodology) fuse the forward pass of a
// Llama-family model into one persistent cooperative kernel whose blocks synchronise inside the
// launch instead of at kernel boundaries, and prefetch weights while they wait. This file is an
// MI355X design of that idea, not a translation of the pages' CUDA:
//
//  * Grid: one 512-thread block per compute unit (256 on MI355X), launched cooperatively so
//    all blocks are co-resident. Each GEMV stage splits its row pairs evenly over all 2048
//    waves; every weight byte is streamed once with coalesced non-temporal dwordx4 loads.
//  * Grid-level synchronisation by tagged hand-offs, not barriers: every value one stage passes
//    to the next (residual, q, K/V of the new position, attention split partials, attention
//    output, SwiGLU output) is written as a word that carries the producing step's tag beside
//    the payload (64-bit words: payload low, tag high; SwiGLU: bf16 high, 16 tag bits low). A
//    consumer block polls exactly the words it needs with agent-coherent (sc1) loads until all
//    carry the expected tag, so it waits for its own producers only and the data arrives with
//    the flag in one round trip. Tags grow by 6 per layer plus 1 per launch (the host advances
//    the base), so words never need clearing. Waits are bounded; a timeout raises a device error
//    flag and every block leaves the kernel.
//  * Prefetch across a hand-off: before a block starts polling a stage's input vector it issues
//    that stage's operand window (row scales, RoPE tables or residual) and its first two weight
//    items into registers; attention issues its K/V loads before q arrives. A hand-off's words
//    reach the other blocks through the memory side, behind the weight reads in flight, so the
//    depth in flight is a trade-off: an item is one 1 KB chunk slot per row for hidden sizes up to
//    2048 and two above (a template parameter), and with two-slot items the second prefetched
//    item leaves a little after the first.
//  * Activations: the GEMV input vector of a stage (RMSNorm output, attention output, SwiGLU
//    output) is staged in LDS as fp32 holding bf16-rounded values (as bf16 for int4 weights),
//    in a swizzled layout so the 16-byte LDS reads of a lane per weight chunk are bank-conflict
//    free.
//  * W8A16: int8 codes convert with one v_cvt_f32_i32 (SDWA byte select, sign extend) per
//    weight and feed an fp32 FMA; the per-row fp32 scale multiplies the wave-reduced sum.
//    W4A16: sign-magnitude codes, eight per dword, laid out so that two masks turn a dword into
//    eight fp8 (e4m3) subnormals of value q * 2^-9; gfx950's fp8-to-bf16 pair conversion and
//    bf16 pair dot products then take two weights per instruction (1.375 VALU per weight).
//    W4A16-G128: the same codes; a lane's 32 columns of a chunk lie in one 128-column group, so
//    the lane's partial sum is multiplied by that group's fp16 scale before it joins the row.
//  * Row pairs: rows are packed at load time so that rows i and i + hd/2 of one head (a RoPE
//    pair) and rows n of gate and up (a SwiGLU pair) are adjacent; one wave computes both rows
//    of a pair, so the RoPE / SwiGLU / residual epilogues need no cross-wave exchange.
//  * Attention: split-KV over (kv head, position range) units, one unit per block. The G query
//    heads of a kv head share every K/V load. Each wave takes 16-position tiles: K and V rows
//    are loaded whole into a per-wave LDS tile, the G heads' scores and the weighted values are
//    bf16 matrix-core products (q and the softmax weights split into high and low bf16 parts),
//    and each head keeps an online softmax in base-2 units. The block's waves then merge in LDS
//    into one tagged partial (values, max, sum) per unit; every block of the kv head merges one
//    slice of the head's outputs over all splits by log-sum-exp weights (DPP segmented
//    reductions) and writes it as tagged bf16 pairs. A context short enough for one split per
//    kv head skips that second merge: the unit writes the normalised output itself.
//  * Matrix cores for attention only: a batch-1 GEMV is a matrix-vector product, far below the
//    MFMA ridge point, so the projections run on the VALU; attention's per-tile products (up to
//    16 heads by 16 positions by hd) are small dense contractions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "amk_kparams.h"

namespace amk {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// agent-coherent accesses (sc1) for data exchanged between blocks
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ldc(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Tagged exchange word: payload in the low 32 bits, the tag of the stage that wrote it in the
// high 32 bits. A 64-bit aligned store is single-copy atomic, so a payload is never seen with
// another stage's tag.
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t payload, uint32_t tag) {
  __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 32-bit exchange word for a bf16 value: the value in the high half, the low 16 bits of the tag
// in the low half (single-copy atomic as well).
__device__ __forceinline__ void st_tag16(uint32_t* p, uint16_t value, uint32_t tag) {
  __hip_atomic_store(p, (static_cast<uint32_t>(value) << 16) | (tag & 0xffffu), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_payload(const uint64_t* p) {
  return __uint_as_float(static_cast<uint32_t>(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
}

// An empty asm that hides a value from the optimizer. Stage functions start from an opaque
// copy of the thread index so the compiler recomputes their (cheap) per-thread addresses
// inside the layer loop instead of hoisting dozens of them out of it and spilling them.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Wave index as a wave-uniform (scalar) value, so per-wave work splits stay in SGPRs.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(opaque(threadIdx.x) >> 6); }

// Raw buffer resource over [base, base + bytes) and a non-temporal 16-byte buffer load. A lane
// whose voffset is kOOB (beyond the resource) receives zeros without a branch.
constexpr int kOOB = static_cast<int>(0x80000000u);
constexpr int kBufCacheNT = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ i32x4 ldbuf(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kBufCacheNT);
}
// Cache policy of the agent-coherent (sc1) 16-byte buffer loads that poll vectors written by
// other blocks in this launch.
constexpr int kBufCacheSC1 = 16;

// ------------------------------------------------------------------------------------------
// bf16 <-> fp32
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(int v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ float bf_hi(int v) { return __uint_as_float(static_cast<uint32_t>(v) & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {  // round to nearest, ties to even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }
__device__ __forceinline__ float i8_to_f32(int v, int k) {
  return static_cast<float>(static_cast<signed char>(static_cast<uint32_t>(v) >> (8 * k)));
}

// ------------------------------------------------------------------------------------------
// cross-lane sums
// ------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  // every lane of the row patterns used here reads a lane of its own row; written as an update
  // with a zero fill so the compiler folds the move into the consuming add / max (one DPP op)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum over the 2^k lanes of each aligned group (k = 3: 8 lanes, k = 4: 16 lanes), in every lane
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror: adds the other quad of each 8-lane half
  if (LANES == 16) v += dpp<0x140>(v);  // row_mirror: adds the other half of each row
  return v;
}
// v from lane (lane ^ OFF) for OFF in {8, 16, 32}, in VALU: a DPP rotate by 8 inside each row of
// 16 lanes, or the gfx950 permlane swaps that exchange rows (16) and halves (32) of the wave.
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
// max / sum over each aligned group of SP lanes (SP a power of two <= 64, wave-uniform), in
// every lane of the group
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
// weight formats and the LDS layout of a GEMV input vector
// ------------------------------------------------------------------------------------------
// BITS per weight. A 1 KB weight chunk covers CW columns and lane L owns LC consecutive columns
// of it (16 bytes). Per chunk the lane reads NR 16-byte words of activations, and one chunk's
// activations span XCS floats of LDS.
template <int FMT> struct Fmt;
template <> struct Fmt<0> { static constexpr int BITS = 16, CW = 512, LC = 8, NR = 1, XCS = 256; };    // bf16
template <> struct Fmt<1> { static constexpr int BITS = 8, CW = 1024, LC = 16, NR = 4, XCS = 1024; };  // int8
template <> struct Fmt<2> { static constexpr int BITS = 4, CW = 2048, LC = 32, NR = 4, XCS = 1024; };  // int4
template <> struct Fmt<3> { static constexpr int BITS = 4, CW = 2048, LC = 32, NR = 4, XCS = 1024; };  // int4, group scales
// Format 3 stores its codes as format 2 does; each run of 128 columns (four lanes' columns of a
// chunk) has an fp16 scale per row. The 16 group scales of a chunk, for both rows of a pair, are
// 64 bytes: dword j holds the scale of group j of row 0 (low half) and of row 1 (high half), and
// the dwords of pair pr, chunk ch start at byte (pr * nch + ch) * 64 of the matrix's scale array.
template <int FMT> constexpr bool kInt4 = FMT == 2 || FMT == 3;
// int8 weights: the activations are fp32 in LDS. Column e is stored at chunk*CW + (k/4)*256 +
// L*4 + k%4, k = e's index inside the lane, so the lane's k/4-th float4 sits at a 16-byte lane
// stride: conflict-free ds_read_b128.
// bf16 and int4 weights: the activations are bf16 in LDS (they are bf16 values). For bf16 the
// vector is in column order (lane L's eight columns are its 16-byte word). For int4 the lane's
// d-th 16-byte word holds its columns 8d .. 8d + 7 in order and sits at 16 * (d * 64 + L) bytes
// into the chunk's 4 KB; swz16 gives the 16-bit index.
template <int FMT>
__device__ __forceinline__ int swz(int e) {
  constexpr int CW = Fmt<FMT>::CW, LC = Fmt<FMT>::LC;
  const int ch = e / CW, r = e - ch * CW, ln = r / LC, k = r - ln * LC;
  return ch * CW + (k >> 2) * 256 + ln * 4 + (k & 3);
}
__device__ __forceinline__ int swz16(int e) {
  const int ch = e >> 11, r = e & 2047, ln = r >> 5, k = r & 31;
  return ch * 2048 + (((k >> 3) * 64 + ln) << 3) + (k & 7);
}
template <int FMT>
__device__ __forceinline__ int padded(int K) {
  constexpr int CW = Fmt<FMT>::CW;
  return (K + CW - 1) / CW * CW;
}
// Stores activation e (a bf16 value held in a float) into a GEMV input vector in LDS; put_x4
// stores columns e .. e + 3 (e a multiple of 4).
template <int FMT>
__device__ __forceinline__ void put_x(float* xs, int e, float v) {
  if constexpr (kInt4<FMT>) reinterpret_cast<uint16_t*>(xs)[swz16(e)] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
  else if constexpr (FMT == 0) reinterpret_cast<uint16_t*>(xs)[e] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
  else xs[swz<FMT>(e)] = v;
}
template <int FMT>
__device__ __forceinline__ void put_x4(float* xs, int e, f32x4 v) {
  if constexpr (FMT != 1) {
    const uint32_t lo = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
    const uint32_t hi = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xffff0000u);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(xs) + (kInt4<FMT> ? swz16(e) : e)) = uint2{lo, hi};
  } else {
    *reinterpret_cast<f32x4*>(xs + swz<FMT>(e)) = v;
  }
}

// Workgroup barrier that waits only for this wave's LDS traffic (lgkmcnt 0): weight loads in
// flight stay in flight across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  wg_barrier();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  wg_barrier();
  return t;
}

__device__ __forceinline__ uint32_t tag_of(const KParams& p, int layer, int which) {
  return p.tag0 + static_cast<uint32_t>(layer * kTagsPerLayer + which);
}
// byte offset of a tagged buffer inside the tagged region
// The step's input token: the launch argument, or the device-resident token of a greedy step
// (read again wherever needed; it does not change during the launch). Out-of-range device tokens
// decode token 0; the launch reports them through the error flag (see the kernel entry).
__device__ __forceinline__ int step_token(const KParams& p) {
  if (p.token_dev == nullptr) return p.token;
  const int t = __builtin_amdgcn_readfirstlane(*p.token_dev);
  return (t >= 0 && t < p.V) ? t : 0;
}

__device__ __forceinline__ int toff(const KParams& p, const uint64_t* buf) {
  return static_cast<int>(reinterpret_cast<const uint8_t*>(buf) - reinterpret_cast<const uint8_t*>(p.tagged));
}

// Raises device error `code` unless another one was raised first in this launch: the first
// raiser also writes the code to the pinned host word, where the next step call finds it without
// synchronising (exactly one write per failed launch).
__device__ __forceinline__ void raise_error(const KParams& p, unsigned code) {
  unsigned expected = 0u;
  if (__hip_atomic_compare_exchange_strong(p.err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT))
    __hip_atomic_store(p.herr, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Per-stage dump of layer l (see amk_set_dump): the slots in the order of the dump layout.
enum { kDH = 0, kDQKV, kDQ, kDO, kDWO, kDXO, kDH2, kDGU, kDM, kDWD, kDXD };
__device__ __forceinline__ float* dump_at(const KParams& p, int l, int slot) {
  if (p.dump == nullptr) return nullptr;
  const int H = p.H, QD = p.nq * p.hd, QKV = QD + 2 * p.nkv * p.hd, F = p.F;
  const int off[11] = {0, H, H + QKV, H + QKV + QD, H + QKV + 2 * QD, 2 * H + QKV + 2 * QD, 3 * H + QKV + 2 * QD,
                       4 * H + QKV + 2 * QD, 4 * H + QKV + 2 * QD + 2 * F, 4 * H + QKV + 2 * QD + 3 * F,
                       5 * H + QKV + 2 * QD + 3 * F};
  return p.dump + static_cast<int64_t>(l) * p.dump_stride + (l < p.L ? off[slot] : 0);
}

// Bound of a hand-off wait, checked after its reload number `it`: false once the step must be
// abandoned. The error word is read every 16 reloads (an error raised elsewhere keeps its code);
// the clock also after the second reload, so that a spin limit of one tick ends the first poll
// that waits at all.
__device__ __forceinline__ bool wait_ok(const KParams& p, unsigned it, uint64_t t_start) {
  const bool round16 = (it & 15u) == 0;
  if (round16 && ldc(p.err) != 0u) return false;
  if ((round16 || it == 2) && wall_clock64() - t_start > p.spin_limit) {
    raise_error(p, kErrTimeout);
    return false;
  }
  return true;
}

// Block-wide poll of nquads 16-byte quads (two tagged words each) of the tagged region: thread t
// owns quads t + 512 b, b < VB (then further batches). When both tags of every quad of a thread
// equal `tag` on the first read (the common case once the producers are done) visit(b, qi,
// payload0, payload1) runs straight away; otherwise the thread re-reads its pending quads until
// they are fresh. off(qi) is the quad's byte offset, or kOOB for a quad to skip. Returns false if
// the step must be abandoned (timeout, or an error raised elsewhere).
template <int VB, class Off, class Visit>
__device__ __forceinline__ bool poll_block(const KParams& p, int nquads, uint32_t tag, Off off, Visit visit) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.tagged, p.tagged_bytes);
  const int tid = opaque(threadIdx.x);
  for (int q0 = 0; q0 < nquads; q0 += kThreads * VB) {
    i32x4 v[VB];
    uint32_t skip = 0;
#pragma unroll
    for (int b = 0; b < VB; ++b) {
      const int qi = q0 + b * kThreads + tid;
      const int o = qi < nquads ? off(qi) : kOOB;
      skip |= (o == kOOB) ? (1u << b) : 0u;
      v[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, kBufCacheSC1);
    }
    auto pending = [&]() {
      uint32_t pend = 0;
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        const bool good = ((skip >> b) & 1u) ||
                          (static_cast<uint32_t>(v[b].y) == tag && static_cast<uint32_t>(v[b].w) == tag);
        pend |= good ? 0u : (1u << b);
      }
      return pend;
    };
    uint32_t pend = pending();
    if (pend != 0u) {
      const uint64_t t_start = wall_clock64();
      unsigned it = 0;
      while (pend != 0u) {
        if (!wait_ok(p, ++it, t_start)) return false;
        __builtin_amdgcn_s_sleep(0);
#pragma unroll
        for (int b = 0; b < VB; ++b)
          if (pend & (1u << b))
            v[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, off(q0 + b * kThreads + tid), 0, kBufCacheSC1);
        pend = pending();
      }
    }
#pragma unroll
    for (int b = 0; b < VB; ++b)
      if (!((skip >> b) & 1u))
        visit(b, q0 + b * kThreads + tid, static_cast<uint32_t>(v[b].x), static_cast<uint32_t>(v[b].z));
  }
  return true;
}

// Block-wide poll of bf16 values in 32-bit tagged words (value << 16 | tag & 0xffff) into the
// GEMV input vector, zero padded: thread t owns quads t + 512 b (four words = four consecutive
// elements, one float4 of the swizzled layout). Returns false if abandoned.
template <int FMT>
__device__ __forceinline__ bool vector_from_words16(const KParams& p, const uint32_t* src, int K, uint32_t tag,
                                                    float* xs) {
  constexpr int VB = 8;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.tagged, p.tagged_bytes);
  const int tid = opaque(threadIdx.x);
  const int ob = static_cast<int>(reinterpret_cast<const uint8_t*>(src) - reinterpret_cast<const uint8_t*>(p.tagged));
  const uint32_t t16 = tag & 0xffffu;
  const int nq = K / 4;
  for (int q0 = 0; q0 < nq; q0 += kThreads * VB) {
    i32x4 v[VB];
#pragma unroll
    for (int b = 0; b < VB; ++b) {
      const int qi = q0 + b * kThreads + tid;
      v[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, qi < nq ? ob + 16 * qi : kOOB, 0, kBufCacheSC1);
    }
    auto pending = [&]() {
      uint32_t pend = 0;
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        const int qi = q0 + b * kThreads + tid;
        const bool good = qi >= nq || (((static_cast<uint32_t>(v[b].x) & 0xffffu) == t16) &&
                                       ((static_cast<uint32_t>(v[b].y) & 0xffffu) == t16) &&
                                       ((static_cast<uint32_t>(v[b].z) & 0xffffu) == t16) &&
                                       ((static_cast<uint32_t>(v[b].w) & 0xffffu) == t16));
        pend |= good ? 0u : (1u << b);
      }
      return pend;
    };
    uint32_t pend = pending();
    if (pend != 0u) {
      const uint64_t t_start = wall_clock64();
      unsigned it = 0;
      while (pend != 0u) {
        if (!wait_ok(p, ++it, t_start)) return false;
        __builtin_amdgcn_s_sleep(0);
#pragma unroll
        for (int b = 0; b < VB; ++b)
          if (pend & (1u << b))
            v[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, ob + 16 * (q0 + b * kThreads + tid), 0, kBufCacheSC1);
        pend = pending();
      }
    }
#pragma unroll
    for (int b = 0; b < VB; ++b) {
      const int qi = q0 + b * kThreads + tid;
      if (qi < nq)
        put_x4<FMT>(xs, 4 * qi, f32x4{bf_hi(v[b].x), bf_hi(v[b].y), bf_hi(v[b].z), bf_hi(v[b].w)});
    }
  }
  for (int e = K + tid; e < padded<FMT>(K); e += kThreads) put_x<FMT>(xs, e, 0.f);
  return true;
}

constexpr int kNormVB = 8;  // RMSNorm inputs up to 2 * 8 * 512 = 8192 elements

// xs <- bf16((x * r) * w) for the thread's element pairs e = 2 (b * 512 + tid), zero padded to
// whole weight chunks; block 0 also writes the values to the dump slot dh (when dumping).
template <int FMT>
__device__ __forceinline__ void norm_out(int H, float r, const float2 (&xv)[kNormVB], const float2 (&wv)[kNormVB],
                                         float* xs, float* dh) {
#pragma clang fp contract(off)
  const int tid = opaque(threadIdx.x);
  const bool dump = dh != nullptr && blockIdx.x == 0;
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) {
    const int e = 2 * (b * kThreads + tid);
    if (e < H) {
      const float h0 = round_bf16((xv[b].x * r) * wv[b].x), h1 = round_bf16((xv[b].y * r) * wv[b].y);
      put_x<FMT>(xs, e, h0);
      put_x<FMT>(xs, e + 1, h1);
      if (dump) *reinterpret_cast<float2*>(dh + e) = float2{h0, h1};
    }
  }
  for (int e = H + tid; e < padded<FMT>(H); e += kThreads) put_x<FMT>(xs, e, 0.f);
}

// xs <- bf16((x * rsqrt(mean(x^2) + eps)) * w) for the first layer, x = the bf16 embedding row,
// zero padded to whole weight chunks.
template <int FMT>
__device__ __forceinline__ void rmsnorm_embed_to_lds(const KParams& p, const float* __restrict__ w, float* xs,
                                                     float* red, float* dh) {
#pragma clang fp contract(off)
  const int H = p.H, tid = opaque(threadIdx.x);
  const uint16_t* row = p.embed + static_cast<size_t>(step_token(p)) * H;
  float2 xv[kNormVB], wv[kNormVB];
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) {
    const int e = 2 * (b * kThreads + tid);
    xv[b] = float2{0.f, 0.f};
    wv[b] = float2{0.f, 0.f};
    if (e < H) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(row + e);
      xv[b] = float2{bf_lo(static_cast<int>(u)), bf_hi(static_cast<int>(u))};
      wv[b] = *reinterpret_cast<const float2*>(w + e);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) ss += xv[b].x * xv[b].x + xv[b].y * xv[b].y;
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + p.eps);
  norm_out<FMT>(H, r, xv, wv, xs, dh);
}

// xs <- RMSNorm of the residual x polled from its tagged words (tag `tag`), zero padded. The
// weights are loaded with the poll, in the same round trip. Returns false if abandoned.
template <int FMT>
__device__ __forceinline__ bool norm_from_x(const KParams& p, const float* __restrict__ w, uint32_t tag, float* xs,
                                            float* red, float* dh) {
#pragma clang fp contract(off)
  const int H = p.H, tid = opaque(threadIdx.x);
  float2 xv[kNormVB], wv[kNormVB];
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) {
    const int e = 2 * (b * kThreads + tid);
    wv[b] = e < H ? *reinterpret_cast<const float2*>(w + e) : float2{0.f, 0.f};
    xv[b] = float2{0.f, 0.f};
  }
  const int ob = toff(p, p.tx);
  const bool ok = poll_block<kNormVB>(p, H / 2, tag, [&](int qi) { return ob + 16 * qi; },
                                      [&](int b, int, uint32_t a, uint32_t c) {
                                        xv[b] = float2{__uint_as_float(a), __uint_as_float(c)};
                                      });
  float ss = 0.f;
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) ss += xv[b].x * xv[b].x + xv[b].y * xv[b].y;
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + p.eps);
  norm_out<FMT>(H, r, xv, wv, xs, dh);
  return ok;
}

// xs <- a bf16 vector of K elements polled from its tagged words (two bf16 per word), zero
// padded. Four consecutive elements land in one float4 of the swizzled layout.
template <int FMT>
__device__ __forceinline__ bool vector_from_words(const KParams& p, const uint64_t* src, int K, uint32_t tag,
                                                  float* xs, float* dv) {
  const int ob = toff(p, src);
  const bool dump = dv != nullptr && blockIdx.x == 0;
  const bool ok = poll_block<8>(p, K / 4, tag, [&](int qi) { return ob + 16 * qi; },
                                [&](int, int qi, uint32_t a, uint32_t c) {
                                  const f32x4 v{bf16_to_f32(a & 0xffffu), bf16_to_f32(a >> 16),
                                                bf16_to_f32(c & 0xffffu), bf16_to_f32(c >> 16)};
                                  put_x4<FMT>(xs, 4 * qi, v);
                                  if (dump) *reinterpret_cast<f32x4*>(dv + 4 * qi) = v;
                                });
  for (int e = K + opaque(threadIdx.x); e < padded<FMT>(K); e += kThreads) put_x<FMT>(xs, e, 0.f);
  return ok;
}

// ------------------------------------------------------------------------------------------
// GEMV stage over row pairs
// ------------------------------------------------------------------------------------------
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// CG (a kernel template parameter, 1 or 2): chunk slots per item, so an item is 2 rows x CG x
// 16 B dwordx4 loads per lane and a wave keeps two items (2 CG KB) in flight. Two slots stream the
// Llama-3-8B shapes fastest; one slot, half the reads queued at each hand-off, is faster for
// hidden sizes up to 2048 (the host picks by hidden size).
constexpr int kSeg = 32; // pairs per operand window (lane j holds the operand of packed row 2*base + j)

// Registers that carry a GEMV stage's operand window and first two items across the wait for
// the stage's input vector.
template <int CG>
struct GemvRegs {
  i32x4 a0[CG], a1[CG], b0[CG], b1[CG];
  uint32_t sa[CG], sb[CG];  // group scales of the items' slots (format 3 only)
  float wA, wB;
};

// How one stage is split. A wave owns the contiguous pair range [pa, pb), processed in
// segments of at most kSeg pairs. Inside a segment, pair k's chunks occupy slots
// [k*cpp, k*cpp + nch) of a padded slot space (cpp = chunks per pair rounded so that items of
// CG slots never straddle a pair unevenly); an item is CG consecutive slots. Slots past a
// row's end or past the segment read zeros, so every item issues the same 8 loads.
struct GemvPlan {
  int RB;   // bytes per row
  int nch;  // 1 KB chunks per row
  int cpp;  // padded slots per pair: 1 or 2 when nch <= CG, else a multiple of CG
  int pa, pb;     // the wave's pairs, as local indices k in [pa, pb)
  int st0, sst;   // local index k is pair st0 + k * sst of the matrix
};
__device__ __forceinline__ int pidx(const GemvPlan& g, int k) { return g.st0 + k * g.sst; }

// Pairs are split over all waves of the grid by a strided map: wave w of block b is stream
// s = w * blocks + b and takes pairs s, s + NW, s + 2 NW, ... (NW = waves in the grid). At any
// moment the grid streams one sliding window of the matrix, consecutive pairs going to
// consecutive blocks (and so to different XCDs), and block b holds pair b of every stage.
template <int FMT, int CG>
__device__ __forceinline__ GemvPlan gemv_plan(int K, int npairs, int wave) {
  GemvPlan g;
  g.RB = K * Fmt<FMT>::BITS / 8;
  g.nch = (g.RB + 1023) >> 10;
  g.cpp = g.nch <= 1 ? 1 : g.nch <= 2 ? 2 : (g.nch + CG - 1) / CG * CG;
  const int NW = gridDim.x * kWaves;
  const int sw = wave * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x);
  g.pa = 0;
  g.pb = sw < npairs ? (npairs - sw + NW - 1) / NW : 0;
  g.st0 = sw;
  g.sst = NW;
  return g;
}

// Position in the slot space of a segment: pair k (relative to the segment base) and slot ch.
struct Cursor {
  int k, ch;
  __device__ __forceinline__ void advance(int cpp) {
    const int n = ch + 1;
    const bool wrap = n == cpp;
    ch = wrap ? 0 : n;
    k += wrap ? 1 : 0;
  }
};

// Eight int4 codes of one dword against their eight activations (bf16, in column order). Byte k
// of the dword holds the magnitude of column k in bits 0..2 and its sign in bit 7, the
// magnitude of column k + 4 in bits 4..6, and the sign of column (k - 1) mod 4 + 4 in bit 3.
// So w & 0x87878787 and (w rotated right by 4) & 0x87878787 are four e4m3 codes each whose
// values are exactly q * 2^-9 (exponent field zero: subnormals); each pair converts to a bf16
// pair exactly and enters a bf16 pair dot product (exact products, fp32 sum). The epilogue
// applies the factor 2^9.
__device__ __forceinline__ float dot8_i4(uint32_t w, const i32x4 x, float acc) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  const uint32_t lo = w & 0x87878787u;
  const uint32_t hi = __builtin_amdgcn_alignbit(w, w, 4) & 0x87878787u;
  // the pairs are taken from one 8-wide bf16 view of the word (this compiler drops the element
  // index of a bit cast of one int lane to a bf16 pair)
  const bf16x8_t xb = __builtin_bit_cast(bf16x8_t, x);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false),
                                        __builtin_shufflevector(xb, xb, 0, 1), acc, false);  // columns 0, 1
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true),
                                        __builtin_shufflevector(xb, xb, 2, 3), acc, false);  // 2, 3
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false),
                                        __builtin_shufflevector(xb, xb, 4, 5), acc, false);  // 4, 5
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true),
                                        __builtin_shufflevector(xb, xb, 6, 7), acc, false);  // 6, 7
  return acc;
}

// The activations of one slot: NR 16-byte reads per lane from the swizzled LDS vector.
template <int FMT>
struct XSlot {
  f32x4 v[Fmt<FMT>::NR];
};
template <int FMT>
__device__ __forceinline__ void load_x(const float* __restrict__ xl, XSlot<FMT>& x) {
#pragma unroll
  for (int k = 0; k < Fmt<FMT>::NR; ++k) x.v[k] = *reinterpret_cast<const f32x4*>(xl + k * 256);
}

template <int FMT>
__device__ __forceinline__ void chunk_fma(const i32x4 w0, const i32x4 w1, const XSlot<FMT>& xs, uint32_t gs,
                                          float& a0, float& a1) {
  if constexpr (FMT == 3) {
    // the lane's 32 columns lie in one group: their sum (in units of 2^-9), times the group's scale
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const i32x4 x = __builtin_bit_cast(i32x4, xs.v[d]);
      p0 = dot8_i4(static_cast<uint32_t>(w0[d]), x, p0);
      p1 = dot8_i4(static_cast<uint32_t>(w1[d]), x, p1);
    }
    const float s0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(gs & 0xffffu)));
    const float s1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(gs >> 16)));
    a0 = __builtin_fmaf(p0, s0, a0);
    a1 = __builtin_fmaf(p1, s1, a1);
  } else if constexpr (FMT == 2) {
    // dword d holds the lane's columns 8d .. 8d + 7; read d of the slot holds their activations
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const i32x4 x = __builtin_bit_cast(i32x4, xs.v[d]);
      a0 = dot8_i4(static_cast<uint32_t>(w0[d]), x, a0);
      a1 = dot8_i4(static_cast<uint32_t>(w1[d]), x, a1);
    }
  } else if constexpr (FMT == 1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f32x4 x = xs.v[d];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a0 = __builtin_fmaf(i8_to_f32(w0[d], k), x[k], a0);
        a1 = __builtin_fmaf(i8_to_f32(w1[d], k), x[k], a1);
      }
    }
  } else {
    // dword d holds the bf16 weights of columns 2d, 2d + 1; so does dword d of the activations
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    const bf16x8_t x = __builtin_bit_cast(bf16x8_t, xs.v[0]);
    const bf16x8_t u0 = __builtin_bit_cast(bf16x8_t, w0), u1 = __builtin_bit_cast(bf16x8_t, w1);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u0, u0, 0, 1), __builtin_shufflevector(x, x, 0, 1), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u1, u1, 0, 1), __builtin_shufflevector(x, x, 0, 1), a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u0, u0, 2, 3), __builtin_shufflevector(x, x, 2, 3), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u1, u1, 2, 3), __builtin_shufflevector(x, x, 2, 3), a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u0, u0, 4, 5), __builtin_shufflevector(x, x, 4, 5), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u1, u1, 4, 5), __builtin_shufflevector(x, x, 4, 5), a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u0, u0, 6, 7), __builtin_shufflevector(x, x, 6, 7), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(u1, u1, 6, 7), __builtin_shufflevector(x, x, 6, 7), a1, false);
  }
}

// Per-pair operands for a window of 32 pairs: lane j holds the value for row j & 1 of the
// window's pair j / 2: A = the row scale of per-row int8 / int4 weights, B = residual input (EPI_RESID) or RoPE cos
// (even j) / sin (odd j) of the pair (EPI_QKV).
template <int FMT, int EPI>
__device__ __forceinline__ void load_window(const KParams& p, const float* __restrict__ Sc, const GemvPlan& g,
                                            int wbase, bool resid_from_embed, float& A, float& B) {
  const int lane = __lane_id();
  const int k = wbase + (lane >> 1);
  const int row = 2 * pidx(g, k) + (lane & 1);
  A = 1.f;
  B = 0.f;
  if (k < g.pb) {
    if (FMT == 1 || FMT == 2) A = Sc[row];  // int4: the epilogue applies the factor 2^9
    if (EPI == EPI_RESID) {
      B = resid_from_embed ? bf16_to_f32(p.embed[static_cast<size_t>(step_token(p)) * p.H + row])
                           : ld_payload(p.tx + row);
    } else if (EPI == EPI_QKV) {
      const int half = p.hd >> 1;
      const int i = (row >> 1) % half;
      B = (row & 1) ? p.rope_sin[static_cast<size_t>(p.pos) * half + i] : p.rope_cos[static_cast<size_t>(p.pos) * half + i];
    }
  }
}

// Lane-0 state an epilogue carries across the pairs of one wave: the greedy argmax of the logits
// seen so far (value, index; rows arrive in increasing order, so a strict compare keeps the
// lowest index among equal values).
struct EpiState {
  float v;
  int i;
};

// Runs in lane 0 for one finished row pair: scale (applied by the caller), then q / K / V with
// RoPE (and the K/V append to the cache), the residual add, SwiGLU, or the logits. Values that
// cross blocks are written as tagged words (tag tg); a SwiGLU output is one 32-bit word. dp is
// the stage's dump slot (null unless dumping): the GEMV outputs and what the epilogue derives.
template <int EPI>
__device__ __forceinline__ void epilogue(const KParams& p, int layer, int pr, float y0, float y1, float b0, float b1,
                                         uint32_t tg, EpiState& st, float* dp) {
#pragma clang fp contract(off)
  if (EPI == EPI_QKV) {
    const int half = p.hd >> 1;
    const int hb = pr / half, i = pr - hb * half;
    float a = y0, b = y1;
    if (hb < p.nq + p.nkv) {
      const float c = b0, s = b1;
      a = y0 * c - y1 * s;
      b = y1 * c + y0 * s;
    }
    if (dp != nullptr) {  // rows hb * hd + i and hb * hd + i + half of q | k | v; then q rotated
      const int QKV = (p.nq + 2 * p.nkv) * p.hd;
      dp[hb * p.hd + i] = y0;
      dp[hb * p.hd + i + half] = y1;
      if (hb < p.nq) {
        dp[QKV + hb * p.hd + i] = a;
        dp[QKV + hb * p.hd + i + half] = b;
      }
    }
    if (hb < p.nq) {
      st_tag(p.tq + hb * p.hd + i, __float_as_uint(a), tg);
      st_tag(p.tq + hb * p.hd + i + half, __float_as_uint(b), tg);
    } else {
      const int kvs = hb < p.nq + p.nkv ? 0 : 1;
      const int g = hb - p.nq - kvs * p.nkv;
      const uint16_t ba = f32_to_bf16(a), bb = f32_to_bf16(b);
      uint16_t* dst = p.kv + ((static_cast<size_t>(layer * 2 + kvs) * p.nkv + g) * p.max_ctx + p.pos) * p.hd;
      dst[i] = ba;
      dst[i + half] = bb;
      st_tag(p.tkv + (kvs * p.nkv + g) * half + i, static_cast<uint32_t>(ba) | (static_cast<uint32_t>(bb) << 16), tg);
    }
  } else if (EPI == EPI_RESID) {
    const float x0 = b0 + y0, x1 = b1 + y1;
    st_tag(p.tx + 2 * pr, __float_as_uint(x0), tg);
    st_tag(p.tx + 2 * pr + 1, __float_as_uint(x1), tg);
    if (dp != nullptr) {  // projection output, then the residual after it
      *reinterpret_cast<float2*>(dp + 2 * pr) = float2{y0, y1};
      *reinterpret_cast<float2*>(dp + p.H + 2 * pr) = float2{x0, x1};
    }
  } else if (EPI == EPI_SWIGLU) {
    const float m = (y0 / (1.0f + expf(-y0))) * y1;
    const uint16_t mb = f32_to_bf16(m);
    st_tag16(reinterpret_cast<uint32_t*>(p.tm) + pr, mb, tg);
    if (dp != nullptr) {  // gate, up, then the SwiGLU output
      dp[pr] = y0;
      dp[p.F + pr] = y1;
      dp[2 * p.F + pr] = bf16_to_f32(mb);
    }
  } else {
    if (p.logits != nullptr) {
      p.logits[2 * pr] = y0;
      p.logits[2 * pr + 1] = y1;
    }
    if (y0 > st.v) {
      st.v = y0;
      st.i = 2 * pr;
    }
    if (y1 > st.v) {
      st.v = y1;
      st.i = 2 * pr + 1;
    }
  }
}

// Issues the two loads of the chunk slot at cursor c (both rows of its pair) and for format 3 the
// slot's group-scale dword (lane L takes group L / 4 of the chunk); advances c by one slot.
// np = pairs in the segment, base = first pair of the segment.
template <int FMT>
__device__ __forceinline__ void issue_slot(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t gsr, const GemvPlan& g,
                                           int base, int np, Cursor& c, i32x4& r0, i32x4& r1, uint32_t& gs) {
  const int lane = __lane_id();
  const bool v = c.ch < g.nch && c.k < np;
  const int off = c.ch * 1024 + lane * 16;
  const int voff = (v && off < g.RB) ? off : kOOB;
  // uniform by construction; readfirstlane keeps the compiler from moving it to VGPRs
  const int pr = v ? pidx(g, base + c.k) : 0;
  const int soff = __builtin_amdgcn_readfirstlane(2 * pr * g.RB);
  r0 = ldbuf(rs, voff, soff);
  r1 = ldbuf(rs, voff, soff + g.RB);
  if constexpr (FMT == 3) {
    const int goff = __builtin_amdgcn_readfirstlane((pr * g.nch + c.ch) * 64);
    gs = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(gsr, v ? (lane >> 2) * 4 : kOOB, goff, kBufCacheNT));
  }
  c.advance(g.cpp);
}

// Issues the CG slots (4 CG loads, plus the format-3 scales) of the item that starts at cursor c.
template <int FMT, int CG>
__device__ __forceinline__ void gemv_issue(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t gsr, const GemvPlan& g,
                                           int base, int np, Cursor& c, i32x4 (&r0)[CG], i32x4 (&r1)[CG],
                                           uint32_t (&gs)[CG]) {
#pragma unroll
  for (int s = 0; s < CG; ++s) issue_slot<FMT>(rs, gsr, g, base, np, c, r0[s], r1[s], gs[s]);
}

// Quantized weights refill each chunk slot of an item right after its FMAs, so its loads leave
// a slot earlier than a refill of the whole item after its last FMA (8B W8A16 0.8%, W4A16 1.3%,
// 1B W8A16 1.4% faster per token); bf16 weights, with far fewer VALU operations per slot, refill
// whole items (slot refills measured 0.5% slower there).
template <int FMT>
constexpr bool kSlotRefill = FMT != 0;
// An odd item count leaves a zero item in the loop's last iteration. int4 stages skip it (a
// branch on a uniform count): with one 2 KB chunk per row, QKV, O and gate/up have odd counts,
// and skipping measured 1.7% faster per token for 8B W4A16. For int8 (only the down projection
// has an odd count) the branch changes the compiler's load waits and measured 2% slower.
template <int FMT>
constexpr bool kSkipZeroItem = kInt4<FMT>;

// Accumulates the item at cursor c into (acc0, acc1); when a slot completes a pair, reduces it
// over the wave and lane 0 runs the epilogue. Slots that read zeros add nothing.
// Slots issue their LDS reads one slot ahead of their FMAs: xn holds the activations of the slot
// at cursor c on entry and of the slot after this item's last one on return. (With slot refills,
// reading ahead is also faster for int8 weights: 1B W8A16 2.1%, 8B 0.2% per token; with item
// refills it had measured 2% slower there.)
//
// With kSlotRefill, each slot's registers are refilled (cursor ci, two items ahead) as soon as
// its FMAs are issued.
template <int FMT, int EPI, int CG>
__device__ __forceinline__ void gemv_compute(const KParams& p, const GemvPlan& g, int base, int np, int layer,
                                             const float* xlane, i32x4 (&r0)[CG], i32x4 (&r1)[CG],
                                             uint32_t (&gs)[CG], float wA, float wB, Cursor& c, float& acc0, float& acc1, uint32_t tg,
                                             EpiState& st, XSlot<FMT>& xn, float* dp, __amdgpu_buffer_rsrc_t rs,
                                             __amdgpu_buffer_rsrc_t gsr, Cursor& ci) {
  constexpr int XCS = Fmt<FMT>::XCS;
#pragma unroll
  for (int s = 0; s < CG; ++s) {
    const XSlot<FMT> xc = xn;
    Cursor cn = c;
    cn.advance(g.cpp);
    load_x<FMT>(xlane + min(cn.ch, g.nch - 1) * XCS, xn);
    // keep the scheduler from hoisting the conversions of all slots at once (register spills)
    __builtin_amdgcn_sched_barrier(0);
    chunk_fma<FMT>(r0[s], r1[s], xc, gs[s], acc0, acc1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kSlotRefill<FMT>) issue_slot<FMT>(rs, gsr, g, base, np, ci, r0[s], r1[s], gs[s]);
    if (c.ch == g.nch - 1 && c.k < np) {
      float y0 = wave_sum(acc0), y1 = wave_sum(acc1);
      acc0 = acc1 = 0.f;
      const int j = 2 * c.k;
      if (FMT == 1 || FMT == 2) {
        y0 *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wA), j));
        y1 *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wA), j + 1));
      }
      if (kInt4<FMT>) {  // the int4 products arrived as q * 2^-9 (exact)
        y0 *= 512.f;
        y1 *= 512.f;
      }
      const float b0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wB), j));
      const float b1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wB), j + 1));
      if (__lane_id() == 0) epilogue<EPI>(p, layer, pidx(g, base + c.k), y0, y1, b0, b1, tg, st, dp);
    }
    c.advance(g.cpp);
  }
}

// Loads the operand window of the segment at `base` and issues the segment's first two items.
template <int FMT, int EPI, int CG>
__device__ __forceinline__ void gemv_segment_start(const KParams& p, __amdgpu_buffer_rsrc_t rs,
                                                   __amdgpu_buffer_rsrc_t gsr, const float* __restrict__ Sc,
                                                   const GemvPlan& g, int base, int np, bool rfe, bool two,
                                                   GemvRegs<CG>& R) {
  load_window<FMT, EPI>(p, Sc, g, base, rfe, R.wA, R.wB);
  Cursor c{0, 0};
  gemv_issue<FMT, CG>(rs, gsr, g, base, np, c, R.a0, R.a1, R.sa);
  if (two) gemv_issue<FMT, CG>(rs, gsr, g, base, np, c, R.b0, R.b1, R.sb);
}

// Buffer resource over a format-3 matrix's group scales (npairs * nch * 64 bytes); for the
// other formats an empty resource that no load uses.
template <int FMT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gscale_rsrc(const float* Sc, const GemvPlan& g, int npairs) {
  return make_rsrc(Sc, FMT == 3 ? static_cast<uint32_t>(npairs * g.nch * 64) : 0u);
}

// Issues the stage's operand window and first two items; called before the block polls the
// stage's input vector, so HBM keeps streaming while the producers of that vector finish. With
// two-slot items the second item leaves about 0.2 us (512 clocks) after the first: the hand-off
// words that the slowest producers store at this moment wait at the memory side behind the reads
// the grid has in flight, and half of this CU's reads are not yet among them (Llama-3-8B shapes
// 0.2-0.7% faster per token; longer delays, and any delay with one-slot items, measured slower).
template <int FMT, int EPI, int CG>
__device__ __forceinline__ void gemv_prefetch(const KParams& p, const uint8_t* __restrict__ W,
                                              const float* __restrict__ Sc, int K, int npairs, bool rfe,
                                              GemvRegs<CG>& R) {
  const GemvPlan g = gemv_plan<FMT, CG>(K, npairs, wave_id());
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, static_cast<uint32_t>(2 * npairs) * g.RB);
  const __amdgpu_buffer_rsrc_t gsr = gscale_rsrc<FMT>(Sc, g, npairs);
  const int np = min(kSeg, g.pb - g.pa);
  gemv_segment_start<FMT, EPI, CG>(p, rs, gsr, Sc, g, g.pa, np, rfe, CG == 1, R);
  if constexpr (CG == 2) {
    __builtin_amdgcn_s_sleep(8);
    Cursor c{0, 0};
    for (int s = 0; s < CG; ++s) c.advance(g.cpp);
    gemv_issue<FMT, CG>(rs, gsr, g, g.pa, np, c, R.b0, R.b1, R.sb);
  }
}

// Runs the stage. Items alternate between the two register buffers, each refilled two items
// ahead of its use; the loop body is branch free apart from the per-pair epilogue, so loads
// stay in flight across iterations. Returns the epilogue state of lane 0 (the wave's argmax for
// the logits stage).
template <int FMT, int EPI, int CG>
__device__ __forceinline__ EpiState gemv_run(const KParams& p, const uint8_t* __restrict__ W,
                                         const float* __restrict__ Sc, int K, int npairs, const float* xs,
                                         int layer, bool rfe, GemvRegs<CG>& R, uint32_t tg, float* dp) {
  const GemvPlan g = gemv_plan<FMT, CG>(K, npairs, wave_id());
  EpiState st{-__builtin_inff(), 0x7fffffff};
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, static_cast<uint32_t>(2 * npairs) * g.RB);
  const __amdgpu_buffer_rsrc_t gsr = gscale_rsrc<FMT>(Sc, g, npairs);
  const float* xlane = xs + __lane_id() * 4;
  for (int base = g.pa; base < g.pb; base += kSeg) {
    const int np = min(kSeg, g.pb - base);
    if (base != g.pa) gemv_segment_start<FMT, EPI, CG>(p, rs, gsr, Sc, g, base, np, rfe, true, R);
    const int items = (np * g.cpp + CG - 1) / CG;
    Cursor ci{0, 0}, cc{0, 0};
    for (int s = 0; s < 2 * CG; ++s) ci.advance(g.cpp);
    float acc0 = 0.f, acc1 = 0.f;
    XSlot<FMT> xn;
    load_x<FMT>(xlane, xn);  // slot 0 of the segment is chunk 0
    for (int it = 0; it < items; it += 2) {
      gemv_compute<FMT, EPI, CG>(p, g, base, np, layer, xlane, R.a0, R.a1, R.sa, R.wA, R.wB, cc, acc0, acc1, tg, st,
                                 xn, dp, rs, gsr, ci);
      if constexpr (!kSlotRefill<FMT>) gemv_issue<FMT, CG>(rs, gsr, g, base, np, ci, R.a0, R.a1, R.sa);
      if (!kSkipZeroItem<FMT> || it + 1 < items) {  // uniform
        gemv_compute<FMT, EPI, CG>(p, g, base, np, layer, xlane, R.b0, R.b1, R.sb, R.wA, R.wB, cc, acc0, acc1, tg,
                                   st, xn, dp, rs, gsr, ci);
        if constexpr (!kSlotRefill<FMT>) gemv_issue<FMT, CG>(rs, gsr, g, base, np, ci, R.b0, R.b1, R.sb);
      }
    }
  }
  return st;
}

// ------------------------------------------------------------------------------------------
// split-KV GQA attention
// ------------------------------------------------------------------------------------------

// A unit (kv head g, split j) covers positions [t0, t1) in tiles of kAttnTile = 16 positions;
// wave w takes tiles w, w + 8, w + 16, ... For a tile, a wave forms the transposed scores of the
// G heads with bf16 matrix-core products (S^T = K Q^T: q, in base-2 units, split into a bf16 high
// and low part, so it keeps 16 significant bits; K is bf16), updates each head's online softmax,
// and adds the transposed weighted values O^T += V^T P^T the same way (P split into high and low
// parts, V bf16). Every product is exact in fp32 and the sums are fp32. In the transposed form a
// lane holds one head (its column) at four positions: the head's tile maximum is a reduction over
// the lane's 4 elements and the 4 lanes of that column, the weights P^T are already the B operand
// of the value product, and the rescaling of the head's values stays inside the lane. The waves'
// (max, sum, values) then merge through LDS into the unit's partial.
//
// K and V are loaded in whole position rows (hd / 8 lanes of 16 bytes per row, so one load
// instruction reads 64 / (hd / 8) complete rows) and reach the MFMA operand layouts through a
// per-wave LDS tile: K with plain 16-byte reads, V with the transposing ds_read_b64_tr_b16.
//
// MFMA operand layouts used (v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x16_bf16): lane l
// holds A[l % 16][k] and B[k][l % 16] for the k of its k block (8 (l / 16) .. + 7, or
// 4 (l / 16) .. + 3), and the result D[4 (l / 16) + r][l % 16] in element r.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// One tile's K and V as loaded: register m of lane l holds the 16 bytes at byte (l % (hd / 8)) * 16
// of position row (64 / (hd / 8)) * m + l / (hd / 8) of the tile.
template <int HD>
struct AttnTile {
  i32x4 k[HD / 32], v[HD / 32];
};
template <int HD>
struct AttnRegs {
  AttnTile<HD> a, b;  // two tiles in flight per wave
};

// Running maxima start at a finite floor below every score, so the softmax weights need no
// special case: exp2(-inf - m) and exp2(floor - m) are both 0 for any score m, and a wave that
// has seen no position keeps weight 0 in the merge.
constexpr float kScoreFloor = -1.0e30f;

// LDS of the stage (byte offsets): per wave a K and a V tile [16][2 HD + 32 bytes] and a result
// row per head [GMAX][HD + 4] fp32 (values, max, sum); then (float offset kQ) q of the G heads as
// bf16 high parts [G][HD] and low parts [G][HD], and K/V(pos) [2][HD] bf16. Matches
// attn_lds_bytes.
template <int HD, int GMAX>
struct AttnLds {
  static constexpr int kVStride = 2 * HD + 32;  // padded: the 16 rows of a transposed read spread over the banks
  static constexpr int kRStride = HD + 4;
  static constexpr int kK = 0;
  static constexpr int kV = kK + kWaves * kAttnTile * kVStride;
  static constexpr int kRes = kV + kWaves * kAttnTile * kVStride;
  static constexpr int kQ = (kRes + kWaves * GMAX * kRStride * 4) / 4;
};

// Split-KV plan of this step: block u < nkv * S owns kv head g = u / S and positions
// [j*T, min((j+1)*T, pos+1)) with j = u % S.
struct AttnUnit {
  int g, j, t0, t1, ntiles;
  bool active;
};
template <int HD>
__device__ __forceinline__ AttnUnit attn_unit(const KParams& p) {
  AttnUnit a;
  const int S = p.S > 0 ? p.S : 1;
  const int u = blockIdx.x;
  a.active = u < p.nkv * p.S;
  a.g = u / S;
  a.j = u - a.g * S;
  a.t0 = a.j * p.T;
  a.t1 = min(a.t0 + p.T, p.pos + 1);
  a.ntiles = a.active ? (a.t1 - a.t0 + kAttnTile - 1) / kAttnTile : 0;
  return a;
}

// buffer resource over the [max_ctx][HD] bf16 K (kv = 0) or V (kv = 1) block of (layer, kv head)
template <int HD>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kv_rsrc(const KParams& p, int layer, int kv, int g) {
  const uint16_t* base = p.kv + ((static_cast<size_t>(layer * 2 + kv) * p.nkv + g) * p.max_ctx) * HD;
  return make_rsrc(base, static_cast<uint32_t>(p.max_ctx) * HD * 2);
}

// K/V loads of tile `tile` of the unit; positions past the unit (or tiles past the last) read
// zeros. The current position's slot may still be in flight from another block's QKV stage; the
// unit that holds pos replaces it with the copy that arrived with q.
template <int HD>
__device__ __forceinline__ void attn_tile_load(const AttnUnit& a, __amdgpu_buffer_rsrc_t kr,
                                               __amdgpu_buffer_rsrc_t vr, int tile, AttnTile<HD>& T) {
  const int lane = __lane_id();
  constexpr int LPP = HD / 8, PPI = 64 / LPP;  // lanes per position row, rows per load
#pragma unroll
  for (int m = 0; m < HD / 32; ++m) {
    const int t = a.t0 + tile * kAttnTile + PPI * m + lane / LPP;
    const bool v = tile < a.ntiles && t < a.t1;
    const int voff = v ? t * (HD * 2) + (lane % LPP) * 16 : kOOB;
    T.k[m] = ldbuf(kr, voff, 0);
    T.v[m] = ldbuf(vr, voff, 0);
  }
}

template <int HD, int GMAX>
__device__ __forceinline__ void attention_prefetch(const KParams& p, int layer, AttnRegs<HD>& R) {
  const int wave = wave_id();
  const AttnUnit a = attn_unit<HD>(p);
  const __amdgpu_buffer_rsrc_t kr = kv_rsrc<HD>(p, layer, 0, a.g), vr = kv_rsrc<HD>(p, layer, 1, a.g);
  attn_tile_load<HD>(a, kr, vr, wave, R.a);
  attn_tile_load<HD>(a, kr, vr, wave + kWaves, R.b);
}

template <int HD, int GMAX>
__device__ __forceinline__ void attention_stage(const KParams& p, int layer, float* smem, AttnRegs<HD>& R) {
  using Lds = AttnLds<HD, GMAX>;
  constexpr int NC = HD / 32;  // 32-dim chunks of the score product
  constexpr int NV = HD / 16;  // 16-dim chunks of the value product
  const float NEG_INF = -__builtin_inff();
  const int S = p.S;
  const int G = p.nq / p.nkv;
  const int tid = opaque(threadIdx.x), lane = tid & 63, wave = wave_id();
  const int col = lane & 15, kb = lane >> 4;  // the lane's MFMA column and k block
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
  uint8_t* vt = lds + Lds::kV + wave * kAttnTile * Lds::kVStride;
  uint8_t* kt = lds + Lds::kK + wave * kAttnTile * Lds::kVStride;
  constexpr int LPP = HD / 8, PPI = 64 / LPP;
  float* res = reinterpret_cast<float*>(lds + Lds::kRes);
  const float* qs = smem + Lds::kQ;
  const uint16_t* kvp = reinterpret_cast<const uint16_t*>(qs + G * HD);  // K(pos) [HD], V(pos) [HD]
  const AttnUnit a = attn_unit<HD>(p);
  const int g = a.g, j = a.j;

  if (a.active) {
    // q as the B operand of K Q^T (lane l: head l % 16, dims c * 32 + 8 (l / 16) ..), already in
    // base-2 units and split into bf16 high and low parts by the q poll; heads past G are 0
    const bf16x8_t* qhs = reinterpret_cast<const bf16x8_t*>(qs);
    const bf16x8_t zero8 = __builtin_bit_cast(bf16x8_t, i32x4{0, 0, 0, 0});
    bf16x8_t qh[NC], ql[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qh[c] = col < G ? qhs[(col * HD + c * 32 + kb * 8) / 8] : zero8;
      ql[c] = col < G ? qhs[(G * HD + col * HD + c * 32 + kb * 8) / 8] : zero8;
    }
    // for head col (the lane's column): the running max (uniform over the head's 4 lanes), this
    // lane's share of the running sum (its positions 4 kb .. 4 kb + 3 of every tile), and the
    // values: element r of o[n] is dim n * 16 + 4 kb + r of head col
    float mrun = kScoreFloor, lrun = 0.f;
    f32x4 o[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int t0 = a.t0, t1 = a.t1, ntiles = a.ntiles;
    const __amdgpu_buffer_rsrc_t kr = kv_rsrc<HD>(p, layer, 0, g), vr = kv_rsrc<HD>(p, layer, 1, g);
    const int ipos = (t0 <= p.pos && p.pos < t1) ? (p.pos - t0) / kAttnTile : -1;  // uniform
    const int cpos = (p.pos - t0) % kAttnTile;

    auto process = [&](int tile, AttnTile<HD>& T) {
      const int row = lane / LPP, cb = (lane % LPP) * 16;
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        *reinterpret_cast<i32x4*>(kt + (PPI * m + row) * Lds::kVStride + cb) = T.k[m];
        *reinterpret_cast<i32x4*>(vt + (PPI * m + row) * Lds::kVStride + cb) = T.v[m];
      }
      if (tile == ipos && lane < LPP) {  // K/V(pos) from the hand-off replace the cache's slot
        *reinterpret_cast<i32x4*>(kt + cpos * Lds::kVStride + lane * 16) = *reinterpret_cast<const i32x4*>(kvp + lane * 8);
        *reinterpret_cast<i32x4*>(vt + cpos * Lds::kVStride + lane * 16) =
            *reinterpret_cast<const i32x4*>(kvp + HD + lane * 8);
      }
      // transposed scores: element r of lane l is position 4 kb + r of the tile for head col; the
      // high and low parts of q accumulate apart (two independent chains), then add
      f32x4 sh = f32x4{0.f, 0.f, 0.f, 0.f}, sl = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8_t kc = *reinterpret_cast<const bf16x8_t*>(kt + col * Lds::kVStride + (c * 32 + kb * 8) * 2);
        sh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, qh[c], sh, 0, 0, 0);
        sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, ql[c], sl, 0, 0, 0);
      }
      const int pb = t0 + tile * kAttnTile + 4 * kb;  // the position of element 0
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = pb + r < t1 ? sh[r] + sl[r] : NEG_INF;
      float tmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      tmax = fmaxf(tmax, xor_lane<16>(tmax));  // the head's other k blocks
      tmax = fmaxf(tmax, xor_lane<32>(tmax));
      const float mnew = fmaxf(mrun, tmax);
      const float corr = __builtin_amdgcn_exp2f(mrun - mnew);
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(sv[r] - mnew);
      lrun = __builtin_fmaf(lrun, corr, (pr[0] + pr[1]) + (pr[2] + pr[3]));
      mrun = mnew;
#pragma unroll
      for (int n = 0; n < NV; ++n) o[n] *= corr;
      // P^T as the B operand of V^T P^T (lane l: head col, positions 4 kb ..): the lane's own
      // weights, split into high and low bf16 parts
      s16x4_t ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 hi = static_cast<__bf16>(pr[e]);
        ph[e] = __builtin_bit_cast(short, hi);
        pl[e] = __builtin_bit_cast(short, static_cast<__bf16>(pr[e] - static_cast<float>(hi)));
      }
      // V^T as the A operand (lane l: dim n * 16 + col, positions 4 kb ..) by ds_read_b64_tr_b16:
      // within each group of 16 lanes, lane i receives element i % 4 of the 8 bytes addressed by
      // lanes 4 e + i / 4 (e = 0..3). Lane 4 e + c of k block kb addresses position 4 kb + e, dims
      // n * 16 + 4 c .., so lane i gets V[4 kb + e][n * 16 + i]. A wave's LDS accesses complete in
      // order, so no barrier is needed between the tile writes and these reads.
      const int vrow = (kb * 4 + (col >> 2)) * Lds::kVStride + 8 * (col & 3);
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const s16x4_t av = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vt + vrow + n * 32));
        o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, ph, o[n], 0, 0, 0);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pl, o[n], 0, 0, 0);
      }
    };

    // two tiles in flight; loads past the unit read zeros, so the loop body has no branch
    for (int tile = wave; tile < ntiles; tile += 2 * kWaves) {
      process(tile, R.a);
      attn_tile_load<HD>(a, kr, vr, tile + 2 * kWaves, R.a);
      if (tile + kWaves < ntiles) process(tile + kWaves, R.b);  // uniform
      attn_tile_load<HD>(a, kr, vr, tile + 3 * kWaves, R.b);
    }

    // this wave's result per head: values, max, and the sum over the head's 4 lanes (waves with
    // no tile write max = floor and zeros, which the merge weighs 0)
    float lsum = lrun + xor_lane<16>(lrun);
    lsum += xor_lane<32>(lsum);
    if (col < G) {
      float* rw = res + (wave * GMAX + col) * Lds::kRStride;
#pragma unroll
      for (int n = 0; n < NV; ++n) *reinterpret_cast<f32x4*>(rw + n * 16 + 4 * kb) = o[n];
      if (kb == 0) {
        rw[HD] = mrun;
        rw[HD + 1] = lsum;
      }
    }
  }
  wg_barrier();
  if (!a.active) return;

  // merge of the 8 waves: weights 2^(m_w - M) with M the largest wave max (finite: some wave holds
  // the unit's first position). A partial is the weighted values, M and the weighted sum; a single
  // split writes the normalised output as bf16 pairs.
  const uint32_t tpart = tag_of(p, layer, kTagPart), to_tag = tag_of(p, layer, kTagO);
  if (S == 1) {
    for (int o2 = tid; o2 < G * HD / 2; o2 += kThreads) {
      const int h = (2 * o2) / HD, d = 2 * o2 - h * HD;
      float M = NEG_INF;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, res[(w * GMAX + h) * Lds::kRStride + HD]);
      float A0 = 0.f, A1 = 0.f, Ls = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* rw = res + (w * GMAX + h) * Lds::kRStride;
        const float e = __builtin_amdgcn_exp2f(rw[HD] - M);
        const float2 v = *reinterpret_cast<const float2*>(rw + d);
        A0 = __builtin_fmaf(v.x, e, A0);
        A1 = __builtin_fmaf(v.y, e, A1);
        Ls = __builtin_fmaf(rw[HD + 1], e, Ls);
      }
      const float inv = 1.0f / Ls;
      st_tag(p.to + ((g * G + h) * HD + d) / 2,
             static_cast<uint32_t>(f32_to_bf16(A0 * inv)) | (static_cast<uint32_t>(f32_to_bf16(A1 * inv)) << 16),
             to_tag);
    }
  } else {
    // one output per thread, so a wave stores a run of consecutive words
    for (int oi = tid; oi < G * HD; oi += kThreads) {
      const int h = oi / HD, d = oi - h * HD;
      float M = NEG_INF;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, res[(w * GMAX + h) * Lds::kRStride + HD]);
      float A = 0.f, Ls = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* rw = res + (w * GMAX + h) * Lds::kRStride;
        const float e = __builtin_amdgcn_exp2f(rw[HD] - M);
        A = __builtin_fmaf(rw[d], e, A);
        Ls = __builtin_fmaf(rw[HD + 1], e, Ls);
      }
      uint64_t* dst = p.tpart + (static_cast<size_t>(g * G + h) * p.s_cap + j) * (HD + 2);
      st_tag(dst + d, __float_as_uint(A), tpart);
      if (d == 0) {
        st_tag(dst + HD, __float_as_uint(M), tpart);
        st_tag(dst + HD + 1, __float_as_uint(Ls), tpart);
      }
    }
  }
}

// The blocks of kv head g each merge one slice of the head's G * HD outputs over its S splits
// (log-sum-exp weights) and write it as tagged bf16 pairs. Thread t holds split t % SP of output
// word w0 + t / SP (plus 512 / SP in a second round, run when the slice reaches it); SP = S rounded
// up to a power of two.
template <int HD>
__device__ __forceinline__ bool attention_merge_slice(const KParams& p, int layer) {
  const float NEG_INF = -__builtin_inff();
  const AttnUnit a = attn_unit<HD>(p);
  if (!a.active || p.S == 1) return true;  // a single split wrote the output itself
  const int G = p.nq / p.nkv, S = p.S, g = a.g, j = a.j;
  const int tid = opaque(threadIdx.x);
  const int nw = G * HD / 2;  // output words of the kv head (2 bf16 each)
  const int w0 = nw * j / S, w1 = nw * (j + 1) / S;
  int SP = 1;
  while (SP < S) SP *= 2;
  const int wpr = kThreads / SP;  // words per round
  const int obase = toff(p, p.tpart);
  float av[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  float mv[2] = {NEG_INF, NEG_INF}, lv[2] = {0.f, 0.f};
  const bool ok = poll_block<4>(
      p, 4 * kThreads, tag_of(p, layer, kTagPart),
      [&](int qi) {
        const int bq = qi / kThreads, t = qi - bq * kThreads;
        const int r = bq >> 1, which = bq & 1;
        const int wd = w0 + r * wpr + t / SP, sp = t % SP;
        if (wd >= w1 || sp >= S) return kOOB;
        const int h = wd / (HD / 2), d = 2 * (wd - h * (HD / 2));
        const int rec = (g * G + h) * p.s_cap + sp;
        return obase + (rec * (HD + 2) + (which ? HD : d)) * 8;
      },
      [&](int bq, int, uint32_t x0, uint32_t x1) {
        if (bq & 1) {
          mv[bq >> 1] = __uint_as_float(x0);
          lv[bq >> 1] = __uint_as_float(x1);
        } else {
          av[bq >> 1][0] = __uint_as_float(x0);
          av[bq >> 1][1] = __uint_as_float(x1);
        }
      });
  const uint32_t to_tag = tag_of(p, layer, kTagO);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (w0 + r * wpr >= w1) break;  // uniform: no word of the slice falls in this round
    const int wd = w0 + r * wpr + tid / SP, sp = tid % SP;
    const bool v = wd < w1 && sp < S;
    const float mj = v ? mv[r] : NEG_INF;
    const float M = seg_max(mj, SP);
    const float e = (mj == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(mj - M);  // base-2 maxima
    // the three weighted sums are independent (one pass of reductions); the output is the
    // values' sums over the sums' sum
    const float Ls = seg_sum(v ? lv[r] * e : 0.f, SP);
    const float s0 = seg_sum(v ? av[r][0] * e : 0.f, SP);
    const float s1 = seg_sum(v ? av[r][1] * e : 0.f, SP);
    if (ok && v && sp == 0) {
      const float inv = 1.0f / Ls;
      const int h = wd / (HD / 2), d = 2 * (wd - h * (HD / 2));
      st_tag(p.to + ((g * G + h) * HD + d) / 2,
             static_cast<uint32_t>(f32_to_bf16(s0 * inv)) | (static_cast<uint32_t>(f32_to_bf16(s1 * inv)) << 16),
             to_tag);
    }
  }
  return ok;
}

// ------------------------------------------------------------------------------------------
// the persistent decode kernel
// ------------------------------------------------------------------------------------------
// q of the unit's G heads into the q area as the score product's operands: q times the
// attention scale and log2(e) (base-2 units, so every softmax weight is one exp2), split into a
// bf16 high part [G][HD] and the bf16 of the remainder [G][HD] (each value converted once, by
// the thread that polls it); for the unit that holds pos, K/V(pos) (bf16 pairs of dims i,
// i + HD/2) into the bf16 area after it. Returns false if abandoned.
template <int HD>
__device__ __forceinline__ bool poll_q_kv(const KParams& p, int layer, float* qs) {
  const AttnUnit a = attn_unit<HD>(p);
  if (!a.active) return true;
  constexpr int half = HD / 2;
  const int G = p.nq / p.nkv;
  const bool has_pos = a.t1 == p.pos + 1;
  const int nq4 = G * HD / 2, nkv4 = has_pos ? half / 2 : 0;
  const int oq = toff(p, p.tq) + a.g * G * HD * 8, ok_ = toff(p, p.tkv) + a.g * half * 8,
            ov = toff(p, p.tkv) + (p.nkv + a.g) * half * 8;
  uint16_t* kvp = reinterpret_cast<uint16_t*>(qs + G * HD);
  uint32_t* qpair = reinterpret_cast<uint32_t*>(qs);  // bf16 pairs: high parts, then low parts
  const float qscale = p.attn_scale * 1.4426950408889634f;
  return poll_block<2>(
      p, nq4 + 2 * nkv4, tag_of(p, layer, kTagQKV),
      [&](int qi) {
        return qi < nq4 ? oq + 16 * qi : (qi < nq4 + nkv4 ? ok_ + 16 * (qi - nq4) : ov + 16 * (qi - nq4 - nkv4));
      },
      [&](int, int qi, uint32_t x0, uint32_t x1) {
        if (qi < nq4) {
          const float a = __uint_as_float(x0) * qscale, b = __uint_as_float(x1) * qscale;
          const __bf16 ah = static_cast<__bf16>(a), bh = static_cast<__bf16>(b);
          const __bf16 al = static_cast<__bf16>(a - static_cast<float>(ah));
          const __bf16 bl = static_cast<__bf16>(b - static_cast<float>(bh));
          qpair[qi] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ah)) |
                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, bh)) << 16);
          qpair[G * HD / 2 + qi] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, al)) |
                                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, bl)) << 16);
        } else {
          const int r = qi - nq4;
          const int kvs = r < nkv4 ? 0 : 1;
          const int i = 2 * (r - kvs * nkv4);
          uint16_t* d = kvp + kvs * HD;
          d[i] = static_cast<uint16_t>(x0 & 0xffffu);
          d[i + half] = static_cast<uint16_t>(x0 >> 16);
          d[i + 1] = static_cast<uint16_t>(x1 & 0xffffu);
          d[i + 1 + half] = static_cast<uint16_t>(x1 >> 16);
        }
      });
}

// Greedy next token (argmax of the logits, ties to the lowest index) of a device-resident step.
// Every block reduces its waves' argmax and publishes it as two tagged words (value bits, index);
// block 0 polls all blocks' words and writes the token. Block 0 therefore writes only after every
// block has finished the lm_head, so the output may alias the step's input token.
__device__ __forceinline__ bool argmax_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}
__device__ __forceinline__ bool greedy_token(const KParams& p, const EpiState& st, float* smem, float* red,
                                             int* ired) {
  const int lane = __lane_id(), wave = wave_id();
  const float wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, st.v), 0));
  const int wi = __builtin_amdgcn_readlane(st.i, 0);
  if (lane == 0) {
    red[wave] = wv;
    ired[wave] = wi;
  }
  wg_barrier();
  const uint32_t tag = tag_of(p, p.L, 0);
  if (threadIdx.x == 0) {
    float bv = red[0];
    int bi = ired[0];
    for (int w = 1; w < kWaves; ++w)
      if (argmax_better(red[w], ired[w], bv, bi)) {
        bv = red[w];
        bi = ired[w];
      }
    st_tag(p.targ + 2 * blockIdx.x, __float_as_uint(bv), tag);
    st_tag(p.targ + 2 * blockIdx.x + 1, static_cast<uint32_t>(bi), tag);
  }
  if (blockIdx.x != 0) return true;
  float* av = smem;
  int* ai = reinterpret_cast<int*>(smem + kThreads);
  const int ob = toff(p, p.targ);
  const bool ok = poll_block<1>(p, static_cast<int>(gridDim.x), tag, [&](int qi) { return ob + 16 * qi; },
                                [&](int, int qi, uint32_t v, uint32_t i) {
                                  av[qi] = __uint_as_float(v);
                                  ai[qi] = static_cast<int>(i);
                                });
  wg_barrier();
  if (ok && threadIdx.x < 64) {  // wave 0: a strided pass over the blocks, then a lane tree
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    for (int b = threadIdx.x; b < static_cast<int>(gridDim.x); b += 64)
      if (argmax_better(av[b], ai[b], bv, bi)) {
        bv = av[b];
        bi = ai[b];
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (argmax_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (threadIdx.x == 0) *p.next_token = bi;
  }
  return ok;
}

template <int HD, int FMT, int GMAX, int CG>
__global__ void __launch_bounds__(kThreads, 1) amk_decode_kernel(const KParams p) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ float red[kWaves];
  __shared__ int ired[kWaves];
  __shared__ int abort_flag;
  if (threadIdx.x == 0) abort_flag = 0;
  const unsigned err0 = ldc(p.err);
  __syncthreads();
  if (err0 != 0u) return;
  if (p.token_dev != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
    const int t = *p.token_dev;
    if (t < 0 || t >= p.V) raise_error(p, kErrBadToken);  // the step decodes token 0 and is abandoned
  }
  uint64_t* trace = p.trace ? p.trace + static_cast<size_t>(blockIdx.x) * p.trace_stride : nullptr;
  int ev = 0;
  auto stamp = [&]() {
    if (trace != nullptr && threadIdx.x == 0) trace[ev] = wall_clock64();
    ++ev;
  };
  stamp();
  float* xs = smem;                                  // GEMV input vector (swizzled)
  float* qs = smem + AttnLds<HD, GMAX>::kQ;          // attention: q (bf16 high, low parts), K/V(pos)
  const int H = p.H, L = p.L;
  const int qkv_pairs = (p.nq + 2 * p.nkv) * (HD / 2);
  const int qdim = p.nq * HD;
  GemvRegs<CG> R;
  AttnRegs<HD> AR;
  bool ok = true;
  // end of a hand-off: the next stage's input is in LDS, or every thread leaves
  auto handoff_done = [&]() -> bool {
    if (!ok) abort_flag = 1;
    wg_barrier();
    if (abort_flag != 0) {
      __builtin_amdgcn_s_waitcnt(0);
      return false;
    }
    return true;
  };

  gemv_prefetch<FMT, EPI_QKV, CG>(p, p.w_qkv, p.s_qkv, H, qkv_pairs, false, R);
  rmsnorm_embed_to_lds<FMT>(p, p.norm_in, xs, red, dump_at(p, 0, kDH));
  stamp();
  wg_barrier();
  for (int l = 0; l < L; ++l) {
    if (l > 0) {  // RMSNorm of the residual written by the previous layer's down stage
      ok = norm_from_x<FMT>(p, p.norm_in + static_cast<size_t>(l) * H, tag_of(p, l - 1, kTagXD), xs, red,
                           dump_at(p, l, kDH));
      stamp();
      if (!handoff_done()) return;
    }
    // QKV GEMV -> RoPE; q, K/V(pos) as tagged words, K/V(pos) also into the cache
    gemv_run<FMT, EPI_QKV, CG>(p, p.w_qkv + l * p.w_qkv_ls, p.s_qkv + l * p.s_qkv_ls, H, qkv_pairs, xs, l, false, R,
                           tag_of(p, l, kTagQKV), dump_at(p, l, kDQKV));
    attention_prefetch<HD, GMAX>(p, l, AR);
    wg_barrier();  // every wave is done with xs
    stamp();
    ok = poll_q_kv<HD>(p, l, qs);
    stamp();
    if (!handoff_done()) return;

    // split-KV attention -> the unit's partial; the kv head's blocks merge one slice each
    attention_stage<HD, GMAX>(p, l, smem, AR);
    stamp();
    ok = attention_merge_slice<HD>(p, l);
    stamp();
    gemv_prefetch<FMT, EPI_RESID, CG>(p, p.w_o + l * p.w_o_ls, p.s_o + l * p.s_o_ls, qdim, H / 2, l == 0, R);
    wg_barrier();  // attention is done with LDS
    if (ok) ok = vector_from_words<FMT>(p, p.to, qdim, tag_of(p, l, kTagO), xs, dump_at(p, l, kDO));
    stamp();
    if (!handoff_done()) return;

    // O-projection + residual
    gemv_run<FMT, EPI_RESID, CG>(p, p.w_o + l * p.w_o_ls, p.s_o + l * p.s_o_ls, qdim, H / 2, xs, l, l == 0, R,
                             tag_of(p, l, kTagXO), dump_at(p, l, kDWO));
    gemv_prefetch<FMT, EPI_SWIGLU, CG>(p, p.w_gu + l * p.w_gu_ls, p.s_gu + l * p.s_gu_ls, H, p.F, false, R);
    wg_barrier();
    stamp();
    ok = norm_from_x<FMT>(p, p.norm_post + static_cast<size_t>(l) * H, tag_of(p, l, kTagXO), xs, red,
                         dump_at(p, l, kDH2));
    stamp();
    if (!handoff_done()) return;

    // gate/up GEMV -> SwiGLU
    gemv_run<FMT, EPI_SWIGLU, CG>(p, p.w_gu + l * p.w_gu_ls, p.s_gu + l * p.s_gu_ls, H, p.F, xs, l, false, R,
                              tag_of(p, l, kTagM), dump_at(p, l, kDGU));
    gemv_prefetch<FMT, EPI_RESID, CG>(p, p.w_d + l * p.w_d_ls, p.s_d + l * p.s_d_ls, p.F, H / 2, false, R);
    wg_barrier();
    stamp();
    ok = vector_from_words16<FMT>(p, reinterpret_cast<const uint32_t*>(p.tm), p.F, tag_of(p, l, kTagM), xs);
    stamp();
    if (!handoff_done()) return;

    // down GEMV + residual
    gemv_run<FMT, EPI_RESID, CG>(p, p.w_d + l * p.w_d_ls, p.s_d + l * p.s_d_ls, p.F, H / 2, xs, l, false, R,
                             tag_of(p, l, kTagXD), dump_at(p, l, kDWD));
    if (l + 1 < L)
      gemv_prefetch<FMT, EPI_QKV, CG>(p, p.w_qkv + (l + 1) * p.w_qkv_ls, p.s_qkv + (l + 1) * p.s_qkv_ls, H, qkv_pairs,
                                  false, R);
    else if (FMT != 0 && p.lm_fmt == 0)  // quantized projections, bf16 lm_head
      gemv_prefetch<0, EPI_LOGITS, CG>(p, p.w_lm, p.s_lm, H, p.V / 2, false, R);
    else
      gemv_prefetch<FMT, EPI_LOGITS, CG>(p, p.w_lm, p.s_lm, H, p.V / 2, false, R);
    wg_barrier();
    stamp();
  }
  // final RMSNorm -> lm_head (in the lm_head's own storage format, which sets the LDS layout)
  const bool head16 = FMT != 0 && p.lm_fmt == 0;
  if (head16) ok = norm_from_x<0>(p, p.norm_final, tag_of(p, L - 1, kTagXD), xs, red, dump_at(p, L, kDH));
  else ok = norm_from_x<FMT>(p, p.norm_final, tag_of(p, L - 1, kTagXD), xs, red, dump_at(p, L, kDH));
  stamp();
  if (!handoff_done()) return;
  const EpiState st = head16 ? gemv_run<0, EPI_LOGITS, CG>(p, p.w_lm, p.s_lm, H, p.V / 2, xs, L, false, R, 0u, nullptr)
                             : gemv_run<FMT, EPI_LOGITS, CG>(p, p.w_lm, p.s_lm, H, p.V / 2, xs, L, false, R, 0u, nullptr);
  wg_barrier();
  stamp();
  if (p.next_token != nullptr) greedy_token(p, st, smem, red, ired);
}

template __global__ void amk_decode_kernel<64, 0, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 1, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 0, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 1, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 0, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 1, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 0, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 1, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 2, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 2, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 2, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 2, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 3, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 3, 4, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 3, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<128, 3, 8, 1>(const KParams);
template __global__ void amk_decode_kernel<64, 0, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<64, 1, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 0, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 1, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<64, 0, 8, 2>(const KParams);
template __global__ void amk_decode_kernel<64, 1, 8, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 0, 8, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 1, 8, 2>(const KParams);
template __global__ void amk_decode_kernel<64, 2, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 2, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<64, 2, 8, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 2, 8, 2>(const KParams);
template __global__ void amk_decode_kernel<64, 3, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 3, 4, 2>(const KParams);
template __global__ void amk_decode_kernel<64, 3, 8, 2>(const KParams);
template __global__ void amk_decode_kernel<128, 3, 8, 2>(const KParams);

// Zeroes n 32-bit words (a model's scratch: error flag and exchange words) before the model is
// used again after a failure; a kernel rather than a memset so that it is safe in graph capture.
__global__ void amk_clear_kernel(uint32_t* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

}  // namespace amk

// host-visible handles of the kernel instantiations (defined in this translation unit)
// fmt: 0 bf16, 1 int8, 2 int4 (row scales), 3 int4 (group scales) projection weights
extern "C" __attribute__((visibility("hidden"))) const void* amk_kernel_handle(int head_dim, int fmt, int gmax,
                                                                                int cg) {
  using namespace amk;
#define AMK_K(HD, F, G, C) (const void*)&amk_decode_kernel<HD, F, G, C>
#define AMK_K4(HD, G, C) {AMK_K(HD, 0, G, C), AMK_K(HD, 1, G, C), AMK_K(HD, 2, G, C), AMK_K(HD, 3, G, C)}
  const void* const t[2][2][2][4] = {{{AMK_K4(64, 4, 1), AMK_K4(64, 8, 1)}, {AMK_K4(128, 4, 1), AMK_K4(128, 8, 1)}},
                                     {{AMK_K4(64, 4, 2), AMK_K4(64, 8, 2)}, {AMK_K4(128, 4, 2), AMK_K4(128, 8, 2)}}};
#undef AMK_K4
#undef AMK_K
  if ((head_dim != 64 && head_dim != 128) || (gmax != 4 && gmax != 8) || fmt < 0 || fmt > 3 || (cg != 1 && cg != 2))
    return nullptr;
  return t[cg - 1][head_dim == 128][gmax == 8][fmt];
}

extern "C" __attribute__((visibility("hidden"))) const void* amk_clear_kernel_handle() {
  return (const void*)&amk::amk_clear_kernel;
}

// Exchange words and error flag of amk_decode_step_noalloc: one array per GPU, held until the
// process ends, shared by every such call on that GPU. Host code never uses the array's name as
// an address (in host code it is a stand-in, not device memory): amk_static_scratch looks the
// device address up with hipGetSymbolAddress, once per device, and callers pass that pointer on.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Device address and size of `scratch` on the current device (looked up on the first call for a
// device, then cached). Returns hipSuccess or the lookup's error.
extern "C" __attribute__((visibility("hidden"))) hipError_t amk_static_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}
