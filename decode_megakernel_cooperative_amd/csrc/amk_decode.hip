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
//    items into registers; attention issues its K/V loads before q arrives.
//  * Activations: the GEMV input vector of a stage (RMSNorm output, attention output, SwiGLU
//    output) is staged in LDS as fp32 holding bf16-rounded values (as bf16 for int4 weights),
//    in a swizzled layout so the 16-byte LDS reads of a lane per weight chunk are bank-conflict
//    free.
//  * W8A16: int8 codes convert with one v_cvt_f32_i32 (SDWA byte select, sign extend) per
//    weight and feed an fp32 FMA; the per-row fp32 scale multiplies the wave-reduced sum.
//    W4A16: sign-magnitude codes, eight per dword, laid out so that two masks turn a dword into
//    eight fp8 (e4m3) subnormals of value q * 2^-9; gfx950's fp8-to-bf16 pair conversion and
//    bf16 pair dot products then take two weights per instruction (1.375 VALU per weight).
//  * Row pairs: rows are packed at load time so that rows i and i + hd/2 of one head (a RoPE
//    pair) and rows n of gate and up (a SwiGLU pair) are adjacent; one wave computes both rows
//    of a pair, so the RoPE / SwiGLU / residual epilogues need no cross-wave exchange.
//  * Attention: split-KV over (kv head, position range) units, one unit per block. The G query
//    heads of a kv head share every K/V load. Each 16-lane row (hd 128) or 8-lane row (hd 64)
//    scores one position per step with DPP row reductions and keeps an online softmax in base-2
//    units; all rows of the block then merge in LDS (one exp2 weight per row and head) into one
//    tagged partial (values, max, sum) per unit; then every block of the kv head merges one
//    slice of the head's outputs over all splits by log-sum-exp weights (DPP segmented
//    reductions) and writes it as tagged bf16 pairs. A context short enough for one split per
//    kv head skips that second merge: the unit writes the normalised output itself.
//  * No MFMA: batch-1 decode is a matrix-vector product, far below the MFMA ridge point.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "amk_kparams.h"

#ifndef AMK_FINE_TRACE
#define AMK_FINE_TRACE 0  // 1: extra trace stamps inside every layer (stage-internal timing)
#endif
#ifndef AMK_KCG
#define AMK_KCG 2         // 1 KB chunk slots per GEMV item (per row)
#endif
#ifndef AMK_STRIDED
#define AMK_STRIDED 2     // how a GEMV stage's row pairs map to the NW waves of the grid:
                          // 2: wave w of block b is stream s = w * blocks + b and takes pairs s,
                          //    s + NW, ...: at any moment the grid streams one sliding window of
                          //    the matrix, consecutive pairs going to consecutive blocks (and so to
                          //    different XCDs); 1: the same with s = b * 8 + w; 0: a contiguous
                          //    range of pairs per wave
#endif
#ifndef AMK_PREFETCH_ITEMS
#define AMK_PREFETCH_ITEMS 2  // GEMV items issued before the barrier in front of a stage (1 or 2)
#endif

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
__device__ __forceinline__ void ldc2(const float* p, float& a, float& b) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  a = __uint_as_float(static_cast<uint32_t>(v));
  b = __uint_as_float(static_cast<uint32_t>(v >> 32));
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc16(uint16_t* p, uint16_t v) {
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
// Agent-coherent (sc1) 16-byte buffer load, for vectors written by other blocks in this launch.
constexpr int kBufCacheSC1 = 16;
__device__ __forceinline__ f32x4 ldbuf_c(__amdgpu_buffer_rsrc_t rs, int voff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kBufCacheSC1);
  return f32x4{__int_as_float(v.x), __int_as_float(v.y), __int_as_float(v.z), __int_as_float(v.w)};
}


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
// grid barrier (the library's barrier microbenchmark only: the decode kernel synchronises by
// tagged hand-offs, whose cost this measures a lower bound against)
// ------------------------------------------------------------------------------------------
struct GridBarrier {
  unsigned* ctr;
  unsigned base;   // barriers completed by earlier launches
  unsigned n;      // barriers completed in this launch
  uint64_t limit;
  unsigned* err;
  uint64_t* trace; // optional per-block timestamps (entry, then arrival/exit of every barrier)
  int ev;

  __device__ __forceinline__ void stamp() {
    if (trace != nullptr && threadIdx.x == 0) trace[ev] = wall_clock64();
    ++ev;
  }

  // Arrival: waits for this block's stores (s_waitcnt 0 per wave, then the workgroup
  // barrier) and adds one to the block's arrival counter. Loads issued after arrive() and
  // before wait() overlap the wait (the next stage's weights are prefetched there).
  __device__ __forceinline__ void arrive() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stamp();
    ++n;
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(ctr + (blockIdx.x & (kBarrierCtrs - 1)) * kCtrStride, 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Wait until every block has arrived n times. Returns false if the step must be abandoned
  // (timeout here or an error raised by another block).
  __device__ __forceinline__ bool wait(int* abort_lds) {
    const unsigned tid = threadIdx.x;
    if (tid < kBarrierCtrs && tid < gridDim.x) {
      const unsigned per = (gridDim.x - tid + kBarrierCtrs - 1) / kBarrierCtrs;
      const unsigned target = (base + n) * per;
      const uint64_t t0 = wall_clock64();
      unsigned it = 0;
      bool bad = false;
      while (static_cast<int>(ldc(ctr + tid * kCtrStride) - target) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if (((++it) & 31u) == 0) {
          if (ldc(err) != 0u) { bad = true; break; }
          if (wall_clock64() - t0 > limit) { stc(err, kErrTimeout); bad = true; break; }
        }
      }
      if (bad) *abort_lds = 1;
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    stamp();
    return *abort_lds == 0;
  }

  __device__ __forceinline__ bool sync(int* abort_lds) {
    arrive();
    return wait(abort_lds);
  }
};

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
  if constexpr (FMT == 2) reinterpret_cast<uint16_t*>(xs)[swz16(e)] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
  else if constexpr (FMT == 0) reinterpret_cast<uint16_t*>(xs)[e] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
  else xs[swz<FMT>(e)] = v;
}
template <int FMT>
__device__ __forceinline__ void put_x4(float* xs, int e, f32x4 v) {
  if constexpr (FMT != 1) {
    const uint32_t lo = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
    const uint32_t hi = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xffff0000u);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(xs) + (FMT == 2 ? swz16(e) : e)) = uint2{lo, hi};
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

// stage-internal stamps (AMK_FINE_TRACE builds only): slot k of layer l after the stage stamps
__device__ __forceinline__ void fstamp(const KParams& p, int l, int k) {
  if (AMK_FINE_TRACE && p.trace != nullptr && threadIdx.x == 0)
    p.trace[static_cast<size_t>(blockIdx.x) * p.trace_stride + 3 + 11 * p.L + l * 16 + k] = wall_clock64();
}
__device__ __forceinline__ int toff(const KParams& p, const uint64_t* buf) {
  return static_cast<int>(reinterpret_cast<const uint8_t*>(buf) - reinterpret_cast<const uint8_t*>(p.tagged));
}

// Bound of a hand-off wait, checked after its reload number `it`: false once the step must be
// abandoned. The error word is read every 16 reloads (an error raised elsewhere keeps its code);
// the clock also after the second reload, so that a spin limit of one tick ends the first poll
// that waits at all.
__device__ __forceinline__ bool wait_ok(const KParams& p, unsigned it, uint64_t t_start) {
  const bool round16 = (it & 15u) == 0;
  if (round16 && ldc(p.err) != 0u) return false;
  if ((round16 || it == 2) && wall_clock64() - t_start > p.spin_limit) {
    stc(p.err, kErrTimeout);
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
        __builtin_amdgcn_s_sleep(2);
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
        __builtin_amdgcn_s_sleep(2);
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

// xs <- bf16((x * rsqrt(mean(x^2) + eps)) * w) for the first layer, x = the bf16 embedding row,
// zero padded to whole weight chunks.
template <int FMT>
__device__ __forceinline__ void rmsnorm_embed_to_lds(const KParams& p, const float* __restrict__ w, float* xs,
                                                     float* red) {
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
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) {
    const int e = 2 * (b * kThreads + tid);
    if (e < H) {
      put_x<FMT>(xs, e, round_bf16((xv[b].x * r) * wv[b].x));
      put_x<FMT>(xs, e + 1, round_bf16((xv[b].y * r) * wv[b].y));
    }
  }
  for (int e = H + tid; e < padded<FMT>(H); e += kThreads) put_x<FMT>(xs, e, 0.f);
}

// xs <- RMSNorm of the residual x polled from its tagged words (tag `tag`), zero padded. The
// weights are loaded with the poll, in the same round trip. Returns false if abandoned.
template <int FMT>
__device__ __forceinline__ bool norm_from_x(const KParams& p, const float* __restrict__ w, uint32_t tag, float* xs,
                                            float* red) {
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
#pragma unroll
  for (int b = 0; b < kNormVB; ++b) {
    const int e = 2 * (b * kThreads + tid);
    if (e < H) {
      put_x<FMT>(xs, e, round_bf16((xv[b].x * r) * wv[b].x));
      put_x<FMT>(xs, e + 1, round_bf16((xv[b].y * r) * wv[b].y));
    }
  }
  for (int e = H + tid; e < padded<FMT>(H); e += kThreads) put_x<FMT>(xs, e, 0.f);
  return ok;
}

// xs <- a bf16 vector of K elements polled from its tagged words (two bf16 per word), zero
// padded. Four consecutive elements land in one float4 of the swizzled layout.
template <int FMT>
__device__ __forceinline__ bool vector_from_words(const KParams& p, const uint64_t* src, int K, uint32_t tag,
                                                  float* xs) {
  const int ob = toff(p, src);
  const bool ok = poll_block<8>(p, K / 4, tag, [&](int qi) { return ob + 16 * qi; },
                                [&](int, int qi, uint32_t a, uint32_t c) {
                                  put_x4<FMT>(xs, 4 * qi,
                                              f32x4{bf16_to_f32(a & 0xffffu), bf16_to_f32(a >> 16),
                                                    bf16_to_f32(c & 0xffffu), bf16_to_f32(c >> 16)});
                                });
  for (int e = K + opaque(threadIdx.x); e < padded<FMT>(K); e += kThreads) put_x<FMT>(xs, e, 0.f);
  return ok;
}

// ------------------------------------------------------------------------------------------
// GEMV stage over row pairs
// ------------------------------------------------------------------------------------------
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

constexpr int kCG = AMK_KCG;  // chunk slots per item: 2 rows x kCG x 16 B dwordx4 loads per lane
constexpr int kSeg = 32; // pairs per operand window (lane j holds the operand of packed row 2*base + j)

// Registers that carry a GEMV stage's operand window and first two items across the wait for
// the stage's input vector.
struct GemvRegs {
  i32x4 a0[kCG], a1[kCG], b0[kCG], b1[kCG];
  float wA, wB;
};

// How one stage is split. A wave owns the contiguous pair range [pa, pb), processed in
// segments of at most kSeg pairs. Inside a segment, pair k's chunks occupy slots
// [k*cpp, k*cpp + nch) of a padded slot space (cpp = chunks per pair rounded so that items of
// kCG slots never straddle a pair unevenly); an item is kCG consecutive slots. Slots past a
// row's end or past the segment read zeros, so every item issues the same 8 loads.
struct GemvPlan {
  int RB;   // bytes per row
  int nch;  // 1 KB chunks per row
  int cpp;  // padded slots per pair: 1, 2 or 4 when nch <= kCG, else a multiple of kCG
  int pa, pb;     // the wave's pairs, as local indices k in [pa, pb)
  int st0, sst;   // local index k is pair st0 + k * sst of the matrix
};
__device__ __forceinline__ int pidx(const GemvPlan& g, int k) { return g.st0 + k * g.sst; }

// Pairs are split over the waves in units of `unit` pairs (2 for gate/up, so a wave's SwiGLU
// outputs fill whole two-value exchange words).
template <int FMT>
__device__ __forceinline__ GemvPlan gemv_plan(int K, int npairs, int wave, int unit) {
  GemvPlan g;
  g.RB = K * Fmt<FMT>::BITS / 8;
  g.nch = (g.RB + 1023) >> 10;
  g.cpp = g.nch <= 1 ? 1 : g.nch <= 2 ? 2 : g.nch <= kCG ? kCG : (g.nch + kCG - 1) / kCG * kCG;
  const int NW = gridDim.x * kWaves, gw = blockIdx.x * kWaves + wave;
  if (AMK_STRIDED) {
    const int sw = AMK_STRIDED == 2 ? wave * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x) : gw;
    g.pa = 0;
    g.pb = sw < npairs ? (npairs - sw + NW - 1) / NW : 0;
    g.st0 = sw;
    g.sst = NW;
    (void)unit;
    return g;
  }
  const int nu = npairs / unit;
  g.pa = unit * static_cast<int>((static_cast<int64_t>(nu) * gw) / NW);
  g.pb = unit * static_cast<int>((static_cast<int64_t>(nu) * (gw + 1)) / NW);
  g.st0 = 0;
  g.sst = 1;
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
__device__ __forceinline__ void chunk_fma(const i32x4 w0, const i32x4 w1, const XSlot<FMT>& xs, float& a0,
                                          float& a1) {
  if constexpr (FMT == 2) {
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
// window's pair j / 2: A = the row scale of int8 / int4 weights, B = residual input (EPI_RESID) or RoPE cos
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
    if (FMT != 0) A = Sc[row];  // int4: the epilogue applies the factor 2^9
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
// cross blocks are written as tagged words (tag tg); a SwiGLU output is one 32-bit word.
template <int EPI>
__device__ __forceinline__ void epilogue(const KParams& p, int layer, int pr, float y0, float y1, float b0, float b1,
                                         uint32_t tg, EpiState& st) {
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
    st_tag(p.tx + 2 * pr, __float_as_uint(b0 + y0), tg);
    st_tag(p.tx + 2 * pr + 1, __float_as_uint(b1 + y1), tg);
  } else if (EPI == EPI_SWIGLU) {
    const float m = (y0 / (1.0f + expf(-y0))) * y1;
    st_tag16(reinterpret_cast<uint32_t*>(p.tm) + pr, f32_to_bf16(m), tg);
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

// Issues the 8 loads of the item that starts at cursor c (advancing c by kCG slots). np = pairs
// in the segment, base = first pair of the segment.
__device__ __forceinline__ void gemv_issue(__amdgpu_buffer_rsrc_t rs, const GemvPlan& g, int base, int np,
                                           Cursor& c, i32x4 (&r0)[kCG], i32x4 (&r1)[kCG]) {
  const int lane = __lane_id();
#pragma unroll
  for (int s = 0; s < kCG; ++s) {
    const bool v = c.ch < g.nch && c.k < np;
    const int off = c.ch * 1024 + lane * 16;
    const int voff = (v && off < g.RB) ? off : kOOB;
    // uniform by construction; readfirstlane keeps the compiler from moving it to VGPRs
    const int soff = __builtin_amdgcn_readfirstlane(v ? 2 * pidx(g, base + c.k) * g.RB : 0);
    r0[s] = ldbuf(rs, voff, soff);
    r1[s] = ldbuf(rs, voff, soff + g.RB);
    c.advance(g.cpp);
  }
}

// Accumulates the item at cursor c into (acc0, acc1); when a slot completes a pair, reduces it
// over the wave and lane 0 runs the epilogue. Slots that read zeros add nothing.
// bf16 and int4 slots issue their LDS reads one slot ahead of their FMAs: xn holds the
// activations of the slot at cursor c on entry and of the slot after this item's last one on
// return. int8 slots read their own activations first: reading one slot ahead measured 2%
// slower per token for int8 weights and 1% faster for bf16 and int4.
template <int FMT, int EPI>
__device__ __forceinline__ void gemv_compute(const KParams& p, const GemvPlan& g, int base, int np, int layer,
                                             const float* xlane, const i32x4 (&r0)[kCG], const i32x4 (&r1)[kCG],
                                             float wA, float wB, Cursor& c, float& acc0, float& acc1, uint32_t tg,
                                             EpiState& st, XSlot<FMT>& xn) {
  constexpr int XCS = Fmt<FMT>::XCS;
#pragma unroll
  for (int s = 0; s < kCG; ++s) {
    XSlot<FMT> xc;
    if constexpr (FMT == 1) {
      load_x<FMT>(xlane + min(c.ch, g.nch - 1) * XCS, xc);
    } else {
      xc = xn;
      Cursor cn = c;
      cn.advance(g.cpp);
      load_x<FMT>(xlane + min(cn.ch, g.nch - 1) * XCS, xn);
    }
    // keep the scheduler from hoisting the conversions of all slots at once (register spills)
    __builtin_amdgcn_sched_barrier(0);
    chunk_fma<FMT>(r0[s], r1[s], xc, acc0, acc1);
    __builtin_amdgcn_sched_barrier(0);
    if (c.ch == g.nch - 1 && c.k < np) {
      float y0 = wave_sum(acc0), y1 = wave_sum(acc1);
      acc0 = acc1 = 0.f;
      const int j = 2 * c.k;
      if (FMT != 0) {
        y0 *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wA), j));
        y1 *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wA), j + 1));
      }
      if (FMT == 2) {  // the int4 products arrived as q * 2^-9 (exact)
        y0 *= 512.f;
        y1 *= 512.f;
      }
      const float b0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wB), j));
      const float b1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wB), j + 1));
      if (__lane_id() == 0) epilogue<EPI>(p, layer, pidx(g, base + c.k), y0, y1, b0, b1, tg, st);
    }
    c.advance(g.cpp);
  }
}

// Loads the operand window of the segment at `base` and issues the segment's first two items.
template <int FMT, int EPI>
__device__ __forceinline__ void gemv_segment_start(const KParams& p, __amdgpu_buffer_rsrc_t rs,
                                                   const float* __restrict__ Sc, const GemvPlan& g, int base,
                                                   int np, bool rfe, bool two, GemvRegs& R) {
  load_window<FMT, EPI>(p, Sc, g, base, rfe, R.wA, R.wB);
  Cursor c{0, 0};
  gemv_issue(rs, g, base, np, c, R.a0, R.a1);
  if (two) gemv_issue(rs, g, base, np, c, R.b0, R.b1);
}

// Issues the stage's operand window and first two items; called before the block polls the
// stage's input vector, so HBM keeps streaming while the producers of that vector finish.
template <int FMT, int EPI>
__device__ __forceinline__ void gemv_prefetch(const KParams& p, const uint8_t* __restrict__ W,
                                              const float* __restrict__ Sc, int K, int npairs, bool rfe,
                                              GemvRegs& R) {
  const GemvPlan g = gemv_plan<FMT>(K, npairs, wave_id(), 1);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, static_cast<uint32_t>(2 * npairs) * g.RB);
  gemv_segment_start<FMT, EPI>(p, rs, Sc, g, g.pa, min(kSeg, g.pb - g.pa), rfe, AMK_PREFETCH_ITEMS > 1, R);
}

// Runs the stage. Items alternate between the two register buffers, each refilled two items
// ahead of its use; the loop body is branch free apart from the per-pair epilogue, so loads
// stay in flight across iterations. Returns the epilogue state of lane 0 (the wave's argmax for
// the logits stage).
template <int FMT, int EPI>
__device__ __forceinline__ EpiState gemv_run(const KParams& p, const uint8_t* __restrict__ W,
                                         const float* __restrict__ Sc, int K, int npairs, const float* xs,
                                         int layer, bool rfe, GemvRegs& R, uint32_t tg) {
  const GemvPlan g = gemv_plan<FMT>(K, npairs, wave_id(), 1);
  EpiState st{-__builtin_inff(), 0x7fffffff};
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, static_cast<uint32_t>(2 * npairs) * g.RB);
  const float* xlane = xs + __lane_id() * 4;
  for (int base = g.pa; base < g.pb; base += kSeg) {
    const int np = min(kSeg, g.pb - base);
    if (base != g.pa) gemv_segment_start<FMT, EPI>(p, rs, Sc, g, base, np, rfe, true, R);
    const int items = (np * g.cpp + kCG - 1) / kCG;
    Cursor ci{0, 0}, cc{0, 0};
    for (int s = 0; s < kCG; ++s) ci.advance(g.cpp);
    if (AMK_PREFETCH_ITEMS > 1 || base != g.pa) {
      for (int s = 0; s < kCG; ++s) ci.advance(g.cpp);
    } else {
      gemv_issue(rs, g, base, np, ci, R.b0, R.b1);  // second item was not prefetched
    }
    float acc0 = 0.f, acc1 = 0.f;
    XSlot<FMT> xn;
    load_x<FMT>(xlane, xn);  // slot 0 of the segment is chunk 0
    if (EPI == EPI_QKV) fstamp(p, layer, 12);
    for (int it = 0; it < items; it += 2) {
      gemv_compute<FMT, EPI>(p, g, base, np, layer, xlane, R.a0, R.a1, R.wA, R.wB, cc, acc0, acc1, tg, st, xn);
      if (EPI == EPI_QKV && it == 0) fstamp(p, layer, 13);
      gemv_issue(rs, g, base, np, ci, R.a0, R.a1);
      if (EPI == EPI_QKV && it == 0) fstamp(p, layer, 14);
      gemv_compute<FMT, EPI>(p, g, base, np, layer, xlane, R.b0, R.b1, R.wA, R.wB, cc, acc0, acc1, tg, st, xn);
      if (EPI == EPI_QKV && it == 0) fstamp(p, layer, 15);
      gemv_issue(rs, g, base, np, ci, R.b0, R.b1);
    }
  }
  return st;
}

// ------------------------------------------------------------------------------------------
// split-KV GQA attention
// ------------------------------------------------------------------------------------------

template <int GMAX>
struct AttnRegs {
  static constexpr int U = GMAX > 4 ? 2 : 4;  // position groups per wave per pipeline step
  i32x4 ka[U], va[U], kb[U], vb[U];           // two pipeline buffers
};

// Running maxima start at a finite floor below every score, so the softmax weights need no
// special case: exp2(-inf - m) and exp2(floor - m) are both 0 for any score m, and a row that has
// seen no position keeps weight 0.
constexpr float kScoreFloor = -1.0e30f;

// LDS of the attention stage, in floats: every row's softmax state (a row is the LPP lanes that
// hold one position of a wave load: [R][GMAX][RS] = values, running max, running sum, merge
// weight, pad), then each head's block max and sum, then q of the G heads and K/V(pos).
template <int HD, int GMAX>
struct AttnLds {
  static constexpr int PPW = 64 / (HD / 8);
  static constexpr int R = kWaves * PPW;
  static constexpr int RS = HD + 4;
  static constexpr int kHeads = R * GMAX * RS;
  static constexpr int kQ = kHeads + 4 * GMAX;
};

// Split-KV plan of this step: block u < nkv * S owns kv head g = u / S and positions
// [j*T, min((j+1)*T, pos+1)) with j = u % S.
struct AttnUnit {
  int g, j, t0, t1, ngroups;
  bool active;
};
template <int HD>
__device__ __forceinline__ AttnUnit attn_unit(const KParams& p) {
  constexpr int PPW = 64 / (HD / 8);
  AttnUnit a;
  const int S = p.S > 0 ? p.S : 1;
  const int u = blockIdx.x;
  a.active = u < p.nkv * p.S;
  a.g = u / S;
  a.j = u - a.g * S;
  a.t0 = a.j * p.T;
  a.t1 = min(a.t0 + p.T, p.pos + 1);
  a.ngroups = a.active ? (a.t1 - a.t0 + PPW - 1) / PPW : 0;
  return a;
}

// K/V loads of one pipeline step of a wave: U groups of PPW positions, one position per row
// of LPP lanes. With skip_pos, the current position (written by this step's QKV stage,
// possibly still in flight) is left out: the prefetch issued before q arrives uses that.
template <int HD, int U>
__device__ __forceinline__ void attn_load(const KParams& p, const AttnUnit& a, __amdgpu_buffer_rsrc_t kr_rs,
                                          __amdgpu_buffer_rsrc_t vr_rs, int gbase, bool skip_pos, i32x4 (&kr)[U],
                                          i32x4 (&vr)[U]) {
  constexpr int LPP = HD / 8, PPW = 64 / LPP;
  const int lane = __lane_id();
  const int ri = lane / LPP, lo = (lane % LPP) * 16;
#pragma unroll
  for (int uu = 0; uu < U; ++uu) {
    const int gg = gbase + uu * kWaves;
    const int t = a.t0 + gg * PPW + ri;
    const bool v = gg < a.ngroups && t < a.t1 && !(skip_pos && t == p.pos);
    const int voff = v ? t * (HD * 2) + lo : kOOB;
    kr[uu] = ldbuf(kr_rs, voff, 0);
    vr[uu] = ldbuf(vr_rs, voff, 0);
  }
}

// buffer resource over the [max_ctx][HD] bf16 K (kv = 0) or V (kv = 1) block of (layer, kv head)
template <int HD>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kv_rsrc(const KParams& p, int layer, int kv, int g) {
  const uint16_t* base = p.kv + ((static_cast<size_t>(layer * 2 + kv) * p.nkv + g) * p.max_ctx) * HD;
  return make_rsrc(base, static_cast<uint32_t>(p.max_ctx) * HD * 2);
}

template <int HD, int GMAX>
__device__ __forceinline__ void attention_prefetch(const KParams& p, int layer, AttnRegs<GMAX>& R) {
  constexpr int U = AttnRegs<GMAX>::U;
  const int wave = wave_id();
  const AttnUnit a = attn_unit<HD>(p);
  const __amdgpu_buffer_rsrc_t kr = kv_rsrc<HD>(p, layer, 0, a.g), vr = kv_rsrc<HD>(p, layer, 1, a.g);
  // all lanes load (out-of-range groups read zeros), so R is written on every path
  attn_load<HD, U>(p, a, kr, vr, wave, true, R.ka, R.va);
  attn_load<HD, U>(p, a, kr, vr, wave + kWaves * U, true, R.kb, R.vb);
}

template <int HD, int GMAX>
__device__ __forceinline__ void attention_stage(const KParams& p, int layer, float* smem, AttnRegs<GMAX>& R) {
  constexpr int kAttnU = AttnRegs<GMAX>::U;
  constexpr int LPP = HD / 8;     // lanes per position (8 bf16 = 16 bytes per lane)
  constexpr int PPW = 64 / LPP;   // positions per wave load
  const float NEG_INF = -__builtin_inff();
  const int S = p.S;
  const int G = p.nq / p.nkv;
  const int tid = opaque(threadIdx.x), lane = tid & 63, wave = wave_id();
  const int li = lane % LPP, ri = lane / LPP, d0 = li * 8;
  using Lds = AttnLds<HD, GMAX>;
  constexpr int NR = Lds::R, RS = Lds::RS;
  float* wp = smem;                   // row states [R][GMAX][RS]
  float* hs = smem + Lds::kHeads;     // per head: block max, block sum
  const float* qs = smem + Lds::kQ;   // q of the G heads [G][HD]
  const uint16_t* kvp = reinterpret_cast<const uint16_t*>(qs + G * HD);  // K(pos) [HD], V(pos) [HD]
  const AttnUnit a = attn_unit<HD>(p);
  const int g = a.g, j = a.j;

  if (a.active) {
    const int t0 = a.t0, t1 = a.t1, ngroups = a.ngroups;
    const __amdgpu_buffer_rsrc_t kb = kv_rsrc<HD>(p, layer, 0, g);
    const __amdgpu_buffer_rsrc_t vb = kv_rsrc<HD>(p, layer, 1, g);
    i32x4 (&KA)[kAttnU] = R.ka;
    i32x4 (&VA)[kAttnU] = R.va;
    i32x4 (&KB)[kAttnU] = R.kb;
    i32x4 (&VB)[kAttnU] = R.vb;
    const int step = kWaves * kAttnU;
    // The current position's K/V are written by this step's QKV stage on another block: plain
    // stores that need not be visible here yet. The unit that holds pos received them with q
    // (LDS); whatever the cache load of that slot returned is replaced before use.
    const int gpos = (t0 <= p.pos && p.pos < t1) ? (p.pos - t0) / PPW : -1;  // uniform
    const int rpos = (p.pos - t0) % PPW;
    auto patch_pos = [&](int gbase, i32x4 (&kr)[kAttnU], i32x4 (&vr)[kAttnU]) {
      const int dg = gpos - gbase;
      if (dg >= 0 && dg < kAttnU * kWaves && dg % kWaves == 0) {  // uniform: at most once per unit
        const i32x4 kl = *reinterpret_cast<const i32x4*>(kvp + li * 8);
        const i32x4 vl = *reinterpret_cast<const i32x4*>(kvp + HD + li * 8);
#pragma unroll
        for (int uu = 0; uu < kAttnU; ++uu) {
          const bool here = uu == dg / kWaves && ri == rpos;
          kr[uu] = here ? kl : kr[uu];
          vr[uu] = here ? vl : vr[uu];
        }
      }
    };
    auto load = [&](int gbase, i32x4 (&kr)[kAttnU], i32x4 (&vr)[kAttnU]) {
      attn_load<HD, kAttnU>(p, a, kb, vb, gbase, false, kr, vr);
    };

    fstamp(p, layer, 0);
    // scores are kept in base-2 units (q pre-scaled by log2(e) / sqrt(HD)), so every softmax
    // weight is one exp2
    const float qscale = p.attn_scale * 1.4426950408889634f;
    float qv[GMAX][8];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < G) {
        const float* qp = qs + h * HD + d0;
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[h][i] = qp[i] * qscale;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[h][i] = 0.f;
      }
    }
    float mr[GMAX], lr[GMAX], acc[GMAX][8];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      mr[h] = kScoreFloor;
      lr[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }

    auto compute = [&](int gbase, const i32x4 (&kr)[kAttnU], const i32x4 (&vr)[kAttnU]) {
      float s[kAttnU][GMAX];
#pragma unroll
      for (int uu = 0; uu < kAttnU; ++uu) {
        const int gg = gbase + uu * kWaves;
        const bool valid = gg < ngroups && (t0 + gg * PPW + ri) < t1;
        if (gg >= ngroups) {  // uniform: no position of this group is in the unit
#pragma unroll
          for (int h = 0; h < GMAX; ++h) s[uu][h] = NEG_INF;
          continue;
        }
        float kf[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          kf[2 * d] = bf_lo(kr[uu][d]);
          kf[2 * d + 1] = bf_hi(kr[uu][d]);
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          float dot = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) dot = __builtin_fmaf(qv[h][i], kf[i], dot);
          dot = group_sum<LPP>(dot);
          s[uu][h] = valid ? dot : NEG_INF;
        }
      }
      // online softmax: new running max, rescale, and this step's weights (all zero while a row
      // has seen no position: its max stays -inf and its sums stay 0)
      float pe[kAttnU][GMAX];
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        if (h >= G) continue;
        float mnew = mr[h];
#pragma unroll
        for (int uu = 0; uu < kAttnU; ++uu) mnew = fmaxf(mnew, s[uu][h]);
        const float corr = __builtin_amdgcn_exp2f(mr[h] - mnew);
        lr[h] *= corr;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] *= corr;
#pragma unroll
        for (int uu = 0; uu < kAttnU; ++uu) {
          pe[uu][h] = __builtin_amdgcn_exp2f(s[uu][h] - mnew);
          lr[h] += pe[uu][h];
        }
        mr[h] = mnew;
      }
      // values: each group's V converted once, shared by the G heads
#pragma unroll
      for (int uu = 0; uu < kAttnU; ++uu) {
        if (gbase + uu * kWaves >= ngroups) continue;  // uniform
        float vf[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          vf[2 * d] = bf_lo(vr[uu][d]);
          vf[2 * d + 1] = bf_hi(vr[uu][d]);
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          if (h >= G) continue;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = __builtin_fmaf(pe[uu][h], vf[i], acc[h][i]);
        }
      }
    };

    // two buffers in flight; loads past the unit read zeros, so the loop body has no branch
    for (int gb = wave; gb < ngroups; gb += 2 * step) {
      patch_pos(gb, KA, VA);
      compute(gb, KA, VA);
      if (gb == wave) fstamp(p, layer, 1);
      load(gb + 2 * step, KA, VA);
      if (gb + step < ngroups) {  // uniform
        patch_pos(gb + step, KB, VB);
        compute(gb + step, KB, VB);
      }
      load(gb + 3 * step, KB, VB);
    }

    // every row's state into LDS (each row saw its own positions); rows that saw none hold
    // max -inf and zero sums
    fstamp(p, layer, 2);
    float* row = wp + (wave * Lds::PPW + ri) * GMAX * RS;
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) continue;
      float* dst = row + h * RS + d0;
      *reinterpret_cast<f32x4*>(dst) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
      if (li == 0) {
        row[h * RS + HD] = mr[h];
        row[h * RS + HD + 1] = lr[h];
      }
    }
  }
  wg_barrier();
  fstamp(p, layer, 3);
  if (!a.active) return;

  // wave h < G: the head's block max M over the R rows, each row's weight 2^(m - M) and the
  // block sum of the rows' sums under those weights
  if (wave < G) {
    const int h = wave;
    float* rp = wp + (min(lane, NR - 1) * GMAX + h) * RS;
    const float m = lane < NR ? rp[HD] : NEG_INF;
    const float M = wave_max(m);  // finite: row 0 of wave 0 holds the unit's first position
    const float w = (m == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m - M);
    const float Ls = wave_sum(lane < NR ? rp[HD + 1] * w : 0.f);
    if (lane < NR) rp[HD + 2] = w;
    if (lane == 0) {
      hs[2 * h] = M;
      hs[2 * h + 1] = Ls;
    }
  }
  wg_barrier();

  // The weighted sum over the rows of each pair of output dims of each head: NS lanes of a quad
  // take every NS-th row (eight rows per batch of LDS reads) and add their sums by DPP. The
  // quad's first lane then writes this unit's tagged partial (values, max, sum) or, for a single
  // split, the attention output.
  const int npair = G * HD / 2;
  const int NS = npair * 4 <= kThreads ? 4 : (npair * 2 <= kThreads ? 2 : 1);  // uniform
  const uint32_t tpart = tag_of(p, layer, kTagPart), to_tag = tag_of(p, layer, kTagO);
  for (int t = tid; t < npair * NS; t += kThreads) {  // NS divides npair * NS: quads stay whole
    const int pi = t / NS, sub = t - pi * NS;
    const int h = pi / (HD / 2), d = 2 * (pi - h * (HD / 2));
    const float* rp = wp + h * RS;
    float A0 = 0.f, A1 = 0.f;
    for (int r0 = sub; r0 < NR; r0 += 8 * NS) {  // NR / NS is a multiple of 8
      float w[8];
      float2 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float* q = rp + (r0 + k * NS) * GMAX * RS;
        w[k] = q[HD + 2];
        v[k] = *reinterpret_cast<const float2*>(q + d);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        A0 = __builtin_fmaf(v[k].x, w[k], A0);
        A1 = __builtin_fmaf(v[k].y, w[k], A1);
      }
    }
    if (NS >= 2) {
      A0 += dpp<0xB1>(A0);
      A1 += dpp<0xB1>(A1);
    }
    if (NS >= 4) {
      A0 += dpp<0x4E>(A0);
      A1 += dpp<0x4E>(A1);
    }
    // every lane of the quad holds both sums now
    const float M = hs[2 * h], Ls = hs[2 * h + 1];
    if (S == 1) {
      if (sub != 0) continue;
      const float inv = 1.0f / Ls;
      st_tag(p.to + ((g * G + h) * HD + d) / 2,
             static_cast<uint32_t>(f32_to_bf16(A0 * inv)) | (static_cast<uint32_t>(f32_to_bf16(A1 * inv)) << 16),
             to_tag);
    } else {
      // lanes 0 and 1 of the quad store the pair's two words with one store instruction, so a
      // wave writes whole runs of consecutive words (whole cache sectors)
      uint64_t* dst = p.tpart + (static_cast<size_t>(g * G + h) * p.s_cap + j) * (HD + 2);
      if (NS >= 2) {
        if (sub < 2) st_tag(dst + d + sub, __float_as_uint(sub == 0 ? A0 : A1), tpart);
      } else {
        st_tag(dst + d, __float_as_uint(A0), tpart);
        st_tag(dst + d + 1, __float_as_uint(A1), tpart);
      }
      if (d == 0 && sub == 0) {
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
  fstamp(p, layer, 4);
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
// q of the unit's G heads (fp32) into qs[G][HD] and, for the unit that holds pos, K/V(pos)
// (bf16 pairs of dims i, i + HD/2) into the bf16 area after it. Returns false if abandoned.
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
  return poll_block<2>(
      p, nq4 + 2 * nkv4, tag_of(p, layer, kTagQKV),
      [&](int qi) {
        return qi < nq4 ? oq + 16 * qi : (qi < nq4 + nkv4 ? ok_ + 16 * (qi - nq4) : ov + 16 * (qi - nq4 - nkv4));
      },
      [&](int, int qi, uint32_t x0, uint32_t x1) {
        if (qi < nq4) {
          qs[2 * qi] = __uint_as_float(x0);
          qs[2 * qi + 1] = __uint_as_float(x1);
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

template <int HD, int FMT, int GMAX>
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
    if (t < 0 || t >= p.V) stc(p.err, kErrBadToken);  // the step decodes token 0 and is abandoned
  }
  uint64_t* trace = p.trace ? p.trace + static_cast<size_t>(blockIdx.x) * p.trace_stride : nullptr;
  int ev = 0;
  auto stamp = [&]() {
    if (trace != nullptr && threadIdx.x == 0) trace[ev] = wall_clock64();
    ++ev;
  };
  stamp();
  float* xs = smem;                                  // GEMV input vector (swizzled)
  float* qs = smem + AttnLds<HD, GMAX>::kQ;          // attention: q, K/V(pos)
  const int H = p.H, L = p.L;
  const int qkv_pairs = (p.nq + 2 * p.nkv) * (HD / 2);
  const int qdim = p.nq * HD;
  GemvRegs R;
  AttnRegs<GMAX> AR;
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

  gemv_prefetch<FMT, EPI_QKV>(p, p.w_qkv, p.s_qkv, H, qkv_pairs, false, R);
  rmsnorm_embed_to_lds<FMT>(p, p.norm_in, xs, red);
  stamp();
  wg_barrier();
  for (int l = 0; l < L; ++l) {
    if (l > 0) {  // RMSNorm of the residual written by the previous layer's down stage
      ok = norm_from_x<FMT>(p, p.norm_in + static_cast<size_t>(l) * H, tag_of(p, l - 1, kTagXD), xs, red);
      stamp();
      if (!handoff_done()) return;
    }
    // QKV GEMV -> RoPE; q, K/V(pos) as tagged words, K/V(pos) also into the cache
    gemv_run<FMT, EPI_QKV>(p, p.w_qkv + l * p.w_qkv_ls, p.s_qkv + l * p.s_qkv_ls, H, qkv_pairs, xs, l, false, R,
                           tag_of(p, l, kTagQKV));
    fstamp(p, l, 5);
    attention_prefetch<HD, GMAX>(p, l, AR);
    fstamp(p, l, 6);
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
    gemv_prefetch<FMT, EPI_RESID>(p, p.w_o + l * p.w_o_ls, p.s_o + l * p.s_o_ls, qdim, H / 2, l == 0, R);
    wg_barrier();  // attention is done with LDS
    if (ok) ok = vector_from_words<FMT>(p, p.to, qdim, tag_of(p, l, kTagO), xs);
    stamp();
    if (!handoff_done()) return;

    // O-projection + residual
    gemv_run<FMT, EPI_RESID>(p, p.w_o + l * p.w_o_ls, p.s_o + l * p.s_o_ls, qdim, H / 2, xs, l, l == 0, R,
                             tag_of(p, l, kTagXO));
    fstamp(p, l, 7);
    gemv_prefetch<FMT, EPI_SWIGLU>(p, p.w_gu + l * p.w_gu_ls, p.s_gu + l * p.s_gu_ls, H, p.F, false, R);
    fstamp(p, l, 8);
    wg_barrier();
    stamp();
    ok = norm_from_x<FMT>(p, p.norm_post + static_cast<size_t>(l) * H, tag_of(p, l, kTagXO), xs, red);
    stamp();
    if (!handoff_done()) return;

    // gate/up GEMV -> SwiGLU
    gemv_run<FMT, EPI_SWIGLU>(p, p.w_gu + l * p.w_gu_ls, p.s_gu + l * p.s_gu_ls, H, p.F, xs, l, false, R,
                              tag_of(p, l, kTagM));
    fstamp(p, l, 9);
    gemv_prefetch<FMT, EPI_RESID>(p, p.w_d + l * p.w_d_ls, p.s_d + l * p.s_d_ls, p.F, H / 2, false, R);
    fstamp(p, l, 10);
    wg_barrier();
    stamp();
    ok = vector_from_words16<FMT>(p, reinterpret_cast<const uint32_t*>(p.tm), p.F, tag_of(p, l, kTagM), xs);
    stamp();
    if (!handoff_done()) return;

    // down GEMV + residual
    gemv_run<FMT, EPI_RESID>(p, p.w_d + l * p.w_d_ls, p.s_d + l * p.s_d_ls, p.F, H / 2, xs, l, false, R,
                             tag_of(p, l, kTagXD));
    fstamp(p, l, 11);
    if (l + 1 < L)
      gemv_prefetch<FMT, EPI_QKV>(p, p.w_qkv + (l + 1) * p.w_qkv_ls, p.s_qkv + (l + 1) * p.s_qkv_ls, H, qkv_pairs,
                                  false, R);
    else if (FMT != 0 && p.lm_fmt == 0)  // quantized projections, bf16 lm_head
      gemv_prefetch<0, EPI_LOGITS>(p, p.w_lm, p.s_lm, H, p.V / 2, false, R);
    else
      gemv_prefetch<FMT, EPI_LOGITS>(p, p.w_lm, p.s_lm, H, p.V / 2, false, R);
    wg_barrier();
    stamp();
  }
  // final RMSNorm -> lm_head (in the lm_head's own storage format, which sets the LDS layout)
  const bool head16 = FMT != 0 && p.lm_fmt == 0;
  if (head16) ok = norm_from_x<0>(p, p.norm_final, tag_of(p, L - 1, kTagXD), xs, red);
  else ok = norm_from_x<FMT>(p, p.norm_final, tag_of(p, L - 1, kTagXD), xs, red);
  stamp();
  if (!handoff_done()) return;
  const EpiState st = head16 ? gemv_run<0, EPI_LOGITS>(p, p.w_lm, p.s_lm, H, p.V / 2, xs, L, false, R, 0u)
                             : gemv_run<FMT, EPI_LOGITS>(p, p.w_lm, p.s_lm, H, p.V / 2, xs, L, false, R, 0u);
  wg_barrier();
  stamp();
  if (p.next_token != nullptr) greedy_token(p, st, smem, red, ired);
}

// barrier microbenchmark: `iters` grid barriers in one persistent launch
__global__ void __launch_bounds__(kThreads, 1) amk_barrier_kernel(unsigned* ctr, unsigned* err, int iters) {
  __shared__ int abort_flag;
  if (threadIdx.x == 0) abort_flag = 0;
  __syncthreads();
  GridBarrier bar{ctr, 0u, 0u, 100000000ull, err, nullptr, 0};
  for (int i = 0; i < iters; ++i)
    if (!bar.sync(&abort_flag)) return;
}

template __global__ void amk_decode_kernel<64, 0, 4>(const KParams);
template __global__ void amk_decode_kernel<64, 1, 4>(const KParams);
template __global__ void amk_decode_kernel<128, 0, 4>(const KParams);
template __global__ void amk_decode_kernel<128, 1, 4>(const KParams);
template __global__ void amk_decode_kernel<64, 0, 8>(const KParams);
template __global__ void amk_decode_kernel<64, 1, 8>(const KParams);
template __global__ void amk_decode_kernel<128, 0, 8>(const KParams);
template __global__ void amk_decode_kernel<128, 1, 8>(const KParams);
template __global__ void amk_decode_kernel<64, 2, 4>(const KParams);
template __global__ void amk_decode_kernel<128, 2, 4>(const KParams);
template __global__ void amk_decode_kernel<64, 2, 8>(const KParams);
template __global__ void amk_decode_kernel<128, 2, 8>(const KParams);

}  // namespace amk

// host-visible handles of the kernel instantiations (defined in this translation unit)
// fmt: 0 bf16, 1 int8, 2 int4 projection weights
extern "C" __attribute__((visibility("hidden"))) const void* amk_kernel_handle(int head_dim, int fmt, int gmax) {
  using namespace amk;
  const void* const t[2][2][3] = {
      {{(const void*)&amk_decode_kernel<64, 0, 4>, (const void*)&amk_decode_kernel<64, 1, 4>,
        (const void*)&amk_decode_kernel<64, 2, 4>},
       {(const void*)&amk_decode_kernel<64, 0, 8>, (const void*)&amk_decode_kernel<64, 1, 8>,
        (const void*)&amk_decode_kernel<64, 2, 8>}},
      {{(const void*)&amk_decode_kernel<128, 0, 4>, (const void*)&amk_decode_kernel<128, 1, 4>,
        (const void*)&amk_decode_kernel<128, 2, 4>},
       {(const void*)&amk_decode_kernel<128, 0, 8>, (const void*)&amk_decode_kernel<128, 1, 8>,
        (const void*)&amk_decode_kernel<128, 2, 8>}}};
  if ((head_dim != 64 && head_dim != 128) || (gmax != 4 && gmax != 8) || fmt < 0 || fmt > 2) return nullptr;
  return t[head_dim == 128][gmax == 8][fmt];
}
extern "C" __attribute__((visibility("hidden"))) const void* amk_barrier_kernel_handle() { return (const void*)&amk::amk_barrier_kernel; }
