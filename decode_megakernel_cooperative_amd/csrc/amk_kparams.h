// Parameter block of the persistent decode kernel (passed by value at launch).
#pragma once
#include <stdint.h>

namespace amk {

constexpr int kThreads = 512;          // threads per persistent block (8 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kCtrStride = 32;         // 32 x 4 B = one 128 B line
constexpr int kAttnTile = 16;          // positions per attention tile (one MFMA column block)

// LDS bytes of the attention stage: per wave a K and a V tile of kAttnTile positions (rows padded
// by 32 bytes) and one result row per head [gmax][hd + 4] fp32; then q of the G heads (bf16 high
// and low parts, 4 bytes per value in all) and K/V of the current position (bf16).
constexpr int attn_lds_bytes(int hd, int gmax, int G) {
  return 2 * kWaves * kAttnTile * (2 * hd + 32) + kWaves * gmax * (hd + 4) * 4 + G * hd * 4 + 4 * hd;
}

// Tags of the exchange words: stage `which` of layer l in a launch writes tag
// tag0 + l * kTagsPerLayer + which; the host advances tag0 by kTagsPerLayer * L + 1 per launch.
constexpr int kTagsPerLayer = 6;
// device error flag values
constexpr unsigned kErrTimeout = 1;   // a hand-off poll exceeded spin_limit
constexpr unsigned kErrBadToken = 2;  // a device-resident input token was outside [0, V)
enum { kTagQKV = 0, kTagPart = 1, kTagO = 2, kTagXO = 3, kTagM = 4, kTagXD = 5 };

struct KParams {
  // model
  int32_t H, L, nq, nkv, hd, F, V, max_ctx;
  float eps, attn_scale;
  // this step
  int32_t token, pos, S, T;
  const int32_t* token_dev;                 // greedy step: input token in device memory (else null)
  int32_t* next_token;                      // greedy step: argmax of the logits (else null)
  // packed weights: per layer, rows are stored in the order the kernel consumes them
  const uint8_t* w_qkv; int64_t w_qkv_ls;   // bytes per layer
  const float* s_qkv;   int64_t s_qkv_ls;   // per layer: fp32 row scales, or the packed fp16 group
                                            // scales of format 3 (stride in floats)
  const uint8_t* w_o;   int64_t w_o_ls;
  const float* s_o;     int64_t s_o_ls;
  const uint8_t* w_gu;  int64_t w_gu_ls;
  const float* s_gu;    int64_t s_gu_ls;
  const uint8_t* w_d;   int64_t w_d_ls;
  const float* s_d;     int64_t s_d_ls;
  const uint8_t* w_lm;
  const float* s_lm;
  int32_t lm_fmt;                           // lm_head storage: 0 bf16, 1 int8 (+ s_lm)
  const uint16_t* embed;                    // bf16 [V][H]
  const float* norm_in;                     // fp32 [L][H]
  const float* norm_post;                   // fp32 [L][H]
  const float* norm_final;                  // fp32 [H]
  const float* rope_cos;                    // fp32 [max_ctx][hd/2]
  const float* rope_sin;
  // caller buffers
  uint16_t* kv;                             // bf16 [L][2][nkv][max_ctx][hd]
  float* logits;                            // fp32 [V]
  // scratch (library-owned)
  int32_t s_cap;                            // split capacity per kv head (partials stride)
  unsigned* err;                            // device error flag
  unsigned* herr;                           // pinned host word: the code of the error that set err
  uint64_t spin_limit;                      // wall-clock ticks per hand-off poll
  // tagged exchange words (low 32 bits payload, high 32 bits tag), all inside one region so a
  // single buffer resource covers them
  uint64_t* tagged; uint32_t tagged_bytes;
  uint64_t* tx;                             // [H] residual (fp32)
  uint64_t* tq;                             // [nq*hd] rotated queries (fp32)
  uint64_t* tkv;                            // [2][nkv][hd/2] K/V of pos, bf16 dims (i, i+hd/2)
  uint64_t* tpart;                          // [nq][s_cap][hd+2] split partials: values, max (base 2), sum
  uint64_t* to;                             // [nq*hd/2] attention output, 2 bf16 per word
  uint64_t* targ;                           // [grid][2] greedy step: each block's argmax (value, index)
  uint64_t* tm;                             // SwiGLU output: [F] 32-bit words bf16 << 16 | tag & 0xffff
  uint32_t tag0;
  uint64_t* trace;                          // optional [grid][trace_stride] wall-clock stamps
  int32_t trace_stride;
  float* dump;                              // optional per-stage dump, dump_stride floats per layer
  int64_t dump_stride;
};

}  // namespace amk
