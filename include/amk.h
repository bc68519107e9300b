/*
 * amk.h — C ABI of the MI355X (gfx950) batch-1 Llama decode library.
 *
 * One call of amk_decode_step runs the whole forward pass of one decoded token as ONE
 * persistent cooperative kernel launch: RMSNorm, QKV GEMV, RoPE, GQA attention over the
 * KV cache, O-projection, SwiGLU gate/up/down GEMVs and the lm_head GEMV, with grid-level
 * synchronisation between dependent stages done by tagged hand-offs: a stage writes its output
 * as words that carry the step's tag, and each consumer block polls the words it needs until
 * they carry that tag (no grid barrier, no counter reset). This follows the problem statement of the
 * decode-megakernel pages: batch-1 decode is bandwidth bound, its latency floor is weight
 * bytes over HBM bandwidth, and per-operator launches plus activation round trips through
 * HBM keep frameworks off that floor (gist.science explainer of AutoMegaKernel, Technical
 * Summary > Problem Statement); the megakernel runs the forward pass of a HuggingFace
 * Llama-family model in one persistent cooperative launch (AutoMegaKernel paper index,
 * Abstract; explainer, Technical Summary > Methodology, Layer 0).
 *
 * Conventions for every function:
 *   - returns int status: AMK_OK (0) or a negative AMK_ERR_* code; no C++ exception or
 *     longjmp crosses this boundary;
 *   - "host" pointers are CPU memory, "device" pointers are GPU memory of the current
 *     device (for example torch.Tensor.data_ptr() of a CUDA/HIP tensor);
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *   - amk_status_string() describes the most recent error of the calling thread.
 */
#ifndef AMK_H_
#define AMK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AMK_OK 0
#define AMK_ERR_INVALID_ARG (-1)     /* null pointer, token/pos/index out of range         */
#define AMK_ERR_UNSUPPORTED (-2)     /* model shape or format outside the supported set    */
#define AMK_ERR_HIP (-3)             /* a HIP runtime call failed (text via status string) */
#define AMK_ERR_COOPERATIVE (-4)     /* the persistent grid cannot be co-resident          */
#define AMK_ERR_SYNC_TIMEOUT (-5)    /* a grid-level wait exceeded its bound (device)      */
#define AMK_ERR_OOM (-6)             /* host or device allocation failed                   */

#define AMK_BF16 0  /* weights stored bf16, fp32 accumulation                              */
#define AMK_W8A16 1 /* weights int8, one fp32 scale per output row; activations bf16      */
#define AMK_W8A16_BF16_HEAD 2 /* AMK_W8A16 projections, lm_head kept bf16 (for a tied model the
                                 head reads the bf16 embedding table; no quantized copy)      */
#define AMK_W4A16 3 /* projections int4 (eight codes per word), one fp32 scale per output row;
                       lm_head kept bf16 as in AMK_W8A16_BF16_HEAD; activations bf16           */
#define AMK_W4A16_G128 4 /* projections int4 as in AMK_W4A16, one fp16 scale per row and group
                            of 128 columns; lm_head kept bf16; activations bf16               */

/* Model description. Weights follow HuggingFace LlamaForCausalLM: pre-norm RMSNorm,
 * rotate-half RoPE with inv_freq_i = rope_theta^(-2i/head_dim), grouped-query attention
 * (q head h reads kv head h / (n_q_heads / n_kv_heads)), SwiGLU MLP, no biases (biased
 * projections are not representable, matching the pages' rejection of unsupported variants,
 * explainer, Technical Summary > Key Contributions). */
typedef struct {
  int32_t hidden;          /* H                                                              */
  int32_t n_layers;        /* L                                                              */
  int32_t n_q_heads;       /* nq                                                             */
  int32_t n_kv_heads;      /* nkv; nq % nkv == 0 and nq / nkv <= 8                           */
  int32_t head_dim;        /* 64 or 128                                                      */
  int32_t ffn;             /* F (intermediate size)                                          */
  int32_t vocab;           /* V                                                              */
  int32_t max_ctx;         /* KV-cache capacity in positions                                 */
  float rms_eps;           /* RMSNorm epsilon                                                */
  float rope_theta;        /* RoPE base                                                      */
  int32_t tied_embeddings; /* 1: lm_head is embed_tokens                                     */
  int32_t weight_format;   /* AMK_BF16, AMK_W8A16, AMK_W8A16_BF16_HEAD, AMK_W4A16 or
                              AMK_W4A16_G128                                                 */
  /* Llama-3 RoPE frequency scaling (the rule Llama 3.1 / 3.2 checkpoints declare; the pages do
   * not describe it): rope_scale_factor <= 1 means none. Otherwise a frequency f with
   * wavelength 2 pi / f shorter than rope_original_ctx / rope_high_freq_factor is kept, one
   * longer than rope_original_ctx / rope_low_freq_factor becomes f / factor, and in between it
   * moves linearly in rope_original_ctx / wavelength from f / factor to f. */
  float rope_scale_factor;
  float rope_low_freq_factor;
  float rope_high_freq_factor;
  int32_t rope_original_ctx;
} amk_config;

typedef struct amk_model amk_model; /* opaque, library-owned */

/* Launch geometry and memory of a loaded model (for tests and benchmarks). */
typedef struct {
  int32_t grid_blocks;          /* persistent blocks (one per compute unit)                 */
  int32_t block_threads;        /* threads per block                                         */
  int32_t lds_bytes;            /* dynamic LDS per block                                     */
  int32_t handoffs_per_step;    /* grid-wide tagged vector exchanges in one decode step
                                   (6 per layer + 1); the launch has no grid barrier        */
  int64_t weight_bytes;         /* device bytes of packed weights + scales + norms           */
  int64_t scratch_bytes;        /* device bytes of library scratch                           */
  int32_t max_splits;           /* upper bound on KV splits per kv head                      */
  int32_t device;               /* HIP device the model lives on                             */
  int64_t dump_layer_floats;    /* floats per layer of the per-stage dump (amk_set_dump)      */
  int64_t dump_floats;          /* floats of a whole dump: n_layers * dump_layer_floats + H  */
  int32_t gemv_item_slots;      /* 1 KB chunk slots per row in a GEMV item of the kernel
                                   variant: 1 for hidden <= 2048, else 2                     */
} amk_info;

/* Copies, packs, (for the quantized formats) quantizes and uploads a model to the current device.
 * host_bf16_tensors: n_tensors host pointers to bf16 bit patterns (uint16), row-major
 *   [out][in] for matrices, in canonical HF order:
 *     embed_tokens [V][H];
 *     per layer: input_layernorm [H], q_proj [nq*hd][H], k_proj [nkv*hd][H],
 *       v_proj [nkv*hd][H], o_proj [H][nq*hd], post_attention_layernorm [H],
 *       gate_proj [F][H], up_proj [F][H], down_proj [H][F];
 *     norm [H]; lm_head [V][H] only when tied_embeddings == 0.
 *   n_tensors must equal 2 + 9 L + (tied ? 0 : 1).
 * W8A16 quantizes every projection and the lm_head (for tied models: a quantized copy of
 * embed_tokens; the embedding gather keeps reading bf16) with amk_quantize_int8.
 * AMK_W8A16_BF16_HEAD quantizes the projections the same way and keeps the lm_head bf16 (the
 * int8-weights reading in which only the projections shrink: the pages quote int8 weight bytes
 * at 0.61 of bf16, a figure a bf16 head explains; gist.science explainer, Experimental
 * Results).
 * AMK_W4A16 quantizes the projections with amk_quantize_int4 and keeps the lm_head bf16 (the
 * pages' int4 weight-only variant: lossy, 2.42x less weight traffic than bf16; gist.science
 * explainer, Technical Summary > Key Contributions; this format streams 1/2.44 of the bf16
 * weight bytes of a SmolLM2-135M or Llama-3.2-1B shape). Device row layout: columns 8i .. 8i + 7
 * in 32-bit word i; byte k of a word holds |q| of column k in bits 0..2 and its sign in bit 7,
 * |q| of column k + 4 in bits 4..6, and the sign of column (k + 3) mod 4 + 4 in bit 3.
 * AMK_W4A16_G128 quantizes the projections with amk_quantize_int4_g128 (one scale per 128
 * columns) and keeps the lm_head bf16: the same codes and code layout as AMK_W4A16, plus 2
 * bytes of scale per 128 weights, 1/2.415 of the bf16 weight bytes on those two shapes. The
 * device holds the 16 scales of each 2048-column chunk of a row pair (both rows) together, 64
 * bytes per pair and chunk.
 * Synchronous. The caller keeps ownership of its host tensors (they may be freed on return);
 * *out receives a model handle owned by the library until amk_free.
 * Errors: INVALID_ARG (null pointers, wrong n_tensors); UNSUPPORTED for a shape outside the
 * supported set: head_dim in {64,128}, nq % nkv == 0, nq/nkv <= 8, hidden, ffn and nq*hd
 * multiples of 16 (of 32 for AMK_W4A16 and AMK_W4A16_G128), vocab even, hidden <= 8192, ffn and nq*hd <= 32768,
 * every packed weight matrix, the embedding and each (layer, K/V, kv head) block of the cache
 * below 2^31 bytes (the kernel addresses them with 32-bit offsets); and, on the current device
 * with G compute units (one persistent block each): nkv <= G, ffn >= G, and for n_layers >= 2
 * (nq + 2 nkv) * head_dim / 2 >= G. The last two give every block at least one row pair of the
 * gate/up and QKV stages, which the tagged hand-offs need: a block then cannot fall a whole
 * layer behind the blocks that overwrite the exchange words it still polls. HIP, OOM,
 * COOPERATIVE (no co-resident persistent grid). */
int amk_load_weights(const amk_config* cfg, const uint16_t* const* host_bf16_tensors,
                     int32_t n_tensors, amk_model** out);

/* Checks a model description against everything amk_load_weights requires of it, for a device
 * with `compute_units` compute units (the persistent grid has one block per unit; MI355X: 256),
 * on the host only: no GPU is needed and nothing is allocated. The pages validate a schedule
 * before it reaches the GPU, so a bad one gets a clean rejection instead of a hang (gist.science
 * explainer, Methodology > Safety Gate); here the schedule is fixed, and what can be rejected is
 * the model shape. Returns AMK_OK, or UNSUPPORTED with the reason in amk_status_string (the
 * conditions are listed at amk_load_weights); INVALID_ARG for a null cfg or compute_units <= 0. */
int amk_validate_config(const amk_config* cfg, int32_t compute_units);

/* Decodes one token: feeds `token` at position `pos`, writes K/V of position `pos` in every
 * layer of `kv_cache`, attends over positions [0, pos] inclusive, and writes fp32 logits.
 * One cooperative kernel launch, ordered on `stream`; returns once it is enqueued, the
 * outputs are valid when the stream reaches that point.
 * kv_cache: device bf16 [L][2 (K, V)][nkv][max_ctx][head_dim], amk_kv_cache_bytes() long,
 *   caller-owned; slots [0, pos) must already hold this sequence's keys/values.
 * logits_out: device fp32 [V], caller-owned.
 * Errors:
 *   - INVALID_ARG for a null handle or pointer, token outside [0, V) or pos outside
 *     [0, max_ctx): checked on the host before any HIP call;
 *   - SYNC_TIMEOUT or INVALID_ARG for a failure of an EARLIER step of this model that has
 *     completed on the device by the time of this call: a hand-off wait that exceeded its bound
 *     (SYNC_TIMEOUT), or an out-of-range device token of a greedy step (INVALID_ARG). The kernel
 *     raising the error writes its code to a word in pinned host memory, which this call reads
 *     without synchronising. The call then launches nothing: it enqueues, on `stream`, the reset
 *     of the model's device state (exchange words and error flag), after which the model is
 *     usable again, and returns the error. The failed step's outputs are undefined (it may have
 *     written some, all or none of its logits, K/V slots and token); steps launched after it
 *     and before the reset did nothing: their logits_out and K/V slots are left unwritten. A
 *     failure whose kernel has not finished yet is reported by a later call or by amk_sync.
 *     The pages require a clean rejection instead of a hung GPU (gist.science explainer,
 *     Methodology > Safety Gate): every wait in the kernel is bounded;
 *   - HIP if the launch fails.
 * Concurrency: one handle must not run two steps at once (they share the scratch). */
int amk_decode_step(amk_model* m, int32_t token, int32_t pos, void* kv_cache,
                    float* logits_out, void* stream);

/* amk_decode_step for callers that cannot allocate device memory around a step: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation. The same forward pass,
 * arguments, outputs and host checks as amk_decode_step, but this call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine): the step's exchange words and error flag
 * live in a file-scope static device array of the library (4 MiB per GPU, held until the process
 * ends; its address is looked up once per device when a model is loaded) instead of the model's
 * scratch. The call first clears the part the model uses (a kernel on `stream`), so it does not
 * depend on what an earlier call on that GPU left there. Every such call on one GPU shares the
 * array: calls that overlap in time on one GPU (other streams, other threads, other models) race
 * and must not be issued. Errors: those of amk_decode_step, and UNSUPPORTED when the model needs
 * more than 4 MiB of exchange words (no shape that amk_load_weights accepts on a 256-CU device
 * needs more than 3 MiB). A failure of this call is reported like that of amk_decode_step (by
 * the model's next call or amk_sync); it does not turn later calls into no-ops. */
int amk_decode_step_noalloc(amk_model* m, int32_t token, int32_t pos, void* kv_cache,
                            float* logits_out, void* stream);

/* Greedy decode step with device-resident tokens (no host round trip per token): the same
 * forward pass as amk_decode_step, but the input token is read from device memory and the step
 * also writes the greedy next token: the argmax over the logits, with ties going to the lowest
 * index. The pages decode greedily (AutoMegaKernel paper index, Abstract); the tie rule is this
 * library's, and it matches numpy.argmax. Passing one step's next_token_out as the next step's
 * token_in (with pos + 1) decodes a sequence with no host synchronisation; such a chain of
 * launches can be captured in a HIP graph.
 * token_in: device int32 [1], read once the launch starts; next_token_out: device int32 [1],
 *   written at the end of the step (it may be the same buffer as token_in);
 * logits_out: device fp32 [V] or NULL (then no logits are written);
 * kv_cache, pos, stream: as for amk_decode_step. All buffers are caller-owned.
 * Errors: INVALID_ARG for a null handle, token_in, kv_cache or next_token_out, or pos outside
 * [0, max_ctx) (host checks, before any HIP call); an earlier step's failure as for
 * amk_decode_step; HIP if the launch fails. A token_in value outside [0, V) cannot be checked
 * on the host: the step then decodes token 0 in its place, its outputs are undefined, and the
 * next call (or amk_sync) reports INVALID_ARG. */
int amk_decode_step_greedy(amk_model* m, const int32_t* token_in, int32_t pos, void* kv_cache,
                           float* logits_out, int32_t* next_token_out, void* stream);

/* Waits for `stream` and reports a device-side error raised by an earlier step of this model
 * that no step call has reported yet (AMK_ERR_SYNC_TIMEOUT for an abandoned hand-off wait,
 * AMK_ERR_INVALID_ARG for an out-of-range device token of a greedy step), then resets the
 * model's device state and waits for the reset, so the model is usable again. Steps launched
 * after the error and before the reset do nothing (their outputs are left unwritten). */
int amk_sync(amk_model* m, void* stream);

/* Bytes of the caller-owned KV cache: L * 2 * nkv * max_ctx * head_dim * 2. 0 for NULL. */
size_t amk_kv_cache_bytes(const amk_model* m);

/* Launch geometry and sizes of a loaded model. */
int amk_get_info(const amk_model* m, amk_info* info);

/* Copies the codes and scales the library uses for canonical tensor `tensor_index` (a quantized
 * projection, or, for AMK_W8A16, the lm_head index 2+9L / embed index 0 for a tied model) back
 * to host memory in canonical [rows][cols] order, one code per int8 (int4 codes unpacked, in
 * [-7, 7]). codes_out: host int8 [rows*cols]; scales_out: host fp32 [rows] (row scales), or,
 * for AMK_W4A16_G128, [rows][ceil(cols / 128)] (the fp16 group scales, widened exactly).
 * Errors: INVALID_ARG for a tensor that is not quantized (including the bf16 head of
 * AMK_W8A16_BF16_HEAD, AMK_W4A16 and AMK_W4A16_G128); UNSUPPORTED for an AMK_BF16 model. */
int amk_export_quantized(const amk_model* m, int32_t tensor_index, int8_t* codes_out,
                         float* scales_out);

/* Host quantizer used by amk_load_weights (no GPU needed): symmetric int8 per output row.
 * For row n: amax = max |w|, s = fp32(amax / 127) by IEEE division, q = clamp(round half to
 * even(fp32(w / s)), -127, 127); an all-zero row gives s = 0 and q = 0. The pages name
 * int8 weight-only (W8A16) megakernels without the scale rule (AutoMegaKernel paper index,
 * Abstract; explainer, Technical Summary > Key Contributions); this per-row rule is the one
 * the W8A16 workload states. w: host bf16 bit patterns [rows][cols]; codes: host int8
 * [rows][cols]; scales: host fp32 [rows]. Errors: INVALID_ARG for null pointers or
 * non-positive sizes. */
int amk_quantize_int8(const uint16_t* w, int64_t rows, int64_t cols, int8_t* codes,
                      float* scales);

/* Host quantizer of AMK_W4A16 (no GPU needed): the same rule at four bits. For row n: amax =
 * max |w|, s = fp32(amax / 7) by IEEE division, q = clamp(round half to even(fp32(w / s)), -7,
 * 7); an all-zero row gives s = 0 and q = 0. The pages name int4 weight-only quantization as
 * lossy with 2.42x less weight traffic (gist.science explainer, Technical Summary > Key
 * Contributions) without its format; this per-row rule is the W8A16 one at four bits.
 * w: host bf16 bit patterns [rows][cols]; codes: host int8 [rows][cols], one code per byte;
 * scales: host fp32 [rows]. Errors: INVALID_ARG for null pointers or non-positive sizes. */
int amk_quantize_int4(const uint16_t* w, int64_t rows, int64_t cols, int8_t* codes,
                      float* scales);

/* Host quantizer of AMK_W4A16_G128 (no GPU needed): the int4 rule applied to each group of 128
 * consecutive columns of a row (a row whose length is not a multiple of 128 ends with a shorter
 * group), with the scale held in IEEE half precision. Per group: amax = max |w|, s =
 * fp16(fp32(amax / 7)) (IEEE fp32 division, then round to nearest even to half precision;
 * values past 65504 saturate to 65504), q = clamp(round half to even(fp32(w / s)), -7, 7); s ==
 * 0 gives q = 0. The pages give the int4 variant no format (gist.science explainer, Technical
 * Summary > Key Contributions); per-group half-precision scales are the usual int4 weight-only
 * layout, and at 128 columns they meet the pages' 2.42x weight-traffic figure most closely.
 * w: host bf16 bit patterns [rows][cols]; codes: host int8 [rows][cols]; scales: host fp32
 * [rows][ceil(cols / 128)] holding the half-precision values exactly. Errors: INVALID_ARG for
 * null pointers or non-positive sizes. */
int amk_quantize_int4_g128(const uint16_t* w, int64_t rows, int64_t cols, int8_t* codes,
                           float* scales);

/* Debug control: bound (in 100 MHz wall-clock ticks) on any single hand-off poll or barrier
 * wait; 0 restores the default (one second). A tiny bound makes steps fail cleanly with
 * SYNC_TIMEOUT, which is how the timeout path is exercised. */
int amk_set_spin_limit(amk_model* m, uint64_t ticks);

/* Debug control: per-block stage timestamps. When trace is non-NULL, every later step of this
 * model writes, for each block b, the 100 MHz wall clock into trace[b * events_per_block + e]:
 * e = 0 at kernel entry; e = 1 + 11 l + k for layer l and k = 0..10: the layer's RMSNorm in
 * LDS, QKV epilogue, q received, attention partial stored, split merge stored, attention output
 * received, O epilogue, RMSNorm 2 in LDS, gate/up epilogue, SwiGLU output received, down
 * epilogue; e = 1 + 11 L when the final RMSNorm is in LDS and e = 2 + 11 L at the end of the
 * lm_head (events_per_block >= 3 + 11 * n_layers).
 * trace: device uint64 [grid_blocks][events_per_block], caller-owned. NULL switches tracing off.
 * Errors: INVALID_ARG for a null handle or a too small events_per_block. */
int amk_set_trace(amk_model* m, uint64_t* trace, int32_t events_per_block);

/* Debug control: per-stage dumps, so each stage of every layer can be checked against the plain
 * definition applied to the kernel's own input for that stage (the pages check the generated
 * kernel's parts in isolation against eager references: gist.science explainer, Methodology >
 * Layer 1). When dump is non-NULL, every later step of this model writes fp32 values into it:
 * for layer l, at dump + l * S (S = amk_info.dump_layer_floats = 6 H + QKV + 2 QD + 3 F with
 * QKV = (nq + 2 nkv) head_dim and QD = nq head_dim), in this order:
 *   h [H]        RMSNorm output that feeds the QKV projection (bf16 values);
 *   qkv [QKV]    QKV projection output before RoPE (row scale applied), q | k | v rows in the
 *                canonical order of q_proj, k_proj, v_proj;
 *   q [QD]       q after RoPE;
 *   o [QD]       attention output (bf16 values), head-major;
 *   wo [H]       O-projection output;
 *   x_o [H]      residual after the O-projection;
 *   h2 [H]       RMSNorm output that feeds gate/up (bf16 values);
 *   gu [2F]      gate outputs [F], then up outputs [F];
 *   m [F]        SwiGLU output (bf16 values);
 *   wd [H]       down-projection output;
 *   x_d [H]      residual after the down projection;
 * then, at dump + L * S, the final RMSNorm output [H] that feeds the lm_head. The K/V of the
 * step's position are in the KV cache and the logits in logits_out. dump: device fp32 of at
 * least floats = amk_info.dump_floats elements, caller-owned. NULL switches dumping off.
 * Errors: INVALID_ARG for a null handle or floats too small. */
int amk_set_dump(amk_model* m, float* dump, int64_t floats);

/* Releases every device and host resource of the handle. NULL is accepted. */
int amk_free(amk_model* m);

/* Text for a status code, including the failing HIP call of the last AMK_ERR_HIP. */
const char* amk_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* AMK_H_ */
