/*
 * hta.h -- C ABI of the MI355X (gfx950) batch-1 codebook-TTS decode library.
 *
 * What it computes (reference pages):
 *  - FlashRT "Higgs Audio v3 TTS-4B" page, summary: a dense Qwen3-4B-shaped
 *    backbone (GQA, SwiGLU, RoPE theta 1e6) driving a fused head of
 *    8 codebooks x 1026 under a delay pattern.
 *  - same page, section 5: the per-frame chain RMSNorm (+quant) -> qkv GEMV ->
 *    q/k-norm + RoPE (+KV write) -> attention -> o_proj GEMV with residual ->
 *    RMSNorm -> gate/up GEMV -> SiLU*mul (+quant) -> down GEMV with residual
 *    -> final RMSNorm (+quant) -> fused head GEMV -> greedy argmax with the
 *    delay mask -> embedding of the chosen codes as the next input.
 *  - same page, section 7: one batched prefill pass over the prompt; a kept
 *    preamble KV is reused and only a suffix is prefilled.
 *  - same page, section 8: FP8 W8A8 with per-tensor static activation scales
 *    (amax / 448) from a BF16 calibration run.
 *  - SGLang-Omni Higgs Audio v3 page, architecture paragraph: the next input
 *    is the sum of the 8 codebook embeddings of the previous frame.
 *
 * Conventions for every call:
 *  - Return value: HTA_OK (0), HTA_DONE (1, decode only) or a negative
 *    error code; hta_last_error() gives a message.  Nothing throws.
 *  - "device" pointers are HIP device addresses (e.g. a torch CUDA tensor's
 *    data_ptr); "host" pointers are ordinary host memory, read or written
 *    before the call returns.
 *  - All GPU work is enqueued on the stream given to hta_create; calls that
 *    return results to the host synchronise that stream.
 *  - A context is not thread-safe; use one per thread.
 *  - The caller owns all device memory (weights, workspace); the library owns
 *    only its graph objects and a small pinned host staging buffer.
 *    hta_destroy must run before the caller frees the workspace, because the
 *    captured graphs reference it.
 */
#ifndef HTA_H
#define HTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HTA_OK = 0,
  HTA_DONE = 1,            /* decode: this step completed the utterance (codebook 7 emitted EOS) */
  HTA_E_ARG = -1,          /* null pointer, size mismatch, bad enum */
  HTA_E_STATE = -2,        /* call out of order (e.g. decode before load) */
  HTA_E_CAPACITY = -3,     /* length + P would exceed max_seq, or P > max_prefill */
  HTA_E_RANGE = -4,        /* token id >= text_vocab or code id >= codebook_size */
  HTA_E_UNSUPPORTED = -5,  /* device is not gfx950, or a shape the kernels do not cover */
  HTA_E_HIP = -6,          /* HIP runtime error; message in hta_last_error */
  HTA_E_TIMEOUT = -7       /* a device-side bounded wait expired (the kernel exited early) */
};

typedef enum { HTA_BF16 = 0, HTA_FP8_E4M3 = 1 } hta_precision;
typedef enum { HTA_SRC_F32 = 0, HTA_SRC_BF16 = 1 } hta_src_dtype;

typedef struct {
  int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, text_vocab;
  int n_codebooks;   /* 8 */
  int codebook_size; /* 1026: codes 0..1023, BOS 1024, EOS 1025 */
  int bos_id, eos_id;
  float rope_theta;  /* 1e6 */
  float rms_eps;     /* 1e-6 */
  int max_seq;       /* KV capacity in positions */
  int max_prefill;   /* largest P accepted by one hta_prefill call */
  int precision;     /* hta_precision */
  int n_streams;     /* utterances decoded together (batched decode); 0 reads as 1 */
} hta_config;

typedef struct hta_ctx hta_ctx;

/* Batched decode (SGLang-Omni Higgs Audio v3 page, performance section: requests decoded
 * concurrently on one GPU).  A context with n_streams = M > 1 holds M independent
 * utterances, each with its own KV cache, delay state and code history, over one copy of
 * the weights.  hta_select_stream picks the stream that hta_prefill, hta_reset,
 * hta_force_codes and hta_read_tap (HIDDEN, LOGITS, STATE, KV) act on.  hta_decode_frame(s)
 * advance every stream by one step per frame in one batched step: the embedding of each
 * stream's previous codes, then per layer the M rows through the same GEMMs (one weight
 * stream shared by all streams), q/k-norm + RoPE + KV write at each stream's own position,
 * decode attention of each row over its own cache (key splits, log-sum-exp combine), and
 * the head with each stream's greedy argmax and delay rule; the whole step is one captured
 * graph.  codes_out then receives n * M * C codes ([frame][stream][codebook]); *n_done
 * the number of streams whose utterance is done; HTA_DONE when all are.  Limits: 2 <= M
 * <= 128 and M <= max_prefill; greedy only (hta_set_sampling gives HTA_E_UNSUPPORTED);
 * hta_calibrate, hta_layer_step, HTA_OPT_TAPS, hta_time_kernels and
 * hta_decode_frames_noalloc need a single-stream context. */

/* Shape limits the kernels support (hta_create returns HTA_E_UNSUPPORTED otherwise):
 * head_dim 64 or 128; hidden, ffn and the q width (n_q_heads * head_dim) multiples of
 * 128, with hidden <= 5120 and ffn, q width <= 10240; GQA group n_q_heads / n_kv_heads
 * of 1, 2 or 4; n_kv_heads <= 32, n_q_heads + n_kv_heads <= 64, kv width <= 2048;
 * n_codebooks <= 16; codebook_size <= 2048.  The decode frame kernel runs one resident
 * block per compute unit (256 on MI355X), and each of its GEMV phases needs at least one
 * row unit per block: q + 2 kv widths, hidden, ffn (gate/up pairs) and n_codebooks *
 * codebook_size must each be at least the compute-unit count. */

/* Create a context for cfg on the current HIP device, enqueueing on hip_stream
 * (a hipStream_t, e.g. torch.cuda.current_stream().cuda_stream; NULL makes the
 * library create a non-blocking stream of its own, destroyed by hta_destroy).  Fails
 * with HTA_E_UNSUPPORTED on a device other than gfx950 or an unsupported shape.
 * *out receives the context. */
int hta_create(const hta_config* cfg, void* hip_stream, hta_ctx** out);

/* Bytes of device workspace the context needs: packed weights, KV cache
 * [layer][kv_head][max_seq][head_dim] bf16 x 2, RoPE table, decode state and
 * scratch.  Usable before hta_create. */
size_t hta_workspace_bytes(const hta_config* cfg);

/* Bind caller-owned device memory of at least hta_workspace_bytes(cfg) bytes,
 * 256-byte aligned.  The library never frees it. */
int hta_bind_workspace(hta_ctx* ctx, void* dev_ptr, size_t bytes);

/* Load weights from device tensors in the fixed order: e_text [Vt][d],
 * e_aud [C][V][d], then per layer g_attn [d], wq [Hq*hd][d], wk [Hkv*hd][d],
 * wv [Hkv*hd][d], g_q [hd], g_k [hd], wo [d][Hq*hd], g_mlp [d], wg [F][d],
 * wu [F][d], wd [d][F]; then g_final [d], w_head [C*V][d]; all row-major,
 * src_dtype elements (hta_src_dtype).  n_tensors must be 4 + 11*n_layers.
 * BF16 contexts store projections, embeddings and head in bfloat16 (RNE);
 * FP8 contexts store projections and head as e4m3 codes with per-row scales
 * max|row| / 448 (FlashRT page, section 8 and its FP8 notes), embeddings in
 * bfloat16.  act_scales (host, FP8 only, else NULL): 4*n_layers+1 static
 * activation scales in site order (per layer: attention input, attention
 * output, MLP input, down input; then the head input).  The source tensors
 * may be freed after the call returns. */
int hta_load_weights(hta_ctx* ctx, const void* const* dev_tensors, int n_tensors, int src_dtype,
                     const float* act_scales);

/* Append a prompt of P text tokens (host int32) at positions len .. len+P-1 in
 * one batched pass that writes the KV cache (FlashRT page, section 7); no head
 * is evaluated.  Errors: HTA_E_RANGE for an id outside [0, text_vocab),
 * HTA_E_CAPACITY if len + P > max_seq or P > max_prefill. */
int hta_prefill(hta_ctx* ctx, const int32_t* tokens, int P);

/* One projection of the prefill on its own (FlashRT page, section 5: the W8A8 / BF16
 * projections of the layer chain; the prefill runs them as batched GEMMs), with the
 * kernels, tile shapes and K split that hta_prefill uses for the same (M, N, K):
 * C[m][n] = sum over k of A[m][k] * W[n][k], products exact and summed in fp32 in
 * 128-element steps of increasing k (split partials added in order), so a row's result
 * does not depend on M.  FP8 context: A [M][K] and W [N][K] are e4m3 codes, the sum is
 * multiplied by a_scale * w_scale[n] (w_scale: float32 [N]).  BF16 context: A and W are
 * bf16 bits; w_scale and a_scale are ignored (w_scale may be NULL).  C: float32 [M][N].
 * All arrays are row-major device memory owned by the caller; the call uses the
 * context's split-partial scratch, runs on its stream and returns once C is written.
 * Limits (HTA_E_ARG otherwise): 1 <= M <= max_prefill; N a multiple of 64, at most the
 * widest projection (q + 2 kv widths, 2 ffn or hidden); K a positive multiple of 128;
 * max(M, N) * K operand bytes below 2 GiB.  HTA_E_STATE without a bound workspace. */
int hta_gemm(hta_ctx* ctx, const void* A, const void* W, const float* w_scale, float a_scale, int M, int N, int K,
             float* C);

/* One decode frame (FlashRT page, section 5): embed the previous codes (all
 * BOS for the first frame), run the backbone at position len, the fused head,
 * the greedy argmax under the delay pattern (lowest id on ties; a NaN logit
 * never wins, so a code is always a valid id); write the 8 delayed codes of this
 * step to codes_out (host).  Returns HTA_OK, or HTA_DONE when this step
 * completed the utterance; later calls keep returning all-EOS frames with the
 * same work.  HTA_E_CAPACITY when len == max_seq. */
int hta_decode_frame(hta_ctx* ctx, int32_t* codes_out);

/* n decode frames back to back with one device-to-host copy at the end;
 * codes_out (host) receives n*C codes; *n_done (may be NULL) receives the
 * number of steps that ended in the done state. */
int hta_decode_frames(hta_ctx* ctx, int n, int32_t* codes_out, int* n_done);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): hta_decode_frames with the same arguments, results
 * and errors, allocating nothing.  The decode frame kernel's exchange words (tagged
 * residual, q/k/v, attention output and partials, SiLU*mul output, logits) and its launch
 * counter / abort flag live in a static device array of the library, 2 MiB per GPU, held
 * until the process ends, instead of the workspace; each call first clears the part its
 * shape uses, then launches the kernel directly (no graph is instantiated).  Every context
 * on one GPU shares that array: calls that overlap in time on one GPU (two streams, two
 * threads) race and must be serialised by the caller.  HTA_E_CAPACITY when the shape's
 * exchange words exceed the array (no shape hta_create accepts on a 256-CU device does);
 * HTA_E_TIMEOUT as for hta_decode_frames. */
int hta_decode_frames_noalloc(hta_ctx* ctx, int n, int32_t* codes_out, int* n_done);

/* Decode policy of the head (FlashRT page, section 4 "Sampling policy", section 5 and
 * section 8 "Decode policy"): temperature 0 (the default) is the greedy argmax;
 * temperature > 0 replaces the argmax of every codebook not forced by the delay rule with
 * a categorical draw: weights exp((z_i - m) / temperature) over the codebook's allowed ids
 * (the greedy path's set; NaN logits weigh nothing), m their largest fp32 logit, and the
 * first id (in id order) whose running weight exceeds u times the total.  u is a uniform
 * in [0, 1): the top 24 bits of word 0 of Philox4x32-10 (Salmon et al., SC'11) keyed by
 * `seed` (low 32 bits first) at counter (step t of the utterance, codebook k, 0, 0), so a
 * fixed seed repeats the same draws.  The draw runs in the frame kernel's head epilogue,
 * in the same launch and graph as the argmax; no top-p or top-k.  Holds until changed;
 * hta_calibrate always runs greedy.  HTA_E_ARG for a negative or non-finite temperature;
 * HTA_E_UNSUPPORTED when n_codebooks * codebook_size fp32 logits exceed 120 KiB. */
int hta_set_sampling(hta_ctx* ctx, float temperature, uint64_t seed);

/* Start a new utterance: keep the KV of positions [0, keep_len) (prefix reuse,
 * FlashRT page, section 4) and reset the delay state.  keep_len = 0 is a cold
 * start; keep_len must not exceed the current length. */
int hta_reset(hta_ctx* ctx, int keep_len);

/* Batched contexts: make stream m (0 <= m < n_streams) the one that the per-stream calls
 * act on (stream 0 after hta_create).  HTA_E_ARG for m out of range. */
int hta_select_stream(hta_ctx* ctx, int m);

/* Teacher forcing: the next frame embeds codes_in (host, C codes each in
 * [0, codebook_size)) instead of the last chosen codes; the EOC bookkeeping
 * follows the forced code of codebook 0. */
int hta_force_codes(hta_ctx* ctx, const int32_t* codes_in);

/* Read device state for tests: tap HTA_TAP_HIDDEN -> float32 [d] final
 * residual of the last frame; HTA_TAP_LOGITS -> float32 [C*V] raw logits of the
 * last frame; HTA_TAP_STATE -> int32 [4 + 2*C] {len, t, eoc, done, prev[C],
 * codes[C]}; HTA_TAP_KV -> bf16 bits [2][Hkv][n][hd] of layer `layer`, n = the
 * number of positions the buffer holds (bytes / (4*Hkv*hd), at most max_seq);
 * HTA_TAP_AMAX -> float32 [4L+1] recorded activation maxima; HTA_TAP_PREFILL_HIDDEN
 * -> float32 [P][d] residual after the last layer of the last prefill;
 * HTA_TAP_W_QKV -> packed q/k/v rows of `layer` ([Hq*hd + 2*Hkv*hd][d], bf16 bits
 * or e4m3 codes); HTA_TAP_S_QKV -> their float32 FP8 row scales;
 * HTA_TAP_W_GU / HTA_TAP_S_GU -> the packed gate/up rows (interleaved
 * gate_0, up_0, gate_1, ...) and scales.  With HTA_OPT_TAPS on:
 * HTA_TAP_LAYER_H -> float32 [n_layers + 1][d], the residual entering each
 * layer of the last decode frame and, last, the final residual;
 * HTA_TAP_PREFILL_LAYER -> float32 [2][P][d], the rows entering and leaving
 * layer HTA_OPT_PREFILL_TAP_LAYER in the last prefill (HTA_E_STATE when the
 * taps are off).  With HTA_OPT_TRACE on, HTA_TAP_TRACE -> uint32
 * [blocks][5 * n_layers + 1][8]: for every block of the persistent frame kernel
 * and every phase of the last frame (per layer: qkv, attention, o_proj,
 * gate/up, down; then the head), the low 32 bits of the 100 MHz constant clock
 * at phase start, inputs ready, weights streamed and phase done, then for the
 * block's first wave: weight packets consumed and row sums closed in the
 * phase, then the clock when the first wave's polls of the phase input were
 * satisfied and when every wave's were (zero where a phase has no polled
 * input; attention phases leave both as they were) (blocks = one per compute unit;
 * entries of phases a block skips are left as they were).
 * With HTA_OPT_TAPS on, HTA_TAP_ACT -> uint16 [5 * n_layers + 1][10240]: for every
 * GEMV phase of the last decode frame (per layer qkv, -, o_proj, gate/up, down; then the
 * head), the input vector the phase multiplies with, as bf16 bits of the rounded values
 * (BF16) or of the e4m3 code values (FP8; every e4m3 value is exact in bf16), in the
 * first hidden / q width / ffn entries of its row (attention rows unused); HTA_TAP_Q ->
 * uint16 [n_layers][Hq][hd]: the bf16 bits of the queries after q-norm and RoPE that the
 * last frame's attention used.
 * A buffer smaller than the tap gives HTA_E_ARG. */
enum { HTA_TAP_HIDDEN = 0, HTA_TAP_LOGITS = 1, HTA_TAP_STATE = 2, HTA_TAP_KV = 3, HTA_TAP_AMAX = 4,
       HTA_TAP_PREFILL_HIDDEN = 5, HTA_TAP_W_QKV = 6, HTA_TAP_S_QKV = 7, HTA_TAP_W_GU = 8, HTA_TAP_S_GU = 9,
       HTA_TAP_LAYER_H = 10, HTA_TAP_PREFILL_LAYER = 11, HTA_TAP_TRACE = 12, HTA_TAP_ACT = 13, HTA_TAP_Q = 14 };
int hta_read_tap(hta_ctx* ctx, int tap, int layer, void* host_out, size_t bytes);

/* FP8 calibration on a BF16 context (FlashRT page, section 8: a short BF16
 * free run of a fixed prompt, scale = amax / 448): reset, prefill the P
 * calibration tokens, decode n_frames frames with the decode frame kernel (fed
 * with forced_codes [n_frames][C] when not NULL, else greedy), recording max |x|
 * at every activation site before its rounding; writes 4*n_layers+1 scales
 * (host) and leaves the context reset to length 0. */
int hta_calibrate(hta_ctx* ctx, const int32_t* tokens, int P, int n_frames, const int32_t* forced_codes,
                  float* scales_out);

/* One decoder layer (the one-layer configuration of the benchmark): on a context with
 * n_layers == 1 (layer must be 0, else HTA_E_UNSUPPORTED), fill the KV cache's positions
 * [0, kv_len - 1) from k_init/v_init (device bf16 [Hkv][kv_len-1][hd], NULL to keep the
 * cache), then run one frame of the decode frame kernel at position kv_len - 1 with
 * h_io (device float32 [d]) as its input in place of the codebook embedding sum, and
 * write the residual leaving the layer back to h_io.  The new key and value land in
 * slot kv_len - 1; the context is left at length kv_len, one step into an utterance. */
int hta_layer_step(hta_ctx* ctx, int layer, int kv_len, const void* k_init, const void* v_init, void* h_io);

/* Un-delay (host only): frames[f][k] = step_codes[f+k][k] for f < n, with
 * n = EOC step if codebook 0 emitted EOS, else T - (C - 1); frames_out needs
 * room for T*C codes; *n_frames receives n. */
int hta_undelay(const int32_t* step_codes, int T, int n_codebooks, int eos_id, int32_t* frames_out, int* n_frames);

/* Streaming hand-off of one utterance (host only; FlashRT page, section 4: a streaming
 * generator whose output equals the one-shot output; Performance section: a deterministic
 * repeated-code stop guard ends runs that never emit EOC before the generation cap).
 * The caller pushes the delayed step codes as it decodes them; the stream un-delays them
 * (frame f is complete once step f + C - 1 is in; with EOC at step e the frames are
 * 0..e-1) and hands out complete frames in whole chunks of chunk_frames while the
 * utterance runs, and all remaining complete frames once it has ended.  The frames handed
 * out, concatenated, equal hta_undelay of every pushed step.
 * Stop guard (the page gives no rule; this reading): after frame f completes, if the
 * last guard_window frames repeat with a period p <= guard_max_period (frame g equals
 * frame g - p for every g of the window after its first p), the stream stops with frames
 * 0..f; guard_window 0 disables it.  Steps pushed after the end are ignored. */
typedef struct hta_stream hta_stream;
enum { HTA_STREAM_RUNNING = 0, HTA_STREAM_DONE = 1, HTA_STREAM_STOPPED = 2, HTA_STREAM_CAPPED = 3 };
/* HTA_E_ARG for n_codebooks outside 1..64, chunk_frames < 1 or negative guard values. */
int hta_stream_create(int n_codebooks, int bos_id, int eos_id, int chunk_frames, int guard_window,
                      int guard_max_period, hta_stream** out);
/* Push n_steps steps (host int32 [n_steps][C]); writes up to max_frames frames (host int32
 * [max_frames][C]) to frames_out and their count to *n_frames; frames beyond max_frames stay
 * queued for the next call (push 0 steps to drain).  *status (may be NULL) receives
 * HTA_STREAM_RUNNING, _DONE (EOC: every frame before it is complete) or _STOPPED (guard). */
int hta_stream_push(hta_stream* s, const int32_t* step_codes, int n_steps, int32_t* frames_out, int max_frames,
                    int* n_frames, int* status);
/* The caller ends a running utterance (its generation cap): the stream becomes
 * HTA_STREAM_CAPPED and hands out every remaining complete frame. */
int hta_stream_finish(hta_stream* s, int32_t* frames_out, int max_frames, int* n_frames);
void hta_stream_destroy(hta_stream* s);

/* Kernel timing for the benchmark: decode n_frames frames, each one launch of the
 * decode frame kernel bracketed by a HIP event pair on the context's stream;
 * avg_us_out (host, n_classes floats) receives the average device time per launch
 * at index HTA_K_FRAME and zero for the other classes (kept for the ABI).  The
 * frames are real decode steps (the state advances). */
enum { HTA_K_EMBED = 0, HTA_K_QKV = 1, HTA_K_ATTN = 2, HTA_K_O = 3, HTA_K_GATEUP = 4, HTA_K_DOWN = 5, HTA_K_HEAD = 6,
       HTA_K_FRAME = 7, HTA_K_COUNT = 8 };
int hta_time_kernels(hta_ctx* ctx, int n_frames, float* avg_us_out, int n_classes);

/* Options: HTA_OPT_USE_GRAPH (default 1) replays the captured position-agnostic
 * frame graph (runs of eight frames replay a graph of eight launches); 0 launches the
 * frame kernel directly (for tests that compare the two).  Every frame is one launch of the persistent decode frame kernel (one
 * resident block per compute unit; blocks hand values to each other through
 * phase-tagged words, no grid barrier; a wait that runs out ends the frame with
 * HTA_E_TIMEOUT).  HTA_OPT_TAPS (default 0) makes decode frames and prefills also
 * write the per-layer residuals and GEMV inputs read by HTA_TAP_LAYER_H,
 * HTA_TAP_ACT and HTA_TAP_PREFILL_LAYER (frames then launch without the graph);
 * HTA_OPT_PREFILL_TAP_LAYER selects the prefill layer (0..n_layers-1, else
 * HTA_E_ARG).  HTA_OPT_TRACE (default 0) records the frame kernel's phase
 * timestamps (HTA_TAP_TRACE).  HTA_OPT_FORCE_TIMEOUT (default 0; for tests of the
 * recovery path) makes every frame's first input wait for a tag no block writes: the
 * bounded wait runs out (0.5 s), every block leaves the kernel, and the decode call
 * returns HTA_E_TIMEOUT with the exchange words cleared; after setting it back to 0,
 * hta_reset starts a clean utterance.  HTA_OPT_FP8_MFMA (default 0; FP8 contexts only,
 * HTA_E_UNSUPPORTED on BF16) multiplies the e4m3 GEMMs of hta_prefill, hta_gemm and
 * the batched step on the e4m3 MFMA instead of widening the codes to bf16: faster, but
 * the instruction sums its products with fewer bits than fp32 (a product 2^-18 beside a
 * product 1 is lost), so results differ from the fp32 sums by up to about 2^-19 of the
 * sum of |products|, short of the fp32 accumulation this library reads into the FP8
 * path (FlashRT page, section 8 names e4m3 W8A8 GEMMs and no accumulation width).  Rows
 * stay independent of M.  Value 1 is unused. */
enum { HTA_OPT_USE_GRAPH = 0, HTA_OPT_TAPS = 2, HTA_OPT_PREFILL_TAP_LAYER = 3, HTA_OPT_TRACE = 4,
       HTA_OPT_FORCE_TIMEOUT = 5, HTA_OPT_FP8_MFMA = 6 };
int hta_set_option(hta_ctx* ctx, int option, int value);

void hta_destroy(hta_ctx* ctx);
const char* hta_last_error(const hta_ctx* ctx);
const char* hta_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HTA_H */
