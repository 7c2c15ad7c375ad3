// Host-side internals: workspace layout, context, kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>
#include <vector>

#include "../../include/hta.h"

namespace hta {

constexpr int kSitesPerLayer = 4;   // attention input, attention output, MLP input, down input
constexpr int kAttnTile = 64;       // keys per attention tile (aligned to absolute positions)
constexpr int kMaxCodebooks = 16;
constexpr int kTraceBlocks = 1024;  // most blocks the persistent kernel's trace records
constexpr size_t kFrameArgsBytes = 1024;  // device slot of the persistent kernel's arguments
constexpr int kActsWidth = 10240;   // widest GEMV input (hidden <= 5120, q width and ffn <= 10240)

// Decode state kept on the device (one per context).
struct DevState {
  int len;    // KV length = position of the next token
  int t;      // decode step within the utterance
  int eoc;    // step at which codebook 0 emitted EOS, -1 if none yet
  int done;   // 1 once the last step completed the utterance
  int prev[kMaxCodebooks];   // codes fed into the next frame
  int codes[kMaxCodebooks];  // codes chosen by the last frame
  int n_done;                // number of steps that ended done (for batched decode)
  int pad[7];
};

// Device pointers of one layer's packed weights.
struct LayerW {
  void* w_qkv;   // [qd + 2 kvd][d]  bf16 or e4m3
  void* w_o;     // [d][qd]
  void* w_gu;    // [2F][d], rows interleaved gate_0, up_0, gate_1, up_1, ...
  void* w_d;     // [d][F]
  float* s_qkv;  // FP8 per-row scales (null for BF16)
  float* s_o;
  float* s_gu;
  float* s_d;
  float* g_attn;  // [d] fp32
  float* g_q;     // [hd]
  float* g_k;     // [hd]
  float* g_mlp;   // [d]
  uint16_t* k_cache;  // [Hkv][max_seq][hd] bf16
  uint16_t* v_cache;
};

struct Layout {
  size_t total = 0;
  // offsets (bytes) of every region
  size_t layer_base, layer_stride;
  size_t off_wqkv, off_wo, off_wgu, off_wd, off_sqkv, off_so, off_sgu, off_sd;
  size_t off_gattn, off_gq, off_gk, off_gmlp, off_k, off_v;
  size_t off_etext, off_eaud, off_gfinal, off_whead, off_shead;
  size_t off_rope_cos, off_rope_sin, off_act_scales, off_amax;
  size_t off_state, off_hist, off_counters;
  size_t off_h, off_qkv, off_attn_part, off_o_act, off_a_act, off_logits;
  size_t off_layer_table, off_xh, off_xqkv, off_xo, off_xa, off_xpart, off_xlogits, off_sync;
  // prefill scratch
  size_t off_tok, off_x, off_u, off_pqkv, off_pq, off_po, off_pgu, off_pa;
  size_t off_taps, off_ptaps, off_tact, off_tq, off_trace, off_fargs, off_fargs_s;
  // batched decode: logits [M][CVp] and attention split partials [M][Hq][splits][hd + 2]
  size_t off_blogits, off_bpart;
  size_t kv_stream_bytes;   // bytes of one stream's K (or V) cache within a layer
  int cv_pad;               // head rows padded to a multiple of 64 (the GEMM's column tile)
  int gemm_cols;            // widest GEMM output the split partials hold (8 splits of max_prefill rows)
  int n_streams, batch_splits;
  int attn_splits;
};

Layout make_layout(const hta_config& c);

struct Ctx {
  hta_config cfg;
  Layout lay;
  hipStream_t stream = nullptr;
  int device = 0;
  char* ws = nullptr;  // bound workspace
  bool weights_loaded = false;
  int len = 0;         // host mirror of DevState::len
  int t = 0;           // host mirror of DevState::t
  bool done = false;
  hipGraph_t frame_graph = nullptr;
  hipGraphExec_t frame_exec = nullptr;
  hipGraph_t frame_graph8 = nullptr;   // eight frame launches in one graph (replayed for runs of 8)
  hipGraphExec_t frame_exec8 = nullptr;
  DevState* h_state = nullptr;  // pinned host staging
  int32_t* h_stage = nullptr;   // pinned host staging for tokens / codes
  size_t h_stage_elems = 0;
  std::string err;
  std::vector<float> h_scales;  // host copy of the activation scales (FP8)
  bool use_graph = true;
  // per-kernel timing: when set, launchers bracket each kernel with events from this pool
  hipEvent_t* tev = nullptr;
  int tev_next = 0, tev_cap = 0;
  int* tev_class = nullptr;
  bool own_stream = false;
  bool frame_ok = false;      // the persistent frame kernel fits this device and shape
  const float* frame_h_in = nullptr;  // frame input override (one-layer steps), or null
  bool frame_record = false;  // the frame records activation maxima (calibration)
  int frame_blocks = 0, frame_splits = 0;
  int num_cus = 256;          // compute units of the device (prefill block-width choice)
  // derived device pointers
  LayerW* layers = nullptr;  // host array of n_layers
  uint16_t* e_text = nullptr;
  uint16_t* e_aud = nullptr;
  float* g_final = nullptr;
  void* w_head = nullptr;
  float* s_head = nullptr;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  float* act_scales = nullptr;  // [4L+1]
  float* amax = nullptr;        // [4L+1]
  DevState* state = nullptr;
  int32_t* hist = nullptr;      // [max_seq][C]
  unsigned* counters = nullptr; // [64]
  float* h = nullptr;           // [d]
  float* qkv = nullptr;         // [qd + 2kvd]
  float* attn_part = nullptr;   // [Hq][splits][hd + 2]
  void* o_act = nullptr;        // [qd]
  void* a_act = nullptr;        // [F]
  float* logits = nullptr;      // [C*V]
  LayerW* d_layers = nullptr;   // device copy of `layers`
  // persistent kernel exchange words (value + phase tag)
  uint64_t* x_h = nullptr;      // [d]
  uint64_t* x_qkv = nullptr;    // [qd + 2kvd]
  uint32_t* x_o = nullptr;      // [qd]
  uint32_t* x_a = nullptr;      // [F]
  uint64_t* x_part = nullptr;   // [Hq][64][hd + 2]
  uint64_t* x_logits = nullptr; // [C*V]
  unsigned* sync = nullptr;     // [0] launch count, [64] abort flag
  int32_t* tok = nullptr;       // [max_prefill]
  float* px = nullptr;          // [Pmax][d]
  void* pu = nullptr;           // [Pmax][max(d, qd, F)] act
  float* pqkv = nullptr;        // [Pmax][qd + 2kvd]
  float* pq = nullptr;          // [Pmax][qd] rotated q (bf16-rounded values)
  void* po = nullptr;           // [Pmax][qd] act
  float* pgu = nullptr;         // [Pmax][2F]
  void* pa = nullptr;           // [Pmax][F] SiLU * mul rows (act)
  int last_prefill_P = 0;
  // test taps: the residual entering every layer of each decode frame (and the final one),
  // and the rows entering / leaving layer prefill_tap_layer of each prefill
  bool taps = false;
  int prefill_tap_layer = 0;
  float* taps_h = nullptr;      // [n_layers + 1][d]
  float* taps_p = nullptr;      // [2][Pmax][d]
  uint16_t* taps_act = nullptr; // [5 * n_layers + 1][kActsWidth] GEMV inputs of the last frame (block 0)
  uint16_t* taps_q = nullptr;   // [n_layers][Hq * hd] rotated queries of the last frame
  bool trace = false;           // persistent frame kernel phase timestamps
  bool fp8_mfma = false;        // e4m3 prefill and batched-step GEMMs on the e4m3 MFMA (opt-in)
  uint32_t* trace_buf = nullptr;  // [kTraceBlocks][5 * n_layers + 1][4]
  void* fargs = nullptr;          // the persistent kernel's arguments (device)
  // captured prefills, one per prompt length P (positions come from the device state)
  struct PrefillGraph { int P; int stream; hipGraphExec_t exec; };  // (prompt length, stream)
  std::vector<PrefillGraph> prefill_graphs;
  // hta_decode_frames_noalloc: the frame kernel's exchange words in the library's static
  // per-device array (its address on this context's device) instead of the workspace
  char* scratch_dev = nullptr;
  size_t static_exch_bytes = 0;   // bytes of that array this shape's exchange words take
  void* fargs_s = nullptr;        // kernel arguments pointing at it (device)
  unsigned* h_status = nullptr;   // pinned host word: the abort flag read back after a decode
  // batched decode (n_streams > 1): the selected stream's state / history / caches are
  // what `state`, `hist` and layers[].k_cache / v_cache point at; the others' host-side
  // lengths and steps are kept here
  int sel = 0;
  std::vector<int> s_len, s_t;
  std::vector<char> s_done;
  DevState* state_base = nullptr;
  int32_t* hist_base = nullptr;
  std::vector<uint16_t*> k_base, v_base;   // stream 0's cache of each layer
  hipGraph_t batch_graph = nullptr;
  hipGraphExec_t batch_exec = nullptr;
  float* b_logits = nullptr;
  float* b_part = nullptr;
  float temperature = 0.0f;       // 0: greedy; > 0: the head draws at this temperature
  bool force_timeout = false;     // frames wait for an input no block writes (recovery tests)
  uint64_t seed = 0;              // the draw's seed
};

// Event pair around one kernel launch when per-kernel timing is on (kernel class k).
inline void time_begin(Ctx& c, int k) {
  if (c.tev && c.tev_next + 2 <= c.tev_cap) {
    c.tev_class[c.tev_next / 2] = k;
    (void)hipEventRecord(c.tev[c.tev_next], c.stream);
  }
}
inline void time_end(Ctx& c) {
  if (c.tev && c.tev_next + 2 <= c.tev_cap) {
    (void)hipEventRecord(c.tev[c.tev_next + 1], c.stream);
    c.tev_next += 2;
  }
}

// ---------------------------------------------------------------- decode state (load.hip)
hipError_t launch_set_prev(Ctx& c, const int32_t* codes);
hipError_t launch_reset_state(Ctx& c, int keep_len);
hipError_t launch_set_len(Ctx& c, int len);

// ---------------------------------------------------------------- persistent frame (frame.hip)
hipError_t frame_setup(Ctx& c);
hipError_t launch_frame_persistent(Ctx& c);
hipError_t launch_frame_args(Ctx& c, void* fargs);  // the same kernel with another argument slot
hipError_t frame_write_args(Ctx& c);
int frame_max_packets(const hta_config& f, int blocks);
int frame_part_capacity();
size_t frame_sample_capacity();  // bytes of LDS that hold a sampling frame's logits

// ---------------------------------------------------------------- launchers (prefill.hip)
hipError_t prefill_setup();  // kernel attributes of the prefill GEMM (once per context)
hipError_t launch_prefill(Ctx& c, int P, bool record);
// C[M][N] = A[M][K] . W[N][K]^T with the prefill's kernels and K split (e4m3: times a_scale * w_scale[n])
hipError_t launch_gemm(Ctx& c, const void* A, const void* W, const float* w_scale, float a_scale, float* C, int M,
                       int N, int K);
hipError_t launch_batch_step(Ctx& c);  // one batched decode step of all n_streams streams

// ---------------------------------------------------------------- launchers (load.hip)
hipError_t launch_pack_rows(void* dst, int dst_row0, int dst_row_stride, const void* src, int src_dtype,
                            int rows, int cols, int to_fp8, float* scales, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const void* src, int src_dtype, size_t n, hipStream_t s);
hipError_t launch_fill_u32(void* dst, uint32_t v, size_t n, hipStream_t s);
hipError_t launch_kv_init(uint16_t* k_cache, uint16_t* v_cache, const void* k_init, const void* v_init,
                          int n_kv, int n, int max_seq, int hd, hipStream_t s);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The frame kernel's tagged exchange words and launch counter / abort flag laid out from
// `base`: residual, q/k/v, attention output, SiLU*mul output, attention partials (for the
// kernel's split count), logits, then 1024 words of sync.  Returns the bytes taken.
struct Exchange {
  uint64_t* xh; uint64_t* xqkv; uint32_t* xo; uint32_t* xa; uint64_t* xpart; uint64_t* xlogits;
  unsigned* sync;
};
inline size_t exchange_layout(const hta_config& f, int splits, char* base, Exchange* x) {
  const size_t d = f.hidden, hd = f.head_dim, qd = (size_t)f.n_q_heads * hd, W = qd + 2 * (size_t)f.n_kv_heads * hd;
  const size_t CV = (size_t)f.n_codebooks * f.codebook_size;
  size_t o = 0;
  auto take = [&](size_t bytes) { char* r = base + o; o = align256(o + bytes); return r; };
  char* xh = take(d * 8);
  char* xqkv = take(W * 8);
  char* xo = take(qd * 4);
  char* xa = take((size_t)f.ffn * 4);
  char* xpart = take((size_t)f.n_q_heads * splits * (hd + 2) * 8);
  char* xlogits = take(CV * 8);
  char* sync = take(1024 * 4);
  if (x) {
    x->xh = reinterpret_cast<uint64_t*>(xh); x->xqkv = reinterpret_cast<uint64_t*>(xqkv);
    x->xo = reinterpret_cast<uint32_t*>(xo); x->xa = reinterpret_cast<uint32_t*>(xa);
    x->xpart = reinterpret_cast<uint64_t*>(xpart); x->xlogits = reinterpret_cast<uint64_t*>(xlogits);
    x->sync = reinterpret_cast<unsigned*>(sync);
  }
  return o;
}

}  // namespace hta
