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
  // prefill scratch
  size_t off_tok, off_x, off_u, off_pqkv, off_pq, off_po, off_pgu, off_pa;
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
  DevState* h_state = nullptr;  // pinned host staging
  int32_t* h_stage = nullptr;   // pinned host staging for tokens / codes
  size_t h_stage_elems = 0;
  std::string err;
  std::vector<float> h_scales;  // host copy of the activation scales (FP8)
  bool use_graph = true;
  bool own_stream = false;
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
  int32_t* tok = nullptr;       // [max_prefill]
  float* px = nullptr;          // [Pmax][d]
  void* pu = nullptr;           // [Pmax][max(d, qd, F)] act
  float* pqkv = nullptr;        // [Pmax][qd + 2kvd]
  float* pq = nullptr;          // [Pmax][qd] rotated q (bf16-rounded values)
  void* po = nullptr;           // [Pmax][qd] act
  float* pgu = nullptr;         // [Pmax][2F]
  int last_prefill_P = 0;
};

// ---------------------------------------------------------------- launchers (decode.hip)
hipError_t launch_frame_begin(Ctx& c);
hipError_t launch_layer_decode(Ctx& c, int layer, float* h, bool record);
hipError_t launch_layer_decode_at(Ctx& c, int layer, float* h, bool record, int pos_override);
hipError_t launch_head(Ctx& c, bool record);
hipError_t launch_set_prev(Ctx& c, const int32_t* codes);
hipError_t launch_reset_state(Ctx& c, int keep_len);
hipError_t launch_set_len(Ctx& c, int len);

// ---------------------------------------------------------------- launchers (prefill.hip)
hipError_t launch_prefill(Ctx& c, int P, bool record);

// ---------------------------------------------------------------- launchers (load.hip)
hipError_t launch_pack_rows(void* dst, int dst_row0, int dst_row_stride, const void* src, int src_dtype,
                            int rows, int cols, int to_fp8, float* scales, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const void* src, int src_dtype, size_t n, hipStream_t s);
hipError_t launch_fill_u32(void* dst, uint32_t v, size_t n, hipStream_t s);
hipError_t launch_kv_init(uint16_t* k_cache, uint16_t* v_cache, const void* k_init, const void* v_init,
                          int n_kv, int n, int max_seq, int hd, hipStream_t s);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace hta
