// Host runtime behind the C ABI (include/hta.h): workspace layout, weight
// packing, the position-agnostic frame graph, prefill, calibration and taps.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "hta_internal.h"

using namespace hta;

struct hta_ctx {
  Ctx c;
};

// Exchange words of hta_decode_frames_noalloc: one array per GPU, held until the process
// ends and shared by every context on that GPU (overlapping calls on one GPU race).  2 MiB
// covers every shape hta_create accepts at 256 frame blocks: at most 1 MiB of attention
// partials (n_q_heads * splits <= 1024 rows of head_dim + 2 words), 256 KiB of logits and
// under 256 KiB for the rest.
constexpr size_t kStaticScratchBytes = 2u << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch` on each GPU, once looked up

// The array's device address on the current device (`device`), looked up once per device.
// The host-side name `scratch` is only a handle for the lookup, never a device address.
hipError_t static_scratch(int device, char** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[device] = static_cast<char*>(p);
  }
  *out = g_scratch_dev[device];
  return hipSuccess;
}
}  // namespace

namespace hta {

float host_act_scale(const Ctx& c, int site) {
  if (c.cfg.precision != HTA_FP8_E4M3) return 1.0f;
  return c.h_scales.empty() ? 1.0f : c.h_scales[site];
}

static int wbytes(const hta_config& c) { return c.precision == HTA_FP8_E4M3 ? 1 : 2; }

Layout make_layout(const hta_config& c) {
  Layout L{};
  const size_t d = c.hidden, hd = c.head_dim, qd = (size_t)c.n_q_heads * hd, kvd = (size_t)c.n_kv_heads * hd;
  const size_t F = c.ffn, W = qd + 2 * kvd, wb = wbytes(c), ms = c.max_seq, Pm = c.max_prefill;
  const size_t CV = (size_t)c.n_codebooks * c.codebook_size;
  const bool fp8 = c.precision == HTA_FP8_E4M3;
  const size_t M = c.n_streams > 1 ? (size_t)c.n_streams : 1;
  const size_t CVp = (CV + 63) / 64 * 64;  // head rows padded for the batched step's GEMM tiles
  L.cv_pad = (int)CVp;
  L.n_streams = (int)M;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  // one layer block
  size_t lo = 0;
  auto ltake = [&](size_t bytes) { size_t r = lo; lo = align256(lo + bytes); return r; };
  L.off_wqkv = ltake(W * d * wb);
  L.off_wo = ltake(d * qd * wb);
  L.off_wgu = ltake(2 * F * d * wb);
  L.off_wd = ltake(d * F * wb);
  L.off_sqkv = ltake(fp8 ? W * 4 : 0);
  L.off_so = ltake(fp8 ? d * 4 : 0);
  L.off_sgu = ltake(fp8 ? 2 * F * 4 : 0);
  L.off_sd = ltake(fp8 ? d * 4 : 0);
  L.off_gattn = ltake(d * 4);
  L.off_gq = ltake(hd * 4);
  L.off_gk = ltake(hd * 4);
  L.off_gmlp = ltake(d * 4);
  L.kv_stream_bytes = (size_t)c.n_kv_heads * ms * hd * 2;
  L.off_k = ltake(M * L.kv_stream_bytes);  // stream m's cache at + m * kv_stream_bytes
  L.off_v = ltake(M * L.kv_stream_bytes);
  L.layer_stride = lo;
  L.layer_base = take(lo * c.n_layers);
  L.off_etext = take((size_t)c.text_vocab * d * 2);
  L.off_eaud = take(CV * d * 2);
  L.off_gfinal = take(d * 4);
  L.off_whead = take(CVp * d * wb);
  L.off_shead = take(fp8 ? CVp * 4 : 0);
  L.off_rope_cos = take(ms * (hd / 2) * 4);
  L.off_rope_sin = take(ms * (hd / 2) * 4);
  const size_t nsites = (size_t)kSitesPerLayer * c.n_layers + 1;
  L.off_act_scales = take(nsites * 4);
  L.off_amax = take(nsites * 4);
  L.off_state = take(M * sizeof(DevState));
  L.off_hist = take(M * ms * c.n_codebooks * 4);
  L.off_counters = take(64 * 4);
  int splits = 256 / c.n_kv_heads;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  L.attn_splits = splits;
  const int part_splits = 64;  // the persistent kernel may use up to 64 splits
  L.off_h = take(d * 4);
  L.off_qkv = take(W * 4);
  L.off_attn_part = take((size_t)c.n_q_heads * part_splits * (hd + 2) * 4);
  L.off_o_act = take(qd * 2);
  L.off_a_act = take(F * 2);
  L.off_logits = take(CV * 4);
  L.off_layer_table = take((size_t)c.n_layers * sizeof(LayerW));
  L.off_xh = take(d * 8);
  L.off_xqkv = take(W * 8);
  L.off_xo = take(qd * 4);
  L.off_xa = take(F * 4);
  L.off_xpart = take((size_t)c.n_q_heads * part_splits * (hd + 2) * 8);
  L.off_xlogits = take(CV * 8);
  L.off_sync = take(1024 * 4);
  L.off_tok = take(Pm * 4);
  L.off_x = take(Pm * d * 4);
  L.off_u = take(Pm * (d > F ? d : F) * 2);
  L.off_pqkv = take(Pm * W * 4);
  L.off_pq = take(Pm * qd * 4);
  L.off_po = take(Pm * qd * 2);
  size_t nmax = W;
  if (2 * F > nmax) nmax = 2 * F;
  if (d > nmax) nmax = d;
  if (M > 1 && CVp > nmax) nmax = CVp;  // the batched step's head GEMM
  L.off_pgu = take(Pm * 2 * F * 4 + 8 * Pm * nmax * 4);  // gate/up rows, then GEMM split partials
  L.gemm_cols = (int)nmax;
  L.off_pa = take(Pm * F * 2);  // SiLU * mul rows (the down projection's input)
  L.off_taps = take(((size_t)c.n_layers + 1) * d * 4);
  L.off_ptaps = take(2 * Pm * d * 4);
  L.off_tact = take((5 * (size_t)c.n_layers + 1) * kActsWidth * 2);
  L.off_tq = take((size_t)c.n_layers * qd * 2);
  L.off_trace = take((size_t)kTraceBlocks * (5 * c.n_layers + 1) * 8 * 4);
  L.off_fargs = take(kFrameArgsBytes);
  L.off_fargs_s = take(kFrameArgsBytes);
  {
    int S = M > 1 ? (int)(256 / ((size_t)c.n_kv_heads * M)) : 1;  // about one block per CU
    L.batch_splits = S < 1 ? 1 : (S > 16 ? 16 : S);
  }
  L.off_blogits = take(M > 1 ? M * CVp * 4 : 0);
  L.off_bpart = take(M > 1 ? M * (size_t)c.n_q_heads * L.batch_splits * (hd + 2) * 4 : 0);
  L.total = o;
  return L;
}

}  // namespace hta

// ---------------------------------------------------------------------------- helpers
static int fail(Ctx& c, int code, const std::string& msg) {
  c.err = msg;
  return code;
}
static int hip_fail(Ctx& c, hipError_t e, const char* where) {
  c.err = std::string(where) + ": " + hipGetErrorString(e);
  return HTA_E_HIP;
}
#define HIPCK(expr, where)                          \
  do {                                              \
    hipError_t _e = (expr);                         \
    if (_e != hipSuccess) return hip_fail(c, _e, where); \
  } while (0)

static bool shape_ok(const hta_config& f, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return false; };
  if (f.n_layers < 1 || f.hidden < 64 || f.n_q_heads < 1 || f.n_kv_heads < 1) return bad("non-positive shape");
  if (f.head_dim != 64 && f.head_dim != 128) return bad("head_dim must be 64 or 128");
  if (f.n_q_heads % f.n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
  {
    const int g = f.n_q_heads / f.n_kv_heads;
    if (g != 1 && g != 2 && g != 4) return bad("GQA group size must be 1, 2 or 4");
  }
  if (f.n_kv_heads > 32) return bad("n_kv_heads above 32 is not supported");
  if (f.n_q_heads + f.n_kv_heads > 64 || f.n_kv_heads * f.head_dim > 2048)
    return bad("n_q_heads + n_kv_heads above 64 or kv width above 2048 exceed the prefill row kernels");
  if (f.hidden % 128 || f.ffn % 128 || (f.n_q_heads * f.head_dim) % 128) return bad("hidden, ffn and q width must be multiples of 128");
  if (f.n_codebooks < 1 || f.n_codebooks > kMaxCodebooks) return bad("n_codebooks must be in 1..16");
  if (f.codebook_size < 2 || f.codebook_size > 2048) return bad("codebook_size must be in 2..2048");
  if (f.bos_id < 0 || f.bos_id >= f.codebook_size || f.eos_id < 0 || f.eos_id >= f.codebook_size) return bad("bos/eos ids out of range");
  if (f.text_vocab < 1) return bad("text_vocab must be positive");
  if (f.max_seq < 2 || f.max_prefill < 1 || f.max_prefill > f.max_seq) return bad("bad max_seq / max_prefill");
  if (f.precision != HTA_BF16 && f.precision != HTA_FP8_E4M3) return bad("unknown precision");
  if (f.n_streams < 0 || f.n_streams > 128) return bad("n_streams must be in 0..128");
  if (f.n_streams > 1 && f.n_streams > f.max_prefill) return bad("n_streams must not exceed max_prefill");
  if (f.hidden > 5120 || f.ffn > 10240 || f.n_q_heads * f.head_dim > 10240)
    return bad("hidden above 5120 or ffn / q width above 10240 exceed the GEMV prologue budget");
  return true;
}

// Point `state`, `hist` and every layer's K/V cache at the selected stream's.
static void point_stream(Ctx& c) {
  const int m = c.sel;
  c.state = c.state_base + m;
  c.hist = c.hist_base + (size_t)m * c.cfg.max_seq * c.cfg.n_codebooks;
  const size_t ke = c.lay.kv_stream_bytes / 2;  // elements
  for (int l = 0; l < c.cfg.n_layers; ++l) {
    c.layers[l].k_cache = c.k_base[l] + (size_t)m * ke;
    c.layers[l].v_cache = c.v_base[l] + (size_t)m * ke;
  }
}

static void set_pointers(Ctx& c) {
  const hta_config& f = c.cfg;
  const Layout& L = c.lay;
  char* w = c.ws;
  const bool fp8 = f.precision == HTA_FP8_E4M3;
  for (int l = 0; l < f.n_layers; ++l) {
    char* b = w + L.layer_base + (size_t)l * L.layer_stride;
    LayerW& lw = c.layers[l];
    lw.w_qkv = b + L.off_wqkv;
    lw.w_o = b + L.off_wo;
    lw.w_gu = b + L.off_wgu;
    lw.w_d = b + L.off_wd;
    lw.s_qkv = fp8 ? reinterpret_cast<float*>(b + L.off_sqkv) : nullptr;
    lw.s_o = fp8 ? reinterpret_cast<float*>(b + L.off_so) : nullptr;
    lw.s_gu = fp8 ? reinterpret_cast<float*>(b + L.off_sgu) : nullptr;
    lw.s_d = fp8 ? reinterpret_cast<float*>(b + L.off_sd) : nullptr;
    lw.g_attn = reinterpret_cast<float*>(b + L.off_gattn);
    lw.g_q = reinterpret_cast<float*>(b + L.off_gq);
    lw.g_k = reinterpret_cast<float*>(b + L.off_gk);
    lw.g_mlp = reinterpret_cast<float*>(b + L.off_gmlp);
    lw.k_cache = reinterpret_cast<uint16_t*>(b + L.off_k);
    lw.v_cache = reinterpret_cast<uint16_t*>(b + L.off_v);
  }
  c.e_text = reinterpret_cast<uint16_t*>(w + L.off_etext);
  c.e_aud = reinterpret_cast<uint16_t*>(w + L.off_eaud);
  c.g_final = reinterpret_cast<float*>(w + L.off_gfinal);
  c.w_head = w + L.off_whead;
  c.s_head = fp8 ? reinterpret_cast<float*>(w + L.off_shead) : nullptr;
  c.rope_cos = reinterpret_cast<float*>(w + L.off_rope_cos);
  c.rope_sin = reinterpret_cast<float*>(w + L.off_rope_sin);
  c.act_scales = reinterpret_cast<float*>(w + L.off_act_scales);
  c.amax = reinterpret_cast<float*>(w + L.off_amax);
  c.state_base = reinterpret_cast<DevState*>(w + L.off_state);
  c.hist_base = reinterpret_cast<int32_t*>(w + L.off_hist);
  c.b_logits = reinterpret_cast<float*>(w + L.off_blogits);
  c.b_part = reinterpret_cast<float*>(w + L.off_bpart);
  c.k_base.assign(f.n_layers, nullptr);
  c.v_base.assign(f.n_layers, nullptr);
  for (int l = 0; l < f.n_layers; ++l) {
    c.k_base[l] = c.layers[l].k_cache;
    c.v_base[l] = c.layers[l].v_cache;
  }
  point_stream(c);
  c.counters = reinterpret_cast<unsigned*>(w + L.off_counters);
  c.h = reinterpret_cast<float*>(w + L.off_h);
  c.qkv = reinterpret_cast<float*>(w + L.off_qkv);
  c.attn_part = reinterpret_cast<float*>(w + L.off_attn_part);
  c.o_act = w + L.off_o_act;
  c.a_act = w + L.off_a_act;
  c.logits = reinterpret_cast<float*>(w + L.off_logits);
  c.d_layers = reinterpret_cast<LayerW*>(w + L.off_layer_table);
  c.x_h = reinterpret_cast<uint64_t*>(w + L.off_xh);
  c.x_qkv = reinterpret_cast<uint64_t*>(w + L.off_xqkv);
  c.x_o = reinterpret_cast<uint32_t*>(w + L.off_xo);
  c.x_a = reinterpret_cast<uint32_t*>(w + L.off_xa);
  c.x_part = reinterpret_cast<uint64_t*>(w + L.off_xpart);
  c.x_logits = reinterpret_cast<uint64_t*>(w + L.off_xlogits);
  c.sync = reinterpret_cast<unsigned*>(w + L.off_sync);
  c.taps_h = reinterpret_cast<float*>(w + L.off_taps);
  c.taps_p = reinterpret_cast<float*>(w + L.off_ptaps);
  c.taps_act = reinterpret_cast<uint16_t*>(w + L.off_tact);
  c.taps_q = reinterpret_cast<uint16_t*>(w + L.off_tq);
  c.trace_buf = reinterpret_cast<uint32_t*>(w + L.off_trace);
  c.fargs = w + L.off_fargs;
  c.fargs_s = w + L.off_fargs_s;
  c.tok = reinterpret_cast<int32_t*>(w + L.off_tok);
  c.px = reinterpret_cast<float*>(w + L.off_x);
  c.pu = w + L.off_u;
  c.pqkv = reinterpret_cast<float*>(w + L.off_pqkv);
  c.pq = reinterpret_cast<float*>(w + L.off_pq);
  c.po = w + L.off_po;
  c.pgu = reinterpret_cast<float*>(w + L.off_pgu);
  c.pa = w + L.off_pa;
}

static void drop_graph(Ctx& c) {
  if (c.batch_exec) (void)hipGraphExecDestroy(c.batch_exec);
  if (c.batch_graph) (void)hipGraphDestroy(c.batch_graph);
  c.batch_exec = nullptr;
  c.batch_graph = nullptr;
  for (auto& g : c.prefill_graphs) (void)hipGraphExecDestroy(g.exec);
  c.prefill_graphs.clear();
  if (c.frame_exec) (void)hipGraphExecDestroy(c.frame_exec);
  if (c.frame_graph) (void)hipGraphDestroy(c.frame_graph);
  c.frame_exec = nullptr;
  c.frame_graph = nullptr;
  if (c.frame_exec8) (void)hipGraphExecDestroy(c.frame_exec8);
  if (c.frame_graph8) (void)hipGraphDestroy(c.frame_graph8);
  c.frame_exec8 = nullptr;
  c.frame_graph8 = nullptr;
}

// Zero the persistent kernel's tagged exchange words and its launch counter / abort flag.
static hipError_t clear_exchange(Ctx& c) {
  const Layout& L = c.lay;
  const size_t n = (L.off_sync + 1024 * 4 - L.off_xh) / 4;
  return launch_fill_u32(c.ws + L.off_xh, 0u, n, c.stream);
}

// The frame graph (one launch of the frame kernel) and a graph of eight launches in a row:
// consecutive frames replayed from one graph start a few microseconds sooner than
// back-to-back replays of the one-launch graph (measured: about 5 us per frame).
static int ensure_graph(Ctx& c) {
  if (c.frame_exec8) return HTA_OK;  // captured last: both graphs are there
  if (c.frame_exec) {                 // a capture that failed half way: start again
    (void)hipGraphExecDestroy(c.frame_exec);
    if (c.frame_graph) (void)hipGraphDestroy(c.frame_graph);
    c.frame_exec = nullptr;
    c.frame_graph = nullptr;
  }
  HIPCK(hipStreamBeginCapture(c.stream, hipStreamCaptureModeRelaxed), "hipStreamBeginCapture");
  hipError_t e = launch_frame_persistent(c);
  hipGraph_t g = nullptr;
  hipError_t e2 = hipStreamEndCapture(c.stream, &g);
  if (e != hipSuccess) { if (g) (void)hipGraphDestroy(g); return hip_fail(c, e, "frame capture"); }
  if (e2 != hipSuccess) return hip_fail(c, e2, "hipStreamEndCapture");
  c.frame_graph = g;
  HIPCK(hipGraphInstantiate(&c.frame_exec, g, nullptr, nullptr, 0), "hipGraphInstantiate");
  HIPCK(hipStreamBeginCapture(c.stream, hipStreamCaptureModeRelaxed), "hipStreamBeginCapture");
  for (int i = 0; i < 8 && e == hipSuccess; ++i) e = launch_frame_persistent(c);
  g = nullptr;
  e2 = hipStreamEndCapture(c.stream, &g);
  if (e != hipSuccess) { if (g) (void)hipGraphDestroy(g); return hip_fail(c, e, "frame capture"); }
  if (e2 != hipSuccess) return hip_fail(c, e2, "hipStreamEndCapture");
  c.frame_graph8 = g;
  HIPCK(hipGraphInstantiate(&c.frame_exec8, g, nullptr, nullptr, 0), "hipGraphInstantiate");
  return HTA_OK;
}

// The prefill of P rows as one graph, captured on first use; at most kMaxPrefillGraphs
// prompt lengths are kept (the oldest is dropped).
constexpr size_t kMaxPrefillGraphs = 16;
static int prefill_graph(Ctx& c, int P, hipGraphExec_t* out) {
  for (const auto& g : c.prefill_graphs)
    if (g.P == P && g.stream == c.sel) { *out = g.exec; return HTA_OK; }
  HIPCK(hipStreamBeginCapture(c.stream, hipStreamCaptureModeRelaxed), "hipStreamBeginCapture");
  hipError_t e = launch_prefill(c, P, false);
  hipGraph_t g = nullptr;
  hipError_t e2 = hipStreamEndCapture(c.stream, &g);
  if (e != hipSuccess) { if (g) (void)hipGraphDestroy(g); return hip_fail(c, e, "prefill capture"); }
  if (e2 != hipSuccess) return hip_fail(c, e2, "hipStreamEndCapture");
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return hip_fail(c, e, "hipGraphInstantiate");
  if (c.prefill_graphs.size() >= kMaxPrefillGraphs) {
    (void)hipGraphExecDestroy(c.prefill_graphs.front().exec);
    c.prefill_graphs.erase(c.prefill_graphs.begin());
  }
  c.prefill_graphs.push_back({P, c.sel, x});
  *out = x;
  return HTA_OK;
}

static int ready(Ctx& c) {
  if (!c.ws) return fail(c, HTA_E_STATE, "no workspace bound");
  if (!c.weights_loaded) return fail(c, HTA_E_STATE, "weights not loaded");
  return HTA_OK;
}

// ---------------------------------------------------------------------------- ABI
extern "C" {

const char* hta_version(void) { return "hta 0.1 gfx950"; }

size_t hta_workspace_bytes(const hta_config* cfg) {
  if (!cfg || !shape_ok(*cfg, nullptr)) return 0;
  return make_layout(*cfg).total;
}

int hta_create(const hta_config* cfg, void* hip_stream, hta_ctx** out) {
  if (!cfg || !out) return HTA_E_ARG;
  *out = nullptr;
  std::string why;
  hta_ctx* x = new (std::nothrow) hta_ctx();
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (!shape_ok(*cfg, &why)) { delete x; return HTA_E_UNSUPPORTED; }
  c.cfg = *cfg;
  hipError_t e = hipGetDevice(&c.device);
  if (e != hipSuccess) { delete x; return HTA_E_HIP; }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c.device) != hipSuccess) { delete x; return HTA_E_HIP; }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) { delete x; return HTA_E_UNSUPPORTED; }
  c.num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
  if (hip_stream) {
    c.stream = static_cast<hipStream_t>(hip_stream);
  } else {
    if (hipStreamCreateWithFlags(&c.stream, hipStreamNonBlocking) != hipSuccess) { delete x; return HTA_E_HIP; }
    c.own_stream = true;
  }
  if (prefill_setup() != hipSuccess) { hta_destroy(x); return HTA_E_HIP; }
  c.lay = make_layout(c.cfg);
  c.layers = new LayerW[c.cfg.n_layers]();
  if (frame_setup(c) == hipSuccess && frame_max_packets(c.cfg, c.frame_blocks) <= frame_part_capacity())
    c.frame_ok = true;
  (void)hipGetLastError();
  {
    // The frame kernel runs one resident block per compute unit, and every block must own
    // rows in every GEMV phase: a block that owned none would not hold back the phase's
    // producers, which could then rewrite an exchange buffer before that block has read it.
    const hta_config& f = c.cfg;
    const long units[5] = {(long)(f.n_q_heads + 2 * f.n_kv_heads) * f.head_dim, f.hidden, f.ffn, f.hidden,
                           (long)f.n_codebooks * f.codebook_size};
    bool rows_ok = true;
    for (long u : units) rows_ok = rows_ok && u >= c.frame_blocks;
    if (!c.frame_ok || !rows_ok) {
      hta_destroy(x);
      return HTA_E_UNSUPPORTED;
    }
  }
  c.h_stage_elems = (size_t)c.cfg.max_seq * c.cfg.n_codebooks * (c.cfg.n_streams > 1 ? c.cfg.n_streams : 1);
  if ((size_t)c.cfg.max_prefill > c.h_stage_elems) c.h_stage_elems = c.cfg.max_prefill;
  if (hipHostMalloc((void**)&c.h_stage, c.h_stage_elems * sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&c.h_state, sizeof(DevState), hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&c.h_status, sizeof(unsigned), hipHostMallocDefault) != hipSuccess) {
    hta_destroy(x);
    return HTA_E_HIP;
  }
  // the static exchange array's address on this device (the current one)
  if (static_scratch(c.device, &c.scratch_dev) != hipSuccess) {
    hta_destroy(x);
    return HTA_E_HIP;
  }
  c.static_exch_bytes = exchange_layout(c.cfg, c.frame_splits, nullptr, nullptr);
  *out = x;
  return HTA_OK;
}

int hta_bind_workspace(hta_ctx* x, void* dev_ptr, size_t bytes) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (!dev_ptr) return fail(c, HTA_E_ARG, "null workspace");
  if (reinterpret_cast<uintptr_t>(dev_ptr) % 256) return fail(c, HTA_E_ARG, "workspace not 256-byte aligned");
  if (bytes < c.lay.total) return fail(c, HTA_E_ARG, "workspace too small");
  drop_graph(c);
  c.ws = static_cast<char*>(dev_ptr);
  c.weights_loaded = false;
  c.sel = 0;
  set_pointers(c);
  const hta_config& f = c.cfg;
  // RoPE table: phi = p * theta^(-2i/hd) in double, stored as float cos / sin
  const int h2 = f.head_dim / 2;
  std::vector<float> cs((size_t)f.max_seq * h2), sn((size_t)f.max_seq * h2);
  for (int p = 0; p < f.max_seq; ++p)
    for (int i = 0; i < h2; ++i) {
      const double inv = std::pow((double)f.rope_theta, -2.0 * i / f.head_dim);
      const double phi = (double)p * inv;
      cs[(size_t)p * h2 + i] = (float)std::cos(phi);
      sn[(size_t)p * h2 + i] = (float)std::sin(phi);
    }
  HIPCK(hipStreamSynchronize(c.stream), "sync");
  HIPCK(hipMemcpy(c.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice), "rope table");
  HIPCK(hipMemcpy(c.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice), "rope table");
  const size_t nsites = (size_t)kSitesPerLayer * f.n_layers + 1;
  HIPCK(launch_fill_u32(c.counters, 0u, 64, c.stream), "fill");
  HIPCK(launch_fill_u32(c.amax, 0u, nsites, c.stream), "fill");
  HIPCK(launch_fill_u32(c.act_scales, 0x3f800000u, nsites, c.stream), "fill");
  const int M = c.lay.n_streams;
  HIPCK(launch_fill_u32(c.state_base, 0u, (size_t)M * sizeof(DevState) / 4, c.stream), "fill");
  HIPCK(clear_exchange(c), "fill");
  for (int m = M - 1; m >= 0; --m) {  // every stream's state; stream 0 stays selected
    c.sel = m;
    point_stream(c);
    HIPCK(launch_reset_state(c, 0), "reset");
  }
  HIPCK(hipStreamSynchronize(c.stream), "sync");
  HIPCK(frame_write_args(c), "frame arguments");
  c.len = 0;
  c.t = 0;
  c.s_len.assign(M, 0);
  c.s_t.assign(M, 0);
  c.s_done.assign(M, 0);
  return HTA_OK;
}

int hta_load_weights(hta_ctx* x, const void* const* t, int n, int src_dtype, const float* act_scales) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  const hta_config& f = c.cfg;
  if (!c.ws) return fail(c, HTA_E_STATE, "no workspace bound");
  if (!t || n != 4 + 11 * f.n_layers) return fail(c, HTA_E_ARG, "expected 4 + 11 * n_layers tensors");
  if (src_dtype != HTA_SRC_F32 && src_dtype != HTA_SRC_BF16) return fail(c, HTA_E_ARG, "bad src dtype");
  for (int i = 0; i < n; ++i) if (!t[i]) return fail(c, HTA_E_ARG, "null weight tensor");
  const bool fp8 = f.precision == HTA_FP8_E4M3;
  if (fp8 && !act_scales) return fail(c, HTA_E_ARG, "FP8 needs activation scales");
  const int nsites = kSitesPerLayer * f.n_layers + 1;
  c.h_scales.assign(nsites, 1.0f);
  if (fp8) {
    for (int i = 0; i < nsites; ++i) {
      if (!(act_scales[i] > 0.0f) || !std::isfinite(act_scales[i])) return fail(c, HTA_E_ARG, "activation scales must be positive");
      c.h_scales[i] = act_scales[i];
    }
  }
  drop_graph(c);
  const int d = f.hidden, hd = f.head_dim, qd = f.n_q_heads * hd, kvd = f.n_kv_heads * hd, F = f.ffn;
  const int CV = f.n_codebooks * f.codebook_size;
  hipStream_t s = c.stream;
  const int q8 = fp8 ? 1 : 0;
  HIPCK(launch_pack_rows(c.e_text, 0, 1, t[0], src_dtype, f.text_vocab, d, 0, nullptr, s), "pack e_text");
  HIPCK(launch_pack_rows(c.e_aud, 0, 1, t[1], src_dtype, CV, d, 0, nullptr, s), "pack e_aud");
  for (int l = 0; l < f.n_layers; ++l) {
    const void* const* T = t + 2 + 11 * l;
    LayerW& L = c.layers[l];
    HIPCK(launch_copy_f32(L.g_attn, T[0], src_dtype, d, s), "gain");
    HIPCK(launch_pack_rows(L.w_qkv, 0, 1, T[1], src_dtype, qd, d, q8, L.s_qkv, s), "pack wq");
    HIPCK(launch_pack_rows(L.w_qkv, qd, 1, T[2], src_dtype, kvd, d, q8, L.s_qkv, s), "pack wk");
    HIPCK(launch_pack_rows(L.w_qkv, qd + kvd, 1, T[3], src_dtype, kvd, d, q8, L.s_qkv, s), "pack wv");
    HIPCK(launch_copy_f32(L.g_q, T[4], src_dtype, hd, s), "gain");
    HIPCK(launch_copy_f32(L.g_k, T[5], src_dtype, hd, s), "gain");
    HIPCK(launch_pack_rows(L.w_o, 0, 1, T[6], src_dtype, d, qd, q8, L.s_o, s), "pack wo");
    HIPCK(launch_copy_f32(L.g_mlp, T[7], src_dtype, d, s), "gain");
    HIPCK(launch_pack_rows(L.w_gu, 0, 2, T[8], src_dtype, F, d, q8, L.s_gu, s), "pack wg");
    HIPCK(launch_pack_rows(L.w_gu, 1, 2, T[9], src_dtype, F, d, q8, L.s_gu, s), "pack wu");
    HIPCK(launch_pack_rows(L.w_d, 0, 1, T[10], src_dtype, d, F, q8, L.s_d, s), "pack wd");
  }
  const void* const* T = t + 2 + 11 * f.n_layers;
  HIPCK(launch_copy_f32(c.g_final, T[0], src_dtype, d, s), "gain");
  HIPCK(launch_pack_rows(c.w_head, 0, 1, T[1], src_dtype, CV, d, q8, c.s_head, s), "pack head");
  if (c.lay.cv_pad > CV) {  // the padded head rows of the batched step's GEMM: zero weights
    const size_t wbh = fp8 ? 1 : 2;
    HIPCK(launch_fill_u32(static_cast<char*>(c.w_head) + (size_t)CV * d * wbh, 0u,
                          (size_t)(c.lay.cv_pad - CV) * d * wbh / 4, s), "fill");
    if (fp8) HIPCK(launch_fill_u32(c.s_head + CV, 0x3f800000u, (size_t)(c.lay.cv_pad - CV), s), "fill");
  }
  HIPCK(hipMemcpyAsync(c.act_scales, c.h_scales.data(), nsites * 4, hipMemcpyHostToDevice, s), "scales");
  HIPCK(hipMemcpyAsync(c.d_layers, c.layers, (size_t)f.n_layers * sizeof(LayerW), hipMemcpyHostToDevice, s), "layer table");
  HIPCK(hipStreamSynchronize(s), "load sync");
  c.weights_loaded = true;
  return HTA_OK;
}

int hta_reset(hta_ctx* x, int keep_len) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (!c.ws) return fail(c, HTA_E_STATE, "no workspace bound");
  if (keep_len < 0 || keep_len > c.len) return fail(c, HTA_E_ARG, "keep_len out of range");
  HIPCK(launch_reset_state(c, keep_len), "reset");
  c.len = keep_len;
  c.t = 0;
  c.done = false;
  return HTA_OK;
}

int hta_select_stream(hta_ctx* x, int m) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (!c.ws) return fail(c, HTA_E_STATE, "no workspace bound");
  if (m < 0 || m >= c.lay.n_streams) return fail(c, HTA_E_ARG, "stream out of range");
  c.s_len[c.sel] = c.len;
  c.s_t[c.sel] = c.t;
  c.s_done[c.sel] = c.done ? 1 : 0;
  c.sel = m;
  point_stream(c);
  c.len = c.s_len[m];
  c.t = c.s_t[m];
  c.done = c.s_done[m] != 0;
  return HTA_OK;
}

int hta_prefill(hta_ctx* x, const int32_t* tokens, int P) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  int r = ready(c);
  if (r) return r;
  if (!tokens || P <= 0) return fail(c, HTA_E_ARG, "empty prompt");
  if (P > c.cfg.max_prefill) return fail(c, HTA_E_CAPACITY, "P exceeds max_prefill");
  if (c.len + P > c.cfg.max_seq) return fail(c, HTA_E_CAPACITY, "prompt exceeds max_seq");
  for (int i = 0; i < P; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.cfg.text_vocab) return fail(c, HTA_E_RANGE, "token id out of range");
  HIPCK(hipStreamSynchronize(c.stream), "sync");
  std::memcpy(c.h_stage, tokens, (size_t)P * 4);
  HIPCK(hipMemcpyAsync(c.tok, c.h_stage, (size_t)P * 4, hipMemcpyHostToDevice, c.stream), "tokens");
  if (c.use_graph && !c.taps) {
    hipGraphExec_t x = nullptr;
    int r2 = prefill_graph(c, P, &x);
    if (r2 != HTA_OK) return r2;
    HIPCK(hipGraphLaunch(x, c.stream), "hipGraphLaunch");
  } else {
    HIPCK(launch_prefill(c, P, false), "prefill");
  }
  HIPCK(launch_set_len(c, c.len + P), "set len");
  HIPCK(hipStreamSynchronize(c.stream), "prefill sync");
  c.len += P;
  c.last_prefill_P = P;
  return HTA_OK;
}

// A bounded wait of the frame kernel expired (every block left the kernel early): clear
// the exchange words so that the next launch starts clean.
static int frame_timed_out(Ctx& c) {
  HIPCK(clear_exchange(c), "fill");
  HIPCK(hipStreamSynchronize(c.stream), "sync");
  return fail(c, HTA_E_TIMEOUT, "a bounded wait of the frame kernel expired; the utterance must be reset");
}

// n frames; with `no_alloc` the frame kernel exchanges through the static per-device array
// (cleared first, launch counter included) and is launched directly, never through the graph.
// n batched steps of every stream (n_streams > 1): the step graph replayed n times, then
// each stream's n codes from its history into codes_out[frame][stream][codebook].
static int decode_batch(Ctx& c, int n, int32_t* codes_out, int* n_done_out) {
  const int M = c.lay.n_streams, C = c.cfg.n_codebooks;
  c.s_len[c.sel] = c.len;
  c.s_t[c.sel] = c.t;
  for (int m = 0; m < M; ++m)
    if (c.s_len[m] + n > c.cfg.max_seq) return fail(c, HTA_E_CAPACITY, "KV cache of a stream full");
  if ((size_t)n * M * C > c.h_stage_elems) return fail(c, HTA_E_ARG, "too many frames for one call");
  if (!c.batch_exec) {
    HIPCK(hipStreamBeginCapture(c.stream, hipStreamCaptureModeRelaxed), "hipStreamBeginCapture");
    hipError_t e = launch_batch_step(c);
    hipGraph_t g = nullptr;
    hipError_t e2 = hipStreamEndCapture(c.stream, &g);
    if (e != hipSuccess) { if (g) (void)hipGraphDestroy(g); return hip_fail(c, e, "batch step capture"); }
    if (e2 != hipSuccess) return hip_fail(c, e2, "hipStreamEndCapture");
    c.batch_graph = g;
    HIPCK(hipGraphInstantiate(&c.batch_exec, g, nullptr, nullptr, 0), "hipGraphInstantiate");
  }
  for (int i = 0; i < n; ++i) HIPCK(hipGraphLaunch(c.batch_exec, c.stream), "hipGraphLaunch");
  for (int m = 0; m < M; ++m)  // stream m's steps t_m .. t_m + n - 1
    HIPCK(hipMemcpy2DAsync(c.h_stage + (size_t)m * C, (size_t)M * C * 4,
                           c.hist_base + ((size_t)m * c.cfg.max_seq + c.s_t[m]) * C, (size_t)C * 4, (size_t)C * 4, n,
                           hipMemcpyDeviceToHost, c.stream), "codes");
  HIPCK(hipStreamSynchronize(c.stream), "decode sync");
  std::vector<DevState> st(M);
  HIPCK(hipMemcpy(st.data(), c.state_base, (size_t)M * sizeof(DevState), hipMemcpyDeviceToHost), "state");
  std::memcpy(codes_out, c.h_stage, (size_t)n * M * C * 4);
  int done = 0;
  for (int m = 0; m < M; ++m) {
    c.s_len[m] += n;
    c.s_t[m] += n;
    c.s_done[m] = st[m].done ? 1 : 0;
    done += c.s_done[m];
    if (st[m].len != c.s_len[m] || st[m].t != c.s_t[m]) return fail(c, HTA_E_STATE, "device state out of step with host");
  }
  c.len = c.s_len[c.sel];
  c.t = c.s_t[c.sel];
  c.done = c.s_done[c.sel] != 0;
  if (n_done_out) *n_done_out = done;
  return done == M ? HTA_DONE : HTA_OK;
}

static int decode_n(Ctx& c, int n, int32_t* codes_out, int* n_done_out, bool no_alloc) {
  int r = ready(c);
  if (r) return r;
  if (n <= 0 || !codes_out) return fail(c, HTA_E_ARG, "bad frame count or output");
  if (c.lay.n_streams > 1) {
    if (no_alloc) return fail(c, HTA_E_UNSUPPORTED, "the allocation-free decode serves single-stream contexts");
    return decode_batch(c, n, codes_out, n_done_out);
  }
  if (c.len + n > c.cfg.max_seq) return fail(c, HTA_E_CAPACITY, "KV cache full");
  const unsigned* abort_word = c.sync + 64;
  if (no_alloc) {
    if (!c.scratch_dev) return fail(c, HTA_E_STATE, "static scratch address not looked up");
    if (c.static_exch_bytes > kStaticScratchBytes)
      return fail(c, HTA_E_CAPACITY, "this shape's exchange words need " + std::to_string(c.static_exch_bytes) +
                                         " bytes; the static scratch array holds " + std::to_string(kStaticScratchBytes));
    Exchange xs;
    exchange_layout(c.cfg, c.frame_splits, c.scratch_dev, &xs);
    abort_word = xs.sync + 64;
    // the previous call on this GPU (any context, any shape) left its tags there
    HIPCK(launch_fill_u32(c.scratch_dev, 0u, c.static_exch_bytes / 4, c.stream), "fill");
    for (int i = 0; i < n; ++i) HIPCK(launch_frame_args(c, c.fargs_s), "frame");
  } else if (c.use_graph && !c.taps) {
    if ((r = ensure_graph(c)) != HTA_OK) return r;
    int i = 0;
    for (; i + 8 <= n; i += 8) HIPCK(hipGraphLaunch(c.frame_exec8, c.stream), "hipGraphLaunch");
    for (; i < n; ++i) HIPCK(hipGraphLaunch(c.frame_exec, c.stream), "hipGraphLaunch");
  } else {
    for (int i = 0; i < n; ++i) HIPCK(launch_frame_persistent(c), "frame");
  }
  const int C = c.cfg.n_codebooks;
  const int t0 = c.t;
  HIPCK(hipMemcpyAsync(c.h_stage, c.hist + (size_t)t0 * C, (size_t)n * C * 4, hipMemcpyDeviceToHost, c.stream), "codes");
  HIPCK(hipMemcpyAsync(c.h_state, c.state, sizeof(DevState), hipMemcpyDeviceToHost, c.stream), "state");
  HIPCK(hipMemcpyAsync(c.h_status, abort_word, sizeof(unsigned), hipMemcpyDeviceToHost, c.stream), "status");
  HIPCK(hipStreamSynchronize(c.stream), "decode sync");
  if (*c.h_status) return frame_timed_out(c);
  std::memcpy(codes_out, c.h_stage, (size_t)n * C * 4);
  c.len += n;
  c.t += n;
  if (c.h_state->len != c.len || c.h_state->t != c.t) return fail(c, HTA_E_STATE, "device state out of step with host");
  c.done = c.h_state->done != 0;
  if (n_done_out) *n_done_out = c.h_state->n_done;
  return c.done ? HTA_DONE : HTA_OK;
}

int hta_decode_frame(hta_ctx* x, int32_t* codes_out) {
  if (!x) return HTA_E_ARG;
  return decode_n(x->c, 1, codes_out, nullptr, false);
}

int hta_decode_frames(hta_ctx* x, int n, int32_t* codes_out, int* n_done) {
  if (!x) return HTA_E_ARG;
  return decode_n(x->c, n, codes_out, n_done, false);
}

int hta_decode_frames_noalloc(hta_ctx* x, int n, int32_t* codes_out, int* n_done) {
  if (!x) return HTA_E_ARG;
  return decode_n(x->c, n, codes_out, n_done, true);
}

int hta_set_sampling(hta_ctx* x, float temperature, uint64_t seed) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (c.lay.n_streams > 1 && temperature != 0.0f) return fail(c, HTA_E_UNSUPPORTED, "batched decode is greedy");
  if (!(temperature >= 0.0f) || !std::isfinite(temperature)) return fail(c, HTA_E_ARG, "temperature must be finite and >= 0");
  const size_t logit_bytes = (size_t)c.cfg.n_codebooks * c.cfg.codebook_size * sizeof(float);
  if (temperature > 0.0f && logit_bytes > frame_sample_capacity())
    return fail(c, HTA_E_UNSUPPORTED, "n_codebooks * codebook_size logits exceed the sampling head's LDS");
  c.temperature = temperature;
  c.seed = seed;
  if (c.ws) HIPCK(frame_write_args(c), "frame arguments");
  return HTA_OK;
}

int hta_force_codes(hta_ctx* x, const int32_t* codes) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (!c.ws) return fail(c, HTA_E_STATE, "no workspace bound");
  if (!codes) return fail(c, HTA_E_ARG, "null codes");
  for (int k = 0; k < c.cfg.n_codebooks; ++k)
    if (codes[k] < 0 || codes[k] >= c.cfg.codebook_size) return fail(c, HTA_E_RANGE, "code out of range");
  HIPCK(launch_set_prev(c, codes), "force codes");
  return HTA_OK;
}

int hta_read_tap(hta_ctx* x, int tap, int layer, void* host_out, size_t bytes) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  const hta_config& f = c.cfg;
  if (!c.ws) return fail(c, HTA_E_STATE, "no workspace bound");
  if (!host_out) return fail(c, HTA_E_ARG, "null output");
  HIPCK(hipStreamSynchronize(c.stream), "sync");
  const int C = f.n_codebooks;
  switch (tap) {
    case HTA_TAP_HIDDEN: {
      if (bytes < (size_t)f.hidden * 4) return fail(c, HTA_E_ARG, "buffer too small");
      // batched: the selected stream's final residual row of the last step
      const float* src = c.lay.n_streams > 1 ? c.px + (size_t)c.sel * f.hidden : c.h;
      HIPCK(hipMemcpy(host_out, src, (size_t)f.hidden * 4, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_LOGITS: {
      const size_t nb = (size_t)C * f.codebook_size * 4;
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      const float* src = c.lay.n_streams > 1 ? c.b_logits + (size_t)c.sel * c.lay.cv_pad : c.logits;
      HIPCK(hipMemcpy(host_out, src, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_STATE: {
      if (bytes < (size_t)(4 + 2 * C) * 4) return fail(c, HTA_E_ARG, "buffer too small");
      DevState s;
      HIPCK(hipMemcpy(&s, c.state, sizeof(s), hipMemcpyDeviceToHost), "tap");
      int32_t* o = static_cast<int32_t*>(host_out);
      o[0] = s.len; o[1] = s.t; o[2] = s.eoc; o[3] = s.done;
      for (int k = 0; k < C; ++k) { o[4 + k] = s.prev[k]; o[4 + C + k] = s.codes[k]; }
      return HTA_OK;
    }
    case HTA_TAP_KV: {
      // as many positions as the buffer holds: bytes / (2 * Hkv * hd * 2), at most max_seq
      if (layer < 0 || layer >= f.n_layers) return fail(c, HTA_E_ARG, "bad layer");
      const size_t per_pos = 2 * (size_t)f.n_kv_heads * f.head_dim * 2;
      size_t npos = bytes / per_pos;
      if (npos > (size_t)f.max_seq) npos = f.max_seq;
      if (npos == 0) return fail(c, HTA_E_ARG, "buffer too small");
      const size_t row = npos * f.head_dim * 2;
      const size_t half = (size_t)f.n_kv_heads * row;
      const size_t pitch = (size_t)f.max_seq * f.head_dim * 2;
      char* o = static_cast<char*>(host_out);
      HIPCK(hipMemcpy2D(o, row, c.layers[layer].k_cache, pitch, row, f.n_kv_heads, hipMemcpyDeviceToHost), "tap");
      HIPCK(hipMemcpy2D(o + half, row, c.layers[layer].v_cache, pitch, row, f.n_kv_heads, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_AMAX: {
      const size_t nb = ((size_t)kSitesPerLayer * f.n_layers + 1) * 4;
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      HIPCK(hipMemcpy(host_out, c.amax, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_PREFILL_HIDDEN: {
      const size_t nb = (size_t)c.last_prefill_P * f.hidden * 4;
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      if (nb) HIPCK(hipMemcpy(host_out, c.px, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_W_QKV:
    case HTA_TAP_S_QKV:
    case HTA_TAP_W_GU:
    case HTA_TAP_S_GU: {
      if (layer < 0 || layer >= f.n_layers) return fail(c, HTA_E_ARG, "bad layer");
      const bool fp8 = f.precision == HTA_FP8_E4M3;
      const bool qkv = tap == HTA_TAP_W_QKV || tap == HTA_TAP_S_QKV;
      const bool scales = tap == HTA_TAP_S_QKV || tap == HTA_TAP_S_GU;
      const size_t rows = qkv ? (size_t)(f.n_q_heads + 2 * f.n_kv_heads) * f.head_dim : (size_t)2 * f.ffn;
      if (scales && !fp8) return fail(c, HTA_E_ARG, "no scales in a BF16 context");
      const size_t nb = scales ? rows * 4 : rows * f.hidden * (fp8 ? 1 : 2);
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      const LayerW& L = c.layers[layer];
      const void* src = scales ? (const void*)(qkv ? L.s_qkv : L.s_gu) : (const void*)(qkv ? L.w_qkv : L.w_gu);
      HIPCK(hipMemcpy(host_out, src, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_LAYER_H: {
      const size_t nb = ((size_t)f.n_layers + 1) * f.hidden * 4;
      if (!c.taps) return fail(c, HTA_E_STATE, "taps are off");
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      HIPCK(hipMemcpy(host_out, c.taps_h, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_PREFILL_LAYER: {
      const size_t nb = (size_t)c.last_prefill_P * f.hidden * 4;
      if (!c.taps) return fail(c, HTA_E_STATE, "taps are off");
      if (bytes < 2 * nb) return fail(c, HTA_E_ARG, "buffer too small");
      if (nb) {
        char* o = static_cast<char*>(host_out);
        HIPCK(hipMemcpy(o, c.taps_p, nb, hipMemcpyDeviceToHost), "tap");
        HIPCK(hipMemcpy(o + nb, c.taps_p + (size_t)f.max_prefill * f.hidden, nb, hipMemcpyDeviceToHost), "tap");
      }
      return HTA_OK;
    }
    case HTA_TAP_ACT: {
      const size_t nb = (5 * (size_t)f.n_layers + 1) * kActsWidth * 2;
      if (!c.taps) return fail(c, HTA_E_STATE, "taps are off");
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      HIPCK(hipMemcpy(host_out, c.taps_act, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_Q: {
      const size_t nb = (size_t)f.n_layers * f.n_q_heads * f.head_dim * 2;
      if (!c.taps) return fail(c, HTA_E_STATE, "taps are off");
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      HIPCK(hipMemcpy(host_out, c.taps_q, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    case HTA_TAP_TRACE: {
      const size_t nb = (size_t)c.frame_blocks * (5 * f.n_layers + 1) * 8 * 4;
      if (!c.trace) return fail(c, HTA_E_STATE, "trace is off");
      if (bytes < nb) return fail(c, HTA_E_ARG, "buffer too small");
      HIPCK(hipMemcpy(host_out, c.trace_buf, nb, hipMemcpyDeviceToHost), "tap");
      return HTA_OK;
    }
    default:
      return fail(c, HTA_E_ARG, "unknown tap");
  }
}

int hta_calibrate(hta_ctx* x, const int32_t* tokens, int P, int n_frames, const int32_t* forced, float* scales_out) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  const hta_config& f = c.cfg;
  int r = ready(c);
  if (r) return r;
  if (f.precision != HTA_BF16) return fail(c, HTA_E_STATE, "calibration runs on a BF16 context");
  if (c.lay.n_streams > 1) return fail(c, HTA_E_UNSUPPORTED, "calibration runs on a single-stream context");
  if (!tokens || P <= 0 || P > f.max_prefill || n_frames < 0 || !scales_out) return fail(c, HTA_E_ARG, "bad calibration arguments");
  if (P + n_frames > f.max_seq) return fail(c, HTA_E_CAPACITY, "calibration run exceeds max_seq");
  for (int i = 0; i < P; ++i)
    if (tokens[i] < 0 || tokens[i] >= f.text_vocab) return fail(c, HTA_E_RANGE, "token id out of range");
  if (forced)
    for (int i = 0; i < n_frames * f.n_codebooks; ++i)
      if (forced[i] < 0 || forced[i] >= f.codebook_size) return fail(c, HTA_E_RANGE, "forced code out of range");
  const int nsites = kSitesPerLayer * f.n_layers + 1;
  c.len = 0;  // cold start
  HIPCK(launch_reset_state(c, 0), "reset");
  HIPCK(launch_fill_u32(c.amax, 0u, nsites, c.stream), "fill");
  HIPCK(hipStreamSynchronize(c.stream), "sync");
  std::memcpy(c.h_stage, tokens, (size_t)P * 4);
  HIPCK(hipMemcpyAsync(c.tok, c.h_stage, (size_t)P * 4, hipMemcpyHostToDevice, c.stream), "tokens");
  HIPCK(launch_prefill(c, P, true), "calibration prefill");
  HIPCK(launch_set_len(c, P), "set len");
  // the frames run on the decode frame kernel itself, recording each site's maximum
  c.frame_record = true;
  const float temperature = c.temperature;  // calibration is a greedy run
  c.temperature = 0.0f;
  HIPCK(frame_write_args(c), "frame arguments");
  hipError_t e = hipSuccess;
  for (int fr = 0; fr < n_frames && e == hipSuccess; ++fr) {
    e = launch_frame_persistent(c);
    if (e == hipSuccess && forced) e = launch_set_prev(c, forced + (size_t)fr * f.n_codebooks);
  }
  c.frame_record = false;
  c.temperature = temperature;
  const hipError_t e2 = frame_write_args(c);  // synchronises the stream first
  if (e != hipSuccess) return hip_fail(c, e, "calibration frame");
  if (e2 != hipSuccess) return hip_fail(c, e2, "frame arguments");
  unsigned aborted = 0;
  HIPCK(hipMemcpy(&aborted, c.sync + 64, sizeof(unsigned), hipMemcpyDeviceToHost), "status");
  if (aborted) return frame_timed_out(c);
  std::vector<float> amax(nsites);
  HIPCK(hipMemcpy(amax.data(), c.amax, nsites * 4, hipMemcpyDeviceToHost), "amax");
  for (int i = 0; i < nsites; ++i) scales_out[i] = amax[i] > 0.0f ? amax[i] / 448.0f : 1.0f;
  c.last_prefill_P = P;
  HIPCK(launch_reset_state(c, 0), "reset");
  HIPCK(hipStreamSynchronize(c.stream), "sync");
  c.len = 0;
  c.t = 0;
  c.done = false;
  return HTA_OK;
}

int hta_layer_step(hta_ctx* x, int layer, int kv_len, const void* k_init, const void* v_init, void* h_io) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  const hta_config& f = c.cfg;
  int r = ready(c);
  if (r) return r;
  if (c.lay.n_streams > 1) return fail(c, HTA_E_UNSUPPORTED, "a single-stream call");
  if (f.n_layers != 1 || layer != 0) return fail(c, HTA_E_UNSUPPORTED, "a layer step runs layer 0 of a one-layer context");
  if (kv_len < 1 || kv_len > f.max_seq) return fail(c, HTA_E_CAPACITY, "kv_len out of range");
  if (!h_io) return fail(c, HTA_E_ARG, "null hidden state");
  if ((k_init == nullptr) != (v_init == nullptr)) return fail(c, HTA_E_ARG, "k_init and v_init go together");
  if (!k_init && kv_len - 1 > c.len) return fail(c, HTA_E_STATE, "the cache holds fewer than kv_len - 1 positions");
  if (k_init)
    HIPCK(launch_kv_init(c.layers[0].k_cache, c.layers[0].v_cache, k_init, v_init, f.n_kv_heads, kv_len - 1,
                         f.max_seq, f.head_dim, c.stream), "kv init");
  // one frame of the decode frame kernel at position kv_len - 1 with h_io as its input
  HIPCK(launch_reset_state(c, kv_len - 1), "reset");
  c.frame_h_in = static_cast<const float*>(h_io);
  hipError_t e = frame_write_args(c);
  if (e == hipSuccess) e = launch_frame_persistent(c);
  c.frame_h_in = nullptr;
  const hipError_t e2 = frame_write_args(c);  // synchronises the stream first
  if (e != hipSuccess) return hip_fail(c, e, "layer step");
  if (e2 != hipSuccess) return hip_fail(c, e2, "frame arguments");
  unsigned aborted = 0;
  HIPCK(hipMemcpy(&aborted, c.sync + 64, sizeof(unsigned), hipMemcpyDeviceToHost), "status");
  if (aborted) return frame_timed_out(c);
  HIPCK(hipMemcpy(h_io, c.h, (size_t)f.hidden * 4, hipMemcpyDeviceToDevice), "layer output");
  c.len = kv_len;
  c.t = 1;
  c.done = false;
  return HTA_OK;
}

int hta_undelay(const int32_t* steps, int T, int C, int eos, int32_t* frames_out, int* n_frames) {
  if (!steps || !frames_out || !n_frames || T < 0 || C < 1) return HTA_E_ARG;
  int eoc = -1;
  for (int t = 0; t < T; ++t)
    if (steps[(size_t)t * C] == eos) { eoc = t; break; }
  int n = eoc >= 0 ? eoc : T - (C - 1);
  if (n < 0) n = 0;
  if (n + C - 1 > T) n = T - (C - 1) < 0 ? 0 : T - (C - 1);
  for (int fr = 0; fr < n; ++fr)
    for (int k = 0; k < C; ++k) frames_out[(size_t)fr * C + k] = steps[(size_t)(fr + k) * C + k];
  *n_frames = n;
  return HTA_OK;
}

int hta_time_kernels(hta_ctx* x, int n_frames, float* avg_us, int n_classes) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  int r = ready(c);
  if (r) return r;
  if (c.lay.n_streams > 1) return fail(c, HTA_E_UNSUPPORTED, "a single-stream call");
  if (n_frames <= 0 || !avg_us || n_classes <= 0) return fail(c, HTA_E_ARG, "bad arguments");
  if (c.len + n_frames > c.cfg.max_seq) return fail(c, HTA_E_CAPACITY, "KV cache full");
  hipEvent_t ev[2];
  HIPCK(hipEventCreate(&ev[0]), "hipEventCreate");
  if (hipEventCreate(&ev[1]) != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return fail(c, HTA_E_HIP, "hipEventCreate");
  }
  int cls = -1;
  double sum = 0.0;
  int rc = HTA_OK;
  for (int fr = 0; fr < n_frames && rc == HTA_OK; ++fr) {
    c.tev = ev;
    c.tev_cap = 2;
    c.tev_next = 0;
    c.tev_class = &cls;
    hipError_t e = launch_frame_persistent(c);
    c.tev = nullptr;
    if (e != hipSuccess) { rc = hip_fail(c, e, "timed frame"); break; }
    if ((e = hipStreamSynchronize(c.stream)) != hipSuccess) { rc = hip_fail(c, e, "sync"); break; }
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, ev[0], ev[1]) == hipSuccess) sum += ms * 1000.0;
    c.len += 1;
    c.t += 1;
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  for (int k = 0; k < n_classes; ++k) avg_us[k] = (k == HTA_K_FRAME && rc == HTA_OK) ? (float)(sum / n_frames) : 0.0f;
  return rc;
}

int hta_set_option(hta_ctx* x, int option, int value) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (option == HTA_OPT_USE_GRAPH) {
    c.use_graph = value != 0;
    return HTA_OK;
  }
  if ((option == HTA_OPT_TAPS || option == HTA_OPT_TRACE || option == HTA_OPT_FORCE_TIMEOUT) && value != 0 &&
      c.lay.n_streams > 1)
    return fail(c, HTA_E_UNSUPPORTED, "a single-stream option");
  if (option == HTA_OPT_TAPS) {
    const bool v = value != 0;
    if (v != c.taps) drop_graph(c);
    c.taps = v;
    HIPCK(frame_write_args(c), "frame arguments");
    return HTA_OK;
  }
  if (option == HTA_OPT_TRACE) {
    const bool v = value != 0;
    if (v != c.trace) drop_graph(c);
    c.trace = v;
    HIPCK(frame_write_args(c), "frame arguments");
    return HTA_OK;
  }
  if (option == HTA_OPT_FORCE_TIMEOUT) {
    c.force_timeout = value != 0;
    HIPCK(frame_write_args(c), "frame arguments");
    return HTA_OK;
  }
  if (option == HTA_OPT_FP8_MFMA) {
    if (value != 0 && c.cfg.precision != HTA_FP8_E4M3)
      return fail(c, HTA_E_UNSUPPORTED, "the e4m3 MFMA option is for FP8 contexts");
    const bool v = value != 0;
    if (v != c.fp8_mfma) drop_graph(c);  // captured prefills and batched steps hold the kernel choice
    c.fp8_mfma = v;
    return HTA_OK;
  }
  if (option == HTA_OPT_PREFILL_TAP_LAYER) {
    if (value < 0 || value >= c.cfg.n_layers) return fail(c, HTA_E_ARG, "tap layer out of range");
    c.prefill_tap_layer = value;
    return HTA_OK;
  }
  return fail(c, HTA_E_ARG, "unknown option");
}

int hta_gemm(hta_ctx* x, const void* A, const void* W, const float* w_scale, float a_scale, int M, int N, int K,
             float* C) {
  if (!x) return HTA_E_ARG;
  Ctx& c = x->c;
  if (!c.ws) return fail(c, HTA_E_STATE, "no workspace bound");
  const bool fp8 = c.cfg.precision == HTA_FP8_E4M3;
  if (!A || !W || !C || (fp8 && !w_scale)) return fail(c, HTA_E_ARG, "null operand");
  if (M < 1 || M > c.cfg.max_prefill) return fail(c, HTA_E_ARG, "M must be in 1..max_prefill");
  if (N < 64 || N % 64 != 0 || N > c.lay.gemm_cols)
    return fail(c, HTA_E_ARG, "N must be a multiple of 64 up to the widest projection");
  if (K < 128 || K % 128 != 0) return fail(c, HTA_E_ARG, "K must be a positive multiple of 128");
  const size_t rows = (size_t)(M > N ? M : N), eb = fp8 ? 1 : 2;
  if (rows * (size_t)K * eb >= ((size_t)1 << 31)) return fail(c, HTA_E_ARG, "operand of 2 GiB or more");
  HIPCK(launch_gemm(c, A, W, w_scale, a_scale, C, M, N, K), "gemm");
  HIPCK(hipStreamSynchronize(c.stream), "gemm sync");
  return HTA_OK;
}

void hta_destroy(hta_ctx* x) {
  if (!x) return;
  Ctx& c = x->c;
  if (c.stream) (void)hipStreamSynchronize(c.stream);
  drop_graph(c);
  if (c.h_stage) (void)hipHostFree(c.h_stage);
  if (c.h_state) (void)hipHostFree(c.h_state);
  if (c.h_status) (void)hipHostFree(c.h_status);
  if (c.own_stream && c.stream) (void)hipStreamDestroy(c.stream);
  delete[] c.layers;
  delete x;
}

const char* hta_last_error(const hta_ctx* x) {
  if (!x) return "null context";
  return x->c.err.c_str();
}

}  // extern "C"
