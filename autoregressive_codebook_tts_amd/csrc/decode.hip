// Decode-step kernels for gfx950: frame input embedding, the M = 1 weight-
// streaming GEMV (fused RMSNorm + activation-rounding prologue, residual /
// SiLU*mul / head epilogues), split-K flash-decoding attention with fused
// q/k-norm + RoPE + KV write and a last-block combine, and the fused head
// argmax + delay-pattern bookkeeping.
//
// Reference: FlashRT "Higgs Audio v3 TTS-4B" page, section 5 (per-frame chain
// and the M = 1 GEMV with fused residual epilogue) and section 8 (FP8 static
// activation scales); SGLang-Omni Higgs Audio v3 page, architecture paragraph
// (summed codebook embedding as next input).
#include "device_common.h"
#include "hta_internal.h"

namespace hta {

// ============================================================================ frame input
// h = sum_k E_aud[k][prev_k]; block 0 also derives the EOC step from the
// fed-back code of codebook 0 (delay pattern bookkeeping).
__global__ __launch_bounds__(256) void k_frame_begin(const uint16_t* __restrict__ e_aud, DevState* st,
                                                     float* __restrict__ h, int d, int C, int V, int eos) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (st->eoc < 0 && st->t > 0 && st->prev[0] == eos) st->eoc = st->t - 1;
  }
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= d) return;
  float s = 0.0f;
  for (int c = 0; c < C; ++c) {
    const int code = st->prev[c];
    s += bf16_to_f32(e_aud[((size_t)c * V + code) * d + k]);
  }
  h[k] = s;
}

// ============================================================================ GEMV
enum Pro { kProNorm = 0, kProAct = 1 };
enum Epi { kEpiStore = 0, kEpiResid = 1, kEpiSilu = 2, kEpiHead = 3 };

struct GemvArgs {
  const void* w;          // [N][K] bf16 or e4m3
  const float* w_scale;   // FP8 per-row scale
  int N, K;
  const float* h;         // norm prologue: input residual [K]
  const float* g;         // norm gain [K]
  float eps;
  const void* x_act;      // act prologue: [K] bf16 bits / e4m3 codes
  float in_scale;         // activation scale of the input site (FP8)
  float* amax_in;         // record slot of the input site (norm prologue), or null
  float* out;             // store / residual target [N]
  void* out_act;          // SiLU epilogue output [N/2]
  float out_scale;        // activation scale of the SiLU output site (FP8)
  float* amax_out;        // record slot of the SiLU output site, or null
  // head epilogue
  unsigned* counter;
  DevState* st;
  int32_t* hist;
  int C, V, bos, eos;
};

template <int P>
struct WTraits;
template <>
struct WTraits<kBF16> { static constexpr int E = 8; static constexpr int B = 2; };
template <>
struct WTraits<kFP8> { static constexpr int E = 16; static constexpr int B = 1; };

// dot of one 16-byte weight packet with E consecutive fp32 activations from LDS
template <int P>
__device__ __forceinline__ float dot16(const uint4& w, const float* __restrict__ x) {
  float s = 0.0f;
  if (P == kBF16) {
    const float4 x0 = *reinterpret_cast<const float4*>(x);
    const float4 x1 = *reinterpret_cast<const float4*>(x + 4);
    s = fmaf(bf16lo(w.x), x0.x, s); s = fmaf(bf16hi(w.x), x0.y, s);
    s = fmaf(bf16lo(w.y), x0.z, s); s = fmaf(bf16hi(w.y), x0.w, s);
    s = fmaf(bf16lo(w.z), x1.x, s); s = fmaf(bf16hi(w.z), x1.y, s);
    s = fmaf(bf16lo(w.w), x1.z, s); s = fmaf(bf16hi(w.w), x1.w, s);
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 xv = *reinterpret_cast<const float4*>(x + 4 * i);
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
      s = fmaf(lo[0], xv.x, s); s = fmaf(lo[1], xv.y, s);
      s = fmaf(hi[0], xv.z, s); s = fmaf(hi[1], xv.w, s);
    }
  }
  return s;
}

template <int P, int ROWS, int PRO, int EPI>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  extern __shared__ float smem[];
  float* xs = smem;            // [K] activations in GEMV units
  __shared__ float red[16];
  __shared__ int sh_flag;
  __shared__ int sh_arg[kMaxCodebooks];
  const int K = a.K, N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // ---- prologue: the input vector in LDS
  if (PRO == kProNorm) {
    float ss = 0.0f;
    for (int k = tid; k < K; k += blockDim.x) { const float v = a.h[k]; ss = fmaf(v, v, ss); }
    ss = block_sum(ss, red);
    const float rstd = 1.0f / sqrtf(ss / (float)K + a.eps);
    float mx = 0.0f;
    for (int k = tid; k < K; k += blockDim.x) {
      const float u = a.h[k] * rstd * a.g[k];
      mx = fmaxf(mx, fabsf(u));
      xs[k] = act_round<P>(u, a.in_scale);
    }
    if (a.amax_in != nullptr && blockIdx.x == 0) {
      mx = block_max(mx, red);
      if (tid == 0) record_amax(a.amax_in, mx);
    }
  } else {
    if (P == kBF16) {
      const uint16_t* x = static_cast<const uint16_t*>(a.x_act);
      for (int k = tid; k < K; k += blockDim.x) xs[k] = bf16_to_f32(x[k]);
    } else {
      const uint8_t* x = static_cast<const uint8_t*>(a.x_act);
      for (int k = tid; k < K; k += blockDim.x) xs[k] = e4m3_to_f32(x[k]);
    }
  }
  __syncthreads();

  // ---- main loop: each wave owns ROWS consecutive rows
  constexpr int E = WTraits<P>::E;
  constexpr int CH = kWave * E;
  constexpr int U = (P == kBF16) ? 4 : 2;
  const int row0 = (blockIdx.x * (blockDim.x >> 6) + wv) * ROWS;
  const int nch = (K + CH - 1) / CH;
  float acc[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;
  if (row0 < N) {
    const uint8_t* wb = static_cast<const uint8_t*>(a.w);
    for (int c0 = 0; c0 < nch; c0 += U) {
      uint4 wr[ROWS][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = (c0 + u) * CH + lane * E;
        const bool ok = (c0 + u < nch) && (e < K);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const int row = row0 + r;
          if (ok && row < N)
            wr[r][u] = ld_stream16(wb + ((size_t)row * K + e) * WTraits<P>::B);
          else
            wr[r][u] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = (c0 + u) * CH + lane * E;
        if ((c0 + u < nch) && (e < K)) {
#pragma unroll
          for (int r = 0; r < ROWS; ++r) acc[r] += dot16<P>(wr[r][u], xs + e);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = wave_sum(acc[r]);

  // ---- epilogue (lane 0 of each wave)
  if (lane == 0 && row0 < N) {
    float y[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int row = row0 + r;
      const float sc = (P == kFP8 && row < N) ? a.in_scale * a.w_scale[row] : 1.0f;
      y[r] = acc[r] * sc;
    }
    if (EPI == kEpiStore || EPI == kEpiHead) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) if (row0 + r < N) a.out[row0 + r] = y[r];
    } else if (EPI == kEpiResid) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) if (row0 + r < N) a.out[row0 + r] += y[r];
    } else {  // SiLU*mul over interleaved (gate, up) row pairs
      float mx = 0.0f;
#pragma unroll
      for (int r = 0; r + 1 < ROWS; r += 2) {
        if (row0 + r + 1 < N) {
          const float v = silu(y[r]) * y[r + 1];
          mx = fmaxf(mx, fabsf(v));
          const int j = (row0 + r) >> 1;
          if (P == kBF16) static_cast<uint16_t*>(a.out_act)[j] = (uint16_t)act_encode<P>(v, a.out_scale);
          else static_cast<uint8_t*>(a.out_act)[j] = (uint8_t)act_encode<P>(v, a.out_scale);
        }
      }
      if (a.amax_out) record_amax(a.amax_out, mx);
    }
  }

  if (EPI != kEpiHead) return;

  // ---- head: the last block to finish takes the per-codebook argmax and the delay step
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(a.counter, 1u);
    sh_flag = (prev == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_flag) return;
  __threadfence();
  const int nw = blockDim.x >> 6;
  for (int k = wv; k < a.C; k += nw) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    const float* lg = a.out + (size_t)k * a.V;
    for (int i = lane; i < a.V; i += kWave) {
      const bool allowed = (i < a.bos) || (k == 0 && i == a.eos);
      if (!allowed) continue;
      const float v = lg[i];
      if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) sh_arg[k] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    DevState* st = a.st;
    const int t = st->t, eoc = st->eoc;
    int codes[kMaxCodebooks];
    for (int k = 0; k < a.C; ++k) {
      int c;
      if (t < k) c = a.bos;
      else if (eoc >= 0 && t >= eoc + k) c = a.eos;
      else c = sh_arg[k];
      codes[k] = c;
    }
    const int eoc2 = eoc >= 0 ? eoc : (codes[0] == a.eos ? t : -1);
    const int done = (eoc2 >= 0 && t >= eoc2 + a.C - 1) ? 1 : 0;
    for (int k = 0; k < a.C; ++k) {
      st->codes[k] = codes[k];
      st->prev[k] = codes[k];
      a.hist[(size_t)t * a.C + k] = codes[k];
    }
    st->t = t + 1;
    st->len = st->len + 1;
    st->done = done;
    st->n_done += done;
    *a.counter = 0u;
    __threadfence();
  }
}

// ============================================================================ attention (decode)
struct AttnArgs {
  const float* qkv;          // [Hq*hd | Hkv*hd | Hkv*hd]
  const float* g_q;
  const float* g_k;
  const float* rope_cos;     // [max_seq][hd/2]
  const float* rope_sin;
  uint16_t* k_cache;         // layer base [Hkv][max_seq][hd]
  uint16_t* v_cache;
  const DevState* st;
  float* part;               // [Hq][splits][hd + 2]
  unsigned* counters;        // [Hkv]
  void* o_act;               // [Hq*hd]
  float o_scale;
  float* amax;               // record slot of the attention-output site
  float eps;
  int max_seq, Hq, Hkv, splits;
  int pos_override;          // >= 0: position to use instead of the state (single-layer step)
};

template <int HD>
__device__ __forceinline__ void norm_rope_head(const float* __restrict__ src, const float* __restrict__ g,
                                               const float* __restrict__ cs, const float* __restrict__ sn,
                                               float eps, int lane, float* __restrict__ dst) {
  constexpr int H2 = HD / 2;
  const bool act = lane < H2;
  const float x0 = act ? src[lane] : 0.0f;
  const float x1 = act ? src[lane + H2] : 0.0f;
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float rstd = 1.0f / sqrtf(ss / (float)HD + eps);
  if (act) {
    const float a = x0 * rstd * g[lane];
    const float b = x1 * rstd * g[lane + H2];
    const float c = cs[lane], s = sn[lane];
    dst[lane] = round_bf16(a * c - b * s);
    dst[lane + H2] = round_bf16(b * c + a * s);
  }
}

template <int P, int HD>
__global__ __launch_bounds__(256) void k_attn_decode(AttnArgs a) {
  constexpr int H2 = HD / 2;
  constexpr int T = kAttnTile;
  __shared__ float qs[4][HD];
  __shared__ float kn[HD], vn[HD];
  __shared__ float Kt[T][HD + 1];
  __shared__ float Vt[T][HD];
  __shared__ float ps[4][T];
  __shared__ int sh_last;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = blockIdx.y, split = blockIdx.x;
  const int G = a.Hq / a.Hkv;
  const int pos = a.pos_override >= 0 ? a.pos_override : a.st->len;
  const int L = pos + 1;
  int chunk = (L + a.splits - 1) / a.splits;
  chunk = (chunk + T - 1) / T * T;
  const int beg = split * chunk;
  const int end = min(L, beg + chunk);
  const float* cs = a.rope_cos + (size_t)pos * H2;
  const float* sn = a.rope_sin + (size_t)pos * H2;

  if (w < G) norm_rope_head<HD>(a.qkv + (size_t)(j * G + w) * HD, a.g_q, cs, sn, a.eps, lane, qs[w]);
  if (w == (G < 4 ? G : 3)) {
    // the new key (q/k-norm + RoPE) and value, rounded to the bf16 cache format
    norm_rope_head<HD>(a.qkv + (size_t)a.Hq * HD + (size_t)j * HD, a.g_k, cs, sn, a.eps, lane, kn);
  }
  __syncthreads();
  if (tid < HD) vn[tid] = round_bf16(a.qkv[(size_t)(a.Hq + a.Hkv) * HD + (size_t)j * HD + tid]);
  __syncthreads();
  uint16_t* kc = a.k_cache + (size_t)j * a.max_seq * HD;
  uint16_t* vc = a.v_cache + (size_t)j * a.max_seq * HD;
  if (beg <= pos && pos < end && tid < HD) {
    kc[(size_t)pos * HD + tid] = (uint16_t)f32_to_bf16(kn[tid]);
    vc[(size_t)pos * HD + tid] = (uint16_t)f32_to_bf16(vn[tid]);
  }

  const float inv_sqrt = 1.0f / sqrtf((float)HD);
  float m = -INFINITY, lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int t0 = beg; t0 < end; t0 += T) {
    // stage the K/V tile in LDS (16-byte packets)
    constexpr int SEG = HD / 8;
    for (int idx = tid; idx < T * SEG; idx += blockDim.x) {
      const int key = idx / SEG, seg = idx % SEG;
      const int kp = t0 + key;
      float kv[8], vv[8];
      if (kp < end && kp != pos) {
        const uint4 kw = *reinterpret_cast<const uint4*>(kc + (size_t)kp * HD + seg * 8);
        const uint4 vw = *reinterpret_cast<const uint4*>(vc + (size_t)kp * HD + seg * 8);
        kv[0] = bf16lo(kw.x); kv[1] = bf16hi(kw.x); kv[2] = bf16lo(kw.y); kv[3] = bf16hi(kw.y);
        kv[4] = bf16lo(kw.z); kv[5] = bf16hi(kw.z); kv[6] = bf16lo(kw.w); kv[7] = bf16hi(kw.w);
        vv[0] = bf16lo(vw.x); vv[1] = bf16hi(vw.x); vv[2] = bf16lo(vw.y); vv[3] = bf16hi(vw.y);
        vv[4] = bf16lo(vw.z); vv[5] = bf16hi(vw.z); vv[6] = bf16lo(vw.w); vv[7] = bf16hi(vw.w);
      } else if (kp == pos && kp < end) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kv[e] = kn[seg * 8 + e]; vv[e] = vn[seg * 8 + e]; }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kv[e] = 0.0f; vv[e] = 0.0f; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) { Kt[key][seg * 8 + e] = kv[e]; Vt[key][seg * 8 + e] = vv[e]; }
    }
    __syncthreads();
    float scale = 1.0f, mnew = m;
    if (w < G) {
      const int kp = t0 + lane;
      float s = -INFINITY;
      if (kp < end) {
        float d = 0.0f;
#pragma unroll 8
        for (int e = 0; e < HD; ++e) d = fmaf(qs[w][e], Kt[lane][e], d);
        s = d * inv_sqrt;
      }
      mnew = fmaxf(m, wave_max(s));
      const float p = (kp < end) ? __expf(s - mnew) : 0.0f;
      scale = __expf(m - mnew);
      lsum = lsum * scale + wave_sum(p);
      ps[w][lane] = p;
    }
    __syncthreads();
    if (w < G) {
      o0 *= scale;
      o1 *= scale;
      for (int kk = 0; kk < T; ++kk) {
        const float p = ps[w][kk];
        if (lane < HD) o0 = fmaf(p, Vt[kk][lane], o0);
        if (HD > 64) o1 = fmaf(p, Vt[kk][(lane + 64) % HD], o1);
      }
      m = mnew;
    }
    __syncthreads();
  }

  // ---- split partial (m, l, o)
  if (w < G) {
    const int h = j * G + w;
    float* pp = a.part + ((size_t)h * a.splits + split) * (HD + 2);
    if (lane < HD) pp[lane] = o0;
    if (HD > 64) pp[lane + 64] = o1;
    if (lane == 0) { pp[HD] = m; pp[HD + 1] = lsum; }
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(a.counters + j, 1u);
    sh_last = (prev == (unsigned)a.splits - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  // ---- the last split block of this kv head merges the partials (log-sum-exp)
  if (w < G) {
    const int h = j * G + w;
    const float* pb = a.part + (size_t)h * a.splits * (HD + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) {
      const float ls = pb[(size_t)s * (HD + 2) + HD + 1];
      if (ls > 0.0f) M = fmaxf(M, pb[(size_t)s * (HD + 2) + HD]);
    }
    float den = 0.0f, n0 = 0.0f, n1 = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
      const float* q = pb + (size_t)s * (HD + 2);
      const float ls = q[HD + 1];
      if (!(ls > 0.0f)) continue;
      const float f = __expf(q[HD] - M);
      den = fmaf(f, ls, den);
      if (lane < HD) n0 = fmaf(f, q[lane], n0);
      if (HD > 64) n1 = fmaf(f, q[lane + 64], n1);
    }
    const float inv = 1.0f / den;
    const float v0 = n0 * inv, v1 = n1 * inv;
    float mx = (lane < HD) ? fabsf(v0) : 0.0f;
    if (HD > 64) mx = fmaxf(mx, fabsf(v1));
    if (P == kBF16) {
      uint16_t* o = static_cast<uint16_t*>(a.o_act) + (size_t)h * HD;
      if (lane < HD) o[lane] = (uint16_t)act_encode<P>(v0, a.o_scale);
      if (HD > 64) o[lane + 64] = (uint16_t)act_encode<P>(v1, a.o_scale);
    } else {
      uint8_t* o = static_cast<uint8_t*>(a.o_act) + (size_t)h * HD;
      if (lane < HD) o[lane] = (uint8_t)act_encode<P>(v0, a.o_scale);
      if (HD > 64) o[lane + 64] = (uint8_t)act_encode<P>(v1, a.o_scale);
    }
    if (a.amax) {
      mx = wave_max(mx);
      if (lane == 0) record_amax(a.amax, mx);
    }
  }
  if (tid == 0) a.counters[j] = 0u;
}

// ============================================================================ small state kernels
__global__ void k_set_prev(DevState* st, int c0, int c1, int c2, int c3, int c4, int c5, int c6, int c7,
                           int c8, int c9, int c10, int c11, int c12, int c13, int c14, int c15, int C) {
  const int cs[16] = {c0, c1, c2, c3, c4, c5, c6, c7, c8, c9, c10, c11, c12, c13, c14, c15};
  if (threadIdx.x < C) st->prev[threadIdx.x] = cs[threadIdx.x];
}

__global__ void k_reset_state(DevState* st, int len, int C, int bos) {
  if (threadIdx.x == 0) {
    st->len = len;
    st->t = 0;
    st->eoc = -1;
    st->done = 0;
    st->n_done = 0;
  }
  if (threadIdx.x < C) {
    st->prev[threadIdx.x] = bos;
    st->codes[threadIdx.x] = bos;
  }
}

__global__ void k_set_len(DevState* st, int len) {
  if (threadIdx.x == 0) st->len = len;
}

// ============================================================================ launchers
template <int P, int ROWS, int PRO, int EPI>
static hipError_t gemv(const Ctx& c, GemvArgs a) {
  const int waves = 4;
  const int rows_per_block = waves * ROWS;
  const int grid = (a.N + rows_per_block - 1) / rows_per_block;
  const size_t lds = (size_t)a.K * sizeof(float);
  hipLaunchKernelGGL((k_gemv<P, ROWS, PRO, EPI>), dim3(grid), dim3(64 * waves), lds, c.stream, a);
  return hipGetLastError();
}

hipError_t launch_frame_begin(Ctx& c) {
  const auto& f = c.cfg;
  hipLaunchKernelGGL(k_frame_begin, dim3((f.hidden + 255) / 256), dim3(256), 0, c.stream, c.e_aud, c.state, c.h,
                     f.hidden, f.n_codebooks, f.codebook_size, f.eos_id);
  return hipGetLastError();
}

// Host copies of the activation scales live in c (set at load); the kernels take them by value.
extern float host_act_scale(const Ctx& c, int site);

template <int P>
static hipError_t layer_decode_p(Ctx& c, int layer, float* h, bool record, int pos_override) {
  const auto& f = c.cfg;
  const LayerW& L = c.layers[layer];
  const int d = f.hidden, hd = f.head_dim, qd = f.n_q_heads * hd, kvd = f.n_kv_heads * hd, F = f.ffn;
  const int s0 = kSitesPerLayer * layer;
  float* amax = record ? c.amax : nullptr;
  hipError_t e;
  // qkv = W_qkv . round(rmsnorm(h))
  {
    GemvArgs a{};
    a.w = L.w_qkv; a.w_scale = L.s_qkv; a.N = qd + 2 * kvd; a.K = d;
    a.h = h; a.g = L.g_attn; a.eps = f.rms_eps; a.in_scale = host_act_scale(c, s0);
    a.amax_in = amax ? amax + s0 : nullptr; a.out = c.qkv;
    if ((e = gemv<P, 4, kProNorm, kEpiStore>(c, a)) != hipSuccess) return e;
  }
  // attention (q/k-norm + RoPE + KV write + split-K + combine)
  {
    AttnArgs a{};
    a.qkv = c.qkv; a.g_q = L.g_q; a.g_k = L.g_k; a.rope_cos = c.rope_cos; a.rope_sin = c.rope_sin;
    a.k_cache = L.k_cache; a.v_cache = L.v_cache; a.st = c.state; a.part = c.attn_part;
    a.counters = c.counters; a.o_act = c.o_act; a.o_scale = host_act_scale(c, s0 + 1);
    a.amax = amax ? amax + s0 + 1 : nullptr; a.eps = f.rms_eps; a.max_seq = f.max_seq;
    a.Hq = f.n_q_heads; a.Hkv = f.n_kv_heads; a.splits = c.lay.attn_splits; a.pos_override = pos_override;
    dim3 grid(a.splits, f.n_kv_heads);
    if (hd == 128) hipLaunchKernelGGL((k_attn_decode<P, 128>), grid, dim3(256), 0, c.stream, a);
    else hipLaunchKernelGGL((k_attn_decode<P, 64>), grid, dim3(256), 0, c.stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // h += W_o . o
  {
    GemvArgs a{};
    a.w = L.w_o; a.w_scale = L.s_o; a.N = d; a.K = qd; a.x_act = c.o_act; a.in_scale = host_act_scale(c, s0 + 1);
    a.out = h;
    if ((e = gemv<P, 1, kProAct, kEpiResid>(c, a)) != hipSuccess) return e;
  }
  // a = round(silu(W_g . u2) * (W_u . u2)), u2 = round(rmsnorm(h))
  {
    GemvArgs a{};
    a.w = L.w_gu; a.w_scale = L.s_gu; a.N = 2 * F; a.K = d;
    a.h = h; a.g = L.g_mlp; a.eps = f.rms_eps; a.in_scale = host_act_scale(c, s0 + 2);
    a.amax_in = amax ? amax + s0 + 2 : nullptr;
    a.out_act = c.a_act; a.out_scale = host_act_scale(c, s0 + 3); a.amax_out = amax ? amax + s0 + 3 : nullptr;
    if ((e = gemv<P, 4, kProNorm, kEpiSilu>(c, a)) != hipSuccess) return e;
  }
  // h += W_d . a
  {
    GemvArgs a{};
    a.w = L.w_d; a.w_scale = L.s_d; a.N = d; a.K = F; a.x_act = c.a_act; a.in_scale = host_act_scale(c, s0 + 3);
    a.out = h;
    if ((e = gemv<P, 1, kProAct, kEpiResid>(c, a)) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_layer_decode_at(Ctx& c, int layer, float* h, bool record, int pos_override) {
  if (c.cfg.precision == HTA_FP8_E4M3) return layer_decode_p<kFP8>(c, layer, h, record, pos_override);
  return layer_decode_p<kBF16>(c, layer, h, record, pos_override);
}

hipError_t launch_layer_decode(Ctx& c, int layer, float* h, bool record) {
  return launch_layer_decode_at(c, layer, h, record, -1);
}

template <int P>
static hipError_t head_p(Ctx& c, bool record) {
  const auto& f = c.cfg;
  const int site = kSitesPerLayer * f.n_layers;
  GemvArgs a{};
  a.w = c.w_head; a.w_scale = c.s_head; a.N = f.n_codebooks * f.codebook_size; a.K = f.hidden;
  a.h = c.h; a.g = c.g_final; a.eps = f.rms_eps; a.in_scale = host_act_scale(c, site);
  a.amax_in = record ? c.amax + site : nullptr; a.out = c.logits;
  a.counter = c.counters + 32; a.st = c.state; a.hist = c.hist;
  a.C = f.n_codebooks; a.V = f.codebook_size; a.bos = f.bos_id; a.eos = f.eos_id;
  return gemv<P, 2, kProNorm, kEpiHead>(c, a);
}

hipError_t launch_head(Ctx& c, bool record) {
  if (c.cfg.precision == HTA_FP8_E4M3) return head_p<kFP8>(c, record);
  return head_p<kBF16>(c, record);
}

hipError_t launch_set_prev(Ctx& c, const int32_t* v) {
  int cs[16] = {0};
  for (int i = 0; i < c.cfg.n_codebooks; ++i) cs[i] = v[i];
  hipLaunchKernelGGL(k_set_prev, dim3(1), dim3(64), 0, c.stream, c.state, cs[0], cs[1], cs[2], cs[3], cs[4], cs[5],
                     cs[6], cs[7], cs[8], cs[9], cs[10], cs[11], cs[12], cs[13], cs[14], cs[15], c.cfg.n_codebooks);
  return hipGetLastError();
}

hipError_t launch_reset_state(Ctx& c, int keep_len) {
  hipLaunchKernelGGL(k_reset_state, dim3(1), dim3(64), 0, c.stream, c.state, keep_len, c.cfg.n_codebooks,
                     c.cfg.bos_id);
  return hipGetLastError();
}

hipError_t launch_set_len(Ctx& c, int len) {
  hipLaunchKernelGGL(k_set_len, dim3(1), dim3(64), 0, c.stream, c.state, len);
  return hipGetLastError();
}

}  // namespace hta
