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
  int code[kMaxCodebooks];
#pragma unroll
  for (int c = 0; c < kMaxCodebooks; ++c) code[c] = c < C ? st->prev[c] : 0;
  float v[kMaxCodebooks];
#pragma unroll
  for (int c = 0; c < kMaxCodebooks; ++c) v[c] = c < C ? bf16_to_f32(e_aud[((size_t)c * V + code[c]) * d + k]) : 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxCodebooks; ++c) s += v[c];  // codebook order
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

// Each wave owns ROWS consecutive rows and issues every 16-byte weight packet of
// those rows (MAXC packets per row and lane) before the prologue, so the
// prologue's own loads and reductions overlap the weight stream.
constexpr int kProMax = 5;  // 16-byte prologue packets per thread (K <= 5120 fp32 / 10240 bf16)

template <int P, int ROWS, int MAXC, int PRO, int EPI>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  extern __shared__ float smem[];
  float* xs = smem;            // [K] activations in GEMV units
  __shared__ float red[16];
  __shared__ int sh_flag;
  __shared__ int sh_arg[kMaxCodebooks];
  const int K = a.K, N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nthr = blockDim.x;
  constexpr int E = WTraits<P>::E;
  constexpr int CH = kWave * E;
  const int row0 = (blockIdx.x * (blockDim.x >> 6) + wv) * ROWS;
  const int nch = (K + CH - 1) / CH;

  // ---- prologue inputs first (small), so they return ahead of the weights
  float4 hv[kProMax], gv[kProMax];
  uint4 xv[kProMax];
  if (PRO == kProNorm) {
#pragma unroll
    for (int p = 0; p < kProMax; ++p) {
      const int idx = (p * nthr + tid) * 4;
      if (idx < K) {
        hv[p] = *reinterpret_cast<const float4*>(a.h + idx);
        gv[p] = *reinterpret_cast<const float4*>(a.g + idx);
      }
    }
  } else {
    constexpr int XE = (P == kBF16) ? 8 : 16;  // elements per 16-byte packet
#pragma unroll
    for (int p = 0; p < kProMax; ++p) {
      const int idx = (p * nthr + tid) * XE;
      if (idx < K) xv[p] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.x_act) + (size_t)idx * WTraits<P>::B);
    }
  }

  // ---- the weight stream of this wave
  uint4 wr[ROWS][MAXC];
  const uint8_t* wb = static_cast<const uint8_t*>(a.w);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = c * CH + lane * E;
    const bool ok = (c < nch) && (e < K);
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int row = row0 + r;
      if (ok && row < N) wr[r][c] = ld_stream16(wb + ((size_t)row * K + e) * WTraits<P>::B);
      else wr[r][c] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // ---- prologue: the input vector in LDS, in GEMV units
  if (PRO == kProNorm) {
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < kProMax; ++p) {
      const int idx = (p * nthr + tid) * 4;
      if (idx < K) {
        ss = fmaf(hv[p].x, hv[p].x, ss); ss = fmaf(hv[p].y, hv[p].y, ss);
        ss = fmaf(hv[p].z, hv[p].z, ss); ss = fmaf(hv[p].w, hv[p].w, ss);
      }
    }
    ss = block_sum(ss, red);
    const float rstd = 1.0f / sqrtf(ss / (float)K + a.eps);
    float mx = 0.0f;
#pragma unroll
    for (int p = 0; p < kProMax; ++p) {
      const int idx = (p * nthr + tid) * 4;
      if (idx < K) {
        const float u0 = hv[p].x * rstd * gv[p].x, u1 = hv[p].y * rstd * gv[p].y;
        const float u2 = hv[p].z * rstd * gv[p].z, u3 = hv[p].w * rstd * gv[p].w;
        mx = fmaxf(fmaxf(mx, fmaxf(fabsf(u0), fabsf(u1))), fmaxf(fabsf(u2), fabsf(u3)));
        xs[idx] = act_round<P>(u0, a.in_scale);
        xs[idx + 1] = act_round<P>(u1, a.in_scale);
        xs[idx + 2] = act_round<P>(u2, a.in_scale);
        xs[idx + 3] = act_round<P>(u3, a.in_scale);
      }
    }
    if (a.amax_in != nullptr && blockIdx.x == 0) {
      mx = block_max(mx, red);
      if (tid == 0) record_amax(a.amax_in, mx);
    }
  } else {
    constexpr int XE = (P == kBF16) ? 8 : 16;
#pragma unroll
    for (int p = 0; p < kProMax; ++p) {
      const int idx = (p * nthr + tid) * XE;
      if (idx < K) {
        const uint32_t ws[4] = {xv[p].x, xv[p].y, xv[p].z, xv[p].w};
        if (P == kBF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) { xs[idx + 2 * q] = bf16lo(ws[q]); xs[idx + 2 * q + 1] = bf16hi(ws[q]); }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[q], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[q], true);
            xs[idx + 4 * q] = lo[0]; xs[idx + 4 * q + 1] = lo[1]; xs[idx + 4 * q + 2] = hi[0]; xs[idx + 4 * q + 3] = hi[1];
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- dot products
  float acc[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = c * CH + lane * E;
    if ((c < nch) && (e < K)) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) acc[r] += dot16<P>(wr[r][c], xs + e);
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
  constexpr int kVPL = 32;  // logits per lane: codebook_size <= 2048
  for (int k = wv; k < a.C; k += nw) {
    const float* lg = a.out + (size_t)k * a.V;
    float v[kVPL];
#pragma unroll
    for (int q = 0; q < kVPL; ++q) {
      const int i = q * kWave + lane;
      v[q] = i < a.V ? lg[i] : -INFINITY;
    }
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kVPL; ++q) {
      const int i = q * kWave + lane;
      const bool allowed = i < a.V && ((i < a.bos) || (k == 0 && i == a.eos));
      // a NaN logit never wins: with every allowed logit NaN the lowest allowed id is
      // chosen, so the code stays a valid embedding row
      const float x = v[q] == v[q] ? v[q] : -INFINITY;
      if (allowed && (x > bv || (x == bv && i < bi))) { bv = x; bi = i; }
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

// Split-K flash decoding.  Grid (splits, Hkv); block = 4 waves, wave w owns q
// head j*G + w of the kv head's group.  Keys are cut into `splits` chunks of a
// whole number of 64-key tiles (the chunk depends only on the length), so
// only ceil(L / chunk) splits hold keys; the others exit at once.  Each active
// split stages its K/V tiles in LDS, keeps an online softmax (m, l, o) and
// writes it; the last active split to finish merges the partials with the
// log-sum-exp rule and writes the rounded attention output.
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
  const int n_active = (L + chunk - 1) / chunk;
  if (split >= n_active) return;
  const int beg = split * chunk;
  const int end = min(L, beg + chunk);
  const float* cs = a.rope_cos + (size_t)pos * H2;
  const float* sn = a.rope_sin + (size_t)pos * H2;

  if (w < G) norm_rope_head<HD>(a.qkv + (size_t)(j * G + w) * HD, a.g_q, cs, sn, a.eps, lane, qs[w]);
  if (w == (G < 4 ? G : 3)) {
    // the new key (q/k-norm + RoPE) and value, rounded to the bf16 cache format
    norm_rope_head<HD>(a.qkv + (size_t)a.Hq * HD + (size_t)j * HD, a.g_k, cs, sn, a.eps, lane, kn);
  }
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
    constexpr int SEG = HD / 8;
    constexpr int PER = T * SEG / 256;  // 16-byte packets per thread per tile
    uint4 kw[PER], vw[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = q * 256 + tid;
      const int key = idx / SEG, seg = idx % SEG;
      const int kp = t0 + key;
      if (kp < end && kp != pos) {
        kw[q] = *reinterpret_cast<const uint4*>(kc + (size_t)kp * HD + seg * 8);
        vw[q] = *reinterpret_cast<const uint4*>(vc + (size_t)kp * HD + seg * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = q * 256 + tid;
      const int key = idx / SEG, seg = idx % SEG;
      const int kp = t0 + key;
      float kv[8], vv[8];
      if (kp < end && kp != pos) {
        const uint32_t ks[4] = {kw[q].x, kw[q].y, kw[q].z, kw[q].w}, vs[4] = {vw[q].x, vw[q].y, vw[q].z, vw[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[2 * e] = bf16lo(ks[e]); kv[2 * e + 1] = bf16hi(ks[e]);
          vv[2 * e] = bf16lo(vs[e]); vv[2 * e + 1] = bf16hi(vs[e]);
        }
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
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll 8
        for (int e = 0; e < HD; e += 2) {
          d0 = fmaf(qs[w][e], Kt[lane][e], d0);
          d1 = fmaf(qs[w][e + 1], Kt[lane][e + 1], d1);
        }
        s = (d0 + d1) * inv_sqrt;
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
      const int nk = min(T, end - t0);
      for (int kk = 0; kk < nk; ++kk) {
        const float p = ps[w][kk];
        if (lane < HD) o0 = fmaf(p, Vt[kk][lane], o0);
        if (HD > 64) o1 = fmaf(p, Vt[kk][(lane + 64) % HD], o1);
      }
      m = mnew;
    }
    __syncthreads();
  }

  // ---- one active split: no merge needed
  if (n_active == 1) {
    if (w < G) {
      const int h = j * G + w;
      const float inv = 1.0f / lsum;
      const float v0 = o0 * inv, v1 = o1 * inv;
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
    return;
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
    sh_last = (prev == (unsigned)n_active - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  // ---- the last active split of this kv head merges the partials (log-sum-exp)
  if (w < G) {
    const int h = j * G + w;
    const float* pb = a.part + (size_t)h * a.splits * (HD + 2);
    // lane s holds split s's (m, l); n_active <= splits <= 64
    const bool has = lane < n_active;
    const float ms = has ? pb[(size_t)lane * (HD + 2) + HD] : -INFINITY;
    const float ls = has ? pb[(size_t)lane * (HD + 2) + HD + 1] : 0.0f;
    const float M = wave_max(ls > 0.0f ? ms : -INFINITY);
    const float f = (ls > 0.0f) ? __expf(ms - M) : 0.0f;
    const float den = wave_sum(f * ls);
    float n0 = 0.0f, n1 = 0.0f;
    for (int s0 = 0; s0 < n_active; s0 += 8) {
      float x0[8], x1[8], fs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sp = s0 + u;
        fs[u] = __shfl(f, sp < n_active ? sp : 0, kWave);
        const float* q = pb + (size_t)sp * (HD + 2);
        x0[u] = (sp < n_active && lane < HD) ? q[lane] : 0.0f;
        x1[u] = (sp < n_active && HD > 64) ? q[lane + 64] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u < n_active) {
          n0 = fmaf(fs[u], x0[u], n0);
          n1 = fmaf(fs[u], x1[u], n1);
        }
      }
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
template <int P, int ROWS, int MAXC, int PRO, int EPI>
static hipError_t gemv_launch(Ctx& c, const GemvArgs& a, int kclass) {
  const int waves = 4;
  const int rows_per_block = waves * ROWS;
  const int grid = (a.N + rows_per_block - 1) / rows_per_block;
  const size_t lds = (size_t)a.K * sizeof(float);
  time_begin(c, kclass);
  hipLaunchKernelGGL((k_gemv<P, ROWS, MAXC, PRO, EPI>), dim3(grid), dim3(64 * waves), lds, c.stream, a);
  time_end(c);
  return hipGetLastError();
}

// Picks the register budget (16-byte packets per row and lane) from K.
template <int P, int ROWS, int PRO, int EPI>
static hipError_t gemv(Ctx& c, GemvArgs a, int kclass) {
  constexpr int CH = kWave * WTraits<P>::E;
  const int nch = (a.K + CH - 1) / CH;
  if (nch <= 2) return gemv_launch<P, ROWS, 2, PRO, EPI>(c, a, kclass);
  if (nch <= 3) return gemv_launch<P, ROWS, 3, PRO, EPI>(c, a, kclass);
  if (nch <= 5) return gemv_launch<P, ROWS, 5, PRO, EPI>(c, a, kclass);
  if constexpr (ROWS == 4) {
    return gemv<P, 2, PRO, EPI>(c, a, kclass);  // wide rows: halve the rows per wave
  } else {
    if (nch <= 8) return gemv_launch<P, ROWS, 8, PRO, EPI>(c, a, kclass);
    if (nch <= 10) return gemv_launch<P, ROWS, 10, PRO, EPI>(c, a, kclass);
    if (nch <= 19) return gemv_launch<P, ROWS, 19, PRO, EPI>(c, a, kclass);
    if (nch <= 32) return gemv_launch<P, ROWS, 32, PRO, EPI>(c, a, kclass);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_frame_begin(Ctx& c) {
  const auto& f = c.cfg;
  time_begin(c, HTA_K_EMBED);
  hipLaunchKernelGGL(k_frame_begin, dim3((f.hidden + 255) / 256), dim3(256), 0, c.stream, c.e_aud, c.state, c.h,
                     f.hidden, f.n_codebooks, f.codebook_size, f.eos_id);
  time_end(c);
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
    if ((e = gemv<P, 4, kProNorm, kEpiStore>(c, a, HTA_K_QKV)) != hipSuccess) return e;
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
    time_begin(c, HTA_K_ATTN);
    if (hd == 128) hipLaunchKernelGGL((k_attn_decode<P, 128>), grid, dim3(256), 0, c.stream, a);
    else hipLaunchKernelGGL((k_attn_decode<P, 64>), grid, dim3(256), 0, c.stream, a);
    time_end(c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // h += W_o . o
  {
    GemvArgs a{};
    a.w = L.w_o; a.w_scale = L.s_o; a.N = d; a.K = qd; a.x_act = c.o_act; a.in_scale = host_act_scale(c, s0 + 1);
    a.out = h;
    if ((e = gemv<P, 1, kProAct, kEpiResid>(c, a, HTA_K_O)) != hipSuccess) return e;
  }
  // a = round(silu(W_g . u2) * (W_u . u2)), u2 = round(rmsnorm(h))
  {
    GemvArgs a{};
    a.w = L.w_gu; a.w_scale = L.s_gu; a.N = 2 * F; a.K = d;
    a.h = h; a.g = L.g_mlp; a.eps = f.rms_eps; a.in_scale = host_act_scale(c, s0 + 2);
    a.amax_in = amax ? amax + s0 + 2 : nullptr;
    a.out_act = c.a_act; a.out_scale = host_act_scale(c, s0 + 3); a.amax_out = amax ? amax + s0 + 3 : nullptr;
    if ((e = gemv<P, 4, kProNorm, kEpiSilu>(c, a, HTA_K_GATEUP)) != hipSuccess) return e;
  }
  // h += W_d . a
  {
    GemvArgs a{};
    a.w = L.w_d; a.w_scale = L.s_d; a.N = d; a.K = F; a.x_act = c.a_act; a.in_scale = host_act_scale(c, s0 + 3);
    a.out = h;
    if ((e = gemv<P, 1, kProAct, kEpiResid>(c, a, HTA_K_DOWN)) != hipSuccess) return e;
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
  return gemv<P, 2, kProNorm, kEpiHead>(c, a, HTA_K_HEAD);
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
