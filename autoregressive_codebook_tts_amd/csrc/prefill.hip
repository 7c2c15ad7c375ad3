// Batched prefill (M = P rows) for gfx950: embedding gather, row RMSNorm +
// activation rounding, MFMA GEMMs (bf16 16x16x32; e4m3 operands widened to
// bf16 in registers) with a
// fixed, P-independent reduction order, fused q/k-norm + RoPE + KV write, and
// causal attention over key tiles aligned to absolute positions.
//
// Reference: FlashRT "Higgs Audio v3 TTS-4B" page, section 7 (the prompt is
// prefilled in one batched M = P forward; a shared preamble's KV is reused and
// the result is bit-identical to a cold prefill) and the Performance section
// (batched BF16/FP8 prefill).  Bit-identity under prefix reuse requires that
// every output row is computed the same way whatever P or the start offset is:
// the GEMM's K order and split depend only on (N, K), and attention walks key
// tiles at absolute multiples of 64.
#include "device_common.h"
#include "hta_internal.h"

namespace hta {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// 8 e4m3 codes (two dwords) -> 8 bf16 values, exactly (hardware pair convert, scale 1).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// One 16x16 tile over a 128-element step on the e4m3 MFMA (the opt-in fast form): each
// lane gives 32 bytes of its A row and of its B row, the 16-byte units u0 and u1 of the
// step, the same units in both operands.  The instruction sums its e4m3 products in groups
// with fewer bits than fp32 (a product 2^-18 beside a product 1 is dropped), so its results
// differ from fp32 accumulation by up to about 2^-19 of the sum of |products|.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_e4m3_step(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
  const i32x8 a{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 b{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  // formats 0 / 0: e4m3 operands; scale operands 0: no block scaling
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

extern float host_act_scale(const Ctx& c, int site);

// ============================================================================ rows
__global__ __launch_bounds__(256) void k_embed_rows(const int32_t* __restrict__ tok, const uint16_t* __restrict__ e_text,
                                                    float* __restrict__ X, int d) {
  const int i = blockIdx.x;
  const size_t t = (size_t)tok[i];
  for (int k = threadIdx.x; k < d; k += blockDim.x) X[(size_t)i * d + k] = bf16_to_f32(e_text[t * d + k]);
}

// The row kernels issue all of a thread's loads before using any (clamped addresses,
// no load under a condition): a loop that loads and uses one element per step waits
// a memory round trip per element.
constexpr int kRowPerMax = 20;  // row elements per thread of the row kernels (rows up to 20 * 256)

// The sum of a column's K-split partials in split order, scaled as k_gemm_reduce
// scales it (the rounding sequence of k_gemm_reduce, so fusing changes no bit).
struct SplitIn {
  const float* part;     // [ks][M][N] partials, or null: no split to add
  int ks;
  long plane;            // M * N
  const float* w_scale;  // e4m3 per-row weight scales, or null
  float in_scale;
};
constexpr int kMaxSplit = 8;  // gemm_ksplit's cap
// out[u] = the split sum at element idx[u] (column col[u]) for U elements; KS >= si.ks.
// Every load is issued before the first add (clamped split indices, no load under a
// condition), so a thread waits one memory round trip, not one per split.
template <int U, int KS>
__device__ __forceinline__ void split_sums(const SplitIn& si, const long (&idx)[U], const int (&col)[U],
                                           float (&out)[U]) {
  float pv[U][KS], ws[U];
  const float* wp = si.w_scale ? si.w_scale : si.part;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int k = 0; k < KS; ++k) pv[u][k] = si.part[(long)min(k, si.ks - 1) * si.plane + idx[u]];
    ws[u] = wp[si.w_scale ? col[u] : 0];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (k < si.ks) s += pv[u][k];
    if (si.w_scale) s *= si.in_scale * ws[u];
    out[u] = s;
  }
}

// block_sum for blocks of exactly NWV waves (the same additions in the same order,
// without the loop over a run-time wave count).
template <int NWV>
__device__ __forceinline__ float block_sum_n(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NWV; ++i) s += red[i];
  return s;
}

// Row RMSNorm + rounding to the GEMV input format.  With a split input, the row is first
// updated as residual += (the split sum of the GEMM that produced it), the work of
// k_gemm_reduce, and the updated residual is stored and normalised.
// NT threads, RP row elements per thread (rows up to NT * RP); KS bounds the split count
// of the input (0: no split input), so that no thread issues loads beyond its row and
// splits.
template <int P, int RP, int KS, int NT>
__global__ __launch_bounds__(NT) void k_rmsnorm_act_rows(float* __restrict__ X, const float* __restrict__ g,
                                                          float eps, void* __restrict__ U, int d, float scale,
                                                          float* amax, SplitIn si) {
  __shared__ float red[16];
  const int i = blockIdx.x;
  float* x = X + (size_t)i * d;
  float xv[RP], gv[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int k = u * NT + threadIdx.x, kc = min(k, d - 1);
    xv[u] = x[kc];
    gv[u] = g[kc];
  }
  if (KS > 0 && si.part) {
    float sv[RP];
    long idx[RP];
    int col[RP];
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      col[u] = min(u * NT + (int)threadIdx.x, d - 1);
      idx[u] = (long)i * d + col[u];
    }
    split_sums<RP, (KS > 0 ? KS : 1)>(si, idx, col, sv);
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      const int k = u * NT + threadIdx.x;
      xv[u] += sv[u];
      if (k < d) x[k] = xv[u];
    }
  }
  float ss = 0.0f;  // over k = tid, tid + NT, ... in increasing order
#pragma unroll
  for (int u = 0; u < RP; ++u)
    if (u * NT + threadIdx.x < d) ss = fmaf(xv[u], xv[u], ss);
  ss = block_sum_n<NT / 64>(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
  // every element's value and code first (elements past the row are clamped copies,
  // computed and never stored), so that the per-element divisions of the e4m3 rounding
  // overlap instead of running one branch at a time
  float v[RP];
  uint32_t code[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    v[u] = xv[u] * rstd * gv[u];
    code[u] = act_encode<P>(v[u], scale);
  }
  float mx = 0.0f;
  auto put = [&](int u) {
    const int k = u * NT + threadIdx.x;
    mx = fmaxf(mx, fabsf(v[u]));
    if (P == kBF16) static_cast<uint16_t*>(U)[(size_t)i * d + k] = (uint16_t)code[u];
    else static_cast<uint8_t*>(U)[(size_t)i * d + k] = (uint8_t)code[u];
  };
  if (d == RP * NT) {  // uniform: every element lies in the row, no store is predicated
#pragma unroll
    for (int u = 0; u < RP; ++u) put(u);
  } else {
#pragma unroll
    for (int u = 0; u < RP; ++u)
      if (u * NT + (int)threadIdx.x < d) put(u);
  }
  if (amax) {
    mx = block_max(mx, red);
    if (threadIdx.x == 0) record_amax(amax, mx);
  }
}

// k_rmsnorm_act_rows over `rows` rows, with the narrowest instantiation for d and si.ks
// (the split bound rounds up: 2, 5 or 8 splits).
template <int P>
static void launch_rmsnorm_rows(hipStream_t st, int rows, float* X, const float* g, float eps, void* U, int d,
                                float scale, float* amax, const SplitIn& si) {
// 512 threads (two waves per SIMD, so that each wave's dependent chains are half as long
// and the other wave covers them); the shape depends on d only, so every caller sums a
// row in the same order.
#define HTA_NORM(RP, KS)                                                                                      \
  hipLaunchKernelGGL((k_rmsnorm_act_rows<P, RP, KS, 512>), dim3(rows), dim3(512), 0, st, X, g, eps, U, d, scale, \
                     amax, si)
  const int ks = si.part ? si.ks : 0;
  if (d <= 5 * 512) {
    if (ks == 0) HTA_NORM(5, 0);
    else if (ks <= 2) HTA_NORM(5, 2);
    else if (ks <= 5) HTA_NORM(5, 5);
    else HTA_NORM(5, 8);
  } else {
    if (ks == 0) HTA_NORM(10, 0);
    else if (ks <= 2) HTA_NORM(10, 2);
    else if (ks <= 5) HTA_NORM(10, 5);
    else HTA_NORM(10, 8);
  }
#undef HTA_NORM
}

template <int P>
__global__ __launch_bounds__(256) void k_silu_mul_rows(const float* __restrict__ GU, void* __restrict__ A, int F,
                                                       float scale, float* amax) {
  __shared__ float red[16];
  const int i = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  float mx = 0.0f;
  if (j < F) {
    const float gt = GU[(size_t)i * 2 * F + 2 * j], up = GU[(size_t)i * 2 * F + 2 * j + 1];
    const float v = silu(gt) * up;
    mx = fabsf(v);
    if (P == kBF16) static_cast<uint16_t*>(A)[(size_t)i * F + j] = (uint16_t)act_encode<P>(v, scale);
    else static_cast<uint8_t*>(A)[(size_t)i * F + j] = (uint8_t)act_encode<P>(v, scale);
  }
  if (amax) {
    mx = block_max(mx, red);
    if (threadIdx.x == 0) record_amax(amax, mx);
  }
}

// q/k RMSNorm + RoPE for one row of heads; rotated values rounded to bf16.
// (x0, x1: the lane's two elements of the head, lane < HD / 2; g0, g1 their gains;
// c, s the rotation of the lane's pair)
// The head row's sum of squares (the wave holds its two halves, x0 and x1, per lane).
__device__ __forceinline__ float norm_ss(float x0, float x1) { return wave_sum(__builtin_fmaf(x0, x0, x1 * x1)); }
// 1 / sqrt(ss / HD + eps) of the row.
template <int HD>
__device__ __forceinline__ float rstd_of(float ss, float eps) { return 1.0f / sqrtf(ss / (float)HD + eps); }
// rstd_of for N <= 64 rows at once: lane i evaluates row i's (the same operations on the
// same value, so the same bits), and each row's result is read back from its lane.
template <int HD, int N>
__device__ __forceinline__ void rstd_rows(const float (&ss)[N], float eps, float (&rstd)[N]) {
  static_assert(N <= 64, "one row per lane");
  const int lane = threadIdx.x & 63;
  float v = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) v = lane == i ? ss[i] : v;
  const float r = rstd_of<HD>(v, eps);
#pragma unroll
  for (int i = 0; i < N; ++i) rstd[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), i));
}
template <int HD>
__device__ __forceinline__ void rope_apply(float rstd, float x0, float x1, float g0, float g1, float c_, float s_,
                                           int lane, float* a_out, float* b_out) {
  constexpr int H2 = HD / 2;
  const bool act = lane < H2;
  const float a = x0 * rstd * (act ? g0 : 0.0f);
  const float b = x1 * rstd * (act ? g1 : 0.0f);
  const float c = act ? c_ : 0.0f, s = act ? s_ : 0.0f;
  // the fused forms are written out: left to contraction, the compiler picks the product
  // to fuse per call site, and two kernels would round the same rotation differently
  *a_out = round_bf16_sel(__builtin_fmaf(a, c, -(b * s)));
  *b_out = round_bf16_sel(__builtin_fmaf(b, c, a * s));
}

// The q/k/v row comes from QKV, or, with a split input, is the split sum of the GEMM's
// partials (the work of k_gemm_reduce, element by element in the same order; at most
// kRopeMaxSplit splits, so that every partial of a thread is loaded in one batch).
// NT threads, HPW heads per wave (Hq + Hkv <= NT / 64 HPW), VPER value elements per
// thread (Hkv HD <= NT VPER) and KS >= the split count (0: no split input), so that no
// thread issues loads beyond its heads and splits.
constexpr int kRopeMaxSplit = 4;
template <int HD, int HPW, int VPER, int KS, int NT>
__global__ __launch_bounds__(NT) void k_qk_rope_rows(const float* __restrict__ QKV, const float* __restrict__ g_q,
                                                      const float* __restrict__ g_k, const float* __restrict__ rope_cos,
                                                      const float* __restrict__ rope_sin, float* __restrict__ Q,
                                                      uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int* __restrict__ len_at,
                                                      int Hq, int Hkv, int max_seq, float eps, int len_stride,
                                                      long kv_stride, SplitIn si) {
  constexpr int H2 = HD / 2;
  // prefill (len_stride 0): row i of a prompt sits at the KV length before the prefill
  // plus i.  Batched decode: row i is stream i, at its own KV length (len_at[i *
  // len_stride]), with its own cache (kv_stride elements after the previous stream's).
  const int i = blockIdx.x;
  const int pos = len_stride ? len_at[(long)i * len_stride] : *len_at + i;
  kc += (long)i * kv_stride;
  vc += (long)i * kv_stride;
  constexpr int nw = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int W = (Hq + 2 * Hkv) * HD;
  const float* row = QKV + (size_t)i * W;
  const float* cs = rope_cos + (size_t)pos * H2;
  const float* sn = rope_sin + (size_t)pos * H2;
  // this wave's heads' values, all loaded before the first is used
  constexpr int kHeadsPerWave = HPW;
  const bool act = lane < H2;
  const int la = act ? lane : 0;
  float x0[kHeadsPerWave], x1[kHeadsPerWave];
  if (KS > 0 && si.part) {
    long idx[2 * kHeadsPerWave];
    int col[2 * kHeadsPerWave];
    float xs[2 * kHeadsPerWave];
#pragma unroll
    for (int t = 0; t < kHeadsPerWave; ++t) {
      const int h = min(w + t * nw, Hq + Hkv - 1);
      col[2 * t] = h * HD + la;
      col[2 * t + 1] = h * HD + la + H2;
      idx[2 * t] = (long)i * W + col[2 * t];
      idx[2 * t + 1] = (long)i * W + col[2 * t + 1];
    }
    split_sums<2 * kHeadsPerWave, (KS > 0 ? KS : 1)>(si, idx, col, xs);
#pragma unroll
    for (int t = 0; t < kHeadsPerWave; ++t) {
      x0[t] = xs[2 * t];
      x1[t] = xs[2 * t + 1];
    }
  } else {
#pragma unroll
    for (int t = 0; t < kHeadsPerWave; ++t) {
      const int h = min(w + t * nw, Hq + Hkv - 1);
      x0[t] = row[(size_t)h * HD + la];
      x1[t] = row[(size_t)h * HD + la + H2];
    }
  }
  const float gq0 = g_q[la], gq1 = g_q[la + H2], gk0 = g_k[la], gk1 = g_k[la + H2];
  const float c_ = cs[la], s_ = sn[la];
  // every head's sum of squares first (independent reductions whose latency overlaps)
  float ss[kHeadsPerWave], rstd[kHeadsPerWave];
#pragma unroll
  for (int t = 0; t < kHeadsPerWave; ++t) ss[t] = norm_ss(act ? x0[t] : 0.0f, act ? x1[t] : 0.0f);
  rstd_rows<HD, kHeadsPerWave>(ss, eps, rstd);
#pragma unroll
  for (int t = 0; t < kHeadsPerWave; ++t) {
    const int h = w + t * nw;
    if (h >= Hq + Hkv) break;
    float a, b;
    if (h < Hq) {
      rope_apply<HD>(rstd[t], act ? x0[t] : 0.0f, act ? x1[t] : 0.0f, gq0, gq1, c_, s_, lane, &a, &b);
      if (lane < H2) {
        Q[(size_t)i * Hq * HD + (size_t)h * HD + lane] = a;
        Q[(size_t)i * Hq * HD + (size_t)h * HD + lane + H2] = b;
      }
    } else {
      const int j = h - Hq;
      rope_apply<HD>(rstd[t], act ? x0[t] : 0.0f, act ? x1[t] : 0.0f, gk0, gk1, c_, s_, lane, &a, &b);
      if (lane < H2) {
        kc[((size_t)j * max_seq + pos) * HD + lane] = (uint16_t)f32_to_bf16(a);
        kc[((size_t)j * max_seq + pos) * HD + lane + H2] = (uint16_t)f32_to_bf16(b);
      }
    }
  }
  constexpr int kVPer = VPER;
  float vv[kVPer];
  if (KS > 0 && si.part) {
    long idx[kVPer];
    int col[kVPer];
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      col[u] = (Hq + Hkv) * HD + min(u * NT + (int)threadIdx.x, Hkv * HD - 1);
      idx[u] = (long)i * W + col[u];
    }
    split_sums<kVPer, (KS > 0 ? KS : 1)>(si, idx, col, vv);
  } else {
#pragma unroll
    for (int u = 0; u < kVPer; ++u) vv[u] = row[(size_t)(Hq + Hkv) * HD + min(u * NT + (int)threadIdx.x, Hkv * HD - 1)];
  }
#pragma unroll
  for (int u = 0; u < kVPer; ++u) {
    const int e = u * NT + threadIdx.x;
    if (e >= Hkv * HD) break;
    const int j = e / HD, dd = e % HD;
    vc[((size_t)j * max_seq + pos) * HD + dd] = (uint16_t)f32_to_bf16(vv[u]);
  }
}

// k_qk_rope_rows over `rows` rows with the narrowest instantiation, 512 threads (two
// waves per SIMD, each with half the heads): 5 heads per wave and 2 value elements per
// thread where the head counts allow (Hq + Hkv <= 40, Hkv HD <= 1024), else 8 and 4;
// split bound 2 or 4.
template <int HD>
static void launch_qk_rope_rows(hipStream_t st, int rows, const float* QKV, const float* g_q, const float* g_k,
                                const float* rope_cos, const float* rope_sin, float* Q, uint16_t* kc, uint16_t* vc,
                                const int* len_at, int Hq, int Hkv, int max_seq, float eps, int len_stride,
                                long kv_stride, const SplitIn& si) {
#define HTA_ROPE(HPW, VPER, KS)                                                                                  \
  hipLaunchKernelGGL((k_qk_rope_rows<HD, HPW, VPER, KS, 512>), dim3(rows), dim3(512), 0, st, QKV, g_q, g_k,      \
                     rope_cos, \
                     rope_sin, Q, kc, vc, len_at, Hq, Hkv, max_seq, eps, len_stride, kv_stride, si)
  const int ks = si.part ? si.ks : 0;
  if (Hq + Hkv <= 40 && Hkv * HD <= 1024) {
    if (ks == 0) HTA_ROPE(5, 2, 0);
    else if (ks <= 2) HTA_ROPE(5, 2, 2);
    else HTA_ROPE(5, 2, 4);
  } else {
    if (ks == 0) HTA_ROPE(8, 4, 0);
    else if (ks <= 2) HTA_ROPE(8, 4, 2);
    else HTA_ROPE(8, 4, 4);
  }
#undef HTA_ROPE
}

// ============================================================================ causal attention
// One block: 16 query rows of one kv head's group of G <= 4 query heads, one wave per
// head; keys in 64-wide tiles at absolute positions 0, 64, 128, ... up to the last
// query's position, shared by the group's waves through LDS.  Per tile and wave:
// S = Q K^T on the bf16 MFMA (q values are bf16-rounded and k is bf16, so the products
// are exact; fp32 accumulation), the online softmax per row in fp32, and O += P V on
// the MFMA with P split into three bf16 parts (P = hi + mid + lo up to 2^-24 of P,
// the precision of the fp32 value; all three are multiplied).  Every row is computed on its own (MFMA rows
// do not mix), so a row's result does not depend on which rows share its block.
// Lane layout of a 16x16x32 MFMA: the A operand row is lane & 15 with k = 8 (lane >> 4)
// .. + 8; the B operand column is lane & 15 with the same k; the result holds rows
// 4 (lane >> 4) + i, column lane & 15.
constexpr int kAttnQT = 16;
template <int HD, int NWV = 4>
struct __align__(16) PrefillAttnLds {
  uint16_t K[kAttnTile][HD + 8];   // [key][dim] (rows padded against bank conflicts)
  uint16_t V[HD][kAttnTile + 8];   // [dim][key], transposed for the P V operand
  float Pm[NWV][kAttnQT][kAttnTile + 4];  // per wave: the tile's probabilities, [row][key]
};

// All-reduce over each 16-lane row with DPP (no LDS round trips): the row mirror, the
// half-row mirror, then quad swaps by 2 and by 1.  Every step pairs each lane with a
// lane whose value has the same summation tree, so all 16 lanes end with the same bits.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_src<0x140, 0xf>(v, 0.0f);  // row_mirror
  v += dpp_src<0x141, 0xf>(v, 0.0f);  // row_half_mirror
  v += dpp_src<0x4e, 0xf>(v, 0.0f);   // quad_perm [2, 3, 0, 1]
  v += dpp_src<0xb1, 0xf>(v, 0.0f);   // quad_perm [1, 0, 3, 2]
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_src<0x140, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0x141, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0x4e, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0xb1, 0xf>(v, -INFINITY));
  return v;
}

__device__ __forceinline__ uint32_t pack_bf16_trunc(float a, float b) {  // exact for bf16 values
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// The attention of one block (kv head j, query rows i0 .. i0 + 15) once this lane's
// A fragments `qa` of its query head are formed.  The block's HB * CW waves: HB = G
// query heads of the group (wave w on head w / CW) or HB = 1 (head hg of the group), CW
// waves per head.  The CW waves of a head each compute the scores and probabilities of
// the whole tile (the same values in every such wave) and P V and the output for their
// own HD / CW output columns; a column's arithmetic is the same whichever wave takes it.
template <int P, int HD, int G, int HB = G, int CW = 1>
__device__ __forceinline__ void attn_prefill_block(const bf16x8 (&qa)[HD / 32], const uint16_t* __restrict__ kc,
                                                   const uint16_t* __restrict__ vc, void* __restrict__ O, int len0,
                                                   int i0, int j, int n_rows, int Hq, int max_seq, float scale,
                                                   float* amax, PrefillAttnLds<HD, HB * CW>& sm, float* red,
                                                   int hg = 0) {
  constexpr int T = kAttnTile, QT = kAttnQT;
  constexpr int NT = HD / 16;   // 16-wide output column tiles
  static_assert(T == 64, "four 16-key blocks per tile");
  static_assert(HB == G || HB == 1, "heads per block");
  static_assert(NT % CW == 0, "column tiles per wave");
  constexpr int NW = NT / CW;   // column tiles of this wave
  constexpr int nthr = 64 * HB * CW;
  constexpr int KC = HD / 32;   // 32-wide k chunks of a q row
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = j * G + (HB == 1 ? hg : w / CW);
  const int nb = (w % CW) * NW;  // first column tile of this wave
  const int r16 = lane & 15, g4 = lane >> 4;
  const int last_pos = len0 + min(i0 + QT, n_rows) - 1;
  const int n_tiles = last_pos / T + 1;
  const uint16_t* kb = kc + (size_t)j * max_seq * HD;
  const uint16_t* vb = vc + (size_t)j * max_seq * HD;
  const float inv_sqrt = 1.0f / sqrtf((float)HD);
  (void)KC;
  f32x4 oacc[NW];
#pragma unroll
  for (int n = 0; n < NW; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.0f; }

  // key/value tile loads: 16-byte segments, every load of a thread issued before its use;
  // the next tile is fetched while the current one is used.  K segments are stored as
  // they come ([key][dim]); V is stored transposed ([dim][key]) for the P V operand, so a
  // thread loads the same segment of two neighbouring keys and writes each dim's pair of
  // values as one 32-bit word: the 32 key pairs of a segment are consecutive words of a
  // row, and the two segments a wave covers land on opposite halves of the banks.
  constexpr int SEG = HD / 8;
  constexpr int NKV = T * SEG / nthr;
  constexpr int NV2 = (T / 2) * SEG / nthr;  // key pairs per thread
  static_assert(NKV * nthr == T * SEG && NV2 * nthr == (T / 2) * SEG, "key tile segments per thread");
  uint4 kr[NKV], va[NV2], vb2[NV2];
  auto load_kv = [&](int t0) {
#pragma unroll
    for (int u = 0; u < NKV; ++u) {
      const int idx = u * nthr + tid;
      const int key = idx / SEG, seg = idx % SEG;
      const int kp = min(t0 + key, last_pos);
      kr[u] = *reinterpret_cast<const uint4*>(kb + (size_t)kp * HD + seg * 8);
    }
#pragma unroll
    for (int u = 0; u < NV2; ++u) {
      const int idx = u * nthr + tid;
      const int pr = idx % (T / 2), seg = idx / (T / 2);
      const int k0 = min(t0 + 2 * pr, last_pos), k1 = min(t0 + 2 * pr + 1, last_pos);
      va[u] = *reinterpret_cast<const uint4*>(vb + (size_t)k0 * HD + seg * 8);
      vb2[u] = *reinterpret_cast<const uint4*>(vb + (size_t)k1 * HD + seg * 8);
    }
  };
  load_kv(0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * T;
    __syncthreads();  // the previous tile is consumed
#pragma unroll
    for (int u = 0; u < NKV; ++u) {
      const int idx = u * nthr + tid;
      const int key = idx / SEG, seg = idx % SEG;
      const bool valid = t0 + key <= last_pos;  // keys past the block's last query are zero
      *reinterpret_cast<uint4*>(&sm.K[key][seg * 8]) = valid ? kr[u] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < NV2; ++u) {
      const int idx = u * nthr + tid;
      const int pr = idx % (T / 2), seg = idx / (T / 2);
      const uint4 v0 = t0 + 2 * pr <= last_pos ? va[u] : make_uint4(0u, 0u, 0u, 0u);
      const uint4 v1 = t0 + 2 * pr + 1 <= last_pos ? vb2[u] : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t a4[4] = {v0.x, v0.y, v0.z, v0.w}, b4[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // dims 2q, 2q + 1 of the segment: (key 2pr, key 2pr + 1) as one word each
        *reinterpret_cast<uint32_t*>(&sm.V[seg * 8 + 2 * q][2 * pr]) = __builtin_amdgcn_perm(b4[q], a4[q], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&sm.V[seg * 8 + 2 * q + 1][2 * pr]) =
            __builtin_amdgcn_perm(b4[q], a4[q], 0x07060302u);
      }
    }
    if (tile + 1 < n_tiles) load_kv(t0 + T);
    __syncthreads();
    // scores of the 16 rows against the tile's 64 keys (four 16-key blocks)
    f32x4 sc[4];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const uint4 b = *reinterpret_cast<const uint4*>(&sm.K[kb4 * 16 + r16][c * 32 + 8 * g4]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
      }
      sc[kb4] = acc;
    }
    float mnew[4], fs[4], psum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g4 + i, qi = i0 + row, qpos = len0 + qi;
      float tmax = -INFINITY;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const int kp = t0 + kb4 * 16 + r16;
        const float v = (qi < n_rows && kp <= qpos) ? sc[kb4][i] * inv_sqrt : -INFINITY;
        sc[kb4][i] = v;
        tmax = fmaxf(tmax, v);
      }
      tmax = row16_max(tmax);
      mnew[i] = fmaxf(m[i], tmax);
      float ps = 0.0f;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const float v = sc[kb4][i];
        const float p = (v == -INFINITY) ? 0.0f : __expf(v - mnew[i]);
        sm.Pm[w][row][kb4 * 16 + r16] = p;
        ps += p;
      }
      ps = row16_sum(ps);
      psum[i] = ps;
      fs[i] = (m[i] == -INFINITY) ? 0.0f : __expf(m[i] - mnew[i]);
      l[i] = l[i] * fs[i] + psum[i];
      m[i] = mnew[i];
    }
#pragma unroll
    for (int n = 0; n < NW; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[n][i] *= fs[i];
    // the wave reads back its probabilities in the other lane order: its LDS writes first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // O += P V: the probabilities (this wave's own LDS rows) as A, in two 32-key chunks
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const float4 pa = *reinterpret_cast<const float4*>(&sm.Pm[w][r16][c2 * 32 + 8 * g4]);
      const float4 pb = *reinterpret_cast<const float4*>(&sm.Pm[w][r16][c2 * 32 + 8 * g4 + 4]);
      const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      // each part is the bf16 truncation of what the parts before it leave (the
      // differences are exact in fp32)
      uint32_t hi[4], mid[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = pv[2 * q], b = pv[2 * q + 1];
        const float ah = __uint_as_float(__float_as_uint(a) & 0xffff0000u), bh = __uint_as_float(__float_as_uint(b) & 0xffff0000u);
        const float ar = a - ah, br = b - bh;
        const float am = __uint_as_float(__float_as_uint(ar) & 0xffff0000u), bm = __uint_as_float(__float_as_uint(br) & 0xffff0000u);
        hi[q] = pack_bf16_trunc(ah, bh);
        mid[q] = pack_bf16_trunc(am, bm);
        lo[q] = pack_bf16_trunc(ar - am, br - bm);
      }
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
      const bf16x8 amid = __builtin_bit_cast(bf16x8, make_uint4(mid[0], mid[1], mid[2], mid[3]));
      const bf16x8 alo = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
      for (int n = 0; n < NW; ++n) {
        const uint4 b = *reinterpret_cast<const uint4*>(&sm.V[(nb + n) * 16 + r16][c2 * 32 + 8 * g4]);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
        oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, oacc[n], 0, 0, 0);
        oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(amid, bv, oacc[n], 0, 0, 0);
        oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, oacc[n], 0, 0, 0);
      }
    }
  }
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = i0 + 4 * g4 + i;
    if (qi >= n_rows) continue;
    const float inv = 1.0f / l[i];
#pragma unroll
    for (int n = 0; n < NW; ++n) {
      const float v = oacc[n][i] * inv;
      mx = fmaxf(mx, fabsf(v));
      const size_t idx = ((size_t)qi * Hq + h) * HD + (nb + n) * 16 + r16;
      if (P == kBF16) static_cast<uint16_t*>(O)[idx] = (uint16_t)act_encode<P>(v, scale);
      else static_cast<uint8_t*>(O)[idx] = (uint8_t)act_encode<P>(v, scale);
    }
  }
  if (amax) {
    mx = block_max(mx, red);
    if (tid == 0) record_amax(amax, mx);
  }
}

// this lane's A fragments of the 16 query rows (row r16; clamped rows are unused) from
// rotated queries held as fp32 values (bf16-exact), row stride `rs` floats
template <int HD>
__device__ __forceinline__ void q_fragments(const float* q0, int rs, int n_rows, int i0, bf16x8 (&qa)[HD / 32]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  const float* qrow = q0 + (size_t)min(i0 + r16, n_rows - 1) * rs;
#pragma unroll
  for (int c = 0; c < HD / 32; ++c) {
    const float4 a = *reinterpret_cast<const float4*>(qrow + c * 32 + 8 * g4);
    const float4 b = *reinterpret_cast<const float4*>(qrow + c * 32 + 8 * g4 + 4);
    const uint4 u = make_uint4(pack_bf16_trunc(a.x, a.y), pack_bf16_trunc(a.z, a.w), pack_bf16_trunc(b.x, b.y),
                               pack_bf16_trunc(b.z, b.w));
    qa[c] = __builtin_bit_cast(bf16x8, u);
  }
}

// CW waves per query head (each with HD / CW output columns).
template <int P, int HD, int G, int CW>
__global__ __launch_bounds__(64 * G * CW) void k_attn_prefill(const float* __restrict__ Q,
                                                           const uint16_t* __restrict__ kc,
                                                           const uint16_t* __restrict__ vc, void* __restrict__ O,
                                                           const int* __restrict__ len_at, int n_rows, int Hq,
                                                           int Hkv, int max_seq, float scale, float* amax) {
  __shared__ PrefillAttnLds<HD, G * CW> sm;
  __shared__ float red[16];
  const int j = blockIdx.x, i0 = blockIdx.y * kAttnQT;
  const int h = j * G + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / CW;
  bf16x8 qa[HD / 32];
  q_fragments<HD>(Q + (size_t)h * HD, Hq * HD, n_rows, i0, qa);
  attn_prefill_block<P, HD, G, G, CW>(qa, kc, vc, O, *len_at, i0, j, n_rows, Hq, max_seq, scale, amax, sm, red);
}

// Prompts of at most 16 rows (one query block): one block per query head (grid: kv heads
// x query heads per kv head).  The block's G waves take the prompt rows w, w + G, ...:
// each rotates the block's query head and the group's key head for its rows (q/k RMSNorm
// + RoPE) and writes their keys and values into the cache (the G blocks of a group store
// the same bits into the same cache rows, and each reads back only rows it has stored
// itself), then the waves share the attention of the query block through the column
// split of attn_prefill_block.  The rotation is norm_ss, rstd_rows and rope_apply on the
// split sums of k_qk_rope_rows and the attention is attn_prefill_block, in the same order,
// so every value is bit-identical to the two-kernel path of longer prompts.  The rotated
// queries stay in LDS (in the key tile area, free until the attention's first tile).
template <int HD>
constexpr bool rope_attn_small_fits() {
  return (size_t)kAttnQT * HD * 4 <= sizeof(uint16_t) * kAttnTile * (HD + 8);
}
// KS >= the split count of the q/k/v input (loads per thread bounded by it).
template <int P, int HD, int G, int KS>
__global__ __launch_bounds__(64 * G) void k_rope_attn_small(
    const float* __restrict__ QKV, SplitIn si, const float* __restrict__ g_q, const float* __restrict__ g_k,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc, void* __restrict__ O, const int* __restrict__ len_at, int n_rows, int Hq, int Hkv,
    int max_seq, float eps, float scale, float* amax) {
  constexpr int H2 = HD / 2, QT = kAttnQT;
  constexpr int R = QT / G;      // prompt rows per wave: w, w + G, ...
  constexpr int VE = HD / 64;    // value elements per lane and row
  constexpr int RU = 4 + VE;     // operands per row: the query pair, the key pair, the values
  static_assert(rope_attn_small_fits<HD>(), "rotated queries in the key tile area");
  __shared__ PrefillAttnLds<HD, G> sm;
  __shared__ float red[16];
  float* qs = reinterpret_cast<float*>(&sm.K[0][0]);  // [QT][HD]
  const int j = blockIdx.x, hg = blockIdx.y;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hq = j * G + hg;
  const int len0 = *len_at;
  const int W = (Hq + 2 * Hkv) * HD;
  const bool act = lane < H2;
  const int la = act ? lane : 0;
  // every operand of this wave's rows (rows past the prompt repeat its last row), loaded
  // before any is used: each row's rotation, the query head's and the key head's two
  // elements and the value head's VE
  float rc[R], rs[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const size_t rp = (size_t)(len0 + min(w + G * t, n_rows - 1)) * H2 + la;
    rc[t] = rope_cos[rp];
    rs[t] = rope_sin[rp];
  }
  float xs[R * RU];
  {
    long idx[R * RU];
    int col[R * RU];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const long r = min(w + G * t, n_rows - 1);
      col[RU * t] = hq * HD + la;
      col[RU * t + 1] = hq * HD + la + H2;
      col[RU * t + 2] = (Hq + j) * HD + la;
      col[RU * t + 3] = (Hq + j) * HD + la + H2;
#pragma unroll
      for (int e = 0; e < VE; ++e) col[RU * t + 4 + e] = (Hq + Hkv + j) * HD + lane + 64 * e;
#pragma unroll
      for (int u = 0; u < RU; ++u) idx[RU * t + u] = r * W + col[RU * t + u];
    }
    if (si.part) {
      split_sums<R * RU, KS>(si, idx, col, xs);
    } else {
#pragma unroll
      for (int u = 0; u < R * RU; ++u) xs[u] = QKV[idx[u]];
    }
  }
  const float gq0 = g_q[la], gq1 = g_q[la + H2], gk0 = g_k[la], gk1 = g_k[la + H2];
  uint16_t* kb = kc + (size_t)j * max_seq * HD;
  uint16_t* vb = vc + (size_t)j * max_seq * HD;
  // every row's sum of squares first (independent reductions: their latency overlaps; a
  // block has one wave per SIMD, nothing else hides it), the 1/rms of all rows in one pass
  // over the lanes, then the rotations.  Rows past the prompt are computed and never
  // stored, so that the row loop has no branch around its arithmetic.
  float ss[2 * R], rstd[2 * R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    ss[t] = norm_ss(act ? xs[RU * t] : 0.0f, act ? xs[RU * t + 1] : 0.0f);
    ss[R + t] = norm_ss(act ? xs[RU * t + 2] : 0.0f, act ? xs[RU * t + 3] : 0.0f);
  }
  rstd_rows<HD, 2 * R>(ss, eps, rstd);
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int r = w + G * t;
    float qa0, qb0, ka0, kb0;
    rope_apply<HD>(rstd[t], act ? xs[RU * t] : 0.0f, act ? xs[RU * t + 1] : 0.0f, gq0, gq1, rc[t], rs[t], lane, &qa0,
                   &qb0);
    rope_apply<HD>(rstd[R + t], act ? xs[RU * t + 2] : 0.0f, act ? xs[RU * t + 3] : 0.0f, gk0, gk1, rc[t], rs[t], lane,
                   &ka0, &kb0);
    if (r < n_rows) {  // uniform
      const int pos = len0 + r;
      if (act) {
        qs[r * HD + lane] = qa0;
        qs[r * HD + lane + H2] = qb0;
        kb[(size_t)pos * HD + lane] = (uint16_t)f32_to_bf16(ka0);
        kb[(size_t)pos * HD + lane + H2] = (uint16_t)f32_to_bf16(kb0);
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) vb[(size_t)pos * HD + lane + 64 * e] = (uint16_t)f32_to_bf16(xs[RU * t + 4 + e]);
    }
  }
  __threadfence_block();  // the block's cache rows, before its tiles read them
  __syncthreads();
  bf16x8 qa[HD / 32];
  q_fragments<HD>(qs, HD, n_rows, 0, qa);
  attn_prefill_block<P, HD, G, 1, G>(qa, kc, vc, O, len0, 0, j, n_rows, Hq, max_seq, scale, amax, sm, red, hg);
}

// ============================================================================ MFMA GEMM, small M
// C[M][N] (+)= A[M][K] . B[N][K]^T, A = activations (bf16 bits / e4m3 codes),
// B = packed weights.  A block computes 16R rows x 64 columns with 4 waves of
// 16R x 16; the K range is split into `ksplit` contiguous parts (a function of N
// and K only) whose partial sums land in Cpart[ksplit][M][N] and are added in
// split order by the row kernel that consumes the output (split_sums) or by
// k_gemm_reduce.  Each 16x16 MFMA tile accumulates its K range in
// increasing order: bf16 in 32-wide chunks; e4m3 per 64-wide chunk, the low 8
// bytes of every lane's 16-byte unit and then the high 8 bytes.  A row's result
// therefore does not depend on M, and the LDS-tiled kernel for larger M computes
// the same products in the same order.
//
// At small M the weights are a stream read once and one block's share of it is
// short, so the stream is latency-bound unless many bytes are requested ahead.
// One 128-element step of the block's 64 B rows and 16R A rows is a stage, fetched
// straight into LDS (global_load_lds_dwordx4) through a ring of NS stages issued
// NS - 1 ahead; the ring takes at most 80 KB, so two blocks share a CU.  Within a
// stage, 16-byte unit u of row r sits at position r * NU + (u ^ swz(r)), so a
// fragment read (16 consecutive rows, one unit each) touches 16 different bank
// groups.  Rows past M fetch row M - 1 (their results are not stored).
// What a GEMM does with a finished output tile when K is not split (the work
// k_gemm_reduce and k_silu_mul_rows do otherwise): mode 0 stores, mode 1 adds to `out`
// (the residual), mode 2 forms SiLU(gate) * up of the interleaved gate/up columns
// and stores it in GEMV units (bf16 bits / e4m3 codes of x / act_scale) into `act`
// [M][N / 2], recording |x| maxima in *amax when amax is set.
struct GemmEpi {
  float* out;
  const float* w_scale;  // e4m3 per-row weight scales, or null
  float in_scale;
  int mode;
  void* act;
  float act_scale;
  float* amax;
};

// the sum of a column's splits, as k_gemm_reduce scales it
__device__ __forceinline__ float epi_scale(const GemmEpi& e, float s, int col) {
  if (e.w_scale) s *= e.in_scale * e.w_scale[col];
  return s;
}
template <int P>
__device__ __forceinline__ float epi_store(const GemmEpi& e, int N, int row, int col, float s) {
  const size_t idx = (size_t)row * N + col;
  if (e.mode == 1) e.out[idx] += s;
  else e.out[idx] = s;
  return 0.0f;
}
template <int P>
__device__ __forceinline__ float epi_silu(const GemmEpi& e, int N, int row, int pair, float g, float u) {
  const float v = silu(g) * u;
  const size_t idx = (size_t)row * (N / 2) + pair;
  if (P == kBF16) static_cast<uint16_t*>(e.act)[idx] = (uint16_t)act_encode<P>(v, e.act_scale);
  else static_cast<uint8_t*>(e.act)[idx] = (uint8_t)act_encode<P>(v, e.act_scale);
  return fabsf(v);
}

// SiLU * up of one 16x16 output tile: the lane of an even column holds the gate values of
// rows row0 .. row0 + 3 (v[0..3], already scaled), its odd neighbour the up values of the
// same rows.  Two exchanges give the even lane the pairs of rows row0 and row0 + 1 and the
// odd lane those of rows row0 + 2 and row0 + 3, so both lanes share the work; each pair's
// arithmetic is that of epi_silu.  Returns the larger |SiLU * up| of the lane's two pairs.
template <int P>
__device__ __forceinline__ float epi_silu_tile(const GemmEpi& e, int N, int M, int row0, int pair, bool odd,
                                               const float (&v)[4]) {
  // the neighbouring lane's values by a DPP quad swap (lane ^ 1), no LDS round trip
  const float s1 = dpp_src<0xb1, 0xf>(odd ? v[0] : v[2], 0.0f);  // even: up of row0; odd: gate of row0 + 2
  const float s2 = dpp_src<0xb1, 0xf>(odd ? v[1] : v[3], 0.0f);  // even: up of row0 + 1; odd: gate of row0 + 3
  const int ra = row0 + (odd ? 2 : 0);
  float mx = 0.0f;
  if (ra < M) mx = epi_silu<P>(e, N, ra, pair, odd ? s1 : v[0], odd ? v[2] : s1);
  if (ra + 1 < M) mx = fmaxf(mx, epi_silu<P>(e, N, ra + 1, pair, odd ? s2 : v[1], odd ? v[3] : s2));
  return mx;
}

// NW waves per block, each computing 16R x 16 (16 NW columns per block).  The ring's
// budget keeps two blocks per CU at NW = 4 and three at NW = 2.
template <int P, int R, int NW>
struct Skinny {
  static constexpr int EB = P == kBF16 ? 2 : 1;
  static constexpr int SK = 128 * EB;                  // bytes of one row per stage
  static constexpr int NU = SK / 16;                   // 16-byte units per row and stage
  static constexpr int U = NU / 4;                     // units per lane per 16-row fragment
  static constexpr int BYTES_B = 16 * NW * SK, BYTES_A = 16 * R * SK, STAGE = BYTES_B + BYTES_A;
  // ring stages in 80 KB for four- and five-wave blocks (one per CU), 52 KB for two-wave
  // blocks (three per CU).  NW = 4: bf16 4 (R = 1), 3 (R = 2), e4m3 8, 6; NW = 5 (bf16,
  // R = 1): 3
  static constexpr int NS = ((NW >= 3 ? 80 : 52) * 1024) / STAGE;
  static constexpr int NB = NU / 4;                    // B fetches per wave and stage
  static constexpr int NA_ALL = R * NU / 4;            // A fetches per stage
  static constexpr int AW = NA_ALL >= NW ? NW : NA_ALL;  // waves that fetch A
  static constexpr int NA = NA_ALL / AW;               // A fetches per fetching wave
  static_assert(NS >= 3 && NA * AW == NA_ALL, "stage shape");
};

__device__ __forceinline__ int skinny_swz(int row, int nu) { return (row ^ (row >> 3)) & (nu - 1); }

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory"); }

template <int P, int R, int NW>
size_t skinny_lds_bytes() { return (size_t)Skinny<P, R, NW>::NS * Skinny<P, R, NW>::STAGE; }

// F8M (e4m3 only): the e4m3 MFMA, one instruction per 128-element step and 16-row fragment.
// Columns: the NW 16-column tiles from blockIdx.y * 16 NW, or (BAL, the bf16 form for up
// to 16 rows) a balanced contiguous run of the N / 16 tiles dealt over the gridDim.y
// blocks of each K split, at most NW tiles a block.  A wave beyond its block's tiles issues no load and computes
// nothing; it is never one of the AW waves that fetch A (the host deals at least AW tiles
// to every block), so every wave's ring waits count exactly the loads it issued.
template <int P, int R, int NW, bool F8M = false, bool BAL = false>
__global__ __launch_bounds__(64 * NW) void k_gemm(const void* __restrict__ A, const void* __restrict__ B,
                                                  float* __restrict__ Cpart, int M, int N, int K, int ksplit,
                                                  GemmEpi epi) {
  using S = Skinny<P, R, NW>;
  static_assert(!F8M || (P == kFP8 && S::U == 2), "the e4m3 MFMA takes a 128-byte step as two units per lane");
  extern __shared__ __align__(16) unsigned char gsm[];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = blockIdx.x * 16 * R, ks = blockIdx.z;
  int n0 = blockIdx.y * 16 * NW, nt = NW;
  if constexpr (BAL) {
    const int ntl = N / 16, nb = gridDim.y;
    const int t0 = (int)((long)blockIdx.y * ntl / nb), t1 = (int)((long)(blockIdx.y + 1) * ntl / nb);
    n0 = 16 * t0;
    nt = t1 - t0;
  }
  const bool on = !BAL || w < nt;  // wave-uniform (always true in the fixed form)
  const int rowbytes = K * S::EB;  // operands below 2^31 bytes
  const int nsteps = K / 128;
  const int s_beg = (int)((long)nsteps * ks / ksplit), s_end = (int)((long)nsteps * (ks + 1) / ksplit);
  const int nst = s_end - s_beg;
  const bool fetch_a = w < S::AW;

  int voffB[S::NB], voffA[S::NA];
#pragma unroll
  for (int j = 0; j < S::NB; ++j) {
    const int p = 64 * (w * S::NB + j) + lane, row = p / S::NU, u = (p % S::NU) ^ skinny_swz(row, S::NU);
    voffB[j] = (n0 + row) * rowbytes + u * 16;
  }
#pragma unroll
  for (int j = 0; j < S::NA; ++j) {
    const int p = 64 * (w * S::NA + j) + lane, row = p / S::NU, u = (p % S::NU) ^ skinny_swz(row, S::NU);
    voffA[j] = min(m0 + row, M - 1) * rowbytes + u * 16;
  }
  const unsigned char* Ab = static_cast<const unsigned char*>(A);
  const unsigned char* Bb = static_cast<const unsigned char*>(B);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)gsm);
  auto issue = [&](int c) {  // fetch step s_beg + c into stage c % NS
    const uint32_t sb = lds0 + (uint32_t)(c % S::NS) * S::STAGE;
    const unsigned char* a = Ab + (size_t)(s_beg + c) * S::SK;
    const unsigned char* b = Bb + (size_t)(s_beg + c) * S::SK;
    if (on) {
#pragma unroll
      for (int j = 0; j < S::NB; ++j) {
        const uint32_t mb = __builtin_amdgcn_readfirstlane(sb + (uint32_t)(w * S::NB + j) * 1024u);
        // weight rows, read once per call: non-temporal, past the caches
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     : : "v"(voffB[j]), "s"(b), "s"(mb) : "memory", "m0");
      }
    }
    if (fetch_a) {
#pragma unroll
      for (int j = 0; j < S::NA; ++j) {
        const uint32_t ma = __builtin_amdgcn_readfirstlane(sb + S::BYTES_B + (uint32_t)(w * S::NA + j) * 1024u);
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     : : "v"(voffA[j]), "s"(a), "s"(ma) : "memory", "m0");
      }
    }
  };
  for (int c = 0; c < S::NS - 1 && c < nst; ++c) issue(c);

  const int g = lane >> 4, r16 = lane & 15;
  int fb[S::U], fa[R][S::U];  // byte offsets of this lane's fragment units within a stage
#pragma unroll
  for (int q = 0; q < S::U; ++q) {
    const int rb = 16 * w + r16;
    fb[q] = (rb * S::NU + ((4 * q + g) ^ skinny_swz(rb, S::NU))) * 16;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int ra = 16 * r + r16;
      fa[r][q] = S::BYTES_B + (ra * S::NU + ((4 * q + g) ^ skinny_swz(ra, S::NU))) * 16;
    }
  }
  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nst; ++c) {
    // stage c has landed once at most the fetches of the NS - 2 younger stages remain
    // (loads land in issue order)
    if (c + S::NS - 2 < nst) {
      if (S::AW == NW || fetch_a) wait_vm<(S::NS - 2) * (S::NB + S::NA)>();
      else wait_vm<(S::NS - 2) * S::NB>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();  // every wave's part of stage c is in, and stage c - 1 is consumed
    if (c + S::NS - 1 < nst) issue(c + S::NS - 1);
    const unsigned char* st = gsm + (c % S::NS) * S::STAGE;
    if (!on) continue;  // wave-uniform: an idle wave only takes part in the barriers
    uint4 bv[S::U], av[R][S::U];
#pragma unroll
    for (int q = 0; q < S::U; ++q) {
      bv[q] = *reinterpret_cast<const uint4*>(st + fb[q]);
#pragma unroll
      for (int r = 0; r < R; ++r) av[r][q] = *reinterpret_cast<const uint4*>(st + fa[r][q]);
    }
    if (P == kBF16) {
#pragma unroll
      for (int q = 0; q < S::U; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r)
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[r][q]),
                                                           __builtin_bit_cast(bf16x8, bv[q]), acc[r], 0, 0, 0);
    } else if (F8M) {
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mfma_e4m3_step(av[r][0], av[r][1], bv[0], bv[1], acc[r]);
    } else {
      // e4m3 operands are widened to bf16 in registers (exact: 4 significant bits) and
      // multiplied on the bf16 MFMA, which accumulates at full fp32 precision; the e4m3
      // MFMA forms accumulate internally with fewer bits
#pragma unroll
      for (int q = 0; q < S::U; ++q) {
        const bf16x8 bl = fp8x8_to_bf16(bv[q].x, bv[q].y), bh = fp8x8_to_bf16(bv[q].z, bv[q].w);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(av[r][q].x, av[r][q].y), bl, acc[r], 0, 0, 0);
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(av[r][q].z, av[r][q].w), bh, acc[r], 0, 0, 0);
        }
      }
    }
  }
  // output layout: lane holds rows 4 * g + i of each 16x16 tile, column lane & 15
  const int col = n0 + 16 * w + r16;
  // the ring is idle once every stage is consumed: its first bytes hold the amax slots
  // (behind block_max's barriers), so the block stays within 80 KB
  float* red = reinterpret_cast<float*>(gsm);
  float mx = 0.0f;
  if (ksplit == 1) {
    // the whole K range is here: the epilogue works from the registers (0 + acc, as the
    // split sum starts from zero)
#pragma unroll
    for (int r = 0; r < R && on; ++r) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sum = 0.0f;
        sum += acc[r][i];
        v[i] = epi_scale(epi, sum, col);
      }
      const int row0 = m0 + 16 * r + 4 * g;
      if (epi.mode == 2) {
        mx = fmaxf(mx, epi_silu_tile<P>(epi, N, M, row0, col / 2, (r16 & 1) != 0, v));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (row0 + i < M) epi_store<P>(epi, N, row0 + i, col, v[i]);
      }
    }
  } else {
    // a split's partial, summed by the consuming row kernel or k_gemm_reduce (a
    // last-arriving block adding the splits here would put three memory round trips on
    // the kernel's tail, more than the reduce's launch)
    float* Cp = Cpart + (size_t)ks * M * N;
    if (!on) return;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * r + 4 * g + i;
        if (row < M) Cp[(size_t)row * N + col] = acc[r][i];
      }
    return;
  }
  if (epi.mode == 2 && epi.amax) {
    mx = block_max(mx, red);
    if (threadIdx.x == 0) record_amax(epi.amax, mx);
  }
}

// ============================================================================ LDS-tiled MFMA GEMM
// For M >= 64.  The products and their order are those of k_gemm (per 16x16 tile:
// bf16 in 32-wide K chunks of increasing K; e4m3 per 64-wide chunk, the low 8 bytes
// of every lane's 16-byte unit and then the high 8 bytes) and so is the K split, so a
// row's result is bit-identical whichever of the two kernels, and whichever tile shape,
// computes it.
// A block computes BM rows x BN columns with 4 waves of 64 rows x BN / (4 / (BM / 64))
// columns.  Per stage, 64 bytes of K of each of the BM A rows and BN B rows are fetched
// straight into LDS (global_load_lds_dwordx4) through a ring of NS stages issued NS - 1
// ahead of the stage being multiplied, so no register holds data in flight and a B tile
// is shared by the waves.  A stage's 16-byte units are swizzled within each row (unit u
// of row r at position 4r + (u ^ ((r >> 2) & 3))), so that a fragment read (16
// consecutive rows, one unit each) touches 16 different bank groups.
// Tile shapes (measured on the 36-layer shapes against the 128 x 128 four-stage tile):
// M >= 256 takes 128 x 128 with three stages (48 KB, three blocks per CU: the 560-608
// block grids then fit in one wave of the chip).  Below that, e4m3 takes 64 x 64 with
// four stages (32 KB), which puts 2-4x more blocks on the CUs than one 128-row tile
// can; bf16 keeps 128 x 128 with four stages, as a 64 x 64 bf16 tile has too few MFMAs
// per stage (8 per wave) for its barrier.
// The grid's blocks are dealt to the 8 XCDs round robin; the kernel maps them back so
// that each XCD walks a contiguous run of tiles (row tiles of one column tile first),
// which then share that column tile's weights in the XCD's L2.
constexpr int kGemmTileMinM = 64;        // smaller M: k_gemm (weights streamed once per 16 or 32 rows)
constexpr int kGemmTileBigM = 256;       // from here: 128 x 128 tiles

template <int BM, int BN, int NS>
struct TileCfg {
  static constexpr int WMW = BM / 64, WNW = 4 / WMW, WN = BN / WNW, NJ = WN / 16;
  static constexpr int HA = BM * 64, HB = BN * 64, STG = HA + HB;  // bytes per stage
  static constexpr int UA = BM * 4, UB = BN * 4;                  // 16-byte units per stage
  static constexpr int LA = UA / 256, LB = UB / 256;                // fetches per wave and stage
  static_assert(WMW * WNW == 4 && NJ >= 1 && WN % 16 == 0, "four waves of 64 x 16k");
  static_assert(LA * 256 == UA && LB * 256 == UB, "every wave fetches the same count");
  static_assert(NS >= 3, "ring of at least three stages");
};

template <int BM, int BN, int NS>
size_t gemm_tile_lds_bytes() { return (size_t)NS * TileCfg<BM, BN, NS>::STG; }

__device__ __forceinline__ int tile_unit_pos(int row, int u) { return row * 4 + (u ^ ((row >> 2) & 3)); }

// F8M (e4m3 only): the e4m3 MFMA over each pair of 64-byte chunks (one 128-element step;
// a lane's units of the two chunks are the units k_gemm's lane takes from the step).
template <int P, int BM, int BN, int NS, bool F8M = false>
__global__ __launch_bounds__(256, F8M ? 3 : 1) void k_gemm_tile(const void* __restrict__ A, const void* __restrict__ B,
                                                   float* __restrict__ Cpart, int M, int N, int K, int ksplit,
                                                   GemmEpi epi) {
  using T = TileCfg<BM, BN, NS>;
  constexpr int NJ = T::NJ, WN = T::WN;
  static_assert(!F8M || P == kFP8, "the e4m3 MFMA form is for e4m3 operands");
  extern __shared__ __align__(16) unsigned char gsm[];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int mt, nt, ks;
  {
    // block L runs on XCD L % 8; give XCD x the contiguous tile run [start(x), start(x) + count(x))
    const int gx = gridDim.x, gy = gridDim.y;
    const int total = gx * gy * (int)gridDim.z;
    const int L = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const int x = L & 7, i = L >> 3, q = total >> 3, r = total & 7;
    const int t = x * q + (x < r ? x : r) + i;
    mt = t % gx;
    nt = (t / gx) % gy;
    ks = t / (gx * gy);
  }
  const int m0 = mt * BM, n0 = nt * BN;
  constexpr int EB = (P == kBF16) ? 2 : 1;
  const int rowbytes = K * EB;  // operands below 2^31 bytes
  const int nsteps = K / 128;   // the split is over 128-element steps, as in k_gemm
  const int s_beg = (int)((long)nsteps * ks / ksplit), s_end = (int)((long)nsteps * (ks + 1) / ksplit);
  constexpr int CPS = 128 * EB / 64;  // 64-byte chunks per 128-element step
  const int c0 = s_beg * CPS, nch = (s_end - s_beg) * CPS;

  // this wave fetches units [64 * (w + 4 j), +64) of each operand's tile
  int voffA[T::LA], voffB[T::LB];
#pragma unroll
  for (int j = 0; j < T::LA; ++j) {
    const int p = 64 * (w + 4 * j) + lane, row = p >> 2, u = (p & 3) ^ ((row >> 2) & 3);
    const int ra = m0 + row < M ? m0 + row : M - 1;  // rows past M fetch row M - 1 (results unused)
    voffA[j] = ra * rowbytes + u * 16;
  }
#pragma unroll
  for (int j = 0; j < T::LB; ++j) {
    const int p = 64 * (w + 4 * j) + lane, row = p >> 2, u = (p & 3) ^ ((row >> 2) & 3);
    voffB[j] = (n0 + row) * rowbytes + u * 16;
  }
  const unsigned char* Ab = static_cast<const unsigned char*>(A);
  const unsigned char* Bb = static_cast<const unsigned char*>(B);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)gsm);
  auto issue = [&](int c) {  // fetch chunk c into stage c % NS
    const uint32_t sb = lds0 + (uint32_t)(c % NS) * T::STG;
    const unsigned char* a = Ab + (size_t)(c0 + c) * 64;
    const unsigned char* b = Bb + (size_t)(c0 + c) * 64;
#pragma unroll
    for (int j = 0; j < T::LA; ++j) {
      const uint32_t ma = __builtin_amdgcn_readfirstlane(sb + (uint32_t)(w + 4 * j) * 1024u);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   : : "v"(voffA[j]), "s"(a), "s"(ma) : "memory", "m0");
    }
#pragma unroll
    for (int j = 0; j < T::LB; ++j) {
      const uint32_t mb = __builtin_amdgcn_readfirstlane(sb + T::HA + (uint32_t)(w + 4 * j) * 1024u);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   : : "v"(voffB[j]), "s"(b), "s"(mb) : "memory", "m0");
    }
  };
  for (int c = 0; c < NS - 1 && c < nch; ++c) issue(c);

  const int wm = w / T::WNW, wn = w % T::WNW, g = lane >> 4, r16 = lane & 15;
  int fa[4], fb[NJ];  // byte offsets of this lane's fragment units within a stage
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = tile_unit_pos(64 * wm + 16 * i + r16, g) * 16;
#pragma unroll
  for (int j = 0; j < NJ; ++j) fb[j] = T::HA + tile_unit_pos(WN * wn + 16 * j + r16, g) * 16;
  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 hav[F8M ? 4 : 1], hbv[F8M ? NJ : 1];  // F8M: the first chunk of the step being multiplied

  for (int c = 0; c < nch; ++c) {
    // chunk c has landed once at most the fetches of the NS - 2 younger chunks remain
    // (LA + LB per chunk and wave; loads land in issue order)
    if (c + NS - 2 < nch) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * (T::LA + T::LB)) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's part of chunk c is in, and chunk c - 1 is consumed
    if (c + NS - 1 < nch) issue(c + NS - 1);
    const unsigned char* st = gsm + (c % NS) * T::STG;
    uint4 av[4], bv[NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const uint4*>(st + fa[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bv[j] = *reinterpret_cast<const uint4*>(st + fb[j]);
    if (P == kBF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                               __builtin_bit_cast(bf16x8, bv[j]), acc[i][j], 0, 0, 0);
    } else if (F8M) {
      // chunks come in step pairs: c0 is even and every step has two chunks
      if ((c & 1) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hav[i] = av[i];
#pragma unroll
        for (int j = 0; j < NJ; ++j) hbv[j] = bv[j];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_e4m3_step(hav[i], av[i], hbv[j], bv[j], acc[i][j]);
      }
    } else {
      bf16x8 al[4], ah[4], bl[NJ], bh[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        al[i] = fp8x8_to_bf16(av[i].x, av[i].y);
        ah[i] = fp8x8_to_bf16(av[i].z, av[i].w);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        bl[j] = fp8x8_to_bf16(bv[j].x, bv[j].y);
        bh[j] = fp8x8_to_bf16(bv[j].z, bv[j].w);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        }
    }
  }
  // output layout: lane holds rows 4 * g + r of each 16x16 tile, column lane & 15
  if (ksplit == 1) {
    // the whole K range is here: the epilogue works from the registers, as in k_gemm
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = n0 + WN * wn + 16 * j + r16;
        const int row0 = m0 + 64 * wm + 16 * i + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float sum = 0.0f;
          sum += acc[i][j][r];
          v[r] = epi_scale(epi, sum, col);
        }
        if (epi.mode == 2) {
          mx = fmaxf(mx, epi_silu_tile<P>(epi, N, M, row0, col / 2, (r16 & 1) != 0, v));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (row0 + r < M) epi_store<P>(epi, N, row0 + r, col, v[r]);
        }
      }
    if (epi.mode == 2 && epi.amax) {
      mx = block_max(mx, reinterpret_cast<float*>(gsm));  // the ring is idle: its first bytes
      if (threadIdx.x == 0) record_amax(epi.amax, mx);
    }
    return;
  }
  float* Cp = Cpart + (size_t)ks * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + WN * wn + 16 * j + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 64 * wm + 16 * i + 4 * g + r;
        if (row < M) Cp[(size_t)row * N + col] = acc[i][j][r];
      }
    }
}

// out = sum over splits (in order) * in_scale * w_scale[n]; mode 0 store, 1 add to out.
__global__ __launch_bounds__(256) void k_gemm_reduce(const float* __restrict__ Cpart, float* __restrict__ out,
                                                     const float* __restrict__ w_scale, float in_scale, int M, int N,
                                                     int ksplit, int resid) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t MN = (size_t)M * N;
  if (idx >= MN) return;
  float pv[8];  // ksplit <= 8
#pragma unroll
  for (int k = 0; k < 8; ++k) pv[k] = Cpart[(size_t)min(k, ksplit - 1) * MN + idx];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < ksplit) s += pv[k];
  if (w_scale) s *= in_scale * w_scale[idx % N];
  if (resid) out[idx] += s;
  else out[idx] = s;
}

// Number of K splits: a function of (N, K) only, so prefix reuse stays bit-identical.  About
// 768 blocks of 16 columns: on the 36-layer shapes this takes o and down to 5 splits and
// q/k/v to 2 (from 7 and 3 at 1024 blocks: -6 % at P = 512, -4 % at P = 128, -2 % at
// P = 13 and -3 % per batched step; 384 and 512 blocks were slower at some P).
static int gemm_ksplit(int N, int K) {
  const int nsteps = K / 128;
  const int nblk = N / 16;
  int s = (768 + nblk - 1) / nblk;
  if (s > 8) s = 8;
  if (s > nsteps) s = nsteps;
  if (s < 1) s = 1;
  return s;
}

static float* split_buffer(Ctx& c) { return c.pgu + (size_t)c.cfg.max_prefill * 2 * c.cfg.ffn; }

// The split partials of the last gemm(..., defer = true) as the next row kernel's input
// (null part when K was not split: the GEMM's epilogue then finished the output).
template <int P>
static SplitIn deferred_split(Ctx& c, int M, int N, int K, const float* w_scale, float in_scale) {
  const int ks = gemm_ksplit(N, K);
  if (ks == 1) return SplitIn{nullptr, 0, 0, nullptr, 1.0f};
  return SplitIn{split_buffer(c), ks, (long)M * N, P == kFP8 ? w_scale : nullptr, in_scale};
}

// The kernel choice for one product (F8M: the e4m3 MFMA form of the same kernels).
template <int P, bool F8M>
static void gemm_launch(Ctx& c, const void* A, const void* B, float* part, int M, int N, int K, int ks,
                        const GemmEpi& epi) {
  if (M < kGemmTileMinM) {
    const int R = M <= 16 ? 1 : 2;
    const int mt = (M + 16 * R - 1) / (16 * R);
    // Block width: the weight stream is dealt to the CUs in whole blocks, so the
    // kernel lasts about as long as the CU with the most columns.  Two-wave blocks
    // (32 columns, three resident per CU) are taken when they lower that maximum.
    // Which block computes a column does not change its arithmetic.
    const long cus = c.num_cus;
    auto max_cols = [&](long width) {
      const long blocks = (long)mt * (N / width) * ks;
      return (blocks + cus - 1) / cus * width;  // columns x splits on the busiest CU
    };
    const long classic = std::min(max_cols(32), max_cols(64));
    // Balanced form (bf16, up to 16 rows): one block per CU and K split, each with a
    // contiguous run of 4 or 5 of the N / 16 column tiles (run lengths differ by at most
    // one), taken where it lowers the busiest CU's columns and every block gets at least
    // the tiles of its waves that fetch A.  (e4m3 measured slower in this form: two or
    // three resident two-wave blocks per CU keep more of its weight stream in flight.)
    if constexpr (P == kBF16) {
      if (R == 1) {
        const int ntl = N / 16;
        int nb = (int)(cus / ks);
        if (nb > ntl) nb = ntl;
        const int tmax = nb > 0 ? (ntl + nb - 1) / nb : 0, tmin = nb > 0 ? ntl / nb : 0;
        if (nb > 0 && 16L * tmax < classic && tmax == 5 && tmin >= Skinny<P, 1, 5>::AW) {
          const dim3 grid(1, nb, ks);
          hipLaunchKernelGGL((k_gemm<P, 1, 5, F8M, true>), grid, dim3(320), (skinny_lds_bytes<P, 1, 5>()), c.stream,
                             A, B, part, M, N, K, ks, epi);
          return;
        }
      }
    }
    const bool narrow = max_cols(32) < max_cols(64);
    if (!narrow) {
      dim3 grid(mt, N / 64, ks);
      if (R == 1)
        hipLaunchKernelGGL((k_gemm<P, 1, 4, F8M>), grid, dim3(256), (skinny_lds_bytes<P, 1, 4>()), c.stream, A, B,
                           part, M, N, K, ks, epi);
      else
        hipLaunchKernelGGL((k_gemm<P, 2, 4, F8M>), grid, dim3(256), (skinny_lds_bytes<P, 2, 4>()), c.stream, A, B,
                           part, M, N, K, ks, epi);
    } else {
      dim3 grid(mt, N / 32, ks);
      if (R == 1)
        hipLaunchKernelGGL((k_gemm<P, 1, 2, F8M>), grid, dim3(128), (skinny_lds_bytes<P, 1, 2>()), c.stream, A, B,
                           part, M, N, K, ks, epi);
      else
        hipLaunchKernelGGL((k_gemm<P, 2, 2, F8M>), grid, dim3(128), (skinny_lds_bytes<P, 2, 2>()), c.stream, A, B,
                           part, M, N, K, ks, epi);
    }
  } else if (N % 128 != 0 || (M < kGemmTileBigM && P == kFP8)) {
    dim3 grid((M + 63) / 64, N / 64, ks);
    hipLaunchKernelGGL((k_gemm_tile<P, 64, 64, 4, F8M>), grid, dim3(256), (gemm_tile_lds_bytes<64, 64, 4>()),
                       c.stream, A, B, part, M, N, K, ks, epi);
  } else if (M < kGemmTileBigM) {
    if constexpr (!F8M) {  // bf16 only (e4m3 takes 64 x 64 below 256 rows)
      dim3 grid((M + 127) / 128, N / 128, ks);
      hipLaunchKernelGGL((k_gemm_tile<P, 128, 128, 4>), grid, dim3(256), (gemm_tile_lds_bytes<128, 128, 4>()),
                         c.stream, A, B, part, M, N, K, ks, epi);
    }
  } else {
    dim3 grid((M + 127) / 128, N / 128, ks);
    hipLaunchKernelGGL((k_gemm_tile<P, 128, 128, 3, F8M>), grid, dim3(256), (gemm_tile_lds_bytes<128, 128, 3>()),
                       c.stream, A, B, part, M, N, K, ks, epi);
  }
}

// defer: with K split, leave the partials for the next row kernel (deferred_split)
// instead of launching k_gemm_reduce; only for outputs without the SiLU epilogue.
template <int P>
static hipError_t gemm(Ctx& c, const void* A, const void* B, const float* w_scale, float in_scale, float* out, int M,
                       int N, int K, int resid, void* act = nullptr, float act_scale = 1.0f, float* amax = nullptr,
                       bool defer = false) {
  if (N % 64 != 0 || K % 128 != 0) return hipErrorInvalidValue;  // the kernels' tiling
  if (defer && act) return hipErrorInvalidValue;
  const int ks = gemm_ksplit(N, K);
  float* part = split_buffer(c);  // split partials after the gate/up buffer
  const GemmEpi epi{out, P == kFP8 ? w_scale : nullptr, in_scale, act ? 2 : (resid ? 1 : 0), act, act_scale, amax};
  hipError_t e;
  if constexpr (P == kFP8) {
    if (c.fp8_mfma) gemm_launch<P, true>(c, A, B, part, M, N, K, ks, epi);
    else gemm_launch<P, false>(c, A, B, part, M, N, K, ks, epi);
  } else {
    gemm_launch<P, false>(c, A, B, part, M, N, K, ks, epi);
  }
  if ((e = hipGetLastError()) != hipSuccess || ks == 1 || defer) return e;  // one split: the epilogue ran in the GEMM
  const size_t MN = (size_t)M * N;
  hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, c.stream, part, out,
                     P == kFP8 ? w_scale : nullptr, in_scale, M, N, ks, resid);
  if ((e = hipGetLastError()) != hipSuccess || !act) return e;
  const int F = N / 2;
  hipLaunchKernelGGL((k_silu_mul_rows<P>), dim3((F + 255) / 256, M), dim3(256), 0, c.stream, out, act, F, act_scale,
                     amax);
  return hipGetLastError();
}

template <int P>
static hipError_t prefill_p(Ctx& c, int Pn, bool record) {
  const auto& f = c.cfg;
  const int d = f.hidden, hd = f.head_dim, Hq = f.n_q_heads, Hkv = f.n_kv_heads;
  const int qd = Hq * hd, kvd = Hkv * hd, F = f.ffn, W = qd + 2 * kvd;
  // the kernels read the first position from the device state (the KV length before this
  // prefill), so a captured prefill of Pn rows serves every position
  const int* len0 = &c.state->len;
  float* amax = record ? c.amax : nullptr;
  // the row kernels' per-thread register batches (k_rmsnorm_act_rows, k_qk_rope_rows)
  if (d > kRowPerMax * 256 || Hq + Hkv > 16 * 4 || kvd > 8 * 256) return hipErrorInvalidValue;
  if (Hq % Hkv != 0 || (Hq / Hkv != 1 && Hq / Hkv != 2 && Hq / Hkv != 4)) return hipErrorInvalidValue;
  hipError_t e;
  hipLaunchKernelGGL(k_embed_rows, dim3(Pn), dim3(256), 0, c.stream, c.tok, c.e_text, c.px, d);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t tap_bytes = (size_t)Pn * d * 4;
  const SplitIn none{nullptr, 0, 0, nullptr, 1.0f};
  bool normed = false;  // c.pu holds this layer's attention input (normed with the last down's split sum)
  for (int layer = 0; layer < f.n_layers; ++layer) {
    const LayerW& L = c.layers[layer];
    const int s0 = kSitesPerLayer * layer;
    const bool tap = c.taps && layer == c.prefill_tap_layer;
    if (tap && (e = hipMemcpyAsync(c.taps_p, c.px, tap_bytes, hipMemcpyDeviceToDevice, c.stream)) != hipSuccess)
      return e;
    if (!normed) {
      launch_rmsnorm_rows<P>(c.stream, Pn, c.px, L.g_attn, f.rms_eps, c.pu,
                         d, host_act_scale(c, s0), amax ? amax + s0 : nullptr, none);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool defer_q = gemm_ksplit(W, d) <= kRopeMaxSplit;  // else k_gemm_reduce finishes the rows
    if ((e = gemm<P>(c, c.pu, L.w_qkv, L.s_qkv, host_act_scale(c, s0), c.pqkv, Pn, W, d, 0, nullptr, 1.0f, nullptr,
                     defer_q)) != hipSuccess)
      return e;
    const SplitIn sq = defer_q ? deferred_split<P>(c, Pn, W, d, L.s_qkv, host_act_scale(c, s0)) : none;
    const int G = Hq / Hkv;
    const float so = host_act_scale(c, s0 + 1);
    float* am = amax ? amax + s0 + 1 : nullptr;
    if (Pn <= kAttnQT) {
      // one query block: rotation and attention in one launch, one block per query head
#define HTA_RA2(HDV, GV, KSV)                                                                                \
  hipLaunchKernelGGL((k_rope_attn_small<P, HDV, GV, KSV>), dim3(Hkv, GV), dim3(64 * GV), 0, c.stream, c.pqkv, sq, \
                     L.g_q, L.g_k, c.rope_cos, c.rope_sin, L.k_cache, L.v_cache, c.po, len0, Pn, Hq, Hkv,         \
                     f.max_seq, f.rms_eps, so, am)
#define HTA_RA(HDV, GV)                            \
  do {                                             \
    if (!sq.part || sq.ks <= 2) HTA_RA2(HDV, GV, 2); \
    else HTA_RA2(HDV, GV, kRopeMaxSplit);            \
  } while (0)
      if (hd == 128 && G == 4) HTA_RA(128, 4);
      else if (hd == 128 && G == 2) HTA_RA(128, 2);
      else if (hd == 128 && G == 1) HTA_RA(128, 1);
      else if (hd == 64 && G == 4) HTA_RA(64, 4);
      else if (hd == 64 && G == 2) HTA_RA(64, 2);
      else if (hd == 64 && G == 1) HTA_RA(64, 1);
      else return hipErrorInvalidValue;
#undef HTA_RA
#undef HTA_RA2
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      if (hd == 128)
        launch_qk_rope_rows<128>(c.stream, Pn, c.pqkv, L.g_q, L.g_k, c.rope_cos, c.rope_sin, c.pq, L.k_cache,
                                 L.v_cache, len0, Hq, Hkv, f.max_seq, f.rms_eps, 0, 0L, sq);
      else
        launch_qk_rope_rows<64>(c.stream, Pn, c.pqkv, L.g_q, L.g_k, c.rope_cos, c.rope_sin, c.pq, L.k_cache,
                                L.v_cache, len0, Hq, Hkv, f.max_seq, f.rms_eps, 0, 0L, sq);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      dim3 grid(Hkv, (Pn + kAttnQT - 1) / kAttnQT);
// one wave per query head: two (each with half the output columns, the scores and
// probabilities computed by both) made the kernel 15 % slower at P = 512
#define HTA_ATTN(HDV, GV)                                                                                         \
  hipLaunchKernelGGL((k_attn_prefill<P, HDV, GV, 1>), grid, dim3(64 * GV), 0, c.stream, c.pq, L.k_cache, L.v_cache, \
                     c.po, len0, Pn, Hq, Hkv, f.max_seq, so, am)
      if (hd == 128 && G == 4) HTA_ATTN(128, 4);
      else if (hd == 128 && G == 2) HTA_ATTN(128, 2);
      else if (hd == 128 && G == 1) HTA_ATTN(128, 1);
      else if (hd == 64 && G == 4) HTA_ATTN(64, 4);
      else if (hd == 64 && G == 2) HTA_ATTN(64, 2);
      else if (hd == 64 && G == 1) HTA_ATTN(64, 1);
      else return hipErrorInvalidValue;
#undef HTA_ATTN
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = gemm<P>(c, c.po, L.w_o, L.s_o, host_act_scale(c, s0 + 1), c.px, Pn, d, qd, 1, nullptr, 1.0f, nullptr,
                     true)) != hipSuccess)
      return e;
    launch_rmsnorm_rows<P>(c.stream, Pn, c.px, L.g_mlp, f.rms_eps, c.pu, d,
                       host_act_scale(c, s0 + 2), amax ? amax + s0 + 2 : nullptr,
                       deferred_split<P>(c, Pn, d, qd, L.s_o, host_act_scale(c, s0 + 1)));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = gemm<P>(c, c.pu, L.w_gu, L.s_gu, host_act_scale(c, s0 + 2), c.pgu, Pn, 2 * F, d, 0, c.pa,
                     host_act_scale(c, s0 + 3), amax ? amax + s0 + 3 : nullptr)) != hipSuccess)
      return e;
    // the next layer's attention norm takes the down projection's split sum (the last
    // layer's residual is finished by the reduce: the prefill emits no norm after it)
    const bool fuse_next = layer + 1 < f.n_layers && gemm_ksplit(d, F) > 1;
    if ((e = gemm<P>(c, c.pa, L.w_d, L.s_d, host_act_scale(c, s0 + 3), c.px, Pn, d, F, 1, nullptr, 1.0f, nullptr,
                     fuse_next)) != hipSuccess)
      return e;
    normed = fuse_next;
    if (fuse_next) {
      const int s1 = s0 + kSitesPerLayer;
      launch_rmsnorm_rows<P>(c.stream, Pn, c.px, c.layers[layer + 1].g_attn,
                         f.rms_eps, c.pu, d, host_act_scale(c, s1), amax ? amax + s1 : nullptr,
                         deferred_split<P>(c, Pn, d, F, L.s_d, host_act_scale(c, s0 + 3)));
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (tap && (e = hipMemcpyAsync(c.taps_p + (size_t)f.max_prefill * d, c.px, tap_bytes, hipMemcpyDeviceToDevice,
                                   c.stream)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

// ============================================================================ batched decode step
// M independent streams (utterances) advance one step together: row m of every row
// buffer is stream m.  The GEMMs are the prefill's (M rows share one weight stream); the
// kernels below are the per-stream parts.

// Row m = the sum of the codebook embeddings of stream m's previous codes (codebooks in
// order, fp32).
__global__ __launch_bounds__(256) void k_embed_codes_rows(const DevState* __restrict__ st,
                                                          const uint16_t* __restrict__ e_aud, float* __restrict__ X,
                                                          int d, int C, int V) {
  const int m = blockIdx.x;
  for (int k = threadIdx.x; k < d; k += blockDim.x) {
    float v = 0.0f;
    for (int c = 0; c < C; ++c) v += bf16_to_f32(e_aud[((size_t)c * V + st[m].prev[c]) * d + k]);
    X[(size_t)m * d + k] = v;
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Decode attention of the batched step: one block per (key split s, kv head j, stream m),
// one wave per query head of the group.  Stream m's query is at position p = its KV
// length (its key and value were just written there); split s takes keys
// [s * chunk, min(p + 1, (s + 1) * chunk)) with chunk = ceil((p + 1) / S) in whole 64-key
// tiles.  Lane l scores key kb + l of a tile (fp32 dot of the bf16 key with the
// bf16-rounded query, scale 1/sqrt(hd)); the wave keeps the online softmax (running
// max and denominator, fp32) and lane l accumulates output dimensions l and l + 64.
// The split's (o[hd], max, denominator) go to part[((m * Hq + h) * S + s) * (hd + 2)].
template <int HD>
__global__ __launch_bounds__(256) void k_attn_rows(const float* __restrict__ Q, const uint16_t* __restrict__ kc,
                                                   const uint16_t* __restrict__ vc, long kv_stride,
                                                   const DevState* __restrict__ st, int Hq, int Hkv, int max_seq,
                                                   float* __restrict__ part) {
  const int S = gridDim.x, s = blockIdx.x, j = blockIdx.y, m = blockIdx.z;
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = j * G + w;
  const int L = st[m].len + 1;
  int chunk = (L + S - 1) / S;
  chunk = (chunk + 63) / 64 * 64;
  const int k0 = s * chunk, k1 = min(L, k0 + chunk);
  __shared__ __align__(16) float sq[4][HD];
  __shared__ float sp[4][64];
  const float* q = Q + ((size_t)m * Hq + h) * HD;
  for (int dd = lane; dd < HD; dd += 64) sq[w][dd] = q[dd];
  __syncthreads();
  const uint16_t* K = kc + (long)m * kv_stride + (size_t)j * max_seq * HD;
  const uint16_t* V = vc + (long)m * kv_stride + (size_t)j * max_seq * HD;
  const float inv_sqrt = 1.0f / sqrtf((float)HD);
  float mrun = -INFINITY, lrun = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int kb = k0; kb < k1; kb += 64) {  // the same trip count in every wave of the block
    const int key = kb + lane;
    const bool ok = key < k1;
    const uint4* kr = reinterpret_cast<const uint4*>(K + (size_t)(ok ? key : k0) * HD);
    float sc = 0.0f;
#pragma unroll
    for (int u = 0; u < HD / 8; ++u) {
      const uint4 k4 = kr[u];
      const float4 qa = *reinterpret_cast<const float4*>(&sq[w][8 * u]);
      const float4 qb = *reinterpret_cast<const float4*>(&sq[w][8 * u + 4]);
      sc = fmaf(qa.x, bf16_lo(k4.x), sc);
      sc = fmaf(qa.y, bf16_hi(k4.x), sc);
      sc = fmaf(qa.z, bf16_lo(k4.y), sc);
      sc = fmaf(qa.w, bf16_hi(k4.y), sc);
      sc = fmaf(qb.x, bf16_lo(k4.z), sc);
      sc = fmaf(qb.y, bf16_hi(k4.z), sc);
      sc = fmaf(qb.z, bf16_lo(k4.w), sc);
      sc = fmaf(qb.w, bf16_hi(k4.w), sc);
    }
    sc = ok ? sc * inv_sqrt : -INFINITY;
    const float mnew = fmaxf(mrun, wave_max(sc));
    const float p = ok ? __expf(sc - mnew) : 0.0f;
    const float scale = __expf(mrun - mnew);
    lrun = lrun * scale + wave_sum(p);
    o0 *= scale;
    o1 *= scale;
    sp[w][lane] = p;
    __syncthreads();
    const int nk = min(64, k1 - kb);
    for (int kk = 0; kk < nk; ++kk) {
      const float pk = sp[w][kk];
      const uint16_t* vr = V + (size_t)(kb + kk) * HD;
      o0 = fmaf(pk, bf16_to_f32(vr[lane]), o0);
      if (HD > 64) o1 = fmaf(pk, bf16_to_f32(vr[lane + 64]), o1);
    }
    mrun = mnew;
    __syncthreads();
  }
  float* pp = part + (((size_t)m * Hq + h) * S + s) * (HD + 2);
  pp[lane] = o0;
  if (HD > 64) pp[lane + 64] = o1;
  if (lane == 0) {
    pp[HD] = mrun;
    pp[HD + 1] = lrun;
  }
}

// Log-sum-exp combine of the splits (those holding keys), then the attention output in
// GEMM units (bf16 bits, or e4m3 codes at the site's static scale): one block per
// (query head, stream), one thread per output dimension.
// SM >= S, the step's split count (every split's partial is loaded before the first is
// used; the clamped indices past S are loaded but not used).
template <int P, int HD, int SM>
__global__ __launch_bounds__(HD) void k_attn_combine(const float* __restrict__ part, int S, int Hq,
                                                      void* __restrict__ O, float scale) {
  const int h = blockIdx.x, m = blockIdx.y, dd = threadIdx.x;
  const float* pp = part + ((size_t)m * Hq + h) * S * (HD + 2);
  float mv[SM], lv[SM], ov[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const float* ps = pp + (size_t)min(s, S - 1) * (HD + 2);
    mv[s] = ps[HD];
    lv[s] = ps[HD + 1];
    ov[s] = ps[dd];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < SM; ++s)
    if (s < S && lv[s] > 0.0f) mx = fmaxf(mx, mv[s]);
  float num = 0.0f, den = 0.0f;
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    if (s < S && lv[s] > 0.0f) {
      const float f = __expf(mv[s] - mx);
      num = fmaf(f, ov[s], num);
      den = fmaf(f, lv[s], den);
    }
  }
  const float v = num / den;
  const size_t idx = ((size_t)m * Hq + h) * HD + dd;
  if (P == kBF16) static_cast<uint16_t*>(O)[idx] = (uint16_t)act_encode<P>(v, scale);
  else static_cast<uint8_t*>(O)[idx] = (uint8_t)act_encode<P>(v, scale);
}

// k_attn_combine with the split bound rounded up to 1, 2, 4, 8 or 16 (the step's S <= 16).
template <int P, int HD>
static void launch_attn_combine(hipStream_t st, int Hq, int M, const float* part, int S, void* O, float scale) {
#define HTA_COMB(SM) \
  hipLaunchKernelGGL((k_attn_combine<P, HD, SM>), dim3(Hq, M), dim3(HD), 0, st, part, S, Hq, O, scale)
  if (S <= 1) HTA_COMB(1);
  else if (S <= 2) HTA_COMB(2);
  else if (S <= 4) HTA_COMB(4);
  else if (S <= 8) HTA_COMB(8);
  else HTA_COMB(16);
#undef HTA_COMB
}

// Each stream's codes of the step: per codebook the greedy argmax over the allowed ids
// (codebook 0: codes and EOS; the others: codes; ties to the lowest id; a NaN logit never
// wins), then the delay rule and the state advance, as in the decode frame kernel.
__global__ __launch_bounds__(256) void k_head_select(const float* __restrict__ logits, int ld,
                                                     DevState* __restrict__ st, int32_t* __restrict__ hist,
                                                     int max_seq, int C, int V, int bos, int eos) {
  const int m = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const float* z = logits + (size_t)m * ld;
  __shared__ int arg[kMaxCodebooks];
  for (int k = w; k < C; k += nw) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = lane; i < V; i += 64) {
      const float v = z[(size_t)k * V + i];
      const bool allowed = (i < bos) || (k == 0 && i == eos);
      const float x = v == v ? v : -INFINITY;
      if (allowed && (x > bv || (x == bv && i < bi))) { bv = x; bi = i; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) arg[k] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    DevState* s = st + m;
    const int t = s->t;
    int eoc = s->eoc;
    if (eoc < 0 && t > 0 && s->prev[0] == eos) eoc = t - 1;  // EOC from the fed-back code
    int codes[kMaxCodebooks];
    for (int k = 0; k < C; ++k) codes[k] = t < k ? bos : ((eoc >= 0 && t >= eoc + k) ? eos : arg[k]);
    const int eoc2 = eoc >= 0 ? eoc : (codes[0] == eos ? t : -1);
    const int done = (eoc2 >= 0 && t >= eoc2 + C - 1) ? 1 : 0;
    for (int k = 0; k < C; ++k) {
      s->codes[k] = codes[k];
      s->prev[k] = codes[k];
      hist[((size_t)m * max_seq + t) * C + k] = codes[k];
    }
    s->eoc = eoc;
    s->t = t + 1;
    s->len = s->len + 1;
    s->done = done;
    s->n_done += done;
  }
}

template <int P>
static hipError_t batch_step_p(Ctx& c) {
  const auto& f = c.cfg;
  const int M = c.lay.n_streams, S = c.lay.batch_splits;
  const int d = f.hidden, hd = f.head_dim, Hq = f.n_q_heads, Hkv = f.n_kv_heads, G = Hq / Hkv;
  const int qd = Hq * hd, kvd = Hkv * hd, F = f.ffn, W = qd + 2 * kvd;
  const long kvs = (long)(c.lay.kv_stream_bytes / 2);
  const int len_stride = (int)(sizeof(DevState) / sizeof(int));
  hipError_t e;
  hipLaunchKernelGGL(k_embed_codes_rows, dim3(M), dim3(256), 0, c.stream, c.state_base, c.e_aud, c.px, d,
                     f.n_codebooks, f.codebook_size);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const SplitIn none{nullptr, 0, 0, nullptr, 1.0f};
  for (int layer = 0; layer < f.n_layers; ++layer) {
    const LayerW& L = c.layers[layer];
    const int s0 = kSitesPerLayer * layer;
    if (layer == 0) {  // later layers' attention inputs are normed with the previous down's split sum
      launch_rmsnorm_rows<P>(c.stream, M, c.px, L.g_attn, f.rms_eps, c.pu,
                         d, host_act_scale(c, s0), nullptr, none);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool defer_q = gemm_ksplit(W, d) <= kRopeMaxSplit;  // else k_gemm_reduce finishes the rows
    if ((e = gemm<P>(c, c.pu, L.w_qkv, L.s_qkv, host_act_scale(c, s0), c.pqkv, M, W, d, 0, nullptr, 1.0f, nullptr,
                     defer_q)) != hipSuccess)
      return e;
    {
      const SplitIn sq = defer_q ? deferred_split<P>(c, M, W, d, L.s_qkv, host_act_scale(c, s0)) : none;
      if (hd == 128)
        launch_qk_rope_rows<128>(c.stream, M, c.pqkv, L.g_q, L.g_k, c.rope_cos, c.rope_sin, c.pq, c.k_base[layer],
                                 c.v_base[layer], &c.state_base->len, Hq, Hkv, f.max_seq, f.rms_eps, len_stride, kvs,
                                 sq);
      else
        launch_qk_rope_rows<64>(c.stream, M, c.pqkv, L.g_q, L.g_k, c.rope_cos, c.rope_sin, c.pq, c.k_base[layer],
                                c.v_base[layer], &c.state_base->len, Hq, Hkv, f.max_seq, f.rms_eps, len_stride, kvs,
                                sq);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (hd == 128)
      hipLaunchKernelGGL(k_attn_rows<128>, dim3(S, Hkv, M), dim3(64 * G), 0, c.stream, c.pq, c.k_base[layer],
                         c.v_base[layer], kvs, c.state_base, Hq, Hkv, f.max_seq, c.b_part);
    else
      hipLaunchKernelGGL(k_attn_rows<64>, dim3(S, Hkv, M), dim3(64 * G), 0, c.stream, c.pq, c.k_base[layer],
                         c.v_base[layer], kvs, c.state_base, Hq, Hkv, f.max_seq, c.b_part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (S > 16) return hipErrorInvalidValue;  // the combine's split bound
    if (hd == 128) launch_attn_combine<P, 128>(c.stream, Hq, M, c.b_part, S, c.po, host_act_scale(c, s0 + 1));
    else launch_attn_combine<P, 64>(c.stream, Hq, M, c.b_part, S, c.po, host_act_scale(c, s0 + 1));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = gemm<P>(c, c.po, L.w_o, L.s_o, host_act_scale(c, s0 + 1), c.px, M, d, qd, 1, nullptr, 1.0f, nullptr,
                     true)) != hipSuccess)
      return e;
    launch_rmsnorm_rows<P>(c.stream, M, c.px, L.g_mlp, f.rms_eps, c.pu, d,
                       host_act_scale(c, s0 + 2), nullptr, deferred_split<P>(c, M, d, qd, L.s_o, host_act_scale(c, s0 + 1)));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = gemm<P>(c, c.pu, L.w_gu, L.s_gu, host_act_scale(c, s0 + 2), c.pgu, M, 2 * F, d, 0, c.pa,
                     host_act_scale(c, s0 + 3), nullptr)) != hipSuccess)
      return e;
    if ((e = gemm<P>(c, c.pa, L.w_d, L.s_d, host_act_scale(c, s0 + 3), c.px, M, d, F, 1, nullptr, 1.0f, nullptr,
                     true)) != hipSuccess)
      return e;
    // the down projection's split sum feeds the next layer's attention norm, or the final norm
    const bool last = layer + 1 == f.n_layers;
    const int s1 = last ? kSitesPerLayer * f.n_layers : s0 + kSitesPerLayer;
    launch_rmsnorm_rows<P>(c.stream, M, c.px,
                       last ? c.g_final : c.layers[layer + 1].g_attn, f.rms_eps, c.pu, d, host_act_scale(c, s1), nullptr,
                       deferred_split<P>(c, M, d, F, L.s_d, host_act_scale(c, s0 + 3)));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = gemm<P>(c, c.pu, c.w_head, c.s_head, host_act_scale(c, kSitesPerLayer * f.n_layers), c.b_logits, M,
                   c.lay.cv_pad, d, 0)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_head_select, dim3(M), dim3(256), 0, c.stream, c.b_logits, c.lay.cv_pad, c.state_base,
                     c.hist_base, f.max_seq, f.n_codebooks, f.codebook_size, f.bos_id, f.eos_id);
  return hipGetLastError();
}

hipError_t launch_batch_step(Ctx& c) {
  if (c.cfg.n_q_heads / c.cfg.n_kv_heads > 4) return hipErrorInvalidValue;  // one wave per head, 256 threads
  if (c.cfg.precision == HTA_FP8_E4M3) return batch_step_p<kFP8>(c);
  return batch_step_p<kBF16>(c);
}

hipError_t prefill_setup() {
  const struct { const void* f; size_t lds; } kernels[] = {
      {(const void*)k_gemm_tile<kBF16, 64, 64, 4>, gemm_tile_lds_bytes<64, 64, 4>()},
      {(const void*)k_gemm_tile<kFP8, 64, 64, 4>, gemm_tile_lds_bytes<64, 64, 4>()},
      {(const void*)k_gemm_tile<kBF16, 128, 128, 3>, gemm_tile_lds_bytes<128, 128, 3>()},
      {(const void*)k_gemm_tile<kBF16, 128, 128, 4>, gemm_tile_lds_bytes<128, 128, 4>()},
      {(const void*)k_gemm_tile<kFP8, 128, 128, 3>, gemm_tile_lds_bytes<128, 128, 3>()},
      {(const void*)k_gemm<kBF16, 1, 4>, skinny_lds_bytes<kBF16, 1, 4>()},
      {(const void*)k_gemm<kBF16, 2, 4>, skinny_lds_bytes<kBF16, 2, 4>()},
      {(const void*)k_gemm<kFP8, 1, 4>, skinny_lds_bytes<kFP8, 1, 4>()},
      {(const void*)k_gemm<kFP8, 2, 4>, skinny_lds_bytes<kFP8, 2, 4>()},
      {(const void*)k_gemm<kBF16, 1, 2>, skinny_lds_bytes<kBF16, 1, 2>()},
      {(const void*)k_gemm<kBF16, 2, 2>, skinny_lds_bytes<kBF16, 2, 2>()},
      {(const void*)k_gemm<kFP8, 1, 2>, skinny_lds_bytes<kFP8, 1, 2>()},
      {(const void*)k_gemm<kFP8, 2, 2>, skinny_lds_bytes<kFP8, 2, 2>()},
      {(const void*)k_gemm<kBF16, 1, 5, false, true>, skinny_lds_bytes<kBF16, 1, 5>()},
      {(const void*)k_gemm_tile<kFP8, 64, 64, 4, true>, gemm_tile_lds_bytes<64, 64, 4>()},
      {(const void*)k_gemm_tile<kFP8, 128, 128, 3, true>, gemm_tile_lds_bytes<128, 128, 3>()},
      {(const void*)k_gemm<kFP8, 1, 4, true>, skinny_lds_bytes<kFP8, 1, 4>()},
      {(const void*)k_gemm<kFP8, 2, 4, true>, skinny_lds_bytes<kFP8, 2, 4>()},
      {(const void*)k_gemm<kFP8, 1, 2, true>, skinny_lds_bytes<kFP8, 1, 2>()},
      {(const void*)k_gemm<kFP8, 2, 2, true>, skinny_lds_bytes<kFP8, 2, 2>()},
  };
  for (const auto& k : kernels) {
    const hipError_t e = hipFuncSetAttribute(k.f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)k.lds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(Ctx& c, const void* A, const void* W, const float* w_scale, float a_scale, float* C, int M,
                       int N, int K) {
  if (c.cfg.precision == HTA_FP8_E4M3) return gemm<kFP8>(c, A, W, w_scale, a_scale, C, M, N, K, 0);
  return gemm<kBF16>(c, A, W, nullptr, 1.0f, C, M, N, K, 0);
}

hipError_t launch_prefill(Ctx& c, int P, bool record) {
  if (c.cfg.precision == HTA_FP8_E4M3) return prefill_p<kFP8>(c, P, record);
  return prefill_p<kBF16>(c, P, record);
}

}  // namespace hta
