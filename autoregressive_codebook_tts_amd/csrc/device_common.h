// Device-side helpers shared by the gfx950 kernels: storage-format conversions,
// wave64 reductions and the activation-rounding rule of each precision.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hta {

constexpr int kWave = 64;
constexpr float kE4m3Max = 448.0f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global (address space 1) views of pointers whose address space the compiler
// cannot infer (e.g. read from a device-side table): they then compile to
// global_* instead of flat_* accesses, and flat accesses would also count
// against lgkmcnt, so every LDS wait or barrier would drain the weight stream.
#define HTA_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const HTA_GLOBAL T* gp(const T* p) { return (const HTA_GLOBAL T*)p; }
template <class T>
__device__ __forceinline__ HTA_GLOBAL T* gpw(T* p) { return (HTA_GLOBAL T*)p; }

// 16-byte streaming load of weight data that is read once per frame.
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(gp(reinterpret_cast<const u32x4*>(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16-byte ordinary global load.
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 v = *gp(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- bfloat16 (raw uint16 bits)
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }
// The same roundings written with selects instead of a branch (the same bits for every
// input, NaN included), for straight-line code on latency-bound paths.
__device__ __forceinline__ uint32_t f32_to_bf16_sel(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : r;
}
__device__ __forceinline__ float round_bf16_sel(float f) { return bf16_to_f32(f32_to_bf16_sel(f)); }

// ---------------------------------------------------------------- OCP e4m3fn
// The hardware convert rounds to nearest even but turns |x| > 464 into NaN, so
// the value is clamped to +-448 first (saturating encode).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  x = fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false) & 0xffu;
}
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// ---------------------------------------------------------------- reductions
// Wave-wide sum / max with DPP: row shifts 1, 2, 4, 8 leave each 16-lane row's
// result in its lane 15, two row broadcasts fold the rows into lane 63, which is
// returned to every lane.  No LDS round trips.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_src(float x, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_src<0x111, 0xf>(v, 0.0f);  // row_shr:1
  v += dpp_src<0x112, 0xf>(v, 0.0f);  // row_shr:2
  v += dpp_src<0x114, 0xf>(v, 0.0f);  // row_shr:4
  v += dpp_src<0x118, 0xf>(v, 0.0f);  // row_shr:8
  v += dpp_src<0x142, 0xa>(v, 0.0f);  // row_bcast:15 into rows 1, 3
  v += dpp_src<0x143, 0xc>(v, 0.0f);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_src<0x111, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0x112, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0x114, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0x118, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0x142, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp_src<0x143, 0xc>(v, -INFINITY));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Block-wide sum for blockDim.x <= 1024; `red` needs blockDim.x / 64 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < nw; ++i) s += red[i];  // fixed order: deterministic
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
  for (int i = 1; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

// Maximum of non-negative floats via their ordered bit patterns (deterministic).
__device__ __forceinline__ void record_amax(float* slot, float v) {
  if (slot) atomicMax(reinterpret_cast<unsigned int*>(slot), __float_as_uint(fabsf(v)));
}

// ---------------------------------------------------------------- activation storage
// Precision of the GEMV inputs: bfloat16 values, or e4m3 codes of x / scale.
enum Prec { kBF16 = 0, kFP8 = 1 };

// Rounded value of x at an activation site, expressed in the units the GEMV
// multiplies with: the bfloat16 value, or the e4m3 code value of x * inv_scale
// (the scale itself is applied in the GEMV epilogue).
template <int P>
__device__ __forceinline__ float act_round(float x, float scale) {
  if (P == kBF16) return round_bf16(x);
  return e4m3_to_f32(f32_to_e4m3(x / scale));
}
// Storage form of the same rounding: bf16 bits (uint16) or e4m3 code (uint8).
template <int P>
__device__ __forceinline__ uint32_t act_encode(float x, float scale) {
  if (P == kBF16) return f32_to_bf16(x);
  return f32_to_e4m3(x / scale);
}
template <int P>
__device__ __forceinline__ float act_decode(uint32_t c) {
  if (P == kBF16) return bf16_to_f32(c);
  return e4m3_to_f32(c);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

}  // namespace hta
