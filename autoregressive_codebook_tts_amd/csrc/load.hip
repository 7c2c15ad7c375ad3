// Weight packing at load time: bf16 storage (round to nearest even) or FP8
// e4m3 codes with per-row scales max|row| / 448 (FlashRT "Higgs Audio v3
// TTS-4B" page, section 8: FP8 W8A8 with per-output-channel weight scales),
// written at a row stride so that gate and up rows interleave and q/k/v rows
// concatenate.  Plus small fill, KV-initialisation and decode-state kernels.
#include "device_common.h"
#include "hta_internal.h"

namespace hta {

__device__ __forceinline__ float load_src(const void* src, int dtype, size_t i) {
  if (dtype == HTA_SRC_F32) return static_cast<const float*>(src)[i];
  return bf16_to_f32(static_cast<const uint16_t*>(src)[i]);
}

__global__ __launch_bounds__(256) void k_pack_rows(void* __restrict__ dst, int dst_row0, int dst_row_stride,
                                                   const void* __restrict__ src, int dtype, int cols, int to_fp8,
                                                   float* __restrict__ scales) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  const size_t drow = (size_t)dst_row0 + (size_t)r * dst_row_stride;
  const size_t sbase = (size_t)r * cols;
  if (!to_fp8) {
    uint16_t* d = static_cast<uint16_t*>(dst) + drow * cols;
    if (dtype == HTA_SRC_BF16) {
      const uint16_t* s = static_cast<const uint16_t*>(src) + sbase;
      for (int k = threadIdx.x; k < cols; k += blockDim.x) d[k] = s[k];
    } else {
      for (int k = threadIdx.x; k < cols; k += blockDim.x) d[k] = (uint16_t)f32_to_bf16(load_src(src, dtype, sbase + k));
    }
    return;
  }
  float mx = 0.0f;
  for (int k = threadIdx.x; k < cols; k += blockDim.x) mx = fmaxf(mx, fabsf(load_src(src, dtype, sbase + k)));
  mx = block_max(mx, red);
  const float s = mx > 0.0f ? mx / kE4m3Max : 1.0f;
  uint8_t* d = static_cast<uint8_t*>(dst) + drow * cols;
  for (int k = threadIdx.x; k < cols; k += blockDim.x) d[k] = (uint8_t)f32_to_e4m3(load_src(src, dtype, sbase + k) / s);
  if (threadIdx.x == 0) scales[drow] = s;
}

__global__ void k_copy_f32(float* __restrict__ dst, const void* __restrict__ src, int dtype, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = load_src(src, dtype, i);
}

__global__ void k_fill_u32(uint32_t* __restrict__ dst, uint32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = v;
}

// K/V rows [Hkv][n][hd] (bf16) into the cache layout [Hkv][max_seq][hd].
__global__ void k_kv_init(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const uint16_t* __restrict__ ki,
                          const uint16_t* __restrict__ vi, int n, int max_seq, int hd) {
  const int j = blockIdx.y;
  const size_t per = (size_t)n * hd;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < per; e += (size_t)gridDim.x * blockDim.x) {
    const size_t p = e / hd, dd = e % hd;
    kc[((size_t)j * max_seq + p) * hd + dd] = ki[(size_t)j * per + e];
    vc[((size_t)j * max_seq + p) * hd + dd] = vi[(size_t)j * per + e];
  }
}

hipError_t launch_pack_rows(void* dst, int dst_row0, int dst_row_stride, const void* src, int src_dtype, int rows,
                            int cols, int to_fp8, float* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_rows, dim3(rows), dim3(256), 0, s, dst, dst_row0, dst_row_stride, src, src_dtype, cols,
                     to_fp8, scales);
  return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const void* src, int src_dtype, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, src, src_dtype, n);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* dst, uint32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, static_cast<uint32_t*>(dst), v, n);
  return hipGetLastError();
}

hipError_t launch_kv_init(uint16_t* k_cache, uint16_t* v_cache, const void* k_init, const void* v_init, int n_kv,
                          int n, int max_seq, int hd, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid(64, n_kv);
  hipLaunchKernelGGL(k_kv_init, grid, dim3(256), 0, s, k_cache, v_cache, static_cast<const uint16_t*>(k_init),
                     static_cast<const uint16_t*>(v_init), n, max_seq, hd);
  return hipGetLastError();
}

// ---------------------------------------------------------------- decode state
__global__ void k_set_prev(DevState* st, int c0, int c1, int c2, int c3, int c4, int c5, int c6, int c7,
                           int c8, int c9, int c10, int c11, int c12, int c13, int c14, int c15, int C) {
  const int cs[16] = {c0, c1, c2, c3, c4, c5, c6, c7, c8, c9, c10, c11, c12, c13, c14, c15};
  if (threadIdx.x < C) st->prev[threadIdx.x] = cs[threadIdx.x];
}

// a new utterance at length len: step 0, no EOC yet, all-BOS codes fed into the first frame
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
