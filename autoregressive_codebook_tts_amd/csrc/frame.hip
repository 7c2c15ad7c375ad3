// Persistent decode-frame kernel for gfx950: the whole frame (embedding,
// n_layers x [qkv GEMV, attention, o_proj GEMV, gate/up GEMV, down GEMV],
// head, argmax + delay bookkeeping) in one cooperative launch, one block per
// compute unit.
//
// Reference: FlashRT "Higgs Audio v3 TTS-4B" page, section 5 (the per-frame
// chain) and section 7 (the decode floor is set by streaming every weight once
// per frame; the frame is replayed as one position-agnostic graph).
//
// Design (MI355X):
//  * Every GEMV phase splits its rows across the blocks; a block's rows are cut
//    into 16-byte-per-lane packets along K (1 KB per wave), dealt round-robin to
//    the block's waves, kD packets per wave in flight.  A register slot is
//    refilled as soon as it is consumed, and the last group of a phase refills
//    from the first group of the next GEMV phase, so the weight stream runs
//    ahead of the activations it will be multiplied with.
//  * No grid barriers.  Every value handed from one block to another inside the
//    launch travels with a tag in the same atomic word (64-bit value+tag, or a
//    16-bit payload with a 16-bit tag); the tag is a running phase number, so a
//    consumer polls exactly the inputs it needs until they carry the current
//    phase's tag.  Producers never wait and need no release fence, and no
//    s_waitcnt ever drains the in-flight weight loads.  A buffer is rewritten
//    only after every consumer of its previous content has finished (each
//    rewrite depends, through the layer's data flow, on all of them).
//  * The exchange words are read and written with agent-scope atomic accesses,
//    coherent across the XCDs' L2s; weights, embeddings and older KV entries
//    are read-only during the launch.
//  * Polls are bounded: a wait longer than kSpinLimit sets an abort flag that
//    every other poll sees, so the grid always drains.
//  * Dot products: bf16 pairs on v_dot2_f32_bf16 (fp32 accumulation); e4m3
//    weights are widened to bf16 pairs in registers first (exact).
#include "device_common.h"
#include "hta_internal.h"

namespace hta {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kFT = 512;            // threads per block
constexpr int kFW = kFT / kWave;    // waves per block
constexpr int kD = 8;               // packets per wave per group
constexpr int kPartMax = 1024;      // packet partial sums per block per phase
constexpr uint64_t kSpinLimit = 50000000ull;  // 0.5 s at the 100 MHz constant clock

struct FrameArgs {
  int d, hd, Hq, Hkv, F, C, V, bos, eos, n_layers, max_seq, splits;
  float eps;
  const LayerW* layers;      // device copy of the per-layer pointers
  const uint16_t* e_aud;
  const float* g_final;
  const void* w_head;
  const float* s_head;
  const float* rope_cos;
  const float* rope_sin;
  const float* act_scales;   // [4L + 1]
  uint64_t* xh;              // [d]    residual            (value | tag << 32)
  uint64_t* xqkv;            // [W]    q, k, v             (value | tag << 32)
  uint32_t* xo;              // [qd]   attention output    (bf16 bits | tag16 << 16)
  uint32_t* xa;              // [F]    SiLU*mul output     (bf16 bits | tag16 << 16)
  uint64_t* xpart;           // [Hq][splits][hd + 2]       (value | tag << 32)
  uint64_t* xlogits;         // [C*V]                      (value | tag << 32)
  float* h_out;              // [d]    final residual (plain, for taps)
  float* logits_out;         // [C*V]  logits (plain, for taps)
  float* taps;               // [n_layers + 1][d] residual entering each layer, or null
  unsigned* sync;            // [0] launch count, [64] abort flag
  DevState* st;
  int32_t* hist;
};

// ---------------------------------------------------------------- tagged exchange words
__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(uint64_t* p, float v, unsigned tag) {
  __hip_atomic_store(gpw(p), ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld32(const uint32_t* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st32(uint32_t* p, uint32_t bits16, unsigned tag) {
  __hip_atomic_store(gpw(p), ((tag & 0xffffu) << 16) | (bits16 & 0xffffu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded poll state of one thread.
struct Poll {
  unsigned* abort_flag;
  uint64_t t0;
  bool ok;
  __device__ void start(unsigned* f) { abort_flag = f; t0 = __builtin_amdgcn_s_memrealtime(); ok = true; }
  // one more round of waiting; false when the frame must be abandoned
  __device__ bool again() {
    __builtin_amdgcn_s_sleep(1);
    if (__hip_atomic_load(gp(abort_flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) { ok = false; return false; }
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
      __hip_atomic_store(gpw(abort_flag), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = false;
      return false;
    }
    return true;
  }
};

// block-wide "everyone's polls succeeded"
__device__ __forceinline__ bool block_ok(bool ok, int* flag) {
  if (threadIdx.x == 0) *flag = 1;
  __syncthreads();
  if (!ok) *flag = 0;
  __syncthreads();
  return *flag != 0;
}

// ---------------------------------------------------------------- packet stream of one GEMV phase
// A block's rows are a run of packets in row-major order (a packet is 16 bytes
// per lane, 1 KB per wave, along K).  Wave w takes the contiguous run
// [w*n/kFW, (w+1)*n/kFW) of the block's n packets, so the waves' work differs by
// at most one packet; lanes accumulate a row across its packets and reduce once
// when the row ends, writing one partial per (row, wave) to LDS.
template <int P>
struct Stream {
  const uint8_t* w;
  int K;        // elements per row
  int r0;       // first row of this block
  int nrows;    // rows of this block
  int nch;      // packets per row
  static constexpr int E = (P == kBF16) ? 8 : 16;  // elements per 16-byte lane packet
  static constexpr int B = (P == kBF16) ? 2 : 1;   // bytes per element
  static constexpr int CH = kWave * E;             // elements per packet
  __device__ int npk() const { return nrows * nch; }
  __device__ int run_begin(int wave) const { return (int)((long)npk() * wave / kFW); }
};

template <int P>
__device__ __forceinline__ Stream<P> make_stream(const void* w, int N, int K, int pair_rows) {
  Stream<P> s;
  s.w = static_cast<const uint8_t*>(w);
  s.K = K;
  const int units = pair_rows ? N / 2 : N;
  const int u0 = (int)((long)units * blockIdx.x / gridDim.x);
  const int u1 = (int)((long)units * (blockIdx.x + 1) / gridDim.x);
  s.r0 = pair_rows ? 2 * u0 : u0;
  s.nrows = pair_rows ? 2 * (u1 - u0) : (u1 - u0);
  s.nch = (K + Stream<P>::CH - 1) / Stream<P>::CH;
  return s;
}

// Position in a wave's run: packet j of the run, at (row, ch).
struct Cursor {
  int j, n;      // packets taken, run length
  int row, ch;   // local row, packet within the row
};

template <int P>
__device__ __forceinline__ Cursor cursor_begin(const Stream<P>& s) {
  const int w = threadIdx.x >> 6;
  Cursor c;
  const int p0 = s.run_begin(w);
  c.j = 0;
  c.n = s.run_begin(w + 1) - p0;
  c.row = s.nch > 0 ? p0 / s.nch : 0;
  c.ch = p0 - c.row * s.nch;
  return c;
}
__device__ __forceinline__ void cursor_step(Cursor& c, int nch) {
  ++c.j;
  if (++c.ch == nch) { c.ch = 0; ++c.row; }
}

// One packet load per call, always issued (an address inside the stream when the
// packet is outside the run or past K, then zeroed), so the number of loads in
// flight is the same on every path and s_waitcnt can count them exactly.
template <int P>
__device__ __forceinline__ uint4 load_at(const Stream<P>& s, const Cursor& c) {
  const int lane = threadIdx.x & 63;
  const int e = c.ch * Stream<P>::CH + lane * Stream<P>::E;
  const bool ok = (c.j < c.n) && (e < s.K);
  const size_t off = ok ? ((size_t)(s.r0 + c.row) * s.K + e) * Stream<P>::B : 0;
  uint4 v = ld_stream16(s.w + off);
  if (!ok) v = make_uint4(0u, 0u, 0u, 0u);
  return v;
}

// bf16-pair dot of one packet with the activations xs (bf16 pairs in LDS)
template <int P>
__device__ __forceinline__ float packet_dot(const uint4& wv, const uint32_t* __restrict__ xs, float s) {
  if (P == kBF16) {
    const uint4 x = *reinterpret_cast<const uint4*>(xs);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.x), __builtin_bit_cast(bf16x2, x.x), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.y), __builtin_bit_cast(bf16x2, x.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.z), __builtin_bit_cast(bf16x2, x.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.w), __builtin_bit_cast(bf16x2, x.w), s, false);
    return s;
  } else {
    const uint4 x0 = *reinterpret_cast<const uint4*>(xs);
    const uint4 x1 = *reinterpret_cast<const uint4*>(xs + 4);
    const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, false);
      const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, true);
      s = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2, xw[2 * i]), s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, xw[2 * i + 1]), s, false);
    }
    return s;
  }
}

// The register ring of one wave: kD packets in flight.  `iss` is the issue
// cursor, kD packets ahead of consumption; while it lies in the phase's own run
// it loads from `s`, after the run it loads from the next phase's run.
template <int P>
struct Ring {
  uint4 buf[kD];
  Cursor iss;
  int iss_next;  // 1: the issue cursor is in the next stream's run
};

template <int P>
__device__ __forceinline__ void ring_prime(Ring<P>& r, const Stream<P>& s) {
  r.iss = cursor_begin(s);
  r.iss_next = 0;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    r.buf[i] = load_at(s, r.iss);
    cursor_step(r.iss, s.nch);
  }
}

// Consume this wave's run of `s` (the ring already holds its first kD packets);
// every consumed slot is refilled kD packets ahead, running on into the first
// kD packets of `next` (if any).  Row partials go to part[row * kFW + wave]; the
// caller zeroes part beforehand.
template <int P>
__device__ __forceinline__ void run_stream(const Stream<P>& s, const Stream<P>& next, Ring<P>& r,
                                           const uint32_t* __restrict__ xs, float* __restrict__ part) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  Cursor c = cursor_begin(s);
  const int ng = (c.n + kD - 1) / kD;
  float acc = 0.0f;
  for (int g = 0; g < ng; ++g) {
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      // consume slot i (pad slots hold zeros)
      const int e = c.ch * Stream<P>::CH + lane * Stream<P>::E;
      acc = packet_dot<P>(r.buf[i], xs + (e < s.K ? e : 0) / 2, acc);
      if (c.j < c.n) {
        const int row = c.row;
        cursor_step(c, s.nch);
        if (c.row != row || c.j == c.n) {
          const float v = wave_sum(acc);
          if (lane == 0) part[row * kFW + w] = v;
          acc = 0.0f;
        }
      } else {
        ++c.j;
      }
      // refill slot i, kD packets ahead (the run is padded to whole groups of kD)
      if (!r.iss_next && r.iss.j >= ng * kD) { r.iss = cursor_begin(next); r.iss_next = 1; }
      const Stream<P>& src = r.iss_next ? next : s;
      r.buf[i] = load_at(src, r.iss);
      cursor_step(r.iss, src.nch);
    }
  }
  if (ng == 0) {
    // nothing of this phase for this wave: prime the ring with the next phase
    r.iss = cursor_begin(next);
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      r.buf[i] = load_at(next, r.iss);
      cursor_step(r.iss, next.nch);
    }
  }
  // the ring holds the first kD packets of `next`; its issue cursor is kD packets into next's run
  r.iss_next = 0;
  __syncthreads();
}

// Sum of a row's per-wave partials in wave order (deterministic); zeroes them for the next phase.
__device__ __forceinline__ float row_sum(float* part, int row) {
  float y = 0.0f;
#pragma unroll
  for (int w = 0; w < kFW; ++w) { y += part[row * kFW + w]; part[row * kFW + w] = 0.0f; }
  return y;
}

// ---------------------------------------------------------------- phase inputs into LDS (bf16 pairs)
template <int P>
__device__ __forceinline__ uint32_t act_bits(float v, float scale) {
  // value in GEMV units (bf16-rounded value, or the e4m3 code value), as bf16 bits (exact)
  return f32_to_bf16(act_round<P>(v, scale));
}

// Tagged words are polled in batches: every load of a batch is issued before any
// tag is checked (one memory round trip per attempt), and only words that did
// not yet carry the expected tag are loaded again.
template <int N>
__device__ __forceinline__ bool poll_batch64(const uint64_t* base, int stride, int count, unsigned tag,
                                             uint64_t (&wv)[N], Poll& pl) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int k = i * stride + t;
    wv[i] = k < count ? ld64(base + k) : ((uint64_t)tag << 32);
  }
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && ((unsigned)(wv[i] >> 32) == tag);
    if (ok) return true;
    if (!pl.again()) return false;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = i * stride + t;
      if ((unsigned)(wv[i] >> 32) != tag) wv[i] = ld64(base + k);
    }
  }
}
template <int N>
__device__ __forceinline__ bool poll_batch32(const uint32_t* base, int stride, int count, unsigned tag,
                                             uint32_t (&wv)[N], Poll& pl) {
  const int t = threadIdx.x;
  const unsigned t16 = tag & 0xffffu;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int k = i * stride + t;
    wv[i] = k < count ? ld32(base + k) : (t16 << 16);
  }
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && ((wv[i] >> 16) == t16);
    if (ok) return true;
    if (!pl.again()) return false;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = i * stride + t;
      if ((wv[i] >> 16) != t16) wv[i] = ld32(base + k);
    }
  }
}

// xs = act(rmsnorm(h) * g), h polled from the tagged residual
template <int P>
__device__ __forceinline__ bool norm_to_lds(const uint64_t* xh, unsigned tag, const float* g, int K, float eps,
                                            float scale, uint32_t* xs, float* red, unsigned* abort_flag, int* okf) {
  Poll pl;
  pl.start(abort_flag);
  constexpr int kMaxPer = 16;  // K <= 16 * kFT
  uint64_t wv[kMaxPer];
  const bool got = poll_batch64<kMaxPer>(xh, kFT, K, tag, wv, pl);
  if (!block_ok(got, okf)) return false;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int k = i * kFT + threadIdx.x;
    const float v = k < K ? __uint_as_float((uint32_t)wv[i]) : 0.0f;
    ss = fmaf(v, v, ss);
  }
  ss = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)K + eps);
  uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int k = i * kFT + threadIdx.x;
    if (k < K) xs16[k] = (uint16_t)act_bits<P>(__uint_as_float((uint32_t)wv[i]) * rstd * *gp(g + k), scale);
  }
  __syncthreads();
  return true;
}

// xs from a tagged exchange buffer already in GEMV units (bf16 bits)
__device__ __forceinline__ bool act_to_lds(const uint32_t* x, unsigned tag, int K, uint32_t* xs,
                                           unsigned* abort_flag, int* okf) {
  Poll pl;
  pl.start(abort_flag);
  constexpr int kMaxPer = 20;  // K <= 20 * kFT
  uint32_t wv[kMaxPer];
  const bool got = poll_batch32<kMaxPer>(x, kFT, K, tag, wv, pl);
  uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int k = i * kFT + threadIdx.x;
    if (k < K) xs16[k] = (uint16_t)(wv[i] & 0xffffu);
  }
  return block_ok(got, okf);
}

// ---------------------------------------------------------------- attention task (split-K, one kv head)
struct AttnLds {
  float qs[8][128];
  float kn[128], vn[128];
  float Kt[kAttnTile][129];
  float Vt[kAttnTile][128];
  float ps[8][kAttnTile];
};

template <int HD>
__device__ __forceinline__ void attn_norm_rope(const uint64_t* src, unsigned tag, const float* g, const float* cs,
                                               const float* sn, float eps, int lane, float* dst, Poll& pl) {
  constexpr int H2 = HD / 2;
  const bool act = lane < H2;
  uint64_t w0 = act ? ld64(src + lane) : ((uint64_t)tag << 32);
  uint64_t w1 = act ? ld64(src + lane + H2) : ((uint64_t)tag << 32);
  while (pl.ok && ((unsigned)(w0 >> 32) != tag || (unsigned)(w1 >> 32) != tag)) {
    if (!pl.again()) break;
    if ((unsigned)(w0 >> 32) != tag) w0 = ld64(src + lane);
    if ((unsigned)(w1 >> 32) != tag) w1 = ld64(src + lane + H2);
  }
  const float x0 = act ? __uint_as_float((uint32_t)w0) : 0.0f;
  const float x1 = act ? __uint_as_float((uint32_t)w1) : 0.0f;
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float rstd = 1.0f / sqrtf(ss / (float)HD + eps);
  if (act) {
    const float a = x0 * rstd * *gp(g + lane);
    const float b = x1 * rstd * *gp(g + lane + H2);
    const float c = *gp(cs + lane), s = *gp(sn + lane);
    dst[lane] = round_bf16(a * c - b * s);
    dst[lane + H2] = round_bf16(b * c + a * s);
  }
}

// One block = one (kv head, key split) task.  Split 0 of each kv head merges the
// other active splits' partials (polled by tag) and publishes the attention output.
// Returns false if the frame was abandoned.
template <int P, int HD>
__device__ __forceinline__ bool attn_task(const FrameArgs a, const LayerW L, int layer, int pos, unsigned tag_qkv,
                          unsigned tag_part, unsigned tag_o, AttnLds& sm, unsigned* abort_flag, int* okf) {
  constexpr int H2 = HD / 2;
  constexpr int T = kAttnTile;
  const int G = a.Hq / a.Hkv;
  const int ntask = a.Hkv * a.splits;
  const int task = blockIdx.x;
  if (task >= ntask) return true;
  const int j = task / a.splits, split = task % a.splits;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nkeys = pos + 1;
  int chunk = (nkeys + a.splits - 1) / a.splits;
  chunk = (chunk + T - 1) / T * T;
  const int n_active = (nkeys + chunk - 1) / chunk;
  if (split >= n_active) return true;
  const int beg = split * chunk, end = min(nkeys, beg + chunk);
  const float* cs = a.rope_cos + (size_t)pos * H2;
  const float* sn = a.rope_sin + (size_t)pos * H2;
  Poll pl;
  pl.start(abort_flag);
  if (w < G) attn_norm_rope<HD>(a.xqkv + (size_t)(j * G + w) * HD, tag_qkv, L.g_q, cs, sn, a.eps, lane, sm.qs[w], pl);
  if (w == G) attn_norm_rope<HD>(a.xqkv + (size_t)a.Hq * HD + (size_t)j * HD, tag_qkv, L.g_k, cs, sn, a.eps, lane, sm.kn, pl);
  if (w == G + 1) {
    const uint64_t* vsrc = a.xqkv + (size_t)(a.Hq + a.Hkv) * HD + (size_t)j * HD;
    const uint64_t want = (uint64_t)tag_qkv << 32;
    uint64_t v0 = lane < HD ? ld64(vsrc + lane) : want;
    uint64_t v1 = HD > 64 ? ld64(vsrc + lane + 64) : want;
    while (pl.ok && ((unsigned)(v0 >> 32) != tag_qkv || (unsigned)(v1 >> 32) != tag_qkv)) {
      if (!pl.again()) break;
      if ((unsigned)(v0 >> 32) != tag_qkv) v0 = ld64(vsrc + lane);
      if ((unsigned)(v1 >> 32) != tag_qkv) v1 = ld64(vsrc + lane + 64);
    }
    if (lane < HD) sm.vn[lane] = round_bf16(__uint_as_float((uint32_t)v0));
    if (HD > 64) sm.vn[lane + 64] = round_bf16(__uint_as_float((uint32_t)v1));
  }
  if (!block_ok(pl.ok, okf)) return false;
  uint16_t* kc = L.k_cache + (size_t)j * a.max_seq * HD;
  uint16_t* vc = L.v_cache + (size_t)j * a.max_seq * HD;
  if (beg <= pos && pos < end && tid < HD) {
    *gpw(kc + (size_t)pos * HD + tid) = (uint16_t)f32_to_bf16(sm.kn[tid]);
    *gpw(vc + (size_t)pos * HD + tid) = (uint16_t)f32_to_bf16(sm.vn[tid]);
  }
  const float inv_sqrt = 1.0f / sqrtf((float)HD);
  float m = -INFINITY, lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
  constexpr int SEG = HD / 8;
  for (int t0 = beg; t0 < end; t0 += T) {
    for (int idx = tid; idx < T * SEG; idx += kFT) {
      const int key = idx / SEG, seg = idx % SEG;
      const int kp = t0 + key;
      float kv[8], vv[8];
      if (kp < end && kp != pos) {
        const uint4 kw = ld16(kc + (size_t)kp * HD + seg * 8);
        const uint4 vw = ld16(vc + (size_t)kp * HD + seg * 8);
        const uint32_t ks[4] = {kw.x, kw.y, kw.z, kw.w}, vs[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[2 * e] = bf16lo(ks[e]); kv[2 * e + 1] = bf16hi(ks[e]);
          vv[2 * e] = bf16lo(vs[e]); vv[2 * e + 1] = bf16hi(vs[e]);
        }
      } else if (kp == pos && kp < end) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kv[e] = sm.kn[seg * 8 + e]; vv[e] = sm.vn[seg * 8 + e]; }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kv[e] = 0.0f; vv[e] = 0.0f; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) { sm.Kt[key][seg * 8 + e] = kv[e]; sm.Vt[key][seg * 8 + e] = vv[e]; }
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
          d0 = fmaf(sm.qs[w][e], sm.Kt[lane][e], d0);
          d1 = fmaf(sm.qs[w][e + 1], sm.Kt[lane][e + 1], d1);
        }
        s = (d0 + d1) * inv_sqrt;
      }
      mnew = fmaxf(m, wave_max(s));
      const float p = (kp < end) ? __expf(s - mnew) : 0.0f;
      scale = __expf(m - mnew);
      lsum = lsum * scale + wave_sum(p);
      sm.ps[w][lane] = p;
    }
    __syncthreads();
    if (w < G) {
      o0 *= scale;
      o1 *= scale;
      const int nk = min(T, end - t0);
      for (int kk = 0; kk < nk; ++kk) {
        const float p = sm.ps[w][kk];
        if (lane < HD) o0 = fmaf(p, sm.Vt[kk][lane], o0);
        if (HD > 64) o1 = fmaf(p, sm.Vt[kk][(lane + 64) % HD], o1);
      }
      m = mnew;
    }
    __syncthreads();
  }
  const float so = P == kFP8 ? *gp(a.act_scales + kSitesPerLayer * layer + 1) : 1.0f;
  if (split != 0) {
    // publish this split's (o, m, l)
    if (w < G) {
      const int h = j * G + w;
      uint64_t* pp = a.xpart + ((size_t)h * a.splits + split) * (HD + 2);
      if (lane < HD) st64(pp + lane, o0, tag_part);
      if (HD > 64) st64(pp + lane + 64, o1, tag_part);
      if (lane == 0) { st64(pp + HD, m, tag_part); st64(pp + HD + 1, lsum, tag_part); }
    }
    return true;
  }
  // split 0: merge with the other active splits (log-sum-exp) and publish the output
  Poll pm;
  pm.start(abort_flag);
  if (w < G) {
    const int h = j * G + w;
    const uint64_t* pb = a.xpart + (size_t)h * a.splits * (HD + 2);
    // lane s (1 <= s < n_active) holds split s's (m, l); lane 0 holds split 0's own
    const bool other = lane > 0 && lane < n_active;
    uint64_t wm = other ? ld64(pb + (size_t)lane * (HD + 2) + HD) : ((uint64_t)tag_part << 32);
    uint64_t wl = other ? ld64(pb + (size_t)lane * (HD + 2) + HD + 1) : ((uint64_t)tag_part << 32);
    while (pm.ok && ((unsigned)(wm >> 32) != tag_part || (unsigned)(wl >> 32) != tag_part)) {
      if (!pm.again()) break;
      if ((unsigned)(wm >> 32) != tag_part) wm = ld64(pb + (size_t)lane * (HD + 2) + HD);
      if ((unsigned)(wl >> 32) != tag_part) wl = ld64(pb + (size_t)lane * (HD + 2) + HD + 1);
    }
    const float ms = other ? __uint_as_float((uint32_t)wm) : (lane == 0 ? m : -INFINITY);
    const float ls = other ? __uint_as_float((uint32_t)wl) : (lane == 0 ? lsum : 0.0f);
    const float M = wave_max(ls > 0.0f ? ms : -INFINITY);
    const float f = (ls > 0.0f) ? __expf(ms - M) : 0.0f;
    const float den = wave_sum(f * ls);
    const float f0 = __shfl(f, 0, kWave);
    float n0 = f0 * o0, n1 = f0 * o1;
    // the other splits' o vectors, 8 splits per batch, each word polled by its own tag
    const uint64_t want = (uint64_t)tag_part << 32;
    for (int sp0 = 1; sp0 < n_active && pm.ok; sp0 += 4) {
      uint64_t x0[4], x1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sp = sp0 + u;
        const uint64_t* q = pb + (size_t)(sp < n_active ? sp : 0) * (HD + 2);
        x0[u] = (sp < n_active && lane < HD) ? ld64(q + lane) : want;
        x1[u] = (sp < n_active && HD > 64) ? ld64(q + lane + 64) : want;
      }
      while (pm.ok) {
        bool ok = true;
#pragma unroll
        for (int u = 0; u < 4; ++u) ok = ok && (unsigned)(x0[u] >> 32) == tag_part && (unsigned)(x1[u] >> 32) == tag_part;
        if (ok || !pm.again()) break;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint64_t* q = pb + (size_t)(sp0 + u) * (HD + 2);
          if ((unsigned)(x0[u] >> 32) != tag_part) x0[u] = ld64(q + lane);
          if ((unsigned)(x1[u] >> 32) != tag_part) x1[u] = ld64(q + lane + 64);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sp = sp0 + u;
        const float fs = __shfl(f, sp < n_active ? sp : 0, kWave);
        if (sp < n_active) {
          n0 = fmaf(fs, __uint_as_float((uint32_t)x0[u]), n0);
          n1 = fmaf(fs, __uint_as_float((uint32_t)x1[u]), n1);
        }
      }
    }
    const float inv = 1.0f / den;
    if (lane < HD) st32(a.xo + (size_t)h * HD + lane, act_bits<P>(n0 * inv, so), tag_o);
    if (HD > 64) st32(a.xo + (size_t)h * HD + lane + 64, act_bits<P>(n1 * inv, so), tag_o);
  }
  return block_ok(pm.ok, okf);
}

// ---------------------------------------------------------------- the frame
// The frame is a sequence of phases: per layer QKV, ATTN, O, GU, DOWN, then
// HEAD.  GEMV phases share one code path (prologue / packet stream / epilogue
// chosen by the phase kind), so the streaming loop exists once in the binary.
enum PhaseKind { kQKV = 0, kATTN = 1, kO = 2, kGU = 3, kDOWN = 4, kHEAD = 5 };

template <int P, int HD>
__device__ __forceinline__ Stream<P> phase_stream(const FrameArgs& a, int phase) {
  const int layer = phase / 5, kind = phase % 5;
  const int d = a.d, qd = a.Hq * HD, W = (a.Hq + 2 * a.Hkv) * HD;
  if (layer >= a.n_layers) return make_stream<P>(a.w_head, a.C * a.V, d, 0);
  const LayerW* L = a.layers + layer;
  switch (kind) {
    case kQKV: return make_stream<P>(L->w_qkv, W, d, 0);
    case kO: return make_stream<P>(L->w_o, d, qd, 0);
    case kGU: return make_stream<P>(L->w_gu, 2 * a.F, d, 1);
    default: return make_stream<P>(L->w_d, d, a.F, 0);
  }
}

template <int P, int HD>
__global__ __launch_bounds__(kFT) void k_frame(FrameArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem_raw);                    // activations, bf16 pairs (<= 10240)
  float* part = reinterpret_cast<float*>(smem_raw + 5120 * 4);              // per-(row, wave) partials
  AttnLds& sm = *reinterpret_cast<AttnLds*>(smem_raw + 5120 * 4 + kPartMax * 4);
  __shared__ float red[16];
  __shared__ int sh_state[4 + kMaxCodebooks];
  __shared__ int okf;
  const int tid = threadIdx.x;
  unsigned* abort_flag = a.sync + 64;
  const unsigned launch = a.sync[0];
  // phase p of the frame tags its outputs with base + 1 + p; the frame input uses base
  const unsigned base = (launch + 1u) * (8u + 8u * (unsigned)a.n_layers);

  if (tid == 0) {
    sh_state[0] = a.st->len;
    sh_state[1] = a.st->t;
    int eoc = a.st->eoc;
    if (eoc < 0 && a.st->t > 0 && a.st->prev[0] == a.eos) eoc = a.st->t - 1;
    sh_state[2] = eoc;
    for (int c = 0; c < a.C; ++c) sh_state[4 + c] = a.st->prev[c];
  }
  __syncthreads();
  const int pos = sh_state[0];
  const int d = a.d;

  Ring<P> ring;
  Stream<P> cur = phase_stream<P, HD>(a, 0);
  ring_prime(ring, cur);
  for (int i = tid; i < kPartMax; i += kFT) part[i] = 0.0f;

  // frame input: h = sum_k E_aud[k][prev_k]; every block forms the whole vector for
  // the first norm and publishes the rows it owns (the O/DOWN row split of d)
  {
    const Stream<P> own = make_stream<P>(nullptr, d, 1, 0);
    constexpr int kMaxPer = 16;
    float hv[kMaxPer];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int k = i * kFT + tid;
      hv[i] = 0.0f;
      if (k < d) {
        float v = 0.0f;
        for (int c = 0; c < a.C; ++c) v += bf16_to_f32(*gp(a.e_aud + ((size_t)c * a.V + sh_state[4 + c]) * d + k));
        hv[i] = v;
        ss = fmaf(v, v, ss);
      }
    }
    for (int r = tid; r < own.nrows; r += kFT) {
      const int k = own.r0 + r;
      float v = 0.0f;
      for (int c = 0; c < a.C; ++c) v += bf16_to_f32(*gp(a.e_aud + ((size_t)c * a.V + sh_state[4 + c]) * d + k));
      st64(a.xh + k, v, base);
      if (a.taps) *gpw(a.taps + k) = v;
    }
    ss = block_sum(ss, red);
    const float rstd = 1.0f / sqrtf(ss / (float)d + a.eps);
    const float sc = P == kFP8 ? a.act_scales[0] : 1.0f;
    const float* g = a.layers[0].g_attn;
    uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int k = i * kFT + tid;
      if (k < d) xs16[k] = (uint16_t)act_bits<P>(hv[i] * rstd * *gp(g + k), sc);
    }
    __syncthreads();
  }

  const int n_phases = 5 * a.n_layers + 1;
  unsigned tag_h = base;   // tag of the residual's latest value
  for (int phase = 0; phase < n_phases; ++phase) {
    const int layer = phase / 5;
    const int kind = layer >= a.n_layers ? kHEAD : phase % 5;
    const unsigned tag = base + 1u + (unsigned)phase;
    if (kind == kATTN) {
      const LayerW L = a.layers[layer];
      // inputs: the QKV phase (tag - 1); partials and output carry this phase's tag
      if (!attn_task<P, HD>(a, L, layer, pos, tag - 1u, tag, tag, sm, abort_flag, &okf)) return;
      continue;
    }
    const int site = kind == kHEAD ? kSitesPerLayer * a.n_layers
                   : kSitesPerLayer * layer + (kind == kQKV ? 0 : kind == kO ? 1 : kind == kGU ? 2 : 3);
    const float sc_in = P == kFP8 ? a.act_scales[site] : 1.0f;
    // ---- prologue: the phase input in LDS
    if (kind == kQKV || kind == kGU || kind == kHEAD) {
      if (!(kind == kQKV && layer == 0)) {
        const float* g = kind == kHEAD ? a.g_final : (kind == kQKV ? a.layers[layer].g_attn : a.layers[layer].g_mlp);
        if (!norm_to_lds<P>(a.xh, tag_h, g, d, a.eps, sc_in, xs, red, abort_flag, &okf)) return;
      }
    } else {
      // O reads the attention output (phase tag - 1), DOWN the SiLU*mul output (tag - 1)
      const uint32_t* src = kind == kO ? a.xo : a.xa;
      const int K = kind == kO ? a.Hq * HD : a.F;
      if (!act_to_lds(src, tag - 1u, K, xs, abort_flag, &okf)) return;
    }
    // ---- stream the weights; the next GEMV phase's first packets follow
    int nphase = phase + 1;
    if (nphase < n_phases && nphase / 5 < a.n_layers && nphase % 5 == kATTN) ++nphase;
    Stream<P> nxt = cur;
    if (nphase < n_phases) nxt = phase_stream<P, HD>(a, nphase);
    else nxt.nrows = 0;
    run_stream<P>(cur, nxt, ring, xs, part);
    // ---- epilogue
    const float* wsc = nullptr;
    if (P == kFP8) {
      if (kind == kHEAD) wsc = a.s_head;
      else {
        const LayerW* L = a.layers + layer;
        wsc = kind == kQKV ? L->s_qkv : kind == kO ? L->s_o : kind == kGU ? L->s_gu : L->s_d;
      }
    }
    if (kind == kGU) {
      const float sc_out = P == kFP8 ? a.act_scales[site + 1] : 1.0f;
      for (int r2 = tid; r2 < cur.nrows / 2; r2 += kFT) {
        const int row = cur.r0 + 2 * r2;
        const float g = row_sum(part, 2 * r2) * (P == kFP8 ? sc_in * *gp(wsc + row) : 1.0f);
        const float u = row_sum(part, 2 * r2 + 1) * (P == kFP8 ? sc_in * *gp(wsc + row + 1) : 1.0f);
        st32(a.xa + row / 2, act_bits<P>(silu(g) * u, sc_out), tag);
      }
    } else {
      for (int r = tid; r < cur.nrows; r += kFT) {
        const int row = cur.r0 + r;
        const float y = row_sum(part, r) * (P == kFP8 ? sc_in * *gp(wsc + row) : 1.0f);
        if (kind == kQKV) {
          st64(a.xqkv + row, y, tag);
        } else if (kind == kHEAD) {
          st64(a.xlogits + row, y, tag);
        } else {
          // O / DOWN: residual update of this block's own rows
          const float hn = __uint_as_float((uint32_t)ld64(a.xh + row)) + y;
          st64(a.xh + row, hn, tag);
          if (kind == kDOWN && layer + 1 == a.n_layers) *gpw(a.h_out + row) = hn;
          if (kind == kDOWN && a.taps) *gpw(a.taps + (size_t)(layer + 1) * d + row) = hn;
        }
      }
      if (kind == kO || kind == kDOWN) tag_h = tag;
    }
    cur = nxt;
  }
  const unsigned tag_logits = base + (unsigned)n_phases;
  if (blockIdx.x != 0) return;

  // ---- block 0: per-codebook argmax over the allowed ids, delay rule, state advance
  __shared__ int sh_arg[kMaxCodebooks];
  __shared__ float sh_bv[2 * kMaxCodebooks];
  __shared__ int sh_bi[2 * kMaxCodebooks];
  const int lane = tid & 63, wv = tid >> 6;
  Poll pl;
  pl.start(abort_flag);
  constexpr int kVPL = 16;  // logits per lane per pass; passes cover codebook_size <= 2048
  for (int kk = wv; kk < a.C * 2; kk += kFW) {
    const int k = kk >> 1, half = kk & 1;
    const uint64_t* lg = a.xlogits + (size_t)k * a.V + half * kVPL * kWave;
    const uint64_t want = (uint64_t)tag_logits << 32;
    uint64_t lw[kVPL];
#pragma unroll
    for (int q = 0; q < kVPL; ++q) {
      const int i = half * kVPL * kWave + q * kWave + lane;
      lw[q] = i < a.V ? ld64(lg + q * kWave + lane) : want;
    }
    while (pl.ok) {
      bool ok = true;
#pragma unroll
      for (int q = 0; q < kVPL; ++q) ok = ok && (unsigned)(lw[q] >> 32) == tag_logits;
      if (ok || !pl.again()) break;
#pragma unroll
      for (int q = 0; q < kVPL; ++q)
        if ((unsigned)(lw[q] >> 32) != tag_logits) lw[q] = ld64(lg + q * kWave + lane);
    }
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kVPL; ++q) {
      const int i = half * kVPL * kWave + q * kWave + lane;
      if (i < a.V) {
        const float v = __uint_as_float((uint32_t)lw[q]);
        *gpw(a.logits_out + (size_t)k * a.V + i) = v;
        const bool allowed = (i < a.bos) || (k == 0 && i == a.eos);
        if (allowed && (v > bv || (v == bv && i < bi))) { bv = v; bi = i; }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) { sh_bv[kk] = bv; sh_bi[kk] = bi; }
  }
  __syncthreads();
  if (tid < a.C) {
    // merge the two halves of each codebook (lower index first on ties)
    const float v0 = sh_bv[2 * tid], v1 = sh_bv[2 * tid + 1];
    const int i0 = sh_bi[2 * tid], i1 = sh_bi[2 * tid + 1];
    sh_arg[tid] = (v1 > v0 || (v1 == v0 && i1 < i0)) ? i1 : i0;
  }
  if (!block_ok(pl.ok, &okf)) return;
  if (tid == 0) {
    DevState* st = a.st;
    const int t = sh_state[1], eoc = sh_state[2];
    for (int k = 0; k < a.C; ++k) {
      int c;
      if (t < k) c = a.bos;
      else if (eoc >= 0 && t >= eoc + k) c = a.eos;
      else c = sh_arg[k];
      sh_arg[k] = c;
    }
    const int eoc2 = eoc >= 0 ? eoc : (sh_arg[0] == a.eos ? t : -1);
    const int done = (eoc2 >= 0 && t >= eoc2 + a.C - 1) ? 1 : 0;
    for (int k = 0; k < a.C; ++k) {
      st->codes[k] = sh_arg[k];
      st->prev[k] = sh_arg[k];
      *gpw(a.hist + (size_t)t * a.C + k) = sh_arg[k];
    }
    st->eoc = eoc;
    st->t = t + 1;
    st->len = pos + 1;
    st->done = done;
    st->n_done += done;
    a.sync[0] = launch + 1u;
  }
}

// ---------------------------------------------------------------- launcher
size_t frame_lds_bytes() { return 5120 * 4 + kPartMax * 4 + sizeof(AttnLds); }

hipError_t launch_frame_persistent(Ctx& c) {
  const hta_config& f = c.cfg;
  FrameArgs a{};
  a.d = f.hidden; a.hd = f.head_dim; a.Hq = f.n_q_heads; a.Hkv = f.n_kv_heads; a.F = f.ffn;
  a.C = f.n_codebooks; a.V = f.codebook_size; a.bos = f.bos_id; a.eos = f.eos_id; a.n_layers = f.n_layers;
  a.max_seq = f.max_seq; a.eps = f.rms_eps;
  a.layers = c.d_layers; a.e_aud = c.e_aud; a.g_final = c.g_final; a.w_head = c.w_head; a.s_head = c.s_head;
  a.rope_cos = c.rope_cos; a.rope_sin = c.rope_sin; a.act_scales = c.act_scales;
  a.xh = c.x_h; a.xqkv = c.x_qkv; a.xo = c.x_o; a.xa = c.x_a; a.xpart = c.x_part; a.xlogits = c.x_logits;
  a.h_out = c.h; a.logits_out = c.logits;
  a.taps = c.taps ? c.taps_h : nullptr;
  a.sync = c.sync; a.st = c.state; a.hist = c.hist;
  a.splits = c.frame_splits;
  const size_t lds = frame_lds_bytes();
  void* args[] = {&a};
  void* fn;
  if (f.precision == HTA_FP8_E4M3) fn = f.head_dim == 128 ? (void*)k_frame<kFP8, 128> : (void*)k_frame<kFP8, 64>;
  else fn = f.head_dim == 128 ? (void*)k_frame<kBF16, 128> : (void*)k_frame<kBF16, 64>;
  time_begin(c, HTA_K_FRAME);
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(c.frame_blocks), dim3(kFT), args, lds, c.stream);
  time_end(c);
  return e;
}

hipError_t frame_setup(Ctx& c) {
  const size_t lds = frame_lds_bytes();
  hipError_t e;
  void* fns[4] = {(void*)k_frame<kFP8, 128>, (void*)k_frame<kFP8, 64>, (void*)k_frame<kBF16, 128>,
                  (void*)k_frame<kBF16, 64>};
  for (void* fn : fns)
    if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess) return e;
  int cus = 0;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c.device)) != hipSuccess) return e;
  void* fn = c.cfg.precision == HTA_FP8_E4M3 ? (c.cfg.head_dim == 128 ? fns[0] : fns[1])
                                             : (c.cfg.head_dim == 128 ? fns[2] : fns[3]);
  int per_cu = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kFT, lds)) != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  c.frame_blocks = cus;  // one block per CU
  int splits = c.frame_blocks / c.cfg.n_kv_heads;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  c.frame_splits = splits;
  return hipSuccess;
}

// Largest number of per-(row, wave) partials any block holds in one phase (must fit kPartMax).
int frame_max_packets(const hta_config& f, int blocks) {
  auto pk = [&](long n, long k, int eb) {
    (void)k; (void)eb;
    const long rows = (n + blocks - 1) / blocks + 2;
    return rows * kFW;
  };
  const int eb = f.precision == HTA_FP8_E4M3 ? 1 : 2;
  const long qd = (long)f.n_q_heads * f.head_dim, W = qd + 2L * f.n_kv_heads * f.head_dim;
  long m = pk(W, f.hidden, eb);
  const long cands[4] = {pk(f.hidden, qd, eb), pk(2L * f.ffn, f.hidden, eb), pk(f.hidden, f.ffn, eb),
                         pk((long)f.n_codebooks * f.codebook_size, f.hidden, eb)};
  for (long v : cands) m = v > m ? v : m;
  if (f.hidden > 16 * kFT) return 1 << 30;  // the norm prologue holds at most 16 values per thread
  return (int)m;
}
int frame_part_capacity() { return kPartMax; }

}  // namespace hta
