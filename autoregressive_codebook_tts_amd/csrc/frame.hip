// Persistent decode-frame kernel for gfx950: the whole frame (embedding,
// n_layers x [qkv GEMV, attention, o_proj GEMV, gate/up GEMV, down GEMV],
// head, argmax + delay bookkeeping) in one launch of one resident block per
// compute unit.
//
// Reference: FlashRT "Higgs Audio v3 TTS-4B" page, section 5 (the per-frame
// chain) and section 7 (the decode floor is set by streaming every weight once
// per frame; the frame is replayed as one position-agnostic graph).
//
// Design (MI355X):
//  * Every GEMV phase splits its rows across the blocks; a block's rows are one
//    contiguous byte range, cut into one piece per wave.  Each wave fetches its
//    pieces, phase after phase, as 1 KB packets straight into an LDS ring of
//    kRD slots (global_load_lds_dwordx4), kRD packets ahead of consumption, so
//    the weight stream runs on through the waits for the next phase's inputs
//    and through attention without holding registers.
//  * Constant operands (norm gains, FP8 row scales, the first attention key
//    tile, RoPE rows) are issued before a phase waits for its inputs.
//  * No grid barriers.  Every value handed from one block to another inside the
//    launch travels with a tag in the same atomic word (64-bit value+tag, or a
//    16-bit payload with a 16-bit tag); the tag is a running phase number, so a
//    consumer polls exactly the inputs it needs until they carry the current
//    phase's tag.  Producers never wait and need no release fence.  A buffer is rewritten
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
constexpr int kRD = 15;             // LDS ring slots (1 KB packets) per wave
constexpr int kPartMax = 1024;      // packet partial sums per block per phase
constexpr uint64_t kSpinLimit = 50000000ull;  // 0.5 s at the 100 MHz constant clock

struct FrameArgs {
  int d, hd, Hq, Hkv, F, C, V, bos, eos, n_layers, max_seq, splits;
  float eps;
  const LayerW* layers;      // device copy of the per-layer pointers
  const unsigned char* wl0;  // layer 0's block; layer l's weights are at wl0 + l * lstride + off_*
  unsigned long long lstride;
  unsigned long long off_wqkv, off_wo, off_wgu, off_wd;
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
  uint16_t* acts;            // [5 * n_layers + 1][kActsWidth] GEMV input of each phase (block 0), or null
  uint16_t* q_tap;           // [n_layers][Hq * hd] rotated queries (bf16), or null
  const float* h_in;         // [d] frame input in place of the codebook embedding sum, or null
  float* amax;               // [4L + 1] max |x| of each activation site before rounding, or null
  uint32_t* trace;           // [blocks][5 * n_layers + 1][8] phase timestamps and counters, or null
  unsigned* sync;            // [0] launch count, [64] abort flag
  DevState* st;
  int32_t* hist;
  float temperature;         // 0: greedy argmax; > 0: categorical draw at this temperature
  uint32_t seed_lo, seed_hi; // the draw's 64-bit seed
  uint32_t input_tag_skew;   // 0; otherwise added to layer 0's attention input tag (a wait that cannot end)
};

// The kernel reads FrameArgs through the constant address space: every field is a
// scalar (s_load) read that never waits on vector-memory counters.
typedef const __attribute__((address_space(4))) FrameArgs CFA;
// The per-layer pointer table is read the same way: a vector load of a pointer
// would need a vector-memory counter wait before its use, and that wait would also
// wait for every weight fetch the ring has in flight.
typedef const __attribute__((address_space(4))) LayerW CLW;
__device__ __forceinline__ CLW* layer_ptrs(CFA& a, int layer) { return (CLW*)a.layers + layer; }
// FP8 row-scale pointer i of a layer (0 qkv, 1 o_proj, 2 gate/up, 3 down): the four
// pointers sit side by side in LayerW, so this is one indexed scalar read (a
// multi-way select over the fields, lowered to branches, picked the wrong field here)
static_assert(offsetof(LayerW, s_o) == offsetof(LayerW, s_qkv) + sizeof(float*) &&
                  offsetof(LayerW, s_gu) == offsetof(LayerW, s_qkv) + 2 * sizeof(float*) &&
                  offsetof(LayerW, s_d) == offsetof(LayerW, s_qkv) + 3 * sizeof(float*),
              "LayerW scale pointers must be adjacent");
__device__ __forceinline__ const float* layer_scales(CFA& a, int layer, int i) {
  typedef const __attribute__((address_space(4))) uint64_t CU64;
  const CU64* p = (const CU64*)((const __attribute__((address_space(4))) char*)layer_ptrs(a, layer) +
                                offsetof(LayerW, s_qkv));
  return reinterpret_cast<const float*>(p[i]);
}
// the static activation scales, likewise (uniform index, scalar read)
__device__ __forceinline__ float act_scale(CFA& a, int site) {
  return ((const __attribute__((address_space(4))) float*)a.act_scales)[site];
}

// ---------------------------------------------------------------- sampling head
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds over the counter
// (c0, c1, 0, 0) with the key (k0, k1) advanced by the two Weyl constants between rounds;
// each round multiplies words 0 and 2 by the round constants into 64-bit products.  The
// draw's uniform is the top 24 bits of output word 0, exact in fp32, in [0, 1).
__device__ __forceinline__ float philox_uniform(uint32_t k0, uint32_t k1, uint32_t c0, uint32_t c1) {
  uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, x0), lo0 = 0xD2511F53u * x0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, x2), lo1 = 0xCD9E8D57u * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
  return (float)(x0 >> 8) * (1.0f / 16777216.0f);
}

// One wave draws codebook k's code from its fp32 logits z[V] (LDS): weights
// exp((z_i - m) / T) over the allowed finite logits, m their maximum; the draw is the
// first id whose running weight (in id order) exceeds u times the total.  Lane l holds
// the contiguous ids [l * c, l * c + c); the running weight is the lane's sequential sum
// added to an inclusive scan of the lane sums.  Returns the id in every lane.
__device__ __forceinline__ int sample_codebook(const float* z, int V, int k, int bos, int eos, float T, float u) {
  const int lane = threadIdx.x & 63;
  const int c = (V + kWave - 1) / kWave;
  const int i0 = lane * c, i1 = min(i0 + c, V);
  auto weight_ok = [&](int i, float v) { return ((i < bos) || (k == 0 && i == eos)) && v == v; };
  float mx = -INFINITY;
  for (int i = i0; i < i1; ++i) {
    const float v = z[i];
    if (weight_ok(i, v)) mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  if (!(mx > -INFINITY)) return 0;  // no allowed finite logit: the lowest allowed id, as the greedy path
  float s = 0.0f;
  for (int i = i0; i < i1; ++i) {
    const float v = z[i];
    if (weight_ok(i, v)) s += expf((v - mx) / T);
  }
  float incl = s;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const float o = __shfl_up(incl, dd, kWave);
    if (lane >= dd) incl += o;
  }
  // (the shuffle runs in every lane: a lane left out of it would read as zero to its neighbour)
  const float prev = __shfl_up(incl, 1, kWave);
  const float excl = lane == 0 ? 0.0f : prev;
  const float target = u * __shfl(incl, kWave - 1, kWave);
  const uint64_t hit = __ballot(incl > target);
  // the lane whose share holds the target; past the end (rounding), the last lane with weight
  const int owner = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(__ballot(s > 0.0f));
  int pick = -1, last = -1;
  if (lane == owner) {
    float acc = excl;
    for (int i = i0; i < i1; ++i) {
      const float v = z[i];
      if (!weight_ok(i, v)) continue;
      const float e = expf((v - mx) / T);
      if (e > 0.0f) last = i;
      acc += e;
      if (acc > target && e > 0.0f) {
        pick = i;
        break;
      }
    }
    if (pick < 0) pick = last;
  }
  return __shfl(pick, owner, kWave);
}

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

// Compiler barrier: loads written before it are issued before it, so that
// operands that do not depend on the frame travel with (or ahead of) a poll
// instead of being sunk to their first use after it.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// An opaque copy of a (wave-uniform) pointer.  Taken inside the phase loop it keeps
// the compiler from hoisting every per-thread address derived from the pointer out
// of the loop, which would hold dozens of 64-bit addresses in registers for the
// whole frame.
template <class T>
__device__ __forceinline__ T* launder(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Bounded poll state of one thread.
struct Poll {
  unsigned* abort_flag;
  uint64_t t0;
  unsigned n;
  bool ok;
  __device__ void start(unsigned* f) { abort_flag = f; t0 = __builtin_amdgcn_s_memrealtime(); n = 0; ok = true; }
  // one more round of waiting; false when the frame must be abandoned.  The abort
  // flag costs a memory round trip, so it is read on every 16th round only.
  __device__ bool again() {
    __builtin_amdgcn_s_sleep(1);
    if ((++n & 15u) == 0u &&
        __hip_atomic_load(gp(abort_flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) { ok = false; return false; }
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
  // every thread reads the same word: take lane 0's, so the branches on it stay uniform
  return __builtin_amdgcn_readfirstlane(*flag) != 0;
}

// ---------------------------------------------------------------- the rows of one GEMV phase
// A block owns the rows [r0, r0 + nrows) of the phase's row-major weight
// matrix: one contiguous byte range.  It is cut into kFW contiguous pieces, one
// per wave, at 16-byte boundaries, so the waves' shares differ by at most 16
// bytes; a wave streams its piece as consecutive 1 KB packets (16 bytes per
// lane), whatever the row length, so no lane is ever idle on a row tail.
template <int P>
struct Stream {
  const uint8_t* w;
  int K;        // elements per row
  int r0;       // first row of this block
  int nrows;    // rows of this block
  static constexpr int E = (P == kBF16) ? 8 : 16;  // elements per 16-byte lane packet
  static constexpr int B = (P == kBF16) ? 2 : 1;   // bytes per element
};

// Rows [r0, r0 + n) of N rows (N / 2 gate/up pairs when pair_rows) for this block.
__device__ __forceinline__ void block_rows(int N, int pair_rows, int* out) {
  const unsigned units = pair_rows ? (unsigned)N / 2u : (unsigned)N;
  const unsigned u0 = units * blockIdx.x / gridDim.x;  // units * gridDim.x < 2^31
  const unsigned u1 = units * (blockIdx.x + 1u) / gridDim.x;
  out[0] = (int)(pair_rows ? 2u * u0 : u0);
  out[1] = (int)(pair_rows ? 2u * (u1 - u0) : (u1 - u0));
}

// `split` is the block's table of rows per GEMV kind in LDS, [2 * kind] = first row,
// [2 * kind + 1] = count, filled once per launch with block_rows.
template <int P>
__device__ __forceinline__ Stream<P> make_stream(const int* split, const void* w, int K, int kind) {
  Stream<P> s;
  s.w = static_cast<const uint8_t*>(w);
  s.K = K;
  // LDS reads are not known to be uniform: take lane 0's so that the issue path stays scalar
  s.r0 = __builtin_amdgcn_readfirstlane(split[2 * kind]);
  s.nrows = __builtin_amdgcn_readfirstlane(split[2 * kind + 1]);
  return s;
}

// One wave's piece of a phase: bytes [b0, b1) counted from the block's first row.
struct Piece {
  const uint8_t* base;  // first byte of the block's first row
  int rowbytes;
  int b0, b1;
  int npk;              // 1 KB packets
};

template <int P>
__device__ __forceinline__ Piece make_piece(const Stream<P>& s) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Piece q;
  q.rowbytes = s.K * Stream<P>::B;
  q.base = s.w + (size_t)s.r0 * q.rowbytes;
  const int total = s.nrows * q.rowbytes;  // a multiple of 16, total * kFW < 2^31
  q.b0 = (total * w / kFW) & ~15;
  q.b1 = w + 1 == kFW ? total : (total * (w + 1) / kFW) & ~15;
  q.npk = (q.b1 - q.b0 + 1023) >> 10;
  return q;
}

// bf16-pair dot of one packet with its activations (bf16 pairs; x1 holds the second
// 16 bytes of an e4m3 packet's activations), in two partial chains
template <int P>
__device__ __forceinline__ float packet_dot(const uint4& wv, const uint4& x0, const uint4& x1) {
  float s0 = 0.0f, s1 = 0.0f;
  if (P == kBF16) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.x), __builtin_bit_cast(bf16x2, x0.x), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.y), __builtin_bit_cast(bf16x2, x0.y), s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.z), __builtin_bit_cast(bf16x2, x0.z), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.w), __builtin_bit_cast(bf16x2, x0.w), s1, false);
  } else {
    const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, false);
      const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, true);
      s0 = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2, xw[2 * i]), s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, xw[2 * i + 1]), s1, false);
    }
  }
  return s0 + s1;
}

// Sum of a row's per-wave partials in wave order (deterministic); zeroes them for the next phase.
// Sum of a row's per-wave partials, which are cleared for the next phase.  The zeros
// come from a register quad that lives for the whole kernel (`zero4`, opaque to the
// compiler): zeros materialised afresh would land in registers that some load on
// another path also writes, and the compiler would wait for that load first.
static_assert(kFW % 4 == 0, "partials are cleared four at a time");
__device__ __forceinline__ float row_sum(float* part, int row, const float4& zero4) {
  float y = 0.0f;
#pragma unroll
  for (int w = 0; w < kFW; ++w) y += part[row * kFW + w];
#pragma unroll
  for (int w = 0; w < kFW; w += 4) *reinterpret_cast<float4*>(part + row * kFW + w) = zero4;
  return y;
}

// ---------------------------------------------------------------- phase inputs into LDS (bf16 pairs)
template <int P>
__device__ __forceinline__ uint32_t act_bits(float v, float scale) {
  // value in GEMV units (bf16-rounded value, or the e4m3 code value), as bf16 bits (exact).
  // An e4m3 code value has at most four significant bits, so its bf16 bits are the upper
  // half of its fp32 bits (the clamp in f32_to_e4m3 leaves no NaN); a bf16 value needs
  // one rounding of v (rounding it again changes no bit).  Both without a branch.
  if (P == kFP8) return __float_as_uint(act_round<P>(v, scale)) >> 16;
  return f32_to_bf16_sel(v);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Store the wave-uniform v to the LDS word p from lane 0 only, without a branch on the
// lane index: such a branch is divergent control flow, and the compiler may merge code
// across it in ways that make the (uniform) fetch state look divergent.  The store
// completes before the statement ends.  The compiler does not see the EXEC writes, so
// each is followed by the wait states that a later DPP or lane-select instruction
// needs after an SALU write of EXEC (five).
__device__ __forceinline__ void lane0_lds_store(float* p, float v) {
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_void_t*)p;
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "s_nop 4\n\t"
      "ds_write_b32 %1, %2\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b64 exec, %0\n\t"
      "s_nop 4"
      : "=&s"(saved) : "v"(addr), "v"(v) : "memory");
}

// A block-wide sum and "every thread's poll succeeded" with one barrier: each wave
// leaves its partial sum and its flag in its own slot of `slots` (2 * kFW floats),
// then every wave adds the partials in wave order (the order block_sum uses).  The
// slots are reused phase after phase; the barriers between two uses keep them apart.
__device__ __forceinline__ bool block_sum_ok(float& v, bool ok, float* slots) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  v = wave_sum(v);
  const float wok = __all(ok) ? 1.0f : 0.0f;
  lane0_lds_store(slots + w, v);
  lane0_lds_store(slots + kFW + w, wok);
  __syncthreads();
  float s = 0.0f, all = 1.0f;
#pragma unroll
  for (int i = 0; i < kFW; ++i) {
    s += slots[i];
    all = fminf(all, slots[kFW + i]);
  }
  v = s;
  return __builtin_amdgcn_readfirstlane(__float_as_uint(all)) != 0u;
}

// The compiler counts only its own vector loads, not the ring's LDS fetches; where it
// cannot prove a load of its own has landed it waits for the whole counter, and that
// wait would also wait for every fetch the ring has in flight.  Right after a poll is
// satisfied the counter is all but empty (loads land in issue order, and the poll's
// were the youngest), so an explicit full wait there costs nothing and leaves the
// compiler nothing pending to guard later in the phase.
// (The compiler barriers keep loads from being moved across the wait.)
__device__ __forceinline__ void settle_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  asm volatile("" ::: "memory");
}

// Tagged words are polled in batches: every load of a batch is issued before any
// tag is checked (one memory round trip per attempt), and a thread that still
// misses a word loads all of its words again.  No load sits under a condition (a
// conditional load becomes a basic block of its own with its counter wait inside,
// which would turn a retry into a chain of round trips): a word past `count`
// re-reads the thread's word of the first row (callers ignore its value; the batch
// size is chosen to fit the input, so there are few such words, and they spread
// over many cache lines rather than piling onto one).  A scheduling barrier after
// the batch keeps the compiler from pulling the checks in between the loads.
// The thread index is laundered per call, so that the word offsets are formed at
// the poll (a few VALU ops) instead of being hoisted out of the phase loop and held
// in registers for the whole frame; they are 32-bit offsets from the uniform base.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
template <class T>
__device__ __forceinline__ const T* word_at(const T* base, int i) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + (uint32_t)i * (uint32_t)sizeof(T));
}
template <int N>
__device__ __forceinline__ void load_batch64(const uint64_t* base, int stride, int count, uint64_t (&wv)[N]) {
  const int t = opaque_tid();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int k = i * stride + t;
    wv[i] = ld64(word_at(base, k < count ? k : min(t, count - 1)));
  }
  __builtin_amdgcn_sched_barrier(0);
}
template <int N>
__device__ __forceinline__ bool poll_batch64(const uint64_t* base, int stride, int count, unsigned tag,
                                             uint64_t (&wv)[N], Poll& pl) {
  load_batch64<N>(base, stride, count, wv);
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && ((unsigned)(wv[i] >> 32) == tag);
    if (ok) return true;
    if (!pl.again()) return false;
    load_batch64<N>(base, stride, count, wv);
  }
}
template <int N>
__device__ __forceinline__ void load_batch32(const uint32_t* base, int stride, int count, uint32_t (&wv)[N]) {
  const int t = opaque_tid();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int k = i * stride + t;
    wv[i] = ld32(word_at(base, k < count ? k : min(t, count - 1)));
  }
  __builtin_amdgcn_sched_barrier(0);
}
template <int N>
__device__ __forceinline__ bool poll_batch32(const uint32_t* base, int stride, int count, unsigned tag,
                                             uint32_t (&wv)[N], Poll& pl) {
  const unsigned t16 = tag & 0xffffu;
  load_batch32<N>(base, stride, count, wv);
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && ((wv[i] >> 16) == t16);
    if (ok) return true;
    if (!pl.again()) return false;
    load_batch32<N>(base, stride, count, wv);
  }
}

// xs = act(rmsnorm(h) * g), h polled from the tagged residual; kMaxPer words per thread
template <int P, int kMaxPer>
__device__ __forceinline__ bool norm_to_lds_n(const uint64_t* xh, unsigned tag, const float* g, int K, float eps,
                                              float scale, uint32_t* xs, float* red, unsigned* abort_flag,
                                              uint32_t (&seen)[2], float* rec) {
  Poll pl;
  pl.start(abort_flag);
  // the gains do not depend on the frame: their loads travel with the first poll round
  float gv[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int k = i * kFT + threadIdx.x;
    gv[i] = k < K ? *gp(g + k) : 0.0f;
  }
  issue_fence();
  uint64_t wv[kMaxPer];
  const bool got = poll_batch64<kMaxPer>(xh, kFT, K, tag, wv, pl);
  settle_loads();
  seen[0] = (uint32_t)__builtin_amdgcn_s_memrealtime();
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int k = i * kFT + threadIdx.x;
    const float v = k < K ? __uint_as_float((uint32_t)wv[i]) : 0.0f;
    ss = fmaf(v, v, ss);
  }
  if (!block_sum_ok(ss, got, red)) return false;  // red: 2 * kFW floats
  seen[1] = (uint32_t)__builtin_amdgcn_s_memrealtime();
  const float rstd = 1.0f / sqrtf(ss / (float)K + eps);
  uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
  // every element's value and code first (elements past K are clamped copies with a zero
  // gain, computed and never stored), so that the per-element divisions overlap
  float u[kMaxPer];
  uint32_t code[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    u[i] = __uint_as_float((uint32_t)wv[i]) * rstd * gv[i];
    code[i] = act_bits<P>(u[i], scale);
  }
  float mx = 0.0f;
  if (K == kMaxPer * kFT) {  // uniform: every element lies in the row, no store is predicated
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      xs16[i * kFT + threadIdx.x] = (uint16_t)code[i];
      mx = fmaxf(mx, fabsf(u[i]));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int k = i * kFT + threadIdx.x;
      if (k < K) {
        xs16[k] = (uint16_t)code[i];
        mx = fmaxf(mx, fabsf(u[i]));
      }
    }
  }
  if (rec != nullptr) {  // calibration: the site's maximum before rounding (uniform branch)
    mx = block_max(mx, red);
    if (threadIdx.x == 0) record_amax(rec, mx);
  }
  __syncthreads();
  return true;
}
template <int P>
__device__ __forceinline__ bool norm_to_lds(const uint64_t* xh, unsigned tag, const float* g, int K, float eps,
                                            float scale, uint32_t* xs, float* red, unsigned* abort_flag,
                                            uint32_t (&seen)[2], float* rec) {
  // K <= 10 * kFT; hidden sizes up to 5 * kFT (2560 at 512 threads) take the short batch
  if (K <= 5 * kFT) return norm_to_lds_n<P, 5>(xh, tag, g, K, eps, scale, xs, red, abort_flag, seen, rec);
  return norm_to_lds_n<P, 10>(xh, tag, g, K, eps, scale, xs, red, abort_flag, seen, rec);
}

// xs from a tagged exchange buffer already in GEMV units (bf16 bits); kMaxPer words per thread
template <int kMaxPer>
__device__ __forceinline__ bool act_to_lds_n(const uint32_t* x, unsigned tag, int K, uint32_t* xs,
                                             unsigned* abort_flag, float* slots, uint32_t (&seen)[2]) {
  Poll pl;
  pl.start(abort_flag);
  uint32_t wv[kMaxPer];
  const bool got = poll_batch32<kMaxPer>(x, kFT, K, tag, wv, pl);
  settle_loads();
  seen[0] = (uint32_t)__builtin_amdgcn_s_memrealtime();
  uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int k = i * kFT + threadIdx.x;
    if (k < K) xs16[k] = (uint16_t)(wv[i] & 0xffffu);
  }
  float unused = 0.0f;
  const bool ok = block_sum_ok(unused, got, slots);  // also makes the xs writes visible
  seen[1] = (uint32_t)__builtin_amdgcn_s_memrealtime();
  return ok;
}
__device__ __forceinline__ bool act_to_lds(const uint32_t* x, unsigned tag, int K, uint32_t* xs,
                                           unsigned* abort_flag, float* slots, uint32_t (&seen)[2]) {
  // K <= 20 * kFT; the attention output (Hq * hd = 4096 at 512 threads) takes the short batch
  if (K <= 8 * kFT) return act_to_lds_n<8>(x, tag, K, xs, abort_flag, slots, seen);
  return act_to_lds_n<20>(x, tag, K, xs, abort_flag, slots, seen);
}

// Phase timestamps for profiling the persistent kernel (the constant 100 MHz clock):
// [0] phase start, [1] inputs ready, [2] weights streamed, [3] phase done; for wave 0
// of the block: [4] weight packets consumed and [5] row sums closed in the phase; and
// (clock again) [6] wave 0's polls of the phase input satisfied, [7] every wave's.
// Trace words are written by every lane of wave 0 (the same value to the same word):
// a branch on the wave index is uniform, where one on the thread index would be a
// divergent branch that the compiler may thread through the whole phase loop.
__device__ __forceinline__ void trace_put(CFA& a, int n_phases, int phase, int i, uint32_t v) {
  if (a.trace != nullptr && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0)
    *gpw(a.trace + ((size_t)blockIdx.x * n_phases + phase) * 8 + i) = __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ void trace_mark(CFA& a, int n_phases, int phase, int i) {
  trace_put(a, n_phases, phase, i, (uint32_t)__builtin_amdgcn_s_memrealtime());
}

// ---------------------------------------------------------------- attention task (split-K, one kv head)
struct AttnLds {
  float qs[4][128];                 // the kv group's rotated queries (group <= 4)
  float kn[128], vn[128];           // this frame's key and value
  uint32_t Kt[kAttnTile][65];       // the tile's keys as bf16 pairs (rows padded against bank conflicts)
  uint32_t Vt[kAttnTile][64];       // the tile's values as bf16 pairs
  float ps[4][kAttnTile];
  float half[8][kAttnTile];         // per (wave, key): the even- or odd-dimension half of a score
  float scl[4];                     // per query head: the tile's rescale of the running output
  float ml[4][2];                   // per query head: this split's (max, denominator)
};
// bytes of the region the GEMV input vector (5120 words) and the attention scratch share
constexpr size_t kFrameShared = ((sizeof(AttnLds) > 5120 * 4 + kPartMax * 4 ? sizeof(AttnLds) : 5120 * 4 + kPartMax * 4) + 15) / 16 * 16;
static_assert(kFW * kRD * 1024 + kFrameShared + 1024 <= 160 * 1024, "frame LDS");

// Half of the dot product of query head qh with key `key` of the tile: the even
// dimensions (low halves of the key words) or, ODD, the odd ones, as two FMA chains
// alternating over the key words, added at the end.
template <int HD, bool ODD>
__device__ __forceinline__ float half_dot(const AttnLds& sm, int qh, int key) {
  float d[2] = {0.0f, 0.0f};
  for (int eb = 0; eb < HD / 2; eb += 16) {  // 16 key words and 32 query values per batch
    uint32_t kk[16];
    float q[32];
#pragma unroll
    for (int u = 0; u < 16; ++u) kk[u] = sm.Kt[key][eb + u];
#pragma unroll
    for (int u = 0; u < 32; u += 4) {
      const float4 q4 = *reinterpret_cast<const float4*>(&sm.qs[qh][2 * eb + u]);
      q[u] = q4.x; q[u + 1] = q4.y; q[u + 2] = q4.z; q[u + 3] = q4.w;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      d[u & 1] = ODD ? fmaf(q[2 * u + 1], bf16hi(kk[u]), d[u & 1]) : fmaf(q[2 * u], bf16lo(kk[u]), d[u & 1]);
  }
  return d[0] + d[1];
}

template <int HD>
__device__ __forceinline__ void attn_norm_rope(const uint64_t* src, unsigned tag, const float* g, const float* cs,
                                               const float* sn, float eps, int lane, float* dst, Poll& pl) {
  constexpr int H2 = HD / 2;
  const bool act = lane < H2;
  // frame-independent operands first, so their latency overlaps the poll
  const float g0 = act ? *gp(g + lane) : 0.0f, g1 = act ? *gp(g + lane + H2) : 0.0f;
  const float c = act ? *gp(cs + lane) : 0.0f, s = act ? *gp(sn + lane) : 0.0f;
  issue_fence();
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
    const float a = x0 * rstd * g0;
    const float b = x1 * rstd * g1;
    dst[lane] = round_bf16_sel(a * c - b * s);
    dst[lane + H2] = round_bf16_sel(b * c + a * s);
  }
}

// One block = one (kv head, key split) task.  Split 0 of each kv head merges the
// other active splits' partials (polled by tag) and publishes the attention output.
// Returns false if the frame was abandoned.
template <int P, int HD>
__device__ __forceinline__ bool attn_task(CFA& a, const LayerW L, int layer, int pos, unsigned tag_qkv,
                          unsigned tag_part, unsigned tag_o, AttnLds& sm, unsigned* abort_flag, int* okf) {
  constexpr int H2 = HD / 2;
  constexpr int T = kAttnTile;
  const int G = a.Hq / a.Hkv;
  const int ntask = a.Hkv * a.splits;
  const int task = blockIdx.x;
  if (task >= ntask) return true;
  const int j = task / a.splits, split = task % a.splits;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nkeys = pos + 1;
  int chunk = (nkeys + a.splits - 1) / a.splits;
  chunk = (chunk + T - 1) / T * T;
  const int n_active = (nkeys + chunk - 1) / chunk;
  if (split >= n_active) return true;
  const int beg = split * chunk, end = min(nkeys, beg + chunk);
  const float* cs = launder(a.rope_cos) + (size_t)pos * H2;
  const float* sn = launder(a.rope_sin) + (size_t)pos * H2;
  uint64_t* xqkv = launder(a.xqkv);
  uint64_t* xpart = launder(a.xpart);
  uint32_t* xo = launder(a.xo);
  uint16_t* kc = L.k_cache + (size_t)j * a.max_seq * HD;
  uint16_t* vc = L.v_cache + (size_t)j * a.max_seq * HD;
  // the first key tile comes from earlier positions only (the new key at pos is
  // written below): load it before waiting for this frame's q, k, v
  constexpr int SEG = HD / 8;                       // 16-byte segments per key
  constexpr int NPT = (T * SEG + kFT - 1) / kFT;    // tile segments per thread
  uint4 kr[NPT], vr[NPT];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = u * kFT + tid;
      const int kp = t0 + idx / SEG, seg = idx % SEG;
      if (idx < T * SEG && kp < end && kp != pos) {
        kr[u] = ld16(kc + (size_t)kp * HD + seg * 8);
        vr[u] = ld16(vc + (size_t)kp * HD + seg * 8);
      } else {
        kr[u] = make_uint4(0u, 0u, 0u, 0u);
        vr[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  load_tile(beg);
  issue_fence();
  Poll pl;
  pl.start(abort_flag);
  if (w < G) attn_norm_rope<HD>(xqkv + (size_t)(j * G + w) * HD, tag_qkv, L.g_q, cs, sn, a.eps, lane, sm.qs[w], pl);
  if (w == G) attn_norm_rope<HD>(xqkv + (size_t)a.Hq * HD + (size_t)j * HD, tag_qkv, L.g_k, cs, sn, a.eps, lane, sm.kn, pl);
  if (w == G + 1) {
    const uint64_t* vsrc = xqkv + (size_t)(a.Hq + a.Hkv) * HD + (size_t)j * HD;
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
  if (a.q_tap != nullptr && split == 0 && tid < G * HD)  // taps: this kv group's rotated queries
    *gpw(a.q_tap + (size_t)layer * a.Hq * HD + (size_t)j * G * HD + tid) = (uint16_t)f32_to_bf16(sm.qs[tid / HD][tid % HD]);
  trace_mark(a, 5 * a.n_layers + 1, 5 * layer + 1, 1);
  const float inv_sqrt = 1.0f / sqrtf((float)HD);
  const bool hi = w >= G;             // the odd-dimension / upper-output wave of a query head
  const int qh = hi ? w - G : w;      // its query head within the group
  float m = -INFINITY, lsum = 0.0f, o = 0.0f;  // (m, lsum) live in the lower wave of each head
  for (int t0 = beg; t0 < end; t0 += T) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = u * kFT + tid;
      if (idx >= T * SEG) continue;
      const int key = idx / SEG, seg = idx % SEG;
      const int kp = t0 + key;
      uint32_t kw[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w}, vw[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
      if (kp == pos && kp < end) {
        // the new key/value (bf16-rounded values, so the conversion is exact)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kw[e] = f32_to_bf16(sm.kn[seg * 8 + 2 * e]) | (f32_to_bf16(sm.kn[seg * 8 + 2 * e + 1]) << 16);
          vw[e] = f32_to_bf16(sm.vn[seg * 8 + 2 * e]) | (f32_to_bf16(sm.vn[seg * 8 + 2 * e + 1]) << 16);
        }
      }
      // keys past the split hold zero words (load_tile zeroed them)
#pragma unroll
      for (int e = 0; e < 4; ++e) { sm.Kt[key][seg * 4 + e] = kw[e]; sm.Vt[key][seg * 4 + e] = vw[e]; }
    }
    // the next tile's loads (into the registers just stored) overlap this tile's work
    if (t0 + T < end) load_tile(t0 + T);
    __syncthreads();
    // Every query head is shared by two waves: wave qh takes the even dimensions (the
    // low halves of the key and value words) and wave qh + G the odd ones of the
    // scores, and dimensions 0..63 and 64..127 of the output.  The two FMA chains of
    // each half and their final additions are those of a single wave's dot product,
    // so the scores and outputs are unchanged.
    float mnew = m;
    if (w < 2 * G) {
      const int kp = t0 + lane;
      float part = 0.0f;
      if (kp < end) part = hi ? half_dot<HD, true>(sm, qh, lane) : half_dot<HD, false>(sm, qh, lane);
      sm.half[w][lane] = part;
    }
    __syncthreads();
    if (w < G) {
      const int kp = t0 + lane;
      const float s = (kp < end) ? (sm.half[w][lane] + sm.half[w + G][lane]) * inv_sqrt : -INFINITY;
      mnew = fmaxf(m, wave_max(s));
      const float p = (kp < end) ? __expf(s - mnew) : 0.0f;
      const float scale = __expf(m - mnew);
      lsum = lsum * scale + wave_sum(p);
      sm.ps[w][lane] = p;
      sm.scl[w] = scale;  // every lane writes the same value
    }
    __syncthreads();
    if (w < 2 * G && (HD > 64 || !hi)) {
      // all T keys of the tile (those past the split have p = 0 and zero values), 16 keys
      // per batch: the batch's LDS reads are issued together, then one FMA chain in key
      // order (the order of the one-kernel-per-phase frame)
      const int dd = hi ? lane + 64 : lane;  // this lane's output dimension
      const int dw = dd >> 1;
      const uint32_t dsh = (dd & 1) ? 0u : 16u;  // bf16 half of the value word: (v << dsh) & hi16
      o *= sm.scl[qh];
      for (int kb = 0; kb < T; kb += 16) {
        float pp[16];
        uint32_t v[16];
#pragma unroll
        for (int u = 0; u < 16; u += 4) {
          const float4 p4 = *reinterpret_cast<const float4*>(&sm.ps[qh][kb + u]);
          pp[u] = p4.x; pp[u + 1] = p4.y; pp[u + 2] = p4.z; pp[u + 3] = p4.w;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = sm.Vt[kb + u][dw];
#pragma unroll
        for (int u = 0; u < 16; ++u) o = fmaf(pp[u], __uint_as_float((v[u] << dsh) & 0xffff0000u), o);
      }
    }
    m = mnew;
    __syncthreads();
  }
  // The last tile issues no prefetch, but the compiler cannot tell: it would take the
  // tile registers for in flight and wait for all vector memory (the ring's fetches
  // too) wherever it reuses them.  Nothing is in flight here by now (the ring's last
  // fetches went out before the QKV epilogue), so a full wait costs nothing.
  settle_loads();
  // this frame's key and value into the cache, for the frames to come (this one took
  // them from LDS): stored after the tiles, so that no tile waits for the stores
  if (beg <= pos && pos < end && tid < HD) {
    *gpw(kc + (size_t)pos * HD + tid) = (uint16_t)f32_to_bf16(sm.kn[tid]);
    *gpw(vc + (size_t)pos * HD + tid) = (uint16_t)f32_to_bf16(sm.vn[tid]);
  }
  trace_mark(a, 5 * a.n_layers + 1, 5 * layer + 1, 2);
  const float so = P == kFP8 ? *gp(a.act_scales + kSitesPerLayer * layer + 1) : 1.0f;
  if (split != 0) {
    // publish this split's (o, m, l)
    if (w < 2 * G && (HD > 64 || !hi)) {
      const int h = j * G + qh;
      uint64_t* pp = xpart + ((size_t)h * a.splits + split) * (HD + 2);
      st64(pp + (hi ? lane + 64 : lane), o, tag_part);
      if (!hi && lane == 0) { st64(pp + HD, m, tag_part); st64(pp + HD + 1, lsum, tag_part); }
    }
    return true;
  }
  // the upper wave of each head takes the split's (m, l) from the lower one
  if (w < G) { sm.ml[w][0] = m; sm.ml[w][1] = lsum; }
  __syncthreads();
  if (hi && w < 2 * G) { m = sm.ml[qh][0]; lsum = sm.ml[qh][1]; }
  // split 0: merge with the other active splits (log-sum-exp) and publish the output.
  // The first round loads every split's (m, l) (lane s holds split s's) together with
  // the o vectors of the first kMB other splits, so a merge of up to kMB + 1 splits
  // costs one memory round trip; each word carries its own tag.
  constexpr int kMB = 8;  // o vectors per round
  Poll pm;
  pm.start(abort_flag);
  if (w < 2 * G && (HD > 64 || !hi)) {
    // both waves of a head form the same merge weights; each merges its half of the output
    const int h = j * G + qh;
    const int dd = hi ? lane + 64 : lane;
    const uint64_t* pb = xpart + (size_t)h * a.splits * (HD + 2);
    const uint64_t want = (uint64_t)tag_part << 32;
    const bool other = lane > 0 && lane < n_active;
    uint64_t wm = other ? ld64(pb + (size_t)lane * (HD + 2) + HD) : want;
    uint64_t wl = other ? ld64(pb + (size_t)lane * (HD + 2) + HD + 1) : want;
    float n = 0.0f, f = 0.0f;
    for (int sp0 = 1; sp0 < n_active || sp0 == 1; sp0 += kMB) {
      uint64_t x[kMB];
#pragma unroll
      for (int u = 0; u < kMB; ++u) {
        const int sp = sp0 + u;
        const uint64_t* q = pb + (size_t)(sp < n_active ? sp : 0) * (HD + 2);
        x[u] = sp < n_active ? ld64(q + dd) : want;
      }
      while (pm.ok) {
        bool ok = (unsigned)(wm >> 32) == tag_part && (unsigned)(wl >> 32) == tag_part;
#pragma unroll
        for (int u = 0; u < kMB; ++u) ok = ok && (unsigned)(x[u] >> 32) == tag_part;
        if (ok || !pm.again()) break;
        if ((unsigned)(wm >> 32) != tag_part) wm = ld64(pb + (size_t)lane * (HD + 2) + HD);
        if ((unsigned)(wl >> 32) != tag_part) wl = ld64(pb + (size_t)lane * (HD + 2) + HD + 1);
#pragma unroll
        for (int u = 0; u < kMB; ++u) {
          const uint64_t* q = pb + (size_t)(sp0 + u) * (HD + 2);
          if ((unsigned)(x[u] >> 32) != tag_part) x[u] = ld64(q + dd);
        }
      }
      if (!pm.ok) break;
      if (sp0 == 1) {  // the merge weights, once every (m, l) is in
        const float ms = other ? __uint_as_float((uint32_t)wm) : (lane == 0 ? m : -INFINITY);
        const float ls = other ? __uint_as_float((uint32_t)wl) : (lane == 0 ? lsum : 0.0f);
        const float M = wave_max(ls > 0.0f ? ms : -INFINITY);
        f = (ls > 0.0f) ? __expf(ms - M) : 0.0f;
        lsum = wave_sum(f * ls);  // the merged denominator
        n = __shfl(f, 0, kWave) * o;
      }
#pragma unroll
      for (int u = 0; u < kMB; ++u) {
        const int sp = sp0 + u;
        const float fs = __shfl(f, sp < n_active ? sp : 0, kWave);
        if (sp < n_active) n = fmaf(fs, __uint_as_float((uint32_t)x[u]), n);
      }
    }
    const float inv = 1.0f / lsum;
    st32(xo + (size_t)h * HD + dd, act_bits<P>(n * inv, so), tag_o);
    if (a.amax != nullptr) {  // calibration: the attention-output site's maximum before rounding
      const float mx = wave_max(fabsf(n * inv));
      if (lane == 0) record_amax(a.amax + kSitesPerLayer * layer + 1, mx);
    }
  }
  return block_ok(pm.ok, okf);
}

// ---------------------------------------------------------------- the frame
// The frame is a sequence of phases: per layer QKV, ATTN, O, GU, DOWN, then
// HEAD.  GEMV phases share one code path (prologue / packet stream / epilogue
// chosen by the phase kind), so the streaming loop exists once in the binary.
enum PhaseKind { kQKV = 0, kATTN = 1, kO = 2, kGU = 3, kDOWN = 4, kHEAD = 5 };

template <int P, int HD>
__device__ __forceinline__ Stream<P> phase_stream(CFA& a, const int* split, int phase) {
  const int layer = phase / 5, kind = phase % 5;
  const int d = a.d, qd = a.Hq * HD;
  if (layer >= a.n_layers) return make_stream<P>(split, a.w_head, d, kHEAD);
  // arithmetic on the argument block only (no dependent load on the issue path)
  const unsigned char* lb = a.wl0 + (size_t)layer * a.lstride;
  switch (kind) {
    case kQKV: return make_stream<P>(split, lb + a.off_wqkv, d, kQKV);
    case kO: return make_stream<P>(split, lb + a.off_wo, qd, kO);
    case kGU: return make_stream<P>(split, lb + a.off_wgu, d, kGU);
    default: return make_stream<P>(split, lb + a.off_wd, a.F, kDOWN);
  }
}

// ---------------------------------------------------------------- weight stream through an LDS ring
// Every wave owns kRD ring slots of 1 KB in LDS.  Its weight packets (its run
// of each GEMV phase, phase after phase through the whole frame) are fetched
// with global_load_lds_dwordx4 straight into the slots, kRD packets ahead of
// consumption, so the fetch runs on across phase boundaries, through the waits
// for the next phase's inputs and through attention, without holding any
// registers.  Loads complete in issue order, so "packet k has landed" is
// "at most issued - k - 1 younger loads are outstanding" (s_waitcnt vmcnt).
typedef const __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ int next_gemv_phase(int phase, int n_layers) {
  int p = phase + 1;
  if (p / 5 < n_layers && p % 5 == kATTN) ++p;
  return p;
}

template <int P>
struct Issuer {
  const uint8_t* next;  // first byte of the next packet to fetch (uniform)
  int left;             // packets of the current piece still to fetch
  int tail;             // bytes of the current piece's last packet (16 .. 1024)
  int phase;            // phase of the current piece; n_phases once all are issued
  int slot;             // ring slot of the next fetch
  uint32_t m0base;      // LDS byte address of this wave's ring
  const int* split;     // the block's rows per GEMV kind (LDS)
};

template <int P>
__device__ __forceinline__ void issuer_piece(Issuer<P>& is, const Piece& q) {
  is.next = q.base + q.b0;
  is.left = q.npk;
  is.tail = q.b1 - q.b0 - (q.npk - 1) * 1024;
}

// Fetch the wave's next packet into the next ring slot.  Exactly one fetch per call:
// once every packet of the frame is issued, the last one is fetched again, so that
// kRD fetches are always in flight and the ring's waits are constant.
template <int P, int HD>
__device__ __forceinline__ void issue_one(CFA& a, Issuer<P>& is, int n_phases) {
  while (is.left == 0 && is.phase < n_phases) {
    is.phase = next_gemv_phase(is.phase, a.n_layers);
    if (is.phase < n_phases) issuer_piece(is, make_piece<P>(phase_stream<P, HD>(a, is.split, is.phase)));
  }
  const int lane16 = 16 * (int)(threadIdx.x & 63);
  const bool real = is.left > 0;
  const uint8_t* src = real ? is.next : is.next - 1024;
  // lanes past the piece's end (its last packet only), and every lane of a repeated
  // fetch, read the packet's first 16 bytes
  const int voff = (!real || (is.left == 1 && lane16 >= is.tail)) ? 0 : lane16;
  // Written as inline assembly so that the compiler does not see an LDS write it
  // cannot attribute to a slot (it would wait for every fetch in flight before each
  // ring read); the ring's waits are the explicit ones in run_stream.  The packet's
  // address is scalar (lane offsets in a VGPR); M0 holds the slot's LDS byte
  // address, and each lane's 16 bytes land at M0 + 16 * lane.  The weights are read
  // once per frame: the non-temporal hint (nt) streams them past the caches, which
  // measured 7.0 TB/s against 6.1 TB/s without it for a plain read of 4 GB.
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(is.m0base + (uint32_t)is.slot * 1024u);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               : : "v"(voff), "s"(src), "s"(m0) : "memory", "m0");
  if (real) {
    is.next += 1024;
    --is.left;
  }
  is.slot = is.slot + 1 == kRD ? 0 : is.slot + 1;
}

template <int P, int HD>
__device__ __forceinline__ void issuer_begin(CFA& a, Issuer<P>& is, unsigned char* ring_w, const int* split,
                                             int n_phases) {
  is.split = split;
  is.m0base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)ring_w);
  is.phase = 0;
  is.slot = 0;
  issuer_piece(is, make_piece<P>(phase_stream<P, HD>(a, split, 0)));
  for (int i = 0; i < kRD; ++i) issue_one<P, HD>(a, is, n_phases);
}

// Wait until every fetch into the ring has landed (before the block leaves the kernel).
__device__ __forceinline__ void ring_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Fetch the wave's next two packets (one issue_one each, with a shorter path where
// neither ends a piece).
template <int P, int HD>
__device__ __forceinline__ void issue_two(CFA& a, Issuer<P>& is, int n_phases) {
  if (is.left >= 3) {
    const int lane16 = 16 * (int)(threadIdx.x & 63);
    const int s2 = is.slot + 1 == kRD ? 0 : is.slot + 1;
    const uint32_t m0a = __builtin_amdgcn_readfirstlane(is.m0base + (uint32_t)is.slot * 1024u);
    const uint32_t m0b = __builtin_amdgcn_readfirstlane(is.m0base + (uint32_t)s2 * 1024u);
    // (two scalar addresses: an instruction offset would move the LDS destination too)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 : : "v"(lane16), "s"(is.next), "s"(m0a) : "memory", "m0");
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 : : "v"(lane16), "s"(is.next + 1024), "s"(m0b) : "memory", "m0");
    is.next += 2048;
    is.left -= 2;
    is.slot = s2 + 1 == kRD ? 0 : s2 + 1;
  } else {
    issue_one<P, HD>(a, is, n_phases);
    issue_one<P, HD>(a, is, n_phases);
  }
}

// Ring waits.  kRD fetches are in flight whenever a step of the stream begins (every
// consumed packet is replaced by one fetch) and loads land in issue order, so the
// oldest n have landed once at most kRD - n younger ones remain outstanding.  Other
// vector memory operations issued since only make a wait longer.
__device__ __forceinline__ void wait_oldest1() { asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kRD - 1) : "memory"); }
__device__ __forceinline__ void wait_oldest2() { asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kRD - 2) : "memory"); }
static_assert(kRD >= 3 && kRD <= 63, "the ring's waits are s_waitcnt vmcnt immediates");

// Position of the byte `off + lane16` of a packet, counted from the start of the row
// it falls in, where `off` (< rb) is the packet's first byte within the open row.
// LONG: rows of at least 1 KB, so at most one row boundary per packet.
template <bool LONG>
__device__ __forceinline__ int byte_in_row(int off, int lane16, int rb) {
  int p = off + lane16;
  if (LONG) return p >= rb ? p - rb : p;
  while (p >= rb) p -= rb;
  return p;
}
template <bool LONG>
__device__ __forceinline__ int next_off(int off, int rb) {
  int o = off + 1024;
  if (LONG) return o >= rb ? o - rb : o;
  while (o >= rb) o -= rb;
  return o;
}

// One packet in registers: 16 weight bytes per lane and their activations.
struct PacketRegs {
  uint4 w, x0, x1;
};

template <int P>
__device__ __forceinline__ void load_packet(PacketRegs& r, const unsigned char* ring_w, int slot, int lane16,
                                            const uint32_t* __restrict__ xs, int p) {
  r.w = *reinterpret_cast<const uint4*>(ring_w + slot * 1024 + lane16);
  const uint32_t* xp = xs + p / Stream<P>::B / 2;
  r.x0 = *reinterpret_cast<const uint4*>(xp);
  if (P == kFP8) r.x1 = *reinterpret_cast<const uint4*>(xp + 4);
}


// Row bookkeeping of one wave's stream: the open row, the current packet's first byte
// in it, and this lane's share of it.
struct RowAcc {
  int row, off;
  float acc;
  uint32_t closes;
};

// Add packet dv (this lane's dot, zero past the piece's end) to the open row; rows that
// end inside the packet are summed over the wave and written to part[row * kFW + w].
template <bool LONG>
__device__ __forceinline__ void add_packet(RowAcc& ra, float dv, int lane, int lane16, int rb, int nrows,
                                           float* __restrict__ part, int w) {
  const int hi = rb - ra.off;  // lanes with lane16 < hi belong to the open row
  if (hi > 1024) {             // the packet lies inside the open row
    ra.acc += dv;
    ra.off += 1024;
    return;
  }
  if (LONG) {  // exactly one row ends inside the packet
    const bool mine = lane16 < hi;
    const float v = wave_sum(ra.acc + (mine ? dv : 0.0f));
    if (ra.row < nrows) lane0_lds_store(part + ra.row * kFW + w, v);
    ra.acc = mine ? 0.0f : dv;
    ++ra.row;
    ++ra.closes;
    ra.off += 1024 - rb;
    return;
  }
  int lo = 0, h = hi;
  while (h <= 1024) {
    const float v = wave_sum(ra.acc + (lane16 >= lo && lane16 < h ? dv : 0.0f));
    if (ra.row < nrows) lane0_lds_store(part + ra.row * kFW + w, v);
    ra.acc = 0.0f;
    ++ra.row;
    ++ra.closes;
    lo = h;
    h += rb;
  }
  ra.acc = lane16 >= lo ? dv : 0.0f;
  ra.off = 1024 - lo;
}

// Consume this wave's piece q from the ring, two packets per step, refilling each
// consumed slot with the wave's next packet.  The open row and the packet's offset in
// it are uniform: a lane's 16 bytes lie in the open row or, where a row ends inside
// the packet, in a later one.  A row's partial sum is written to part[row * kFW +
// wave] when the row ends (rows local to the block; the caller zeroes part
// beforehand).  `cslot` is the ring slot of the next packet.
template <int P, int HD, bool LONG>
__device__ __forceinline__ void stream_piece(CFA& a, const Piece& q, int nrows, Issuer<P>& is, int& cslot,
                                             const unsigned char* ring_w, const uint32_t* __restrict__ xs,
                                             float* __restrict__ part, int n_phases, uint32_t& closes) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane16 = 16 * lane;
  const int rb = q.rowbytes;
  const int last_bytes = q.b1 - q.b0 - (q.npk - 1) * 1024;
  RowAcc ra;
  ra.row = q.b0 / rb;
  ra.off = q.b0 - ra.row * rb;
  ra.acc = 0.0f;
  ra.closes = 0;
  // Every load the compiler knows of has landed here (the prologue's polls are younger
  // than the ring's fetches, so the ring has landed too).  Saying so with a wait it can
  // see keeps it from waiting for vector memory inside the loop.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
  int i = 0;
  for (; i + 2 <= q.npk; i += 2) {
    wait_oldest2();
    const int s1 = cslot + 1 == kRD ? 0 : cslot + 1;
    const int off1 = next_off<LONG>(ra.off, rb);
    PacketRegs A, B;
    load_packet<P>(A, ring_w, cslot, lane16, xs, byte_in_row<LONG>(ra.off, lane16, rb));
    load_packet<P>(B, ring_w, s1, lane16, xs, byte_in_row<LONG>(off1, lane16, rb));
    const float d0 = packet_dot<P>(A.w, A.x0, A.x1);
    float d1 = packet_dot<P>(B.w, B.x0, B.x1);
    if (i + 2 == q.npk && lane16 >= last_bytes) d1 = 0.0f;  // past the piece's end
    add_packet<LONG>(ra, d0, lane, lane16, rb, nrows, part, w);
    add_packet<LONG>(ra, d1, lane, lane16, rb, nrows, part, w);
    cslot = s1 + 1 == kRD ? 0 : s1 + 1;
    issue_two<P, HD>(a, is, n_phases);
  }
  if (i < q.npk) {  // odd count: the piece's last packet
    wait_oldest1();
    PacketRegs A;
    load_packet<P>(A, ring_w, cslot, lane16, xs, byte_in_row<LONG>(ra.off, lane16, rb));
    float d0 = packet_dot<P>(A.w, A.x0, A.x1);
    if (lane16 >= last_bytes) d0 = 0.0f;
    add_packet<LONG>(ra, d0, lane, lane16, rb, nrows, part, w);
    cslot = cslot + 1 == kRD ? 0 : cslot + 1;
    issue_one<P, HD>(a, is, n_phases);
  }
  // the open row's share (zero where the piece ended on a row end)
  if (ra.row < nrows) lane0_lds_store(part + ra.row * kFW + w, wave_sum(ra.acc));
  closes = ra.closes;
}

template <int P, int HD>
__device__ __forceinline__ void run_stream(CFA& a, const Stream<P>& s, Issuer<P>& is, int& cslot,
                                           const unsigned char* ring_w, const uint32_t* __restrict__ xs,
                                           float* __restrict__ part, int n_phases, int phase) {
  const Piece q = make_piece<P>(s);
  if (q.npk > 0) {
    uint32_t closes = 0;
    if (q.rowbytes >= 1024)
      stream_piece<P, HD, true>(a, q, s.nrows, is, cslot, ring_w, xs, part, n_phases, closes);
    else
      stream_piece<P, HD, false>(a, q, s.nrows, is, cslot, ring_w, xs, part, n_phases, closes);
    trace_put(a, n_phases, phase, 4, (uint32_t)q.npk);
    trace_put(a, n_phases, phase, 5, closes);
  }
  __syncthreads();
}

template <int P, int HD>
__global__ __launch_bounds__(kFT) void k_frame(const FrameArgs* ap_generic) {
  CFA* ap = (CFA*)ap_generic;
  CFA& a = *ap;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  unsigned char* ring_w = smem_raw + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kRD * 1024;  // this wave's ring
  unsigned char* lds1 = smem_raw + kFW * kRD * 1024;
  // the attention task's scratch shares its bytes with the GEMV input vector: the QKV
  // stream ends on a barrier before attention starts, and a barrier follows the task
  // before the o_proj input is written
  uint32_t* xs = reinterpret_cast<uint32_t*>(lds1);                          // activations, bf16 pairs (<= 10240)
  AttnLds& sm = *reinterpret_cast<AttnLds*>(lds1);
  float* part = reinterpret_cast<float*>(lds1 + 5120 * 4);                   // per-(row, wave) partials
  __shared__ float red[2 * kFW];  // block reductions; (sum, flag) slots of block_sum_ok
  __shared__ int sh_state[4 + kMaxCodebooks];
  __shared__ int okf;
  __shared__ int split[12];  // this block's rows per GEMV kind
  const int tid = threadIdx.x;
  unsigned* abort_flag = a.sync + 64;
  const unsigned launch = a.sync[0];
  // phase p of the frame tags its outputs with base + 1 + p; the frame input uses base
  const unsigned base = (launch + 1u) * (8u + 8u * (unsigned)a.n_layers);

  if (tid == 0) {
    // its own laundered view of the arguments: a load here that the compiler merged with
    // the same load after the branch would make that value (and the issue path) divergent
    CFA& a = *launder(ap);
    sh_state[0] = a.st->len;
    sh_state[1] = a.st->t;
    int eoc = a.st->eoc;
    if (eoc < 0 && a.st->t > 0 && a.st->prev[0] == a.eos) eoc = a.st->t - 1;
    sh_state[2] = eoc;
    for (int c = 0; c < a.C; ++c) sh_state[4 + c] = a.st->prev[c];
    block_rows((a.Hq + 2 * a.Hkv) * HD, 0, split + 2 * kQKV);
    block_rows(a.d, 0, split + 2 * kO);
    block_rows(2 * a.F, 1, split + 2 * kGU);
    block_rows(a.d, 0, split + 2 * kDOWN);
    block_rows(a.C * a.V, 0, split + 2 * kHEAD);
  }
  __syncthreads();
  const int pos = __builtin_amdgcn_readfirstlane(sh_state[0]);  // uniform (LDS reads are not known to be)
  const int d = a.d;

  const int n_phases = 5 * a.n_layers + 1;
  Issuer<P> is;
  issuer_begin<P, HD>(a, is, ring_w, split, n_phases);
  int cslot = 0;  // ring slot of the next packet to consume
  float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  asm volatile("" : "+v"(zero4.x), "+v"(zero4.y), "+v"(zero4.z), "+v"(zero4.w));
  for (int i = tid; i < kPartMax; i += kFT) part[i] = 0.0f;

  // frame input: h = sum_k E_aud[k][prev_k] (or, for a one-layer step, the given h_in);
  // every block forms the whole vector for the first norm and publishes the rows it owns
  // (the O/DOWN row split of d).  The owned rows (at most one per thread) stay in h_own
  // for the residual updates.
  float h_own = 0.0f;
  {
    const Stream<P> own = make_stream<P>(split, nullptr, 1, kO);
    constexpr int kMaxPer = 10;  // d <= 10 * kFT
    const float* h_in = a.h_in;
    auto input = [&](int k) {
      if (h_in != nullptr) return *gp(h_in + k);
      float v = 0.0f;
#pragma unroll 1
      for (int c = 0; c < a.C; ++c) v += bf16_to_f32(*gp(a.e_aud + ((size_t)c * a.V + sh_state[4 + c]) * d + k));
      return v;
    };
    float hv[kMaxPer];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int k = i * kFT + tid;
      hv[i] = 0.0f;
      if (k < d) {
        const float v = input(k);
        hv[i] = v;
        ss = fmaf(v, v, ss);
      }
    }
    if (tid < own.nrows) {
      const int k = own.r0 + tid;
      const float v = input(k);
      h_own = v;
      st64(a.xh + k, v, base);
      if (a.taps) *gpw(a.taps + k) = v;
    }
    ss = block_sum(ss, red);
    const float rstd = 1.0f / sqrtf(ss / (float)d + a.eps);
    const float sc = P == kFP8 ? act_scale(a, 0) : 1.0f;
    const float* g = layer_ptrs(a, 0)->g_attn;
    uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int k = i * kFT + tid;
      if (k < d) {
        const float u = hv[i] * rstd * *gp(g + k);
        xs16[k] = (uint16_t)act_bits<P>(u, sc);
        mx = fmaxf(mx, fabsf(u));
      }
    }
    if (a.amax != nullptr && blockIdx.x == 0) {  // calibration: layer 0's attention-input site
      mx = block_max(mx, red);
      if (tid == 0) record_amax(a.amax, mx);
    }
    __syncthreads();
  }
  settle_loads();  // nothing of the prologue's is left pending at the phase loop's entry

  unsigned tag_h = base;   // tag of the residual's latest value
  for (int phase = 0; phase < n_phases; ++phase) {
    const int layer = phase / 5;
    const int kind = layer >= a.n_layers ? kHEAD : phase % 5;
    CFA& a = *launder(ap);
    const unsigned tag = base + 1u + (unsigned)phase;
    trace_mark(a, n_phases, phase, 0);
    uint64_t* xh = launder(a.xh);
    if (kind == kATTN) {
      const LayerW L = a.layers[layer];
      // inputs: the QKV phase (tag - 1); partials and output carry this phase's tag.  (A
      // forced-timeout run skews layer 0's input tag, the frame's first polled one: no
      // block writes it.)
      const unsigned tag_in = layer == 0 ? tag - 1u + a.input_tag_skew : tag - 1u;
      if (!attn_task<P, HD>(a, L, layer, pos, tag_in, tag, tag, sm, abort_flag, &okf)) { ring_drain(); return; }
      __syncthreads();  // the task's scratch is the next phase's input vector and partials
      if (tid < kPartMax / 4) reinterpret_cast<float4*>(part)[tid] = zero4;
      trace_mark(a, n_phases, phase, 3);
      continue;
    }
    const int site = kind == kHEAD ? kSitesPerLayer * a.n_layers
                   : kSitesPerLayer * layer + (kind == kQKV ? 0 : kind == kO ? 1 : kind == kGU ? 2 : 3);
    const float sc_in = P == kFP8 ? act_scale(a, site) : 1.0f;
    const Stream<P> cur = phase_stream<P, HD>(a, split, phase);
    // FP8 row scales of this block's rows (at most one row, or one gate/up pair, per
    // thread), loaded before the prologue's poll and settled right after it (below):
    // the poll's own wait has landed everything older by then, whereas a first use
    // in the epilogue would wait for every weight fetch the ring has in flight
    // Every thread loads (threads past the block's rows load row 0's scale, unused):
    // a default value written into the register before a conditional load would
    // make the compiler wait for every load in flight first.
    float ws0 = 1.0f, ws1 = 1.0f;
    if (P == kFP8) {
      const float* wsc = kind == kHEAD ? a.s_head : layer_scales(a, layer, kind == kQKV ? 0 : kind - 1);
      const int n = kind == kGU ? cur.nrows / 2 : cur.nrows;
      const int i = tid < n ? tid : 0;
      const int r = tid < n ? cur.r0 + (kind == kGU ? 2 * i : i) : 0;
      ws0 = *gp(wsc + r);
      ws1 = *gp(wsc + r + (kind == kGU ? 1 : 0));
      issue_fence();
    }
    // ---- prologue: the phase input in LDS
    uint32_t seen[2] = {0u, 0u};
    if (kind == kQKV || kind == kGU || kind == kHEAD) {
      if (!(kind == kQKV && layer == 0)) {
        const float* g = kind == kHEAD ? a.g_final : (kind == kQKV ? layer_ptrs(a, layer)->g_attn : layer_ptrs(a, layer)->g_mlp);
        float* rec = (a.amax != nullptr && blockIdx.x == 0) ? a.amax + site : nullptr;
        if (!norm_to_lds<P>(xh, tag_h, g, d, a.eps, sc_in, xs, red, abort_flag, seen, rec)) { ring_drain(); return; }
      } else {
        settle_loads();  // layer 0's input was formed in the frame prologue: nothing is in flight
      }
    } else {
      // O reads the attention output (phase tag - 1), DOWN the SiLU*mul output (tag - 1)
      const uint32_t* src = kind == kO ? launder(a.xo) : launder(a.xa);
      const int K = kind == kO ? a.Hq * HD : a.F;
      if (!act_to_lds(src, tag - 1u, K, xs, abort_flag, red, seen)) { ring_drain(); return; }
    }
    if (P == kFP8) asm volatile("" : "+v"(ws0), "+v"(ws1));  // the scale loads land here
    if (a.acts != nullptr && blockIdx.x == 0) {  // taps: this phase's GEMV input vector
      const int K = kind == kO ? a.Hq * HD : (kind == kDOWN ? a.F : d);
      const uint16_t* xs16 = reinterpret_cast<const uint16_t*>(xs);
      for (int k = tid; k < K; k += kFT) *gpw(a.acts + (size_t)phase * kActsWidth + k) = xs16[k];
    }
    trace_mark(a, n_phases, phase, 1);
    trace_put(a, n_phases, phase, 6, seen[0]);
    trace_put(a, n_phases, phase, 7, seen[1]);
    // ---- stream the weights from the ring (its fetches run ahead into the next phases)
    run_stream<P, HD>(a, cur, is, cslot, ring_w, xs, part, n_phases, phase);
    trace_mark(a, n_phases, phase, 2);
    // ---- epilogue (rows per block <= 128 < kFT, so one row or pair per thread)
    if (kind == kGU) {
      const float sc_out = P == kFP8 ? act_scale(a, site + 1) : 1.0f;
      float mx = 0.0f;
      if (tid < cur.nrows / 2) {
        const int row = cur.r0 + 2 * tid;
        const float g = row_sum(part, 2 * tid, zero4) * (P == kFP8 ? sc_in * ws0 : 1.0f);
        const float u = row_sum(part, 2 * tid + 1, zero4) * (P == kFP8 ? sc_in * ws1 : 1.0f);
        const float v = silu(g) * u;
        st32(launder(a.xa) + row / 2, act_bits<P>(v, sc_out), tag);
        mx = fabsf(v);
      }
      if (a.amax != nullptr) {  // calibration: the down-input site's maximum before rounding
        mx = wave_max(mx);
        if ((tid & 63) == 0) record_amax(a.amax + site + 1, mx);
      }
    } else {
      if (tid < cur.nrows) {
        const int row = cur.r0 + tid;
        const float y = row_sum(part, tid, zero4) * (P == kFP8 ? sc_in * ws0 : 1.0f);
        if (kind == kQKV) {
          st64(launder(a.xqkv) + row, y, tag);
        } else if (kind == kHEAD) {
          st64(launder(a.xlogits) + row, y, tag);
        } else {
          // O / DOWN: residual update of this block's own rows (the same rows as the frame input's)
          const float hn = h_own + y;
          h_own = hn;
          st64(xh + row, hn, tag);
          if (kind == kDOWN && layer + 1 == a.n_layers) *gpw(a.h_out + row) = hn;
          if (kind == kDOWN && a.taps) *gpw(a.taps + (size_t)(layer + 1) * d + row) = hn;
        }
      }
      if (kind == kO || kind == kDOWN) tag_h = tag;
    }
    trace_mark(a, n_phases, phase, 3);
  }
  ring_drain();  // every packet was consumed by the head phase; nothing is left in flight
  const unsigned tag_logits = base + (unsigned)n_phases;
  if (blockIdx.x != 0) return;
  // every wave of the block has drained its ring: a sampling run keeps the logits there
  __syncthreads();
  const bool sampling = a.temperature > 0.0f;
  float* lgs = reinterpret_cast<float*>(smem_raw);  // [C][V] logits (sampling)

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
    while (pl.ok) {  // a lane that still misses a logit reloads all of its logits
      bool ok = true;
#pragma unroll
      for (int q = 0; q < kVPL; ++q) ok = ok && (unsigned)(lw[q] >> 32) == tag_logits;
      if (ok || !pl.again()) break;
#pragma unroll
      for (int q = 0; q < kVPL; ++q) {
        const int i = half * kVPL * kWave + q * kWave + lane;
        const uint64_t v = ld64(lg + (i < a.V ? q * kWave + lane : 0));
        lw[q] = i < a.V ? v : want;
      }
    }
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kVPL; ++q) {
      const int i = half * kVPL * kWave + q * kWave + lane;
      if (i < a.V) {
        const float v = __uint_as_float((uint32_t)lw[q]);
        *gpw(a.logits_out + (size_t)k * a.V + i) = v;
        if (sampling) lgs[(size_t)k * a.V + i] = v;
        const bool allowed = (i < a.bos) || (k == 0 && i == a.eos);
        // a NaN logit never wins: with every allowed logit NaN the lowest allowed id is
        // chosen, so the code stays a valid embedding row
        const float x = v == v ? v : -INFINITY;
        if (allowed && (x > bv || (x == bv && i < bi))) { bv = x; bi = i; }
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
  if (sampling) {  // the draw replaces the argmax (block_ok's barriers ordered the LDS logits)
    const int t = sh_state[1];
    for (int k = wv; k < a.C; k += kFW) {
      const float u = philox_uniform(a.seed_lo, a.seed_hi, (uint32_t)t, (uint32_t)k);
      const int id = sample_codebook(lgs + (size_t)k * a.V, a.V, k, a.bos, a.eos, a.temperature, u);
      if (lane == 0) sh_arg[k] = id;
    }
    __syncthreads();
  }
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
size_t frame_lds_bytes() { return (size_t)kFW * kRD * 1024 + kFrameShared; }

// The kernel reads its arguments from device memory (fields are re-read where
// they are used instead of pinning dozens of scalar registers for the whole
// frame); they are written when the workspace is bound and when an option that
// changes them is set, never while a frame runs.
hipError_t frame_write_args(Ctx& c) {
  static_assert(sizeof(FrameArgs) <= kFrameArgsBytes, "FrameArgs does not fit its workspace slot");
  if (!c.frame_ok || !c.fargs) return hipSuccess;
  const hta_config& f = c.cfg;
  FrameArgs a{};
  a.d = f.hidden; a.hd = f.head_dim; a.Hq = f.n_q_heads; a.Hkv = f.n_kv_heads; a.F = f.ffn;
  a.C = f.n_codebooks; a.V = f.codebook_size; a.bos = f.bos_id; a.eos = f.eos_id; a.n_layers = f.n_layers;
  a.max_seq = f.max_seq; a.eps = f.rms_eps;
  a.layers = c.d_layers;
  a.wl0 = reinterpret_cast<const unsigned char*>(c.ws + c.lay.layer_base);
  a.lstride = c.lay.layer_stride;
  a.off_wqkv = c.lay.off_wqkv; a.off_wo = c.lay.off_wo; a.off_wgu = c.lay.off_wgu; a.off_wd = c.lay.off_wd;
  a.e_aud = c.e_aud; a.g_final = c.g_final; a.w_head = c.w_head; a.s_head = c.s_head;
  a.rope_cos = c.rope_cos; a.rope_sin = c.rope_sin; a.act_scales = c.act_scales;
  a.xh = c.x_h; a.xqkv = c.x_qkv; a.xo = c.x_o; a.xa = c.x_a; a.xpart = c.x_part; a.xlogits = c.x_logits;
  a.h_out = c.h; a.logits_out = c.logits;
  a.taps = c.taps ? c.taps_h : nullptr;
  a.acts = c.taps ? c.taps_act : nullptr;
  a.q_tap = c.taps ? c.taps_q : nullptr;
  a.h_in = c.frame_h_in;
  a.amax = c.frame_record ? c.amax : nullptr;
  a.trace = c.trace ? c.trace_buf : nullptr;
  a.sync = c.sync; a.st = c.state; a.hist = c.hist;
  a.splits = c.frame_splits;
  a.temperature = c.temperature;
  a.input_tag_skew = c.force_timeout ? 0x40000000u : 0u;
  a.seed_lo = (uint32_t)c.seed;
  a.seed_hi = (uint32_t)(c.seed >> 32);
  hipError_t e = hipStreamSynchronize(c.stream);
  if (e != hipSuccess) return e;
  if ((e = hipMemcpy(c.fargs, &a, sizeof(a), hipMemcpyHostToDevice)) != hipSuccess) return e;
  if (!c.scratch_dev || !c.fargs_s) return hipSuccess;
  // the same arguments with the exchange words in the static per-device array
  Exchange x;
  exchange_layout(f, c.frame_splits, c.scratch_dev, &x);
  a.xh = x.xh; a.xqkv = x.xqkv; a.xo = x.xo; a.xa = x.xa; a.xpart = x.xpart; a.xlogits = x.xlogits;
  a.sync = x.sync;
  return hipMemcpy(c.fargs_s, &a, sizeof(a), hipMemcpyHostToDevice);
}

hipError_t launch_frame_persistent(Ctx& c) { return launch_frame_args(c, c.fargs); }

hipError_t launch_frame_args(Ctx& c, void* fargs) {
  const hta_config& f = c.cfg;
  const size_t lds = frame_lds_bytes();
  void* ap = fargs;
  void* args[] = {&ap};
  void* fn;
  if (f.precision == HTA_FP8_E4M3) fn = f.head_dim == 128 ? (void*)k_frame<kFP8, 128> : (void*)k_frame<kFP8, 64>;
  else fn = f.head_dim == 128 ? (void*)k_frame<kBF16, 128> : (void*)k_frame<kBF16, 64>;
  time_begin(c, HTA_K_FRAME);
  // One block per CU, each CU able to hold one (checked at set-up), and nothing else on
  // the stream: the blocks are all resident.  An ordinary launch: a cooperative one,
  // which would guarantee it, adds about 20 us per frame; should a block ever not be
  // placed, the bounded waits end the frame with HTA_E_TIMEOUT instead of a hang.
  hipError_t e = hipLaunchKernel(fn, dim3(c.frame_blocks), dim3(kFT), args, lds, c.stream);
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
  c.frame_blocks = cus < kTraceBlocks ? cus : kTraceBlocks;  // one block per CU
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
size_t frame_sample_capacity() { return (size_t)kFW * kRD * 1024; }

}  // namespace hta
