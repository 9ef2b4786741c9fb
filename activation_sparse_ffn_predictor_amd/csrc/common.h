// Shared device helpers and launch declarations of libsffn (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

#include <mutex>

namespace sffn {

constexpr int WAVE = 64;
constexpr float NORM_EPS = 1e-6f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float8v __attribute__((ext_vector_type(8)));

// v from another lane of the same 16-lane row, by a DPP control (VALU latency, no LDS crossbar): 0xB1 swaps lane
// pairs, 0x4E swaps pairs of pairs, 0x141 mirrors each half row (lane i <- 7 - i), 0x140 mirrors the row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// sum over each aligned 16-lane row; every lane of the row gets it
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

// sum over the wave; every lane gets it (row sums by DPP, then the four rows read as scalars)
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// max over the wave; every lane gets it (as wave_sum)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// sum over aligned groups of G lanes (G a power of two <= 64); every lane of the group gets the sum
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if (G >= 2) v += dpp_f<0xB1>(v);
  if (G >= 4) v += dpp_f<0x4E>(v);
  if (G >= 8) v += dpp_f<0x141>(v);
  if (G >= 16) v += dpp_f<0x140>(v);
  if (G >= 32) v += __shfl_xor(v, 16, WAVE);
  if (G >= 64) v += __shfl_xor(v, 32, WAVE);
  return v;
}

// Buffer loads (MUBUF, raw): one resource descriptor per tensor in scalar registers, a 32-bit byte offset per
// lane. A lane whose offset is at or past the tensor's byte size reads zeros (hardware range check), so guarded
// loads need neither branches nor selects and every load of a lane can be in flight at once. Tensors must be
// smaller than 2 GiB; OOB is the offset used for lanes with nothing to load.
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
constexpr uint32_t OOB = 0x80000000u;
struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Buf(const void* p, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000)) {}
  __device__ __forceinline__ uint4 ld16(uint32_t off) const {
    const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ __forceinline__ float4 ldf4(uint32_t off) const {
    const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
  __device__ __forceinline__ uint2 ld8(uint32_t off) const {
    const v2u32 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v.x, v.y);
  }
  __device__ __forceinline__ uint64_t ldu64(uint32_t off) const {
    const v2u32 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return (uint64_t)v.x | ((uint64_t)v.y << 32);
  }
  __device__ __forceinline__ float ldf(uint32_t off) const {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  }
  __device__ __forceinline__ uint32_t ldu(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
  }
  __device__ __forceinline__ _Float16 ldh16(uint32_t off) const {  // one fp16 value
    return __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
  }
  __device__ __forceinline__ uint32_t ldu16(uint32_t off) const {  // one 16-bit value, zero-extended
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  }
  __device__ __forceinline__ float ldh(uint32_t off) const {  // one fp16 value, widened
    const unsigned short b = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    return (float)__builtin_bit_cast(_Float16, b);
  }
};
__device__ __forceinline__ uint32_t boff(bool ok, uint32_t off) { return ok ? off : OOB; }

__device__ __forceinline__ void f16x8_to_f32(const uint4& u, float* f) {
  half8 h = __builtin_bit_cast(half8, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}

__device__ __forceinline__ float dot8(const uint4& u, const float* x) {
  half8 h = __builtin_bit_cast(half8, u);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf((float)h[i], x[i], s);
  return s;
}

// block-wide inclusive->exclusive scan helper for up to 1024 threads (values in registers)
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_tmp /* NT/64 + 1 ints */, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += t;
  }
  if (lane == 63) lds_tmp[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < NT / 64; ++i) { int c = lds_tmp[i]; lds_tmp[i] = run; run += c; }
    lds_tmp[NT / 64] = run;
  }
  __syncthreads();
  total = lds_tmp[NT / 64];
  return lds_tmp[w] + inc - v;
}

// Staging of x into LDS (fp32, token stride D) for kernels that overlap it with other loads: stage_load issues
// the straight-line global loads into registers (every load before the first use; thread t holds float4
// k * NT + t, k < XPT), stage_store writes them to LDS (the caller synchronises), stage_norm normalises in LDS.
template <int NT, int XPT>
__device__ __forceinline__ void stage_load(const float* __restrict__ x, int n4, float4 (&v)[XPT]) {
  const Buf bx(x, (uint32_t)n4 * 16u);
#pragma unroll
  for (int k = 0; k < XPT; ++k) {
    const int i = k * NT + threadIdx.x;
    v[k] = bx.ldf4(boff(i < n4, (uint32_t)i * 16u));
  }
}
template <int NT, int XPT>
__device__ __forceinline__ void stage_store(float* xs, int n4, const float4 (&v)[XPT]) {
  float4* dst = reinterpret_cast<float4*>(xs);
#pragma unroll
  for (int k = 0; k < XPT; ++k) {
    const int i = k * NT + threadIdx.x;
    if (i < n4) dst[i] = v[k];
  }
}
// Normalise one token (B == 1) whose D values are spread over the block's registers before they are stored:
// thread t holds float4 k*NT + t (k < XPT, valid iff < n4). Single pass with a shift (x - x0, x0 = x[0]) for
// the sums, one block reduction (wave sums, then NT/64 partials in wave order). red: 2 * NT/64 floats.
template <int NT, int XPT>
__device__ __forceinline__ void block_norm_regs(float4 (&v)[XPT], int n4, float x0, float* red) {
  constexpr int NWB = NT / 64;
  float s = 0.f, q = 0.f;
#pragma unroll
  for (int k = 0; k < XPT; ++k) {
    if (k * NT + (int)threadIdx.x < n4) {
      const float a = v[k].x - x0, b = v[k].y - x0, c = v[k].z - x0, d = v[k].w - x0;
      s += (a + b) + (c + d);
      q = fmaf(a, a, q); q = fmaf(b, b, q); q = fmaf(c, c, q); q = fmaf(d, d, q);
    }
  }
  s = wave_sum(s);
  q = wave_sum(q);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[w] = s; red[NWB + w] = q; }
  __syncthreads();
  float ts = 0.f, tq = 0.f;
#pragma unroll
  for (int i = 0; i < NWB; ++i) { ts += red[i]; tq += red[NWB + i]; }
  const float n = (float)(n4 * 4);
  const float m = ts / n;                         // mean of x - x0
  const float var = fmaxf(tq / n - m * m, 0.f);
  const float mu = x0 + m;
  const float sc = 1.0f / sqrtf(var + NORM_EPS);
#pragma unroll
  for (int k = 0; k < XPT; ++k) {
    v[k].x = (v[k].x - mu) * sc; v[k].y = (v[k].y - mu) * sc;
    v[k].z = (v[k].z - mu) * sc; v[k].w = (v[k].w - mu) * sc;
  }
}

// Normalise nb tokens of length D held in LDS (centre, unit variance); red: 2 * (NT/64) * nb floats. Starts and
// ends with a block barrier.
template <int NT>
__device__ __forceinline__ void stage_norm(float* xs, int nb, int D, float* red) {
  constexpr int NWB = NT / 64;
  const int w = threadIdx.x >> 6;
  float* rs_ = red;
  float* rq_ = red + NWB * nb;
  __syncthreads();
  for (int b = 0; b < nb; ++b) {
    float s = 0.f;
    for (int i = threadIdx.x; i < D; i += NT) s += xs[(size_t)b * D + i];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) rs_[w * nb + b] = s;
  }
  __syncthreads();
  for (int b = 0; b < nb; ++b) {
    float tot = 0.f;
    for (int i = 0; i < NWB; ++i) tot += rs_[i * nb + b];
    const float mu = tot / (float)D;
    float q = 0.f;
    for (int i = threadIdx.x; i < D; i += NT) { const float d = xs[(size_t)b * D + i] - mu; q = fmaf(d, d, q); }
    q = wave_sum(q);
    if ((threadIdx.x & 63) == 0) rq_[w * nb + b] = q;
  }
  __syncthreads();
  for (int b = 0; b < nb; ++b) {
    float tot = 0.f, totq = 0.f;
    for (int i = 0; i < NWB; ++i) { tot += rs_[i * nb + b]; totq += rq_[i * nb + b]; }
    const float mu = tot / (float)D;
    const float sc = 1.0f / sqrtf(totq / (float)D + NORM_EPS);
    for (int i = threadIdx.x; i < D; i += NT) xs[(size_t)b * D + i] = (xs[(size_t)b * D + i] - mu) * sc;
  }
  __syncthreads();
}

// Workgroup barrier for LDS data only: waits for this wave's LDS accesses, not for its outstanding global loads
// (those stay in flight across the barrier). The empty asm keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maximum (no wait)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup i runs on XCD i % 8) and every XCD has its own
// L2. For a grid of G = 8 * per workgroups, xcd_slice maps workgroup i to slice (i % 8) * per + i / 8, so
// neighbouring slices -- which share cache lines when a slice is narrower than a line -- run on one XCD and
// share its L2 instead of fetching the same lines once per XCD.
__device__ __forceinline__ int xcd_slice(int i, int G) {
  return (i & 7) * (G >> 3) + (i >> 3);
}

// Mask word t with the bits of neurons >= F cleared (callers may pass any bit pattern there).
__device__ __forceinline__ uint64_t mask_word(const uint64_t* __restrict__ mask, int t, int nw, int F) {
  uint64_t w = mask[t];
  if (t == nw - 1 && (F & 63)) w &= (1ull << (F & 63)) - 1ull;
  return w;
}

// Position of the k-th set bit (0-based, k < popcount) of a 64-bit word, by halving.
__device__ __forceinline__ int select_bit(uint64_t w, int k) {
  int pos = 0;
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const uint64_t lowmask = (h == 64) ? ~0ull : ((1ull << h) - 1ull);
    const int c = __popcll(w & lowmask);
    if (k >= c) { k -= c; w >>= h; pos += h; }
  }
  return pos;
}

// The ids of the rows a block owns when dense index i goes to block i % G (G >= 64): bids[k] = the neuron with
// dense index blk + G * k. Thread t owns mask word t (one word per thread: nw <= blockDim.x) and roff[t] = set
// bits before it; owned indices are G >= 64 apart, so a word holds at most one, found by a rank select. The
// caller synchronises before reading bids.
__device__ __forceinline__ void block_row_ids(const uint64_t* wl, const int* roff, int nw, int blk, int G, int* bids) {
  const int t = threadIdx.x;
  if (t < nw) {
    const uint64_t word = wl[t];
    const int base = roff[t];
    int k = (blk - base) % G;                          // rank in the word of the first owned index >= base
    if (k < 0) k += G;
    if (k < __popcll(word)) bids[(base + k - blk) / G] = 64 * t + select_bit(word, k);
  }
}

// Locate the i-th set bit (0-based, dense index i < total) of the mask. words: the mask words, in LDS or
// global memory (bits above F are ignored). roff[T] = exclusive prefix of set bits over thread ranges of wpt words
// each. Wave-uniform result: the stored neuron id.
__device__ __forceinline__ int locate(const uint64_t* words, const int* roff, int nranges, int wpt, int nw, int F,
                                      int i) {
  int lo = 0, hi = nranges - 1;  // largest T with roff[T] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (roff[mid] <= i) lo = mid; else hi = mid - 1;
  }
  int rem = i - roff[lo];
  int t = lo * wpt;
  uint64_t word = 0;
  for (; t < nw; ++t) {
    word = words[t];
    if (t == nw - 1 && (F & 63)) word &= (1ull << (F & 63)) - 1ull;
    const int cnt = __popcll(word);
    if (rem < cnt) break;
    rem -= cnt;
  }
  if (t >= nw) return 0;  // unreachable for i < total; keeps every later access in bounds
  const int lane = threadIdx.x & 63;
  const bool bit = (word >> lane) & 1ull;
  const int pre = __popcll(word & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  const unsigned long long sel = __ballot(bit && pre == rem);
  return t * 64 + (__ffsll((long long)sel) - 1);
}

// Per-block prefix over the mask: thread T owns words [T*wpt, T*wpt + wpt); roff[T] = set bits before its range.
// When wl != nullptr (nw <= NT * WMAX) the words, cleared above F, are also copied to LDS (wl[0..nw)) for locate.
// All of a thread's word loads are issued before the first use. Returns the total number of set bits.
template <int NT, int WMAX>
__device__ __forceinline__ int mask_prefix(const uint64_t* __restrict__ mask, int nw, int F, int wpt, uint64_t* wl,
                                           int* roff, int* tmp) {
  const int t0 = threadIdx.x * wpt;
  int cnt = 0;
  if (wpt <= WMAX) {
    const Buf bm(mask, (uint32_t)nw * 8u);
    uint64_t wr[WMAX];
#pragma unroll
    for (int k = 0; k < WMAX; ++k) {
      const int t = t0 + k;
      wr[k] = bm.ldu64(boff(k < wpt && t < nw, (uint32_t)t * 8u));
    }
#pragma unroll
    for (int k = 0; k < WMAX; ++k) {
      const int t = t0 + k;
      if (k < wpt && t < nw) {
        if (t == nw - 1 && (F & 63)) wr[k] &= (1ull << (F & 63)) - 1ull;
        cnt += __popcll(wr[k]);
        if (wl) wl[t] = wr[k];
      }
    }
  } else {
    for (int t = t0; t < min(nw, t0 + wpt); ++t) cnt += __popcll(mask_word(mask, t, nw, F));
  }
  int total;
  const int ex = block_exclusive_scan<NT>(cnt, tmp, total);
  roff[threadIdx.x] = ex;
  __syncthreads();
  return total;
}

}  // namespace sffn

// ---- host helper: allow a kernel all the LDS its static allocation leaves (160 KiB per workgroup on gfx950).
// Returns the dynamic bytes available in *avail.
inline hipError_t allow_dynamic_lds(const void* func, size_t* avail) {
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, func);
  if (e != hipSuccess) return e;
  const size_t total = 160 * 1024;
  *avail = total > fa.sharedSizeBytes ? total - fa.sharedSizeBytes : 0;
  return hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, (int)*avail);
}

#ifndef SFFN_MAX_DEVICES
#define SFFN_MAX_DEVICES 64
#endif
// The dynamic LDS limit of one kernel, set on the current device by its first launch there. Thread-safe: the
// attribute is set exactly once per device (std::call_once), and every caller then reads the stored result.
// One static instance per kernel (a function-local static of the launcher).
struct LdsLimit {
  std::once_flag once[SFFN_MAX_DEVICES];
  size_t avail[SFFN_MAX_DEVICES] = {};
  hipError_t err[SFFN_MAX_DEVICES] = {};
  hipError_t get(const void* func, size_t* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SFFN_MAX_DEVICES) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] { err[dev] = allow_dynamic_lds(func, &avail[dev]); });
    *out = avail[dev];
    return err[dev];
  }
};

// ---- profiling hook (api.hip): while kernel id `kid` is being profiled (sffn_profile_begin), hands out the next
// pair of events. The launch then records the kernel's own start and end timestamps into them
// (hipExtLaunchKernelGGL), the same clock a kernel trace reads; otherwise the plain launch is used.
bool sffn_prof_events(int kid, hipEvent_t* start, hipEvent_t* stop);

#define SFFN_LAUNCH(kid, kern, grid, block, shm, st, ...)                                   \
  do {                                                                                       \
    hipEvent_t sffn_e0_, sffn_e1_;                                                           \
    if (sffn_prof_events(kid, &sffn_e0_, &sffn_e1_))                                         \
      hipExtLaunchKernelGGL(kern, grid, block, shm, st, sffn_e0_, sffn_e1_, 0, __VA_ARGS__); \
    else                                                                                     \
      hipLaunchKernelGGL(kern, grid, block, shm, st, __VA_ARGS__);                           \
  } while (0)

// ---- launchers (host side), defined in the kernel files; return hipError_t of the launch
hipError_t sffn_launch_predict(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D,
                               int F, int r, float tau, int n_hot, uint64_t* mask, float* logits, float* hbuf,
                               hipStream_t st);
hipError_t sffn_launch_predict_hb(const void* P1, const float* x, int x_norm, int B, int D, int r, float* hbuf,
                                  hipStream_t st);
hipError_t sffn_launch_predict_zb(const void* P2, const float* c, const float* hbuf, int B, int F, int r, float tau,
                                  int n_hot, uint64_t* mask, float* logits, hipStream_t st);
hipError_t sffn_launch_forward(int act, const void* Wg, const float* bg, const void* Wu, const float* bu,
                               const void* WdT, const float* x, int x_norm, int B, int D, int F, const uint64_t* mask,
                               int32_t* active, int32_t* n_active, float* y, float* abuf, hipStream_t st);
hipError_t sffn_launch_forward_q4(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu,
                                  const void* su, const float* bu, const uint8_t* qd, const void* sd, const float* x,
                                  int x_norm, int B, int D, int F, const uint64_t* mask, int32_t* active,
                                  int32_t* n_active, float* y, float* abuf, hipStream_t st);
// single-token fused row + column gather (fused.hip): usable when sffn_fused_ok(B, D, F)
bool sffn_fused_ok(int B, int D, int F, int act, bool q4);
hipError_t sffn_launch_fused(int act, const void* Wg, const float* bg, const void* Wu, const float* bu,
                             const void* WdT, const float* x, int x_norm, int D, int F, const uint64_t* mask,
                             int32_t* active, int32_t* n_active, float* part, int G, float* y, hipStream_t st);
hipError_t sffn_launch_fused_q4(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu,
                                const void* su, const float* bu, const uint8_t* qd, const void* sd, const float* x,
                                int x_norm, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active,
                                float* part, int G, float* y, hipStream_t st);

// single-token layer with the predictor's second stage folded into the row gather (decode.hip)
bool sffn_decode_ok(int act, int D, int F, int r, int G);
size_t sffn_decode_dec_bytes(int G);
hipError_t sffn_launch_decode(int act, const void* P2, const float* c, const float* h, int r, float tau, int n_hot,
                              const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                              const float* x, int x_norm, int D, int F, uint32_t* dec, float* logits, float* part,
                              int G, uint64_t* mask, int32_t* active, int32_t* n_active, float* y, hipStream_t st);
hipError_t sffn_launch_predict_h(const void* P1, const float* x, int x_norm, int D, int r, float* hbuf,
                                 hipStream_t st);

// multi-token (union-mask) path, matrix cores (union.hip)
hipError_t sffn_launch_norm_tokens(const float* x, int B, int D, float* xn, hipStream_t st);
// (hf, hs non-NULL: stage 2 through sffn_launch_predict_mz with those fragment buffers, else k_mt_z)
hipError_t sffn_launch_predict_mt(const void* P1, const void* P2, const float* c, const float* x, int B, int D, int F,
                                  int r, float tau, int n_hot, uint64_t* mask, float* logits, float* hbuf,
                                  float* hpart, int KSH, void* hf, float* hs, hipStream_t st);
// union row gather tiled over 64 rows with every token tile (union_rows.hip): token fragments from x (normalised
// when x_norm) into xf (sffn_ur_xf_bytes) and the tokens' powers of two into xs, then the row kernel
size_t sffn_ur_xf_bytes(int B, int D, bool exact);
int sffn_ur_shares(int B);   // k shares per 64 union rows (> 1: partial pre-activations in `pre`, then combined)
int sffn_ur_bmax_shift(int B);   // log2 of the union rows per entry of the largest-|a| table
hipError_t sffn_launch_rows_ur(int act, bool q4, bool exact, const void* Wg, const void* Sg, const float* bg,
                               const void* Wu, const void* Su, const float* bu, const float* x, int x_norm, int B,
                               int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf,
                               float* bmax, void* xf, float* xs, float* pre, hipStream_t st);
// multi-token predictor stage 2 from h [B, r] (hparts > 0, at most 16: the sum of hparts partials [hparts][B][r]): h
// split into fragments in hf (sffn_ur_xf_bytes(B, r, true)) and hs
hipError_t sffn_launch_predict_mz(const void* P2, const float* c, const float* h, int hparts, int B, int F, int r,
                                  float tau, int n_hot, uint64_t* mask, float* logits, void* hf, float* hs,
                                  hipStream_t st);
// activations (octet order, 64-row tiles written whole) from the k shares' partial pre-activations, and the
// largest |a| per 64 rows and token into bmax
hipError_t sffn_launch_act_combine(int act, const float* pre, int KSP, const int32_t* active, const int32_t* n_active,
                                   const float* bias, int B, int F, float* abuf, float* bmax, hipStream_t st);
hipError_t sffn_launch_sum_parts(const float* part, int KS, int n, float* y, hipStream_t st);
// union down projection on the matrix cores (union_down.hip): KS shares of the union rows, each with its tokens'
// power-of-two scale from bmax (one entry per 2^rbs rows), partial sums into part [KS][B][D], then y = their sum
int sffn_ud_shares(int D, int ks_max);
hipError_t sffn_launch_down_ud(bool q4, bool exact, const void* Wd, const void* Sd, const int32_t* active,
                               const int32_t* n_active, const float* abuf, const float* bmax, int rbs, int B, int D,
                               int F, float* part, int KS, float* y, hipStream_t st);
