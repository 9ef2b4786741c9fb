// Shared device helpers and launch declarations of libsffn (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace sffn {

constexpr int WAVE = 64;
constexpr float RMS_EPS = 1e-6f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// sum over aligned groups of G lanes (G a power of two <= 64); every lane of the group gets the sum
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

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

// Stage xn[b, d] for b < nb, d < D into LDS (fp32, row stride D), normalising each token by its RMS if asked.
// Every thread of the block takes part. red: >= (NT/64) * nb floats of LDS scratch. Deterministic: per-wave
// partial sums are combined in wave order.
template <int NT>
__device__ __forceinline__ void stage_x(const float* __restrict__ x, int nb, int D, int x_rms, float* xs, float* red) {
  const int n4 = D >> 2;  // D % 8 == 0
  for (int b = 0; b < nb; ++b) {
    const float4* src = reinterpret_cast<const float4*>(x + (size_t)b * D);
    float4* dst = reinterpret_cast<float4*>(xs + (size_t)b * D);
    for (int i = threadIdx.x; i < n4; i += NT) dst[i] = src[i];
  }
  __syncthreads();
  if (!x_rms) return;
  const int w = threadIdx.x >> 6;
  for (int b = 0; b < nb; ++b) {
    float s = 0.f;
    for (int i = threadIdx.x; i < D; i += NT) { float v = xs[(size_t)b * D + i]; s = fmaf(v, v, s); }
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[w * nb + b] = s;
  }
  __syncthreads();
  for (int b = 0; b < nb; ++b) {
    float tot = 0.f;
    for (int i = 0; i < NT / 64; ++i) tot += red[i * nb + b];
    const float sc = 1.0f / sqrtf(tot / (float)D + RMS_EPS);
    for (int i = threadIdx.x; i < D; i += NT) xs[(size_t)b * D + i] *= sc;
  }
  __syncthreads();
}

// Mask word t with the bits of neurons >= F cleared (callers may pass any bit pattern there).
__device__ __forceinline__ uint64_t mask_word(const uint64_t* __restrict__ mask, int t, int nw, int F) {
  uint64_t w = mask[t];
  if (t == nw - 1 && (F & 63)) w &= (1ull << (F & 63)) - 1ull;
  return w;
}

// Locate the i-th set bit (0-based, dense index i < total) of the mask. roff[T] = exclusive prefix of set bits
// over thread ranges of WPT words each. Wave-uniform result: the stored neuron id.
__device__ __forceinline__ int locate(const uint64_t* __restrict__ mask, const int* roff, int nranges, int wpt, int nw,
                                      int F, int i) {
  int lo = 0, hi = nranges - 1;  // largest T with roff[T] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (roff[mid] <= i) lo = mid; else hi = mid - 1;
  }
  int rem = i - roff[lo];
  int t = lo * wpt;
  uint64_t word = 0;
  for (; t < nw; ++t) {
    word = mask_word(mask, t, nw, F);
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

// Per-block prefix over mask words: each thread owns WPT consecutive words; roff[t] = set bits before range t.
template <int NT>
__device__ __forceinline__ int mask_prefix(const uint64_t* __restrict__ mask, int nw, int F, int wpt, int* roff,
                                           int* tmp) {
  const int t0 = threadIdx.x * wpt;
  int cnt = 0;
  for (int t = t0; t < min(nw, t0 + wpt); ++t) cnt += __popcll(mask_word(mask, t, nw, F));
  int total;
  const int ex = block_exclusive_scan<NT>(cnt, tmp, total);
  roff[threadIdx.x] = ex;
  __syncthreads();
  return total;
}

}  // namespace sffn

// ---- launchers (host side), defined in the kernel files; return hipError_t of the launch
hipError_t sffn_launch_predict(const void* P1, const void* P2, const float* c, const float* x, int x_rms, int B, int D,
                               int F, int r, float tau, uint64_t* mask, float* logits, float* hbuf, hipStream_t st);
hipError_t sffn_launch_forward(int act, const void* Wg, const float* bg, const void* Wu, const float* bu,
                               const void* WdT, const float* x, int x_rms, int B, int D, int F, const uint64_t* mask,
                               int32_t* active, int32_t* n_active, float* y, float* abuf, hipStream_t st);
hipError_t sffn_launch_forward_q4(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu,
                                  const void* su, const float* bu, const uint8_t* qd, const void* sd, const float* x,
                                  int x_rms, int B, int D, int F, const uint64_t* mask, int32_t* active,
                                  int32_t* n_active, float* y, float* abuf, hipStream_t st);
