// Seeded, counter-based synthetic input generator (host and device).
//
// Every element of every synthetic tensor is a pure function of
// (seed, tensor tag, layer/step, logical element index), so any slice of a
// tensor can be regenerated anywhere -- on the GPU to fill HBM in place, or on
// the host to feed a CPU checker -- with bit-identical results.
//
// Random bits: Philox4x32 with 10 rounds, from Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3" (SC'11). Counter =
// (idx_lo, idx_hi, tag, layer), key = (seed_lo, seed_hi).
//
// Value transforms use only integer arithmetic plus a single correctly rounded
// fp32 operation and an integer-only fp32->fp16 round-to-nearest-even
// conversion, so host and device agree bit for bit:
//   normal  : Irwin-Hall sum of eight 16-bit uniforms, centred (an integer n
//             with |n| <= 262140), then (float)n * scale, scale = sigma/std.
//   q4      : low 4 bits of the first output word (uniform on 0..15).
//   uniform : 24-bit uniform u in [0,1), value = fmaf(u, width, lo).
//
// This file holds no part of the sparse-FFN computation; it only makes inputs.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <thread>
#include <vector>
#include <algorithm>
#include <cstdlib>

namespace {

struct P4 { uint32_t v[4]; };

__host__ __device__ inline void mulhilo32(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  hi = (uint32_t)(p >> 32);
  lo = (uint32_t)p;
}

__host__ __device__ inline P4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(M0, c0, hi0, lo0);
    mulhilo32(M1, c2, hi1, lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0; k1 += W1;
  }
  P4 o; o.v[0] = c0; o.v[1] = c1; o.v[2] = c2; o.v[3] = c3;
  return o;
}

__host__ __device__ inline P4 draw(uint64_t seed, uint32_t tag, uint32_t layer, uint64_t idx) {
  return philox4x32_10((uint32_t)idx, (uint32_t)(idx >> 32), tag, layer, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// centred Irwin-Hall sum of eight 16-bit uniforms (mean 8*32767.5 = 262140)
__host__ __device__ inline int32_t ih8(const P4& o) {
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += (int32_t)(o.v[j] & 0xFFFFu) + (int32_t)(o.v[j] >> 16);
  return s - 262140;
}

// fp32 -> fp16 bits, round to nearest, ties to even, written with integer operations only so that host and
// device give the same bits without depending on a conversion instruction's rounding mode.
__host__ __device__ inline uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);           // NaN
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);          // >= 65520 rounds to infinity
  if (ax < 0x38800000u) {                                            // below 2^-14: fp16 subnormal or zero
    const int e = (int)(ax >> 23);
    if (e < 102) return (uint16_t)sign;                              // < 2^-25: rounds to zero
    const uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
    const int sh = 126 - e;                                          // 14..24
    uint32_t r = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
    if (rem > half || (rem == half && (r & 1u))) ++r;
    return (uint16_t)(sign | r);
  }
  uint32_t r = (((ax >> 23) - 112u) << 10) | ((ax & 0x7FFFFFu) >> 13);
  const uint32_t rem = ax & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;           // a carry may step into the exponent
  return (uint16_t)(sign | r);
}

enum Kind { K_NORMAL_F16 = 0, K_NORMAL_F32 = 1, K_Q4 = 2, K_UNIFORM_F16 = 3 };

__host__ __device__ inline void gen_one(int kind, void* out, uint64_t i, uint64_t seed, uint32_t tag, uint32_t layer,
                                        uint64_t start, float a, float b) {
  P4 o = draw(seed, tag, layer, start + i);
  switch (kind) {
    case K_NORMAL_F16: {
      float w = (float)ih8(o) * a;
      ((uint16_t*)out)[i] = f32_to_f16_bits(w);
      break;
    }
    case K_NORMAL_F32: {
      ((float*)out)[i] = (float)ih8(o) * a;
      break;
    }
    case K_Q4: {
      ((uint8_t*)out)[i] = (uint8_t)(o.v[0] & 15u);
      break;
    }
    default: {
      float u = (float)(o.v[1] >> 8) * (1.0f / 16777216.0f);
      ((uint16_t*)out)[i] = f32_to_f16_bits(fmaf(u, b, a));
      break;
    }
  }
}

__global__ void k_fill(int kind, void* out, uint64_t count, uint64_t seed, uint32_t tag, uint32_t layer,
                       uint64_t start, float a, float b) {
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride) gen_one(kind, out, i, seed, tag, layer, start, a, b);
}

int fill(int kind, void* out, int on_device, uint64_t seed, uint32_t tag, uint32_t layer, uint64_t start,
         uint64_t count, float a, float b, void* stream) {
  if (!out && count) return 1;
  if (count == 0) return 0;
  if (on_device) {
    uint64_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, kind, out, count, seed,
                       tag, layer, start, a, b);
    return hipGetLastError() == hipSuccess ? 0 : 2;
  }
  unsigned nt = std::thread::hardware_concurrency();
  const char* env = std::getenv("SYNTH_THREADS");
  if (env) nt = (unsigned)std::atoi(env);
  if (nt < 1) nt = 1;
  if (nt > 16) nt = 16;
  if (count < (1u << 16)) nt = 1;
  std::vector<std::thread> th;
  uint64_t per = (count + nt - 1) / nt;
  for (unsigned t = 0; t < nt; ++t) {
    uint64_t lo = t * per, hi = std::min<uint64_t>(count, lo + per);
    if (lo >= hi) break;
    th.emplace_back([=]() {
      for (uint64_t i = lo; i < hi; ++i) gen_one(kind, out, i, seed, tag, layer, start, a, b);
    });
  }
  for (auto& t : th) t.join();
  return 0;
}

}  // namespace

extern "C" {

// The fp32 -> fp16 conversion used by the fills (host), for tests.
void synth_f32_to_f16(const float* in, uint16_t* out, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_f16_bits(in[i]);
}

// Raw Philox4x32-10 block, for known-answer tests.
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  P4 o = philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int j = 0; j < 4; ++j) out[j] = o.v[j];
}

// out[i] = fp16((float)IH8(start+i) * scale), i < count. Returns 0 on success.
int synth_fill_normal_f16(void* out, int on_device, uint64_t seed, uint32_t tag, uint32_t layer, uint64_t start,
                          uint64_t count, float scale, void* stream) {
  return fill(K_NORMAL_F16, out, on_device, seed, tag, layer, start, count, scale, 0.f, stream);
}
// out[i] = (float)IH8(start+i) * scale.
int synth_fill_normal_f32(float* out, int on_device, uint64_t seed, uint32_t tag, uint32_t layer, uint64_t start,
                          uint64_t count, float scale, void* stream) {
  return fill(K_NORMAL_F32, out, on_device, seed, tag, layer, start, count, scale, 0.f, stream);
}
// out[i] = uniform integer in [0, 15], one per byte.
int synth_fill_q4(uint8_t* out, int on_device, uint64_t seed, uint32_t tag, uint32_t layer, uint64_t start,
                  uint64_t count, void* stream) {
  return fill(K_Q4, out, on_device, seed, tag, layer, start, count, 0.f, 0.f, stream);
}
// out[i] = fp16(fmaf(u, width, lo)), u a 24-bit uniform in [0, 1).
int synth_fill_uniform_f16(void* out, int on_device, uint64_t seed, uint32_t tag, uint32_t layer, uint64_t start,
                           uint64_t count, float lo, float width, void* stream) {
  return fill(K_UNIFORM_F16, out, on_device, seed, tag, layer, start, count, lo, width, stream);
}

}  // extern "C"
