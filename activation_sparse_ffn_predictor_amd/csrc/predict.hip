// Activation predictor: h = P1 xn (fp32), z = P2 h + c, mask bit = OR over tokens of (z > tau).
//
// PowerInfer pages, Turkish article, "Adaptive sparsity predictors" and "Online stage": a small per-layer
// predictor runs on every token and marks the neurons that will fire. Here it is the low-rank form
// P2 (P1 x) + c with a sigmoid threshold t, decided in logit space (tau = ln(t / (1 - t))).
//
// Kernel 1 (k_pred_h): one wave per row of P1. Every lane issues all of its 16-byte loads of the row before
// waiting, x is staged once per block in LDS (optionally RMS-normalised), the row dot products are reduced
// across the wave. h stays fp32.
// Kernel 2 (k_pred_z): one block per 64 neurons (one mask word). Groups of LPR lanes read one 2r-byte row of
// P2 with 16-byte loads; h sits in LDS; the group reduces, compares with tau, and wave 0 turns the 64
// decisions into the mask word with a wavefront ballot.
#include "common.h"

using namespace sffn;

namespace {

constexpr int NT = 256;          // threads per block
constexpr int X_LDS_FLOATS = 16384;  // x staging budget (64 KB)

template <int NCH>
__global__ __launch_bounds__(NT) void k_pred_h(const uint4* __restrict__ P1, const float* __restrict__ x, int x_rms,
                                               int B, int D, int r, float* __restrict__ h) {
  extern __shared__ float lds[];
  const int TB = max(1, min(B, X_LDS_FLOATS / D));
  float* xs = lds;                       // [TB, D]
  float* red = lds + (size_t)TB * D;     // [(NT/64) * TB]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x * (NT / 64) + w;
  const int nc = D >> 3;
  uint4 wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    wv[i] = (j < r && c < nc) ? P1[(size_t)j * nc + c] : make_uint4(0u, 0u, 0u, 0u);
  }
  for (int tb = 0; tb < B; tb += TB) {
    const int nb = min(TB, B - tb);
    stage_x<NT>(x + (size_t)tb * D, nb, D, x_rms, xs, red);
    for (int b = 0; b < nb; ++b) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < nc) {
          const float4* xp = reinterpret_cast<const float4*>(xs + (size_t)b * D + 8 * c);
          float4 x0 = xp[0], x1 = xp[1];
          float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          acc += dot8(wv[i], xv);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0 && j < r) h[(size_t)(tb + b) * r + j] = acc;
    }
    __syncthreads();  // xs is overwritten by the next token group
  }
}

// LPR lanes per P2 row (power of two, 8..64), ROUNDS chunk rounds per row (1 or 2).
template <int LPR, int ROUNDS>
__global__ __launch_bounds__(NT) void k_pred_z(const uint4* __restrict__ P2, const float* __restrict__ c,
                                               const float* __restrict__ h, int B, int F, int r, float tau,
                                               uint64_t* __restrict__ mask, float* __restrict__ logits) {
  constexpr int RPI = 64 / LPR;        // rows per load instruction
  constexpr int RPW = 16;              // rows per wave
  constexpr int NI = RPW / RPI;        // load instructions per chunk round
  extern __shared__ float lds[];
  float* hs = lds;                                     // [B, r]
  int* flags = reinterpret_cast<int*>(lds + (size_t)B * r);  // [64]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane / LPR, csub = lane % LPR;
  const int cpr = r >> 3;              // 16-byte chunks per row
  const int base = blockIdx.x * 64 + w * RPW;

  uint4 wv[ROUNDS][NI];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = base + i * RPI + rsub;
      const int cc = q * LPR + csub;
      wv[q][i] = (k < F && cc < cpr) ? P2[(size_t)k * cpr + cc] : make_uint4(0u, 0u, 0u, 0u);
    }
  for (int i = threadIdx.x; i < B * r; i += NT) hs[i] = h[i];
  __syncthreads();

  bool pred[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) pred[i] = false;
  for (int b = 0; b < B; ++b) {
    const float* hb = hs + (size_t)b * r;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < ROUNDS; ++q) {
        const int cc = q * LPR + csub;
        if (cc < cpr) {
          const float4* hp = reinterpret_cast<const float4*>(hb + 8 * cc);
          float4 h0 = hp[0], h1 = hp[1];
          float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
          acc += dot8(wv[q][i], hv);
        }
      }
      acc = group_sum<LPR>(acc);
      const int k = base + i * RPI + rsub;
      if (csub == 0 && k < F) {
        const float z = acc + (c ? c[k] : 0.f);
        pred[i] = pred[i] || (z > tau);
        if (logits) logits[(size_t)b * F + k] = z;
      }
    }
  }
  if (csub == 0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) flags[w * RPW + i * RPI + rsub] = pred[i] ? 1 : 0;
  }
  __syncthreads();
  if (w == 0) {
    const int k = blockIdx.x * 64 + lane;
    const bool bit = (k < F) && flags[lane] != 0;
    const unsigned long long word = __ballot(bit);
    if (lane == 0) mask[blockIdx.x] = (uint64_t)word;
  }
}

template <int NCH>
hipError_t launch_h(const void* P1, const float* x, int x_rms, int B, int D, int r, float* h, hipStream_t st) {
  const int TB = std::max(1, std::min(B, X_LDS_FLOATS / D));
  const size_t lds = ((size_t)TB * D + (NT / 64) * TB) * sizeof(float);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_pred_h<NCH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(X_LDS_FLOATS * 4 + 4096));
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int grid = (r + NT / 64 - 1) / (NT / 64);
  hipLaunchKernelGGL(k_pred_h<NCH>, dim3(grid), dim3(NT), lds, st, (const uint4*)P1, x, x_rms, B, D, r, h);
  return hipGetLastError();
}

template <int LPR, int ROUNDS>
hipError_t launch_z(const void* P2, const float* c, const float* h, int B, int F, int r, float tau, uint64_t* mask,
                    float* logits, hipStream_t st) {
  const size_t lds = (size_t)B * r * sizeof(float) + 64 * sizeof(int);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_pred_z<LPR, ROUNDS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * 4 + 256);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int grid = (F + 63) / 64;
  hipLaunchKernelGGL((k_pred_z<LPR, ROUNDS>), dim3(grid), dim3(NT), lds, st, (const uint4*)P2, c, h, B, F, r, tau,
                     mask, logits);
  return hipGetLastError();
}

}  // namespace

hipError_t sffn_launch_predict(const void* P1, const void* P2, const float* c, const float* x, int x_rms, int B, int D,
                               int F, int r, float tau, uint64_t* mask, float* logits, float* hbuf, hipStream_t st) {
  const int nch = (D / 8 + 63) / 64;
  hipError_t e;
  if (nch <= 1) e = launch_h<1>(P1, x, x_rms, B, D, r, hbuf, st);
  else if (nch <= 2) e = launch_h<2>(P1, x, x_rms, B, D, r, hbuf, st);
  else if (nch <= 4) e = launch_h<4>(P1, x, x_rms, B, D, r, hbuf, st);
  else if (nch <= 8) e = launch_h<8>(P1, x, x_rms, B, D, r, hbuf, st);
  else if (nch <= 10) e = launch_h<10>(P1, x, x_rms, B, D, r, hbuf, st);
  else if (nch <= 16) e = launch_h<16>(P1, x, x_rms, B, D, r, hbuf, st);
  else e = launch_h<32>(P1, x, x_rms, B, D, r, hbuf, st);
  if (e != hipSuccess) return e;
  const int cpr = r / 8;
  int lpr = 8;
  while (lpr * 2 <= cpr && lpr < 64) lpr *= 2;
  const int rounds = (cpr + lpr - 1) / lpr;  // 1 or 2 for r <= 1024
  switch (lpr * 10 + rounds) {
    case 81: return launch_z<8, 1>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    case 82: return launch_z<8, 2>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    case 161: return launch_z<16, 1>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    case 162: return launch_z<16, 2>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    case 321: return launch_z<32, 1>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    case 322: return launch_z<32, 2>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    case 641: return launch_z<64, 1>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    case 642: return launch_z<64, 2>(P2, c, hbuf, B, F, r, tau, mask, logits, st);
    default: return hipErrorInvalidValue;
  }
}
