// Activation predictor: h = P1 xn (fp32), z = P2 h + c, mask bit = OR over tokens of (z > tau).
//
// PowerInfer pages, Turkish article, "Adaptive sparsity predictors" and "Online stage": a small per-layer
// predictor runs on every token and marks the neurons that will fire. Here it is the low-rank form
// P2 (P1 x) + c with a sigmoid threshold t, decided in logit space (tau = ln(t / (1 - t))).
//
// Both kernels cost one dependent memory round trip: every global load is issued branch-free (clamped address,
// value selected afterwards) before the first use, so all of them are in flight together.
// Kernel 1 (k_pred_h): one 64-thread block (one wave) per row of P1. Lane l owns the 16-byte chunks
//   c = l + 64 i of its row and loads them with the matching 8 floats of x; the optional normalisation of x
//   (mean, then centred variance) is two wave reductions over registers; the row dot product is reduced
//   across the wave. h stays fp32.
// Kernel 2 (k_pred_z): one block per 64 neurons (one mask word), 16 neurons per wave. Groups of LPR lanes read
//   one 2r-byte row of P2 with 16-byte loads together with the matching slice of h and the bias; the group
//   reduces, compares with tau, and wave 0 turns the 64 decisions into the mask word with a wavefront ballot.
#include "common.h"

using namespace sffn;

namespace {

constexpr int NT = 256;

template <int NCH>
__global__ __launch_bounds__(64) void k_pred_h(const uint4* __restrict__ P1, const float* __restrict__ x, int x_norm,
                                               int B, int D, int r, float* __restrict__ h) {
  const int lane = threadIdx.x;
  const int j = blockIdx.x;
  const int nc = D >> 3;
  const Buf bp(P1, (uint32_t)r * (uint32_t)D * 2u);
  const Buf bx(x, (uint32_t)B * (uint32_t)D * 4u);
  uint4 wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    wv[i] = bp.ld16(boff(c < nc, ((uint32_t)j * nc + c) * 16u));
  }
  float4 xr[NCH][2];
  auto load_x = [&](int b) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      const uint32_t o = ((uint32_t)b * D + 8u * c) * 4u;
      xr[i][0] = bx.ldf4(boff(c < nc, o));
      xr[i][1] = bx.ldf4(boff(c < nc, o + 16u));
    }
  };
  load_x(0);  // before any loop: in flight together with the row of P1
  for (int b = 0; b < B; ++b) {
    if (b > 0) load_x(b);
    if (x_norm) wave_norm_regs<NCH, 2>(xr, nc, D);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float xv[8] = {xr[i][0].x, xr[i][0].y, xr[i][0].z, xr[i][0].w,
                           xr[i][1].x, xr[i][1].y, xr[i][1].z, xr[i][1].w};
      acc += dot8(wv[i], xv);
    }
    acc = wave_sum(acc);
    if (lane == 0) h[(size_t)b * r + j] = acc;
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
  __shared__ int flags[64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane / LPR, csub = lane % LPR;
  const int cpr = r >> 3;              // 16-byte chunks per row
  const int base = blockIdx.x * 64 + w * RPW;

  const Buf bp(P2, (uint32_t)F * (uint32_t)r * 2u);
  const Buf bc(c ? (const void*)c : (const void*)P2, c ? (uint32_t)F * 4u : 0u);   // no bias: every load is 0
  const Buf bh(h, (uint32_t)B * (uint32_t)r * 4u);
  uint4 wv[ROUNDS][NI];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = base + i * RPI + rsub;
      const int cc = q * LPR + csub;
      wv[q][i] = bp.ld16(boff(k < F && cc < cpr, ((uint32_t)k * cpr + cc) * 16u));
    }
  float cb[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int k = base + i * RPI + rsub;
    cb[i] = bc.ldf(boff(k < F, (uint32_t)k * 4u));
  }
  bool pred[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) pred[i] = false;
  float hv[ROUNDS][8];
  auto load_h = [&](int b) {
#pragma unroll
    for (int q = 0; q < ROUNDS; ++q) {
      const int cc = q * LPR + csub;
      const bool ok = cc < cpr;
      const float4 h0 = bh.ldf4(boff(ok, ((uint32_t)b * r + 8u * cc) * 4u));
      const float4 h1 = bh.ldf4(boff(ok, ((uint32_t)b * r + 8u * cc + 4u) * 4u));
      hv[q][0] = h0.x; hv[q][1] = h0.y; hv[q][2] = h0.z; hv[q][3] = h0.w;
      hv[q][4] = h1.x; hv[q][5] = h1.y; hv[q][6] = h1.z; hv[q][7] = h1.w;
    }
  };
  load_h(0);  // before any loop: in flight together with the P2 rows
  for (int b = 0; b < B; ++b) {
    if (b > 0) load_h(b);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < ROUNDS; ++q) acc += dot8(wv[q][i], hv[q]);
      acc = group_sum<LPR>(acc);
      const int k = base + i * RPI + rsub;
      if (csub == 0 && k < F) {
        const float z = acc + cb[i];
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
hipError_t launch_h(const void* P1, const float* x, int x_norm, int B, int D, int r, float* h, hipStream_t st) {
  sffn_prof_before(0, st);
  hipLaunchKernelGGL(k_pred_h<NCH>, dim3(r), dim3(64), 0, st, (const uint4*)P1, x, x_norm, B, D, r, h);
  sffn_prof_after(0, st);
  return hipGetLastError();
}

template <int LPR, int ROUNDS>
hipError_t launch_z(const void* P2, const float* c, const float* h, int B, int F, int r, float tau, uint64_t* mask,
                    float* logits, hipStream_t st) {
  const int grid = (F + 63) / 64;
  sffn_prof_before(1, st);
  hipLaunchKernelGGL((k_pred_z<LPR, ROUNDS>), dim3(grid), dim3(NT), 0, st, (const uint4*)P2, c, h, B, F, r, tau,
                     mask, logits);
  sffn_prof_after(1, st);
  return hipGetLastError();
}

}  // namespace

hipError_t sffn_launch_predict(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D,
                               int F, int r, float tau, uint64_t* mask, float* logits, float* hbuf, hipStream_t st) {
  const int nch = (D / 8 + 63) / 64;
  hipError_t e;
  if (nch <= 1) e = launch_h<1>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 2) e = launch_h<2>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 4) e = launch_h<4>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 8) e = launch_h<8>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 10) e = launch_h<10>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 16) e = launch_h<16>(P1, x, x_norm, B, D, r, hbuf, st);
  else e = launch_h<32>(P1, x, x_norm, B, D, r, hbuf, st);
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
