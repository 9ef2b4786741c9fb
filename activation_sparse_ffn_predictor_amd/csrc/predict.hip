// Activation predictor: h = P1 xn (fp32), z = P2 h + c, mask bit = OR over tokens of (z > tau).
//
// PowerInfer pages, Turkish article, "Adaptive sparsity predictors" and "Online stage": a small per-layer
// predictor runs on every token and marks the neurons that will fire. Here it is the low-rank form
// P2 (P1 x) + c with a sigmoid threshold t, decided in logit space (tau = ln(t / (1 - t))).
//
// Both kernels cost one dependent memory round trip: every global load is issued branch-free (buffer loads whose
// out-of-range offsets read 0) before the first use, so all of them are in flight together.
// Kernel 1 (k_pred_h): one 256-thread block per row of P1. Thread t owns the 16-byte chunks c = t + 256 m of the
//   row and loads them with the matching 8 floats of x. One block reduction of four sums gives the row dot
//   product and, for the optional normalisation of x, the statistics: with x' = x - x[0] (a shift that keeps the
//   single-pass variance well conditioned), mu' = mean(x'), var = mean(x'^2) - mu'^2 and
//   P1[j] . (x - mean) / sqrt(var + eps) = (sum P1[j] x' - mu' sum P1[j]) / sqrt(var + eps). h stays fp32.
// Kernel 2 (k_pred_z): one wave per 16 neurons, four waves per block (one mask word per block), no block
//   barrier. Groups of LPR lanes read one 2r-byte row of P2 with 16-byte loads together with the matching slice
//   of h and the bias; the group reduces and compares with tau, a wavefront ballot gathers the wave's 16
//   decisions, and the wave stores them as its 16-bit quarter of the mask word.
#include "common.h"

using namespace sffn;

namespace {

constexpr int NT = 256;
#ifndef SFFN_Z_LPR_MAX
#define SFFN_Z_LPR_MAX 8         // lanes per P2 row in the stage-2 kernel (fewer lanes: more chunk rounds per lane)
#endif

constexpr int NTH = 256;

template <int NCH>
__global__ __launch_bounds__(NTH) void k_pred_h(const uint4* __restrict__ P1, const float* __restrict__ x, int x_norm,
                                                int D, int r, float* __restrict__ h) {
  __shared__ float red[4][NTH / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x;
  const int nc = D >> 3;
  const Buf bp(P1, (uint32_t)r * (uint32_t)D * 2u);
  const Buf bx(x, (uint32_t)D * 4u);
  // one round trip: x, its first element (the shift) and the row of P1, all issued before the first use
  float4 xr[NCH][2];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + NTH * i;
    xr[i][0] = bx.ldf4(boff(c < nc, 32u * c));
    xr[i][1] = bx.ldf4(boff(c < nc, 32u * c + 16u));
  }
  const float x0 = bx.ldf(boff(x_norm != 0, 0u));
  uint4 wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + NTH * i;
    wv[i] = bp.ld16(boff(c < nc, ((uint32_t)j * nc + c) * 16u));
  }
  __builtin_amdgcn_sched_barrier(0);
  float spx = 0.f, sp = 0.f, sx = 0.f, sxx = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + NTH * i;
    if (c < nc) {
      float pf[8];
      f16x8_to_f32(wv[i], pf);
      const float xv[8] = {xr[i][0].x, xr[i][0].y, xr[i][0].z, xr[i][0].w,
                           xr[i][1].x, xr[i][1].y, xr[i][1].z, xr[i][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = xv[e] - x0;
        spx = fmaf(pf[e], d, spx);
        sp += pf[e];
        sx += d;
        sxx = fmaf(d, d, sxx);
      }
    }
  }
  spx = wave_sum(spx);
  if (x_norm) { sp = wave_sum(sp); sx = wave_sum(sx); sxx = wave_sum(sxx); }
  if (lane == 0) { red[0][w] = spx; red[1][w] = sp; red[2][w] = sx; red[3][w] = sxx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int ww = 0; ww < NTH / 64; ++ww) t[k] += red[k][ww];
    float hv = t[0];
    if (x_norm) {
      const float mu = t[2] / (float)D;
      const float var = fmaxf(t[3] / (float)D - mu * mu, 0.f);
      hv = (t[0] - mu * t[1]) / sqrtf(var + NORM_EPS);
    }
    h[j] = hv;
  }
}

// Kernel 1 for a few tokens (k_pred_hb, 2 <= B <= 8): one 512-thread block per row of P1; the row is read once
// and every token's x with it. Tokens are taken TB at a time (TB = the batch rounded up to 2, 4 or 8, at most 4
// when D > 8192; a batch within one group costs one round trip); per token the same four sums as k_pred_h,
// reduced together. h[b][j] is complete: no partial sums, no separate
// normalisation of x.
constexpr int NTB = 512;

template <int NCH, int TB>
__global__ __launch_bounds__(NTB) void k_pred_hb(const uint4* __restrict__ P1, const float* __restrict__ x,
                                                 int x_norm, int B, int D, int r, float* __restrict__ h) {
  constexpr int NV = 3 * TB + 1;                       // per token: sum p x', sum x', sum x'^2; then sum p
  __shared__ float red[NV][NTB / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x;
  const int nc = D >> 3;
  const Buf bp(P1, (uint32_t)r * (uint32_t)D * 2u);
  const Buf bx(x, (uint32_t)B * (uint32_t)D * 4u);
  uint4 wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + NTB * i;
    wv[i] = bp.ld16(boff(c < nc, ((uint32_t)j * nc + c) * 16u));
  }
  for (int b0 = 0; b0 < B; b0 += TB) {                 // token groups (block-uniform)
    // x of the group's tokens and their first elements (the shifts), all issued before the first use
    float4 xr[TB][NCH][2];
    float x0[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const bool okt = b0 + t < B;
      const uint32_t tb = (uint32_t)(b0 + t) * (uint32_t)D * 4u;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = threadIdx.x + NTB * i;
        xr[t][i][0] = bx.ldf4(boff(okt && c < nc, tb + 32u * c));
        xr[t][i][1] = bx.ldf4(boff(okt && c < nc, tb + 32u * c + 16u));
      }
      x0[t] = bx.ldf(boff(okt && x_norm != 0, tb));
    }
    __builtin_amdgcn_sched_barrier(0);
    float v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + NTB * i;
      if (c < nc) {
        float pf[8];
        f16x8_to_f32(wv[i], pf);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[3 * TB] += pf[e];
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const float xv[8] = {xr[t][i][0].x, xr[t][i][0].y, xr[t][i][0].z, xr[t][i][0].w,
                               xr[t][i][1].x, xr[t][i][1].y, xr[t][i][1].z, xr[t][i][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = xv[e] - x0[t];
            v[3 * t] = fmaf(pf[e], d, v[3 * t]);
            v[3 * t + 1] += d;
            v[3 * t + 2] = fmaf(d, d, v[3 * t + 2]);
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (k % 3 != 0 && !x_norm) continue;             // the statistics and sum p only when x is normalised
      v[k] = wave_sum(v[k]);
      if (lane == 0) red[k][w] = v[k];
    }
    __syncthreads();
    if (threadIdx.x < TB && b0 + (int)threadIdx.x < B) {
      const int t = threadIdx.x;
      float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < NTB / 64; ++ww) {
        s[0] += red[3 * t][ww];
        if (x_norm) { s[1] += red[3 * t + 1][ww]; s[2] += red[3 * t + 2][ww]; s[3] += red[3 * TB][ww]; }
      }
      float hv = s[0];
      if (x_norm) {
        const float mu = s[1] / (float)D;
        const float var = fmaxf(s[2] / (float)D - mu * mu, 0.f);
        hv = (s[0] - mu * s[3]) / sqrtf(var + NORM_EPS);
      }
      h[(size_t)(b0 + t) * r + j] = hv;
    }
    __syncthreads();                                   // red is reused by the next token group
  }
}

// LPR lanes per P2 row (power of two, 8..64), ROUNDS chunk rounds per row (1 or 2). One token (larger batches
// take the matrix-core kernels).
template <int LPR, int ROUNDS>
__global__ __launch_bounds__(NT) void k_pred_z(const uint4* __restrict__ P2, const float* __restrict__ c,
                                               const float* __restrict__ h, int F, int r, float tau, int n_hot,
                                               uint64_t* __restrict__ mask, float* __restrict__ logits) {
  constexpr int RPI = 64 / LPR;        // rows per load instruction
  constexpr int RPW = 16;              // rows per wave = one 16-bit quarter of a mask word
  constexpr int NI = RPW / RPI;        // load instructions per chunk round
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane / LPR, csub = lane % LPR;
  const int cpr = r >> 3;              // 16-byte chunks per row
  const int base = blockIdx.x * 64 + w * RPW;

  const Buf bp(P2, (uint32_t)F * (uint32_t)r * 2u);
  const Buf bc(c ? (const void*)c : (const void*)P2, c ? (uint32_t)F * 4u : 0u);   // no bias: every load is 0
  const Buf bh(h, (uint32_t)r * 4u);
  // one round trip: P2 rows, h slice and biases are all issued before the first use (P2 first: its addresses
  // need no loaded value)
  uint4 wv[ROUNDS][NI];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = base + i * RPI + rsub;
      const int cc = q * LPR + csub;
      wv[q][i] = bp.ld16(boff(k < F && k >= n_hot && cc < cpr, ((uint32_t)k * cpr + cc) * 16u));
    }
  float hv[ROUNDS][8];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    const int cc = q * LPR + csub;
    const bool ok = cc < cpr;
    const float4 h0 = bh.ldf4(boff(ok, 32u * cc));
    const float4 h1 = bh.ldf4(boff(ok, 32u * cc + 16u));
    hv[q][0] = h0.x; hv[q][1] = h0.y; hv[q][2] = h0.z; hv[q][3] = h0.w;
    hv[q][4] = h1.x; hv[q][5] = h1.y; hv[q][6] = h1.z; hv[q][7] = h1.w;
  }
  float cb[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int k = base + i * RPI + rsub;
    cb[i] = bc.ldf(boff(k < F && k >= n_hot, (uint32_t)k * 4u));
  }
  __builtin_amdgcn_sched_barrier(0);
  // decisions: instruction i, row group q sits at lane q * LPR
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < ROUNDS; ++q) acc += dot8(wv[q][i], hv[q]);
    acc = group_sum<LPR>(acc);
    const int k = base + i * RPI + rsub;
    const float z = k < n_hot ? INFINITY : acc + cb[i];   // the always-active prefix: no row was read
    const bool on = csub == 0 && k < F && z > tau;
    if (logits && csub == 0 && k < F) logits[k] = z;
    const unsigned long long bal = __ballot(on);
#pragma unroll
    for (int q = 0; q < RPI; ++q)
      if ((bal >> (q * LPR)) & 1ull) bits |= 1u << (i * RPI + q);
  }
  if (lane == 0) reinterpret_cast<uint16_t*>(mask)[(size_t)blockIdx.x * 4 + w] = (uint16_t)bits;
}

// Kernel 2 for a few tokens (k_pred_zb, 2 <= B <= 4): the k_pred_z layout, with the tokens' h staged in LDS so that
// each row of P2 is read once for all of them. Every token's logit is computed and stored; the mask bit is the OR
// of the tokens' decisions (the union mask of the batch). P2 rows, h and the biases are issued together: one round
// trip, then one block barrier for the LDS copy of h.
template <int LPR, int ROUNDS, int TB>
__global__ __launch_bounds__(NT) void k_pred_zb(const uint4* __restrict__ P2, const float* __restrict__ c,
                                                const float* __restrict__ h, int B, int F, int r, float tau,
                                                int n_hot, uint64_t* __restrict__ mask, float* __restrict__ logits) {
  constexpr int RPI = 64 / LPR;
  constexpr int RPW = 16;
  constexpr int NI = RPW / RPI;
  constexpr int RMAX = 8 * LPR * ROUNDS;               // h elements per token held in LDS (r <= RMAX)
  constexpr int NHL = (TB * RMAX / 4 + NT - 1) / NT;   // float4 loads per thread for the LDS copy
  __shared__ float4 hs4[TB * RMAX / 4];
  const float* hs = reinterpret_cast<const float*>(hs4);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane / LPR, csub = lane % LPR;
  const int cpr = r >> 3;
  const int base = blockIdx.x * 64 + w * RPW;

  const Buf bp(P2, (uint32_t)F * (uint32_t)r * 2u);
  const Buf bc(c ? (const void*)c : (const void*)P2, c ? (uint32_t)F * 4u : 0u);
  const Buf bh(h, (uint32_t)B * (uint32_t)r * 4u);
  uint4 wv[ROUNDS][NI];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = base + i * RPI + rsub;
      const int cc = q * LPR + csub;
      wv[q][i] = bp.ld16(boff(k < F && k >= n_hot && cc < cpr, ((uint32_t)k * cpr + cc) * 16u));
    }
  float4 hl[NHL];
#pragma unroll
  for (int l = 0; l < NHL; ++l) {
    const int e = (threadIdx.x + NT * l) * 4;          // LDS element: token e / RMAX, h index e % RMAX
    const int t = e / RMAX, j = e % RMAX;
    hl[l] = bh.ldf4(boff(t < B && j < r, ((uint32_t)t * r + j) * 4u));   // r % 8 == 0: j < r means j + 4 <= r
  }
  float cb[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int k = base + i * RPI + rsub;
    cb[i] = bc.ldf(boff(k < F && k >= n_hot, (uint32_t)k * 4u));
  }
#pragma unroll
  for (int l = 0; l < NHL; ++l)
    if (threadIdx.x + NT * l < TB * RMAX / 4) hs4[threadIdx.x + NT * l] = hl[l];
  __syncthreads();
  bool any[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) any[i] = false;
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    if (t >= B) break;                                 // block-uniform
    float acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = 0.f;
#pragma unroll
    for (int q = 0; q < ROUNDS; ++q) {
      const int cc = q * LPR + csub;                   // cc >= cpr: the P2 chunk read 0 and the LDS slot holds 0
      const float4 h0 = *reinterpret_cast<const float4*>(hs + t * RMAX + 8 * cc);
      const float4 h1 = *reinterpret_cast<const float4*>(hs + t * RMAX + 8 * cc + 4);
      const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[i] += dot8(wv[q][i], hv);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float s = group_sum<LPR>(acc[i]);
      const int k = base + i * RPI + rsub;
      const float z = k < n_hot ? INFINITY : s + cb[i];
      if (logits && csub == 0 && k < F) logits[(size_t)t * F + k] = z;
      any[i] = any[i] || z > tau;
    }
  }
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int k = base + i * RPI + rsub;
    const unsigned long long bal = __ballot(csub == 0 && k < F && any[i]);
#pragma unroll
    for (int q = 0; q < RPI; ++q)
      if ((bal >> (q * LPR)) & 1ull) bits |= 1u << (i * RPI + q);
  }
  if (lane == 0) reinterpret_cast<uint16_t*>(mask)[(size_t)blockIdx.x * 4 + w] = (uint16_t)bits;
}

template <int NCH>
hipError_t launch_h(const void* P1, const float* x, int x_norm, int B, int D, int r, float* h, hipStream_t st) {
  SFFN_LAUNCH(0, k_pred_h<NCH>, dim3(r), dim3(NTH), 0, st, (const uint4*)P1, x, x_norm, D, r, h);
  return hipGetLastError();
}

template <int NCH, int TB>
hipError_t launch_hb(const void* P1, const float* x, int x_norm, int B, int D, int r, float* h, hipStream_t st) {
  SFFN_LAUNCH(0, (k_pred_hb<NCH, TB>), dim3(r), dim3(NTB), 0, st, (const uint4*)P1, x, x_norm, B, D, r, h);
  return hipGetLastError();
}

template <int LPR, int ROUNDS>
hipError_t launch_z(const void* P2, const float* c, const float* h, int B, int F, int r, float tau, int n_hot,
                    uint64_t* mask, float* logits, hipStream_t st) {
  const int grid = (F + 63) / 64;
  SFFN_LAUNCH(1, (k_pred_z<LPR, ROUNDS>), dim3(grid), dim3(NT), 0, st, (const uint4*)P2, c, h, F, r, tau, n_hot, mask,
              logits);
  return hipGetLastError();
}

template <int LPR, int ROUNDS, int TB>
hipError_t launch_zb(const void* P2, const float* c, const float* h, int B, int F, int r, float tau, int n_hot,
                     uint64_t* mask, float* logits, hipStream_t st) {
  SFFN_LAUNCH(1, (k_pred_zb<LPR, ROUNDS, TB>), dim3((F + 63) / 64), dim3(NT), 0, st, (const uint4*)P2, c, h, B, F, r,
              tau, n_hot, mask, logits);
  return hipGetLastError();
}

// stage-2 shape for rank r: lanes per P2 row (8 .. SFFN_Z_LPR_MAX) and chunk rounds per lane, as 100 lpr + rounds
int z_shape(int r) {
  const int cpr = r / 8;
  int lpr = 8;
  while (lpr * 2 <= cpr && lpr < SFFN_Z_LPR_MAX) lpr *= 2;
  int rounds = 1;
  while (rounds * lpr < cpr) rounds *= 2;   // cpr <= 128: at most 16 rounds of 8 lanes
  return lpr * 100 + rounds;
}

template <int TB>
hipError_t dispatch_zb(const void* P2, const float* c, const float* h, int B, int F, int r, float tau, int n_hot,
                       uint64_t* mask, float* logits, hipStream_t st) {
#define ZB(L, R) return launch_zb<L, R, TB>(P2, c, h, B, F, r, tau, n_hot, mask, logits, st)
  switch (z_shape(r)) {
    case 801: ZB(8, 1);
    case 802: ZB(8, 2);
    case 804: ZB(8, 4);
    case 808: ZB(8, 8);
    case 816: ZB(8, 16);
    case 1601: ZB(16, 1);
    case 1602: ZB(16, 2);
    case 1604: ZB(16, 4);
    case 1608: ZB(16, 8);
    case 3201: ZB(32, 1);
    case 3202: ZB(32, 2);
    case 3204: ZB(32, 4);
    case 6401: ZB(64, 1);
    case 6402: ZB(64, 2);
    default: return hipErrorInvalidValue;
  }
#undef ZB
}

}  // namespace

hipError_t sffn_launch_predict(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D,
                               int F, int r, float tau, int n_hot, uint64_t* mask, float* logits, float* hbuf,
                               hipStream_t st) {
  if (B != 1) return hipErrorInvalidValue;   // batches of several tokens take the matrix-core kernels
  const int nch = (D / 8 + NTH - 1) / NTH;   // 16-byte chunks per thread (D <= 16384: at most 8)
  hipError_t e;
  if (nch <= 1) e = launch_h<1>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 2) e = launch_h<2>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 3) e = launch_h<3>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 4) e = launch_h<4>(P1, x, x_norm, B, D, r, hbuf, st);
  else if (nch <= 6) e = launch_h<6>(P1, x, x_norm, B, D, r, hbuf, st);
  else e = launch_h<8>(P1, x, x_norm, B, D, r, hbuf, st);
  if (e != hipSuccess) return e;
  switch (z_shape(r)) {
    case 801: return launch_z<8, 1>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 802: return launch_z<8, 2>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 804: return launch_z<8, 4>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 808: return launch_z<8, 8>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 816: return launch_z<8, 16>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 1601: return launch_z<16, 1>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 1602: return launch_z<16, 2>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 1604: return launch_z<16, 4>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 1608: return launch_z<16, 8>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 3201: return launch_z<32, 1>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 3202: return launch_z<32, 2>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 3204: return launch_z<32, 4>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 6401: return launch_z<64, 1>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    case 6402: return launch_z<64, 2>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
    default: return hipErrorInvalidValue;
  }
}

// Stage 1 alone for one token: h[j] (fp32, [r]) with the optional normalisation folded in.
hipError_t sffn_launch_predict_h(const void* P1, const float* x, int x_norm, int D, int r, float* hbuf,
                                 hipStream_t st) {
  const int nch = (D / 8 + NTH - 1) / NTH;
  if (nch <= 1) return launch_h<1>(P1, x, x_norm, 1, D, r, hbuf, st);
  if (nch <= 2) return launch_h<2>(P1, x, x_norm, 1, D, r, hbuf, st);
  if (nch <= 3) return launch_h<3>(P1, x, x_norm, 1, D, r, hbuf, st);
  if (nch <= 4) return launch_h<4>(P1, x, x_norm, 1, D, r, hbuf, st);
  if (nch <= 6) return launch_h<6>(P1, x, x_norm, 1, D, r, hbuf, st);
  return launch_h<8>(P1, x, x_norm, 1, D, r, hbuf, st);
}

// Stage 1 for 2 <= B <= 8 tokens: h[b][j] (fp32, [B][r]) with the optional per-token normalisation folded in.
hipError_t sffn_launch_predict_hb(const void* P1, const float* x, int x_norm, int B, int D, int r, float* hbuf,
                                  hipStream_t st) {
  if (B < 2 || B > 8) return hipErrorInvalidValue;
  const int nch = (D / 8 + NTB - 1) / NTB;   // 16-byte chunks per thread (D <= 16384: at most 4)
  if (nch <= 1) {
    if (B <= 2) return launch_hb<1, 2>(P1, x, x_norm, B, D, r, hbuf, st);
    if (B <= 4) return launch_hb<1, 4>(P1, x, x_norm, B, D, r, hbuf, st);
    return launch_hb<1, 8>(P1, x, x_norm, B, D, r, hbuf, st);
  }
  if (nch <= 2) {
    if (B <= 2) return launch_hb<2, 2>(P1, x, x_norm, B, D, r, hbuf, st);
    if (B <= 4) return launch_hb<2, 4>(P1, x, x_norm, B, D, r, hbuf, st);
    return launch_hb<2, 8>(P1, x, x_norm, B, D, r, hbuf, st);
  }
  if (B <= 2) return launch_hb<4, 2>(P1, x, x_norm, B, D, r, hbuf, st);
  return launch_hb<4, 4>(P1, x, x_norm, B, D, r, hbuf, st);
}

// Stage 2 for 2 <= B <= 4 tokens: logits [B][F] (optional) and the union mask from h [B][r]. (At 8 tokens the
// matrix-core kernel is the faster one.)
hipError_t sffn_launch_predict_zb(const void* P2, const float* c, const float* hbuf, int B, int F, int r, float tau,
                                  int n_hot, uint64_t* mask, float* logits, hipStream_t st) {
  if (B < 2 || B > 4) return hipErrorInvalidValue;
  if (B <= 2) return dispatch_zb<2>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
  return dispatch_zb<4>(P2, c, hbuf, B, F, r, tau, n_hot, mask, logits, st);
}
