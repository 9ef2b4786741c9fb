// Neuron-aware sparse FFN with Q4_0 weights, VALU path (decode batches, B <= 8 with B * D <= 16384).
//
// PowerInfer pages, Indonesian digest, "Quantization": INT4 Q4_0 weights are supported and optimised. Reading
// used here: blocks of 32 consecutive weights along d_model in every neuron's row of W_gate / W_up / W_downT,
// w = (q - 8) * s, q in 0..15, one fp16 scale per block. Byte i of a block's 16 nibble bytes holds element i
// (low nibble) and element 16 + i (high nibble).
//
// Dequantisation happens in registers: nibbles are split with two masks per dword, converted with
// byte-to-float conversions, and the "- 8" is folded out of the inner loop (sum (q - 8) x = sum q x - 8 sum x,
// with the per-block sums of x precomputed in LDS for the row gather, and sum of a * s carried per lane for the
// column gather). Every product is exact in fp32 before accumulation.
//
// Work split and compaction are those of the fp16 path: k_upgate_q4 (mask -> ids, row gather, fused
// activation) and k_down_q4 (each block owns 256 output columns = 8 Q4 blocks of every W_downT row).
#include "common.h"

using namespace sffn;

namespace {

constexpr int NT_UP = 256;
constexpr int X_LDS_FLOATS = 16384;

__device__ __forceinline__ float q4_block_dot(const uint4& nib, const float* __restrict__ xb /* 32 floats in LDS */) {
  const uint32_t wds[4] = {nib.x, nib.y, nib.z, nib.w};
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = wds[k] & 0x0F0F0F0Fu, hi = (wds[k] >> 4) & 0x0F0F0F0Fu;
    const float4 xl = *reinterpret_cast<const float4*>(xb + 4 * k);
    const float4 xh = *reinterpret_cast<const float4*>(xb + 16 + 4 * k);
    s = fmaf((float)(lo & 0xFF), xl.x, s);
    s = fmaf((float)((lo >> 8) & 0xFF), xl.y, s);
    s = fmaf((float)((lo >> 16) & 0xFF), xl.z, s);
    s = fmaf((float)(lo >> 24), xl.w, s);
    s = fmaf((float)(hi & 0xFF), xh.x, s);
    s = fmaf((float)((hi >> 8) & 0xFF), xh.y, s);
    s = fmaf((float)((hi >> 16) & 0xFF), xh.z, s);
    s = fmaf((float)(hi >> 24), xh.w, s);
  }
  return s;
}

template <int B, int ACT, int NQ>
__global__ __launch_bounds__(NT_UP) void k_upgate_q4(const uint4* __restrict__ qg, const _Float16* __restrict__ sg,
                                                     const float* __restrict__ bg, const uint4* __restrict__ qu,
                                                     const _Float16* __restrict__ su, const float* __restrict__ bu,
                                                     const float* __restrict__ x, int x_rms, int D, int F,
                                                     const uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                     int32_t* __restrict__ n_active, float* __restrict__ abuf) {
  extern __shared__ float lds[];
  const int nblk = D >> 5;                                   // Q4 blocks per row
  float* xs = lds;                                           // [B, D]
  float* xsum = xs + (size_t)B * D;                          // [B, nblk]
  float* red = xsum + (size_t)B * nblk;                      // [(NT/64) * B]
  int* roff = reinterpret_cast<int*>(red + (NT_UP / 64) * B);  // [NT_UP]
  int* tmp = roff + NT_UP;
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NT_UP - 1) / NT_UP;
  const int n = mask_prefix<NT_UP>(mask, nw, F, wpt, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int NW = gridDim.x * (NT_UP / 64);
  const int g0 = blockIdx.x * (NT_UP / 64);
  if (g0 >= n) return;
  stage_x<NT_UP>(x, B, D, x_rms, xs, red);
  for (int t = threadIdx.x; t < B * nblk; t += NT_UP) {
    const float* p = xs + (size_t)(t / nblk) * D + 32 * (t % nblk);
    float s = 0.f;
    for (int e = 0; e < 32; ++e) s += p[e];
    xsum[t] = s;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  for (int i = g0 + (threadIdx.x >> 6); i < n; i += NW) {
    const int id = locate(mask, roff, NT_UP, wpt, nw, F, i);
    if (lane == 0) active[i] = id;
    uint4 nu[NQ], ng[NQ];
    float fu[NQ], fg[NQ];
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int c = lane + 64 * m;
      const bool ok = c < nblk;
      const size_t o = (size_t)id * nblk + c;
      nu[m] = ok ? qu[o] : make_uint4(0u, 0u, 0u, 0u);
      fu[m] = ok ? (float)su[o] : 0.f;
      if (ACT == 1) {
        ng[m] = ok ? qg[o] : make_uint4(0u, 0u, 0u, 0u);
        fg[m] = ok ? (float)sg[o] : 0.f;
      }
    }
    float au[B], ag[B];
#pragma unroll
    for (int b = 0; b < B; ++b) { au[b] = 0.f; ag[b] = 0.f; }
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int c = lane + 64 * m;
      if (c < nblk) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float* xb = xs + (size_t)b * D + 32 * c;
          const float xsb = xsum[b * nblk + c];
          au[b] = fmaf(fu[m], q4_block_dot(nu[m], xb) - 8.f * xsb, au[b]);
          if (ACT == 1) ag[b] = fmaf(fg[m], q4_block_dot(ng[m], xb) - 8.f * xsb, ag[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float u = wave_sum(au[b]);
      float a;
      if (ACT == 1) {
        const float g = wave_sum(ag[b]) + (bg ? bg[id] : 0.f);
        a = fmaxf(g, 0.f) * u;
      } else {
        a = fmaxf(u + (bu ? bu[id] : 0.f), 0.f);
      }
      if (lane == 0) abuf[(size_t)i * B + b] = a;
    }
  }
}

constexpr int NT_DN = 1024;
constexpr int QSW = 256;               // output columns per block (8 Q4 blocks of each row)
template <int B> struct QD {
  static constexpr int CPL = B <= 2 ? 32 : 16;   // columns per lane
  static constexpr int LPR = QSW / CPL;          // lanes per row slice
  static constexpr int RPI = 64 / LPR;           // rows per wave instruction
  static constexpr int CH = B == 1 ? 4096 : 8192 / B;
};
constexpr int QDU = 4;                 // row slices in flight per lane

template <int B>
__global__ __launch_bounds__(NT_DN) void k_down_q4(const uint8_t* __restrict__ qd, const _Float16* __restrict__ sd,
                                                   const int32_t* __restrict__ active,
                                                   const int32_t* __restrict__ n_active,
                                                   const float* __restrict__ abuf, int D, float* __restrict__ y) {
  constexpr int CPL = QD<B>::CPL, LPR = QD<B>::LPR, RPI = QD<B>::RPI, CH = QD<B>::CH;
  constexpr int NWV = NT_DN / 64;
  __shared__ int ids[CH];
  __shared__ float as[CH * B];
  __shared__ float red[NWV * B * 64];     // per wave: B x 64 columns per pass
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nblk = D >> 5;
  const int rsub = lane / LPR, lsub = lane % LPR;
  const int col0 = blockIdx.x * QSW + lsub * CPL;       // first column of this lane
  const int qblk = col0 >> 5;                           // Q4 block of this lane
  const int half = (CPL == 16) ? ((col0 >> 4) & 1) : 0; // which 8-byte half (16-column lanes)
  const bool colok = col0 < D;
  const int n = *n_active;
  float acc[B][CPL];
  float sas[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    sas[b] = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[b][e] = 0.f;
  }
  for (int r0 = 0; r0 < n; r0 += CH) {
    const int nr = min(CH, n - r0);
    __syncthreads();
    for (int i = threadIdx.x; i < nr; i += NT_DN) ids[i] = active[r0 + i];
    for (int i = threadIdx.x; i < nr * B; i += NT_DN) as[i] = abuf[(size_t)r0 * B + i];
    __syncthreads();
    for (int base = w * RPI + rsub; base < nr; base += NWV * RPI * QDU) {
      uint32_t nib[QDU][CPL / 8];
      float sc[QDU];
#pragma unroll
      for (int u = 0; u < QDU; ++u) {
        const int i = base + u * NWV * RPI;
        const bool ok = i < nr && colok;
        const size_t row = ok ? (size_t)ids[i] : 0;
        if (CPL == 32) {
          const uint4 v = ok ? *reinterpret_cast<const uint4*>(qd + row * (D >> 1) + (size_t)qblk * 16)
                             : make_uint4(0u, 0u, 0u, 0u);
          nib[u][0] = v.x; nib[u][1] = v.y; nib[u][2] = v.z; nib[u][3] = v.w;
        } else {
          const uint2 v = ok ? *reinterpret_cast<const uint2*>(qd + row * (D >> 1) + (size_t)qblk * 16 + half * 8)
                             : make_uint2(0u, 0u);
          nib[u][0] = v.x; nib[u][1] = v.y;
        }
        sc[u] = ok ? (float)sd[row * nblk + qblk] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < QDU; ++u) {
        const int i = base + u * NWV * RPI;
        if (i < nr) {
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const float as_ = as[i * B + b] * sc[u];
            sas[b] += as_;
#pragma unroll
            for (int k = 0; k < CPL / 8; ++k) {
              const uint32_t lo = nib[u][k] & 0x0F0F0F0Fu, hi = (nib[u][k] >> 4) & 0x0F0F0F0Fu;
              // lane-local element order: [0, CPL/2) low nibbles, [CPL/2, CPL) high nibbles
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                acc[b][4 * k + j] = fmaf(as_, (float)((lo >> (8 * j)) & 0xFF), acc[b][4 * k + j]);
                acc[b][CPL / 2 + 4 * k + j] = fmaf(as_, (float)((hi >> (8 * j)) & 0xFF), acc[b][CPL / 2 + 4 * k + j]);
              }
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float v = fmaf(-8.f, sas[b], acc[b][e]);
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, WAVE);
      acc[b][e] = v;
    }
  // lane-local element e -> column: low half e -> col0 + e (CPL=32) / col0 + e (CPL=16, e < 8);
  // high half e -> the element 16 positions later in the Q4 block
  auto col_of = [&](int e) -> int {
    if (CPL == 32) return e < 16 ? col0 + e : col0 + 16 + (e - 16) - 16 + 16;  // col0 + e for both halves
    return e < 8 ? (qblk * 32 + half * 8 + e) : (qblk * 32 + 16 + half * 8 + (e - 8));
  };
  float* red_w = red + (size_t)w * B * 64;
  for (int pass = 0; pass < QSW / 64; ++pass) {
    // columns [pass*64, pass*64+64) of the block's 256
    __syncthreads();
    if (lane < LPR) {
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const int cc = col_of(e) - blockIdx.x * QSW - pass * 64;
          if (cc >= 0 && cc < 64) red_w[b * 64 + cc] = acc[b][e];
        }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < B * 64; t += NT_DN) {
      const int b = t / 64, cc = t % 64;
      float s = 0.f;
      for (int ww = 0; ww < NWV; ++ww) s += red[(size_t)ww * B * 64 + b * 64 + cc];
      const int d = blockIdx.x * QSW + pass * 64 + cc;
      if (d < D) y[(size_t)b * D + d] = s;
    }
  }
}

template <int B, int ACT, int NQ>
hipError_t launch_up(const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu, const void* su,
                     const float* bu, const float* x, int x_rms, int D, int F, const uint64_t* mask, int32_t* active,
                     int32_t* n_active, float* abuf, hipStream_t st) {
  const int nblk = D / 32;
  const size_t lds = ((size_t)B * D + (size_t)B * nblk + (NT_UP / 64) * B) * sizeof(float) +
                     (NT_UP + NT_UP / 64 + 1) * sizeof(int);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_upgate_q4<B, ACT, NQ>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, X_LDS_FLOATS * 4 + 16384);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int grid = std::max(1, std::min((F + 3) / 4, 512));
  hipLaunchKernelGGL((k_upgate_q4<B, ACT, NQ>), dim3(grid), dim3(NT_UP), lds, st, (const uint4*)qg,
                     (const _Float16*)sg, bg, (const uint4*)qu, (const _Float16*)su, bu, x, x_rms, D, F, mask, active,
                     n_active, abuf);
  return hipGetLastError();
}

template <int B, int ACT>
hipError_t dispatch_up(int nq, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu, const void* su,
                       const float* bu, const float* x, int x_rms, int D, int F, const uint64_t* mask, int32_t* active,
                       int32_t* n_active, float* abuf, hipStream_t st) {
#define UPQ(N) return launch_up<B, ACT, N>(qg, sg, bg, qu, su, bu, x, x_rms, D, F, mask, active, n_active, abuf, st)
  if (nq <= 1) UPQ(1);
  if (nq <= 2) UPQ(2);
  if (nq <= 4) UPQ(4);
  UPQ(8);
#undef UPQ
}

template <int B>
hipError_t forward_b(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu, const void* su,
                     const float* bu, const uint8_t* qd, const void* sd, const float* x, int x_rms, int D, int F,
                     const uint64_t* mask, int32_t* active, int32_t* n_active, float* y, float* abuf, hipStream_t st) {
  const int nq = (D / 32 + 63) / 64;
  hipError_t e = act == 1
                     ? dispatch_up<B, 1>(nq, qg, sg, bg, qu, su, bu, x, x_rms, D, F, mask, active, n_active, abuf, st)
                     : dispatch_up<B, 0>(nq, qg, sg, bg, qu, su, bu, x, x_rms, D, F, mask, active, n_active, abuf, st);
  if (e != hipSuccess) return e;
  const int grid = (D + QSW - 1) / QSW;
  hipLaunchKernelGGL(k_down_q4<B>, dim3(grid), dim3(NT_DN), 0, st, qd, (const _Float16*)sd, active, n_active, abuf, D,
                     y);
  return hipGetLastError();
}

}  // namespace

hipError_t sffn_launch_forward_q4(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu,
                                  const void* su, const float* bu, const uint8_t* qd, const void* sd, const float* x,
                                  int x_rms, int B, int D, int F, const uint64_t* mask, int32_t* active,
                                  int32_t* n_active, float* y, float* abuf, hipStream_t st) {
  switch (B) {
    case 1: return forward_b<1>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    case 2: return forward_b<2>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    case 4: return forward_b<4>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    case 8: return forward_b<8>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    default: return hipErrorInvalidValue;
  }
}
