// Neuron-aware sparse FFN, fp16 weights, VALU path (decode batches, B <= 8 with B * D <= 16384).
//
// PowerInfer pages, Turkish article, "Neuron-aware operator" and "Online stage": the operator reads only the
// rows and columns of the weight matrices that belong to predicted-active neurons and never builds a dense
// copy. Here a neuron k owns row k of W_gate / W_up and row k of W_downT (= column k of W_down), all in the
// caller's stored neuron order.
//
// Kernel 1 (k_upgate): compaction + row gather + fused activation.
//   Every block turns the predictor's mask words into prefix offsets (popcounts, block scan). Wave g then
//   takes dense indices g, g + NW, ...: it finds the word holding the i-th set bit (binary search over the
//   per-thread range offsets), picks the bit with a wavefront ballot over lane ranks, writes active[i], and
//   reads that neuron's gate/up rows with every 16-byte load in flight before the first use. The row dot
//   products are reduced across the wave and the activation is applied in registers; a[i, b] goes to the
//   workspace.
// Kernel 2 (k_down): column gather. Each block owns SW = 64 output columns (128 bytes of every W_downT row)
//   and walks all active rows, so no cross-block reduction is needed: (id, a) pairs are staged in LDS,
//   groups of 8 lanes read one row slice with 16-byte loads, partial sums are reduced across lanes and then
//   across waves through LDS.
#include "common.h"

using namespace sffn;

namespace {

constexpr int NT_UP = 256;
constexpr int X_LDS_FLOATS = 16384;

template <int B, int ACT, int NCH>
__global__ __launch_bounds__(NT_UP) void k_upgate(const uint4* __restrict__ Wg, const float* __restrict__ bg,
                                                  const uint4* __restrict__ Wu, const float* __restrict__ bu,
                                                  const float* __restrict__ x, int x_rms, int D, int F,
                                                  const uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                  int32_t* __restrict__ n_active, float* __restrict__ abuf) {
  extern __shared__ float lds[];
  float* xs = lds;                                         // [B, D]
  float* red = lds + (size_t)B * D;                        // [(NT/64) * B]
  int* roff = reinterpret_cast<int*>(red + (NT_UP / 64) * B);  // [NT_UP]
  int* tmp = roff + NT_UP;                                 // [NT_UP/64 + 1]
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NT_UP - 1) / NT_UP;
  const int n = mask_prefix<NT_UP>(mask, nw, F, wpt, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int NW = gridDim.x * (NT_UP / 64);
  const int g0 = blockIdx.x * (NT_UP / 64);
  if (g0 >= n) return;  // block-uniform: no work for any wave of this block
  stage_x<NT_UP>(x, B, D, x_rms, xs, red);
  const int lane = threadIdx.x & 63;
  const int nc = D >> 3;
  for (int i = g0 + (threadIdx.x >> 6); i < n; i += NW) {
    const int id = locate(mask, roff, NT_UP, wpt, nw, F, i);
    if (lane == 0) active[i] = id;
    uint4 wu[NCH], wg[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = lane + 64 * m;
      const bool ok = c < nc;
      wu[m] = ok ? Wu[(size_t)id * nc + c] : make_uint4(0u, 0u, 0u, 0u);
      if (ACT == 1) wg[m] = ok ? Wg[(size_t)id * nc + c] : make_uint4(0u, 0u, 0u, 0u);
    }
    float au[B], ag[B];
#pragma unroll
    for (int b = 0; b < B; ++b) { au[b] = 0.f; ag[b] = 0.f; }
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = lane + 64 * m;
      if (c < nc) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float4* xp = reinterpret_cast<const float4*>(xs + (size_t)b * D + 8 * c);
          const float4 x0 = xp[0], x1 = xp[1];
          const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          au[b] += dot8(wu[m], xv);
          if (ACT == 1) ag[b] += dot8(wg[m], xv);
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

constexpr int NT_DN = 1024;     // 16 waves
constexpr int SW = 64;          // output columns per block (128-byte row slices)
constexpr int DLPR = SW / 8;    // lanes per row slice (8)
constexpr int DRPI = 64 / DLPR; // rows per wave instruction (8)
constexpr int DU = 8;           // row slices in flight per lane
// rows staged in LDS per round: ids [CH] + activations [CH * B] + reduction [16 * B * SW] fit in ~72 KB
template <int B> struct DownCH { static constexpr int v = B == 1 ? 4096 : 8192 / B; };

template <int B>
__global__ __launch_bounds__(NT_DN) void k_down(const uint4* __restrict__ WdT, const int32_t* __restrict__ active,
                                                const int32_t* __restrict__ n_active, const float* __restrict__ abuf,
                                                int D, float* __restrict__ y) {
  constexpr int CH = DownCH<B>::v;
  __shared__ int ids[CH];
  __shared__ float as[CH * B];
  __shared__ float red[(NT_DN / 64) * B * SW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nc = D >> 3;
  const int cchunk = blockIdx.x * DLPR + (lane % DLPR);  // 16-byte chunk index of this lane's 8 columns
  const bool colok = cchunk < nc;
  const int rsub = lane / DLPR;
  const int n = *n_active;
  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;

  for (int r0 = 0; r0 < n; r0 += CH) {
    const int nr = min(CH, n - r0);
    __syncthreads();
    for (int i = threadIdx.x; i < nr; i += NT_DN) ids[i] = active[r0 + i];
    for (int i = threadIdx.x; i < nr * B; i += NT_DN) as[i] = abuf[(size_t)r0 * B + i];
    __syncthreads();
    for (int base = w * DRPI + rsub; base < nr; base += (NT_DN / 64) * DRPI * DU) {
      uint4 wv[DU];
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const int i = base + u * (NT_DN / 64) * DRPI;
        wv[u] = (i < nr && colok) ? WdT[(size_t)ids[i] * nc + cchunk] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const int i = base + u * (NT_DN / 64) * DRPI;
        if (i < nr) {
          float wf[8];
          f16x8_to_f32(wv[u], wf);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const float av = as[i * B + b];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[b][e] = fmaf(av, wf[e], acc[b][e]);
          }
        }
      }
    }
  }
  // reduce over the DRPI row groups of the wave (lanes with equal lane % DLPR)
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[b][e];
#pragma unroll
      for (int o = DLPR; o < 64; o <<= 1) v += __shfl_xor(v, o, WAVE);
      acc[b][e] = v;
    }
  if (lane < DLPR) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(w * B + b) * SW + lane * 8 + e] = acc[b][e];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < B * SW; t += NT_DN) {
    const int b = t / SW, col = t % SW;
    float s = 0.f;
    for (int ww = 0; ww < NT_DN / 64; ++ww) s += red[(ww * B + b) * SW + col];
    const int d = blockIdx.x * SW + col;
    if (d < D) y[(size_t)b * D + d] = s;
  }
}

template <int B, int ACT, int NCH>
hipError_t launch_up(const void* Wg, const float* bg, const void* Wu, const float* bu, const float* x, int x_rms, int D,
                     int F, const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf, hipStream_t st) {
  const size_t lds = ((size_t)B * D + (NT_UP / 64) * B) * sizeof(float) + (NT_UP + NT_UP / 64 + 1) * sizeof(int);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_upgate<B, ACT, NCH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       X_LDS_FLOATS * 4 + 8192);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int grid = std::max(1, std::min((F + 3) / 4, 512));
  hipLaunchKernelGGL((k_upgate<B, ACT, NCH>), dim3(grid), dim3(NT_UP), lds, st, (const uint4*)Wg, bg,
                     (const uint4*)Wu, bu, x, x_rms, D, F, mask, active, n_active, abuf);
  return hipGetLastError();
}

template <int B, int ACT>
hipError_t dispatch_up(int nch, const void* Wg, const float* bg, const void* Wu, const float* bu, const float* x,
                       int x_rms, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf,
                       hipStream_t st) {
#define UP(N) return launch_up<B, ACT, N>(Wg, bg, Wu, bu, x, x_rms, D, F, mask, active, n_active, abuf, st)
  if (nch <= 1) UP(1);
  if (nch <= 2) UP(2);
  if (nch <= 4) UP(4);
  if (nch <= 8) UP(8);
  if (nch <= 10) UP(10);
  if (nch <= 16) UP(16);
  UP(32);
#undef UP
}

template <int B>
hipError_t launch_down(const void* WdT, const int32_t* active, const int32_t* n_active, const float* abuf, int D,
                       float* y, hipStream_t st) {
  const int grid = (D + SW - 1) / SW;
  hipLaunchKernelGGL(k_down<B>, dim3(grid), dim3(NT_DN), 0, st, (const uint4*)WdT, active, n_active, abuf, D, y);
  return hipGetLastError();
}

template <int B>
hipError_t forward_b(int act, const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                     const float* x, int x_rms, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active,
                     float* y, float* abuf, hipStream_t st) {
  const int nch = (D / 8 + 63) / 64;
  hipError_t e = act == 1 ? dispatch_up<B, 1>(nch, Wg, bg, Wu, bu, x, x_rms, D, F, mask, active, n_active, abuf, st)
                          : dispatch_up<B, 0>(nch, Wg, bg, Wu, bu, x, x_rms, D, F, mask, active, n_active, abuf, st);
  if (e != hipSuccess) return e;
  return launch_down<B>(WdT, active, n_active, abuf, D, y, st);
}

}  // namespace

hipError_t sffn_launch_forward(int act, const void* Wg, const float* bg, const void* Wu, const float* bu,
                               const void* WdT, const float* x, int x_rms, int B, int D, int F, const uint64_t* mask,
                               int32_t* active, int32_t* n_active, float* y, float* abuf, hipStream_t st) {
  switch (B) {
    case 1: return forward_b<1>(act, Wg, bg, Wu, bu, WdT, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    case 2: return forward_b<2>(act, Wg, bg, Wu, bu, WdT, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    case 4: return forward_b<4>(act, Wg, bg, Wu, bu, WdT, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    case 8: return forward_b<8>(act, Wg, bg, Wu, bu, WdT, x, x_rms, D, F, mask, active, n_active, y, abuf, st);
    default: return hipErrorInvalidValue;
  }
}
