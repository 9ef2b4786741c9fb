// Neuron-aware sparse FFN, fp16 weights, VALU path (decode batches, B <= 8 with B * D <= 16384).
//
// PowerInfer pages, Turkish article, "Neuron-aware operator" and "Online stage": the operator reads only the
// rows and columns of the weight matrices that belong to predicted-active neurons and never builds a dense
// copy. Here a neuron k owns row k of W_gate / W_up and row k of W_downT (= column k of W_down), all in the
// caller's stored neuron order.
//
// Kernel 1 (k_upgate): compaction + row gather + fused activation, two dependent memory round trips.
//   Round 1: every thread loads its mask words and its share of x, both before either is used. Popcounts and a
//   block scan give prefix offsets over thread ranges. Dense index i goes to block i % G, wave (i / G) % 4, so
//   the active rows spread over every block (and CU) evenly; blocks with no index stop here. Each wave finds
//   the word holding its first i-th set bit (binary search over range offsets, then a wavefront ballot over
//   lane ranks) and, round 2, issues that neuron's gate/up row loads (16 bytes per lane, all in flight
//   together) before x is normalised and staged in LDS, so the staging hides under the row fetch. Row dot
//   products are reduced across the wave, the activation is applied in registers, and a[i, b] goes to the
//   workspace at the dense index i together with active[i].
// Kernel 2 (k_down): column gather, two dependent round trips. Each block owns SW output columns (2*SW bytes
//   of every W_downT row) and walks all active rows, so no cross-block reduction is needed and y is written
//   once, deterministically. Round 1: n_active and the ids that kernel 1 wrote to active[] (issued together,
//   the ids speculatively); round 2: groups of SW/8 lanes read one row slice with 16-byte loads together with
//   a[i, b] (dense, coalesced), DU rows per lane in flight. Partial sums are reduced across lanes, then across
//   waves through LDS.
#include "common.h"

using namespace sffn;

namespace {

#ifndef SFFN_UP_NT
#define SFFN_UP_NT 256           // threads per block of the row gather
#endif
#ifndef SFFN_UP_GRID
#define SFFN_UP_GRID 512         // blocks of the row gather (dense index i -> block i % grid)
#endif
constexpr int NT_UP = SFFN_UP_NT;
#ifndef SFFN_DOWN_XCD
#define SFFN_DOWN_XCD 1          // XCD-aware order of the column slices of the column gather
#endif
constexpr int WMAX = 2;           // mask words per thread kept in registers / LDS (F <= 32768; larger F reads them from memory)

template <int B, int ACT, int NCH>
__global__ __launch_bounds__(NT_UP) void k_upgate(const uint4* __restrict__ Wg, const float* __restrict__ bg,
                                                  const uint4* __restrict__ Wu, const float* __restrict__ bu,
                                                  const float* __restrict__ x, int x_norm, int D, int F,
                                                  const uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                  int32_t* __restrict__ n_active, float* __restrict__ abuf) {
  extern __shared__ uint64_t lds64[];
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NT_UP - 1) / NT_UP;
  const bool words_lds = wpt <= WMAX;
  uint64_t* wl = lds64;                                                       // [nw] if words_lds
  int* roff = reinterpret_cast<int*>(wl + (words_lds ? ((nw + 1) & ~1) : 0));  // [NT_UP], 16-byte aligned
  int* tmp = roff + NT_UP;                                                    // [NT_UP/64 + 1]
  float* xs = reinterpret_cast<float*>(tmp + NT_UP / 64 + 4);                 // [B, D]
  float* red = xs + (size_t)B * D;                                            // [2 * (NT/64) * B]
  const int lane = threadIdx.x & 63;
  const int nc = D >> 3;
  const int n4 = (B * D) >> 2;
  constexpr int XPT = (128 * B * NCH + NT_UP - 1) / NT_UP;   // float4 of x per thread: B * D / 4 <= 128 * B * NCH

  // round 1: x and the mask words, all loads issued before any use
  float4 xv4[XPT];
  stage_load<NT_UP, XPT>(x, n4, xv4);
  const float x0 = x[0];                   // shift for the single-pass statistics (B == 1)
  const int n = mask_prefix<NT_UP, WMAX>(mask, nw, F, wpt, words_lds ? wl : nullptr, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int G = gridDim.x;
  if ((int)blockIdx.x >= n) return;  // block-uniform: no dense index maps to this block
  const uint64_t* words = words_lds ? wl : mask;
  const uint32_t wbytes = (uint32_t)F * (uint32_t)D * 2u;
  const Buf bwu(Wu, wbytes);
  const Buf bwg(ACT == 1 ? (const void*)Wg : (const void*)Wu, ACT == 1 ? wbytes : 0u);
  const float* bp = ACT == 1 ? bg : bu;
  const Buf bbias(bp ? (const void*)bp : (const void*)Wu, bp ? (uint32_t)F * 4u : 0u);   // no bias: 0
  const int NW = G * (NT_UP / 64);
  int i = (int)blockIdx.x + G * (threadIdx.x >> 6);
  uint4 wu[NCH], wg[NCH];
  float bias = 0.f;
  int id = 0;
  auto issue = [&]() {  // round 2 for dense index i: the neuron's rows and bias
    id = locate(words, roff, NT_UP, wpt, nw, F, i);
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = lane + 64 * m;
      const uint32_t o = boff(c < nc, ((uint32_t)id * nc + c) * 16u);
      wu[m] = bwu.ld16(o);
      if (ACT == 1) wg[m] = bwg.ld16(o);
    }
    bias = bbias.ldf((uint32_t)id * 4u);
  };
  const bool have = i < n;            // wave-uniform
  if (have) issue();
  // x: normalised and staged while the first rows are in flight
  if constexpr (B == 1) {
    if (x_norm) block_norm_regs<NT_UP, XPT>(xv4, n4, x0, red);
    stage_store<NT_UP, XPT>(xs, n4, xv4);
    __syncthreads();
  } else {
    stage_store<NT_UP, XPT>(xs, n4, xv4);
    if (x_norm) stage_norm<NT_UP>(xs, B, D, red);
    else __syncthreads();
  }
  if (!have) return;
  for (;;) {
    if (lane == 0) active[i] = id;
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
          const float4 xa = xp[0], xb = xp[1];
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
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
        const float g = wave_sum(ag[b]) + bias;
        a = fmaxf(g, 0.f) * u;
      } else {
        a = fmaxf(u + bias, 0.f);
        if (ACT == 2) a *= a;
      }
      if (lane == 0) abuf[(size_t)i * B + b] = a;
    }
    i += NW;
    if (i >= n) break;
    issue();
  }
}

// Column gather: B tokens, SW columns per block, NT threads, DU row slices in flight per lane.
template <int B>
struct DownCfg;
template <> struct DownCfg<1> { static constexpr int NT = 512, DU = 16; };
template <> struct DownCfg<2> { static constexpr int NT = 512, DU = 16; };
template <> struct DownCfg<4> { static constexpr int NT = 512, DU = 12; };
template <> struct DownCfg<8> { static constexpr int NT = 512, DU = 8; };

// One pass of the column gather over rows k0 + w * RPI + rsub + u * NWV * RPI (u < DU): every row-slice and
// activation load is issued before the first multiply-add (the scheduling barrier keeps the compiler from
// interleaving them, which would leave only a few loads in flight per lane).
template <int B, int LPR, int RPI, int NWV, int DU>
__device__ __forceinline__ void down_pass(const Buf& bwd, const Buf& ba, const uint32_t (&ids)[DU], int k0, int n,
                                          int w, int rsub, bool colok, int nc, int cchunk, float (&acc)[B][8]) {
  uint4 wv[DU];
  float av[DU][B];
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    const int i = k0 + w * RPI + rsub + u * NWV * RPI;
    const bool ok = i < n;
    wv[u] = bwd.ld16(boff(ok && colok, (ids[u] * nc + cchunk) * 16u));
#pragma unroll
    for (int b = 0; b < B; ++b) av[u][b] = ba.ldf(boff(ok, ((uint32_t)i * B + b) * 4u));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    float wf[8];
    f16x8_to_f32(wv[u], wf);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[b][e] = fmaf(av[u][b], wf[e], acc[b][e]);
  }
}

template <int B, int SW>
__global__ __launch_bounds__(DownCfg<B>::NT) void k_down(const uint4* __restrict__ WdT,
                                                         const int32_t* __restrict__ active,
                                                         const int32_t* __restrict__ n_active,
                                                         const float* __restrict__ abuf, int D, int F,
                                                         float* __restrict__ y) {
  constexpr int NT = DownCfg<B>::NT, DU = DownCfg<B>::DU;
  constexpr int LPR = SW / 8;                        // lanes per row slice (16 bytes each)
  constexpr int RPI = 64 / LPR;                      // rows per wave instruction
  constexpr int NWV = NT / 64;
  constexpr int STRIDE = NWV * RPI * DU;             // rows per block pass
  __shared__ float red[NWV * B * SW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nc = D >> 3;
  const int slice = SFFN_DOWN_XCD ? xcd_slice(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  if (slice * SW >= D) return;                          // block-uniform: padding of the grid to 8 * per
  const int cchunk = slice * LPR + (lane % LPR);        // 16-byte chunk of this lane's 8 columns
  const bool colok = cchunk < nc;
  const int rsub = lane / LPR;
  const Buf bwd(WdT, (uint32_t)F * (uint32_t)D * 2u);
  const Buf ba(abuf, (uint32_t)F * (uint32_t)B * 4u);
  const Buf bid(active, (uint32_t)F * 4u);
  const Buf bn(n_active, 4u);
  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;

  auto load_ids = [&](int k0, uint32_t (&ids)[DU]) {  // speculative, bounded by F
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int i = k0 + w * RPI + rsub + u * NWV * RPI;
      ids[u] = bid.ldu(boff(i < F, (uint32_t)i * 4u));
    }
  };
  // round 1: the count and the first pass's ids together; round 2: that pass's rows and activations
  const int nraw = (int)bn.ldu(0u);
  uint32_t ids[DU];
  load_ids(0, ids);
  const int n = min(max(nraw, 0), F);
  down_pass<B, LPR, RPI, NWV, DU>(bwd, ba, ids, 0, n, w, rsub, colok, nc, cchunk, acc);
  for (int k0 = STRIDE; k0 < n; k0 += STRIDE) {       // more rows than one pass holds
    load_ids(k0, ids);
    down_pass<B, LPR, RPI, NWV, DU>(bwd, ba, ids, k0, n, w, rsub, colok, nc, cchunk, acc);
  }
  // reduce over the row groups of the wave (lanes with equal lane % LPR), then across waves
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[b][e];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, WAVE);
      acc[b][e] = v;
    }
  if (lane < LPR) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(w * B + b) * SW + lane * 8 + e] = acc[b][e];
  }
  __syncthreads();
  for (int tt = threadIdx.x; tt < B * SW; tt += NT) {
    const int b = tt / SW, col = tt % SW;
    float s = 0.f;
    for (int ww = 0; ww < NWV; ++ww) s += red[(ww * B + b) * SW + col];
    const int d = slice * SW + col;
    if (d < D) y[(size_t)b * D + d] = s;
  }
}

template <int B, int ACT, int NCH>
hipError_t launch_up(const void* Wg, const float* bg, const void* Wu, const float* bu, const float* x, int x_norm, int D,
                     int F, const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf, hipStream_t st) {
  const int nw = (F + 63) / 64;
  const int wpt = (nw + NT_UP - 1) / NT_UP;
  const size_t lds_scan = (wpt <= WMAX ? (size_t)((nw + 1) & ~1) * 8 : 0) + (NT_UP + NT_UP / 64 + 4) * sizeof(int);
  const int grid = std::max(1, std::min((F + 3) / 4, SFFN_UP_GRID));
  const size_t lds = lds_scan + ((size_t)B * D + 2 * (NT_UP / 64) * B) * sizeof(float);
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_upgate<B, ACT, NCH>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail) return hipErrorInvalidValue;
  SFFN_LAUNCH(2, (k_upgate<B, ACT, NCH>), dim3(grid), dim3(NT_UP), lds, st, (const uint4*)Wg, bg,
              (const uint4*)Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf);
  return hipGetLastError();
}

template <int B, int ACT>
hipError_t dispatch_up(int nch, const void* Wg, const float* bg, const void* Wu, const float* bu, const float* x,
                       int x_norm, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf,
                       hipStream_t st) {
#define UP(N) return launch_up<B, ACT, N>(Wg, bg, Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf, st)
  if (nch <= 1) UP(1);
  if (nch <= 2) UP(2);
  if (nch <= 4) UP(4);
  if (nch <= 8) UP(8);
  if (nch <= 10) UP(10);
  if (nch <= 16) UP(16);
  UP(32);
#undef UP
}

// Output columns per block of the column gather; with the XCD-aware slice order neighbouring slices share L2.
#ifndef SFFN_DOWN_SW
#define SFFN_DOWN_SW 32
#endif
constexpr int DOWN_SW = SFFN_DOWN_SW;

template <int B>
hipError_t launch_down(const void* WdT, const int32_t* active, const int32_t* n_active, const float* abuf, int D,
                       int F, float* y, hipStream_t st) {
  const int slices = (D + DOWN_SW - 1) / DOWN_SW;
  const int grid = SFFN_DOWN_XCD ? (slices + 7) / 8 * 8 : slices;
  SFFN_LAUNCH(3, (k_down<B, DOWN_SW>), dim3(grid), dim3(DownCfg<B>::NT), 0, st, (const uint4*)WdT, active, n_active,
              abuf, D, F, y);
  return hipGetLastError();
}

template <int B>
hipError_t forward_b(int act, const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                     const float* x, int x_norm, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active,
                     float* y, float* abuf, hipStream_t st) {
  const int nch = (D / 8 + 63) / 64;
  hipError_t e =
      act == 1   ? dispatch_up<B, 1>(nch, Wg, bg, Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf, st)
      : act == 2 ? dispatch_up<B, 2>(nch, Wg, bg, Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf, st)
                 : dispatch_up<B, 0>(nch, Wg, bg, Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf, st);
  if (e != hipSuccess) return e;
  return launch_down<B>(WdT, active, n_active, abuf, D, F, y, st);
}

}  // namespace

hipError_t sffn_launch_forward(int act, const void* Wg, const float* bg, const void* Wu, const float* bu,
                               const void* WdT, const float* x, int x_norm, int B, int D, int F, const uint64_t* mask,
                               int32_t* active, int32_t* n_active, float* y, float* abuf, hipStream_t st) {
  switch (B) {
    case 1: return forward_b<1>(act, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    case 2: return forward_b<2>(act, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    case 4: return forward_b<4>(act, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    case 8: return forward_b<8>(act, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    default: return hipErrorInvalidValue;
  }
}
