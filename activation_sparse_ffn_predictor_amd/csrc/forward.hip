// Neuron-aware sparse FFN, fp16 weights, VALU path (decode batches, B <= 8 with B * D <= 16384).
//
// PowerInfer pages, Turkish article, "Neuron-aware operator" and "Online stage": the operator reads only the
// rows and columns of the weight matrices that belong to predicted-active neurons and never builds a dense
// copy. Here a neuron k owns row k of W_gate / W_up and row k of W_downT (= column k of W_down), all in the
// caller's stored neuron order.
//
// Kernel 1 (k_upgate): compaction + row gather + fused activation, two dependent memory round trips.
//   Round 1: every thread loads its mask words and its share of x, both before either is used. Popcounts and a
//   block scan give prefix offsets over thread ranges; blocks with no work stop here. x goes to LDS (normalised
//   there if asked), the words stay in LDS. Wave g takes dense indices g, g + NW, ...: it finds the word holding
//   the i-th set bit (binary search over range offsets, then a wavefront ballot over lane ranks), writes
//   active[i] and, round 2, reads that neuron's gate/up rows with every 16-byte load in flight before the first
//   use. Row dot products are reduced across the wave, the activation is applied in registers, and a[i, b]
//   goes to the workspace at the dense index i.
// Kernel 2 (k_down): column gather, two dependent round trips. Each block owns SW output columns (2*SW bytes
//   of every W_downT row) and walks all active rows, so no cross-block reduction is needed. Round 1: the mask
//   words; the block compacts them into an LDS list of ids (popcount prefix across waves, mbcnt-style ranks in a
//   word); list position = dense index, since both kernels enumerate set bits in ascending order. Round 2:
//   groups of SW/8 lanes read one row slice with 16-byte loads together with a[i, b], up to DU rows per lane
//   in flight. Partial sums are reduced across lanes, then across waves through LDS.
#include "common.h"

using namespace sffn;

namespace {

constexpr int NT_UP = 256;
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
  constexpr int XPT = (B * NCH + 1) / 2;   // float4 of x per thread: B * D / (4 * NT_UP) <= B * NCH / 2

  // round 1: x and the mask words, all loads issued before any use
  float4 xv4[XPT];
  stage_load<NT_UP, XPT>(x, n4, xv4);
  const float x0 = x[0];                   // shift for the single-pass statistics (B == 1)
  const int n = mask_prefix<NT_UP, WMAX>(mask, nw, F, wpt, words_lds ? wl : nullptr, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int NW = gridDim.x * (NT_UP / 64);
  const int g0 = blockIdx.x * (NT_UP / 64);
  if (g0 >= n) return;  // block-uniform: no work for any wave of this block
  if constexpr (B == 1) {
    if (x_norm) block_norm_regs<NT_UP, XPT>(xv4, n4, x0, red);
    stage_store<NT_UP, XPT>(xs, n4, xv4);
    __syncthreads();
  } else {
    stage_store<NT_UP, XPT>(xs, n4, xv4);
    if (x_norm) stage_norm<NT_UP>(xs, B, D, red);
    else __syncthreads();
  }
  const uint64_t* words = words_lds ? wl : mask;
  const uint32_t wbytes = (uint32_t)F * (uint32_t)D * 2u;
  const Buf bwu(Wu, wbytes);
  const Buf bwg(ACT == 1 ? (const void*)Wg : (const void*)Wu, ACT == 1 ? wbytes : 0u);
  const float* bp = ACT == 1 ? bg : bu;
  const Buf bbias(bp ? (const void*)bp : (const void*)Wu, bp ? (uint32_t)F * 4u : 0u);   // no bias: 0

  for (int i = g0 + (threadIdx.x >> 6); i < n; i += NW) {
    const int id = locate(words, roff, NT_UP, wpt, nw, F, i);
    if (lane == 0) active[i] = id;
    // round 2: the neuron's rows and bias
    uint4 wu[NCH], wg[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = lane + 64 * m;
      const uint32_t o = boff(c < nc, ((uint32_t)id * nc + c) * 16u);
      wu[m] = bwu.ld16(o);
      if (ACT == 1) wg[m] = bwg.ld16(o);
    }
    const float bias = bbias.ldf((uint32_t)id * 4u);
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
        const float g = wave_sum(ag[b]) + bias;
        a = fmaxf(g, 0.f) * u;
      } else {
        a = fmaxf(u + bias, 0.f);
      }
      if (lane == 0) abuf[(size_t)i * B + b] = a;
    }
  }
}

constexpr int NT_DN = 1024;   // 16 waves
constexpr int NWV = NT_DN / 64;
constexpr int LIST_WORDS = 512;  // mask words compacted per round (32768 neurons)

template <int B, int SW>
struct DownCfg {
  static constexpr int LPR = SW / 8;                 // lanes per row slice (16 bytes each)
  static constexpr int RPI = 64 / LPR;               // rows per wave instruction
  static constexpr int DU = 16;                      // row slices in flight per lane
};

template <int B, int SW>
__global__ __launch_bounds__(NT_DN) void k_down(const uint4* __restrict__ WdT, const uint64_t* __restrict__ mask,
                                                const float* __restrict__ abuf, int D, int F,
                                                float* __restrict__ y) {
  using C = DownCfg<B, SW>;
  extern __shared__ int list[];                      // [min(nw, LIST_WORDS) * 64] ids
  __shared__ int cnt[NWV + 1];
  __shared__ float red[NWV * B * SW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nc = D >> 3;
  const int cchunk = blockIdx.x * C::LPR + (lane % C::LPR);  // 16-byte chunk of this lane's 8 columns
  const bool colok = cchunk < nc;
  const int rsub = lane / C::LPR;
  const int nw = (F + 63) >> 6;
  const Buf bm(mask, (uint32_t)nw * 8u);
  const Buf bwd(WdT, (uint32_t)F * (uint32_t)D * 2u);
  const Buf ba(abuf, (uint32_t)F * (uint32_t)B * 4u);
  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;

  int done = 0;                                      // set bits in earlier rounds (dense index base)
  for (int w0 = 0; w0 < nw; w0 += LIST_WORDS) {
    const int nwr = min(LIST_WORDS, nw - w0);
    const int wpw = (nwr + NWV - 1) / NWV;           // words per wave (<= 32)
    // round 1: this wave's mask words (lane k holds word k of the wave's range)
    const int t = w0 + w * wpw + lane;
    const uint64_t cw = bm.ldu64(boff(lane < wpw && t < w0 + nwr, (uint32_t)t * 8u));
    if (w0 > 0) __syncthreads();                     // the previous round's list is no longer read
    const int nr = compact_words<NT_DN>(cw, w0, nwr, wpw, nw, F, list, cnt);
    // round 2: row slices and activations
    for (int base = w * C::RPI + rsub; base < nr; base += NWV * C::RPI * C::DU) {
      uint4 wv[C::DU];
      float av[C::DU][B];
#pragma unroll
      for (int u = 0; u < C::DU; ++u) {
        const int i = base + u * NWV * C::RPI;
        const bool ok = i < nr;
        const uint32_t id = ok ? (uint32_t)list[i] : 0u;
        wv[u] = bwd.ld16(boff(ok && colok, (id * nc + cchunk) * 16u));
#pragma unroll
        for (int b = 0; b < B; ++b) av[u][b] = ba.ldf(boff(ok, ((uint32_t)(done + i) * B + b) * 4u));
      }
#pragma unroll
      for (int u = 0; u < C::DU; ++u) {
        float wf[8];
        f16x8_to_f32(wv[u], wf);
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[b][e] = fmaf(av[u][b], wf[e], acc[b][e]);
      }
    }
    done += nr;
  }
  // reduce over the row groups of the wave (lanes with equal lane % LPR), then across waves
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[b][e];
#pragma unroll
      for (int o = C::LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, WAVE);
      acc[b][e] = v;
    }
  if (lane < C::LPR) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(w * B + b) * SW + lane * 8 + e] = acc[b][e];
  }
  __syncthreads();
  for (int tt = threadIdx.x; tt < B * SW; tt += NT_DN) {
    const int b = tt / SW, col = tt % SW;
    float s = 0.f;
    for (int ww = 0; ww < NWV; ++ww) s += red[(ww * B + b) * SW + col];
    const int d = blockIdx.x * SW + col;
    if (d < D) y[(size_t)b * D + d] = s;
  }
}

template <int B, int ACT, int NCH>
hipError_t launch_up(const void* Wg, const float* bg, const void* Wu, const float* bu, const float* x, int x_norm, int D,
                     int F, const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf, hipStream_t st) {
  const int nw = (F + 63) / 64;
  const int wpt = (nw + NT_UP - 1) / NT_UP;
  const size_t lds = (wpt <= WMAX ? (size_t)((nw + 1) & ~1) * 8 : 0) + (NT_UP + NT_UP / 64 + 4) * sizeof(int) +
                     ((size_t)B * D + 2 * (NT_UP / 64) * B) * sizeof(float);
  static size_t avail = 0;
  if (!avail) {
    hipError_t ea = allow_dynamic_lds((const void*)k_upgate<B, ACT, NCH>, &avail);
    if (ea != hipSuccess) return ea;
  }
  if (lds > avail) return hipErrorInvalidValue;
  const int grid = std::max(1, std::min((F + 3) / 4, 512));
  sffn_prof_before(2, st);
  hipLaunchKernelGGL((k_upgate<B, ACT, NCH>), dim3(grid), dim3(NT_UP), lds, st, (const uint4*)Wg, bg,
                     (const uint4*)Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf);
  sffn_prof_after(2, st);
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

constexpr int DOWN_SW = 32;

template <int B>
hipError_t launch_down(const void* WdT, const uint64_t* mask, const float* abuf, int D, int F, float* y,
                       hipStream_t st) {
  const int nw = (F + 63) / 64;
  const size_t lds = (size_t)std::min(nw, LIST_WORDS) * 64 * sizeof(int);
  static size_t avail = 0;
  if (!avail) {
    hipError_t ea = allow_dynamic_lds((const void*)k_down<B, DOWN_SW>, &avail);
    if (ea != hipSuccess) return ea;
  }
  if (lds > avail) return hipErrorInvalidValue;
  const int grid = (D + DOWN_SW - 1) / DOWN_SW;
  sffn_prof_before(3, st);
  hipLaunchKernelGGL((k_down<B, DOWN_SW>), dim3(grid), dim3(NT_DN), lds, st, (const uint4*)WdT, mask, abuf, D, F, y);
  sffn_prof_after(3, st);
  return hipGetLastError();
}

template <int B>
hipError_t forward_b(int act, const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                     const float* x, int x_norm, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active,
                     float* y, float* abuf, hipStream_t st) {
  const int nch = (D / 8 + 63) / 64;
  hipError_t e = act == 1 ? dispatch_up<B, 1>(nch, Wg, bg, Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf, st)
                          : dispatch_up<B, 0>(nch, Wg, bg, Wu, bu, x, x_norm, D, F, mask, active, n_active, abuf, st);
  if (e != hipSuccess) return e;
  return launch_down<B>(WdT, mask, abuf, D, F, y, st);
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
