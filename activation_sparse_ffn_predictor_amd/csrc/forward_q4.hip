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
// Work split and compaction are those of the fp16 path: k_upgate_q4 (mask -> ids, balanced dense-index
// mapping, first rows in flight while x is staged, row gather, fused activation) and k_down_q4 (reads the ids
// kernel 1 wrote to active[]; each block owns 128 output columns = 4 Q4 blocks of every W_downT row; a lane
// reads half a block: 8 nibble bytes and the scale).
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
constexpr int WMAX = 2;            // mask words per thread in registers / LDS (F <= 32768; larger F reads them from memory)

// sum over a Q4 block of q_e * x_e: nib = 16 nibble bytes, xl/xh = x of the low-nibble (elements 0..15) and
// high-nibble (elements 16..31) halves of the block, as four float4 each.
__device__ __forceinline__ float q4_block_dot(const uint4& nib, const float4* xl, const float4* xh) {
  const uint32_t wds[4] = {nib.x, nib.y, nib.z, nib.w};
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = wds[k] & 0x0F0F0F0Fu, hi = (wds[k] >> 4) & 0x0F0F0F0Fu;
    s = fmaf((float)(lo & 0xFF), xl[k].x, s);
    s = fmaf((float)((lo >> 8) & 0xFF), xl[k].y, s);
    s = fmaf((float)((lo >> 16) & 0xFF), xl[k].z, s);
    s = fmaf((float)(lo >> 24), xl[k].w, s);
    s = fmaf((float)(hi & 0xFF), xh[k].x, s);
    s = fmaf((float)((hi >> 8) & 0xFF), xh[k].y, s);
    s = fmaf((float)((hi >> 16) & 0xFF), xh[k].z, s);
    s = fmaf((float)(hi >> 24), xh[k].w, s);
  }
  return s;
}

__device__ __forceinline__ float sum4(const float4& v) { return (v.x + v.y) + (v.z + v.w); }

template <int B, int ACT, int NQ>
__global__ __launch_bounds__(NT_UP) void k_upgate_q4(const uint4* __restrict__ qg, const _Float16* __restrict__ sg,
                                                     const float* __restrict__ bg, const uint4* __restrict__ qu,
                                                     const _Float16* __restrict__ su, const float* __restrict__ bu,
                                                     const float* __restrict__ x, int x_norm, int D, int F,
                                                     const uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                     int32_t* __restrict__ n_active, float* __restrict__ abuf) {
  extern __shared__ uint64_t lds64[];
  const int nblk = D >> 5;                                   // Q4 blocks per row
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NT_UP - 1) / NT_UP;
  const bool words_lds = wpt <= WMAX;
  uint64_t* wl = lds64;
  int* roff = reinterpret_cast<int*>(wl + (words_lds ? ((nw + 1) & ~1) : 0));
  int* tmp = roff + NT_UP;
  float* xs = reinterpret_cast<float*>(tmp + NT_UP / 64 + 4);  // [B, D], then xsum [B, nblk], then red
  float* xsum = xs + (size_t)B * D;
  float* red = xsum + (size_t)B * nblk;
  const int lane = threadIdx.x & 63;
  const int n4 = (B * D) >> 2;
  constexpr int XPT = (512 * B * NQ + NT_UP - 1) / NT_UP;   // float4 of x per thread: B * D / 4 <= 512 * B * NQ

  // round 1: x and the mask words, all loads issued before any use
  float4 xv4[XPT];
  stage_load<NT_UP, XPT>(x, n4, xv4);
  const float x0 = x[0];
  const int n = mask_prefix<NT_UP, WMAX>(mask, nw, F, wpt, words_lds ? wl : nullptr, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int G = gridDim.x;
  if ((int)blockIdx.x >= n) return;  // block-uniform: no dense index maps to this block
  const uint64_t* words = words_lds ? wl : mask;
  const uint32_t qbytes = (uint32_t)F * (uint32_t)nblk * 16u, sbytes = (uint32_t)F * (uint32_t)nblk * 2u;
  const Buf bqu(qu, qbytes), bsu(su, sbytes);
  const Buf bqg(ACT == 1 ? (const void*)qg : (const void*)qu, ACT == 1 ? qbytes : 0u);
  const Buf bsg(ACT == 1 ? (const void*)sg : (const void*)su, ACT == 1 ? sbytes : 0u);
  const float* bp = ACT == 1 ? bg : bu;
  const Buf bbias(bp ? (const void*)bp : (const void*)qu, bp ? (uint32_t)F * 4u : 0u);   // no bias: 0
  const int NW = G * (NT_UP / 64);
  int i = (int)blockIdx.x + G * (threadIdx.x >> 6);
  uint4 nu[NQ], ng[NQ];
  float fu[NQ], fg[NQ];
  float bias = 0.f;
  int id = 0;
  auto issue = [&]() {  // round 2 for dense index i: the neuron's nibbles, scales and bias
    id = locate(words, roff, NT_UP, wpt, nw, F, i);
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int c = lane + 64 * m;
      const bool ok = c < nblk;
      const uint32_t o = (uint32_t)id * nblk + c;
      nu[m] = bqu.ld16(boff(ok, o * 16u));
      fu[m] = bsu.ldh(boff(ok, o * 2u));
      if (ACT == 1) {
        ng[m] = bqg.ld16(boff(ok, o * 16u));
        fg[m] = bsg.ldh(boff(ok, o * 2u));
      }
    }
    bias = bbias.ldf((uint32_t)id * 4u);
  };
  const bool have = i < n;            // wave-uniform
  if (have) issue();
  // x: normalised, staged and summed per Q4 block while the first rows are in flight
  if constexpr (B == 1) {
    if (x_norm) block_norm_regs<NT_UP, XPT>(xv4, n4, x0, red);
    stage_store<NT_UP, XPT>(xs, n4, xv4);
    __syncthreads();
  } else {
    stage_store<NT_UP, XPT>(xs, n4, xv4);
    if (x_norm) stage_norm<NT_UP>(xs, B, D, red);
    else __syncthreads();
  }
  for (int t = threadIdx.x; t < B * nblk; t += NT_UP) {
    const float4* p = reinterpret_cast<const float4*>(xs + (size_t)(t / nblk) * D + 32 * (t % nblk));
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) v += sum4(p[k]);
    xsum[t] = v;
  }
  __syncthreads();
  if (!have) return;
  for (;;) {
    if (lane == 0) active[i] = id;
    float au[B], ag[B];
#pragma unroll
    for (int b = 0; b < B; ++b) { au[b] = 0.f; ag[b] = 0.f; }
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int c = lane + 64 * m;
      if (c < nblk) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float4* xl = reinterpret_cast<const float4*>(xs + (size_t)b * D + 32 * c);
          const float xsb = xsum[b * nblk + c];
          au[b] = fmaf(fu[m], q4_block_dot(nu[m], xl, xl + 4) - 8.f * xsb, au[b]);
          if (ACT == 1) ag[b] = fmaf(fg[m], q4_block_dot(ng[m], xl, xl + 4) - 8.f * xsb, ag[b]);
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

#ifndef SFFN_DOWN_XCD
#define SFFN_DOWN_XCD 1                // XCD-aware order of the column slices of the column gather
#endif
#ifndef SFFN_Q4_DOWN_SW
#define SFFN_Q4_DOWN_SW 64
#endif
constexpr int QSW = SFFN_Q4_DOWN_SW;   // output columns per block (QSW / 32 Q4 blocks of each row)
constexpr int QCPL = 16;               // columns per lane (half a Q4 block: 8 nibble bytes)
constexpr int QLPR = QSW / QCPL;       // lanes per row slice (8)
constexpr int QRPI = 64 / QLPR;        // rows per wave instruction (8)
template <int B> struct QD;            // threads per block, row slices in flight per lane (3 loads each)
template <> struct QD<1> { static constexpr int NT = 512, DU = 16; };
template <> struct QD<2> { static constexpr int NT = 512, DU = 12; };
template <> struct QD<4> { static constexpr int NT = 512, DU = 8; };
template <> struct QD<8> { static constexpr int NT = 512, DU = 2; };

template <int B>
__global__ __launch_bounds__(QD<B>::NT) void k_down_q4(const uint8_t* __restrict__ qd, const _Float16* __restrict__ sd,
                                                       const int32_t* __restrict__ active,
                                                       const int32_t* __restrict__ n_active,
                                                       const float* __restrict__ abuf, int D, int F,
                                                       float* __restrict__ y) {
  constexpr int NT = QD<B>::NT, DU = QD<B>::DU, NWV = NT / 64, STRIDE = NWV * QRPI * DU;
  __shared__ float red[NWV * B * QSW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nblk = D >> 5;
  const int rsub = lane / QLPR, lsub = lane % QLPR;
  const int slice = SFFN_DOWN_XCD ? xcd_slice(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  if (slice * QSW >= D) return;               // block-uniform: padding of the grid to 8 * per
  const int col0 = slice * QSW + lsub * QCPL;
  const int qblk = col0 >> 5;                 // Q4 block of this lane
  const int half = (col0 >> 4) & 1;           // which 8-byte half of the block's nibbles
  const bool colok = col0 < D;
  const Buf bqd(qd, (uint32_t)F * (uint32_t)(D >> 1));
  const Buf bsd(sd, (uint32_t)F * (uint32_t)nblk * 2u);
  const Buf ba(abuf, (uint32_t)F * (uint32_t)B * 4u);
  const Buf bid(active, (uint32_t)F * 4u);
  const Buf bn(n_active, 4u);
  float acc[B][QCPL];
  float sas[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    sas[b] = 0.f;
#pragma unroll
    for (int e = 0; e < QCPL; ++e) acc[b][e] = 0.f;
  }
  auto load_ids = [&](int k0, uint32_t (&ids)[DU]) {  // speculative, bounded by F
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int i = k0 + w * QRPI + rsub + u * NWV * QRPI;
      ids[u] = bid.ldu(boff(i < F, (uint32_t)i * 4u));
    }
  };
  // one pass: every nibble, scale and activation load is issued before the first multiply-add (the scheduling
  // barrier keeps the compiler from interleaving them, which would leave few loads in flight per lane)
  auto pass = [&](int k0, int n, const uint32_t (&ids)[DU]) {
    uint2 nib[DU];
    float sc[DU];
    float av[DU][B];
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int i = k0 + w * QRPI + rsub + u * NWV * QRPI;
      const bool ok = i < n;
      const uint32_t row = ids[u];
      nib[u] = bqd.ld8(boff(ok && colok, row * (uint32_t)(D >> 1) + (uint32_t)qblk * 16u + (uint32_t)half * 8u));
      sc[u] = bsd.ldh(boff(ok && colok, (row * nblk + qblk) * 2u));
#pragma unroll
      for (int b = 0; b < B; ++b) av[u][b] = ba.ldf(boff(ok, ((uint32_t)i * B + b) * 4u));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < DU; ++u) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float as_ = av[u][b] * sc[u];
        sas[b] += as_;
        const uint32_t wds[2] = {nib[u].x, nib[u].y};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t lo = wds[k] & 0x0F0F0F0Fu, hi = (wds[k] >> 4) & 0x0F0F0F0Fu;
          // lane-local element e: e < 8 low nibbles (block elements 8*half + e),
          // e >= 8 high nibbles (block elements 16 + 8*half + e - 8)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[b][4 * k + j] = fmaf(as_, (float)((lo >> (8 * j)) & 0xFF), acc[b][4 * k + j]);
            acc[b][8 + 4 * k + j] = fmaf(as_, (float)((hi >> (8 * j)) & 0xFF), acc[b][8 + 4 * k + j]);
          }
        }
      }
    }
  };
  // round 1: the count and the first pass's ids together; round 2: that pass's nibbles, scales, activations
  const int nraw = (int)bn.ldu(0u);
  uint32_t ids[DU];
  load_ids(0, ids);
  const int n = min(max(nraw, 0), F);
  pass(0, n, ids);
  for (int k0 = STRIDE; k0 < n; k0 += STRIDE) {       // more rows than one pass holds
    load_ids(k0, ids);
    pass(k0, n, ids);
  }
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < QCPL; ++e) {
      float v = fmaf(-8.f, sas[b], acc[b][e]);
#pragma unroll
      for (int o = QLPR; o < 64; o <<= 1) v += __shfl_xor(v, o, WAVE);
      acc[b][e] = v;
    }
  if (lane < QLPR) {
    const int cb = qblk * 32 - slice * QSW;        // first column of the lane's Q4 block, block-relative
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int e = 0; e < QCPL; ++e) {
        const int cc = e < 8 ? cb + 8 * half + e : cb + 16 + 8 * half + (e - 8);
        red[(w * B + b) * QSW + cc] = acc[b][e];
      }
  }
  __syncthreads();
  for (int tt = threadIdx.x; tt < B * QSW; tt += NT) {
    const int b = tt / QSW, cc = tt % QSW;
    float s = 0.f;
    for (int ww = 0; ww < NWV; ++ww) s += red[(ww * B + b) * QSW + cc];
    const int d = slice * QSW + cc;
    if (d < D) y[(size_t)b * D + d] = s;
  }
}

template <int B, int ACT, int NQ>
hipError_t launch_up(const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu, const void* su,
                     const float* bu, const float* x, int x_norm, int D, int F, const uint64_t* mask, int32_t* active,
                     int32_t* n_active, float* abuf, hipStream_t st) {
  const int nblk = D / 32;
  const int nw = (F + 63) / 64;
  const int wpt = (nw + NT_UP - 1) / NT_UP;
  const size_t lds = (wpt <= WMAX ? (size_t)((nw + 1) & ~1) * 8 : 0) + (NT_UP + NT_UP / 64 + 4) * sizeof(int) +
                     ((size_t)B * D + (size_t)B * nblk + 2 * (NT_UP / 64) * B) * sizeof(float);
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_upgate_q4<B, ACT, NQ>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail) return hipErrorInvalidValue;
  const int grid = std::max(1, std::min((F + 3) / 4, SFFN_UP_GRID));
  SFFN_LAUNCH(2, (k_upgate_q4<B, ACT, NQ>), dim3(grid), dim3(NT_UP), lds, st, (const uint4*)qg,
                     (const _Float16*)sg, bg, (const uint4*)qu, (const _Float16*)su, bu, x, x_norm, D, F, mask, active,
                     n_active, abuf);
  return hipGetLastError();
}

template <int B, int ACT>
hipError_t dispatch_up(int nq, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu, const void* su,
                       const float* bu, const float* x, int x_norm, int D, int F, const uint64_t* mask, int32_t* active,
                       int32_t* n_active, float* abuf, hipStream_t st) {
#define UPQ(N) return launch_up<B, ACT, N>(qg, sg, bg, qu, su, bu, x, x_norm, D, F, mask, active, n_active, abuf, st)
  if (nq <= 1) UPQ(1);
  if (nq <= 2) UPQ(2);
  if (nq <= 4) UPQ(4);
  UPQ(8);
#undef UPQ
}

template <int B>
hipError_t forward_b(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu, const void* su,
                     const float* bu, const uint8_t* qd, const void* sd, const float* x, int x_norm, int D, int F,
                     const uint64_t* mask, int32_t* active, int32_t* n_active, float* y, float* abuf, hipStream_t st) {
  const int nq = (D / 32 + 63) / 64;
  hipError_t e =
      act == 1   ? dispatch_up<B, 1>(nq, qg, sg, bg, qu, su, bu, x, x_norm, D, F, mask, active, n_active, abuf, st)
      : act == 2 ? dispatch_up<B, 2>(nq, qg, sg, bg, qu, su, bu, x, x_norm, D, F, mask, active, n_active, abuf, st)
                 : dispatch_up<B, 0>(nq, qg, sg, bg, qu, su, bu, x, x_norm, D, F, mask, active, n_active, abuf, st);
  if (e != hipSuccess) return e;
  const int slices = (D + QSW - 1) / QSW;
  const int grid = SFFN_DOWN_XCD ? (slices + 7) / 8 * 8 : slices;
  SFFN_LAUNCH(3, k_down_q4<B>, dim3(grid), dim3(QD<B>::NT), 0, st, qd, (const _Float16*)sd, active, n_active, abuf, D,
              F, y);
  return hipGetLastError();
}

}  // namespace

hipError_t sffn_launch_forward_q4(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu,
                                  const void* su, const float* bu, const uint8_t* qd, const void* sd, const float* x,
                                  int x_norm, int B, int D, int F, const uint64_t* mask, int32_t* active,
                                  int32_t* n_active, float* y, float* abuf, hipStream_t st) {
  switch (B) {
    case 1: return forward_b<1>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    case 2: return forward_b<2>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    case 4: return forward_b<4>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    case 8: return forward_b<8>(act, qg, sg, bg, qu, su, bu, qd, sd, x, x_norm, D, F, mask, active, n_active, y, abuf, st);
    default: return hipErrorInvalidValue;
  }
}
