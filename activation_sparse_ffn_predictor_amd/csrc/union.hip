// Multi-token (union-mask) path, B > 1: matrix-core (MFMA) kernels for gfx950.
//
// The pages' decode is one token at a time; with several tokens the predicted-active sets are merged (one
// mask, the union over tokens) and every token is computed over that union, so each active row of the
// weights is read once for the whole batch ("Neuron-aware operator", Turkish article). Each step below is a
// small GEMM over gathered rows, so it runs on v_mfma_f32_16x16x32_f16:
//   A operand: 16 weight rows x 32 k (lane l: row l % 16, k 8*(l/16)..+8 -- one 16-byte load of a neuron-major
//              row), B operand: 32 k x 16 tokens (lane l: token l % 16), D: 16 rows x 16 tokens (lane l holds
//              rows 4*(l/16)+i of token l % 16).
// fp32 activations enter as two fp16 halves, x = hi + lo (hi = fp16(x), lo = fp16(x - hi)); weights are exact
// in fp16 (Q4_0: q - 8 is exact, the block scale is applied to the fp32 result of each 32-wide k block). So
// every product is exact and accumulation is fp32, like the single-token path.
//
// Kernels:
//   k_norm_tokens : per-token normalisation of x into the workspace (when the layer input is normalised)
//   k_mt_h        : partial h = P1 x over a share of d, 16 rows of P1 per block, shares over blocks (grid y),
//                   split again over 8 waves with an LDS reduction; k_sum_parts adds the shares in fixed order
//   k_mt_z        : z = P2 h + c, 64 neurons per block (one mask word), OR over tokens by ballot
//   k_mt_rows     : compaction + W_gate / W_up row gather over 16 active neurons per block, k split over 8
//                   waves, fused activation, dense activations a[i, b]
//   k_mt_down     : y partial sums over a slice of 128 columns and every KS-th step of 64 active rows (ids from
//                   the row kernel's active[]); W_downT tiles are staged in LDS and read transposed as the B
//                   operand; activations (times the Q4 block scale) are the A operand; next step loaded ahead
//   k_sum_parts   : y = sum of the partial sums
#include "common.h"

using namespace sffn;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const half8& a, const half8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// x = hi + lo with hi = fp16(x), lo = fp16(x - hi)
__device__ __forceinline__ void split8(const float* v, half8& hi, half8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)v[i];
    hi[i] = h;
    lo[i] = (_Float16)(v[i] - (float)h);
  }
}

// Q4_0: the 8 elements 8*j .. 8*j+7 of a 32-element block (j = 0..3) as exact fp16 (q - 8).
// p = the 8 nibble bytes (8*(j & 1) .. +8) of the block; low nibbles for j < 2, high for j >= 2.
__device__ __forceinline__ half8 q4_to_half8(const uint2& p, int j) {
  const uint32_t sh = (j >> 1) * 4;
  const uint32_t w0 = (p.x >> sh) & 0x0F0F0F0Fu, w1 = (p.y >> sh) & 0x0F0F0F0Fu;
  half8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (_Float16)((int)((w0 >> (8 * i)) & 0xFF) - 8);
    h[4 + i] = (_Float16)((int)((w1 >> (8 * i)) & 0xFF) - 8);
  }
  return h;
}

constexpr int NTN = 512;

// per-token normalisation (centre, unit variance): one block per token; every load of the token is issued at
// once, the statistics are single-pass about x[0] (block_norm_regs) and the result is written from registers
template <int XPT>
__global__ __launch_bounds__(NTN) void k_norm_tokens(const float* __restrict__ x, int D, float* __restrict__ xn) {
  __shared__ float red[2 * (NTN / 64)];
  const int n4 = D >> 2;
  const float* xb = x + (size_t)blockIdx.x * D;
  float4 v[XPT];
  stage_load<NTN, XPT>(xb, n4, v);
  const float x0 = xb[0];
  block_norm_regs<NTN, XPT>(v, n4, x0, red);
  float4* ob = reinterpret_cast<float4*>(xn + (size_t)blockIdx.x * D);
#pragma unroll
  for (int k = 0; k < XPT; ++k) {
    const int i = k * NTN + (int)threadIdx.x;
    if (i < n4) ob[i] = v[k];
  }
}

// B operand for token tile t at k block kb: lane l reads x[t*16 + l%16][32 kb + 8 (l/16) .. +8] (fp32) and splits it
__device__ __forceinline__ void load_xtile(const Buf& bx, int B, int K, int t, int kb, half8& hi, half8& lo) {
  const int lane = threadIdx.x & 63;
  const int tok = t * 16 + (lane & 15);
  const int k = kb * 32 + (lane >> 4) * 8;
  const bool ok = tok < B && k < K;
  const uint32_t o = ((uint32_t)tok * K + k) * 4u;
  const float4 a = bx.ldf4(boff(ok, o)), b = bx.ldf4(boff(ok, o + 16u));
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  split8(v, hi, lo);
}

// raw fp32 B-operand values of token tile t at k block kb (split into fp16 halves at use)
struct XRaw { float4 a, b; };
__device__ __forceinline__ XRaw load_xraw(const Buf& bx, int B, int K, int t, int kb) {
  const int lane = threadIdx.x & 63;
  const int tok = t * 16 + (lane & 15);
  const int k = kb * 32 + (lane >> 4) * 8;
  const bool ok = tok < B && k < K;
  const uint32_t o = ((uint32_t)tok * K + k) * 4u;
  return XRaw{bx.ldf4(boff(ok, o)), bx.ldf4(boff(ok, o + 16u))};
}
__device__ __forceinline__ void split_xraw(const XRaw& r, half8& hi, half8& lo) {
  const float v[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
  split8(v, hi, lo);
}

// k blocks whose loads are issued together (one memory round trip per chunk), by token tiles
template <int NTT> struct KChunk { static constexpr int CH = NTT == 1 ? 8 : (NTT == 2 ? 4 : 2); };

constexpr int NTK = 512;            // 8 waves split the k dimension
constexpr int KW = NTK / 64;

// Partial h over one of gridDim.y shares of d: hp[ks][b][j] = sum_{d in share ks} P1[j, d] x[b, d]; block = 16
// rows of P1 and one share of the k range, split again over the 8 waves.
template <int NTT>
__global__ __launch_bounds__(NTK) void k_mt_h(const uint4* __restrict__ P1, const float* __restrict__ x, int B, int D,
                                              int r, float* __restrict__ hp) {
  __shared__ f32x4 part[KW][NTT][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j0 = blockIdx.x * 16;
  const int KB = (D + 31) / 32;
  const int KSH = gridDim.y, ks = blockIdx.y;
  const int kps = (KB + KSH - 1) / KSH;                  // k blocks of this share
  const int ks0 = ks * kps, ks1 = min(KB, ks0 + kps);
  const int kpw = (kps + KW - 1) / KW;
  const int kb0 = ks0 + w * kpw, kb1 = min(ks1, kb0 + kpw);
  const Buf bp(P1, (uint32_t)r * D * 2u), bx(x, (uint32_t)B * D * 4u);
  const int row = j0 + (lane & 15);
  f32x4 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int CH = KChunk<NTT>::CH;
  for (int c0 = kb0; c0 < kb1; c0 += CH) {
    uint4 av[CH];
    XRaw xr[CH][NTT];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int kb = c0 + q;
      const int k = kb * 32 + (lane >> 4) * 8;
      av[q] = bp.ld16(boff(kb < kb1 && row < r && k < D, ((uint32_t)row * D + k) * 2u));
#pragma unroll
      for (int t = 0; t < NTT; ++t) xr[q][t] = load_xraw(bx, B, kb < kb1 ? D : 0, t, kb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const half8 a = __builtin_bit_cast(half8, av[q]);
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        half8 xh, xl;
        split_xraw(xr[q][t], xh, xl);
        acc[t] = mfma16(a, xl, mfma16(a, xh, acc[t]));
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NTT; ++t) part[w][t][lane] = acc[t];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      f32x4 s = part[0][t][lane];
      for (int ww = 1; ww < KW; ++ww) s += part[ww][t][lane];
      const int tok = t * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + (lane >> 4) * 4 + i;
        if (tok < B && j < r) hp[((size_t)ks * B + tok) * r + j] = s[i];
      }
    }
  }
}

// z = P2 h + c; mask word per block (64 neurons = 4 waves x 16)
template <int NTT>
__global__ __launch_bounds__(256) void k_mt_z(const uint4* __restrict__ P2, const float* __restrict__ c,
                                              const float* __restrict__ h, int B, int F, int r, float tau,
                                              int n_hot, uint64_t* __restrict__ mask,
                                              float* __restrict__ logits) {
  __shared__ uint32_t bits16[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k0 = blockIdx.x * 64 + w * 16;
  const int KB = (r + 31) / 32;
  const Buf bp(P2, (uint32_t)F * r * 2u), bh(h, (uint32_t)B * r * 4u);
  const Buf bc(c ? (const void*)c : (const void*)P2, c ? (uint32_t)F * 4u : 0u);
  const int row = k0 + (lane & 15);
  f32x4 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int CH = KChunk<NTT>::CH;
  for (int c0 = 0; c0 < KB; c0 += CH) {
    uint4 av[CH];
    XRaw hr[CH][NTT];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int kb = c0 + q;
      const int k = kb * 32 + (lane >> 4) * 8;
      av[q] = bp.ld16(boff(kb < KB && row < F && row >= n_hot && k < r, ((uint32_t)row * r + k) * 2u));
#pragma unroll
      for (int t = 0; t < NTT; ++t) hr[q][t] = load_xraw(bh, B, kb < KB ? r : 0, t, kb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const half8 a = __builtin_bit_cast(half8, av[q]);
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        half8 hh, hl;
        split_xraw(hr[q][t], hh, hl);
        acc[t] = mfma16(a, hl, mfma16(a, hh, acc[t]));
      }
    }
  }
  // lane l holds rows 4*(l/16)+i of token l%16 (per token tile)
  float cb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = k0 + (lane >> 4) * 4 + i;
    cb[i] = bc.ldf(boff(kk < F && kk >= n_hot, (uint32_t)kk * 4u));
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = k0 + (lane >> 4) * 4 + i;
    bool any = false;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int tok = t * 16 + (lane & 15);
      const float z = kk < n_hot ? INFINITY : acc[t][i] + cb[i];   // always-active prefix: no row was read
      const bool valid = tok < B && kk < F;
      if (valid && logits) logits[(size_t)tok * F + kk] = z;
      any = any || (valid && z > tau);
    }
    const unsigned long long bal = __ballot(any);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if ((bal >> (16 * g)) & 0xFFFFull) word |= 1u << (g * 4 + i);
  }
  if (lane == 0) bits16[w] = word;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t m = (uint64_t)bits16[0] | ((uint64_t)bits16[1] << 16) | ((uint64_t)bits16[2] << 32) |
                       ((uint64_t)bits16[3] << 48);
    mask[blockIdx.x] = m;
  }
}

// per-lane version of locate: stored id of dense index i (i < total)
__device__ __forceinline__ int locate_lane(const uint64_t* words, const int* roff, int nranges, int wpt, int nw, int F,
                                           int i) {
  int lo = 0, hi = nranges - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (roff[mid] <= i) lo = mid; else hi = mid - 1;
  }
  int rem = i - roff[lo];
  for (int t = lo * wpt; t < nw; ++t) {
    uint64_t word = words[t];
    if (t == nw - 1 && (F & 63)) word &= (1ull << (F & 63)) - 1ull;
    const int cnt = __popcll(word);
    if (rem < cnt) return t * 64 + select_bit(word, rem);
    rem -= cnt;
  }
  return 0;
}

constexpr int WMAXU = 2;

// Active-row gather with fused activation, 16 dense indices per block, k split over 8 waves.
// Q4: W = nibble planes + scale planes. ACT 1 = ReGLU (gate + up), 0 = ReLU (up), 2 = squared ReLU (up).
// KSP > 1 splits k over KSP blocks per 16 rows, block t * KSP + ks taking share ks (the shares of a tile are
// neighbours in dispatch order, so both start with the first blocks; with the shares in a second grid dimension
// they came after every first share, most of them blocks without rows, and 8 tokens gained nothing): each
// writes its partial pre-activations
// (up, and gate for ReGLU, no bias) to pre[(ks * 2 + mat) * F * B + i * B + token] and k_act_combine applies
// the activation; with KSP = 1 the block writes the activations itself.
template <int NTT, int ACT, bool Q4>
__global__ __launch_bounds__(NTK) void k_mt_rows(const void* __restrict__ Wg, const void* __restrict__ Sg,
                                                 const float* __restrict__ bg, const void* __restrict__ Wu,
                                                 const void* __restrict__ Su, const float* __restrict__ bu,
                                                 const float* __restrict__ x, int B, int D, int F,
                                                 const uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                 int32_t* __restrict__ n_active, float* __restrict__ abuf,
                                                 float* __restrict__ pre, int KSP) {
  constexpr bool GT = ACT == 1;                        // gated (ReGLU): a gate row per neuron
  extern __shared__ uint64_t lds64[];
  __shared__ f32x4 part[KW][GT ? 2 : 1][NTT][64];
  __shared__ int ids16[16];
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NTK - 1) / NTK;
  const bool words_lds = wpt <= WMAXU;
  uint64_t* wl = lds64;
  int* roff = reinterpret_cast<int*>(wl + (words_lds ? ((nw + 1) & ~1) : 0));
  int* tmp = roff + NTK;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = mask_prefix<NTK, WMAXU>(mask, nw, F, wpt, words_lds ? wl : nullptr, roff, tmp);
  const int ksp = blockIdx.x % KSP;
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int i0 = (blockIdx.x / KSP) * 16;
  if (i0 >= n) return;
  const uint64_t* words = words_lds ? wl : mask;
  if (threadIdx.x < 16) {
    const int i = i0 + threadIdx.x;
    const int id = i < n ? locate_lane(words, roff, NTK, wpt, nw, F, i) : -1;
    ids16[threadIdx.x] = id;
    if (id >= 0 && ksp == 0) active[i] = id;
  }
  __syncthreads();
  const int idl = ids16[lane & 15];                      // A-operand row of this lane (-1: none)
  const int KB = (D + 31) / 32;
  const int KBh = (KB + KSP - 1) / KSP;                  // k blocks of this block's share
  const int kbs = ksp * KBh, kbe = min(KB, kbs + KBh);
  const int kpw = (kbe - kbs + KW - 1) / KW;
  const int kb0 = kbs + w * kpw, kb1 = min(kbe, kb0 + kpw);
  const Buf bx(x, (uint32_t)B * D * 4u);
  const int nblk = D >> 5;
  const uint32_t wbytes = Q4 ? (uint32_t)F * (uint32_t)(D >> 1) : (uint32_t)F * D * 2u;
  const uint32_t sbytes = (uint32_t)F * nblk * 2u;
  const Buf bwu(Wu, wbytes), bwg(GT ? Wg : Wu, GT ? wbytes : 0u);
  const Buf bsu(Q4 ? Su : Wu, Q4 ? sbytes : 0u), bsg(Q4 && GT ? Sg : Wu, Q4 && GT ? sbytes : 0u);
  // rows of this lane's 4 outputs (D layout): 4*(l/16)+i
  int idr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) idr[i] = ids16[(lane >> 4) * 4 + i];
  f32x4 au[NTT], ag[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) { au[t] = f32x4{0.f, 0.f, 0.f, 0.f}; ag[t] = au[t]; }
  // Double-buffered chunks of CH k blocks: the next chunk's weight rows (or nibbles and scales) and x tiles are
  // issued before the current chunk's matrix-core work, so consecutive round trips overlap.
  // one token tile: 2 k blocks per chunk, so that the fp16 kernels stay within 128 VGPRs and two blocks share a
  // CU (more rows in flight per CU than longer chunks give)
  constexpr int CH = NTT == 1 ? 2 : (KChunk<NTT>::CH / 2 > 0 ? KChunk<NTT>::CH / 2 : 1);
  struct Chunk {
    uint4 wu[CH], wg[CH];
    uint2 qu[CH], qg[CH];
    float su[CH][4], sg[CH][4];
    XRaw xr[CH][NTT];
  };
  auto load_chunk = [&](int c0, Chunk& C) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int kb = c0 + q;
      const int k = kb * 32 + (lane >> 4) * 8;
      const bool ok = kb < kb1 && idl >= 0 && k < D;
      if constexpr (Q4) {
        const uint32_t o = (uint32_t)(ok ? idl : 0) * (uint32_t)(D >> 1) + (uint32_t)kb * 16u + ((lane >> 4) & 1) * 8u;
        C.qu[q] = bwu.ld8(boff(ok, o));
        if (GT) C.qg[q] = bwg.ld8(boff(ok, o));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool okr = kb < kb1 && idr[i] >= 0;
          const uint32_t so = ((uint32_t)(okr ? idr[i] : 0) * nblk + kb) * 2u;
          C.su[q][i] = bsu.ldh(boff(okr, so));
          if (GT) C.sg[q][i] = bsg.ldh(boff(okr, so));
        }
      } else {
        const uint32_t o = ((uint32_t)(ok ? idl : 0) * D + k) * 2u;
        C.wu[q] = bwu.ld16(boff(ok, o));
        if (GT) C.wg[q] = bwg.ld16(boff(ok, o));
      }
#pragma unroll
      for (int t = 0; t < NTT; ++t) C.xr[q][t] = load_xraw(bx, B, kb < kb1 ? D : 0, t, kb);
    }
  };
  auto compute_chunk = [&](const Chunk& C) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      half8 a_u, a_g;
      if constexpr (Q4) {
        a_u = q4_to_half8(C.qu[q], lane >> 4);
        if (GT) a_g = q4_to_half8(C.qg[q], lane >> 4);
      } else {
        a_u = __builtin_bit_cast(half8, C.wu[q]);
        if (GT) a_g = __builtin_bit_cast(half8, C.wg[q]);
      }
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        half8 xh, xl;
        split_xraw(C.xr[q][t], xh, xl);
        if constexpr (Q4) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const f32x4 pu = mfma16(a_u, xl, mfma16(a_u, xh, z));
#pragma unroll
          for (int i = 0; i < 4; ++i) au[t][i] = fmaf(C.su[q][i], pu[i], au[t][i]);
          if (GT) {
            const f32x4 pg = mfma16(a_g, xl, mfma16(a_g, xh, z));
#pragma unroll
            for (int i = 0; i < 4; ++i) ag[t][i] = fmaf(C.sg[q][i], pg[i], ag[t][i]);
          }
        } else {
          au[t] = mfma16(a_u, xl, mfma16(a_u, xh, au[t]));
          if (GT) ag[t] = mfma16(a_g, xl, mfma16(a_g, xh, ag[t]));
        }
      }
    }
  };
  Chunk cA, cB;
  if (kb0 < kb1) load_chunk(kb0, cA);
  for (int c0 = kb0; c0 < kb1; c0 += 2 * CH) {
    if (c0 + CH < kb1) load_chunk(c0 + CH, cB);
    __builtin_amdgcn_sched_barrier(0);
    compute_chunk(cA);
    if (c0 + CH >= kb1) break;
    if (c0 + 2 * CH < kb1) load_chunk(c0 + 2 * CH, cA);
    __builtin_amdgcn_sched_barrier(0);
    compute_chunk(cB);
  }
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    part[w][0][t][lane] = au[t];
    if (GT) part[w][1][t][lane] = ag[t];
  }
  __syncthreads();
  if (w == 0 && KSP > 1) {                             // partial pre-activations of this share of k
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      f32x4 u = part[0][0][t][lane], g = f32x4{0.f, 0.f, 0.f, 0.f};
      if (GT) g = part[0][1][t][lane];
      for (int ww = 1; ww < KW; ++ww) {
        u += part[ww][0][t][lane];
        if (GT) g += part[ww][1][t][lane];
      }
      const int tok = t * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = i0 + (lane >> 4) * 4 + i;
        if (tok < B && ii < n) {
          const size_t e = (size_t)ii * B + tok;
          pre[(size_t)(2 * ksp) * F * B + e] = u[i];
          if (GT) pre[(size_t)(2 * ksp + 1) * F * B + e] = g[i];
        }
      }
    }
  } else if (w == 0) {
    const float* bp = GT ? bg : bu;
    float bias[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[i] = (bp && idr[i] >= 0) ? bp[idr[i]] : 0.f;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      f32x4 u = part[0][0][t][lane], g = f32x4{0.f, 0.f, 0.f, 0.f};
      if (GT) g = part[0][1][t][lane];
      for (int ww = 1; ww < KW; ++ww) {
        u += part[ww][0][t][lane];
        if (GT) g += part[ww][1][t][lane];
      }
      const int tok = t * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = i0 + (lane >> 4) * 4 + i;
        float a;
        if (GT) {
          a = fmaxf(g[i] + bias[i], 0.f) * u[i];
        } else {
          a = fmaxf(u[i] + bias[i], 0.f);
          if (ACT == 2) a *= a;
        }
        if (tok < B && ii < n) abuf[(size_t)ii * B + tok] = a;
      }
    }
  }
}

// Activations from the k-split partials of k_mt_rows: entry e = i * B + token of the n * B active ones,
// a = act(sum over the KSP shares in order, bias of neuron active[i]).
template <int ACT>
__global__ __launch_bounds__(256) void k_act_combine(const float* __restrict__ pre, int KSP,
                                                     const int32_t* __restrict__ active,
                                                     const int32_t* __restrict__ n_active,
                                                     const float* __restrict__ bias, int B, int F,
                                                     float* __restrict__ abuf) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int n = min(max(*n_active, 0), F);
  if (e >= n * B) return;
  const size_t FB = (size_t)F * B;
  float u = 0.f, g = 0.f;
  for (int k = 0; k < KSP; ++k) {
    u += pre[(size_t)(2 * k) * FB + e];
    if (ACT == 1) g += pre[(size_t)(2 * k + 1) * FB + e];
  }
  const float b = bias ? bias[active[e / B]] : 0.f;
  float a;
  if (ACT == 1) {
    a = fmaxf(g + b, 0.f) * u;
  } else {
    a = fmaxf(u + b, 0.f);
    if (ACT == 2) a *= a;
  }
  abuf[e] = a;
}

constexpr int DN_T = 512;            // 8 waves
constexpr int DS_COLS = 128;         // output columns per block (8 waves x 16)
constexpr int DS_K = 64;             // active rows per step (two 32-row MFMA k steps)

// Partial y over a slice of 128 columns; part_out: [KS][B][D]. Row split ks takes the steps s = ks, ks + KS, ...
// of DS_K consecutive dense indices, reading the ids the row kernel wrote to active[]. All of the block's ids are
// staged in LDS first (one round trip, speculatively up to F); then every step's weight tile, scales and
// activations are loaded into registers ahead of use: two steps ahead in two register sets taken in turn (up to
// 32 tokens), else one step ahead, so each step's round trip overlaps the matrix-core work before it.
template <int NTT, bool Q4>
__global__ __launch_bounds__(DN_T) void k_mt_down(const void* __restrict__ Wd, const void* __restrict__ Sd,
                                                  const int32_t* __restrict__ active,
                                                  const int32_t* __restrict__ n_active,
                                                  const float* __restrict__ abuf, int B, int D, int F,
                                                  float* __restrict__ part_out) {
  extern __shared__ int ids_lds[];                     // [M * DS_K] ids of this block's steps
  __shared__ _Float16 wt[DS_K][DS_COLS + 8];           // fp16 weights or exact (q - 8), padded rows
  __shared__ float at[DS_K][65];                       // activations [row][token]
  __shared__ float st[DS_K][DS_COLS / 32];             // Q4: scales of the slice's 32-column blocks
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int KS = gridDim.y, ks = blockIdx.y;
  const int c0 = blockIdx.x * DS_COLS;
  const int nblk = D >> 5;
  const int M = (F + DS_K * KS - 1) / (DS_K * KS);     // steps of this block at most
  const Buf bw(Wd, Q4 ? (uint32_t)F * (uint32_t)(D >> 1) : (uint32_t)F * D * 2u);
  const Buf bs(Q4 ? Sd : Wd, Q4 ? (uint32_t)F * nblk * 2u : 0u);
  const Buf ba(abuf, (uint32_t)F * B * 4u);
  const Buf bid(active, (uint32_t)F * 4u);
  const Buf bn(n_active, 4u);
  // round 1: all of this block's ids (speculatively, bounded by F: 8 per thread per round, one round for
  // M DS_K <= 4096) and the count, issued after the first round's ids so that one wait covers both
  int v[8];
  auto ids_load = [&](int e0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = e0 + threadIdx.x + DN_T * k;
      const int i = (ks + KS * (e / DS_K)) * DS_K + (e % DS_K);
      v[k] = (int)bid.ldu(boff(e < M * DS_K && i < F, (uint32_t)i * 4u));
    }
  };
  auto ids_store = [&](int e0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = e0 + threadIdx.x + DN_T * k;
      if (e < M * DS_K) ids_lds[e] = v[k];
    }
  };
  ids_load(0);
  const int nraw = (int)bn.ldu(0u);
  ids_store(0);
  for (int e0 = 8 * DN_T; e0 < M * DS_K; e0 += 8 * DN_T) {
    ids_load(e0);
    ids_store(e0);
  }
  const int n = min(max(nraw, 0), F);
  __syncthreads();
  // staging roles: fp16 tiles as 2 x (32 rows x 16 parts of 8 columns); Q4 as 64 rows x 8 half-blocks, scales
  // as 64 rows x 4 blocks; activations 8 per thread
  // two register sets (loads two steps ahead) up to 32 tokens; beyond, the registers they take would leave
  // one block per CU instead of two
  constexpr bool TWO_SETS = NTT <= 2;
  constexpr int NT16 = 16 * NTT;                       // token slots of the activation tile
  constexpr int NAV = DS_K * NT16 / DN_T;              // activation loads per thread per step (2 NTT)
  struct Regs { uint4 w16[2]; uint2 nib; float sc; float av[NAV]; };
  auto load_step = [&](int m, Regs& R) {
    const int base = (ks + KS * m) * DS_K;           // dense index of the step's first row
    if constexpr (Q4) {
      const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
      const int i = base + row;
      const bool ok = i < n;
      const uint32_t id = (uint32_t)ids_lds[ok ? m * DS_K + row : 0];   // i < n: step m is one of the M staged
      const int q = part >> 1, hh = part & 1;
      const int blk = (c0 >> 5) + q;
      R.nib = bw.ld8(boff(ok && blk < nblk, id * (uint32_t)(D >> 1) + (uint32_t)blk * 16u + hh * 8u));
      const int srow = threadIdx.x >> 2, sq = threadIdx.x & 3;
      const int si = base + srow;
      const bool sok = threadIdx.x < DS_K * 4 && si < n && (c0 >> 5) + sq < nblk;
      const uint32_t sid = (uint32_t)ids_lds[sok ? m * DS_K + srow : 0];
      R.sc = bs.ldh(boff(sok, (sid * nblk + (c0 >> 5) + sq) * 2u));
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int row = (threadIdx.x >> 4) + 32 * p, part = threadIdx.x & 15;
        const int i = base + row;
        const int cc = c0 + part * 8;
        const bool ok = i < n && cc < D;
        const uint32_t id = (uint32_t)ids_lds[i < n ? m * DS_K + row : 0];
        R.w16[p] = bw.ld16(boff(ok, (id * D + cc) * 2u));
      }
    }
#pragma unroll
    for (int k = 0; k < NAV; ++k) {
      const int e = threadIdx.x + DN_T * k;            // DS_K * NT16 = NAV * DN_T entries
      const int kr = e / NT16, tok = e % NT16;
      const int i = base + kr;
      R.av[k] = ba.ldf(boff(i < n && tok < B, ((uint32_t)i * B + tok) * 4u));
    }
  };
  auto store_step = [&](const Regs& R) {
    if constexpr (Q4) {
      const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
      const int q = part >> 1, hh = part & 1;
      // 8 nibble bytes = half of a 32-column block: elements 8h..8h+7 (low) and 16+8h..16+8h+7 (high)
      const half8 lo8 = q4_to_half8(R.nib, hh), hi8 = q4_to_half8(R.nib, 2 + hh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wt[row][q * 32 + hh * 8 + e] = lo8[e];
        wt[row][q * 32 + 16 + hh * 8 + e] = hi8[e];
      }
      if (threadIdx.x < DS_K * 4) st[threadIdx.x >> 2][threadIdx.x & 3] = R.sc;
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int row = (threadIdx.x >> 4) + 32 * p, part = threadIdx.x & 15;
        *reinterpret_cast<uint4*>(&wt[row][part * 8]) = R.w16[p];
      }
    }
#pragma unroll
    for (int k = 0; k < NAV; ++k) {
      const int e = threadIdx.x + DN_T * k;
      at[e / NT16][e % NT16] = R.av[k];
    }
  };
  f32x4 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one step: tile to LDS, the step two ahead into the freed registers (branch-free: rows past n read 0), then
  // the matrix-core work while two steps' loads are in flight
  auto step = [&](Regs& R, int mm) {
    store_step(R);
    __syncthreads();
    load_step(mm + (TWO_SETS ? 2 : 1), R);
#pragma unroll
    for (int kc = 0; kc < DS_K / 32; ++kc) {
      // B operand: rows k = 8*(l/16)+i of column 16w + l%16 (read transposed from LDS)
      half8 bop;
#pragma unroll
      for (int i = 0; i < 8; ++i) bop[i] = wt[kc * 32 + (lane >> 4) * 8 + i][w * 16 + (lane & 15)];
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        float av[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kr = kc * 32 + (lane >> 4) * 8 + i;
          float a = at[kr][t * 16 + (lane & 15)];
          if constexpr (Q4) a *= st[kr][w >> 1];         // this wave's 16 columns lie in block w / 2
          av[i] = a;
        }
        half8 ah, al;
        split8(av, ah, al);
        acc[t] = mfma16(al, bop, mfma16(ah, bop, acc[t]));
      }
    }
    __syncthreads();
  };
  // steps of this block: m with (ks + KS m) DS_K < n; taken in pairs so that every loop iteration issues and
  // waits for the same loads (the wait before each tile store then leaves the other set in flight)
  const int nst = max(0, ((n + DS_K - 1) / DS_K - ks + KS - 1) / KS);
  if constexpr (TWO_SETS) {
    Regs R0, R1;
    load_step(0, R0);
    load_step(1, R1);
    int m = 0;
    for (; m + 1 < nst; m += 2) {
      step(R0, m);
      step(R1, m + 1);
    }
    if (m < nst) step(R0, m);
  } else {
    Regs R0;
    load_step(0, R0);
    for (int m = 0; m < nst; ++m) step(R0, m);
  }
  // D layout: lane l holds tokens 16t + 4(l/16) + i of column 16w + l%16
  const int col = c0 + w * 16 + (lane & 15);
#pragma unroll
  for (int t = 0; t < NTT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = t * 16 + (lane >> 4) * 4 + i;
      if (tok < B && col < D) part_out[((size_t)ks * B + tok) * D + col] = acc[t][i];
    }
}

__global__ void k_sum_parts(const float* __restrict__ part, int KS, int n, float* __restrict__ y) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < KS; ++k) s += part[(size_t)k * n + i];
  y[i] = s;
}

template <int NTT>
hipError_t predict_mt(const void* P1, const void* P2, const float* c, const float* x, int B, int D, int F, int r,
                      float tau, int n_hot, uint64_t* mask, float* logits, float* hbuf, float* hpart, int KSH,
                      hipStream_t st) {
  hipError_t e;
  if (KSH > 0) {                                       // else hbuf holds h already
    SFFN_LAUNCH(0, k_mt_h<NTT>, dim3((r + 15) / 16, KSH), dim3(NTK), 0, st, (const uint4*)P1, x, B, D, r, hpart);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nh = B * r;
    hipLaunchKernelGGL(k_sum_parts, dim3((nh + 255) / 256), dim3(256), 0, st, hpart, KSH, nh, hbuf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  SFFN_LAUNCH(1, k_mt_z<NTT>, dim3((F + 63) / 64), dim3(256), 0, st, (const uint4*)P2, c, hbuf, B, F, r, tau, n_hot,
              mask, logits);
  return hipGetLastError();
}

template <int NTT, int ACT, bool Q4>
hipError_t rows_mt(const void* Wg, const void* Sg, const float* bg, const void* Wu, const void* Su, const float* bu,
                   const float* x, int B, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active,
                   float* abuf, float* pre, int KSP, hipStream_t st) {
  const int nw = (F + 63) / 64;
  const int wpt = (nw + NTK - 1) / NTK;
  const size_t lds = (wpt <= WMAXU ? (size_t)((nw + 1) & ~1) * 8 : 0) + (NTK + NTK / 64 + 4) * sizeof(int);
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_mt_rows<NTT, ACT, Q4>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail) return hipErrorInvalidValue;
  if (KSP < 1 || (KSP > 1 && !pre)) return hipErrorInvalidValue;
  SFFN_LAUNCH(2, (k_mt_rows<NTT, ACT, Q4>), dim3((F + 15) / 16 * KSP), dim3(NTK), lds, st, Wg, Sg, bg, Wu, Su, bu, x,
              B, D, F, mask, active, n_active, abuf, pre, KSP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || KSP == 1) return e;
  hipLaunchKernelGGL(k_act_combine<ACT>, dim3((F * B + 255) / 256), dim3(256), 0, st, pre, KSP, active, n_active,
                     ACT == 1 ? bg : bu, B, F, abuf);
  return hipGetLastError();
}

template <int NTT, bool Q4>
hipError_t down_mt(const void* Wd, const void* Sd, const int32_t* active, const int32_t* n_active, const float* abuf,
                   int B, int D, int F, float* part, int KS, float* y, hipStream_t st) {
  const int M = (F + DS_K * KS - 1) / (DS_K * KS);
  const size_t lds = (size_t)M * DS_K * sizeof(int);
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_mt_down<NTT, Q4>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail) return hipErrorInvalidValue;
  SFFN_LAUNCH(3, (k_mt_down<NTT, Q4>), dim3((D + DS_COLS - 1) / DS_COLS, KS), dim3(DN_T), lds, st, Wd, Sd, active,
              n_active, abuf, B, D, F, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = B * D;
  hipLaunchKernelGGL(k_sum_parts, dim3((n + 255) / 256), dim3(256), 0, st, part, KS, n, y);
  return hipGetLastError();
}

}  // namespace

// Activations from KSP shares of partial pre-activations (row kernels with a k split); see k_act_combine.
hipError_t sffn_launch_act_combine(int act, const float* pre, int KSP, const int32_t* active, const int32_t* n_active,
                                   const float* bias, int B, int F, float* abuf, hipStream_t st) {
  const dim3 grid((F * B + 255) / 256);
  if (act == 1) hipLaunchKernelGGL(k_act_combine<1>, grid, dim3(256), 0, st, pre, KSP, active, n_active, bias, B, F, abuf);
  else if (act == 2) hipLaunchKernelGGL(k_act_combine<2>, grid, dim3(256), 0, st, pre, KSP, active, n_active, bias, B, F, abuf);
  else hipLaunchKernelGGL(k_act_combine<0>, grid, dim3(256), 0, st, pre, KSP, active, n_active, bias, B, F, abuf);
  return hipGetLastError();
}

// ---- entry points used by the C ABI for B > 1
hipError_t sffn_launch_norm_tokens(const float* x, int B, int D, float* xn, hipStream_t st) {
  const int xpt = (D / 4 + NTN - 1) / NTN;
  if (xpt <= 1) hipLaunchKernelGGL(k_norm_tokens<1>, dim3(B), dim3(NTN), 0, st, x, D, xn);
  else if (xpt <= 2) hipLaunchKernelGGL(k_norm_tokens<2>, dim3(B), dim3(NTN), 0, st, x, D, xn);
  else if (xpt <= 4) hipLaunchKernelGGL(k_norm_tokens<4>, dim3(B), dim3(NTN), 0, st, x, D, xn);
  else if (xpt <= 8) hipLaunchKernelGGL(k_norm_tokens<8>, dim3(B), dim3(NTN), 0, st, x, D, xn);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t sffn_launch_predict_mt(const void* P1, const void* P2, const float* c, const float* x, int B, int D, int F,
                                  int r, float tau, int n_hot, uint64_t* mask, float* logits, float* hbuf,
                                  float* hpart, int KSH, hipStream_t st) {
  const int ntt = (B + 15) / 16;
  switch (ntt) {
    case 1: return predict_mt<1>(P1, P2, c, x, B, D, F, r, tau, n_hot, mask, logits, hbuf, hpart, KSH, st);
    case 2: return predict_mt<2>(P1, P2, c, x, B, D, F, r, tau, n_hot, mask, logits, hbuf, hpart, KSH, st);
    case 3: return predict_mt<3>(P1, P2, c, x, B, D, F, r, tau, n_hot, mask, logits, hbuf, hpart, KSH, st);
    case 4: return predict_mt<4>(P1, P2, c, x, B, D, F, r, tau, n_hot, mask, logits, hbuf, hpart, KSH, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t sffn_launch_rows_mt(int act, bool q4, const void* Wg, const void* Sg, const float* bg, const void* Wu,
                               const void* Su, const float* bu, const float* x, int B, int D, int F,
                               const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf, float* pre,
                               int KSP, hipStream_t st) {
  const int ntt = (B + 15) / 16;
#define RMT(N, A, Q) \
  return rows_mt<N, A, Q>(Wg, Sg, bg, Wu, Su, bu, x, B, D, F, mask, active, n_active, abuf, pre, KSP, st)
#define RMT_A(N) \
  if (act == 1) { if (q4) RMT(N, 1, true); RMT(N, 1, false); } \
  if (act == 2) { if (q4) RMT(N, 2, true); RMT(N, 2, false); } \
  if (q4) RMT(N, 0, true); \
  RMT(N, 0, false);
  switch (ntt) {
    case 1: RMT_A(1)
    case 2: RMT_A(2)
    case 3: RMT_A(3)
    case 4: RMT_A(4)
    default: return hipErrorInvalidValue;
  }
#undef RMT_A
#undef RMT
}

hipError_t sffn_launch_down_mt(bool q4, const void* Wd, const void* Sd, const int32_t* active,
                               const int32_t* n_active, const float* abuf, int B, int D, int F, float* part, int KS,
                               float* y, hipStream_t st) {
  const int ntt = (B + 15) / 16;
#define DMT(N) return q4 ? down_mt<N, true>(Wd, Sd, active, n_active, abuf, B, D, F, part, KS, y, st) \
                         : down_mt<N, false>(Wd, Sd, active, n_active, abuf, B, D, F, part, KS, y, st)
  switch (ntt) {
    case 1: DMT(1);
    case 2: DMT(2);
    case 3: DMT(3);
    case 4: DMT(4);
    default: return hipErrorInvalidValue;
  }
#undef DMT
}
