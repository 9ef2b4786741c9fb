// Multi-token (union-mask) path, B > 1: the predictor on the matrix cores, and the small kernels around the
// union row and down projections (union_rows.hip, union_down.hip).
//
// The pages' decode is one token at a time; with several tokens the predicted-active sets are merged (one
// mask, the union over tokens) and every token is computed over that union, so each active row of the
// weights is read once for the whole batch ("Neuron-aware operator", Turkish article). The predictor's two
// stages are small GEMMs, so they run on v_mfma_f32_16x16x32_f16:
//   A operand: 16 weight rows x 32 k (lane l: row l % 16, k 8*(l/16)..+8 -- one 16-byte load of a neuron-major
//              row), B operand: 32 k x 16 tokens (lane l: token l % 16), D: 16 rows x 16 tokens (lane l holds
//              rows 4*(l/16)+i of token l % 16).
// fp32 token values enter as two fp16 halves, x = hi + lo (hi = fp16(x), lo = fp16(x - hi)); P1 and P2 are fp16,
// so every product is exact and accumulation is fp32, like the single-token path.
//
// Kernels:
//   k_norm_tokens : per-token normalisation of x into the workspace (when the layer input is normalised)
//   k_mt_h        : partial h = P1 x over a share of d, 16 rows of P1 per block, shares over blocks (grid y),
//                   split again over 8 waves with an LDS reduction; k_sum_parts adds the shares in fixed order
//   k_mt_z        : z = P2 h + c, 64 neurons per block (one mask word), OR over tokens by ballot
//   k_act_combine : activations from the row kernel's k shares (union_rows.hip), in octet order
//   k_sum_parts   : y = sum of the partial sums (also those of the down projection, union_down.hip)
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
// mh_tiles(NTT) rows of P1 and one share of the k range, split again over the 8 waves. Every lane's tokens (loaded
// and split once per k block) serve the block's row tiles, so two row tiles per block halve the reads of x, which
// outweigh P1's from 2 token tiles on (70B, 64 tokens: 14.3 -> 11.0 us; 13B, 16 tokens: 6.4 -> 6.6 us).
constexpr int mh_tiles(int ntt) { return ntt >= 2 ? 2 : 1; }

template <int NTT>
__global__ __launch_bounds__(NTK) void k_mt_h(const uint4* __restrict__ P1, const float* __restrict__ x, int B, int D,
                                              int r, float* __restrict__ hp) {
  constexpr int RT = mh_tiles(NTT);
  __shared__ f32x4 part[KW][RT][NTT][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j0 = blockIdx.x * 16 * RT;
  const int KB = (D + 31) / 32;
  const int KSH = gridDim.y, ks = blockIdx.y;
  const int kps = (KB + KSH - 1) / KSH;                  // k blocks of this share
  const int ks0 = ks * kps, ks1 = min(KB, ks0 + kps);
  const int kpw = (kps + KW - 1) / KW;
  const int kb0 = ks0 + w * kpw, kb1 = min(ks1, kb0 + kpw);
  const Buf bp(P1, (uint32_t)r * D * 2u), bx(x, (uint32_t)B * D * 4u);
  f32x4 acc[RT][NTT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int CH = KChunk<NTT>::CH;
  for (int c0 = kb0; c0 < kb1; c0 += CH) {
    uint4 av[CH][RT];
    XRaw xr[CH][NTT];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int kb = c0 + q;
      const int k = kb * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int row = j0 + 16 * rt + (lane & 15);
        av[q][rt] = bp.ld16(boff(kb < kb1 && row < r && k < D, ((uint32_t)row * D + k) * 2u));
      }
#pragma unroll
      for (int t = 0; t < NTT; ++t) xr[q][t] = load_xraw(bx, B, kb < kb1 ? D : 0, t, kb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        half8 xh, xl;
        split_xraw(xr[q][t], xh, xl);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const half8 a = __builtin_bit_cast(half8, av[q][rt]);
          acc[rt][t] = mfma16(a, xl, mfma16(a, xh, acc[rt][t]));
        }
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NTT; ++t) part[w][rt][t][lane] = acc[rt][t];
  __syncthreads();
  if (w < RT) {                                        // wave rt adds row tile rt's partials in wave order
    const int rt = w;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      f32x4 s = part[0][rt][t][lane];
      for (int ww = 1; ww < KW; ++ww) s += part[ww][rt][t][lane];
      const int tok = t * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 16 * rt + (lane >> 4) * 4 + i;
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

// Activations from the k-split partials of the row kernels: one workgroup per 64 union rows; pre holds entry
// e = i * B + token of the n * B active ones, a = act(sum over the KSP shares in order, bias of neuron active[i]).
// The 64 x BP tile (BP = B rounded up to 16) is written whole in octet order, a[i, b] at
// ((i / 8) * BP + b) * 8 + i % 8, zero past n and B; bmax receives the tile's largest |a| per token,
// bmax[(i / 64) * B + token].
constexpr int KSP_MAX = 8;           // k shares of the union row kernel at most

template <int ACT>
__global__ __launch_bounds__(256) void k_act_combine(const float* __restrict__ pre, int KSP,
                                                     const int32_t* __restrict__ active,
                                                     const int32_t* __restrict__ n_active,
                                                     const float* __restrict__ bias, int B, int F,
                                                     float* __restrict__ abuf, float* __restrict__ bmax) {
  __shared__ uint32_t smx[64];
  const int n = min(max(*n_active, 0), F);
  const int i0 = blockIdx.x * 64;
  if (i0 >= n) return;                                 // block-uniform
  if (threadIdx.x < 64) smx[threadIdx.x] = 0u;
  __syncthreads();
  const int BP = (B + 15) & ~15;
  const uint32_t FB = (uint32_t)F * (uint32_t)B;
  const Buf bp(pre, (uint32_t)KSP * 2u * FB * 4u), bid(active, (uint32_t)F * 4u);
  const Buf bbi(bias ? (const void*)bias : (const void*)pre, bias ? (uint32_t)F * 4u : 0u);   // no bias: 0
  // groups of 4 elements per thread: every share's loads and the row ids in one round trip, the biases in a
  // second (an element at a time, the row id and bias loads had made two dependent round trips per element)
  constexpr int EG = 4;
  for (int g0 = 0; g0 < 64 * BP; g0 += 256 * EG) {   // block-uniform
    float vu[EG][KSP_MAX], vg[EG][KSP_MAX];
    int id[EG];
    bool ok[EG];
#pragma unroll
    for (int j = 0; j < EG; ++j) {
      const int q = g0 + j * 256 + (int)threadIdx.x;
      const int b = (q >> 3) % BP, i = i0 + (q / (8 * BP)) * 8 + (q & 7);
      ok[j] = q < 64 * BP && i < n && b < B;
      const uint32_t e = ok[j] ? (uint32_t)i * (uint32_t)B + (uint32_t)b : 0u;
#pragma unroll
      for (int k = 0; k < KSP_MAX; ++k) {
        vu[j][k] = bp.ldf(boff(ok[j] && k < KSP, ((uint32_t)(2 * k) * FB + e) * 4u));
        vg[j][k] = ACT == 1 ? bp.ldf(boff(ok[j] && k < KSP, ((uint32_t)(2 * k + 1) * FB + e) * 4u)) : 0.f;
      }
      id[j] = (int)bid.ldu(boff(ok[j], (uint32_t)(ok[j] ? i : 0) * 4u));
    }
    float bi[EG];
#pragma unroll
    for (int j = 0; j < EG; ++j) bi[j] = bbi.ldf(boff(ok[j], (uint32_t)id[j] * 4u));
#pragma unroll
    for (int j = 0; j < EG; ++j) {
      const int q = g0 + j * 256 + (int)threadIdx.x;
      float a = 0.f;
      if (ok[j]) {
        float u = 0.f, g = 0.f;
#pragma unroll
        for (int k = 0; k < KSP_MAX; ++k) {          // in share order (shares past KSP read 0)
          u += vu[j][k];
          if (ACT == 1) g += vg[j][k];
        }
        if (ACT == 1) {
          a = fmaxf(g + bi[j], 0.f) * u;
        } else {
          a = fmaxf(u + bi[j], 0.f);
          if (ACT == 2) a *= a;
        }
        atomicMax(&smx[(q >> 3) % BP], __float_as_uint(fabsf(a)));   // LDS; non-negative floats order as bits
      }
      if (q < 64 * BP) abuf[(size_t)i0 * BP + q] = a;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < B) bmax[(size_t)blockIdx.x * B + threadIdx.x] = __uint_as_float(smx[threadIdx.x]);
}

// Every share's load is issued before the first add (a loop over the runtime KS had each load wait for the
// previous one: one round trip per share), then the shares are added in order.
constexpr int SUM_PARTS_MAX = 16;
__global__ __launch_bounds__(256) void k_sum_parts(const float* __restrict__ part, int KS, int n,
                                                   float* __restrict__ y) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const Buf bp(part, (uint32_t)KS * (uint32_t)n * 4u);
  float v[SUM_PARTS_MAX];
#pragma unroll
  for (int k = 0; k < SUM_PARTS_MAX; ++k) v[k] = bp.ldf(boff(i < n && k < KS, ((uint32_t)k * (uint32_t)n + i) * 4u));
  if (i >= n) return;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < SUM_PARTS_MAX; ++k)
    if (k < KS) s += v[k];
  y[i] = s;
}

template <int NTT>
hipError_t predict_mt(const void* P1, const void* P2, const float* c, const float* x, int B, int D, int F, int r,
                      float tau, int n_hot, uint64_t* mask, float* logits, float* hbuf, float* hpart, int KSH,
                      void* hf, float* hs, hipStream_t st) {
  hipError_t e;
  if (KSH > 0) {                                       // else hbuf holds h already
    SFFN_LAUNCH(0, k_mt_h<NTT>, dim3((r + 16 * mh_tiles(NTT) - 1) / (16 * mh_tiles(NTT)), KSH), dim3(NTK), 0, st,
                (const uint4*)P1, x, B, D, r, hpart);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (hf)                                            // the split adds the partials itself (one launch fewer)
      return sffn_launch_predict_mz(P2, c, hpart, KSH, B, F, r, tau, n_hot, mask, logits, hf, hs, st);
    const int nh = B * r;
    if (KSH > SUM_PARTS_MAX || (size_t)KSH * nh * 4 >= ((size_t)1 << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_sum_parts, dim3((nh + 255) / 256), dim3(256), 0, st, hpart, KSH, nh, hbuf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (hf)                                              // h split once, P2 streamed on the 64-row tiling
    return sffn_launch_predict_mz(P2, c, hbuf, 0, B, F, r, tau, n_hot, mask, logits, hf, hs, st);
  SFFN_LAUNCH(1, k_mt_z<NTT>, dim3((F + 63) / 64), dim3(256), 0, st, (const uint4*)P2, c, hbuf, B, F, r, tau, n_hot,
              mask, logits);
  return hipGetLastError();
}

}  // namespace

// Activations from KSP shares of partial pre-activations (row kernels with a k split); see k_act_combine.
hipError_t sffn_launch_act_combine(int act, const float* pre, int KSP, const int32_t* active, const int32_t* n_active,
                                   const float* bias, int B, int F, float* abuf, float* bmax, hipStream_t st) {
  if (KSP < 1 || KSP > KSP_MAX || (size_t)KSP * 2 * F * B * 4 >= ((size_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((F + 63) / 64), blk(256);
  if (act == 1) hipLaunchKernelGGL(k_act_combine<1>, grid, blk, 0, st, pre, KSP, active, n_active, bias, B, F, abuf, bmax);
  else if (act == 2) hipLaunchKernelGGL(k_act_combine<2>, grid, blk, 0, st, pre, KSP, active, n_active, bias, B, F, abuf, bmax);
  else hipLaunchKernelGGL(k_act_combine<0>, grid, blk, 0, st, pre, KSP, active, n_active, bias, B, F, abuf, bmax);
  return hipGetLastError();
}

// y[i] = sum of the KS partials part[k * n + i], in share order
hipError_t sffn_launch_sum_parts(const float* part, int KS, int n, float* y, hipStream_t st) {
  if (KS < 1 || KS > SUM_PARTS_MAX || (size_t)KS * n * 4 >= ((size_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sum_parts, dim3((n + 255) / 256), dim3(256), 0, st, part, KS, n, y);
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
                                  float* hpart, int KSH, void* hf, float* hs, hipStream_t st) {
  const int ntt = (B + 15) / 16;
#define PMT(N) return predict_mt<N>(P1, P2, c, x, B, D, F, r, tau, n_hot, mask, logits, hbuf, hpart, KSH, hf, hs, st)
  switch (ntt) {
    case 1: PMT(1);
    case 2: PMT(2);
    case 3: PMT(3);
    case 4: PMT(4);
    default: return hipErrorInvalidValue;
  }
#undef PMT
}
