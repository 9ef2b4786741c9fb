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
//   k_mt_h        : h = P1 x, 16 rows of P1 per block, k split over 8 waves, LDS reduction
//   k_mt_z        : z = P2 h + c, 64 neurons per block (one mask word), OR over tokens by ballot
//   k_mt_rows     : compaction + W_gate / W_up row gather over 16 active neurons per block, k split over 8
//                   waves, fused activation, dense activations a[i, b]
//   k_mt_down     : y partial sums over a slice of 128 columns and a share of the active rows; W_downT tiles
//                   are staged in LDS and read transposed as the B operand; activations (times the Q4 block
//                   scale) are the A operand
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

constexpr int NTN = 256;

// per-token normalisation (centre, unit variance): one block per token
__global__ __launch_bounds__(NTN) void k_norm_tokens(const float* __restrict__ x, int D, float* __restrict__ xn) {
  __shared__ float red[2 * (NTN / 64)];
  const float* xb = x + (size_t)blockIdx.x * D;
  float* ob = xn + (size_t)blockIdx.x * D;
  const int w = threadIdx.x >> 6;
  float s = 0.f;
  for (int i = threadIdx.x; i < D; i += NTN) s += xb[i];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[w] = s;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < NTN / 64; ++i) t += red[i];
  const float mu = t / (float)D;
  float q = 0.f;
  for (int i = threadIdx.x; i < D; i += NTN) { const float d = xb[i] - mu; q = fmaf(d, d, q); }
  q = wave_sum(q);
  if ((threadIdx.x & 63) == 0) red[NTN / 64 + w] = q;
  __syncthreads();
  float tq = 0.f;
  for (int i = 0; i < NTN / 64; ++i) tq += red[NTN / 64 + i];
  const float sc = 1.0f / sqrtf(tq / (float)D + NORM_EPS);
  for (int i = threadIdx.x; i < D; i += NTN) ob[i] = (xb[i] - mu) * sc;
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

constexpr int NTK = 512;            // 8 waves split the k dimension
constexpr int KW = NTK / 64;

// h[b, j] = sum_d P1[j, d] x[b, d]; block = 16 rows of P1
template <int NTT>
__global__ __launch_bounds__(NTK) void k_mt_h(const uint4* __restrict__ P1, const float* __restrict__ x, int B, int D,
                                              int r, float* __restrict__ h) {
  __shared__ f32x4 part[KW][NTT][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j0 = blockIdx.x * 16;
  const int KB = (D + 31) / 32;
  const int kpw = (KB + KW - 1) / KW;
  const int kb0 = w * kpw, kb1 = min(KB, kb0 + kpw);
  const Buf bp(P1, (uint32_t)r * D * 2u), bx(x, (uint32_t)B * D * 4u);
  const int row = j0 + (lane & 15);
  f32x4 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = kb0; kb < kb1; ++kb) {
    const int k = kb * 32 + (lane >> 4) * 8;
    const uint4 av = bp.ld16(boff(row < r && k < D, ((uint32_t)row * D + k) * 2u));
    half8 xh[NTT], xl[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) load_xtile(bx, B, D, t, kb, xh[t], xl[t]);
    const half8 a = __builtin_bit_cast(half8, av);
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[t] = mfma16(a, xl[t], mfma16(a, xh[t], acc[t]));
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
        if (tok < B && j < r) h[(size_t)tok * r + j] = s[i];
      }
    }
  }
}

// z = P2 h + c; mask word per block (64 neurons = 4 waves x 16)
template <int NTT>
__global__ __launch_bounds__(256) void k_mt_z(const uint4* __restrict__ P2, const float* __restrict__ c,
                                              const float* __restrict__ h, int B, int F, int r, float tau,
                                              uint64_t* __restrict__ mask, float* __restrict__ logits) {
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
  for (int kb = 0; kb < KB; ++kb) {
    const int k = kb * 32 + (lane >> 4) * 8;
    const uint4 av = bp.ld16(boff(row < F && k < r, ((uint32_t)row * r + k) * 2u));
    half8 hh[NTT], hl[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) load_xtile(bh, B, r, t, kb, hh[t], hl[t]);
    const half8 a = __builtin_bit_cast(half8, av);
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[t] = mfma16(a, hl[t], mfma16(a, hh[t], acc[t]));
  }
  // lane l holds rows 4*(l/16)+i of token l%16 (per token tile)
  float cb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = k0 + (lane >> 4) * 4 + i;
    cb[i] = bc.ldf(boff(kk < F, (uint32_t)kk * 4u));
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = k0 + (lane >> 4) * 4 + i;
    bool any = false;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int tok = t * 16 + (lane & 15);
      const float z = acc[t][i] + cb[i];
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

// the i-th set bit of a 64-bit word (i < popcount), by halving
__device__ __forceinline__ int select_bit(uint64_t w, int i) {
  int pos = 0;
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    const uint64_t lowmask = (half == 64) ? ~0ull : ((1ull << half) - 1ull);
    const int c = __popcll(w & lowmask);
    if (i >= c) { i -= c; w >>= half; pos += half; }
    else w &= lowmask;
  }
  return pos;
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
// Q4: W = nibble planes + scale planes. ACT 1 = ReGLU (gate + up), 0 = ReLU (up).
template <int NTT, int ACT, bool Q4>
__global__ __launch_bounds__(NTK) void k_mt_rows(const void* __restrict__ Wg, const void* __restrict__ Sg,
                                                 const float* __restrict__ bg, const void* __restrict__ Wu,
                                                 const void* __restrict__ Su, const float* __restrict__ bu,
                                                 const float* __restrict__ x, int B, int D, int F,
                                                 const uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                 int32_t* __restrict__ n_active, float* __restrict__ abuf) {
  extern __shared__ uint64_t lds64[];
  __shared__ f32x4 part[KW][ACT + 1][NTT][64];
  __shared__ int ids16[16];
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NTK - 1) / NTK;
  const bool words_lds = wpt <= WMAXU;
  uint64_t* wl = lds64;
  int* roff = reinterpret_cast<int*>(wl + (words_lds ? ((nw + 1) & ~1) : 0));
  int* tmp = roff + NTK;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = mask_prefix<NTK, WMAXU>(mask, nw, F, wpt, words_lds ? wl : nullptr, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int i0 = blockIdx.x * 16;
  if (i0 >= n) return;
  const uint64_t* words = words_lds ? wl : mask;
  if (threadIdx.x < 16) {
    const int i = i0 + threadIdx.x;
    const int id = i < n ? locate_lane(words, roff, NTK, wpt, nw, F, i) : -1;
    ids16[threadIdx.x] = id;
    if (id >= 0) active[i] = id;
  }
  __syncthreads();
  const int idl = ids16[lane & 15];                      // A-operand row of this lane (-1: none)
  const int KB = (D + 31) / 32;
  const int kpw = (KB + KW - 1) / KW;
  const int kb0 = w * kpw, kb1 = min(KB, kb0 + kpw);
  const Buf bx(x, (uint32_t)B * D * 4u);
  const int nblk = D >> 5;
  const uint32_t wbytes = Q4 ? (uint32_t)F * (uint32_t)(D >> 1) : (uint32_t)F * D * 2u;
  const uint32_t sbytes = (uint32_t)F * nblk * 2u;
  const Buf bwu(Wu, wbytes), bwg(ACT ? Wg : Wu, ACT ? wbytes : 0u);
  const Buf bsu(Q4 ? Su : Wu, Q4 ? sbytes : 0u), bsg(Q4 && ACT ? Sg : Wu, Q4 && ACT ? sbytes : 0u);
  // rows of this lane's 4 outputs (D layout): 4*(l/16)+i
  int idr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) idr[i] = ids16[(lane >> 4) * 4 + i];
  f32x4 au[NTT], ag[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) { au[t] = f32x4{0.f, 0.f, 0.f, 0.f}; ag[t] = au[t]; }
  for (int kb = kb0; kb < kb1; ++kb) {
    const int k = kb * 32 + (lane >> 4) * 8;
    const bool ok = idl >= 0 && k < D;
    half8 a_u, a_g;
    float su4[4], sg4[4];
    if constexpr (Q4) {
      const uint32_t o = (uint32_t)(ok ? idl : 0) * (uint32_t)(D >> 1) + (uint32_t)kb * 16u + ((lane >> 4) & 1) * 8u;
      a_u = q4_to_half8(bwu.ld8(boff(ok, o)), lane >> 4);
      if (ACT) a_g = q4_to_half8(bwg.ld8(boff(ok, o)), lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool okr = idr[i] >= 0;
        const uint32_t so = ((uint32_t)(okr ? idr[i] : 0) * nblk + kb) * 2u;
        su4[i] = bsu.ldh(boff(okr, so));
        if (ACT) sg4[i] = bsg.ldh(boff(okr, so));
      }
    } else {
      const uint32_t o = ((uint32_t)(ok ? idl : 0) * D + k) * 2u;
      a_u = __builtin_bit_cast(half8, bwu.ld16(boff(ok, o)));
      if (ACT) a_g = __builtin_bit_cast(half8, bwg.ld16(boff(ok, o)));
    }
    half8 xh[NTT], xl[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) load_xtile(bx, B, D, t, kb, xh[t], xl[t]);
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      if constexpr (Q4) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 pu = mfma16(a_u, xl[t], mfma16(a_u, xh[t], z));
#pragma unroll
        for (int i = 0; i < 4; ++i) au[t][i] = fmaf(su4[i], pu[i], au[t][i]);
        if (ACT) {
          const f32x4 pg = mfma16(a_g, xl[t], mfma16(a_g, xh[t], z));
#pragma unroll
          for (int i = 0; i < 4; ++i) ag[t][i] = fmaf(sg4[i], pg[i], ag[t][i]);
        }
      } else {
        au[t] = mfma16(a_u, xl[t], mfma16(a_u, xh[t], au[t]));
        if (ACT) ag[t] = mfma16(a_g, xl[t], mfma16(a_g, xh[t], ag[t]));
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    part[w][0][t][lane] = au[t];
    if (ACT) part[w][ACT][t][lane] = ag[t];
  }
  __syncthreads();
  if (w == 0) {
    const float* bp = ACT ? bg : bu;
    float bias[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[i] = (bp && idr[i] >= 0) ? bp[idr[i]] : 0.f;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      f32x4 u = part[0][0][t][lane], g = f32x4{0.f, 0.f, 0.f, 0.f};
      if (ACT) g = part[0][ACT][t][lane];
      for (int ww = 1; ww < KW; ++ww) {
        u += part[ww][0][t][lane];
        if (ACT) g += part[ww][ACT][t][lane];
      }
      const int tok = t * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = i0 + (lane >> 4) * 4 + i;
        float a;
        if (ACT) a = fmaxf(g[i] + bias[i], 0.f) * u[i];
        else a = fmaxf(u[i] + bias[i], 0.f);
        if (tok < B && ii < n) abuf[(size_t)ii * B + tok] = a;
      }
    }
  }
}

constexpr int DN_T = 512;            // 8 waves
constexpr int DS_COLS = 128;         // output columns per block (8 waves x 16)
constexpr int DS_K = 32;             // active rows per step

// Partial y over a slice of 128 columns and a share of the active rows; part_out: [KS][B][D].
// The whole mask is compacted once per block (nw <= 512 words: one word per lane and wave).
template <int NTT, bool Q4>
__global__ __launch_bounds__(DN_T) void k_mt_down(const void* __restrict__ Wd, const void* __restrict__ Sd,
                                                  const uint64_t* __restrict__ mask, const float* __restrict__ abuf,
                                                  int B, int D, int F, float* __restrict__ part_out) {
  extern __shared__ int list[];                        // [nw * 64] compacted ids
  __shared__ int cnt[DN_T / 64 + 1];
  __shared__ _Float16 wt[DS_K][DS_COLS + 8];           // fp16 weights or exact (q - 8), padded rows
  __shared__ float at[DS_K][65];                       // activations [row][token]
  __shared__ float st[DS_K][DS_COLS / 32];             // Q4: scales of the slice's 32-column blocks
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nw = (F + 63) >> 6;
  const int KS = gridDim.y, ks = blockIdx.y;
  const int c0 = blockIdx.x * DS_COLS;
  const int nblk = D >> 5;
  const Buf bm(mask, (uint32_t)nw * 8u);
  const Buf bw(Wd, Q4 ? (uint32_t)F * (uint32_t)(D >> 1) : (uint32_t)F * D * 2u);
  const Buf bs(Q4 ? Sd : Wd, Q4 ? (uint32_t)F * nblk * 2u : 0u);
  const Buf ba(abuf, (uint32_t)F * B * 4u);
  const int wpw = (nw + DN_T / 64 - 1) / (DN_T / 64);  // <= 64 (host keeps nw <= 512)
  const int tw = w * wpw + lane;
  const uint64_t cw = bm.ldu64(boff(lane < wpw && tw < nw, (uint32_t)tw * 8u));
  const int total = compact_words<DN_T>(cw, 0, nw, wpw, nw, F, list, cnt);
  const int per_ks = (total + KS - 1) / KS;
  const int j0 = ks * per_ks, j1 = min(total, j0 + per_ks);
  f32x4 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int srow = threadIdx.x >> 4, spart = threadIdx.x & 15;   // staging: 32 rows x 16 parts
  for (int jb = j0; jb < j1; jb += DS_K) {
    {
      const int j = jb + srow;
      const bool ok = j < j1;
      const uint32_t id = ok ? (uint32_t)list[j] : 0u;
      if constexpr (Q4) {
        if (spart < 8) {
          // 8 nibble bytes = half of a 32-column block: elements 8h..8h+7 (low) and 16+8h..16+8h+7 (high)
          const int q = spart >> 1, hh = spart & 1;
          const int blk = (c0 >> 5) + q;
          const uint2 pbytes = bw.ld8(boff(ok && blk < nblk, id * (uint32_t)(D >> 1) + (uint32_t)blk * 16u + hh * 8u));
          const half8 lo8 = q4_to_half8(pbytes, hh), hi8 = q4_to_half8(pbytes, 2 + hh);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            wt[srow][q * 32 + hh * 8 + e] = lo8[e];
            wt[srow][q * 32 + 16 + hh * 8 + e] = hi8[e];
          }
        } else if (spart < 8 + DS_COLS / 32) {
          const int q = spart - 8;
          const int blk = (c0 >> 5) + q;
          st[srow][q] = bs.ldh(boff(ok && blk < nblk, (id * nblk + blk) * 2u));
        }
      } else {
        const int cc = c0 + spart * 8;
        const uint4 v = bw.ld16(boff(ok && cc < D, (id * D + cc) * 2u));
        *reinterpret_cast<uint4*>(&wt[srow][spart * 8]) = v;
      }
      for (int e = threadIdx.x; e < DS_K * 64; e += DN_T) {
        const int kr = e >> 6, tok = e & 63;
        const int jj = jb + kr;
        at[kr][tok] = ba.ldf(boff(jj < j1 && tok < B, ((uint32_t)jj * B + tok) * 4u));
      }
    }
    __syncthreads();
    // B operand: rows k = 8*(l/16)+i of column 16w + l%16 (read transposed from LDS)
    half8 bop;
#pragma unroll
    for (int i = 0; i < 8; ++i) bop[i] = wt[(lane >> 4) * 8 + i][w * 16 + (lane & 15)];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      float av[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kr = (lane >> 4) * 8 + i;
        float a = at[kr][t * 16 + (lane & 15)];
        if constexpr (Q4) a *= st[kr][w >> 1];           // this wave's 16 columns lie in block w / 2
        av[i] = a;
      }
      half8 ah, al;
      split8(av, ah, al);
      acc[t] = mfma16(al, bop, mfma16(ah, bop, acc[t]));
    }
    __syncthreads();
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
                      float tau, uint64_t* mask, float* logits, float* hbuf, hipStream_t st) {
  SFFN_LAUNCH(0, k_mt_h<NTT>, dim3((r + 15) / 16), dim3(NTK), 0, st, (const uint4*)P1, x, B, D, r, hbuf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SFFN_LAUNCH(1, k_mt_z<NTT>, dim3((F + 63) / 64), dim3(256), 0, st, (const uint4*)P2, c, hbuf, B, F, r, tau, mask,
                     logits);
  return hipGetLastError();
}

template <int NTT, int ACT, bool Q4>
hipError_t rows_mt(const void* Wg, const void* Sg, const float* bg, const void* Wu, const void* Su, const float* bu,
                   const float* x, int B, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active,
                   float* abuf, hipStream_t st) {
  const int nw = (F + 63) / 64;
  const int wpt = (nw + NTK - 1) / NTK;
  const size_t lds = (wpt <= WMAXU ? (size_t)((nw + 1) & ~1) * 8 : 0) + (NTK + NTK / 64 + 4) * sizeof(int);
  static size_t avail = 0;
  if (!avail) {
    hipError_t ea = allow_dynamic_lds((const void*)k_mt_rows<NTT, ACT, Q4>, &avail);
    if (ea != hipSuccess) return ea;
  }
  if (lds > avail) return hipErrorInvalidValue;
  SFFN_LAUNCH(2, (k_mt_rows<NTT, ACT, Q4>), dim3((F + 15) / 16), dim3(NTK), lds, st, Wg, Sg, bg, Wu, Su, bu, x, B,
                     D, F, mask, active, n_active, abuf);
  return hipGetLastError();
}

template <int NTT, bool Q4>
hipError_t down_mt(const void* Wd, const void* Sd, const uint64_t* mask, const float* abuf, int B, int D, int F,
                   float* part, int KS, float* y, hipStream_t st) {
  const int nw = (F + 63) / 64;
  const size_t lds = (size_t)nw * 64 * sizeof(int);
  static size_t avail = 0;
  if (!avail) {
    hipError_t ea = allow_dynamic_lds((const void*)k_mt_down<NTT, Q4>, &avail);
    if (ea != hipSuccess) return ea;
  }
  if (lds > avail) return hipErrorInvalidValue;
  SFFN_LAUNCH(3, (k_mt_down<NTT, Q4>), dim3((D + DS_COLS - 1) / DS_COLS, KS), dim3(DN_T), lds, st, Wd, Sd, mask,
                     abuf, B, D, F, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = B * D;
  hipLaunchKernelGGL(k_sum_parts, dim3((n + 255) / 256), dim3(256), 0, st, part, KS, n, y);
  return hipGetLastError();
}

}  // namespace

// ---- entry points used by the C ABI for B > 1
hipError_t sffn_launch_norm_tokens(const float* x, int B, int D, float* xn, hipStream_t st) {
  hipLaunchKernelGGL(k_norm_tokens, dim3(B), dim3(NTN), 0, st, x, D, xn);
  return hipGetLastError();
}

hipError_t sffn_launch_predict_mt(const void* P1, const void* P2, const float* c, const float* x, int B, int D, int F,
                                  int r, float tau, uint64_t* mask, float* logits, float* hbuf, hipStream_t st) {
  const int ntt = (B + 15) / 16;
  switch (ntt) {
    case 1: return predict_mt<1>(P1, P2, c, x, B, D, F, r, tau, mask, logits, hbuf, st);
    case 2: return predict_mt<2>(P1, P2, c, x, B, D, F, r, tau, mask, logits, hbuf, st);
    case 3: return predict_mt<3>(P1, P2, c, x, B, D, F, r, tau, mask, logits, hbuf, st);
    case 4: return predict_mt<4>(P1, P2, c, x, B, D, F, r, tau, mask, logits, hbuf, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t sffn_launch_rows_mt(int act, bool q4, const void* Wg, const void* Sg, const float* bg, const void* Wu,
                               const void* Su, const float* bu, const float* x, int B, int D, int F,
                               const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf, hipStream_t st) {
  const int ntt = (B + 15) / 16;
#define RMT(N, A, Q) return rows_mt<N, A, Q>(Wg, Sg, bg, Wu, Su, bu, x, B, D, F, mask, active, n_active, abuf, st)
#define RMT_A(N) \
  if (act == 1) { if (q4) RMT(N, 1, true); RMT(N, 1, false); } \
  else { if (q4) RMT(N, 0, true); RMT(N, 0, false); }
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

hipError_t sffn_launch_down_mt(bool q4, const void* Wd, const void* Sd, const uint64_t* mask, const float* abuf, int B,
                               int D, int F, float* part, int KS, float* y, hipStream_t st) {
  const int ntt = (B + 15) / 16;
#define DMT(N) return q4 ? down_mt<N, true>(Wd, Sd, mask, abuf, B, D, F, part, KS, y, st) \
                         : down_mt<N, false>(Wd, Sd, mask, abuf, B, D, F, part, KS, y, st)
  switch (ntt) {
    case 1: DMT(1);
    case 2: DMT(2);
    case 3: DMT(3);
    case 4: DMT(4);
    default: return hipErrorInvalidValue;
  }
#undef DMT
}
