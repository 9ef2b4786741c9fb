// Multi-token down projection on the matrix cores: y[b, :] = sum over union rows i of a[i, b] W_downT[active[i], :].
//
// PowerInfer pages, Turkish article, "Neuron-aware operator": only the columns of W_down (rows of W_downT) of the
// union neurons are read, each once for all tokens. As a GEMM, M = tokens, N = D columns, K = union rows, on
// v_mfma_f32_16x16x32_f16 (A: 16 tokens x 32 rows, lane l: token l % 16, rows 8 (l / 16) .. + 8; B: 32 rows x 16
// columns, lane l: column l % 16, the same rows; D: lane l holds tokens 4 (l / 16) + i of column l % 16).
//
// Activations arrive from the row kernels in octet order: a[i, b] at float ((i / 8) * BP + b) * 8 + i % 8, BP the
// token count rounded up to 16, rows past the union and tokens past B zero. An A-operand lane (8 consecutive rows of
// one token) is then 32 contiguous bytes, and a step's 64 rows x BP tokens one contiguous block.
// The weights are stored neuron-major (a neuron's row runs along D) while a B-operand lane needs 8 neurons at one
// column, so every tile is transposed once on its way through LDS.
// k_ud (workgroups of 4 or 8 waves, 256 columns x every token tile, KS workgroups over the union rows, split by the
// device-side union size): the workgroup stages the ids of its share of union rows in LDS, then walks them in steps
// of 64 or 32 rows (two or one MFMA k chunks). Per step each thread loads a piece of W_downT of 4 neurons x 16 or 8
// columns (Q4_0: 8 or 4 nibble bytes and the block scale per neuron; fp16: two 16- or 8-byte loads per neuron) and
// its share of 16-byte pieces of the activations, and writes them, converted to fp16, as operand fragments into LDS
// (8 bytes per column and 4 neurons; 8 bytes per token and 4 rows). Loads run three steps ahead of the matrix-core
// work in four register sets, with no branch in the loop: rows past the union and steps past the share read neuron
// 0's weights against zero activations. The fragment buffers are double-buffered with one barrier per step. Each
// wave multiplies its 64 or 32 columns by every token tile; with 8 waves two share a SIMD, so one's LDS and barrier
// waits overlap the other's matrix-core work.
// Activations enter multiplied by a per-token power of two 2^(15 - e), with 2^e above their largest magnitude over
// the workgroup's share of rows (from the per-64-row maxima the row kernels write), so every value lies inside
// fp16's range with its full precision; the partial sums are scaled back before they are written. Q4_0 weights
// enter as fp16((q - 8) s) (one rounding) with fp16 activations; fp16 weights enter exactly, with the activations as
// one fp16 operand or, EXACT, as two halves (hi + lo). k_sum_parts (union.hip) adds the KS partials in fixed order.
#include "common.h"

using namespace sffn;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const half8& a, const half8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

constexpr int CTD = 256;             // columns per workgroup: 16 column tiles
constexpr int UD_PAD = 7;            // steps of ids past a share: the ring reads up to 6 steps beyond its last

template <int NW, int KR, int NTT, bool Q4, bool EXACT>
__global__ __launch_bounds__(64 * NW) void k_ud(const void* __restrict__ Wd, const void* __restrict__ Sd,
                                            const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
                                            const float* __restrict__ abuf, const float* __restrict__ bmax,
                                            int rbs, int B, int D, int F, int M, float* __restrict__ part) {
  // KR union rows per step (64 or 32: 2 or 1 MFMA k chunks). M: the most 64-row blocks one share can hold (sizes
  // the ids in LDS, with UD_PAD steps of padding); bmax holds the largest |a| per token of every row tile of 2^rbs
  // rows (rbs = 4 or 6)
  static_assert(!(Q4 && EXACT), "Q4_0 weights take fp16 activations");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(KR == 64 || KR == 32, "64 or 32 rows per step");
  constexpr int NTD = 64 * NW;
  constexpr int KC = KR / 32;                          // MFMA k chunks per step
  constexpr int UPQ = NTD / (KR / 4);                  // staging units per neuron quad
  static_assert(UPQ == 16 || UPQ == 32, "16 or 32 units per quad");
  constexpr int CW = 128 / UPQ;                        // columns per staging unit and half block
  constexpr int NHA = EXACT ? 2 : 1;                   // activation planes (hi, lo)
  constexpr int BP = NTT * 16;                         // token stride of the activations
  constexpr int NPC = KR * NTT * 4;                    // 16-byte activation pieces per step
  extern __shared__ __align__(16) int ids[];           // [64 M + UD_PAD KR] ids of this share's union rows
  __shared__ uint4 Bl[2][KC][16][64];                  // weight fragments [buffer][k chunk][column tile][slot]
  __shared__ uint4 Al[2][KC][NTT][NHA][64];            // activation fragments [buffer][k chunk][token tile][plane]
  __shared__ uint2 junk[NPC % NTD ? NHA : 1][NPC % NTD ? NTD : 1];   // landing slots of pieces a thread lacks
  __shared__ float smx[NTD / 64][64];
  __shared__ float inv_s[64];                          // per token: 2^(15 - e), max |a| < 2^e over this share
  __shared__ float scl[64];                            // and its inverse 2^(e - 15)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int KS = gridDim.y, ks = blockIdx.y;
  const int c0 = blockIdx.x * CTD;
  const int nblk = D >> 5;
  // the union rows in KS shares of whole 64-row blocks
  const int n = min(max((int)Buf(n_active, 4u).ldu(0u), 0), F);
  const int Mn = min(((n + 63) / 64 + KS - 1) / KS, M);
  const int total = Mn * 64;
  const int ibase = ks * total;                        // dense index of this workgroup's first row
  // the row-block maxima of this share and the ids (0 past the union and past the share) in one round trip
  {
    const Buf bm(bmax, (uint32_t)((F + (1 << rbs) - 1) >> rbs) * (uint32_t)B * 4u);
    const Buf bid(active, (uint32_t)n * 4u);
    const int tok = threadIdx.x & 63, sub = threadIdx.x >> 6;
    const int ne = Mn << (6 - rbs);                    // table entries (row tiles of 2^rbs rows) of this share
    float m = 0.f;
    for (int b0 = 0; b0 < ne; b0 += 8 * (NTD / 64)) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int b = b0 + sub + (NTD / 64) * k;
        v[k] = bm.ldf(boff(b < ne && tok < B, ((uint32_t)(ks * ne + b) * (uint32_t)B + (uint32_t)tok) * 4u));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int b = b0 + sub + (NTD / 64) * k;
        if (ibase + (b << rbs) < n) m = fmaxf(m, v[k]);   // row tiles past n hold stale maxima
      }
    }
    smx[sub][tok] = m;
    const int tot_p = total + UD_PAD * KR;
    for (int e0 = 0; e0 < tot_p; e0 += 8 * NTD) {
      int v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = e0 + (int)threadIdx.x + NTD * k;
        v[k] = (int)bid.ldu(boff(e < total, (uint32_t)(ibase + e) * 4u));   // 0 past the share
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = e0 + (int)threadIdx.x + NTD * k;
        if (e < tot_p) ids[e] = v[k];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < NTD / 64; ++i) mx = fmaxf(mx, smx[i][t]);
    int ex = 0;
    if (mx > 0.f) (void)frexpf(mx, &ex);
    const int p = min(15 - ex, 126);
    inv_s[t] = ldexpf(1.f, p);
    scl[t] = ldexpf(1.f, -p);
  }
  __syncthreads();
  const int nst = (max(0, min(total, n - ibase)) + KR - 1) / KR;       // steps with rows
  const int nst4 = (nst + 3) / 4 * 4;                  // padded to rounds of four

  // weight roles: a thread stages 4 neurons (quad nq: neurons 4 nq .. + 3 of the step) at CW columns: column
  // unit cu, 32-column block wb = cu / 2, offset wo: columns 32 wb + wo + (0..CW-1) and 32 wb + 16 + wo + (0..CW-1),
  // which Q4_0 holds in the low and high nibbles of the same CW bytes. 16 units per quad (CW = 8): nq = t / 16,
  // cu = t % 16, wo = 8 (cu % 2). 32 units per quad (CW = 4; wave w, lane l): nq = 2 w + l % 2, cu = (l / 2) % 16,
  // wo = 8 (cu % 2) + 4 (l / 32). Either way a half-wave holds both quads of a lane group at 16 distinct columns,
  // so its fragment writes fall in distinct banks.
  const int nq = UPQ == 16 ? (int)threadIdx.x >> 4 : 2 * w + (lane & 1);
  const int cu = UPQ == 16 ? lane & 15 : (lane >> 1) & 15;
  const int wb = cu >> 1, wo = (cu & 1) * 8 + (UPQ == 16 ? 0 : (lane >> 5) * 4);
  const int kcw = nq >> 3, lgw = (nq >> 1) & 3, hfw = nq & 1;   // fragment k chunk, lane group, 8-byte half
  const uint32_t nbytes = Q4 ? (uint32_t)F * (uint32_t)(D >> 1) : (uint32_t)F * (uint32_t)D * 2u;
  const Buf bw(Wd, nbytes);
  const Buf bs(Q4 ? Sd : Wd, Q4 ? (uint32_t)F * (uint32_t)nblk * 2u : 0u);
  const int jb = (c0 >> 5) + wb;                       // the weights' 32-column block
  const int cl = c0 + 32 * wb + wo;
  // per-thread column part of every weight offset; OOB (>= 2^31, above any tensor) for columns past D
  const uint32_t rowb = Q4 ? (uint32_t)(D >> 1) : (uint32_t)D * 2u;
  const uint32_t cb0 = Q4 ? (jb < nblk ? (uint32_t)jb * 16u + (uint32_t)wo : OOB) : (cl < D ? (uint32_t)cl * 2u : OOB);
  const uint32_t cb1 = Q4 ? 0u : (cl + 16 < D ? (uint32_t)(cl + 16) * 2u : OOB);
  const uint32_t cbs = jb < nblk ? (uint32_t)jb * 2u : OOB;
  const int jbx = (c0 >> 5) + ((lane >> 3) & 7);       // the block of the scale this lane loads for its wave
  const uint32_t cbx = jbx < nblk ? (uint32_t)jbx * 2u : OOB;
  // activation roles: the step's block has NPC pieces of 16 bytes; piece g = NTD j + t (j < AP) is octet
  // g / (2 BP), token (g / 2) % BP, half g % 2 (rows 4 (g % 2) .. + 3 of the octet). A thread past the last piece
  // reads nothing (out-of-range offset) and writes its zeros to its own junk slot.
  constexpr int AP = (NPC + NTD - 1) / NTD;
  const int nr = min(((n + 63) >> 6) << 6, ((F + 63) >> 6) << 6);
  const Buf ba(abuf, (uint32_t)nr * (uint32_t)BP * 4u);   // rows past the union's last 64-row block read 0
  uint32_t aoff[AP];
  float asc[AP];
  int aslot[AP];                                       // Al slot in uint2 units within [buffer][plane 0]; -1: none
#pragma unroll
  for (int j = 0; j < AP; ++j) {
    const int g = NTD * j + (int)threadIdx.x;
    const bool real = g < NPC;
    const int oc = g / (2 * BP), tk = (g >> 1) % BP, h = g & 1;
    aoff[j] = real ? ((uint32_t)((ibase >> 3) + oc) * (uint32_t)BP + (uint32_t)tk) * 32u + (uint32_t)h * 16u : OOB;
    asc[j] = real ? inv_s[tk] : 0.f;
    const int kc = oc >> 2, lg = oc & 3;
    aslot[j] = real ? ((((kc * NTT + (tk >> 4)) * NHA) * 64) + (tk & 15) + 16 * lg) * 2 + h : -1;
  }
  const uint32_t astep = (uint32_t)KR * (uint32_t)BP * 4u;     // bytes of one step's activations

  constexpr int QW = CW / 4;                           // Q4_0: 32-bit words of nibble bytes per neuron
  constexpr int HW = CW / 2;                           // fp16: 32-bit words per neuron and half block
  // Q4_0 block scales: with 32 units per quad a wave needs 64 distinct (neuron, block) scales, 4 per lane; lane L
  // loads the one of neuron 4 (2 w + L % 2) + (L / 2) % 4 at column block (L / 8) % 8 and the lanes exchange them
  // (ds_bpermute) instead of each issuing 4 loads of 2 bytes. Same box, 70B: 32 tokens 60.8 -> 48.1 us per layer;
  // at 4 token tiles no gain (65.3 -> 66.3), so those keep the 4 loads.
  constexpr bool SX = Q4 && UPQ == 32 && NTT < 4;
  constexpr int SS = Q4 ? (SX ? 1 : 4) : 1;
  struct Set {
    uint32_t q[Q4 ? 4 : 1][QW];                        // Q4_0: CW nibble bytes per neuron
    uint32_t s[SS];                                    // Q4_0: block scales' fp16 bits
    uint32_t h[Q4 ? 1 : 4][2][HW];                     // fp16: CW + CW columns per neuron
    float4 a[AP];
  };
  // The set's registers are first read in stage, after the previous phase's barrier: the empty asm keeps the
  // compiler from hoisting their conversion next to the loads, which would wait for loads issued one phase ago.
  auto pin = [](Set& S) {
#pragma unroll
    for (int e = 0; e < SS; ++e) asm volatile("" : "+v"(S.s[e]));
#pragma unroll
    for (int e = 0; e < (Q4 ? 4 : 1); ++e) {
#pragma unroll
      for (int k = 0; k < QW; ++k) asm volatile("" : "+v"(S.q[e][k]));
    }
#pragma unroll
    for (int e = 0; e < (Q4 ? 1 : 4); ++e)
#pragma unroll
      for (int k = 0; k < HW; ++k) asm volatile("" : "+v"(S.h[e][0][k]), "+v"(S.h[e][1][k]));
#pragma unroll
    for (int j = 0; j < AP; ++j) asm volatile("" : "+v"(S.a[j].x), "+v"(S.a[j].y), "+v"(S.a[j].z), "+v"(S.a[j].w));
  };
  auto load = [&](int st, Set& S) {
    const int4 id4 = *reinterpret_cast<const int4*>(&ids[st * KR + 4 * nq]);
    const uint32_t id[4] = {(uint32_t)id4.x, (uint32_t)id4.y, (uint32_t)id4.z, (uint32_t)id4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (Q4) {
        if constexpr (QW == 2) {
          const uint2 v = bw.ld8(id[e] * rowb + cb0);
          S.q[e][0] = v.x;
          S.q[e][QW - 1] = v.y;
        } else {
          S.q[e][0] = bw.ldu(id[e] * rowb + cb0);
        }
        if constexpr (!SX) S.s[e] = bs.ldu16(id[e] * (uint32_t)nblk * 2u + cbs);
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t o = id[e] * rowb + (hh ? cb1 : cb0);
          if constexpr (HW == 4) {
            const uint4 v = bw.ld16(o);
            S.h[e][hh][0] = v.x; S.h[e][hh][1] = v.y; S.h[e][hh][HW - 2] = v.z; S.h[e][hh][HW - 1] = v.w;
          } else {
            const uint2 v = bw.ld8(o);
            S.h[e][hh][0] = v.x; S.h[e][hh][HW - 1] = v.y;
          }
        }
      }
    }
    if constexpr (SX) {                                // this lane's one scale of the wave's 64
      const int es = (lane >> 1) & 3;
      const uint32_t ids_ = es == 0 ? id[0] : es == 1 ? id[1] : es == 2 ? id[2] : id[3];
      S.s[0] = bs.ldu16(ids_ * (uint32_t)nblk * 2u + cbx);
    }
    const uint32_t ast = st < nst ? (uint32_t)st * astep : OOB;   // steps past the share's rows read zeros
#pragma unroll
    for (int j = 0; j < AP; ++j) S.a[j] = ba.ldf4(aoff[j] + ast);
  };
  // fragment slots: a column tile's 64 slots hold (lane group g, column c) at 16 g + (c ^ (tile / 2 % 8)), so
  // a 16-lane read stays a permutation of one 256-byte row
  auto stage = [&](Set& S, int buf) {
    pin(S);
    half2v lo[4][HW], hi[4][HW];                       // [neuron][column pair]: columns wo.., 16 + wo..
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (Q4) {
        const uint32_t ex = 0x64646464u;               // v_perm_b32 pool: 0..3 second source, 4..7 first
        const half2v off = {(_Float16)1032.f, (_Float16)1032.f};
        const uint32_t se = SX ? (uint32_t)__shfl((int)S.s[0], (lane & 1) + 2 * e + 8 * wb, 64) : S.s[SX ? 0 : e];
        const half2v s2 = __builtin_bit_cast(half2v, se * 0x10001u);
#pragma unroll
        for (int k = 0; k < QW; ++k) {
          const uint32_t l4 = S.q[e][k] & 0x0F0F0F0Fu, h4 = (S.q[e][k] >> 4) & 0x0F0F0F0Fu;
          lo[e][2 * k] = (__builtin_bit_cast(half2v, __builtin_amdgcn_perm(l4, ex, 0x00050004u)) - off) * s2;
          lo[e][2 * k + 1] = (__builtin_bit_cast(half2v, __builtin_amdgcn_perm(l4, ex, 0x00070006u)) - off) * s2;
          hi[e][2 * k] = (__builtin_bit_cast(half2v, __builtin_amdgcn_perm(h4, ex, 0x00050004u)) - off) * s2;
          hi[e][2 * k + 1] = (__builtin_bit_cast(half2v, __builtin_amdgcn_perm(h4, ex, 0x00070006u)) - off) * s2;
        }
      } else {
#pragma unroll
        for (int p = 0; p < HW; ++p) {
          lo[e][p] = __builtin_bit_cast(half2v, S.h[e][0][p]);
          hi[e][p] = __builtin_bit_cast(half2v, S.h[e][1][p]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int ln = 16 * lgw + ((wo + c) ^ wb);
      const half4 vlo = {lo[0][c >> 1][c & 1], lo[1][c >> 1][c & 1], lo[2][c >> 1][c & 1], lo[3][c >> 1][c & 1]};
      const half4 vhi = {hi[0][c >> 1][c & 1], hi[1][c >> 1][c & 1], hi[2][c >> 1][c & 1], hi[3][c >> 1][c & 1]};
      reinterpret_cast<uint2*>(&Bl[buf][kcw][2 * wb][ln])[hfw] = __builtin_bit_cast(uint2, vlo);
      reinterpret_cast<uint2*>(&Bl[buf][kcw][2 * wb + 1][ln])[hfw] = __builtin_bit_cast(uint2, vhi);
    }
#pragma unroll
    for (int j = 0; j < AP; ++j) {
      const float v[4] = {S.a[j].x * asc[j], S.a[j].y * asc[j], S.a[j].z * asc[j], S.a[j].w * asc[j]};
      half4 vh, vl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vh[e] = (_Float16)v[e];
        vl[e] = (_Float16)(v[e] - (float)vh[e]);
      }
      const bool real = NPC % NTD == 0 || aslot[j] >= 0;
      uint2* al = reinterpret_cast<uint2*>(&Al[buf][0][0][0][0]);
      uint2* dh = real ? &al[aslot[j]] : &junk[0][NPC % NTD ? threadIdx.x : 0];
      *dh = __builtin_bit_cast(uint2, vh);
      if (EXACT) {
        uint2* dl = real ? &al[aslot[j] + 128] : &junk[NPC % NTD ? NHA - 1 : 0][NPC % NTD ? threadIdx.x : 0];
        *dl = __builtin_bit_cast(uint2, vl);
      }
    }
  };
  constexpr int CPW = 16 / NW;                         // column tiles per wave
  f32x4 acc[NTT][CPW];
#pragma unroll
  for (int t = 0; t < NTT; ++t)
#pragma unroll
    for (int c = 0; c < CPW; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      half8 bop[CPW];
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int tile = CPW * w + c;
        bop[c] = __builtin_bit_cast(half8, Bl[buf][kc][tile][(lane & 48) | ((lane & 15) ^ ((tile >> 1) & 7))]);
      }
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        const half8 ah = __builtin_bit_cast(half8, Al[buf][kc][t][0][lane]);
#pragma unroll
        for (int c = 0; c < CPW; ++c) acc[t][c] = mfma16(ah, bop[c], acc[t][c]);
        if constexpr (EXACT) {
          const half8 al = __builtin_bit_cast(half8, Al[buf][kc][t][NHA - 1][lane]);
#pragma unroll
          for (int c = 0; c < CPW; ++c) acc[t][c] = mfma16(al, bop[c], acc[t][c]);
        }
      }
    }
  };
  // four register sets: a phase loads step s + 3, computes step s (fragments in buffer s % 2) and stages step s + 1
  Set S0, S1, S2, S3;
  load(0, S0);
  load(1, S1);
  load(2, S2);
  stage(S0, 0);
  __syncthreads();
  for (int s = 0; s < nst4; s += 4) {
    load(s + 3, S3);
    compute(0);
    stage(S1, 1);
    __syncthreads();
    load(s + 4, S0);
    compute(1);
    stage(S2, 0);
    __syncthreads();
    load(s + 5, S1);
    compute(0);
    stage(S3, 1);
    __syncthreads();
    load(s + 6, S2);
    compute(1);
    stage(S0, 0);
    __syncthreads();
  }
  // partial sums with the tokens' powers of two undone: lane l holds tokens 4 (l / 16) + i of column l % 16 of
  // column tile CPW w + c
#pragma unroll
  for (int t = 0; t < NTT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = t * 16 + (lane >> 4) * 4 + i;
      if (tok >= B) continue;
      const float sc = scl[tok];
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int col = c0 + 16 * CPW * w + 16 * c + (lane & 15);
        if (col < D) part[((size_t)ks * B + tok) * D + col] = acc[t][c][i] * sc;
      }
    }
}

template <int NW, int KR, int NTT, bool Q4, bool EXACT>
hipError_t launch_ud(const void* Wd, const void* Sd, const int32_t* active, const int32_t* n_active,
                     const float* abuf, const float* bmax, int rbs, int B, int D, int F, float* part, int KS, float* y,
                     hipStream_t st) {
  const int M = (F + 64 * KS - 1) / (64 * KS);         // 64-row blocks per workgroup at most
  const size_t lds = ((size_t)M * 64 + (size_t)UD_PAD * KR) * sizeof(int);
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_ud<NW, KR, NTT, Q4, EXACT>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail) return hipErrorInvalidValue;
  SFFN_LAUNCH(3, (k_ud<NW, KR, NTT, Q4, EXACT>), dim3((D + CTD - 1) / CTD, KS), dim3(64 * NW), lds, st, Wd, Sd,
              active, n_active, abuf, bmax, rbs, B, D, F, M, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sffn_launch_sum_parts(part, KS, B * D, y, st);
}

// Waves and rows per step of k_ud by weight format and token tiles. fp16: 4 waves with 32-row steps (half the LDS
// of 64-row steps, so two or three workgroups share a CU) up to 3 token tiles, 8 waves with 64-row steps at 4.
// Q4_0: 64-row steps, 8 waves from 2 token tiles. Same box, one 13B or 70B layer per launch: fp16 4 tokens 13.8 ->
// 12.6 us, 8 tokens 19.7 -> 18.4, 32 tokens 35.4 -> 29.7 (against 8 waves), 40 tokens 44.0 -> 35.0, 64 tokens
// 46.0 -> 46.8; Q4_0 8 tokens 32.6 -> 38.1, 32 tokens 60.4 -> 63.2, 64 tokens 64.2 -> 80.0 (there the 4-wave
// kernel needs 262 registers).
constexpr int ud_waves(bool q4, int ntt) { return ntt >= 4 || (q4 && ntt >= 2) ? 8 : 4; }
constexpr int ud_rows(bool q4, int ntt) { return q4 || ntt >= 4 ? 64 : 32; }

template <int NTT>
hipError_t ud_q(bool q4, bool exact, const void* Wd, const void* Sd, const int32_t* active, const int32_t* n_active,
                const float* abuf, const float* bmax, int rbs, int B, int D, int F, float* part, int KS, float* y,
                hipStream_t st) {
  if (q4)
    return launch_ud<ud_waves(true, NTT), ud_rows(true, NTT), NTT, true, false>(Wd, Sd, active, n_active, abuf, bmax,
                                                                                 rbs, B, D, F, part, KS, y, st);
  if (exact)
    return launch_ud<ud_waves(false, NTT), ud_rows(false, NTT), NTT, false, true>(Wd, Sd, active, n_active, abuf, bmax,
                                                                                   rbs, B, D, F, part, KS, y, st);
  return launch_ud<ud_waves(false, NTT), ud_rows(false, NTT), NTT, false, false>(Wd, Sd, active, n_active, abuf, bmax,
                                                                                  rbs, B, D, F, part, KS, y, st);
}

}  // namespace

// Shares of the union rows for the down projection: enough workgroups of 256 columns to cover the CUs once.
int sffn_ud_shares(int D, int ks_max) {
  const int ct = (D + CTD - 1) / CTD;
  return std::max(1, std::min(ks_max, (256 + ct - 1) / ct));
}

hipError_t sffn_launch_down_ud(bool q4, bool exact, const void* Wd, const void* Sd, const int32_t* active,
                               const int32_t* n_active, const float* abuf, const float* bmax, int rbs, int B, int D,
                               int F, float* part, int KS, float* y, hipStream_t st) {
  if (rbs != 4 && rbs != 6) return hipErrorInvalidValue;
  switch ((B + 15) / 16) {
    case 1: return ud_q<1>(q4, exact, Wd, Sd, active, n_active, abuf, bmax, rbs, B, D, F, part, KS, y, st);
    case 2: return ud_q<2>(q4, exact, Wd, Sd, active, n_active, abuf, bmax, rbs, B, D, F, part, KS, y, st);
    case 3: return ud_q<3>(q4, exact, Wd, Sd, active, n_active, abuf, bmax, rbs, B, D, F, part, KS, y, st);
    case 4: return ud_q<4>(q4, exact, Wd, Sd, active, n_active, abuf, bmax, rbs, B, D, F, part, KS, y, st);
    default: return hipErrorInvalidValue;
  }
}
