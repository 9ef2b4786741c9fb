// Single-token sparse FFN in one pass over the active rows: row gather, activation and column gather fused.
//
// PowerInfer pages, Turkish article, "Neuron-aware operator": only the rows of W_gate / W_up and of W_downT that
// belong to predicted-active neurons are read. Here each neuron's three rows are read in the same memory round
// trip, and the down projection is accumulated where the activation is computed, so the activations never go
// through memory and the column gather needs no launch of its own.
//
// k_fused1 (up to 256 blocks of 8 waves): round 1 loads x and the mask words; a block scan gives each thread the
// set bits before its mask word and the active count n. G = max(64, ceil(n / 8)) of the blocks (at most all) take
// rows, so that a block's rows fill one pass; dense index i goes to block i % G, a near-equal share each. A
// block's rows are G apart in dense order, so a mask word holds at most one of them: each thread finds its word's
// one by a rank select, and the block has the ids of all its rows in LDS at once. The gather (rowgather.h,
// shared with the folded kernel of decode.hip): per pass of 8 rows, each wave
// issues the loads of its row of W_gate / W_up and every thread the loads of its 16-byte chunks of the pass's 8
// rows of W_downT, all together and before x is normalised and staged. Each wave reduces its row dot products to
// the activation a_i; the 8 activations go through LDS and every thread adds a_i * W_downT[id_i, its chunks] in
// row order. The block's partial sum of y over its rows is written to part[block][D].
// k_fused1_q4: the same for Q4_0 rows (nibbles and fp16 block scales). x is scaled by a power of two (from its
// largest magnitude) and staged in LDS as fp16, in pieces laid out so that the lane of a Q4 block reads its 32
// values without bank conflicts; each pair of nibbles becomes exact fp16 (q - 8) and meets its pair of x in a
// packed dot product (v_dot2, exact products, fp32 sum). The pass's W_downT nibble rows are loaded straight into
// LDS (buffer loads with the LDS destination) instead of registers.
// k_sum_rows: y[d] = sum over the blocks b < min(G, n) that took rows of part[b][d] in a fixed order (16 groups per
// column, each summed in block order, then the groups in order); all of a thread's loads are issued together.
// Every sum has a fixed order, so the results do not depend on timing.
#include "common.h"
#include "rowgather.h"

using namespace sffn;

namespace {

constexpr int NT_F = 512;            // 8 waves: rows per block pass
constexpr int FW = NT_F / 64;
constexpr int WMAX_F = 1;            // mask words per thread kept in LDS (nw <= 512)
#ifndef SFFN_Q4_FUSED_RPW
#define SFFN_Q4_FUSED_RPW 1          // Q4_0 rows per wave per pass (measured best at the 70B shape: 1, over 2 and 3)
#endif

// The blocks that take rows, out of the Gmax launched, for n active rows: just enough for one pass of `pass` rows
// each (at least 64, so that a mask word holds at most one row of a block). Fuller blocks mean fewer partial sums
// of y and fewer idle slots in a pass (same box, one pass per block: 13B 1011 -> 1040, 40B 493 -> 499 tokens/s
// against all 256). k_sum_rows takes the same count from n.
__device__ __forceinline__ int fused_blocks(int n, int Gmax, int pass) {
  return min(Gmax, max(64, (n + pass - 1) / pass));
}
// The most rows a block can take (the length of its row-id list in LDS): one pass while n <= pass * Gmax, else
// ceil(n / Gmax) <= ceil(F / Gmax).
__host__ __device__ __forceinline__ int fused_max_rows(int F, int Gmax, int pass) {
  return max(pass, (F + Gmax - 1) / Gmax);
}

template <int ACT, int NCH, int DCH>
__global__ __launch_bounds__(NT_F) void k_fused1(const uint4* __restrict__ Wg, const float* __restrict__ bg,
                                                 const uint4* __restrict__ Wu, const float* __restrict__ bu,
                                                 const uint4* __restrict__ WdT, const float* __restrict__ x,
                                                 int x_norm, int D, int F, const uint64_t* __restrict__ mask,
                                                 int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                                 float* __restrict__ part) {
  extern __shared__ uint64_t lds64[];
  const int nw = (F + 63) >> 6;
  uint64_t* wl = lds64;                                                  // [nw] mask words
  int* roff = reinterpret_cast<int*>(wl + ((nw + 1) & ~1));              // [NT_F] range offsets
  int* tmp = roff + NT_F;                                                // [NT_F/64 + 1] scan scratch
  float* av = reinterpret_cast<float*>(tmp + NT_F / 64 + 4);             // [FW] activations of the pass
  float* red = av + FW;                                                  // [2 * FW] normalisation scratch
  float* xs = red + 2 * FW + 4;                                          // [D] x (16-byte aligned)
  int* bids = reinterpret_cast<int*>(xs + D);                            // [fused_max_rows] the block's row ids
  const int n4 = D >> 2;
  constexpr int XPT = (128 * NCH + NT_F - 1) / NT_F;   // float4 of x per thread: D / 4 <= 128 * NCH

  // round 1: x and the mask words, all loads issued before any use
  float4 xv4[XPT];
  stage_load<NT_F, XPT>(x, n4, xv4);
  const float x0 = x[0];                               // shift for the single-pass statistics
  const int n = mask_prefix<NT_F, WMAX_F>(mask, nw, F, 1, wl, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int G = fused_blocks(n, gridDim.x, FW);
  if ((int)blockIdx.x >= min(G, n)) return;           // block-uniform: no row here; its partial is never read
  // the block's rows: dense indices blk + G * k, k < nrow, their ids in LDS (one rank select per mask word)
  const int blk = blockIdx.x;
  const int nrow = (n - blk + G - 1) / G;
  block_row_ids(wl, roff, nw, blk, G, bids);
  lds_barrier();
  gather_rows<ACT, NCH, DCH, NT_F, XPT, true>(bids, nrow, Wg, bg, Wu, bu, WdT, D, F, x_norm, x0, xv4, xs, red, av,
                                              part, active, blk, G);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// the fp16 value whose bits are the low half of s, widened
__device__ __forceinline__ float h16f(uint32_t s) { return (float)__builtin_bit_cast(_Float16, (uint16_t)s); }

// sum over a Q4 block of (q_e - 8) x_e: nib = the block's 16 nibble bytes (byte i: element i low, 16 + i high);
// xp[j] = x[4 j .. 4 j + 3] as two fp16 pairs. v_perm_b32 puts each nibble byte under the exponent byte 0x64 (byte
// pool: selector 0..3 = second source, 4..7 = first source), 1032 is subtracted exactly, and v_dot2 multiplies
// the pairs (exact products) into an fp32 sum.
__device__ __forceinline__ float q4_dot_x16(const uint4& nib, const half2v (&xp)[8][2]) {
  const uint32_t wds[4] = {nib.x, nib.y, nib.z, nib.w};
  const uint32_t e = 0x64646464u;
  const half2v off = {(_Float16)1032.f, (_Float16)1032.f};
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = wds[k] & 0x0F0F0F0Fu, hi = (wds[k] >> 4) & 0x0F0F0F0Fu;
    const half2v a0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(lo, e, 0x00050004u)) - off;
    const half2v a1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(lo, e, 0x00070006u)) - off;
    const half2v a2 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hi, e, 0x00050004u)) - off;
    const half2v a3 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hi, e, 0x00070006u)) - off;
    s = __builtin_amdgcn_fdot2(a0, xp[k][0], s, false);
    s = __builtin_amdgcn_fdot2(a1, xp[k][1], s, false);
    s = __builtin_amdgcn_fdot2(a2, xp[4 + k][0], s, false);
    s = __builtin_amdgcn_fdot2(a3, xp[4 + k][1], s, false);
  }
  return s;
}

// Q4_0 form: gate/up rows as nibbles + block scales, dotted with x in packed fp16 (q4_dot_x16); thread t owns
// half-block t of every W_downT row (8 nibble bytes = 16 columns, and the block scale), takes each nibble as the
// exact fp16 1024 + q in an fp32 FMA, and carries sum(a * s) for the "- 1032" of its columns. NQ: Q4 blocks per lane of a row; D <= 32 * NT_F (one half-block per thread).
template <int ACT, int NQ, int RPW>
__global__ __launch_bounds__(NT_F) void k_fused1_q4(const uint4* __restrict__ qg, const _Float16* __restrict__ sg,
                                                    const float* __restrict__ bg, const uint4* __restrict__ qu,
                                                    const _Float16* __restrict__ su, const float* __restrict__ bu,
                                                    const uint8_t* __restrict__ qd, const _Float16* __restrict__ sd,
                                                    const float* __restrict__ x, int x_norm, int D, int F,
                                                    const uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                    int32_t* __restrict__ n_active, float* __restrict__ part) {
  extern __shared__ uint64_t lds64[];
  const int nw = (F + 63) >> 6;
  const int nblk = D >> 5;
  uint64_t* wl = lds64;                                                  // [nw] mask words
  int* roff = reinterpret_cast<int*>(wl + ((nw + 1) & ~1));              // [NT_F] range offsets
  int* tmp = roff + NT_F;                                                // [NT_F/64 + 1] scan scratch
  constexpr int NS = FW * RPW;                                           // rows (slots) per pass
  float* av = reinterpret_cast<float*>(tmp + NT_F / 64 + 4);             // [NS] activations of the pass
  float* red = av + NS;                                                  // [3 * FW] normalisation / max scratch
  uint2* xt = reinterpret_cast<uint2*>(red + 3 * FW + 4);                // [8][D / 32] x as fp16 pieces (16-B aligned)
  int* bids = reinterpret_cast<int*>(xt + 8 * nblk);                    // [fused_max_rows] the block's row ids
  const uint32_t rstride = (uint32_t)NQ * 1024u;       // 1 kB pieces (64 lanes x 16 bytes) of a nibble row
  uint8_t* sdn = reinterpret_cast<uint8_t*>(lds64) +   // [NS][rstride] the pass's W_downT nibble rows
                 ((reinterpret_cast<uintptr_t>(bids + fused_max_rows(F, gridDim.x, FW * RPW)) -
                   reinterpret_cast<uintptr_t>(lds64) + 15) & ~(uintptr_t)15);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n4 = D >> 2;
  constexpr int XPT = (512 * NQ + NT_F - 1) / NT_F;    // float4 of x per thread: D / 4 <= 512 * NQ

  float4 xv4[XPT];
  stage_load<NT_F, XPT>(x, n4, xv4);
  const float x0 = x[0];
  const int n = mask_prefix<NT_F, WMAX_F>(mask, nw, F, 1, wl, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int G = fused_blocks(n, gridDim.x, FW * RPW);
  if ((int)blockIdx.x >= min(G, n)) return;           // block-uniform: no row here; its partial is never read
  const uint32_t qbytes = (uint32_t)F * (uint32_t)nblk * 16u, sbytes = (uint32_t)F * (uint32_t)nblk * 2u;
  const Buf bqu(qu, qbytes), bsu(su, sbytes), bqd(qd, qbytes), bsd(sd, sbytes);
  const Buf bqg(ACT == 1 ? (const void*)qg : (const void*)qu, ACT == 1 ? qbytes : 0u);
  const Buf bsg(ACT == 1 ? (const void*)sg : (const void*)su, ACT == 1 ? sbytes : 0u);
  const float* bp = ACT == 1 ? bg : bu;
  const Buf bbias(bp ? (const void*)bp : (const void*)qu, bp ? (uint32_t)F * 4u : 0u);   // no bias: 0
  // this thread's half-block of W_downT rows
  const int hb = threadIdx.x;                          // half-block index: Q4 block hb / 2, half hb % 2
  const bool hok = hb < 2 * nblk;
  const uint32_t hoff = (uint32_t)(hb >> 1) * 16u + (uint32_t)(hb & 1) * 8u;

  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  float sas = 0.f;

  // x: normalised, scaled by a power of two and staged in LDS as fp16 while the first pass's rows are in flight.
  // The block's largest |x| sets the power 2^(15 - e) (2^e above it), so every value lies inside fp16's range with
  // its full precision; the dot products are scaled back by 2^(e - 15).
  // piece j of Q4 block c (x[32 c + 4 j .. + 3], four fp16) sits at xt[j * nblk + c]: the lane that owns block c
  // reads its 8 pieces as words c, c + nblk, ..., so a wave reads 64 consecutive 8-byte words per step (no LDS
  // bank conflicts)
  float xinv = 1.f;
  auto stage_x = [&]() {
    if (x_norm) block_norm_regs<NT_F, XPT>(xv4, n4, x0, red);
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < XPT; ++k)
      if (k * NT_F + (int)threadIdx.x < n4)
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv4[k].x), fabsf(xv4[k].y)), fmaxf(fabsf(xv4[k].z), fabsf(xv4[k].w))));
    mx = wave_max(mx);
    if (lane == 0) red[2 * FW + w] = mx;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < FW; ++i) mx = fmaxf(mx, red[2 * FW + i]);
    int ex = 0;
    if (mx > 0.f) (void)frexpf(mx, &ex);
    const int pw = min(15 - ex, 126);
    const float xsc = ldexpf(1.f, pw);
    xinv = ldexpf(1.f, -pw);
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int i = k * NT_F + (int)threadIdx.x;       // float4 i: piece i % 8 of block i / 8
      if (i < n4) {
        const half4 hv = {(_Float16)(xv4[k].x * xsc), (_Float16)(xv4[k].y * xsc), (_Float16)(xv4[k].z * xsc),
                          (_Float16)(xv4[k].w * xsc)};
        xt[(i & 7) * nblk + (i >> 3)] = __builtin_bit_cast(uint2, hv);
      }
    }
    lds_barrier();
  };
  // A pass takes NS = 8 * RPW rows: slot s (dense index k0 + G * s) runs on wave s % 8 as its row s / 8, so a
  // block with up to NS rows reads them all in one round trip. The wave of a slot also issues the loads of the
  // slot's W_downT nibble row straight into LDS (no registers), in the same round trip as its gate/up rows.
  const int wv = __builtin_amdgcn_readfirstlane(w);   // wave index, in a scalar register (LDS load bases)
  // the block's rows: dense indices blk + G * k, k < nrow, their ids in LDS (one rank select per mask word)
  const int blk = blockIdx.x;
  const int nrow = (n - blk + G - 1) / G;
  block_row_ids(wl, roff, nw, blk, G, bids);
  lds_barrier();
  struct Pass {
    int idr[RPW];
    uint4 nu[RPW][NQ], ng[RPW][NQ];
    uint32_t fu[RPW][NQ], fg[RPW][NQ];                 // block scales' fp16 bits (32-bit: kept in registers)
    float bias[RPW];
    uint32_t ds[NS];                                   // this thread's block scale of every W_downT row (fp16 bits)
  };
  auto issue = [&](int k0, Pass& P) {                  // rows past nrow read nothing (out-of-range offsets)
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int kr = k0 + w + FW * r;
      const bool have = kr < nrow;                     // wave-uniform
      P.idr[r] = have ? bids[kr] : -1;
      const uint32_t row = (uint32_t)(have ? P.idr[r] : 0);
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
        const int c = lane + 64 * m;
        const bool ok = have && c < nblk;
        const uint32_t o = row * nblk + c;
        P.nu[r][m] = bqu.ld16(boff(ok, o * 16u));
        P.fu[r][m] = bsu.ldu16(boff(ok, o * 2u));
        if (ACT == 1) {
          P.ng[r][m] = bqg.ld16(boff(ok, o * 16u));
          P.fg[r][m] = bsg.ldu16(boff(ok, o * 2u));
        }
      }
      P.bias[r] = bbias.ldf(boff(have, row * 4u));
      uint8_t* dst = sdn + (uint32_t)(wv + FW * r) * rstride;
#pragma unroll
      for (int c = 0; c < NQ; ++c) {                   // the slot's nibble row, 1 kB per load
        const uint32_t o = (uint32_t)c * 1024u + (uint32_t)lane * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            bqd.r, (__attribute__((address_space(3))) void*)(dst + c * 1024), 16,
            boff(have && o < (uint32_t)nblk * 16u, row * (uint32_t)nblk * 16u + o), 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int idj = k0 + j < nrow ? bids[k0 + j] : -1;
      const bool ok = idj >= 0 && hok;
      const uint32_t row = (uint32_t)(idj >= 0 ? idj : 0);
      P.ds[j] = bsd.ldu16(boff(ok, (row * nblk + (hb >> 1)) * 2u));
    }
  };
  auto compute = [&](int k0, const Pass& P) {
    // dot products of the wave's rows: Q4 block m of the lane outer (its 8 pieces of x read once from LDS for
    // all of the wave's rows), rows inner. A word of nibbles holds elements 4 k .. 4 k + 3 (low nibbles) and
    // 16 + 4 k .. (high); each pair becomes exact fp16 (q - 8) (0x64qq is 1024 + q) and meets its pair of x in
    // a packed dot product with fp32 accumulation.
    float au[RPW], ag[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) au[r] = ag[r] = 0.f;
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int c = lane + 64 * m;
      if (c < nblk) {
        half2v xp[8][2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint2 v = xt[j * nblk + c];
          xp[j][0] = __builtin_bit_cast(half2v, v.x);
          xp[j][1] = __builtin_bit_cast(half2v, v.y);
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          if (P.idr[r] >= 0) {                         // wave-uniform
            au[r] = fmaf(h16f(P.fu[r][m]), q4_dot_x16(P.nu[r][m], xp), au[r]);
            if (ACT == 1) ag[r] = fmaf(h16f(P.fg[r][m]), q4_dot_x16(P.ng[r][m], xp), ag[r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (P.idr[r] >= 0) {                             // wave-uniform
        const float u = wave_sum(au[r]) * xinv;
        float a;
        if (ACT == 1) {
          const float g = wave_sum(ag[r]) * xinv + P.bias[r];
          a = fmaxf(g, 0.f) * u;
        } else {
          a = fmaxf(u + P.bias[r], 0.f);
          if (ACT == 2) a *= a;
        }
        if (lane == 0) { av[w + FW * r] = a; active[blk + G * (k0 + w + FW * r)] = P.idr[r]; }
      } else if (lane == 0) {
        av[w + FW * r] = 0.f;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);                     // this wave's nibble rows have landed in LDS
    lds_barrier();
    // column gather of the pass, rows in slot order: element e < 8 is low nibble e of the half (block element
    // 8 * half + e), e >= 8 the high nibble (block element 16 + 8 * half + e - 8)
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float as_ = av[j] * h16f(P.ds[j]);
      sas += as_;
      const uint2 dj = hok ? *reinterpret_cast<const uint2*>(sdn + (uint32_t)j * rstride + hoff) : make_uint2(0u, 0u);
      const uint32_t wds[2] = {dj.x, dj.y};
#pragma unroll
      for (int k = 0; k < 2; ++k) {                    // nibbles as exact fp16 1024 + q (0x64qq), fp32 FMA with
        const uint32_t lo = wds[k] & 0x0F0F0F0Fu, hi = (wds[k] >> 4) & 0x0F0F0F0Fu;   // fp16 operands
        const half2v l0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(lo, 0x64646464u, 0x00050004u));
        const half2v l1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(lo, 0x64646464u, 0x00070006u));
        const half2v h0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hi, 0x64646464u, 0x00050004u));
        const half2v h1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(hi, 0x64646464u, 0x00070006u));
        acc[4 * k + 0] = fmaf(as_, (float)l0[0], acc[4 * k + 0]);
        acc[4 * k + 1] = fmaf(as_, (float)l0[1], acc[4 * k + 1]);
        acc[4 * k + 2] = fmaf(as_, (float)l1[0], acc[4 * k + 2]);
        acc[4 * k + 3] = fmaf(as_, (float)l1[1], acc[4 * k + 3]);
        acc[8 + 4 * k + 0] = fmaf(as_, (float)h0[0], acc[8 + 4 * k + 0]);
        acc[8 + 4 * k + 1] = fmaf(as_, (float)h0[1], acc[8 + 4 * k + 1]);
        acc[8 + 4 * k + 2] = fmaf(as_, (float)h1[0], acc[8 + 4 * k + 2]);
        acc[8 + 4 * k + 3] = fmaf(as_, (float)h1[1], acc[8 + 4 * k + 3]);
      }
    }
    lds_barrier();                                     // av is rewritten by the next pass
  };
  for (int k0 = 0; k0 < nrow; k0 += NS) {              // passes (block-uniform); row k0 + s in slot s
    Pass P;
    issue(k0, P);
    if (k0 == 0) stage_x();                            // while the first pass's rows are in flight
    compute(k0, P);
  }
  if (hok) {
    float* pb = part + (size_t)blockIdx.x * D + 32 * (hb >> 1) + 8 * (hb & 1);
    float4* lo = reinterpret_cast<float4*>(pb);
    float4* hi = reinterpret_cast<float4*>(pb + 16);
    const float c8 = -1032.f * sas;                    // the nibbles entered as 1024 + q
    lo[0] = make_float4(acc[0] + c8, acc[1] + c8, acc[2] + c8, acc[3] + c8);
    lo[1] = make_float4(acc[4] + c8, acc[5] + c8, acc[6] + c8, acc[7] + c8);
    hi[0] = make_float4(acc[8] + c8, acc[9] + c8, acc[10] + c8, acc[11] + c8);
    hi[1] = make_float4(acc[12] + c8, acc[13] + c8, acc[14] + c8, acc[15] + c8);
  }
}

constexpr int NT_S = 512;            // 32 columns x 16 groups of blocks
constexpr int SC = 32;
constexpr int SG = NT_S / SC;
constexpr int SPG = 16;              // partials per group: G <= SG * SPG = 256

__global__ __launch_bounds__(NT_S) void k_sum_rows(const float* __restrict__ part, const int32_t* __restrict__ n_active,
                                                   int G, int pass, int D, float* __restrict__ y) {
  __shared__ float red[SG][SC];
  const int c = threadIdx.x % SC, g = threadIdx.x / SC;
  const int col = blockIdx.x * SC + c;
  const Buf bp(part, (uint32_t)G * (uint32_t)D * 4u);
  // every load of the thread, n_active included, is issued before the first use (group g takes blocks g,
  // g + SG, ...); partials of blocks that wrote none are loaded too and dropped by a select afterwards, so the
  // partial loads need not wait for n_active
  float v[SPG];
#pragma unroll
  for (int k = 0; k < SPG; ++k) {
    const int b = g + SG * k;
    v[k] = bp.ldf(boff(b < G && col < D, ((uint32_t)b * D + col) * 4u));
  }
  const int na = max(*n_active, 0);
  const int nb = min(fused_blocks(na, G, pass), na);   // blocks that wrote a partial
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < SPG; ++k) s += (g + SG * k < nb) ? v[k] : 0.f;
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && col < D) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < SG; ++k) t += red[k][c];
    y[col] = t;
  }
}

template <int ACT, int NCH, int DCH>
hipError_t launch_fused(const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                        const float* x, int x_norm, int D, int F, const uint64_t* mask, int32_t* active,
                        int32_t* n_active, float* part, int G, float* y, hipStream_t st) {
  const int nw = (F + 63) / 64;
  if (G < 64) return hipErrorInvalidValue;            // one owned row per mask word at most
  const size_t lds = (size_t)((nw + 1) & ~1) * 8 + (NT_F + NT_F / 64 + 4) * sizeof(int) +
                     (FW + 2 * FW + 4 + (size_t)D) * sizeof(float) + (size_t)fused_max_rows(F, G, FW) * sizeof(int) +
                     16;
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_fused1<ACT, NCH, DCH>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail) return hipErrorInvalidValue;
  SFFN_LAUNCH(2, (k_fused1<ACT, NCH, DCH>), dim3(G), dim3(NT_F), lds, st, (const uint4*)Wg, bg, (const uint4*)Wu, bu,
              (const uint4*)WdT, x, x_norm, D, F, mask, active, n_active, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (G > SG * SPG) return hipErrorInvalidValue;
  SFFN_LAUNCH(3, k_sum_rows, dim3((D + SC - 1) / SC), dim3(NT_S), 0, st, part, n_active, G, FW, D, y);
  return hipGetLastError();
}

template <int ACT>
hipError_t dispatch_fused(const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                          const float* x, int x_norm, int D, int F, const uint64_t* mask, int32_t* active,
                          int32_t* n_active, float* part, int G, float* y, hipStream_t st) {
  const int nch = (D / 8 + 63) / 64;
#define FU(N, Q) return launch_fused<ACT, N, Q>(Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, part, G, y, st)
  if (nch <= 2) FU(2, 1);          // D <= 1024
  if (nch <= 4) FU(4, 1);          // D <= 2048
  if (nch <= 8) FU(8, 1);          // D <= 4096
  if (nch <= 10) FU(10, 2);        // D <= 5120
  if constexpr (ACT != 1) FU(16, 2);  // D <= 8192 (ReLU, squared ReLU: one matrix; ReGLU rows this wide keep two kernels)
  return hipErrorInvalidValue;
#undef FU
}

template <int ACT, int NQ, int RPW>
hipError_t launch_fused_q4(const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu, const void* su,
                           const float* bu, const uint8_t* qd, const void* sd, const float* x, int x_norm, int D, int F,
                           const uint64_t* mask, int32_t* active, int32_t* n_active, float* part, int G, float* y,
                           hipStream_t st) {
  const int nw = (F + 63) / 64;
  constexpr int NS = FW * RPW;
  if (G < 64) return hipErrorInvalidValue;            // one owned row per mask word at most
  const size_t lds = (size_t)((nw + 1) & ~1) * 8 + (NT_F + NT_F / 64 + 4) * sizeof(int) +
                     (NS + 3 * FW + 4 + (size_t)D / 2) * sizeof(float) +
                     (size_t)fused_max_rows(F, G, NS) * sizeof(int) +
                     16 + (size_t)NS * NQ * 1024;   // + the pass's nibble rows (16-byte aligned)
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_fused1_q4<ACT, NQ, RPW>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail || G > SG * SPG) return hipErrorInvalidValue;
  SFFN_LAUNCH(2, (k_fused1_q4<ACT, NQ, RPW>), dim3(G), dim3(NT_F), lds, st, (const uint4*)qg, (const _Float16*)sg, bg,
              (const uint4*)qu, (const _Float16*)su, bu, qd, (const _Float16*)sd, x, x_norm, D, F, mask, active,
              n_active, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SFFN_LAUNCH(3, k_sum_rows, dim3((D + SC - 1) / SC), dim3(NT_S), 0, st, part, n_active, G, NS, D, y);
  return hipGetLastError();
}

}  // namespace

hipError_t sffn_launch_fused_q4(int act, const uint8_t* qg, const void* sg, const float* bg, const uint8_t* qu,
                                const void* su, const float* bu, const uint8_t* qd, const void* sd, const float* x,
                                int x_norm, int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active,
                                float* part, int G, float* y, hipStream_t st) {
  const int nq = (D / 32 + 63) / 64;   // Q4 blocks per lane of a row
#define FQ(A, N) return launch_fused_q4<A, N, SFFN_Q4_FUSED_RPW>(qg, sg, bg, qu, su, bu, qd, sd, x, x_norm, D, F, mask, active, n_active, part, G, y, st)
  if (act == 1) {
    if (nq <= 1) FQ(1, 1);
    if (nq <= 2) FQ(1, 2);
    FQ(1, 4);
  }
  if (act == 2) {
    if (nq <= 1) FQ(2, 1);
    if (nq <= 2) FQ(2, 2);
    FQ(2, 4);
  }
  if (nq <= 1) FQ(0, 1);
  if (nq <= 2) FQ(0, 2);
  FQ(0, 4);
#undef FQ
}

// Fused single-token forward: F <= 32768 (mask words fit one per thread); fp16: D <= 5120 (ReGLU: gate, up and
// down chunks in registers) or D <= 8192 (ReLU); Q4_0: D <= 8192 (one half-block of every W_downT row per thread).
bool sffn_fused_ok(int B, int D, int F, int act, bool q4) {
  if (B != 1 || F > 32768) return false;
  if (q4) return D <= 8192;
  return D <= 5120 || (act != 1 && D <= 8192);
}

hipError_t sffn_launch_fused(int act, const void* Wg, const float* bg, const void* Wu, const float* bu,
                             const void* WdT, const float* x, int x_norm, int D, int F, const uint64_t* mask,
                             int32_t* active, int32_t* n_active, float* part, int G, float* y, hipStream_t st) {
  switch (act) {
    case 1: return dispatch_fused<1>(Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, part, G, y, st);
    case 2: return dispatch_fused<2>(Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, part, G, y, st);
    default: return dispatch_fused<0>(Wg, bg, Wu, bu, WdT, x, x_norm, D, F, mask, active, n_active, part, G, y, st);
  }
}
