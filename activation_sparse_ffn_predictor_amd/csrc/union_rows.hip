// Multi-token row gather on the matrix cores, tiled so that the token operand is read once per 64 union rows.
//
// PowerInfer pages, Turkish article, "Neuron-aware operator": only the rows of W_gate / W_up of predicted-active
// neurons are read; with several tokens the masks are merged and each union row is read once for all of them.
// Per layer this is a GEMM of the union rows [n x D] with the tokens [D x B] (n up to F, B <= 64), on
// v_mfma_f32_16x16x32_f16 (A: 16 rows x 32 k, lane l: row l % 16, 8 k values of lane group j = l / 16; B: 32 k x 16
// tokens, lane l: token l % 16, the same 8 k values; D: lane l holds rows 4 (l / 16) + i of token l % 16).
//
// k order. A dot product may take its k terms in any order, so the MFMA k slots are assigned to suit the loads:
// k blocks of 32 go in quads. Q4_0: in MFMA q (0..3) of quad g, lane group j takes elements 8 q .. 8 q + 7 of k
// block 4 g + j, so a lane holds one whole block of its row per quad (one 16-byte load of nibbles) and the four
// lanes of a row read 64 contiguous bytes. fp16 ("block-major"): in MFMA q of quad g, lane group j takes elements
// 8 j .. 8 j + 7 of k block 4 g + q, so each of the quad's four 16-byte loads reads one block, 64 contiguous bytes
// per row. The token fragments are written in the matching order.
//
// k_split_x (one workgroup per token slot): normalises the token (optional, as every entry point's x_norm),
// scales it by a power of two 2^-e with 2^e the smallest power above max |x| (exact, and it keeps every value
// inside fp16's range), and writes the B-operand fragments, fragment f = (quad, q, token tile) as 64 lanes x 16
// bytes, so a wave reads one as a contiguous kilobyte. EXACT adds a plane of fp16 residuals (x = hi + lo, the
// single-token kernels' fp32 to within 2^-22); without it the operand is fp16(x). PACK (EXACT, up to 8 tokens)
// puts both halves in one plane: lane columns 0..7 the tokens' hi halves, 8..15 their lo halves.
//
// k_ur (workgroups of 4 or 8 waves, 64 dense indices each, one 16-row tile per wave and, with 8 waves, one k half
// of every chunk per wave; every token tile; KS workgroups per 64 rows split the quads): the workgroup's union rows
// come from the mask (block scan of the words' popcounts, then a search per row). Quads are walked in chunks; per
// chunk each thread loads a share of the next chunk's token fragments (into registers, then LDS, double-buffered:
// all waves read them) and its row's k blocks of weights two chunks ahead (Q4_0 nibbles and block scales, or fp16)
// in a ring of three register sets. The chunk count is padded to a multiple of three (the padding reads nothing:
// out-of-range buffer loads return 0). Q4_0 weights become exact fp16 (q - 8) through the exponent trick (0x64qq
// is 1024 + q in fp16), times the block scale in fp16 (one rounding per weight; the whole block's scale is one
// lane's, so no per-block fp32 step is needed). fp16 weights enter as they are; with EXACT each token operand is
// two fp16 halves and every product is exact (PACK: both halves in one operand, one product per k block, the
// lo columns added to the hi ones in the epilogue). With two k halves the second half's sums meet the first's in LDS,
// always added in that order. The epilogue undoes the token's power of two and, with one share, adds the bias and
// applies the activation; with KS shares each writes its partial pre-activations and k_act_combine (union.hip)
// adds them in share order.
#include "common.h"

using namespace sffn;

#define GT_BIAS(A, bg, bu) ((A) == 1 ? (bg) : (bu))

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const half8& a, const half8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Q4_0: elements 8 q .. 8 q + 7 of a 32-element block as exact fp16 (q - 8). w = the block's 16 nibble bytes (byte
// i: element i low, element 16 + i high): q = 0, 1 take the low nibbles of bytes 8 q .., q = 2, 3 the high nibbles
// of bytes 8 (q - 2) ... Each byte goes under the fp16 exponent pattern 0x64 (0x64nn = 1024 + n exactly), then
// 1032 is subtracted.
__device__ __forceinline__ half8 q4_half8(const uint4& w, int q) {
  const uint32_t px = (q & 1) ? w.z : w.x, py = (q & 1) ? w.w : w.y;
  const uint32_t sh = (uint32_t)(q >> 1) * 4u;
  const uint32_t w0 = (px >> sh) & 0x0F0F0F0Fu, w1 = (py >> sh) & 0x0F0F0F0Fu;
  const uint32_t e = 0x64646464u;
  // v_perm_b32 byte pool: selector 0..3 = second source's bytes, 4..7 = first source's bytes
  const uint32_t h0 = __builtin_amdgcn_perm(w0, e, 0x00050004u), h1 = __builtin_amdgcn_perm(w0, e, 0x00070006u);
  const uint32_t h2 = __builtin_amdgcn_perm(w1, e, 0x00050004u), h3 = __builtin_amdgcn_perm(w1, e, 0x00070006u);
  const half2v off = {(_Float16)1032.f, (_Float16)1032.f};
  const half2v a0 = __builtin_bit_cast(half2v, h0) - off, a1 = __builtin_bit_cast(half2v, h1) - off;
  const half2v a2 = __builtin_bit_cast(half2v, h2) - off, a3 = __builtin_bit_cast(half2v, h3) - off;
  half8 r;
  r[0] = a0[0]; r[1] = a0[1]; r[2] = a1[0]; r[3] = a1[1];
  r[4] = a2[0]; r[5] = a2[1]; r[6] = a3[0]; r[7] = a3[1];
  return r;
}

// eight copies of the fp16 value whose bits are the low half of s
__device__ __forceinline__ half8 splat8(uint32_t s) {
  const uint32_t d = s * 0x10001u;
  return __builtin_bit_cast(half8, make_uint4(d, d, d, d));
}

constexpr int NTX = 256;

// One workgroup per token slot tok < NTT * 16 (slots >= B are zero). xf: [KB][NTT][NH][64] uint4, NH = 2 with EXACT
// (hi, lo). xs[tok] = 2^e, the power of two the fragments are divided by. With nparts > 0 (XPT = 1) the values are
// the sum of nparts partials x[p][B][D], added in share order (as k_sum_parts adds them).
// PACK (EXACT, NTT = 1, B <= 8): one plane whose lane columns 0..7 hold the tokens' hi halves and 8..15 their lo
// halves, so that one matrix-core product takes both (slots 8..15 write nothing).
constexpr int SPLIT_PARTS_MAX = 16;
template <int XPT, bool EXACT, bool PERM, bool PACK = false>
__global__ __launch_bounds__(NTX) void k_split_x(const float* __restrict__ x, int x_norm, int B, int D, int NTT,
                                                 uint4* __restrict__ xf, float* __restrict__ xs, int nparts) {
  static_assert(!PACK || EXACT, "packed planes are the hi and lo halves");
  constexpr int NH = EXACT && !PACK ? 2 : 1;
  __shared__ float red[2 * (NTX / 64) + 4];
  const int tok = blockIdx.x;
  if (PACK && tok >= 8) return;                        // block-uniform
  const bool real = tok < B;
  const int n4 = real ? D >> 2 : 0;                    // padding slots load nothing (all zero)
  const float* xb = x + (size_t)(real ? tok : 0) * D;
  float4 v[XPT];
  if constexpr (XPT == 1) {
    if (nparts > 0) {                                  // every share's load issued before the first add
      const Buf bp(x, (uint32_t)nparts * (uint32_t)B * (uint32_t)D * 4u);
      const bool ok = (int)threadIdx.x < n4;
      float4 u[SPLIT_PARTS_MAX];
#pragma unroll
      for (int k = 0; k < SPLIT_PARTS_MAX; ++k)
        u[k] = bp.ldf4(boff(ok && k < nparts, ((uint32_t)(k * B + tok) * (uint32_t)D + 4u * threadIdx.x) * 4u));
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < SPLIT_PARTS_MAX; ++k)
        if (k < nparts) { acc.x += u[k].x; acc.y += u[k].y; acc.z += u[k].z; acc.w += u[k].w; }
      v[0] = acc;
    } else {
      stage_load<NTX, XPT>(xb, n4, v);
    }
  } else {
    stage_load<NTX, XPT>(xb, n4, v);
  }
  if (real && x_norm) block_norm_regs<NTX, XPT>(v, n4, xb[0], red);
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < XPT; ++k)
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v[k].x), fabsf(v[k].y)), fmaxf(fabsf(v[k].z), fabsf(v[k].w))));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, WAVE));
  __syncthreads();                                     // red may still be read by block_norm_regs' last step
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < NTX / 64; ++i) mx = fmaxf(mx, red[i]);
  int ex = 0;
  if (mx > 0.f) (void)frexpf(mx, &ex);                 // mx = f 2^ex, f in [0.5, 1): |x| 2^-ex < 1
  const float inv = ldexpf(1.f, -ex);
  if (threadIdx.x == 0) xs[tok] = ldexpf(1.f, ex);
  const int t = tok >> 4, tl = tok & 15;
  // element e: k block kb = e / 32, 8-element group q = (e % 32) / 8. Q4_0 order: fragment 4 (kb / 4) + q (quad
  // kb / 4, MFMA q), lane group kb % 4; block-major (PERM): fragment kb (quad kb / 4, MFMA kb % 4), lane group q.
  // float4 i holds elements 4 i .. 4 i + 3, half i % 2 of an 8-element group
  auto slot = [&](int kb, int q, int h) {
    const int f = PERM ? kb : (kb >> 2) * 4 + q, lg = PERM ? q : kb & 3;
    if constexpr (PACK) return ((size_t)f * NTT + t) * 64 + (size_t)(lg * 16 + tl + 8 * h);
    return (((size_t)f * NTT + t) * NH + h) * 64 + (size_t)(lg * 16 + tl);
  };
#pragma unroll
  for (int k = 0; k < XPT; ++k) {
    const int i = k * NTX + (int)threadIdx.x;
    if (i < (D >> 2)) {
      const int kb = i >> 3, q = (i >> 1) & 3, hf = i & 1;
      const float a[4] = {v[k].x * inv, v[k].y * inv, v[k].z * inv, v[k].w * inv};
      _Float16 hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (_Float16)a[e];
        lo[e] = (_Float16)(a[e] - (float)hi[e]);
      }
      uint2* dh = reinterpret_cast<uint2*>(xf + slot(kb, q, 0)) + hf;
      *dh = make_uint2(__builtin_bit_cast(uint32_t, half2v{hi[0], hi[1]}),
                       __builtin_bit_cast(uint32_t, half2v{hi[2], hi[3]}));
      if (EXACT) {
        uint2* dl = reinterpret_cast<uint2*>(xf + slot(kb, q, 1)) + hf;
        *dl = make_uint2(__builtin_bit_cast(uint32_t, half2v{lo[0], lo[1]}),
                         __builtin_bit_cast(uint32_t, half2v{lo[2], lo[3]}));
      }
    }
  }
  // 8-element groups at or past D, up to the end of the last quad, are zero
  const int KQ = (D + 127) >> 7;                       // quads
  for (int gi = (D >> 3) + (int)threadIdx.x; gi < KQ * 16; gi += NTX) {
    xf[slot(gi >> 2, gi & 3, 0)] = make_uint4(0u, 0u, 0u, 0u);
    if (EXACT) xf[slot(gi >> 2, gi & 3, 1)] = make_uint4(0u, 0u, 0u, 0u);
  }
}

constexpr int NTR = 256;             // 4 waves
constexpr int WMAXR = 2;             // mask words per thread kept in LDS (F <= 32768)

// k blocks per chunk: 8 for Q4_0 (two quads: 32 bytes of a row per lane and matrix), 4 for fp16 (a quad: 64 bytes)
template <bool Q4> struct URChunk { static constexpr int KC = Q4 ? 8 : 4; };

// fp16 token fragments and weight loads of k_ur with KH k halves in block-major k order (see the k order note
// above). Measured at the 13B shape: with one k half 8 tokens 33.9 -> 30.6 us, 32 tokens 79.2 -> 69.3 us per
// layer; with two (64 tokens) 85.3 -> 90.7 us, so those keep the Q4_0 order.
constexpr bool ur_block_major(bool q4, int kh) { return !q4 && kh == 1; }

// k_ur: RT row tiles of 16 rows (4 or 8) and KH k halves (1 or 2); NW = RT KH waves, wave w takes row tile w % RT
// and k half w / RT of every chunk
template <int RT, int KH, int NTT, int ACT, bool Q4, bool EXACT, bool PACK>
__global__ __launch_bounds__(64 * RT * KH) __attribute__((amdgpu_waves_per_eu(RT * KH >= 8 ? 4 : 2)))
void k_ur(const void* __restrict__ Wg, const void* __restrict__ Sg,
          const float* __restrict__ bg, const void* __restrict__ Wu,
          const void* __restrict__ Su, const float* __restrict__ bu,
          const uint4* __restrict__ xf, const float* __restrict__ xsc, int B,
          int D, int F, const uint64_t* __restrict__ mask,
          int32_t* __restrict__ active, int32_t* __restrict__ n_active,
          float* __restrict__ abuf, float* __restrict__ bmax,
          float* __restrict__ pre, int KS) {
  static_assert(!(Q4 && EXACT), "Q4_0 rows take fp16 tokens");
  static_assert((RT == 4 || RT == 8) && (KH == 1 || KH == 2), "4 or 8 row tiles, 1 or 2 k halves");
  static_assert(!PACK || (EXACT && NTT == 1), "packed planes: exact tokens of one tile");
  constexpr int NW = RT * KH;
  constexpr int NTU = 64 * NW;
  constexpr int RB = 16 * RT;                          // union rows per workgroup
  constexpr bool GT = ACT == 1;                        // ReGLU: a gate row per neuron
  constexpr int NH = EXACT && !PACK ? 2 : 1;           // token fragment planes (hi, lo; PACK: both in one)
  constexpr int KC = URChunk<Q4>::KC;
  constexpr int QC = KC / 4;                           // quads per chunk
  constexpr int XT = KC * NTT * NH * 64;               // uint4 of token fragments per chunk
  constexpr int XV = (XT + NTU - 1) / NTU;             // per thread
  // a wave's part of a chunk: Q4_0 GQW of the chunk's two quads (per quad a lane's whole k block, one 16-byte
  // load), fp16 QW of the quad's four 8-element groups
  constexpr int GQW = Q4 ? QC / KH : 1;
  constexpr int QW = Q4 ? 4 : 4 / KH;
  constexpr int WV = Q4 ? GQW : QW;                    // uint4 of weights per lane and matrix per chunk
  constexpr int NM = GT ? 2 : 1;                       // weight matrices (up, gate)
  __shared__ int roff[NTU];
  __shared__ int tmp[NTU / 64 + 4];
  __shared__ int ids[RB];
  // token fragments of two chunks; after the last chunk the k halves' sums [row tile][token tile][up, gate][lane]
  constexpr int XLN = 2 * XT > RT * NTT * 2 * 64 ? 2 * XT : RT * NTT * 2 * 64;
  __shared__ uint4 xlraw[XLN];
  uint4 (*xl)[XT] = reinterpret_cast<uint4 (*)[XT]>(xlraw);
  __shared__ uint4 xjunk[XT % NTU ? NTU : 1];          // landing slots of the fragment pieces a thread lacks
  // Q4_0 block scales of two chunks: [buffer][matrix][row][the chunk's 8 blocks], loaded 16 bytes per row by the
  // first NM RB / 64 waves with the token fragments (per lane and quad they would be 2-byte loads from 16 rows)
  __shared__ uint4 sl[Q4 ? 2 : 1][NM][Q4 ? RB : 1];
  // the mask words are needed only before the first chunk: they share the token fragments' space
  static_assert(sizeof(xlraw) >= WMAXR * NTU * sizeof(uint64_t), "mask words fit in the fragment buffers");
  uint64_t* wl = reinterpret_cast<uint64_t*>(&xl[0][0]);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rt = w % RT, kh = w / RT;                  // row tile, k half
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NTU - 1) / NTU;
  const int n = mask_prefix<NTU, WMAXR>(mask, nw, F, wpt, wl, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int ks = blockIdx.x % KS;                      // the shares of 64 rows are neighbours in dispatch order
  const int i0 = (blockIdx.x / KS) * RB;
  if (i0 >= n) return;                                 // block-uniform
  if (threadIdx.x < RB) {
    const int i = i0 + threadIdx.x;
    int id = -1;
    if (i < n) {                                       // the (i - roff)-th set bit after word range T * wpt
      int lo = 0, hi = NTU - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (roff[mid] <= i) lo = mid; else hi = mid - 1;
      }
      int rem = i - roff[lo];
      for (int tw = lo * wpt; tw < nw; ++tw) {
        const int cnt = __popcll(wl[tw]);
        if (rem < cnt) { id = tw * 64 + select_bit(wl[tw], rem); break; }
        rem -= cnt;
      }
      if (ks == 0) active[i] = id;
    }
    ids[threadIdx.x] = id;
  }
  __syncthreads();
  const int idl = ids[rt * 16 + (lane & 15)];          // this lane's A-operand row (-1: none)
  // the epilogue's biases and token powers of two: with one k half loaded now, so that they arrive with the first
  // chunks instead of costing a round trip after the last one (with two k halves the registers are short: in the
  // epilogue)
  float ebias[4], esx[NTT];
  auto load_epi = [&]() {
    const float* bp = GT ? bg : bu;
    const Buf bb(bp ? (const void*)bp : (const void*)xsc, bp ? (uint32_t)F * 4u : 0u);   // no bias: 0
    const Buf bs(xsc, (uint32_t)NTT * 64u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = ids[rt * 16 + (lane >> 4) * 4 + i];
      ebias[i] = bb.ldf(boff(KS == 1 && id >= 0, (uint32_t)(id >= 0 ? id : 0) * 4u));
    }
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int tok = t * 16 + (lane & 15);
      esx[t] = bs.ldf(boff(tok < B, (uint32_t)tok * 4u));
    }
  };
  if constexpr (KH == 1) load_epi();
  const int jq = lane >> 4;                            // lane group: the k block of a quad this lane holds
  const int KB = (D + 31) >> 5, nblk = D >> 5;
  const int KQ = (KB + 3) >> 2;                        // quads
  const int KQS = (KQ + KS - 1) / KS;                  // quads of one share
  const int q0 = ks * KQS, q1 = min(KQ, q0 + KQS);     // this share's quads
  const int nch = ((max(q1 - q0, 0) + QC - 1) / QC + 2) / 3 * 3;   // chunks, padded to rounds of three
  const Buf bx(xf, (uint32_t)q1 * 4u * NTT * NH * 1024u);           // quads past the share read 0
  const uint32_t wbytes = Q4 ? (uint32_t)F * (uint32_t)(D >> 1) : (uint32_t)F * (uint32_t)D * 2u;
  const uint32_t sbytes = Q4 ? (uint32_t)F * (uint32_t)nblk * 2u : 0u;
  const Buf bwu(Wu, wbytes), bwg(GT ? Wg : Wu, GT ? wbytes : 0u);
  const Buf bsu(Q4 ? Su : Wu, sbytes), bsg(Q4 && GT ? Sg : Wu, GT ? sbytes : 0u);
  const uint32_t row = (uint32_t)(idl >= 0 ? idl : 0);
  const int gqh = Q4 ? kh * GQW : 0;                   // the wave's first quad within the chunk
  const int qh = Q4 ? 0 : kh * QW;                     // fp16: the wave's first 8-element group

  struct Set {
    uint4 wu[WV], wg[WV];
  };
  uint4 xv[XV];                                        // this thread's share of the next chunk's token fragments
  uint4 sv;                                            // Q4_0, first NM waves: the next chunk's scales of one row
  const int wu0 = __builtin_amdgcn_readfirstlane(w);   // wave index in a scalar register (selects the matrix)
  const int smat = wu0 % NM, sblk = wu0 / NM;          // staging waves: matrix, 64-row block
  const int srow = ids[(sblk < RB / 64 ? sblk : 0) * 64 + lane];   // the row whose scales this lane stages
  auto load_x = [&](int c) {
    const int g0 = q0 + c * QC;                        // first quad of the chunk
#pragma unroll
    for (int m = 0; m < XV; ++m) {
      const int p = m * NTU + (int)threadIdx.x;
      xv[m] = bx.ld16(boff(XT % NTU == 0 || p < XT, ((uint32_t)g0 * 4u * NTT * NH * 64 + (uint32_t)p) * 16u));
    }
    if constexpr (Q4) {
      // the chunk's 8 blocks: 16 bytes of the row's scales (past the row's last block they belong to the next
      // row, harmless: there the tokens are zero; past the tensor they read 0)
      const uint32_t so = ((uint32_t)(srow >= 0 ? srow : 0) * nblk + (uint32_t)g0 * 4u) * 2u;
      const bool ok = srow >= 0 && g0 < q1 && sblk < RB / 64;
      sv = (smat == 1 ? bsg : bsu).ld16(boff(ok, so));
    }
  };
  auto load_w = [&](int c, Set& S) {
#pragma unroll
    for (int i = 0; i < GQW; ++i) {
    const int g = q0 + c * QC + gqh + i;
    const int kb = g * 4 + jq;                         // Q4_0: this lane's k block of the quad
    const bool ok = g < q1 && kb < KB && idl >= 0;
    const bool okh = g < q1 && idl >= 0;               // fp16: the element bound is checked per load
    if constexpr (Q4) {
      const uint32_t o = row * (uint32_t)(D >> 1) + (uint32_t)kb * 16u;
      S.wu[i] = bwu.ld16(boff(ok, o));
      if (GT) S.wg[i] = bwg.ld16(boff(ok, o));
    } else {
#pragma unroll
      for (int j = 0; j < WV; ++j) {                   // block-major: elements 8 jq .. 8 jq + 7 of block 4 g + q,
        constexpr bool BM = ur_block_major(Q4, KH);    // else elements 8 q .. 8 q + 7 of block kb
        const int k = BM ? (g * 4 + qh + j) * 32 + jq * 8 : kb * 32 + (qh + j) * 8;
        const bool v = BM ? okh && k < D : ok && k < D;
        const uint32_t o = (row * (uint32_t)D + (uint32_t)k) * 2u;
        S.wu[j] = bwu.ld16(boff(v, o));
        if (GT) S.wg[j] = bwg.ld16(boff(v, o));
      }
    }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int m = 0; m < XV; ++m) {
      const int p = m * NTU + (int)threadIdx.x;
      uint4* d = (XT % NTU == 0 || p < XT) ? &xl[buf][p] : &xjunk[threadIdx.x];
      *d = xv[m];
    }
    if (Q4 && sblk < RB / 64) sl[Q4 ? buf : 0][smat][Q4 ? (sblk < RB / 64 ? sblk : 0) * 64 + lane : 0] = sv;
  };
  f32x4 au[NTT], ag[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) { au[t] = f32x4{0.f, 0.f, 0.f, 0.f}; ag[t] = au[t]; }
  auto compute = [&](const Set& S, int buf) {
#pragma unroll
    for (int i = 0; i < GQW; ++i)
#pragma unroll
    for (int j = 0; j < QW; ++j) {
      const int q = qh + j;
      half8 a_u, a_g;
      if constexpr (Q4) {                              // fp16((q - 8) s): one rounding per weight
        const int blk = 4 * (gqh + i) + jq;            // this lane's block within the chunk
        const int srw = rt * 16 + (lane & 15);
        const uint32_t su = reinterpret_cast<const uint16_t*>(&sl[Q4 ? buf : 0][0][Q4 ? srw : 0])[blk];
        a_u = q4_half8(S.wu[i], q) * splat8(su);
        if (GT) {
          const uint32_t sg = reinterpret_cast<const uint16_t*>(&sl[Q4 ? buf : 0][NM - 1][Q4 ? srw : 0])[blk];
          a_g = q4_half8(S.wg[i], q) * splat8(sg);
        }
      } else {
        a_u = __builtin_bit_cast(half8, S.wu[j]);
        if (GT) a_g = __builtin_bit_cast(half8, S.wg[j]);
      }
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        const int f = (((gqh + i) * 4 + q) * NTT + t) * NH;
        const half8 xh = __builtin_bit_cast(half8, xl[buf][f * 64 + lane]);
        if constexpr (EXACT && !PACK) {
          const half8 xo = __builtin_bit_cast(half8, xl[buf][(f + 1) * 64 + lane]);
          au[t] = mfma16(a_u, xo, mfma16(a_u, xh, au[t]));
          if (GT) ag[t] = mfma16(a_g, xo, mfma16(a_g, xh, ag[t]));
        } else {
          au[t] = mfma16(a_u, xh, au[t]);
          if (GT) ag[t] = mfma16(a_g, xh, ag[t]);
        }
      }
    }
  };
  // weights two chunks ahead in three register sets, tokens one chunk ahead (from L2): step c loads chunk c + 1's
  // tokens and chunk c + 2's weights, computes chunk c (its tokens in LDS buffer c % 2) and stages chunk c + 1's
  // tokens into the other buffer
  Set S0, S1, S2;
  load_x(0);
  load_w(0, S0);
  load_w(1, S1);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 3) {                   // nch is a multiple of 3
    load_x(c + 1);
    load_w(c + 2, S2);
    compute(S0, c & 1);
    store_x((c + 1) & 1);
    __syncthreads();
    load_x(c + 2);
    load_w(c + 3, S0);
    compute(S1, (c + 1) & 1);
    store_x(c & 1);
    __syncthreads();
    load_x(c + 3);
    load_w(c + 4, S1);
    compute(S2, c & 1);
    store_x((c + 1) & 1);
    __syncthreads();
  }
  // the k halves meet: the second half's sums go through LDS (xl is free: every wave is past its last chunk) and
  // the first half adds them, always in this order
  f32x4* red = reinterpret_cast<f32x4*>(&xl[0][0]);   // [row tile][token tile][up, gate][64 lanes]
  if (KH == 2 && kh == 1) {
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      red[((rt * NTT + t) * 2) * 64 + lane] = au[t];
      if (GT) red[((rt * NTT + t) * 2 + 1) * 64 + lane] = ag[t];
    }
  }
  if (KH == 2) __syncthreads();
  if (KH == 2 && kh == 0) {
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      au[t] += red[((rt * NTT + t) * 2) * 64 + lane];
      if (GT) ag[t] += red[((rt * NTT + t) * 2 + 1) * 64 + lane];
    }
  }
  // epilogue (first half): the token's power of two back; one share: bias and activation, else the partial
  // pre-activations
  float amx[NTT];                                      // largest |a| of this lane's rows, per token tile
  if (PACK && kh == 0) {                               // column t + 8 holds the lo half's sums of token t < 8
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      au[0][i] += __shfl_xor(au[0][i], 8, 64);
      if (GT) ag[0][i] += __shfl_xor(ag[0][i], 8, 64);
    }
  }
  if (kh == 0) {
    if constexpr (KH == 2) load_epi();
    const size_t FB = (size_t)F * B;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      amx[t] = 0.f;
      const int tok = t * 16 + (lane & 15);
      const int r0 = i0 + rt * 16 + (lane >> 4) * 4;   // this lane's 4 rows: half an octet
      const float sx = esx[t];
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = r0 + i;
        const float u = au[t][i] * sx, g = ag[t][i] * sx;
        float a = 0.f;
        if (KS > 1) {
          if (tok < B && ii < n) {
            const size_t e = (size_t)ii * B + tok;
            pre[(size_t)(2 * ks) * FB + e] = u;
            if (GT) pre[(size_t)(2 * ks + 1) * FB + e] = g;
          }
          continue;
        }
        if (GT) {
          a = fmaxf(g + ebias[i], 0.f) * u;
        } else {
          a = fmaxf(u + ebias[i], 0.f);
          if (ACT == 2) a *= a;
        }
        a4[i] = (tok < B && ii < n) ? a : 0.f;         // the 64-row tile is written whole: zeros past n and B
        amx[t] = fmaxf(amx[t], fabsf(a4[i]));
      }
      if (KS == 1)   // octet order: ((row / 8) * 16 NTT + token) * 8 + row % 8
        *reinterpret_cast<float4*>(&abuf[((size_t)(r0 >> 3) * (NTT * 16) + tok) * 8 + (r0 & 7)]) =
            make_float4(a4[0], a4[1], a4[2], a4[3]);
    }
  }
  if (KS > 1) return;                                  // k_act_combine writes the maxima
  // the workgroup's largest |a| per token: over the lane groups (rows), then over the row tiles
  __syncthreads();                                     // every read of red is done
  float* smx = reinterpret_cast<float*>(&xl[0][0]);    // [RT row tiles][64 tokens]
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      float m = amx[t];
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (lane < 16) smx[rt * 64 + t * 16 + lane] = m;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < B * (RB / 64)) {             // one entry per 64-row block and token
    const int t = threadIdx.x % B, b = threadIdx.x / B;
    const float* sm = smx + b * 256;
    bmax[(size_t)(i0 / 64 + b) * B + t] = fmaxf(fmaxf(sm[t], sm[64 + t]), fmaxf(sm[128 + t], sm[192 + t]));
  }
}

// A few tokens (B <= UR16_MAX_B): 16 union rows per workgroup and the k range split over its 4 waves, so that a small
// union still spreads over many workgroups without a second kernel to combine k shares. Wave w takes a contiguous
// quarter of the quads; per quad each lane loads its row's k block (as in k_ur) and its own token fragments
// straight from xf (no LDS staging: no two waves share a quad). Loads run two quads ahead in a ring of three
// register sets. The waves' partial sums meet in LDS and wave 0 adds them in wave order, applies bias and
// activation, and writes the tile (octet order, zeros past n and B) and its largest |a| per token
// (bmax[(i0 / 16) * B + token]). Workgroups past the union but inside its last 64-row block write a zero tile.
constexpr int R16 = 16;
// Up to 6 tokens the 16-row kernel (k split over the waves of a workgroup) runs; beyond, its token fragments, read
// again by every 16-row workgroup, cost more than the k-share combine of the 64-row kernel. Measured at the 13B
// shape with the packed fragments (same box): 5 tokens 1967 -> 2114 tokens/s with the 16-row kernel, 6 tokens
// 2252 -> 2321, 8 tokens 2692 -> 2654 (falcon 40B 2078 -> 2067, 7B 3773 -> 3905).
constexpr int UR16_MAX_B = 6;


template <int ACT, bool Q4, bool EXACT, bool PACK>
__global__ __launch_bounds__(NTR) void k_ur16(const void* __restrict__ Wg, const void* __restrict__ Sg,
                                              const float* __restrict__ bg, const void* __restrict__ Wu,
                                              const void* __restrict__ Su, const float* __restrict__ bu,
                                              const uint4* __restrict__ xf, const float* __restrict__ xsc, int B,
                                              int D, int F, const uint64_t* __restrict__ mask,
                                              int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                              float* __restrict__ abuf, float* __restrict__ bmax) {
  static_assert(!(Q4 && EXACT), "Q4_0 rows take fp16 tokens");
  static_assert(!PACK || EXACT, "packed planes are the hi and lo halves");
  constexpr bool GT = ACT == 1;                        // ReGLU: a gate row per neuron
  constexpr int NH = EXACT && !PACK ? 2 : 1;           // token fragment planes (hi, lo; PACK: both in one)
  constexpr int WV = Q4 ? 1 : 4;                       // uint4 of weights per lane and matrix per quad
  __shared__ uint64_t wl[WMAXR * NTR];                 // mask words
  __shared__ int roff[NTR];
  __shared__ int tmp[NTR / 64 + 4];
  __shared__ int ids[R16];
  __shared__ f32x4 red[3][2][64];                      // waves 1..3's partial sums (up, gate)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nw = (F + 63) >> 6;
  const int wpt = (nw + NTR - 1) / NTR;
  const int n = mask_prefix<NTR, WMAXR>(mask, nw, F, wpt, wl, roff, tmp);
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_active = n;
  const int i0 = blockIdx.x * R16;
  if (i0 >= n) {                                       // block-uniform
    if (i0 < ((n + 63) & ~63)) {                       // inside the union's last 64-row block: a zero tile
      const int r = threadIdx.x >> 4, tok = threadIdx.x & 15, i = i0 + r;
      abuf[((size_t)(i >> 3) * 16 + tok) * 8 + (i & 7)] = 0.f;
    }
    return;
  }
  if (threadIdx.x < R16) {
    const int i = i0 + threadIdx.x;
    int id = -1;
    if (i < n) {                                       // the (i - roff)-th set bit after word range T * wpt
      int lo = 0, hi = NTR - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (roff[mid] <= i) lo = mid; else hi = mid - 1;
      }
      int rem = i - roff[lo];
      for (int tw = lo * wpt; tw < nw; ++tw) {
        const int cnt = __popcll(wl[tw]);
        if (rem < cnt) { id = tw * 64 + select_bit(wl[tw], rem); break; }
        rem -= cnt;
      }
      active[i] = id;
    }
    ids[threadIdx.x] = id;
  }
  __syncthreads();
  const int idl = ids[lane & 15];                      // this lane's A-operand row (-1: none)
  // the epilogue's biases and token power of two (wave 0), loaded now so that they arrive with the first quads
  float ebias[4], esx;
  {
    const float* bp = GT ? bg : bu;
    const Buf bb(bp ? (const void*)bp : (const void*)xsc, bp ? (uint32_t)F * 4u : 0u);   // no bias: 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = ids[(lane >> 4) * 4 + i];
      ebias[i] = bb.ldf(boff(w == 0 && id >= 0, (uint32_t)(id >= 0 ? id : 0) * 4u));
    }
    esx = Buf(xsc, 64u).ldf(boff(w == 0 && (lane & 15) < B, (uint32_t)(lane & 15) * 4u));
  }
  const int jq = lane >> 4;                            // lane group: the k block of a quad this lane holds
  const int KB = (D + 31) >> 5, nblk = D >> 5;
  const int KQ = (KB + 3) >> 2;                        // quads
  const int KQW = (KQ + 3) >> 2;                       // quads of one wave
  const int q0 = w * KQW, q1 = min(KQ, q0 + KQW);      // this wave's quads
  const int nq3 = (max(q1 - q0, 0) + 2) / 3 * 3;       // padded to rounds of three (the padding reads nothing)
  const Buf bx(xf, (uint32_t)KQ * 4u * (uint32_t)NH * 1024u);
  const uint32_t wbytes = Q4 ? (uint32_t)F * (uint32_t)(D >> 1) : (uint32_t)F * (uint32_t)D * 2u;
  const uint32_t sbytes = Q4 ? (uint32_t)F * (uint32_t)nblk * 2u : 0u;
  const Buf bwu(Wu, wbytes), bwg(GT ? Wg : Wu, GT ? wbytes : 0u);
  const Buf bsu(Q4 ? Su : Wu, sbytes), bsg(Q4 && GT ? Sg : Wu, GT ? sbytes : 0u);
  const uint32_t row = (uint32_t)(idl >= 0 ? idl : 0);
  struct Set {
    uint4 wu[WV], wg[WV];
    uint32_t su, sg;                                   // block scales' fp16 bits (32-bit: kept in registers)
    uint4 xv[4][NH];
  };
  auto load = [&](int g, Set& S) {                     // quad g of the wave's range (past q1: nothing)
    const int kb = g * 4 + jq;                         // Q4_0: this lane's k block of the quad
    const bool ok = g < q1 && kb < KB && idl >= 0;
    const bool okh = g < q1 && idl >= 0;               // fp16: the element bound is checked per load
    if constexpr (Q4) {
      const uint32_t o = row * (uint32_t)(D >> 1) + (uint32_t)kb * 16u;
      S.wu[0] = bwu.ld16(boff(ok, o));
      if (GT) S.wg[0] = bwg.ld16(boff(ok, o));
      const uint32_t so = (row * nblk + kb) * 2u;
      S.su = bsu.ldu16(boff(ok, so));
      if (GT) S.sg = bsg.ldu16(boff(ok, so));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {                    // block-major: elements 8 jq .. 8 jq + 7 of block 4 g + q
        const int k = (g * 4 + q) * 32 + jq * 8;
        const uint32_t o = (row * (uint32_t)D + (uint32_t)k) * 2u;
        S.wu[q] = bwu.ld16(boff(okh && k < D, o));
        if (GT) S.wg[q] = bwg.ld16(boff(okh && k < D, o));
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        S.xv[q][h] = bx.ld16(boff(g < q1, (((uint32_t)(g * 4 + q) * NH + h) * 64u + lane) * 16u));
  };
  f32x4 au = {0.f, 0.f, 0.f, 0.f}, ag = au;
  auto compute = [&](const Set& S) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half8 a_u, a_g;
      if constexpr (Q4) {                              // fp16((q - 8) s): one rounding per weight
        a_u = q4_half8(S.wu[0], q) * splat8(S.su);
        if (GT) a_g = q4_half8(S.wg[0], q) * splat8(S.sg);
      } else {
        a_u = __builtin_bit_cast(half8, S.wu[q]);
        if (GT) a_g = __builtin_bit_cast(half8, S.wg[q]);
      }
      const half8 xh = __builtin_bit_cast(half8, S.xv[q][0]);
      if constexpr (EXACT && !PACK) {
        const half8 xo = __builtin_bit_cast(half8, S.xv[q][NH - 1]);
        au = mfma16(a_u, xo, mfma16(a_u, xh, au));
        if (GT) ag = mfma16(a_g, xo, mfma16(a_g, xh, ag));
      } else {
        au = mfma16(a_u, xh, au);
        if (GT) ag = mfma16(a_g, xh, ag);
      }
    }
  };
  Set S0, S1, S2;
  load(q0, S0);
  load(q0 + 1, S1);
  for (int c = 0; c < nq3; c += 3) {                   // nq3 is a multiple of 3
    load(q0 + c + 2, S2);
    compute(S0);
    load(q0 + c + 3, S0);
    compute(S1);
    load(q0 + c + 4, S1);
    compute(S2);
  }
  // the waves' partial sums, added in wave order by wave 0
  if (w > 0) {
    red[w - 1][0][lane] = au;
    if (GT) red[w - 1][1][lane] = ag;
  }
  __syncthreads();
  if (w > 0) return;                                   // wave-uniform
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    au += red[k][0][lane];
    if (GT) ag += red[k][1][lane];
  }
  // epilogue: lane l holds rows 4 (l / 16) + i of token l % 16; the token's power of two back, bias, activation
  if constexpr (PACK) {                                // column t + 8 holds the lo half's sums of token t < 8
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      au[i] += __shfl_xor(au[i], 8, 64);
      if (GT) ag[i] += __shfl_xor(ag[i], 8, 64);
    }
  }
  const int tok = lane & 15;
  const int r0 = i0 + (lane >> 4) * 4;                 // this lane's 4 rows: half an octet
  const float sx = esx;
  float a4[4], amx = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ii = r0 + i;
    const float bias = ebias[i];
    const float u = au[i] * sx, g = ag[i] * sx;
    float a;
    if (GT) {
      a = fmaxf(g + bias, 0.f) * u;
    } else {
      a = fmaxf(u + bias, 0.f);
      if (ACT == 2) a *= a;
    }
    a4[i] = (tok < B && ii < n) ? a : 0.f;
    amx = fmaxf(amx, fabsf(a4[i]));
  }
  *reinterpret_cast<float4*>(&abuf[((size_t)(r0 >> 3) * 16 + tok) * 8 + (r0 & 7)]) =
      make_float4(a4[0], a4[1], a4[2], a4[3]);
  amx = fmaxf(amx, __shfl_xor(amx, 16, 64));
  amx = fmaxf(amx, __shfl_xor(amx, 32, 64));
  if (lane < B) bmax[(size_t)(i0 / R16) * B + lane] = amx;
}

// The predictor's second stage for a batch of tokens on the same tiling (PowerInfer pages, Turkish article,
// "Adaptive sparsity predictors": z = P2 h + c per token, a neuron marked if any token's z passes the threshold).
// h [B, r] is first split by k_split_x into token fragments (scaled by a power of two per token, two fp16 planes);
// k_mz then streams every row of P2 (64 neurons per workgroup, 16 per wave, 4 k blocks per chunk, two chunks
// ahead in three register sets, the chunk's fragments shared through LDS) and takes exact products into fp32 sums.
// Epilogue: z = sum * 2^e + c (the always-active prefix: +inf, its row never read), optional logits[token][neuron],
// and the OR over tokens by ballot into the block's mask word.
template <int RT, int NTT>
__global__ __launch_bounds__(64 * RT) void k_mz(const void* __restrict__ P2, const float* __restrict__ c,
                                                const uint4* __restrict__ hf, const float* __restrict__ hsc, int B,
                                                int F, int r, float tau, int n_hot, uint64_t* __restrict__ mask,
                                                float* __restrict__ logits) {
  // RT waves of 16 neurons each (4 or 8): every chunk of h fragments staged serves 16 RT neurons
  constexpr int NT = 64 * RT;
  constexpr int NH = 2, KC = 4;                        // two fp16 planes; 4 k blocks (a quad) per chunk
  constexpr int XV = KC * NTT * NH * 64 / NT;
  static_assert(XV * NT == KC * NTT * NH * 64, "fragment share");
  __shared__ uint4 xl[2][KC * NTT * NH * 64];          // token fragments of two chunks
  __shared__ uint32_t bits16[RT];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16 * RT + w * 16;
  const int rl = row0 + (lane & 15);                   // this lane's A-operand row
  const bool live = rl < F && rl >= n_hot;             // the prefix reads no row
  const uint32_t row = (uint32_t)(live ? rl : 0);
  const int jq = lane >> 4;
  const int KB = (r + 31) >> 5, KQ = (KB + 3) >> 2;
  const int nch = (KQ + 2) / 3 * 3;                    // chunks (one quad each), padded to rounds of three
  const Buf bx(hf, (uint32_t)KQ * 4u * NTT * NH * 1024u);   // chunks past KQ read 0
  const Buf bw(P2, (uint32_t)F * (uint32_t)r * 2u);
  struct Set {
    uint4 xv[XV];
    uint4 wv[4];
  };
  auto load = [&](int g, Set& S) {
#pragma unroll
    for (int m = 0; m < XV; ++m)
      S.xv[m] = bx.ld16(((uint32_t)g * 4u * NTT * NH * 64 + (uint32_t)(m * NT) + threadIdx.x) * 16u);
    const bool ok = g < KQ && live;
#pragma unroll
    for (int q = 0; q < 4; ++q) {                      // block-major: elements 8 jq .. 8 jq + 7 of block 4 g + q
      const int k = (g * 4 + q) * 32 + jq * 8;
      S.wv[q] = bw.ld16(boff(ok && k < r, (row * (uint32_t)r + (uint32_t)k) * 2u));
    }
  };
  auto store_x = [&](const Set& S, int buf) {
#pragma unroll
    for (int m = 0; m < XV; ++m) xl[buf][m * NT + threadIdx.x] = S.xv[m];
  };
  f32x4 az[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) az[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Set& S, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const half8 a = __builtin_bit_cast(half8, S.wv[q]);
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        const int f = (q * NTT + t) * NH;
        const half8 xh = __builtin_bit_cast(half8, xl[buf][f * 64 + lane]);
        const half8 xo = __builtin_bit_cast(half8, xl[buf][(f + 1) * 64 + lane]);
        az[t] = mfma16(a, xo, mfma16(a, xh, az[t]));
      }
    }
  };
  Set S0, S1, S2;
  load(0, S0);
  load(1, S1);
  store_x(S0, 0);
  __syncthreads();
  for (int cc = 0; cc < nch; cc += 3) {                // nch is a multiple of 3
    load(cc + 2, S2);
    compute(S0, cc & 1);
    store_x(S1, (cc + 1) & 1);
    __syncthreads();
    load(cc + 3, S0);
    compute(S1, (cc + 1) & 1);
    store_x(S2, cc & 1);
    __syncthreads();
    load(cc + 4, S1);
    compute(S2, cc & 1);
    store_x(S0, (cc + 1) & 1);
    __syncthreads();
  }
  // lane l holds neurons row0 + 4 (l / 16) + i of token t * 16 + l % 16
  const Buf bc(c ? (const void*)c : (const void*)P2, c ? (uint32_t)F * 4u : 0u);   // no bias: every load is 0
  float cb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = row0 + (lane >> 4) * 4 + i;
    cb[i] = bc.ldf(boff(kk < F && kk >= n_hot, (uint32_t)kk * 4u));
  }
  float sx[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    const int tok = t * 16 + (lane & 15);
    sx[t] = tok < B ? hsc[tok] : 0.f;
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = row0 + (lane >> 4) * 4 + i;
    bool any = false;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int tok = t * 16 + (lane & 15);
      const float z = kk < n_hot ? INFINITY : fmaf(az[t][i], sx[t], cb[i]);
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
  const int wi = blockIdx.x * (RT / 4) + (int)threadIdx.x;   // one mask word per 64 neurons (those below F)
  if ((int)threadIdx.x < RT / 4 && wi < (F + 63) / 64) {
    const int h = threadIdx.x;
    mask[wi] = (uint64_t)bits16[4 * h] | ((uint64_t)bits16[4 * h + 1] << 16) | ((uint64_t)bits16[4 * h + 2] << 32) |
               ((uint64_t)bits16[4 * h + 3] << 48);
  }
}

template <int XPT, bool EXACT, bool PERM, bool PACK = false>
hipError_t launch_split_x(const float* x, int x_norm, int B, int D, int NTT, uint4* xf, float* xs, hipStream_t st,
                          int nparts = 0) {
  if (PACK && (NTT != 1 || B > 8)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_split_x<XPT, EXACT, PERM, PACK>), dim3(PACK ? 8 : NTT * 16), dim3(NTX), 0, st, x, x_norm, B,
                     D, NTT, xf, xs, nparts);
  return hipGetLastError();
}

template <bool EXACT, bool PERM, bool PACK = false>
hipError_t split_x_xpt(int xpt, const float* x, int x_norm, int B, int D, int NTT, uint4* xf, float* xs,
                       hipStream_t st) {
  if (xpt <= 1) return launch_split_x<1, EXACT, PERM, PACK>(x, x_norm, B, D, NTT, xf, xs, st);
  if (xpt <= 2) return launch_split_x<2, EXACT, PERM, PACK>(x, x_norm, B, D, NTT, xf, xs, st);
  if (xpt <= 4) return launch_split_x<4, EXACT, PERM, PACK>(x, x_norm, B, D, NTT, xf, xs, st);
  if (xpt <= 8) return launch_split_x<8, EXACT, PERM, PACK>(x, x_norm, B, D, NTT, xf, xs, st);
  if (xpt <= 16) return launch_split_x<16, EXACT, PERM, PACK>(x, x_norm, B, D, NTT, xf, xs, st);
  return hipErrorInvalidValue;
}

// k halves of k_ur by token tiles. Measured at the 13B shape: 64 tokens 101 -> 85 us per layer with two (8 waves);
// 32 tokens (2 tiles) the same either way; 8 and 16 tokens the same.
constexpr int ur_halves(int ntt) { return ntt >= 4 ? 2 : 1; }
// Row tiles of k_ur (16 rows each): 8 where a union of up to F rows would give more than 1.5 workgroups of 64 rows
// per CU (UR_WIDE_ROWS), with two k halves: every token fragment loaded then serves 128 rows instead of 64.
constexpr int UR_WIDE_ROWS = 384 * 64;

template <int NTT, int ACT, bool Q4, bool EXACT>
hipError_t launch_ur(const void* Wg, const void* Sg, const float* bg, const void* Wu, const void* Su, const float* bu,
                     const float* x, int x_norm, int B, int D, int F, const uint64_t* mask, int32_t* active,
                     int32_t* n_active, float* abuf, float* bmax, uint4* xf, float* xs, float* pre, int KS,
                     hipStream_t st) {
  const int xpt = (D / 4 + NTX - 1) / NTX;
  hipError_t e;
  static_assert(!(Q4 && EXACT), "Q4_0 rows take fp16 tokens");
  // the fragment order of the row kernel that runs (k_ur16, up to UR16_MAX_B tokens: fp16 block-major)
  constexpr bool BMUR = ur_block_major(Q4, ur_halves(NTT));
  // up to 8 tokens with fp16 rows and exact tokens: hi and lo packed in one plane (block-major, as both row kernels
  // read fp16 rows there)
  constexpr bool PK = NTT == 1 && !Q4 && EXACT;
  static_assert(UR16_MAX_B <= 8 && (!PK || BMUR), "packed planes hold up to 8 tokens");
  const bool ur16 = NTT == 1 && B <= UR16_MAX_B;
  const bool pack = PK && B <= 8;
  if (pack)
    e = split_x_xpt<EXACT, true, PK>(xpt, x, x_norm, B, D, NTT, xf, xs, st);
  else
    e = (ur16 ? !Q4 : BMUR) ? split_x_xpt<EXACT, true>(xpt, x, x_norm, B, D, NTT, xf, xs, st)
                            : split_x_xpt<EXACT, false>(xpt, x, x_norm, B, D, NTT, xf, xs, st);
  if (e != hipSuccess) return e;
  if ((F + 63) / 64 > WMAXR * NTR || KS < 1 || (KS > 1 && !pre)) return hipErrorInvalidValue;
  if (ur16) {                                          // 16-row workgroups, k split over the waves
    SFFN_LAUNCH(2, (k_ur16<ACT, Q4, EXACT, PK>), dim3((F + R16 - 1) / R16), dim3(NTR), 0, st, Wg, Sg, bg, Wu, Su, bu,
                (const uint4*)xf, xs, B, D, F, mask, active, n_active, abuf, bmax);
    return hipGetLastError();
  }
  constexpr int KH = ur_halves(NTT);
  if constexpr (KH == 2) {
    if (F > UR_WIDE_ROWS) {
      SFFN_LAUNCH(2, (k_ur<8, KH, NTT, ACT, Q4, EXACT, false>), dim3((F + 127) / 128 * KS), dim3(64 * 8 * KH), 0, st,
                  Wg, Sg, bg, Wu, Su, bu, (const uint4*)xf, xs, B, D, F, mask, active, n_active, abuf, bmax, pre, KS);
      e = hipGetLastError();
      if (e != hipSuccess || KS == 1) return e;
      return sffn_launch_act_combine(ACT, pre, KS, active, n_active, GT_BIAS(ACT, bg, bu), B, F, abuf, bmax, st);
    }
  }
  if (pack) {
    SFFN_LAUNCH(2, (k_ur<4, KH, NTT, ACT, Q4, EXACT, PK>), dim3((F + 63) / 64 * KS), dim3(64 * 4 * KH), 0, st, Wg,
                Sg, bg, Wu, Su, bu, (const uint4*)xf, xs, B, D, F, mask, active, n_active, abuf, bmax, pre, KS);
  } else {
    SFFN_LAUNCH(2, (k_ur<4, KH, NTT, ACT, Q4, EXACT, false>), dim3((F + 63) / 64 * KS), dim3(64 * 4 * KH), 0, st, Wg,
                Sg, bg, Wu, Su, bu, (const uint4*)xf, xs, B, D, F, mask, active, n_active, abuf, bmax, pre, KS);
  }
  e = hipGetLastError();
  if (e != hipSuccess || KS == 1) return e;
  return sffn_launch_act_combine(ACT, pre, KS, active, n_active, GT_BIAS(ACT, bg, bu), B, F, abuf, bmax, st);
}

// Q4_0 rows always take fp16 tokens (the weights are rounded to fp16 with their scale); fp16 rows take them as
// two halves when EXACT
template <int NTT, bool EXACT>
hipError_t ur_act(int act, bool q4, const void* Wg, const void* Sg, const float* bg, const void* Wu, const void* Su,
                  const float* bu, const float* x, int x_norm, int B, int D, int F, const uint64_t* mask,
                  int32_t* active, int32_t* n_active, float* abuf, float* bmax, uint4* xf, float* xs, float* pre,
                  int KS, hipStream_t st) {
#define UR(A, Q, E) return launch_ur<NTT, A, Q, E>(Wg, Sg, bg, Wu, Su, bu, x, x_norm, B, D, F, mask, active, \
                                                   n_active, abuf, bmax, xf, xs, pre, KS, st)
  if (act == 1) { if (q4) UR(1, true, false); UR(1, false, EXACT); }
  if (act == 2) { if (q4) UR(2, true, false); UR(2, false, EXACT); }
  if (q4) UR(0, true, false);
  UR(0, false, EXACT);
#undef UR
}

template <int NTT>
hipError_t launch_mz(const void* P2, const float* c, const float* h, int hparts, int B, int F, int r, float tau,
                     int n_hot, uint64_t* mask, float* logits, uint4* hf, float* hs, hipStream_t st) {
  const int xpt = (r / 4 + NTX - 1) / NTX;
  hipError_t e;
  if (hparts > SPLIT_PARTS_MAX) return hipErrorInvalidValue;
  if (xpt <= 1) e = launch_split_x<1, true, true>(h, 0, B, r, NTT, hf, hs, st, hparts);
  else return hipErrorInvalidValue;                    // r <= 1024
  if (e != hipSuccess) return e;
  if (F > UR_WIDE_ROWS) {                              // large layers: 128 neurons per workgroup (as k_ur)
    SFFN_LAUNCH(1, (k_mz<8, NTT>), dim3((F + 127) / 128), dim3(512), 0, st, P2, c, (const uint4*)hf, hs, B, F, r, tau,
                n_hot, mask, logits);
  } else {
    SFFN_LAUNCH(1, (k_mz<4, NTT>), dim3((F + 63) / 64), dim3(256), 0, st, P2, c, (const uint4*)hf, hs, B, F, r, tau,
                n_hot, mask, logits);
  }
  return hipGetLastError();
}

}  // namespace

// Predictor stage 2 for B tokens from h [B, r] (fp32; hparts > 0: the sum of hparts partials [hparts][B][r]) on the
// matrix cores: h split into token fragments in hf (sffn_ur_xf_bytes(B, r, true) bytes) with its powers of two in
// hs, then z, threshold and the union mask.
hipError_t sffn_launch_predict_mz(const void* P2, const float* c, const float* h, int hparts, int B, int F, int r,
                                  float tau, int n_hot, uint64_t* mask, float* logits, void* hf, float* hs,
                                  hipStream_t st) {
  if (r % 8 || r > 1024) return hipErrorInvalidValue;
  switch ((B + 15) / 16) {
    case 1: return launch_mz<1>(P2, c, h, hparts, B, F, r, tau, n_hot, mask, logits, (uint4*)hf, hs, st);
    case 2: return launch_mz<2>(P2, c, h, hparts, B, F, r, tau, n_hot, mask, logits, (uint4*)hf, hs, st);
    case 3: return launch_mz<3>(P2, c, h, hparts, B, F, r, tau, n_hot, mask, logits, (uint4*)hf, hs, st);
    case 4: return launch_mz<4>(P2, c, h, hparts, B, F, r, tau, n_hot, mask, logits, (uint4*)hf, hs, st);
    default: return hipErrorInvalidValue;
  }
}

// Bytes of the token fragments k_split_x writes for B tokens of D values (EXACT: two planes): whole quads of k blocks.
size_t sffn_ur_xf_bytes(int B, int D, bool exact) {
  return (size_t)((D + 127) / 128) * 4 * ((B + 15) / 16) * (exact ? 2 : 1) * 1024;
}

// Shares of the k range per 64 union rows: few tokens mean few union rows, so more shares keep the CUs busy.
int sffn_ur_shares(int B) { return B <= UR16_MAX_B ? 1 : (B <= 8 ? 8 : (B <= 16 ? 4 : (B <= 32 ? 2 : 1))); }

// log2 of the union rows per entry of the row kernels' largest-|a| table: 16-row tiles for the 16-row kernel, else 64
int sffn_ur_bmax_shift(int B) { return B <= UR16_MAX_B ? 4 : 6; }

hipError_t sffn_launch_rows_ur(int act, bool q4, bool exact, const void* Wg, const void* Sg, const float* bg,
                               const void* Wu, const void* Su, const float* bu, const float* x, int x_norm, int B,
                               int D, int F, const uint64_t* mask, int32_t* active, int32_t* n_active, float* abuf,
                               float* bmax, void* xf, float* xs, float* pre, hipStream_t st) {
  const int ntt = (B + 15) / 16;
  const int KS = sffn_ur_shares(B);
#define URN(N) return exact ? ur_act<N, true>(act, q4, Wg, Sg, bg, Wu, Su, bu, x, x_norm, B, D, F, mask, active,   \
                                              n_active, abuf, bmax, (uint4*)xf, xs, pre, KS, st)                      \
                            : ur_act<N, false>(act, q4, Wg, Sg, bg, Wu, Su, bu, x, x_norm, B, D, F, mask, active,  \
                                               n_active, abuf, bmax, (uint4*)xf, xs, pre, KS, st)
  switch (ntt) {
    case 1: URN(1);
    case 2: URN(2);
    case 3: URN(3);
    case 4: URN(4);
    default: return hipErrorInvalidValue;
  }
#undef URN
}
