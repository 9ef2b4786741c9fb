// Single-token layer with the predictor's second stage folded into the row gather.
//
// PowerInfer pages, Turkish article: "Adaptive sparsity predictors" (the predictor runs on every token and marks
// the neurons that will fire) and "Neuron-aware operator" (only the marked neurons' rows and columns are read).
// The separate path runs h = P1 x, then z = P2 h + c with the threshold into a mask, then the row gather over
// the mask: three dependent phases. Here the second and third share one kernel, so a layer costs one launch and
// one dependent round trip less; the results are those of the separate calls.
//
// k_decode1 (G = 256 blocks of 8 waves): block b owns the stored neurons k = b + G j (j = 0, 1, ...), so every
// block holds a near-equal share of every probability band of a hot-first order. Round 1 issues, all before the
// first use: h, x, the P2 rows of the block's neurons (8 lanes per row, 16-byte chunks, a power-of-two number R
// of chunk rounds per row) and their biases. h goes to LDS while the rows are in flight; each lane's chunk dot
// products are summed over the R rounds in a fixed pairwise order, then over the 8 lanes of the row, and
// compared with tau (the always-active prefix k < n_hot is forced on; its P2 rows and biases are never loaded:
// their offsets are out of range, which reads 0 without a memory request). A ballot gives each wave's 8
// decisions per row step; they land in an LDS bitmap of the block's rows, and the block's active neurons, in
// ascending order, are picked from it by rank select. The gather that follows is k_fused1's (rowgather.h): per pass of 8
// rows each wave issues its row of W_gate / W_up and every thread its chunks of the pass's 8 W_downT rows, all
// together; x is normalised and staged while they are in flight; the activations go through LDS and every thread
// adds a_i W_downT[id_i, its chunks] in row order into the block's partial sum of y. Every block writes its
// partial (zeros if it has no active neuron) and its decision bitmap.
// k_sum_asm: y[d] = sum over the G partials in a fixed order (as k_sum_rows); extra blocks, 8 mask words each,
// assemble the blocks' bitmaps into the mask words and write the ascending ids of the set bits to active[] and
// their count to n_active.
#include "common.h"
#include "rowgather.h"

using namespace sffn;

namespace {

constexpr int NT_D = 512;            // 8 waves: rows per gather pass
constexpr int FWD = NT_D / 64;
constexpr int ZL = 8;                // lanes per P2 row
constexpr int ZRW = 64 / ZL;         // P2 rows per wave load instruction
constexpr int ZRS = ZRW * FWD;       // rows per row step of the block (64)
constexpr int ZS = 4;                // 16-byte P2 chunks in flight per lane: row steps x chunk rounds <= ZS
constexpr int JW = 4;                // 32-bit words of a block's decision bitmap: owned rows j < 128 (F <= 32768)

template <int ACT, int NCH, int DCH>
__global__ __launch_bounds__(NT_D) void k_decode1(const uint4* __restrict__ P2, const float* __restrict__ c,
                                                  const float* __restrict__ h, int r, int lr, float tau, int n_hot,
                                                  const uint4* __restrict__ Wg, const float* __restrict__ bg,
                                                  const uint4* __restrict__ Wu, const float* __restrict__ bu,
                                                  const uint4* __restrict__ WdT, const float* __restrict__ x,
                                                  int x_norm, int D, int F, uint32_t* __restrict__ dec,
                                                  float* __restrict__ logits, float* __restrict__ part) {
  extern __shared__ float4 lds4[];
  float* hs = reinterpret_cast<float*>(lds4);                        // [1024] h
  float* xs = hs + 1024;                                             // [D] x
  float* av = xs + D;                                                // [FWD] activations of the pass
  float* red = av + FWD;                                             // [2 * FWD + 4] normalisation scratch
  uint8_t* bits8 = reinterpret_cast<uint8_t*>(red + 2 * FWD + 4);    // [ZS * FWD] decision bytes, byte j / 8
  int* bids = reinterpret_cast<int*>(bits8 + ZS * FWD);              // [32 * JW] the block's active neuron ids
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = gridDim.x, blk = blockIdx.x;
  const int n4 = D >> 2;
  const int cpr = r >> 3;                              // 16-byte chunks per P2 row
  constexpr int XPT = (128 * NCH + NT_D - 1) / NT_D;
  const int rsub = lane / ZL, csub = lane % ZL;
  const int R = 1 << lr;                               // chunk rounds per P2 row (block-uniform)

  // round 1: h, x, the block's P2 rows and biases, every load issued before the first use (h first)
  const Buf bh(h, (uint32_t)r * 4u);
  const float4 hv = bh.ldf4(boff(4 * (int)threadIdx.x < r, threadIdx.x * 16u));
  float4 xv4[XPT];
  stage_load<NT_D, XPT>(x, n4, xv4);
  const float x0 = x[0];                               // shift for the single-pass statistics
  const Buf bp(P2, (uint32_t)F * (uint32_t)r * 2u);
  const Buf bc(c ? (const void*)c : (const void*)P2, c ? (uint32_t)F * 4u : 0u);   // no bias: every load is 0
  uint4 pv[ZS];
  float cb[ZS];
#pragma unroll
  for (int s = 0; s < ZS; ++s) {
    const int i = s >> lr, q = s & (R - 1);            // row step, chunk round
    const int k = blk + G * (i * ZRS + w * ZRW + rsub);
    const int cc = q * ZL + csub;
    const bool row = k < F && k >= n_hot;
    pv[s] = bp.ld16(boff(row && cc < cpr, ((uint32_t)k * cpr + cc) * 16u));
    cb[s] = bc.ldf(boff(row && q == 0, (uint32_t)k * 4u));
  }
  __builtin_amdgcn_sched_barrier(0);
  if ((int)threadIdx.x < ZS * FWD / 4) reinterpret_cast<uint32_t*>(bits8)[threadIdx.x] = 0u;   // rows never decided
  if (4 * (int)threadIdx.x < r) reinterpret_cast<float4*>(hs)[threadIdx.x] = hv;
  lds_barrier();

  // z of the block's rows: chunk dot products, summed over the R rounds (pairwise, fixed order), then over the
  // row's 8 lanes
  float d[ZS];
#pragma unroll
  for (int s = 0; s < ZS; ++s) {
    const int cc = (s & (R - 1)) * ZL + csub;
    float hv8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (cc < cpr) {
      const float4 a = *reinterpret_cast<const float4*>(hs + 8 * cc);
      const float4 b = *reinterpret_cast<const float4*>(hs + 8 * cc + 4);
      hv8[0] = a.x; hv8[1] = a.y; hv8[2] = a.z; hv8[3] = a.w; hv8[4] = b.x; hv8[5] = b.y; hv8[6] = b.z; hv8[7] = b.w;
    }
    d[s] = dot8(pv[s], hv8);
  }
#pragma unroll
  for (int o = 1; o < ZS; o <<= 1)
    if (o < R) {
#pragma unroll
      for (int s = 0; s + o < ZS; s += 2 * o) d[s] += d[s + o];
    }
#pragma unroll
  for (int s = 0; s < ZS; ++s) {
    if (s & (R - 1)) continue;                         // block-uniform
    const int i = s >> lr;
    const int k = blk + G * (i * ZRS + w * ZRW + rsub);
    const float zs = group_sum<ZL>(d[s]) + cb[s];
    const float z = k < n_hot ? INFINITY : zs;         // the always-active prefix: no row was read
    const bool own = csub == 0 && k < F;
    if (logits && own) logits[k] = z;
    const unsigned long long bal = __ballot(own && z > tau);
    uint32_t b8 = 0;
#pragma unroll
    for (int q = 0; q < ZRW; ++q)
      if ((bal >> (q * ZL)) & 1ull) b8 |= 1u << q;
    if (lane == 0) bits8[i * FWD + w] = (uint8_t)b8;   // rows i * 64 + w * 8 + (0..7): byte (row / 8)
  }
  lds_barrier();

  // the block's active rows in ascending order: the t-th set bit of the bitmap is row t of the gather
  const uint32_t* bw = reinterpret_cast<const uint32_t*>(bits8);
  uint32_t words[JW];
  int nrow = 0;
#pragma unroll
  for (int q = 0; q < JW; ++q) { words[q] = bw[q]; nrow += __popc(words[q]); }
  if ((int)threadIdx.x < nrow) {
    int t = threadIdx.x, q = 0;
#pragma unroll
    for (int qq = 0; qq < JW - 1; ++qq)
      if (q == qq && t >= __popc(words[qq])) { t -= __popc(words[qq]); q = qq + 1; }
    bids[threadIdx.x] = blk + G * (32 * q + select_bit((uint64_t)words[q], t));
  }
  if ((int)threadIdx.x < JW) dec[threadIdx.x * G + blk] = bw[threadIdx.x];
  lds_barrier();

  gather_rows<ACT, NCH, DCH, NT_D, XPT, false>(bids, nrow, Wg, bg, Wu, bu, WdT, D, F, x_norm, x0, xv4, xs, red, av,
                                               part, nullptr, 0, 0);   // every block writes its partial
}

constexpr int NT_S = 512;            // 32 columns x 16 groups of blocks
constexpr int GD = 256;              // workgroups of the folded kernel (the neuron-to-block map k % GD)
constexpr int SC = 32;
constexpr int SG = NT_S / SC;
constexpr int SPG = 16;              // partials per group: G <= SG * SPG = 256

// Blocks 0 .. ncol - 1: y over 32 columns each, the G = 256 partials summed in a fixed order. Blocks ncol + a:
// mask words 8a .. 8a + 7 (neuron k = block k % 256, owned row k / 256), the ascending ids of their set bits, and
// (a == 0) their total count. Each assembler block reads all 256 bitmaps (4 KiB, the same lines for every block);
// neurons below its first one, 512 a, are the bitmaps' rows below 2 a, so its offset in active[] is a popcount
// of those rows. One wave per word: lane e takes the bitmap of block (64 t + e) % 256, a ballot forms the word,
// and each lane writes its own bit's id.
__global__ __launch_bounds__(NT_S) void k_sum_asm(const float* __restrict__ part, int G, int D, int ncol,
                                                  float* __restrict__ y, const uint32_t* __restrict__ dec, int F,
                                                  uint64_t* __restrict__ mask, int32_t* __restrict__ active,
                                                  int32_t* __restrict__ n_active) {
  __shared__ float red[SG][SC];
  __shared__ uint32_t dl[JW * GD];
  __shared__ int cnt[2][NT_S / 64];
  __shared__ uint64_t wl[NT_S / 64];
  if ((int)blockIdx.x >= ncol) {                       // block-uniform: an assembler
    constexpr int NWV = NT_S / 64;                     // words per assembler block (one per wave)
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int a = blockIdx.x - ncol;
    const int nw = (F + 63) >> 6;
    const int jlo = 2 * a;                             // rows of the bitmaps below this block's first neuron
    constexpr int EPT = JW * GD / NT_S;                // bitmap words per thread
    const Buf bd(dec, (uint32_t)(JW * GD) * 4u);
    uint32_t v[EPT];
#pragma unroll
    for (int m = 0; m < EPT; ++m) v[m] = bd.ldu((threadIdx.x + NT_S * m) * 4u);
    int below = 0, all = 0;
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
      const int e = threadIdx.x + NT_S * m;            // word q = e / GD of block e % GD: rows 32 q .. 32 q + 31
      dl[e] = v[m];
      const int lo = jlo - 32 * (e / GD);              // rows of this word below jlo
      const uint32_t keep = lo >= 32 ? ~0u : (lo <= 0 ? 0u : ((1u << lo) - 1u));
      below += __popc(v[m] & keep);
      all += __popc(v[m]);
    }
    below = (int)wave_sum((float)below);               // exact: counts below 2^24
    all = (int)wave_sum((float)all);
    if (lane == 0) { cnt[0][w] = below; cnt[1][w] = all; }
    __syncthreads();
    int pre = 0, total = 0;
#pragma unroll
    for (int i = 0; i < NWV; ++i) { pre += cnt[0][i]; total += cnt[1][i]; }
    if (a == 0 && threadIdx.x == 0) *n_active = total;
    const int t = NWV * a + w;                         // this wave's mask word
    uint64_t word = 0;
    if (t < nw) {                                      // wave-uniform
      const int k = 64 * t + lane;
      const int j = k / GD;
      word = __ballot(k < F && ((dl[(j >> 5) * GD + (k % GD)] >> (j & 31)) & 1u));
      if (lane == 0) mask[t] = word;
    }
    if (lane == 0) wl[w] = word;
    __syncthreads();
    int off = pre;
    for (int i = 0; i < w; ++i) off += __popcll(wl[i]);
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
    if ((word >> lane) & 1ull) active[off + __popcll(word & lt)] = 64 * t + lane;
    return;
  }
  const int c = threadIdx.x % SC, g = threadIdx.x / SC;
  const int col = blockIdx.x * SC + c;
  const Buf bp(part, (uint32_t)G * (uint32_t)D * 4u);
  float v[SPG];
#pragma unroll
  for (int k = 0; k < SPG; ++k) {
    const int b = g + SG * k;
    v[k] = bp.ldf(boff(b < G && col < D, ((uint32_t)b * D + col) * 4u));
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < SPG; ++k) s += v[k];
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && col < D) {
    float tt = 0.f;
#pragma unroll
    for (int k = 0; k < SG; ++k) tt += red[k][c];
    y[col] = tt;
  }
}

// log2 of the chunk rounds per P2 row: rounds = the power of two >= ceil(r / 64) (8 lanes of 16 bytes per round)
int z_log_rounds(int r) {
  const int need = (r / 8 + ZL - 1) / ZL;
  int lr = 0;
  while ((1 << lr) < need) ++lr;
  return lr;
}

template <int ACT, int NCH, int DCH>
hipError_t launch_decode(const void* P2, const float* c, const float* h, int r, float tau, int n_hot, const void* Wg,
                         const float* bg, const void* Wu, const float* bu, const void* WdT, const float* x, int x_norm,
                         int D, int F, uint32_t* dec, float* logits, float* part, int G, uint64_t* mask,
                         int32_t* active, int32_t* n_active, float* y, hipStream_t st) {
  const size_t lds = (1024 + (size_t)D + FWD + 2 * FWD + 4) * sizeof(float) + ZS * FWD + 32 * JW * sizeof(int);
  static LdsLimit lds_limit;   // per kernel, set once per device
  size_t avail = 0;
  hipError_t ea = lds_limit.get((const void*)k_decode1<ACT, NCH, DCH>, &avail);
  if (ea != hipSuccess) return ea;
  if (lds > avail || G != GD) return hipErrorInvalidValue;
  SFFN_LAUNCH(2, (k_decode1<ACT, NCH, DCH>), dim3(G), dim3(NT_D), lds, st, (const uint4*)P2, c, h, r, z_log_rounds(r), tau,
              n_hot, (const uint4*)Wg, bg, (const uint4*)Wu, bu, (const uint4*)WdT, x, x_norm, D, F, dec, logits,
              part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ncol = (D + SC - 1) / SC, nasm = ((F + 63) / 64 + NT_S / 64 - 1) / (NT_S / 64);
  SFFN_LAUNCH(3, k_sum_asm, dim3(ncol + nasm), dim3(NT_S), 0, st, part, G, D, ncol, y, dec, F, mask, active, n_active);
  return hipGetLastError();
}

// P2 chunks per lane the block's rows need: row steps of 64 owned rows x chunk rounds
int z_slots(int F, int r) { return ((F + GD - 1) / GD + ZRS - 1) / ZRS << z_log_rounds(r); }

template <int ACT>
hipError_t dispatch_decode(const void* P2, const float* c, const float* h, int r, float tau, int n_hot,
                           const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                           const float* x, int x_norm, int D, int F, uint32_t* dec, float* logits, float* part, int G,
                           uint64_t* mask, int32_t* active, int32_t* n_active, float* y, hipStream_t st) {
  const int nch = (D / 8 + 63) / 64;
#define DE(N, Q) return launch_decode<ACT, N, Q>(P2, c, h, r, tau, n_hot, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, dec, \
                                                 logits, part, G, mask, active, n_active, y, st)
  if (nch <= 2) DE(2, 1);          // D <= 1024
  if (nch <= 4) DE(4, 1);          // D <= 2048
  if (nch <= 8) DE(8, 1);          // D <= 4096
  if (nch <= 10) DE(10, 2);        // D <= 5120
  if constexpr (ACT != 1) DE(16, 2);  // D <= 8192 (one matrix besides W_downT)
  return hipErrorInvalidValue;
#undef DE
}

}  // namespace

// The folded single-token layer applies where it measured faster than the separate kernels: fp16, D <= 4096,
// F <= 32768, and the block's P2 chunks fit four per lane (ceil(ceil(F / 256) / 64) row steps x chunk rounds
// <= 4). Measured: 7B shape 1414 -> 1467 tokens/s; 13B shape (D = 5120) 1018 either way; 40B shape (D = 8192, 16
// chunks per lane) 498 -> 485.
bool sffn_decode_ok(int act, int D, int F, int r, int G) {
  if (!sffn_fused_ok(1, D, F, act, false) || D > 4096 || G != GD) return false;
  return z_slots(F, r) <= ZS && (F + GD - 1) / GD <= 32 * JW;
}

size_t sffn_decode_dec_bytes(int G) { return (size_t)JW * G * sizeof(uint32_t); }

hipError_t sffn_launch_decode(int act, const void* P2, const float* c, const float* h, int r, float tau, int n_hot,
                              const void* Wg, const float* bg, const void* Wu, const float* bu, const void* WdT,
                              const float* x, int x_norm, int D, int F, uint32_t* dec, float* logits, float* part,
                              int G, uint64_t* mask, int32_t* active, int32_t* n_active, float* y, hipStream_t st) {
  switch (act) {
    case 1: return dispatch_decode<1>(P2, c, h, r, tau, n_hot, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, dec, logits, part,
                                      G, mask, active, n_active, y, st);
    case 2: return dispatch_decode<2>(P2, c, h, r, tau, n_hot, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, dec, logits, part,
                                      G, mask, active, n_active, y, st);
    default: return dispatch_decode<0>(P2, c, h, r, tau, n_hot, Wg, bg, Wu, bu, WdT, x, x_norm, D, F, dec, logits,
                                       part, G, mask, active, n_active, y, st);
  }
}
