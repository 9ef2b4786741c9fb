// Single-token row gather shared by the fused kernels (fused.hip, decode.hip).
//
// PowerInfer pages, Turkish article, "Neuron-aware operator": only the rows of W_gate / W_up and of W_downT that
// belong to the block's active neurons are read. Per pass of NT / 64 rows each wave issues the loads of its row of
// W_gate / W_up and every thread the loads of its 16-byte chunks of the pass's rows of W_downT, all together; on
// the first pass x is normalised (optionally) and staged in LDS while they are in flight. Each wave reduces its
// dot products to the activation a_i; the activations go through LDS and every thread adds a_i W_downT[id_i, its
// chunks] in row order. The block's partial sum of y over its rows is then written to part[block][D].
#pragma once
#include "common.h"

namespace sffn {

// ACT: 0 ReLU, 1 ReGLU (gate and up rows), 2 squared ReLU. bids[0 .. nrow): the block's neuron ids, in LDS.
// IDS: also store id k of pass row k at active[ids_base + ids_stride * k].
template <int ACT, int NCH, int DCH, int NT, int XPT, bool IDS>
__device__ __forceinline__ void gather_rows(const int* bids, int nrow, const void* Wg, const float* bg, const void* Wu,
                                            const float* bu, const void* WdT, int D, int F, int x_norm, float x0,
                                            float4 (&xv4)[XPT], float* xs, float* red, float* av, float* part,
                                            int32_t* active, int ids_base, int ids_stride) {
  constexpr int FW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nc = D >> 3, n4 = D >> 2;
  const uint32_t wbytes = (uint32_t)F * (uint32_t)D * 2u;
  const Buf bwu(Wu, wbytes), bwd(WdT, wbytes);
  const Buf bwg(ACT == 1 ? Wg : Wu, ACT == 1 ? wbytes : 0u);
  const float* bp = ACT == 1 ? bg : bu;
  const Buf bbias(bp ? (const void*)bp : Wu, bp ? (uint32_t)F * 4u : 0u);   // no bias: 0
  float acc[DCH][8];
#pragma unroll
  for (int q = 0; q < DCH; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
  const bool wq_last = (int)__builtin_amdgcn_readfirstlane(threadIdx.x) + NT * (DCH - 1) < nc;   // wave-uniform

  bool first = true;
  for (int k0 = 0; k0 < nrow; k0 += FW) {              // passes (block-uniform); row k0 + w on wave w
    const int k = k0 + w;
    const bool have = k < nrow;                        // wave-uniform
    // this wave's neuron, its gate/up rows and bias; then the pass's W_downT rows, all issued together
    int id = -1;
    uint4 wu[NCH], wg[NCH];
    float bias = 0.f;
    if (have) {
      id = bids[k];
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const int c = lane + 64 * m;
        const uint32_t o = boff(c < nc, ((uint32_t)id * nc + c) * 16u);
        wu[m] = bwu.ld16(o);
        if (ACT == 1) wg[m] = bwg.ld16(o);
      }
      bias = bbias.ldf((uint32_t)id * 4u);
    }
    uint4 wd[FW][DCH];
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int idj = k0 + j < nrow ? bids[k0 + j] : -1;
#pragma unroll
      for (int q = 0; q < DCH; ++q) {
        const int c = threadIdx.x + NT * q;
        if (q == DCH - 1 && !wq_last) {                // chunks past the row end on this whole wave: no load
          wd[j][q] = make_uint4(0u, 0u, 0u, 0u);
          continue;
        }
        wd[j][q] = bwd.ld16(boff(idj >= 0 && c < nc, ((uint32_t)(idj >= 0 ? idj : 0) * nc + c) * 16u));
      }
    }
    if (first) {                                       // x: normalised and staged while the rows are in flight
      if (x_norm) block_norm_regs<NT, XPT>(xv4, n4, x0, red);
      stage_store<NT, XPT>(xs, n4, xv4);
      lds_barrier();
      first = false;
    }
    if (have) {
      float au = 0.f, ag = 0.f;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const int c = lane + 64 * m;
        if (c < nc) {
          const float4* xp = reinterpret_cast<const float4*>(xs + 8 * c);
          const float4 xa = xp[0], xb = xp[1];
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
          au += dot8(wu[m], xv);
          if (ACT == 1) ag += dot8(wg[m], xv);
        }
      }
      const float u = wave_sum(au);
      float a;
      if (ACT == 1) {
        const float g = wave_sum(ag) + bias;
        a = fmaxf(g, 0.f) * u;
      } else {
        a = fmaxf(u + bias, 0.f);
        if (ACT == 2) a *= a;
      }
      if (lane == 0) {
        av[w] = a;
        if (IDS) active[ids_base + ids_stride * k] = id;
      }
    } else if (lane == 0) {
      av[w] = 0.f;
    }
    lds_barrier();
    // column gather of the pass, rows in wave order
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const float aj = av[j];
#pragma unroll
      for (int q = 0; q < DCH; ++q) {
        float wf[8];
        f16x8_to_f32(wd[j][q], wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(aj, wf[e], acc[q][e]);
      }
    }
    lds_barrier();                                     // ids / av are rewritten by the next pass
  }
  float* pb = part + (size_t)blockIdx.x * D;
#pragma unroll
  for (int q = 0; q < DCH; ++q) {
    const int c = threadIdx.x + NT * q;
    if (c < nc) {
      float4* o = reinterpret_cast<float4*>(pb + 8 * c);
      o[0] = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
      o[1] = make_float4(acc[q][4], acc[q][5], acc[q][6], acc[q][7]);
    }
  }
}

}  // namespace sffn
