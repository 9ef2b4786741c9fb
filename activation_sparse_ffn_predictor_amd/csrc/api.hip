// C ABI of libsffn: argument checks (host only, before anything is enqueued) and dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/sffn.h"
#include "common.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();   // reported here: do not leave it pending for the caller's next HIP call
  return fail(SFFN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int MAX_B = 64, MAX_D = 16384, MAX_F = 1 << 22, MAX_R = 1024, MAX_BR = 32768;
#ifndef SFFN_MAX_BD_VALU
#define SFFN_MAX_BD_VALU 16384
#endif
constexpr int MAX_BD_VALU = SFFN_MAX_BD_VALU;   // decode-batch kernels (B in {2, 4, 8}): B * D <= this
constexpr int MAX_F_UNION = 32768;   // union kernels compact the whole mask in one block
constexpr int KS_MAX = 16;           // k shares of the multi-token predictor's first stage
constexpr int UD_KS_MAX = 16;        // row shares of the union down projection
constexpr int MZ_MIN_B = 17;         // tokens from which the predictor's stage 2 runs on pre-split h fragments
constexpr int G_FUSED = 256;         // blocks (= partial sums of y) of the fused single-token forward
// fp16 weights in the union kernels: up to this many tokens the tokens and activations enter the matrix cores as
// exact fp16 hi + lo halves (packed into one operand plane, at no measured cost); beyond, as one fp16 value each
// (relative 2^-11, as with Q4_0 weights), which saves a second product per k block. Same box, 13B layer:
// 16 tokens 4292 -> 4365, 32 tokens 5871 -> 6183, 64 tokens 9336 -> 9911 tokens/s.
#ifndef SFFN_UNION_EXACT_MAX_B
#define SFFN_UNION_EXACT_MAX_B 8
#endif
bool union_exact(int B) { return B <= SFFN_UNION_EXACT_MAX_B; }
constexpr size_t MAX_TENSOR = (size_t)1 << 31;   // buffer loads address each tensor with 31-bit byte offsets
#ifndef SFFN_NOALLOC_SCRATCH_BYTES
#define SFFN_NOALLOC_SCRATCH_BYTES (16u << 20)   // device scratch of sffn_decode_noalloc, per GPU
#endif

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool al(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Predictor rank and P2 [F, r] fp16: the kernels address P2 with 31-bit byte offsets (buffer loads).
int check_rank(int F, int r) {
  if (r < 8 || r > MAX_R || r % 8) return fail(SFFN_ERR_SHAPE, "r=%d: need 8 <= r <= %d, r %% 8 == 0", r, MAX_R);
  if ((size_t)F * r * 2 >= MAX_TENSOR) return fail(SFFN_ERR_SHAPE, "F=%d, r=%d: P2 reaches 2 GiB", F, r);
  return SFFN_OK;
}

int check_common(int B, int D, int F) {
  if (B < 1 || B > MAX_B) return fail(SFFN_ERR_SHAPE, "B=%d outside [1, %d]", B, MAX_B);
  if (D < 8 || D > MAX_D || D % 8) return fail(SFFN_ERR_SHAPE, "D=%d: need 8 <= D <= %d, D %% 8 == 0", D, MAX_D);
  if (F < 1 || F > MAX_F) return fail(SFFN_ERR_SHAPE, "F=%d outside [1, %d]", F, MAX_F);
  if ((size_t)F * D * 2 >= MAX_TENSOR || (size_t)F * B * 4 >= MAX_TENSOR)
    return fail(SFFN_ERR_SHAPE, "F=%d, D=%d, B=%d: a tensor reaches 2 GiB", F, D, B);
  return SFFN_OK;
}

// Which kernels serve a call: B == 1 and B == 2 (with B * D <= 16384) take the decode kernels (x staged once per
// block in LDS); so do B in {4, 8} with B * D <= 16384 when F is too large for the union kernels' one-workgroup
// compaction. Every other batch takes the union kernels on the matrix cores, which measured faster from B = 4 on
// (7B shape: 2667 against 2218 tokens/s at B = 4) and slower at B = 2 (1465 against 1624).
bool decode_batch(int B, int D, int F) {
  if (B == 1) return true;
  if ((size_t)B * D > MAX_BD_VALU) return false;
  return B == 2 || ((B == 4 || B == 8) && F > MAX_F_UNION);
}

// Workspace layout, each part 256-byte aligned:
//   [activations a: F * B fp32, for B > 1 at least the union kernels' 64-row tiles of 16-token tiles
//    (ceil(F / 64) 64 x ceil(B / 16) 16 fp32); for B == 1 at least the decision bitmaps of the folded single-token
//    layer]
//   [B > 1: normalised x: B * D fp32]
//   [partial y: UD_KS_MAX * B * D fp32 for B > 1, G_FUSED * D fp32 for B == 1]
//   [B > 1: partial pre-activations][B > 1: token fragments and powers of two][B > 1: largest-|a| table]
//   [predictor h: B * r fp32]
size_t ws_a_bytes(int B, int F) {
  const size_t tiles = B > 1 ? (size_t)((F + 63) / 64) * 64 * ((B + 15) / 16) * 16 * sizeof(float) : 0;
  return align256(std::max({(size_t)F * B * sizeof(float), tiles,
                            B == 1 ? sffn_decode_dec_bytes(G_FUSED) : (size_t)0}));
}
size_t ws_xn_bytes(int B, int D) { return B > 1 ? align256((size_t)B * D * sizeof(float)) : 0; }
size_t ws_part_bytes(int B, int D) {
  static_assert(UD_KS_MAX >= KS_MAX, "the partials region serves both");
  return align256((size_t)(B > 1 ? UD_KS_MAX * B : G_FUSED) * D * sizeof(float));
}
// B > 1: partial pre-activations of the union row kernel's k shares, [KS][2][F][B] fp32 (KS > 1 up to 32 tokens)
size_t ws_pre_bytes(int B, int F) {
  const int ks = sffn_ur_shares(B);
  return B > 1 && ks > 1 ? align256((size_t)ks * 2 * F * B * sizeof(float)) : 0;
}
// B > 1: the union row kernel's token fragments (two fp16 planes) and the tokens' powers of two (16 per tile)
size_t ws_xf_bytes(int B, int D) {
  return B > 1 ? align256(sffn_ur_xf_bytes(B, D, true)) + align256((size_t)((B + 15) / 16) * 16 * sizeof(float)) : 0;
}
// B > 1: the row kernels' largest |activation| per row tile (16 or 64 union rows) and token, [tiles][B] fp32
size_t ws_bmax_bytes(int B, int F) {
  const int t = 1 << sffn_ur_bmax_shift(B);
  return B > 1 ? align256((size_t)((F + t - 1) / t) * B * sizeof(float)) : 0;
}
size_t ws_forward_bytes(int B, int D, int F) {
  return ws_a_bytes(B, F) + ws_xn_bytes(B, D) + ws_part_bytes(B, D) + ws_pre_bytes(B, F) + ws_xf_bytes(B, D) +
         ws_bmax_bytes(B, F);
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(SFFN_ERR_NULL, "workspace is NULL");
  if (!al(ws, 256)) return fail(SFFN_ERR_ALIGN, "workspace not 256-byte aligned");
  if (ws_bytes < need) return fail(SFFN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return SFFN_OK;
}

int check_union(int B, int D, int F) {
  if (!decode_batch(B, D, F) && F > MAX_F_UNION)
    return fail(SFFN_ERR_SHAPE, "forward: B=%d with D=%d takes the union kernels, which need F <= %d (F=%d)", B, D,
                MAX_F_UNION, F);
  return SFFN_OK;
}

float* ws_abuf(void* ws) { return (float*)ws; }
float* ws_xn(void* ws, int B, int F) { return (float*)((char*)ws + ws_a_bytes(B, F)); }
float* ws_part(void* ws, int B, int D, int F) { return (float*)((char*)ws + ws_a_bytes(B, F) + ws_xn_bytes(B, D)); }
float* ws_hbuf(void* ws, int B, int D, int F) { return (float*)((char*)ws + ws_forward_bytes(B, D, F)); }
float* ws_pre(void* ws, int B, int D, int F) {
  return (float*)((char*)ws + ws_a_bytes(B, F) + ws_xn_bytes(B, D) + ws_part_bytes(B, D));
}
void* ws_xf(void* ws, int B, int D, int F) { return (char*)ws_pre(ws, B, D, F) + ws_pre_bytes(B, F); }
float* ws_xs(void* ws, int B, int D, int F) {
  return (float*)((char*)ws_xf(ws, B, D, F) + align256(sffn_ur_xf_bytes(B, D, true)));
}
float* ws_bmax(void* ws, int B, int D, int F) { return (float*)((char*)ws_xf(ws, B, D, F) + ws_xf_bytes(B, D)); }

struct Prof {
  int kernel = -1;
  int max = 0;
  int used = 0;
  hipEvent_t* ev = nullptr;   // 2 * max events
};
thread_local Prof g_prof;

void prof_free() {
  if (g_prof.ev) {
    for (int i = 0; i < 2 * g_prof.max; ++i) hipEventDestroy(g_prof.ev[i]);
    delete[] g_prof.ev;
  }
  g_prof = Prof();
}

}  // namespace

bool sffn_prof_events(int kid, hipEvent_t* start, hipEvent_t* stop) {
  if (g_prof.kernel != kid || g_prof.used >= g_prof.max) return false;
  *start = g_prof.ev[2 * g_prof.used];
  *stop = g_prof.ev[2 * g_prof.used + 1];
  ++g_prof.used;
  return true;
}

namespace {

// Union path (B > 1 outside the decode batches): optional token normalisation, row gather + activation, down
// projection in row splits, sum of the splits.
hipError_t run_union(int act, bool q4, const void* Wg, const void* Sg, const float* bg, const void* Wu, const void* Su,
                     const float* bu, const void* Wd, const void* Sd, const float* x, int x_norm, int B, int D, int F,
                     const uint64_t* mask, int32_t* active, int32_t* n_active, float* y, void* ws, hipStream_t st) {
  hipError_t e = sffn_launch_rows_ur(act, q4, union_exact(B), Wg, Sg, bg, Wu, Su, bu, x, x_norm, B, D, F, mask, active,
                                     n_active, ws_abuf(ws), ws_bmax(ws, B, D, F), ws_xf(ws, B, D, F),
                                     ws_xs(ws, B, D, F), ws_pre(ws, B, D, F), st);
  if (e != hipSuccess) return e;
  return sffn_launch_down_ud(q4, union_exact(B), Wd, Sd, active, n_active, ws_abuf(ws), ws_bmax(ws, B, D, F),
                             sffn_ur_bmax_shift(B), B, D, F, ws_part(ws, B, D, F), sffn_ud_shares(D, UD_KS_MAX), y, st);
}

}  // namespace

extern "C" {

int sffn_profile_begin(int kernel, int max_launches) {
  g_err[0] = 0;
  if (kernel < SFFN_K_PRED_H || kernel > SFFN_K_COLS || max_launches < 1)
    return fail(SFFN_ERR_ARG, "profile: bad kernel %d or count %d", kernel, max_launches);
  prof_free();
  g_prof.ev = new hipEvent_t[2 * (size_t)max_launches];
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipError_t e = hipEventCreate(&g_prof.ev[i]);
    if (e != hipSuccess) {
      for (int k = 0; k < i; ++k) hipEventDestroy(g_prof.ev[k]);
      delete[] g_prof.ev;
      g_prof = Prof();
      return hip_fail(e, "profile: hipEventCreate");
    }
  }
  g_prof.kernel = kernel;
  g_prof.max = max_launches;
  return SFFN_OK;
}

int sffn_profile_end(float* ms, int max) {
  g_err[0] = 0;
  if (g_prof.kernel < 0) return -fail(SFFN_ERR_ARG, "profile: not started");
  const int n = g_prof.used;
  int rc = n;
  if (n > 0) {
    hipError_t e = hipEventSynchronize(g_prof.ev[2 * n - 1]);
    if (e != hipSuccess) rc = -hip_fail(e, "profile: hipEventSynchronize");
    for (int i = 0; rc >= 0 && i < n && i < max && ms; ++i) {
      e = hipEventElapsedTime(&ms[i], g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
      if (e != hipSuccess) rc = -hip_fail(e, "profile: hipEventElapsedTime");
    }
  }
  prof_free();
  return rc;
}


const char* sffn_status_string(int s) {
  switch (s) {
    case SFFN_OK: return "ok";
    case SFFN_ERR_NULL: return "null pointer";
    case SFFN_ERR_SHAPE: return "shape out of range";
    case SFFN_ERR_ALIGN: return "misaligned pointer";
    case SFFN_ERR_WORKSPACE: return "workspace too small";
    case SFFN_ERR_ACT: return "bad activation or missing operand";
    case SFFN_ERR_ARG: return "bad argument";
    case SFFN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sffn_last_error(void) { return g_err; }

size_t sffn_workspace_size(int B, int D, int F, int r) {
  if (B < 1 || D < 1 || F < 1 || r < 1) return 0;
  return ws_forward_bytes(B, D, F) + align256((size_t)B * r * sizeof(float));
}

int sffn_mask_words(int F) { return F < 1 ? 0 : (F + 63) / 64; }

int sffn_forward_path(int act, int q4, int B, int D, int F) {
  if (act != SFFN_ACT_RELU && act != SFFN_ACT_REGLU && act != SFFN_ACT_SQRELU) return -1;
  if (sffn_fused_ok(B, D, F, act, q4 != 0)) return SFFN_PATH_FUSED;
  return decode_batch(B, D, F) ? SFFN_PATH_DECODE : SFFN_PATH_UNION;
}

static int predict_impl(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D,
                        int F, int r, float t, int n_hot, uint64_t* mask, float* logits, void* ws, size_t ws_bytes,
                        void* stream) {
  g_err[0] = 0;
  if (!P1 || !P2 || !x || !mask) return fail(SFFN_ERR_NULL, "predict: P1, P2, x and mask are required");
  int s = check_common(B, D, F);
  if (s) return s;
  if (n_hot < 0 || n_hot > F) return fail(SFFN_ERR_ARG, "n_hot=%d outside 0..F=%d", n_hot, F);
  s = check_rank(F, r);
  if (s) return s;
  if ((long)B * r > MAX_BR) return fail(SFFN_ERR_SHAPE, "B*r=%ld > %d", (long)B * r, MAX_BR);
  if (!(t > 0.f && t < 1.f)) return fail(SFFN_ERR_ARG, "threshold t=%g outside (0, 1)", (double)t);
  if (!al(P1, 16) || !al(P2, 16) || !al(x, 16) || !al(mask, 8) || (c && !al(c, 4)) || (logits && !al(logits, 4)))
    return fail(SFFN_ERR_ALIGN, "predict: misaligned pointer");
  s = check_ws(ws, ws_bytes, sffn_workspace_size(B, D, F, r));
  if (s) return s;
  const float tau = (float)log((double)t / (1.0 - (double)t));
  hipStream_t st = (hipStream_t)stream;
  float* h = ws_hbuf(ws, B, D, F);
  hipError_t e;
  if (B == 1) {
    e = sffn_launch_predict(P1, P2, c, x, x_norm, B, D, F, r, tau, n_hot, mask, logits, h, st);
  } else if (B <= 8) {
    // a few tokens: h in one kernel (each P1 row read once with every token, normalisation folded in), then z
    e = sffn_launch_predict_hb(P1, x, x_norm, B, D, r, h, st);
    // z: vector-ALU kernel for up to 4 tokens, matrix-core kernel beyond (measured: equal at 4, faster at 8)
    if (e == hipSuccess)
      e = B <= 4 ? sffn_launch_predict_zb(P2, c, h, B, F, r, tau, n_hot, mask, logits, st)
                 : sffn_launch_predict_mt(P1, P2, c, x, B, D, F, r, tau, n_hot, mask, logits, h, nullptr, 0,
                                          nullptr, nullptr, st);
  } else {
    const float* xin = x;
    e = hipSuccess;
    if (x_norm) {
      e = sffn_launch_norm_tokens(x, B, D, ws_xn(ws, B, F), st);
      xin = ws_xn(ws, B, F);
    }
    // shares of d for the union predictor's first stage; their partial sums use the partials region
    // (KS_MAX * B * D floats >= ksh * B * r): 16 shares with the two-row-tile blocks from 17 tokens on, 8 below
    // (about 256 blocks either way at r = 512)
    const int ksm = B > 16 ? KS_MAX : KS_MAX / 2;
    const int ksh = std::max(1, std::min({ksm, D / 32 > 0 ? D / 32 : 1, (ksm * D) / r}));
    // stage 2 on pre-split h fragments (in the union row kernel's token-fragment region, free until the forward
    // call) from 17 tokens; below, its split launch costs more than the fragments save
    const bool mz = B > MZ_MIN_B - 1 && sffn_ur_xf_bytes(B, r, true) <= sffn_ur_xf_bytes(B, D, true);
    if (e == hipSuccess)
      e = sffn_launch_predict_mt(P1, P2, c, xin, B, D, F, r, tau, n_hot, mask, logits, h, ws_part(ws, B, D, F), ksh,
                                 mz ? ws_xf(ws, B, D, F) : nullptr, mz ? ws_xs(ws, B, D, F) : nullptr, st);
  }
  return e == hipSuccess ? SFFN_OK : hip_fail(e, "predict launch");
}

int sffn_predict(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D, int F, int r,
                 float t, uint64_t* mask, float* logits, void* ws, size_t ws_bytes, void* stream) {
  return predict_impl(P1, P2, c, x, x_norm, B, D, F, r, t, 0, mask, logits, ws, ws_bytes, stream);
}

int sffn_predict_hot(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D, int F,
                     int r, float t, int n_hot, uint64_t* mask, float* logits, void* ws, size_t ws_bytes, void* stream) {
  return predict_impl(P1, P2, c, x, x_norm, B, D, F, r, t, n_hot, mask, logits, ws, ws_bytes, stream);
}

int sffn_decode_path(int act, int q4, int D, int F, int r) {
  if (act != SFFN_ACT_RELU && act != SFFN_ACT_REGLU && act != SFFN_ACT_SQRELU) return -1;
  return !q4 && sffn_decode_ok(act, D, F, r, G_FUSED) ? SFFN_DECODE_FOLDED : SFFN_DECODE_SEPARATE;
}

int sffn_decode(int act, const void* P1, const void* P2, const float* c, float t, int n_hot, const void* W_gate,
                const float* b_gate, const void* W_up, const float* b_up, const void* W_downT, const float* x,
                int x_norm, int D, int F, int r, uint64_t* mask, int32_t* active, int32_t* n_active, float* y,
                float* logits, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (act != SFFN_ACT_RELU && act != SFFN_ACT_REGLU && act != SFFN_ACT_SQRELU)
    return fail(SFFN_ERR_ACT, "unknown activation %d", act);
  if (act == SFFN_ACT_REGLU && !W_gate) return fail(SFFN_ERR_ACT, "ReGLU needs W_gate");
  const int path = sffn_decode_path(act, 0, D, F, r);
  if (path == SFFN_DECODE_SEPARATE) {                  // the separate predictor and forward calls
    int s = predict_impl(P1, P2, c, x, x_norm, 1, D, F, r, t, n_hot, mask, logits, ws, ws_bytes, stream);
    if (s) return s;
    return sffn_forward(act, W_gate, b_gate, W_up, b_up, W_downT, x, x_norm, 1, D, F, mask, active, n_active, y, ws,
                        ws_bytes, stream);
  }
  if (!P1 || !P2 || !x || !mask || !W_up || !W_downT || !active || !n_active || !y)
    return fail(SFFN_ERR_NULL, "decode: P1, P2, x, W_up, W_downT, mask, active, n_active and y are required");
  int s = check_common(1, D, F);
  if (s) return s;
  s = check_rank(F, r);
  if (s) return s;
  if (!(t > 0.f && t < 1.f)) return fail(SFFN_ERR_ARG, "threshold t=%g outside (0, 1)", (double)t);
  if (n_hot < 0 || n_hot > F) return fail(SFFN_ERR_ARG, "n_hot=%d outside 0..F=%d", n_hot, F);
  if (!al(P1, 16) || !al(P2, 16) || !al(x, 16) || !al(mask, 8) || (c && !al(c, 4)) || (logits && !al(logits, 4)) ||
      (act == SFFN_ACT_REGLU && !al(W_gate, 16)) || !al(W_up, 16) || !al(W_downT, 16) || !al(active, 4) ||
      !al(n_active, 4) || !al(y, 16) || (b_gate && !al(b_gate, 4)) || (b_up && !al(b_up, 4)))
    return fail(SFFN_ERR_ALIGN, "decode: misaligned pointer");
  s = check_ws(ws, ws_bytes, sffn_workspace_size(1, D, F, r));
  if (s) return s;
  const float tau = (float)log((double)t / (1.0 - (double)t));
  const bool g = act == SFFN_ACT_REGLU;
  hipStream_t st = (hipStream_t)stream;
  float* h = ws_hbuf(ws, 1, D, F);
  hipError_t e = sffn_launch_predict_h(P1, x, x_norm, D, r, h, st);
  if (e == hipSuccess)
    e = sffn_launch_decode(act, P2, c, h, r, tau, n_hot, g ? W_gate : nullptr, g ? b_gate : nullptr, W_up,
                           g ? nullptr : b_up, W_downT, x, x_norm, D, F, (uint32_t*)ws_abuf(ws), logits,
                           ws_part(ws, 1, D, F), G_FUSED, mask, active, n_active, y, st);
  return e == hipSuccess ? SFFN_OK : hip_fail(e, "decode launch");
}

}  // extern "C"

namespace {

// Device scratch of sffn_decode_noalloc: one array per GPU, allocated with the code object when the library is
// loaded on that device and kept until the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: kernels and copies only ever get the per-device address from hipGetSymbolAddress.
constexpr size_t NOALLOC_BYTES = (size_t)SFFN_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

struct ScratchAddr {
  std::once_flag once[SFFN_MAX_DEVICES];
  void* ptr[SFFN_MAX_DEVICES] = {};
  hipError_t err[SFFN_MAX_DEVICES] = {};
};
ScratchAddr g_scratch;

// The current device's address of `scratch`, looked up once per device (with that device current).
hipError_t scratch_addr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SFFN_MAX_DEVICES) return hipErrorInvalidDevice;
  std::call_once(g_scratch.once[dev], [dev] {
    void* p = nullptr;
    g_scratch.err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch.ptr[dev] = g_scratch.err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch.err[dev] != hipSuccess) return g_scratch.err[dev];
  if (!g_scratch.ptr[dev] || !al(g_scratch.ptr[dev], 256)) return hipErrorInvalidSymbol;
  *out = g_scratch.ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t sffn_noalloc_scratch_bytes(void) { return NOALLOC_BYTES; }

int sffn_decode_noalloc(int act, const void* P1, const void* P2, const float* c, float t, int n_hot,
                        const void* W_gate, const float* b_gate, const void* W_up, const float* b_up,
                        const void* W_downT, const float* x, int x_norm, int D, int F, int r, uint64_t* mask,
                        int32_t* active, int32_t* n_active, float* y, float* logits, void* stream) {
  g_err[0] = 0;
  if (D < 1 || F < 1 || r < 1) return fail(SFFN_ERR_SHAPE, "decode_noalloc: D=%d, F=%d, r=%d", D, F, r);
  const size_t need = sffn_workspace_size(1, D, F, r);
  if (need > NOALLOC_BYTES)
    return fail(SFFN_ERR_WORKSPACE,
                "decode_noalloc: D=%d, F=%d, r=%d need %zu bytes of scratch, beyond its fixed %zu; use sffn_decode "
                "with a workspace", D, F, r, need, NOALLOC_BYTES);
  void* ws = nullptr;
  const hipError_t e = scratch_addr(&ws);
  if (e != hipSuccess) return hip_fail(e, "decode_noalloc: scratch address");
  return sffn_decode(act, P1, P2, c, t, n_hot, W_gate, b_gate, W_up, b_up, W_downT, x, x_norm, D, F, r, mask, active,
                     n_active, y, logits, ws, NOALLOC_BYTES, stream);
}

int sffn_forward(int act, const void* W_gate, const float* b_gate, const void* W_up, const float* b_up,
                 const void* W_downT, const float* x, int x_norm, int B, int D, int F, const uint64_t* mask,
                 int32_t* active, int32_t* n_active, float* y, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (act != SFFN_ACT_RELU && act != SFFN_ACT_REGLU && act != SFFN_ACT_SQRELU)
    return fail(SFFN_ERR_ACT, "unknown activation %d", act);
  if (act == SFFN_ACT_REGLU && !W_gate) return fail(SFFN_ERR_ACT, "ReGLU needs W_gate");
  if (!W_up || !W_downT || !x || !mask || !active || !n_active || !y)
    return fail(SFFN_ERR_NULL, "forward: W_up, W_downT, x, mask, active, n_active and y are required");
  int s = check_common(B, D, F);
  if (s) return s;
  s = check_union(B, D, F);
  if (s) return s;
  if ((act == SFFN_ACT_REGLU && !al(W_gate, 16)) || !al(W_up, 16) || !al(W_downT, 16) || !al(x, 16) ||
      !al(mask, 8) || !al(active, 4) || !al(n_active, 4) || !al(y, 16) || (b_gate && !al(b_gate, 4)) ||
      (b_up && !al(b_up, 4)))
    return fail(SFFN_ERR_ALIGN, "forward: misaligned pointer");
  s = check_ws(ws, ws_bytes, ws_forward_bytes(B, D, F));
  if (s) return s;
  const bool g = act == SFFN_ACT_REGLU;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (sffn_fused_ok(B, D, F, act, false)) {
    e = sffn_launch_fused(act, g ? W_gate : nullptr, g ? b_gate : nullptr, W_up, g ? nullptr : b_up, W_downT, x,
                          x_norm, D, F, mask, active, n_active, ws_part(ws, B, D, F), G_FUSED, y, st);
  } else if (decode_batch(B, D, F)) {
    e = sffn_launch_forward(act, g ? W_gate : nullptr, g ? b_gate : nullptr, W_up, g ? nullptr : b_up, W_downT, x,
                            x_norm, B, D, F, mask, active, n_active, y, ws_abuf(ws), st);
  } else {
    e = run_union(act, false, g ? W_gate : nullptr, nullptr, g ? b_gate : nullptr, W_up, nullptr, g ? nullptr : b_up,
                  W_downT, nullptr, x, x_norm, B, D, F, mask, active, n_active, y, ws, st);
  }
  return e == hipSuccess ? SFFN_OK : hip_fail(e, "forward launch");
}

int sffn_forward_q4(int act, sffn_q4 W_gate, const float* b_gate, sffn_q4 W_up, const float* b_up, sffn_q4 W_downT,
                    const float* x, int x_norm, int B, int D, int F, const uint64_t* mask, int32_t* active,
                    int32_t* n_active, float* y, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (act != SFFN_ACT_RELU && act != SFFN_ACT_REGLU && act != SFFN_ACT_SQRELU)
    return fail(SFFN_ERR_ACT, "unknown activation %d", act);
  if (act == SFFN_ACT_REGLU && (!W_gate.q || !W_gate.s)) return fail(SFFN_ERR_ACT, "ReGLU needs W_gate");
  if (!W_up.q || !W_up.s || !W_downT.q || !W_downT.s || !x || !mask || !active || !n_active || !y)
    return fail(SFFN_ERR_NULL, "forward_q4: W_up, W_downT, x, mask, active, n_active and y are required");
  int s = check_common(B, D, F);
  if (s) return s;
  if (D % 32) return fail(SFFN_ERR_SHAPE, "forward_q4: D=%d not a multiple of 32", D);
  s = check_union(B, D, F);
  if (s) return s;
  if ((act == SFFN_ACT_REGLU && (!al(W_gate.q, 16) || !al(W_gate.s, 2))) || !al(W_up.q, 16) || !al(W_up.s, 2) ||
      !al(W_downT.q, 16) || !al(W_downT.s, 2) || !al(x, 16) || !al(mask, 8) || !al(active, 4) ||
      !al(n_active, 4) || !al(y, 16) || (b_gate && !al(b_gate, 4)) || (b_up && !al(b_up, 4)))
    return fail(SFFN_ERR_ALIGN, "forward_q4: misaligned pointer");
  s = check_ws(ws, ws_bytes, ws_forward_bytes(B, D, F));
  if (s) return s;
  const bool g = act == SFFN_ACT_REGLU;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (sffn_fused_ok(B, D, F, act, true)) {
    e = sffn_launch_fused_q4(act, g ? W_gate.q : nullptr, g ? W_gate.s : nullptr, g ? b_gate : nullptr, W_up.q, W_up.s,
                             g ? nullptr : b_up, W_downT.q, W_downT.s, x, x_norm, D, F, mask, active, n_active,
                             ws_part(ws, B, D, F), G_FUSED, y, st);
  } else if (decode_batch(B, D, F)) {
    e = sffn_launch_forward_q4(act, g ? W_gate.q : nullptr, g ? W_gate.s : nullptr, g ? b_gate : nullptr, W_up.q,
                               W_up.s, g ? nullptr : b_up, W_downT.q, W_downT.s, x, x_norm, B, D, F, mask, active,
                               n_active, y, ws_abuf(ws), st);
  } else {
    e = run_union(act, true, g ? W_gate.q : nullptr, g ? W_gate.s : nullptr, g ? b_gate : nullptr, W_up.q, W_up.s,
                  g ? nullptr : b_up, W_downT.q, W_downT.s, x, x_norm, B, D, F, mask, active, n_active, y, ws, st);
  }
  return e == hipSuccess ? SFFN_OK : hip_fail(e, "forward_q4 launch");
}

}  // extern "C"
