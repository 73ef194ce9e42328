// Host side of libpi.so: context and scratch, argument checks, kernel selection, stack
// runner with HIP graphs. See include/pi.h for the contract of every entry point.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pi.h"
#include "pi_mfma.hpp"

using namespace pi;

struct pi_ctx {
  int device = 0;
  hipStream_t stream = nullptr;
  int max_batch = 0, max_d = 0, max_ffn = 0, max_rank = 0;
  int cus = 256;
  size_t lds_max = 65536;
  uint8_t* ws = nullptr;
  size_t ws_bytes = 0;
  float* z = nullptr;           // [max_batch][max_rank]
  uint64_t* mtok = nullptr;     // [max_batch][max_ffn/64]
  uint64_t* munion = nullptr;   // [max_ffn/64]
  int32_t* idx = nullptr;       // [max_ffn]
  int32_t* nbuf = nullptr;      // [16]
  float* a = nullptr;           // [max_ffn][NB] on the vector path (NB = batch class 1/2/4/8), by neuron id
  float* hp = nullptr;          // slice partials of the column-sliced up GEMV
  int mask_mode = PI_MASK_UNION; // masking of batches (pi_ctx_set_mask_mode)
  int down_g = 8;               // partial sums the last enqueued down projection left in part
  size_t hp_cap = 0;            // floats in hp
  float* part = nullptr;        // [32][max_batch][max_d] down-projection partial sums (groups or K splits)
  float* y = nullptr;           // [max_batch][max_d]
  float* ssq = nullptr;         // [GLUE_SLICES_MAX][2]: k_glue_sum's slice sums of squares
  uint8_t* xbuf[2] = {nullptr, nullptr};  // [max_batch][max_d] fp32-sized
  uint8_t* xstage = nullptr;    // [max_batch][max_d] fp32-sized
  int32_t* nlog = nullptr;      // [NLOG_CAP]
  // batched (matrix-core) path
  float* zpart = nullptr;       // [MM_KS1][max_batch][max_rank]
  half_t* zhi = nullptr;        // [max_batch][max_rank]
  half_t* zlo = nullptr;
  half_t* a16 = nullptr;        // [32 or 64][lda] activations at compacted positions
  int lda = 0;
  std::string err;
  // cached graph of one stack step, captured on a private stream (the caller's stream may be
  // the null stream, which cannot be captured) and launched on the caller's stream
  hipStream_t cap_stream = nullptr;
  hipGraphExec_t gexec = nullptr;
  std::vector<uint64_t> g_layers;  // serial numbers of the captured step's layers
  int g_B = 0;
  // per-kernel event timing (pi_stack_profile only)
  bool profiling = false;
  std::vector<hipEvent_t> ev;     // pairs: ev[2i] before, ev[2i+1] after launch i
  std::vector<int> ev_class;
  size_t ev_used = 0;
};

struct pi_ffn {
  pi_ffn_desc desc;
  pi_ctx* ctx;
  uint64_t serial;  // unique per pi_ffn_create in this process: the key of a captured stack step
};

static std::atomic<uint64_t> g_ffn_serial{1};

namespace {

constexpr int NLOG_CAP = 4096;

pi_status fail(pi_ctx* ctx, pi_status s, const char* fmt, ...) {
  if (ctx != nullptr) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->err = buf;
  }
  return s;
}

#define PI_HIP(ctx, call)                                                                        \
  do {                                                                                           \
    hipError_t e_ = (call);                                                                      \
    if (e_ != hipSuccess) return fail((ctx), PI_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The next free pair of profiling events, tagged with a kernel class.
void prof_slot(pi_ctx* c, int klass, hipEvent_t* e0, hipEvent_t* e1) {
  if (c->ev_used * 2 + 2 > c->ev.size()) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return;
    }
    c->ev.push_back(a);
    c->ev.push_back(b);
    c->ev_class.push_back(klass);
  }
  const size_t slot = c->ev_used++;
  c->ev_class[slot] = klass;
  *e0 = c->ev[2 * slot];
  *e1 = c->ev[2 * slot + 1];
}

// One kernel launch (`block` threads per workgroup; BLOCK for launch_k) on the context's stream. When profiling,
// the dispatch itself carries a pair of events (hipExtLaunchKernelGGL), so the pair times the
// kernel's execution, not the queueing around it.
template <typename... P, typename... A>
hipError_t launch_kb(pi_ctx* c, int klass, void (*kern)(P...), dim3 grid, int block, size_t lds, A... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (c->profiling) prof_slot(c, klass, &e0, &e1);
  if (e0 != nullptr)
    hipExtLaunchKernelGGL(kern, grid, dim3(block), (uint32_t)lds, c->stream, e0, e1, 0u, static_cast<P>(args)...);
  else
    hipLaunchKernelGGL(kern, grid, dim3(block), lds, c->stream, static_cast<P>(args)...);
  return hipGetLastError();
}
template <typename... P, typename... A>
hipError_t launch_k(pi_ctx* c, int klass, void (*kern)(P...), dim3 grid, size_t lds, A... args) {
  return launch_kb(c, klass, kern, grid, BLOCK, lds, args...);
}
enum { K_STAGE1 = 0, K_STAGE2, K_TRUEMASK, K_UP, K_DOWN, K_REDUCE, K_COUNT };
static_assert(K_COUNT == PI_KERNEL_CLASSES, "kernel classes out of sync with pi.h");
static_assert(PI_ACT_RELU == ACT_RELU && PI_ACT_REGLU == ACT_REGLU && PI_ACT_SQRELU == ACT_SQRELU,
              "activation codes out of sync with pi.h");

LayerDev to_dev(const pi_ffn_desc& d) {
  LayerDev L;
  L.d = d.d;
  L.ffn = d.ffn;
  L.rank = d.rank;
  L.hot_prefix = d.hot_prefix;
  L.act = d.act;
  L.wtype = d.wtype;
  L.threshold = d.threshold;
  L.w_up = static_cast<const uint8_t*>(d.w_up);
  L.w_gate = static_cast<const uint8_t*>(d.w_gate);
  L.w_down_t = static_cast<const uint8_t*>(d.w_down_t);
  L.s_up = d.s_up;
  L.s_gate = d.s_gate;
  L.s_down = d.s_down;
  L.b = d.b;
  L.p_w1 = d.p_w1;
  L.p_w2 = d.p_w2;
  L.p_b = d.p_b;
  return L;
}

constexpr int nb_for(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }
size_t x_elem(int wtype) { return wtype == PI_W_F32 ? 4 : 2; }

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// ---------------------------------------------------------------- kernel dispatch tables

constexpr size_t X_LDS_BUDGET = 65536;  // LDS for staged x that still leaves room for 2 workgroups per CU

// Width of the x column windows for NB tokens of `xe`-byte elements: d when x fits in the LDS
// budget, else the largest multiple of 512 columns that does. 4 KB of the workgroup's LDS
// stay free for the kernels' own shared arrays.
int x_window(const pi_ctx* c, int NB, int d, size_t xe, size_t budget) {
  const size_t cap = std::min(budget, c->lds_max - 4096);
  if ((size_t)NB * d * xe <= cap) return d;
  return std::max(512, (int)(cap / (NB * xe)) / 512 * 512);
}

template <int NB>
pi_status launch_stage1_nb(pi_ctx* c, const LayerDev& L, const XIn& xin, int B) {
  const int dc = x_window(c, NB, L.d, 2, X_LDS_BUDGET);
  const size_t lds = (size_t)NB * dc * 2;
  PI_HIP(c, allow_lds(k_stage1<NB>, lds));
  const int grid = (L.rank + NWAVES - 1) / NWAVES;
  PI_HIP(c, launch_k(c, K_STAGE1, k_stage1<NB>, dim3(grid), lds, L, xin, B, dc, c->z));
  return PI_OK;
}

// Stage 1 of 2..8 tokens of given x (d <= 512 PF): two waves per W1 row, each with its whole
// share in flight from entry. Measured on MI355X against k_stage1 (one wave per row, W1 in
// windows): OPT-6.7B at 4 tokens 7.6 -> 5.6 us, Llama-2-70B at 8 tokens 13.7 -> 10.6 us,
// OPT-175B at 8 tokens 19.3 -> 14.5 us; one wave per row with the whole row in flight left
// OPT-175B at 19.5 us, and four waves per row were no better than two.
template <int NB, int PF>
pi_status launch_stage1_x_t(pi_ctx* c, const LayerDev& L, const void* x, int B) {
  const int dc = x_window(c, NB, L.d, 2, X_LDS_BUDGET);
  const size_t lds = (size_t)NB * dc * 2;
  constexpr int KS = 2;
  auto kern = k_stage1_x<NB, PF, KS>;
  PI_HIP(c, allow_lds(kern, lds));
  const int grid = (L.rank + NWAVES - 1) / NWAVES;
  PI_HIP(c, launch_kb(c, K_STAGE1, kern, dim3(grid), BLOCK * KS, lds, L, static_cast<const half_t*>(x), B, dc,
                      c->z));
  return PI_OK;
}
template <int NB>
pi_status launch_stage1_x(pi_ctx* c, const LayerDev& L, const void* x, int B) {
  if (L.d <= 512 * 8) return launch_stage1_x_t<NB, 8>(c, L, x, B);
  if (L.d <= 512 * 16) return launch_stage1_x_t<NB, 16>(c, L, x, B);
  if (L.d <= 512 * 24) return launch_stage1_x_t<NB, 24>(c, L, x, B);
  return launch_stage1_x_t<NB, 32>(c, L, x, B);
}

// Stage 1 at one token that finishes the glue started by k_glue_sum (xin.ssq != nullptr), two
// waves per W1 row (OPT-175B 8.4 -> 7.7 us per layer against one, Falcon-40B 6.2 -> 5.7,
// Llama-2-70B 6.2 -> 5.4 on MI355X). The first 2/3 of each wave's share goes out at entry,
// behind u's loads; the rest once x is formed. Measured with one wave per row at the OPT-175B
// shape (d = 12288, 24 chunks per lane): 9.0 us with the
// whole row issued at entry, 9.6 with none, 8.7 with 8 chunks, 8.2 with 16.
template <int PF>
pi_status launch_stage1_g1_t(pi_ctx* c, const LayerDev& L, const XIn& xin) {
  const size_t lds = (size_t)L.d * 2;
  constexpr int KS = 2;
  auto kern = k_stage1_g1<PF, PF * 2 / 3, KS>;
  PI_HIP(c, allow_lds(kern, lds));
  const int grid = (L.rank + NWAVES - 1) / NWAVES;
  PI_HIP(c, launch_kb(c, K_STAGE1, kern, dim3(grid), BLOCK * KS, lds, L, xin.y, xin.ssq, xin.nsl,
                      static_cast<const half_t*>(xin.x), static_cast<half_t*>(xin.x_out), c->z));
  return PI_OK;
}

// The two-step glue applies to one token of fp16 x with d <= 4 * BLOCK * GLUE_SLICES_MAX.
bool glue_split_ok(int d, size_t xe) { return xe == 2 && d % 8 == 0 && d <= 4 * BLOCK * GLUE_SLICES_MAX; }

// k_glue_sum over the previous layer's partial sums (one token): u into c->y, the slices'
// sums of squares into c->ssq; returns the slice count through nsl.
pi_status launch_glue_sum(pi_ctx* c, int d, const float* center, int* nsl) {
  *nsl = (d / 4 + BLOCK - 1) / BLOCK;
  const dim3 grid(*nsl);
  switch (c->down_g) {
    case 8: PI_HIP(c, launch_k(c, K_REDUCE, k_glue_sum<8>, grid, 0, c->part, d, center, d, c->y, c->ssq)); break;
    case 16: PI_HIP(c, launch_k(c, K_REDUCE, k_glue_sum<16>, grid, 0, c->part, d, center, d, c->y, c->ssq)); break;
    default: return fail(c, PI_ERR_UNSUPPORTED, "glue over %d partial sums", c->down_g);
  }
  return PI_OK;
}

// k_glue_parts over the previous layer's partial sums (2..8 tokens); glue_parts_ok says
// where it applies (elsewhere k_reduce adds the partials and k_glue follows).
template <int G, bool XF32>
pi_status launch_glue_parts_g(pi_ctx* c, int B, int d, const float* center, const void* x_prev, void* x_out) {
  const int J = (d / 4 + GLUE_NTH - 1) / GLUE_NTH;
  const float* part = c->part;
  const int gs = B * d;
  switch (J) {
    case 1: PI_HIP(c, launch_kb(c, K_REDUCE, k_glue_parts<G, 1, XF32>, dim3(B), GLUE_NTH, 0, part, gs, center, x_prev, d, x_out)); break;
    case 2: PI_HIP(c, launch_kb(c, K_REDUCE, k_glue_parts<G, 2, XF32>, dim3(B), GLUE_NTH, 0, part, gs, center, x_prev, d, x_out)); break;
    case 3: PI_HIP(c, launch_kb(c, K_REDUCE, k_glue_parts<G, 3, XF32>, dim3(B), GLUE_NTH, 0, part, gs, center, x_prev, d, x_out)); break;
    default: PI_HIP(c, launch_kb(c, K_REDUCE, k_glue_parts<G, 4, XF32>, dim3(B), GLUE_NTH, 0, part, gs, center, x_prev, d, x_out));
  }
  return PI_OK;
}
bool glue_parts_ok(const pi_ctx* c, int d) {
  return d % 4 == 0 && d <= 4 * GLUE_NTH * 4 && (c->down_g == 8 || c->down_g == 16);
}
template <bool XF32>
pi_status launch_glue_parts(pi_ctx* c, int B, int d, const float* center, const void* x_prev, void* x_out) {
  switch (c->down_g) {
    case 8: return launch_glue_parts_g<8, XF32>(c, B, d, center, x_prev, x_out);
    default: return launch_glue_parts_g<16, XF32>(c, B, d, center, x_prev, x_out);
  }
}

pi_status launch_stage1(pi_ctx* c, const LayerDev& L, const XIn& xin, int B) {
  if (xin.ssq != nullptr) {
    if (B != 1 || !glue_split_ok(L.d, 2)) return fail(c, PI_ERR_INVALID, "split glue needs one token and d <= 16384");
    if (L.d <= 512 * 8) return launch_stage1_g1_t<8>(c, L, xin);
    if (L.d <= 512 * 16) return launch_stage1_g1_t<16>(c, L, xin);
    if (L.d <= 512 * 24) return launch_stage1_g1_t<24>(c, L, xin);
    return launch_stage1_g1_t<32>(c, L, xin);
  }
  if (xin.y == nullptr && B >= 2 && L.d <= 512 * 32 && L.d % 8 == 0) {
    switch (nb_for(B)) {
      case 2: return launch_stage1_x<2>(c, L, xin.x, B);
      case 4: return launch_stage1_x<4>(c, L, xin.x, B);
      default: return launch_stage1_x<8>(c, L, xin.x, B);
    }
  }
  switch (nb_for(B)) {
    case 1: return launch_stage1_nb<1>(c, L, xin, B);
    case 2: return launch_stage1_nb<2>(c, L, xin, B);
    case 4: return launch_stage1_nb<4>(c, L, xin, B);
    default: return launch_stage1_nb<8>(c, L, xin, B);
  }
}

// Stage 2 of the predictor; with `up`, also the activations of each workgroup's own active
// neurons (x read from `x`, a dense [B][ffn]).
constexpr int STAGE2_TILE = 32;  // neurons per workgroup in predictor stage 2

template <int NB, int CPL, bool UP, int WT, int ACT>
pi_status launch_stage2_t(pi_ctx* c, const LayerDev& L, int B, uint64_t* mtok, float* logits, const void* x) {
  const size_t xe = (WT == W_F32) ? 4 : 2;
  const int xw = UP ? x_window(c, NB, L.d, xe, c->lds_max) : L.d;
  // z in LDS at 8 tokens without the activations ([NB][rank] fp16 hi and lo)
  const size_t lds = UP ? (size_t)NB * xw * xe : (NB >= 8 ? (size_t)NB * L.rank * 4 : 0);
  auto kern = k_stage2<NB, CPL, UP, WT, ACT>;
  PI_HIP(c, allow_lds(kern, lds));
  PI_HIP(c, launch_k(c, K_STAGE2, kern, dim3(L.ffn / STAGE2_TILE), lds, L, c->z, B, mtok, c->munion, logits, x, xw,
                     c->a));
  return PI_OK;
}

template <int NB, int CPL>
pi_status launch_stage2_c(pi_ctx* c, const LayerDev& L, int B, uint64_t* mtok, float* logits, const void* x) {
  if (x == nullptr) return launch_stage2_t<NB, CPL, false, W_F16, ACT_RELU>(c, L, B, mtok, logits, x);
  if (L.wtype != W_F16 && L.wtype != W_Q4) return fail(c, PI_ERR_UNSUPPORTED, "no predictor path for this weight type");
  if (L.wtype == W_F16) {
    switch (L.act) {
      case ACT_RELU: return launch_stage2_t<NB, CPL, true, W_F16, ACT_RELU>(c, L, B, mtok, logits, x);
      case ACT_REGLU: return launch_stage2_t<NB, CPL, true, W_F16, ACT_REGLU>(c, L, B, mtok, logits, x);
      default: return launch_stage2_t<NB, CPL, true, W_F16, ACT_SQRELU>(c, L, B, mtok, logits, x);
    }
  }
  switch (L.act) {
    case ACT_RELU: return launch_stage2_t<NB, CPL, true, W_Q4, ACT_RELU>(c, L, B, mtok, logits, x);
    case ACT_REGLU: return launch_stage2_t<NB, CPL, true, W_Q4, ACT_REGLU>(c, L, B, mtok, logits, x);
    default: return launch_stage2_t<NB, CPL, true, W_Q4, ACT_SQRELU>(c, L, B, mtok, logits, x);
  }
}

template <int NB>
pi_status launch_stage2_nb(pi_ctx* c, const LayerDev& L, int B, uint64_t* mtok, float* logits, const void* x) {
  if (L.rank <= 512) return launch_stage2_c<NB, 1>(c, L, B, mtok, logits, x);
  return launch_stage2_c<NB, 2>(c, L, B, mtok, logits, x);
}

pi_status launch_stage2(pi_ctx* c, const LayerDev& L, int B, uint64_t* mtok, float* logits, const void* x) {
  switch (nb_for(B)) {
    case 1: return launch_stage2_nb<1>(c, L, B, mtok, logits, x);
    case 2: return launch_stage2_nb<2>(c, L, B, mtok, logits, x);
    case 4: return launch_stage2_nb<4>(c, L, B, mtok, logits, x);
    default: return launch_stage2_nb<8>(c, L, B, mtok, logits, x);
  }
}

template <int WT, int NB, bool UP>
pi_status launch_truemask_t(pi_ctx* c, const LayerDev& L, const XIn& xin, int B, uint64_t* mtok, float* logits) {
  constexpr bool XF32 = WT == W_F32;
  const size_t lds = (size_t)NB * L.d * (XF32 ? 4 : 2);
  if (lds + 4096 > c->lds_max) return fail(c, PI_ERR_UNSUPPORTED, "batch %d x d %d does not fit in LDS", B, L.d);
  if (xin.y != nullptr && (L.d > 4 * BLOCK * GLUE_J || xin.ny > GLUE_NY))
    return fail(c, PI_ERR_UNSUPPORTED, "chained layers without a predictor need d <= %d", 4 * BLOCK * GLUE_J);
  auto kern = k_truemask<WT, NB, XF32, UP>;
  PI_HIP(c, allow_lds(kern, lds));
  PI_HIP(c, launch_k(c, K_TRUEMASK, kern, dim3(L.ffn / 64), lds, L, xin, B, mtok, c->munion, logits, c->a));
  return PI_OK;
}

template <int WT, bool UP>
pi_status launch_truemask_w(pi_ctx* c, const LayerDev& L, const XIn& xin, int B, uint64_t* mtok, float* logits) {
  switch (nb_for(B)) {
    case 1: return launch_truemask_t<WT, 1, UP>(c, L, xin, B, mtok, logits);
    case 2: return launch_truemask_t<WT, 2, UP>(c, L, xin, B, mtok, logits);
    case 4: return launch_truemask_t<WT, 4, UP>(c, L, xin, B, mtok, logits);
    default: return launch_truemask_t<WT, 8, UP>(c, L, xin, B, mtok, logits);
  }
}

pi_status launch_truemask(pi_ctx* c, const LayerDev& L, const XIn& xin, int B, uint64_t* mtok, float* logits,
                          bool up) {
  switch (L.wtype) {
    case W_F32: return up ? launch_truemask_w<W_F32, true>(c, L, xin, B, mtok, logits)
                          : launch_truemask_w<W_F32, false>(c, L, xin, B, mtok, logits);
    case W_F16: return up ? launch_truemask_w<W_F16, true>(c, L, xin, B, mtok, logits)
                          : launch_truemask_w<W_F16, false>(c, L, xin, B, mtok, logits);
    default: return up ? launch_truemask_w<W_Q4, true>(c, L, xin, B, mtok, logits)
                       : launch_truemask_w<W_Q4, false>(c, L, xin, B, mtok, logits);
  }
}

template <int WT, int ACT, int NB>
pi_status launch_up_t(pi_ctx* c, const LayerDev& L, const void* x, int B, const int32_t* idx_in, const int32_t* n_in) {
  const size_t xe = (WT == W_F32) ? 4 : 2;
  const int xw = x_window(c, NB, L.d, xe, c->lds_max);
  const size_t lds = (size_t)NB * xw * xe;
  auto kern = k_up<WT, ACT, NB>;
  PI_HIP(c, allow_lds(kern, lds));
  constexpr int CH = NWAVES * ActPW<ACT>::PW;
  const int grid = std::max(1, std::min((L.ffn + CH - 1) / CH, 8 * c->cus));
  PI_HIP(c, launch_k(c, K_UP, kern, dim3(grid), lds, L, x, B, xw, idx_in, n_in, c->a));
  return PI_OK;
}

template <int WT, int ACT>
pi_status launch_up_a(pi_ctx* c, const LayerDev& L, const void* x, int B, const int32_t* idx_in, const int32_t* n_in) {
  switch (nb_for(B)) {
    case 1: return launch_up_t<WT, ACT, 1>(c, L, x, B, idx_in, n_in);
    case 2: return launch_up_t<WT, ACT, 2>(c, L, x, B, idx_in, n_in);
    case 4: return launch_up_t<WT, ACT, 4>(c, L, x, B, idx_in, n_in);
    default: return launch_up_t<WT, ACT, 8>(c, L, x, B, idx_in, n_in);
  }
}

template <int ACT>
pi_status launch_up_w(pi_ctx* c, const LayerDev& L, const void* x, int B, const int32_t* idx_in, const int32_t* n_in) {
  switch (L.wtype) {
    case W_F32: return launch_up_a<W_F32, ACT>(c, L, x, B, idx_in, n_in);
    case W_F16: return launch_up_a<W_F16, ACT>(c, L, x, B, idx_in, n_in);
    default: return launch_up_a<W_Q4, ACT>(c, L, x, B, idx_in, n_in);
  }
}

pi_status launch_up(pi_ctx* c, const LayerDev& L, const void* x, int B, const int32_t* idx_in, const int32_t* n_in) {
  switch (L.act) {
    case ACT_RELU: return launch_up_w<ACT_RELU>(c, L, x, B, idx_in, n_in);
    case ACT_REGLU: return launch_up_w<ACT_REGLU>(c, L, x, B, idx_in, n_in);
    default: return launch_up_w<ACT_SQRELU>(c, L, x, B, idx_in, n_in);
  }
}

// Separate up GEMV over column slices of x (k_up_cols, + k_act_fin for several slices)
// instead of stage 2's fused activations. Always when x of the batch is larger than
// X_LDS_BUDGET: the fused kernels would stage all of x in every workgroup, one workgroup per
// CU. Also where the fused activations make stage 2's tail long: Q4_0 rows (dequantisation),
// rows of 8192 or more columns, and 5..8 tokens. Measured on MI355X against the fused path
// (tokens/s of the layer stacks): OPT-175B Q4_0 +10% at 1 token and +12% at 2; Falcon-40B
// 0/+2/+4% at 1/2/4 tokens; Llama-2-70B +1/+2/+2%; OPT-6.7B (d = 4096) -10/-8/-5% at 1/2/4
// tokens and +19% at 8. Slices are sw columns wide, a multiple of 512 whose x fits the budget.
constexpr int UPC_WGS_PER_CU = 2;
constexpr bool up_cols(int NB, int d, size_t xe) { return (size_t)NB * d * xe > X_LDS_BUDGET; }
constexpr int up_cols_width(int NB, size_t xe) { return (int)(X_LDS_BUDGET / (NB * xe)) / 512 * 512; }
size_t x_elem(const LayerDev& L) { return L.wtype == W_F32 ? 4 : 2; }
bool use_up_cols(const LayerDev& L, int B) {
  const int NB = nb_for(B);
  return B <= 8 && (up_cols(NB, L.d, x_elem(L)) || L.wtype == W_Q4 || L.d >= 8192 || NB >= 8);
}

// Floats of hp for a context's limits: the largest slices x 2 rows x tokens x ffn over the
// batch classes and element sizes that take the column-sliced path.
constexpr size_t up_cols_floats(int max_batch, int max_d, int max_ffn) {
  size_t m = 0;
  const int nb_max = nb_for(max_batch < 8 ? max_batch : 8);
  for (int NB = 1; NB <= nb_max; NB *= 2)
    for (size_t xe = 2; xe <= 4; xe += 2)
      if (up_cols(NB, max_d, xe)) {
        const int sw = up_cols_width(NB, xe);
        const size_t f = (size_t)((max_d + sw - 1) / sw) * 2 * NB * max_ffn;
        m = f > m ? f : m;
      }
  return m;
}

template <int WT, int ACT, int NB>
pi_status launch_up_cols_t(pi_ctx* c, const LayerDev& L, const void* x, int B, const uint64_t* words,
                           const int32_t* idx_in, const int32_t* n_in) {
  typedef typename XType<WT == W_F32>::T XT;
  // one slice when x fits: then only d (rounded up to 512) columns of LDS
  const int sw = std::min(up_cols_width(NB, sizeof(XT)), (L.d + 511) / 512 * 512);
  const int S = (L.d + sw - 1) / sw;
  constexpr int NR = (ACT == ACT_REGLU) ? 2 : 1;
  if (S > 1 && (size_t)S * NR * B * L.ffn > c->hp_cap)
    return fail(c, PI_ERR_UNSUPPORTED, "layer %dx%d exceeds the context's slice buffer", L.d, L.ffn);
  const int W = L.ffn / 64;
  const size_t lds = (size_t)NB * sw * sizeof(XT) + UPC_PMAX * 4 + (words ? (size_t)W * 8 + (size_t)(W + 1) * 4 : 0);
  if (lds + 256 > c->lds_max) return fail(c, PI_ERR_UNSUPPORTED, "ffn %d too large for the sliced up GEMV", L.ffn);
  auto kern = k_up_cols<WT, ACT, NB>;
  PI_HIP(c, allow_lds(kern, lds));
  // one round of workgroups: at most UPC_WGS_PER_CU per CU (their LDS allows no more)
  const int chunks = std::max((L.ffn + UPC_PMAX - 1) / UPC_PMAX, std::max(1, UPC_WGS_PER_CU * c->cus / S));
  PI_HIP(c, launch_k(c, K_UP, kern, dim3(S, chunks), lds, L, x, B, sw, words, idx_in, n_in, c->hp, c->a));
  if (S > 1)
    PI_HIP(c, launch_k(c, K_REDUCE, k_act_fin<ACT>, dim3((L.ffn + BLOCK - 1) / BLOCK), 0, L, B, S,
                       (const float*)c->hp, words, idx_in, n_in, c->a));
  return PI_OK;
}

template <int WT, int ACT>
pi_status launch_up_cols_a(pi_ctx* c, const LayerDev& L, const void* x, int B, const uint64_t* words,
                           const int32_t* idx_in, const int32_t* n_in) {
  switch (nb_for(B)) {
    case 1: return launch_up_cols_t<WT, ACT, 1>(c, L, x, B, words, idx_in, n_in);
    case 2: return launch_up_cols_t<WT, ACT, 2>(c, L, x, B, words, idx_in, n_in);
    case 4: return launch_up_cols_t<WT, ACT, 4>(c, L, x, B, words, idx_in, n_in);
    default: return launch_up_cols_t<WT, ACT, 8>(c, L, x, B, words, idx_in, n_in);
  }
}

template <int ACT>
pi_status launch_up_cols_w(pi_ctx* c, const LayerDev& L, const void* x, int B, const uint64_t* words,
                           const int32_t* idx_in, const int32_t* n_in) {
  switch (L.wtype) {
    case W_F32: return launch_up_cols_a<W_F32, ACT>(c, L, x, B, words, idx_in, n_in);
    case W_F16: return launch_up_cols_a<W_F16, ACT>(c, L, x, B, words, idx_in, n_in);
    default: return launch_up_cols_a<W_Q4, ACT>(c, L, x, B, words, idx_in, n_in);
  }
}

// The gathered up GEMV on Q4_0 rows at 1..8 tokens (k_upq): the slice of x (NB x 4 KB per
// block per lane) stays within 128 KB of LDS, so one workgroup per CU; blocks per lane rounded
// up to an instantiated count (extra blocks are masked); two neurons per wave and round. The
// grid is one round of resident workgroups, at least one per 64 units of 16 bits. Measured on
// MI355X at the OPT-175B shape and one token (before the swizzled x): 14.5 us per layer against
// 18.3 us for k_up_cols; 33 us with 3 neurons per wave and round (registers spill); with
// 256-thread workgroups (3 per CU) 17.8 us, the third workgroup on a CU staging x behind the
// others' row loads. fp16 rows stay on k_up_cols (Falcon-40B 17.0 against 19.2 us,
// Llama-2-70B 27.4 against 29.0 us with a 256-thread version of this kernel).
constexpr size_t UPQ_X_BUDGET = 128 * 1024;

template <int ACT, int NB, int SB>
pi_status launch_upq_t(pi_ctx* c, const LayerDev& L, const void* x, int B, int S, const uint64_t* words,
                       const int32_t* idx_in, const int32_t* n_in) {
  constexpr int NR = (ACT == ACT_REGLU) ? 2 : 1;
  if (S > 1 && (size_t)S * NR * B * L.ffn > c->hp_cap)
    return fail(c, PI_ERR_UNSUPPORTED, "layer %dx%d exceeds the context's slice buffer", L.d, L.ffn);
  // 16 waves, two neurons per wave and round. Measured on MI355X at the OPT-175B shape and 8
  // tokens: 86.6 us per layer; 12 waves with the next round's rows loading during this one's
  // arithmetic 88.5 us; 8 waves with 4 neurons per round (half the LDS reads of x), pipelined,
  // 102 us. The kernel is VALU- and LDS-bound there: about 180 VALU instructions per block and
  // row (16 dot2 per token), 57% VALU-busy.
  constexpr int NTH = 1024;
  const size_t lds = (size_t)NB * 4 * WAVE * SB * 16 + (size_t)NTH * 4 + (size_t)(L.ffn / 64) * 8;
  auto kern = k_upq<ACT, NB, SB, 2, NTH>;
  PI_HIP(c, allow_lds(kern, lds));
  int per_cu = 0;
  PI_HIP(c, hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, NTH, lds));
  const int resident = std::max(1, per_cu) * c->cus;
  // chunks of the neuron list: at most NTH candidates each, at least one workgroup per CU
  const int W = L.ffn / 64;
  int nc, upw = 0;
  if (words != nullptr && NB <= 2) {
    nc = std::min(4 * W, std::max((4 * W + NTH / 16 - 1) / (NTH / 16), std::max(1, resident / S)));
    upw = (4 * W + nc - 1) / nc;
  } else {
    nc = std::max((L.ffn + NTH - 1) / NTH, std::max(1, resident / S));
  }
  PI_HIP(c, launch_kb(c, K_UP, kern, dim3(S, nc), NTH, lds, L, static_cast<const half_t*>(x), B, words, upw,
                      idx_in, n_in, c->hp, c->a));
  if (S > 1)
    PI_HIP(c, launch_k(c, K_REDUCE, k_act_fin<ACT>, dim3((L.ffn + BLOCK - 1) / BLOCK), 0, L, B, S,
                       (const float*)c->hp, words, idx_in, n_in, c->a));
  return PI_OK;
}

// Slices and blocks per lane of k_upq for NB tokens; false where it does not apply.
bool upq_geometry(const pi_ctx* c, const LayerDev& L, int NB, int* S, int* SB) {
  if (L.wtype != W_Q4) return false;
  // its buffer loads address the rows with 32-bit offsets, and an offset of BUF_OOB must lie
  // past them (larger rows take k_up_cols)
  if ((size_t)L.ffn * (L.d / 32) * 16 >= BUF_OOB) return false;
  const int nbl = (L.d / 32 + WAVE - 1) / WAVE;  // blocks per lane over the whole row
  const int sb_max = (int)(UPQ_X_BUDGET / ((size_t)NB * 4 * WAVE * 16));
  const int s = (nbl + sb_max - 1) / sb_max;
  const int sb = (nbl + s - 1) / s;
  if (sb > 6) return false;
  *S = s;
  *SB = sb <= 2 ? 2 : sb <= 3 ? 3 : 6;
  // x of the slice, the neuron list and the union words must fit the workgroup's LDS
  return (size_t)NB * 4 * WAVE * *SB * 16 <= UPQ_X_BUDGET &&
         UPQ_X_BUDGET + (size_t)UPQ_LIST * 4 + (size_t)(L.ffn / 64) * 8 <= c->lds_max;
}

template <int ACT, int NB>
pi_status launch_upq_b(pi_ctx* c, const LayerDev& L, const void* x, int B, int S, int SB, const uint64_t* words,
                       const int32_t* idx_in, const int32_t* n_in) {
  switch (SB) {
    case 2: return launch_upq_t<ACT, NB, 2>(c, L, x, B, S, words, idx_in, n_in);
    case 3: return launch_upq_t<ACT, NB, 3>(c, L, x, B, S, words, idx_in, n_in);
    default: return launch_upq_t<ACT, NB, 6>(c, L, x, B, S, words, idx_in, n_in);
  }
}

template <int ACT>
pi_status launch_upq_a(pi_ctx* c, const LayerDev& L, const void* x, int B, int S, int SB, const uint64_t* words,
                       const int32_t* idx_in, const int32_t* n_in) {
  switch (nb_for(B)) {
    case 1: return launch_upq_b<ACT, 1>(c, L, x, B, S, SB, words, idx_in, n_in);
    case 2: return launch_upq_b<ACT, 2>(c, L, x, B, S, SB, words, idx_in, n_in);
    case 4: return launch_upq_b<ACT, 4>(c, L, x, B, S, SB, words, idx_in, n_in);
    default: return launch_upq_b<ACT, 8>(c, L, x, B, S, SB, words, idx_in, n_in);
  }
}

// a of the active neurons from the union words (words != nullptr) or an index list.
pi_status launch_up_cols(pi_ctx* c, const LayerDev& L, const void* x, int B, const uint64_t* words,
                         const int32_t* idx_in, const int32_t* n_in) {
  int S = 0, SB = 0;
  if (B <= 8 && upq_geometry(c, L, nb_for(B), &S, &SB)) {
    switch (L.act) {
      case ACT_RELU: return launch_upq_a<ACT_RELU>(c, L, x, B, S, SB, words, idx_in, n_in);
      case ACT_REGLU: return launch_upq_a<ACT_REGLU>(c, L, x, B, S, SB, words, idx_in, n_in);
      default: return launch_upq_a<ACT_SQRELU>(c, L, x, B, S, SB, words, idx_in, n_in);
    }
  }
  switch (L.act) {
    case ACT_RELU: return launch_up_cols_w<ACT_RELU>(c, L, x, B, words, idx_in, n_in);
    case ACT_REGLU: return launch_up_cols_w<ACT_REGLU>(c, L, x, B, words, idx_in, n_in);
    default: return launch_up_cols_w<ACT_SQRELU>(c, L, x, B, words, idx_in, n_in);
  }
}

// Down projection over the active neurons (from the union words, SCAN, which also writes idx
// and n; or from a given index list) into G partial sums, then (y != nullptr) their sum into
// y. With y == nullptr the partials stay in c->part for the next layer's glue, and c->down_g
// says how many there are.
constexpr int DOWN_G = 8;        // partial sums (groups) at 1..2 tokens
constexpr int DOWN_G_WIDE = 16;  // at 3..8 tokens, whose union lists are longer
constexpr int down_groups(int NB) { return NB >= 4 ? DOWN_G_WIDE : DOWN_G; }
constexpr int MM_KS1 = 32;  // K splits of the batched predictor stage 1
constexpr int MM_KSD = 32;  // K splits of the batched down projection

template <int WT, int NB, bool SCAN, int G, int SQ = 0, int UO = 0>
pi_status launch_down_g(pi_ctx* c, const LayerDev& L, int B, const int32_t* idx_in, const int32_t* n_in, float* y,
                        int32_t* idx_out, int32_t* n_out, int32_t* n_log, const uint64_t* tok_mask) {
  constexpr int SQE = SQ ? SQ : 4;
  constexpr int U = UO ? UO : (WT == W_Q4) ? (NB == 1 ? 8 : 4) : (NB >= 4 ? 4 : 8);
  const int W = L.ffn / 64;
  // the group's list (+ its per-token bits), then the slots' column sums; or the compaction
  // block's words and prefix
  constexpr size_t lds_red = (size_t)(BLOCK / DownGeom<WT, SQE>::SEG) * (DownGeom<WT, SQE>::SW + 1) * 4;
  const size_t lds = std::max({(size_t)down_list_cap(W, G) * 5, lds_red,
                               SCAN ? (size_t)W * 8 + (size_t)(W + 1) * 4 : (size_t)0});
  constexpr size_t lds_static = 256;
  if (lds + lds_static > c->lds_max)
    return fail(c, PI_ERR_UNSUPPORTED, "ffn %d too large for the down projection", L.ffn);
  auto kern = k_down_part<WT, NB, SCAN, U, G, SQE>;
  PI_HIP(c, allow_lds(kern, lds));
  const int S = (L.d + DownGeom<WT, SQE>::SW - 1) / DownGeom<WT, SQE>::SW;
  // SCAN: one more block writes idx and n
  PI_HIP(c, launch_k(c, K_DOWN, kern, dim3(G * S + (SCAN ? 1 : 0)), lds, L, B, c->munion, idx_in, n_in, c->a, tok_mask,
                     c->part, idx_out, n_out, n_log));
  c->down_g = G;
  if (y != nullptr) {
    const int BD = B * L.d;
    PI_HIP(c, launch_k(c, K_REDUCE, k_reduce, dim3((BD + WAVE - 1) / WAVE), 0, c->part, G, BD, y));
  }
  return PI_OK;
}

// Q4_0 rows at 4..8 tokens: k_down_q4x, G groups, U list items per slot and round.
template <int NB, bool SCAN, int G, int U>
pi_status launch_down_q4x(pi_ctx* c, const LayerDev& L, int B, const int32_t* idx_in, const int32_t* n_in, float* y,
                          int32_t* idx_out, int32_t* n_out, int32_t* n_log, const uint64_t* tok_mask) {
  // its buffer loads address the rows with 32-bit offsets, and an offset of BUF_OOB must lie
  // past them
  if ((size_t)L.ffn * (L.d / 32) * 16 >= BUF_OOB)
    return fail(c, PI_ERR_UNSUPPORTED, "Q4_0 down rows of %d x %d exceed 2 GiB", L.ffn, L.d);
  const int W = L.ffn / 64;
  constexpr size_t lds_red = (size_t)(BLOCK / 16) * (128 + 1) * 4;
  const size_t lds = std::max({(size_t)down_list_cap(W, G) * 5, lds_red,
                               SCAN ? (size_t)W * 8 + (size_t)(W + 1) * 4 : (size_t)0});
  if (lds + 256 > c->lds_max) return fail(c, PI_ERR_UNSUPPORTED, "ffn %d too large for the down projection", L.ffn);
  auto kern = k_down_q4x<NB, SCAN, G, U>;
  PI_HIP(c, allow_lds(kern, lds));
  const int S = (L.d + 127) / 128;
  PI_HIP(c, launch_k(c, K_DOWN, kern, dim3(G * S + (SCAN ? 1 : 0)), lds, L, B, c->munion, idx_in, n_in, c->a, tok_mask,
                     c->part, idx_out, n_out, n_log));
  c->down_g = G;
  if (y != nullptr) {
    const int BD = B * L.d;
    PI_HIP(c, launch_k(c, K_REDUCE, k_reduce, dim3((BD + WAVE - 1) / WAVE), 0, c->part, G, BD, y));
  }
  return PI_OK;
}

// fp16/fp32 rows of 8192+ columns at 1..2 tokens: 16 lanes (256 contiguous bytes of a row)
// per neuron and slice, 8 groups. Measured on MI355X (same box) against 8 lanes and 4 groups:
// Llama-2-70B down 16.3 -> 15.2-15.5 us per layer, Falcon-40B 16.4-16.9 -> 15.4-15.8 us
// (16 lanes with 4 groups 18.6-19.6 us, 32 lanes with 8 groups 18.9-19.0 us); at OPT-6.7B
// (d = 4096) 16 lanes were no faster, so it keeps 8 lanes and 8 groups.
template <int WT, int NB, bool SCAN>
pi_status launch_down_t(pi_ctx* c, const LayerDev& L, int B, const int32_t* idx_in, const int32_t* n_in, float* y,
                        int32_t* idx_out, int32_t* n_out, int32_t* n_log, const uint64_t* tok_mask) {
  if constexpr (WT == W_Q4 && NB == 1) {
    // Q4_0 rows at one token: 8 lanes (8 blocks, 128 code bytes) per neuron and slice, 16
    // groups, 4 list items in flight per slot. Measured on MI355X at the OPT-175B shape against
    // 4 lanes, 8 groups and 8 items: 19.8 -> 17.0 us per layer (8 items: 18.5; 16 lanes with
    // 16 or 32 groups: 21-24; 4 lanes with 16 groups: 22).
    return launch_down_g<WT, NB, SCAN, 16, 8, 4>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
  }
  if constexpr (WT != W_Q4 && NB <= 2) {
    if (L.d >= 8192)
      return launch_down_g<WT, NB, SCAN, DOWN_G, 16>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
  }
  if constexpr (WT == W_Q4 && NB >= 4) {
    // 8 groups at 4..8 tokens of Q4_0 rows: one round of resident workgroups at the OPT-175B
    // shape (16 groups took two; 133 -> 128 us per layer at 8 tokens on MI355X)
    return launch_down_q4x<NB, SCAN, 8, 4>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
  } else {
    return launch_down_g<WT, NB, SCAN, down_groups(NB)>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
  }
}

template <int WT, bool SCAN>
pi_status launch_down_w(pi_ctx* c, const LayerDev& L, int B, const int32_t* idx_in, const int32_t* n_in, float* y,
                        int32_t* idx_out, int32_t* n_out, int32_t* n_log, const uint64_t* tok_mask) {
  switch (nb_for(B)) {
    case 1: return launch_down_t<WT, 1, SCAN>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
    case 2: return launch_down_t<WT, 2, SCAN>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
    case 4: return launch_down_t<WT, 4, SCAN>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
    default: return launch_down_t<WT, 8, SCAN>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
  }
}

template <bool SCAN>
pi_status launch_down(pi_ctx* c, const LayerDev& L, int B, const int32_t* idx_in, const int32_t* n_in, float* y,
                      int32_t* idx_out, int32_t* n_out, int32_t* n_log, const uint64_t* tok_mask) {
  switch (L.wtype) {
    case W_F32: return launch_down_w<W_F32, SCAN>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
    case W_F16: return launch_down_w<W_F16, SCAN>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
    default: return launch_down_w<W_Q4, SCAN>(c, L, B, idx_in, n_in, y, idx_out, n_out, n_log, tok_mask);
  }
}

// Forget the cached stack step (it holds the layers' weight pointers and the context's mode).
void drop_graph(pi_ctx* c) {
  if (c->gexec != nullptr) (void)hipGraphExecDestroy(c->gexec);
  c->gexec = nullptr;
  c->g_layers.clear();
  c->g_B = 0;
}

pi_status launch_compact(pi_ctx* c, int ffn, int32_t* idx, int32_t* n) {
  const int W = ffn / 64;
  hipLaunchKernelGGL(k_compact, dim3((W + BLOCK - 1) / BLOCK), dim3(BLOCK), 0, c->stream, c->munion, W, idx, n,
                     (int32_t*)nullptr);
  PI_HIP(c, hipGetLastError());
  return PI_OK;
}

// ---------------------------------------------------------------- scratch layout

// Byte offsets of the scratch buffers in one block (each 256-byte aligned), for batches up to
// max_batch tokens and layers up to max_d x max_ffn with rank up to max_rank. `stack`: also
// the stack runner's x buffers and count log. Batches above 8 tokens add the matrix-core
// path's buffers.
struct WsLayout {
  size_t z, mt, mu, idx, n, a, hp, part, y, ss, x0, x1, xs, nlog, zp, zh, zl, a16, total;
  size_t hp_floats, lda;
  bool mm;
};

constexpr size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

constexpr WsLayout ws_layout(int max_batch, int max_d, int max_ffn, int max_rank, bool stack) {
  WsLayout o{};
  const size_t B = max_batch, D = max_d, F = max_ffn, R = max_rank > 8 ? max_rank : 8;
  const size_t nbv = (size_t)nb_for(max_batch < 8 ? max_batch : 8);
  o.mm = max_batch > 8;
  size_t off = 0;
  o.z = off; off += al256(B * R * 4);
  o.mt = off; off += al256(B * (F / 64) * 8);
  o.mu = off; off += al256((F / 64) * 8);
  o.idx = off; off += al256(F * 4);
  o.n = off; off += al256(16 * 4);
  o.a = off; off += al256((B > nbv ? B : nbv) * F * 4);
  o.hp_floats = up_cols_floats(max_batch, max_d, max_ffn);
  o.hp = off; off += al256(o.hp_floats * 4);
  const size_t groups = o.mm ? (DOWN_G_WIDE > MM_KSD ? DOWN_G_WIDE : MM_KSD) : DOWN_G_WIDE;
  o.part = off; off += al256(groups * B * D * 4);
  o.y = off; off += al256(B * D * 4);
  o.ss = off; off += al256((size_t)GLUE_SLICES_MAX * 2 * 4);
  o.x0 = off; off += stack ? al256(B * D * 4) : 0;
  o.x1 = off; off += stack ? al256(B * D * 4) : 0;
  o.xs = off; off += stack ? al256(B * D * 4) : 0;
  o.nlog = off; off += stack ? al256(NLOG_CAP * 4) : 0;
  o.lda = (F + 15) / 16 * 16;
  o.zp = off; off += o.mm ? al256((size_t)MM_KS1 * B * R * 4) : 0;
  o.zh = off; off += o.mm ? al256(B * R * 2) : 0;
  o.zl = off; off += o.mm ? al256(B * R * 2) : 0;
  o.a16 = off; off += o.mm ? al256((size_t)(B > 32 ? 64 : 32) * o.lda * 2) : 0;
  o.total = off;
  return o;
}

// Point a context's scratch fields into the block at ws laid out by o.
void ws_assign(pi_ctx* c, uint8_t* ws, const WsLayout& o) {
  c->ws = ws;
  c->ws_bytes = o.total;
  c->z = reinterpret_cast<float*>(ws + o.z);
  c->mtok = reinterpret_cast<uint64_t*>(ws + o.mt);
  c->munion = reinterpret_cast<uint64_t*>(ws + o.mu);
  c->idx = reinterpret_cast<int32_t*>(ws + o.idx);
  c->nbuf = reinterpret_cast<int32_t*>(ws + o.n);
  c->a = reinterpret_cast<float*>(ws + o.a);
  c->hp = reinterpret_cast<float*>(ws + o.hp);
  c->hp_cap = o.hp_floats;
  c->part = reinterpret_cast<float*>(ws + o.part);
  c->y = reinterpret_cast<float*>(ws + o.y);
  c->ssq = reinterpret_cast<float*>(ws + o.ss);
  c->xbuf[0] = ws + o.x0;
  c->xbuf[1] = ws + o.x1;
  c->xstage = ws + o.xs;
  c->nlog = reinterpret_cast<int32_t*>(ws + o.nlog);
  if (o.mm) {
    c->zpart = reinterpret_cast<float*>(ws + o.zp);
    c->zhi = reinterpret_cast<half_t*>(ws + o.zh);
    c->zlo = reinterpret_cast<half_t*>(ws + o.zl);
    c->a16 = reinterpret_cast<half_t*>(ws + o.a16);
    c->lda = (int)o.lda;
  }
}

// ---------------------------------------------------------------- argument checks

pi_status check_batch(pi_ctx* c, const pi_ffn_desc& d, int B) {
  if (B < 1) return fail(c, PI_ERR_INVALID, "B must be >= 1 (got %d)", B);
  if (B > c->max_batch) return fail(c, PI_ERR_INVALID, "B %d exceeds the context's max_batch %d", B, c->max_batch);
  if (B > 8) {
    if (B > 64) return fail(c, PI_ERR_UNSUPPORTED, "batch %d: batches run up to 64 tokens", B);
    if (d.wtype != PI_W_F16)
      return fail(c, PI_ERR_UNSUPPORTED, "batches above 8 tokens run on fp16 weights (matrix cores)");
    if (d.d % 16 || d.rank % 16)
      return fail(c, PI_ERR_UNSUPPORTED, "batches above 8 tokens need d and rank multiples of 16");
    return PI_OK;
  }
  return PI_OK;
}

pi_status check_dev_ptr(pi_ctx* c, const void* p, const char* name, bool nullable = false) {
  if (p == nullptr) return nullable ? PI_OK : fail(c, PI_ERR_INVALID, "%s is NULL", name);
  if (!aligned16(p)) return fail(c, PI_ERR_INVALID, "%s is not 16-byte aligned", name);
  return PI_OK;
}

#define PI_TRY(expr)                 \
  do {                               \
    pi_status s_ = (expr);           \
    if (s_ != PI_OK) return s_;      \
  } while (0)

// A layer description against the limits of ctx (shapes, types, pointers).
pi_status check_desc(pi_ctx* ctx, const pi_ffn_desc& d) {
  if (d.d < 8 || d.d % 8) return fail(ctx, PI_ERR_INVALID, "d must be a positive multiple of 8 (got %d)", d.d);
  if (d.ffn < 64 || d.ffn % 64) return fail(ctx, PI_ERR_INVALID, "ffn must be a positive multiple of 64 (got %d)", d.ffn);
  if (d.rank < 0 || d.rank % 8) return fail(ctx, PI_ERR_INVALID, "rank must be 0 or a multiple of 8 (got %d)", d.rank);
  if (d.rank > 1024) return fail(ctx, PI_ERR_UNSUPPORTED, "rank %d above 1024", d.rank);
  if (d.d > ctx->max_d || d.ffn > ctx->max_ffn || d.rank > ctx->max_rank)
    return fail(ctx, PI_ERR_INVALID, "layer %dx%d rank %d exceeds the context (%dx%d rank %d)", d.d, d.ffn, d.rank,
                ctx->max_d, ctx->max_ffn, ctx->max_rank);
  if (d.act != PI_ACT_RELU && d.act != PI_ACT_REGLU && d.act != PI_ACT_SQRELU)
    return fail(ctx, PI_ERR_INVALID, "unknown activation %d", d.act);
  if (d.wtype != PI_W_F32 && d.wtype != PI_W_F16 && d.wtype != PI_W_Q4_0)
    return fail(ctx, PI_ERR_INVALID, "unknown weight type %d", d.wtype);
  if (d.wtype == PI_W_Q4_0 && d.d % 32) return fail(ctx, PI_ERR_INVALID, "Q4_0 needs d %% 32 == 0 (got %d)", d.d);
  if (d.wtype == PI_W_F32 && d.rank > 0)
    return fail(ctx, PI_ERR_UNSUPPORTED, "the predictor runs on fp16 tokens: fp32 layers take rank 0");
  PI_TRY(check_dev_ptr(ctx, d.w_up, "w_up"));
  PI_TRY(check_dev_ptr(ctx, d.w_down_t, "w_down_t"));
  PI_TRY(check_dev_ptr(ctx, d.b, "b"));
  if (d.act == PI_ACT_REGLU) PI_TRY(check_dev_ptr(ctx, d.w_gate, "w_gate"));
  if (d.wtype == PI_W_Q4_0) {
    PI_TRY(check_dev_ptr(ctx, d.s_up, "s_up"));
    PI_TRY(check_dev_ptr(ctx, d.s_down, "s_down"));
    if (d.act == PI_ACT_REGLU) PI_TRY(check_dev_ptr(ctx, d.s_gate, "s_gate"));
  }
  if (d.rank > 0) {
    PI_TRY(check_dev_ptr(ctx, d.p_w1, "p_w1"));
    PI_TRY(check_dev_ptr(ctx, d.p_w2, "p_w2"));
    PI_TRY(check_dev_ptr(ctx, d.p_b, "p_b"));
  }
  if (d.hot_prefix < 0 || d.hot_prefix > d.ffn)
    return fail(ctx, PI_ERR_INVALID, "hot_prefix %d outside [0, ffn %d]", d.hot_prefix, d.ffn);
  if (d.hot_prefix > 0 && d.rank == 0)
    return fail(ctx, PI_ERR_UNSUPPORTED, "a hot prefix needs a predictor layer (rank > 0)");
  PI_TRY(check_dev_ptr(ctx, d.y_center, "y_center", true));
  return PI_OK;
}

// ---------------------------------------------------------------- batched path (9..64 tokens)

// One tiled product (k_mm_gemm) over `ncols` output columns and ks K splits.
template <int EPI, int ACT, bool HILO>
pi_status launch_mm(pi_ctx* c, const MmRows& p, int ncols, int ks, int klass) {
  constexpr int NPW = (EPI == EPI_ACT && ACT == ACT_REGLU) ? 32 : 64;
  const size_t lds = mm_gemm_lds<HILO>();
  auto kern = k_mm_gemm<EPI, ACT, HILO>;
  PI_HIP(c, allow_lds(kern, lds));
  PI_HIP(c, launch_k(c, klass, kern, dim3((ncols + NPW - 1) / NPW, ks), lds, p));
  return PI_OK;
}

pi_status mm_predict(pi_ctx* c, const LayerDev& L, const half_t* x, int B, uint32_t* mtok, float* logits) {
  MmRows p{};
  p.B = B;
  p.threshold = L.threshold;
  p.ffn = L.ffn;
  if (L.rank > 0) {
    // stage 1: K-split partial sums of X W1^T, then z as fp16 hi + lo
    p.x = x;
    p.K = L.d;
    p.ldx = L.d;
    p.w0 = reinterpret_cast<const half_t*>(L.p_w1);
    p.N = L.rank;
    const int nt = (L.rank + 63) / 64;
    int ks = std::max(1, std::min(MM_KS1, 512 / nt));
    p.ks_len = ((L.d + ks - 1) / ks + MG_KC - 1) / MG_KC * MG_KC;
    ks = (L.d + p.ks_len - 1) / p.ks_len;
    p.part = c->zpart;
    PI_TRY((launch_mm<EPI_PART, ACT_RELU, false>(c, p, L.rank, ks, K_STAGE1)));
    const int BN = B * L.rank;
    PI_HIP(c, launch_k(c, K_REDUCE, k_reduce_hilo, dim3((BN + BLOCK - 1) / BLOCK), 0, c->zpart, ks, BN, c->zhi,
                       c->zlo));
    // stage 2: v = Z W2^T + b_p with the mask epilogue
    MmRows q{};
    q.x = c->zhi;
    q.x_lo = c->zlo;
    q.B = B;
    q.K = L.rank;
    q.ldx = L.rank;
    q.w0 = reinterpret_cast<const half_t*>(L.p_w2);
    q.N = L.ffn;
    q.ks_len = L.rank;
    q.bias = L.p_b;
    q.threshold = L.threshold;
    q.mask_tok = mtok;
    q.mask_union = reinterpret_cast<uint32_t*>(c->munion);
    q.logits = logits;
    q.ffn = L.ffn;
    q.hot_prefix = L.hot_prefix;
    return launch_mm<EPI_MASK, ACT_RELU, true>(c, q, L.ffn, 1, K_STAGE2);
  }
  // no predictor: the true pre-activation of the masked projection
  p.x = x;
  p.K = L.d;
  p.ldx = L.d;
  p.w0 = reinterpret_cast<const half_t*>(L.act == ACT_REGLU ? L.w_gate : L.w_up);
  p.N = L.ffn;
  p.ks_len = L.d;
  p.bias = L.b;
  p.mask_tok = mtok;
  p.mask_union = reinterpret_cast<uint32_t*>(c->munion);
  p.logits = logits;
  return launch_mm<EPI_MASK, ACT_RELU, false>(c, p, L.ffn, 1, K_TRUEMASK);
}

pi_status mm_ffn(pi_ctx* c, const LayerDev& L, const half_t* x, int B, const int32_t* idx, const int32_t* n,
                 float* y, const uint32_t* tok_mask) {
  MmRows p{};
  p.x = x;
  p.B = B;
  p.K = L.d;
  p.ldx = L.d;
  p.w0 = reinterpret_cast<const half_t*>(L.act == ACT_REGLU ? L.w_gate : L.w_up);
  p.w1 = reinterpret_cast<const half_t*>(L.w_up);
  p.idx = idx;
  p.n_dev = n;
  p.ks_len = L.d;
  p.bias = L.b;
  p.a16 = c->a16;
  p.lda = c->lda;
  p.ffn = L.ffn;
  p.tok_mask = tok_mask;
  switch (L.act) {
    case ACT_RELU: PI_TRY((launch_mm<EPI_ACT, ACT_RELU, false>(c, p, L.ffn, 1, K_UP))); break;
    case ACT_REGLU: PI_TRY((launch_mm<EPI_ACT, ACT_REGLU, false>(c, p, L.ffn, 1, K_UP))); break;
    default: PI_TRY((launch_mm<EPI_ACT, ACT_SQRELU, false>(c, p, L.ffn, 1, K_UP))); break;
  }
  MmDown q{};
  q.a16 = c->a16;
  q.lda = c->lda;
  q.B = B;
  q.wd = reinterpret_cast<const half_t*>(L.w_down_t);
  q.idx = idx;
  q.n_dev = n;
  q.ffn = L.ffn;
  q.d = L.d;
  // K splits: enough workgroups to fill the chip, each split at most MD_SPLIT_MAX positions
  const int cblocks = (L.d + MD_COLS - 1) / MD_COLS;
  int ks = std::min(MM_KSD, std::max((1024 + cblocks - 1) / cblocks, (L.ffn + MD_SPLIT_MAX - 1) / MD_SPLIT_MAX));
  q.ks_len = ((L.ffn + ks - 1) / ks + 15) / 16 * 16;
  if (q.ks_len > MD_SPLIT_MAX) return fail(c, PI_ERR_UNSUPPORTED, "ffn %d too large for the batched path", L.ffn);
  ks = (L.ffn + q.ks_len - 1) / q.ks_len;
  q.part = c->part;
  PI_HIP(c, launch_k(c, K_DOWN, k_mm_down, dim3(cblocks, ks), 0, q));
  const int BD = B * L.d;
  PI_HIP(c, launch_k(c, K_REDUCE, k_reduce, dim3((BD + WAVE - 1) / WAVE), 0, c->part, ks, BD, y));
  return PI_OK;
}

pi_status launch_compact_log(pi_ctx* c, int ffn, int32_t* idx, int32_t* n, int32_t* n_log) {
  const int W = ffn / 64;
  PI_HIP(c, launch_k(c, K_REDUCE, k_compact, dim3((W + BLOCK - 1) / BLOCK), 0, c->munion, W, idx, n, n_log));
  return PI_OK;
}

pi_status batched_predict(pi_ctx* c, const LayerDev& L, const void* x, int B, uint64_t* mask, float* logits) {
  uint32_t* mt = reinterpret_cast<uint32_t*>(mask);
  const half_t* xh = static_cast<const half_t*>(x);
  return mm_predict(c, L, xh, B, mt, logits);
}

pi_status batched_ffn(pi_ctx* c, const LayerDev& L, const void* x, int B, const int32_t* idx, const int32_t* n,
                      float* y, const uint32_t* tok_mask) {
  const half_t* xh = static_cast<const half_t*>(x);
  return mm_ffn(c, L, xh, B, idx, n, y, tok_mask);
}

pi_status enqueue_batched(pi_ctx* c, const pi_ffn* f, const void* x, int B, float* y, uint64_t* mask, int32_t* idx,
                          int32_t* n, int32_t* n_log) {
  const LayerDev L = to_dev(f->desc);
  const bool per_tok = c->mask_mode == PI_MASK_PER_TOKEN;
  if (per_tok && mask == nullptr) mask = c->mtok;
  PI_TRY(batched_predict(c, L, x, B, mask, nullptr));
  PI_TRY(launch_compact_log(c, L.ffn, idx, n, n_log));
  return batched_ffn(c, L, x, B, idx, n, y, per_tok ? reinterpret_cast<const uint32_t*>(mask) : nullptr);
}

// Enqueue the whole layer for one batch: three kernels. xin: where x comes from; x_cur: the
// layer's input in global memory as the activation step reads it (xin.x, or xin.x_out when
// xin applies the glue; written by workgroup 0 of the first kernel).
pi_status enqueue_layer(pi_ctx* c, const pi_ffn* f, const XIn& xin, const void* x_cur, int B, float* y,
                        uint64_t* mask, int32_t* idx, int32_t* n, int32_t* n_log) {
  const LayerDev L = to_dev(f->desc);
  // per-token masking needs the tokens' masks: the context's when the caller takes none
  const bool per_tok = c->mask_mode == PI_MASK_PER_TOKEN && B > 1;
  if (per_tok && mask == nullptr) mask = c->mtok;
  if (L.rank > 0) {
    PI_TRY(launch_stage1(c, L, xin, B));
    if (use_up_cols(L, B)) {
      PI_TRY(launch_stage2(c, L, B, mask, nullptr, nullptr));
      PI_TRY(launch_up_cols(c, L, x_cur, B, c->munion, nullptr, nullptr));
    } else {
      PI_TRY(launch_stage2(c, L, B, mask, nullptr, x_cur));
    }
  } else {
    PI_TRY(launch_truemask(c, L, xin, B, mask, nullptr, true));
  }
  return launch_down<true>(c, L, B, nullptr, nullptr, y, idx, n, n_log, per_tok ? mask : nullptr);
}

// ---------------------------------------------------------------- allocation-free layer

// Scratch of pi_layer_noalloc: one fixed device array, which every GPU the library runs on
// holds (at its own address) until the process ends. Sized for batches up to NOALLOC_B
// tokens and layers up to NOALLOC_D x NOALLOC_F with rank up to NOALLOC_R, laid out like a
// context's scratch without the stack runner's buffers.
constexpr int NOALLOC_B = 8, NOALLOC_D = 12288, NOALLOC_F = 49152, NOALLOC_R = 1024;
constexpr int NOALLOC_DEVICES = 64;
constexpr WsLayout NOALLOC_LAYOUT = ws_layout(NOALLOC_B, NOALLOC_D, NOALLOC_F, NOALLOC_R, false);
static_assert(NOALLOC_LAYOUT.total <= (size_t)32 << 20, "the fixed scratch stays modest");

__device__ __align__(256) uint8_t scratch[NOALLOC_LAYOUT.total];

// Per device: the array's device address (from hipGetSymbolAddress with that device current;
// the symbol's host-side name is not a device address) and the limits the launches need.
struct NoallocDev {
  void* ptr = nullptr;
  int cus = 256;
  size_t lds_max = 65536;
};
std::mutex g_noalloc_mu;
NoallocDev g_noalloc[NOALLOC_DEVICES];

pi_status noalloc_device(int device, NoallocDev* out) {
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoallocDev& dv = g_noalloc[device];
  if (dv.ptr == nullptr) {
    if (hipSetDevice(device) != hipSuccess) return PI_ERR_HIP;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return PI_ERR_HIP;
    }
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && cus > 0)
      dv.cus = cus;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, device) == hipSuccess && lds > 0)
      dv.lds_max = (size_t)lds;
    dv.ptr = ptr;
  }
  *out = dv;
  return PI_OK;
}

}  // namespace

// ======================================================================== exported ABI

extern "C" {

int32_t pi_abi_version(void) { return PI_ABI_VERSION; }

const char* pi_status_str(pi_status s) {
  switch (s) {
    case PI_OK: return "ok";
    case PI_ERR_INVALID: return "invalid argument";
    case PI_ERR_UNSUPPORTED: return "unsupported";
    case PI_ERR_OOM: return "out of device memory";
    case PI_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pi_last_error(const pi_ctx* ctx) { return ctx == nullptr ? "" : ctx->err.c_str(); }

pi_status pi_ctx_create(int32_t device, void* hip_stream, int32_t max_batch, int32_t max_d, int32_t max_ffn,
                        int32_t max_rank, pi_ctx** out) {
  if (out == nullptr) return PI_ERR_INVALID;
  *out = nullptr;
  if (max_batch < 1 || max_d < 8 || max_ffn < 64 || max_rank < 0 || max_d % 8 || max_ffn % 64)
    return PI_ERR_INVALID;
  pi_ctx* c = new (std::nothrow) pi_ctx();
  if (c == nullptr) return PI_ERR_OOM;
  c->device = device;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->max_batch = max_batch;
  c->max_d = max_d;
  c->max_ffn = max_ffn;
  c->max_rank = max_rank;
  if (hipSetDevice(device) != hipSuccess) {
    delete c;
    return PI_ERR_HIP;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) == hipSuccess) {
    c->cus = prop.multiProcessorCount;
    c->lds_max = prop.sharedMemPerBlock;
  }
  const WsLayout o = ws_layout(max_batch, max_d, max_ffn, max_rank, true);
  uint8_t* ws = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&ws), o.total) != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return PI_ERR_OOM;
  }
  if (hipMemset(ws, 0, o.total) != hipSuccess) {
    (void)hipFree(ws);
    delete c;
    return PI_ERR_HIP;
  }
  ws_assign(c, ws, o);
  if (hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) != hipSuccess) {
    (void)hipFree(c->ws);
    delete c;
    return PI_ERR_HIP;
  }
  *out = c;
  return PI_OK;
}

void pi_ctx_destroy(pi_ctx* ctx) {
  if (ctx == nullptr) return;
  (void)hipSetDevice(ctx->device);
  if (ctx->gexec != nullptr) (void)hipGraphExecDestroy(ctx->gexec);
  if (ctx->cap_stream != nullptr) (void)hipStreamDestroy(ctx->cap_stream);
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  if (ctx->ws != nullptr) (void)hipFree(ctx->ws);
  delete ctx;
}

pi_status pi_ctx_set_stream(pi_ctx* ctx, void* hip_stream) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  drop_graph(ctx);
  return PI_OK;
}

pi_status pi_ctx_set_mask_mode(pi_ctx* ctx, int32_t mode) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (mode != PI_MASK_UNION && mode != PI_MASK_PER_TOKEN) return fail(ctx, PI_ERR_INVALID, "unknown mask mode %d", mode);
  if (mode != ctx->mask_mode) drop_graph(ctx);  // a captured stack step has the old mode baked in
  ctx->mask_mode = mode;
  return PI_OK;
}

pi_status pi_ffn_create(pi_ctx* ctx, const pi_ffn_desc* desc, pi_ffn** out) {
  if (ctx == nullptr || out == nullptr) return PI_ERR_INVALID;
  *out = nullptr;
  if (desc == nullptr) return fail(ctx, PI_ERR_INVALID, "desc is NULL");
  const pi_ffn_desc& d = *desc;
  PI_TRY(check_desc(ctx, d));
  pi_ffn* f = new (std::nothrow) pi_ffn();
  if (f == nullptr) return fail(ctx, PI_ERR_OOM, "host allocation failed");
  f->desc = d;
  f->ctx = ctx;
  f->serial = g_ffn_serial.fetch_add(1);
  *out = f;
  return PI_OK;
}

void pi_ffn_destroy(pi_ffn* ffn) {
  if (ffn == nullptr) return;
  // a captured stack step holding this layer's pointers is dropped with it
  pi_ctx* c = ffn->ctx;
  if (c != nullptr && std::find(c->g_layers.begin(), c->g_layers.end(), ffn->serial) != c->g_layers.end()) {
    (void)hipSetDevice(c->device);
    drop_graph(c);
  }
  delete ffn;
}

pi_status pi_predict(pi_ctx* ctx, const pi_ffn* ffn, const void* x, int32_t B, uint64_t* mask, int32_t* idx,
                     int32_t* n_active, float* logits_out) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (ffn == nullptr) return fail(ctx, PI_ERR_INVALID, "ffn is NULL");
  PI_TRY(check_batch(ctx, ffn->desc, B));
  PI_TRY(check_dev_ptr(ctx, x, "x"));
  PI_TRY(check_dev_ptr(ctx, mask, "mask"));
  PI_TRY(check_dev_ptr(ctx, idx, "idx"));
  PI_TRY(check_dev_ptr(ctx, n_active, "n_active"));
  PI_TRY(check_dev_ptr(ctx, logits_out, "logits_out", true));
  PI_HIP(ctx, hipSetDevice(ctx->device));
  const LayerDev L = to_dev(ffn->desc);
  if (B > 8) {
    PI_TRY(batched_predict(ctx, L, x, B, mask, logits_out));
    return launch_compact(ctx, L.ffn, idx, n_active);
  }
  const XIn xin{x, nullptr, nullptr, 1, 0};
  if (L.rank > 0) {
    PI_TRY(launch_stage1(ctx, L, xin, B));
    PI_TRY(launch_stage2(ctx, L, B, mask, logits_out, nullptr));
  } else {
    PI_TRY(launch_truemask(ctx, L, xin, B, mask, logits_out, false));
  }
  return launch_compact(ctx, L.ffn, idx, n_active);
}

pi_status pi_sparse_ffn(pi_ctx* ctx, const pi_ffn* ffn, const void* x, int32_t B, const int32_t* idx,
                        const int32_t* n_active, float* y) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (ffn == nullptr) return fail(ctx, PI_ERR_INVALID, "ffn is NULL");
  PI_TRY(check_batch(ctx, ffn->desc, B));
  PI_TRY(check_dev_ptr(ctx, x, "x"));
  PI_TRY(check_dev_ptr(ctx, idx, "idx"));
  PI_TRY(check_dev_ptr(ctx, n_active, "n_active"));
  PI_TRY(check_dev_ptr(ctx, y, "y"));
  PI_HIP(ctx, hipSetDevice(ctx->device));
  const LayerDev L = to_dev(ffn->desc);
  if (B > 8) return batched_ffn(ctx, L, x, B, idx, n_active, y, nullptr);
  if (use_up_cols(L, B)) PI_TRY(launch_up_cols(ctx, L, x, B, nullptr, idx, n_active));
  else PI_TRY(launch_up(ctx, L, x, B, idx, n_active));
  return launch_down<false>(ctx, L, B, idx, n_active, y, nullptr, nullptr, nullptr, nullptr);
}

pi_status pi_layer(pi_ctx* ctx, const pi_ffn* ffn, const void* x, int32_t B, float* y, uint64_t* mask, int32_t* idx,
                   int32_t* n_active) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (ffn == nullptr) return fail(ctx, PI_ERR_INVALID, "ffn is NULL");
  PI_TRY(check_batch(ctx, ffn->desc, B));
  PI_TRY(check_dev_ptr(ctx, x, "x"));
  PI_TRY(check_dev_ptr(ctx, y, "y"));
  PI_TRY(check_dev_ptr(ctx, mask, "mask", true));
  PI_TRY(check_dev_ptr(ctx, idx, "idx", true));
  PI_TRY(check_dev_ptr(ctx, n_active, "n_active", true));
  PI_HIP(ctx, hipSetDevice(ctx->device));
  if (B > 8)
    return enqueue_batched(ctx, ffn, x, B, y, mask, idx ? idx : ctx->idx, n_active ? n_active : ctx->nbuf, nullptr);
  const XIn xin{x, nullptr, nullptr, 1, 0};
  return enqueue_layer(ctx, ffn, xin, x, B, y, mask, idx ? idx : ctx->idx, n_active ? n_active : ctx->nbuf, nullptr);
}

pi_status pi_layer_noalloc(int32_t device, void* hip_stream, const pi_ffn_desc* desc, const void* x, int32_t B,
                           float* y, uint64_t* mask, int32_t* idx, int32_t* n_active) {
  if (desc == nullptr || device < 0 || device >= NOALLOC_DEVICES || B < 1) return PI_ERR_INVALID;
  if (B > NOALLOC_B || desc->d > NOALLOC_D || desc->ffn > NOALLOC_F || desc->rank > NOALLOC_R)
    return PI_ERR_UNSUPPORTED;
  NoallocDev dv;
  PI_TRY(noalloc_device(device, &dv));
  // a host-side context over the device's fixed scratch: nothing is allocated on the device
  pi_ctx c;
  c.device = device;
  c.stream = static_cast<hipStream_t>(hip_stream);
  c.max_batch = NOALLOC_B;
  c.max_d = NOALLOC_D;
  c.max_ffn = NOALLOC_F;
  c.max_rank = NOALLOC_R;
  c.cus = dv.cus;
  c.lds_max = dv.lds_max;
  ws_assign(&c, static_cast<uint8_t*>(dv.ptr), NOALLOC_LAYOUT);
  PI_TRY(check_desc(&c, *desc));
  PI_TRY(check_batch(&c, *desc, B));
  PI_TRY(check_dev_ptr(&c, x, "x"));
  PI_TRY(check_dev_ptr(&c, y, "y"));
  PI_TRY(check_dev_ptr(&c, mask, "mask", true));
  PI_TRY(check_dev_ptr(&c, idx, "idx", true));
  PI_TRY(check_dev_ptr(&c, n_active, "n_active", true));
  if (hipSetDevice(device) != hipSuccess) return PI_ERR_HIP;
  pi_ffn f{*desc, &c, 0};
  const XIn xin{x, nullptr, nullptr, 1, 0, nullptr};
  return enqueue_layer(&c, &f, xin, x, B, y, mask, idx ? idx : c.idx, n_active ? n_active : c.nbuf, nullptr);
}

pi_status pi_q4_dequant(pi_ctx* ctx, const uint8_t* codes, const uint16_t* scales, int32_t rows, int32_t d,
                        float* out) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (rows < 0 || d <= 0 || d % 32) return fail(ctx, PI_ERR_INVALID, "rows %d, d %d: need rows >= 0 and d %% 32 == 0", rows, d);
  PI_TRY(check_dev_ptr(ctx, codes, "codes"));
  PI_TRY(check_dev_ptr(ctx, scales, "scales"));
  PI_TRY(check_dev_ptr(ctx, out, "out"));
  if (rows == 0) return PI_OK;
  PI_HIP(ctx, hipSetDevice(ctx->device));
  const long long nblocks = (long long)rows * (d / 32);
  PI_HIP(ctx, launch_k(ctx, K_REDUCE, k_q4_dequant, dim3((unsigned)((nblocks + BLOCK - 1) / BLOCK)), 0, codes, scales,
                       nblocks, out));
  return PI_OK;
}

pi_status pi_compact(pi_ctx* ctx, const float* v, int32_t B, int32_t ffn, float threshold, uint64_t* mask,
                     int32_t* idx, int32_t* n_active) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (B < 1 || B > ctx->max_batch) return fail(ctx, PI_ERR_INVALID, "B %d out of range 1..%d", B, ctx->max_batch);
  if (B > 8) return fail(ctx, PI_ERR_UNSUPPORTED, "pi_compact handles batches of 1..8");
  if (ffn < 64 || ffn % 64 || ffn > ctx->max_ffn)
    return fail(ctx, PI_ERR_INVALID, "ffn must be a multiple of 64 up to %d (got %d)", ctx->max_ffn, ffn);
  PI_TRY(check_dev_ptr(ctx, v, "v"));
  PI_TRY(check_dev_ptr(ctx, mask, "mask"));
  PI_TRY(check_dev_ptr(ctx, idx, "idx"));
  PI_TRY(check_dev_ptr(ctx, n_active, "n_active"));
  PI_HIP(ctx, hipSetDevice(ctx->device));
  const dim3 grid(ffn / 64);
  switch (nb_for(B)) {
    case 1: hipLaunchKernelGGL(k_threshold<1>, grid, dim3(WAVE), 0, ctx->stream, v, B, ffn, threshold, mask, ctx->munion); break;
    case 2: hipLaunchKernelGGL(k_threshold<2>, grid, dim3(WAVE), 0, ctx->stream, v, B, ffn, threshold, mask, ctx->munion); break;
    case 4: hipLaunchKernelGGL(k_threshold<4>, grid, dim3(WAVE), 0, ctx->stream, v, B, ffn, threshold, mask, ctx->munion); break;
    default: hipLaunchKernelGGL(k_threshold<8>, grid, dim3(WAVE), 0, ctx->stream, v, B, ffn, threshold, mask, ctx->munion); break;
  }
  PI_HIP(ctx, hipGetLastError());
  return launch_compact(ctx, ffn, idx, n_active);
}

pi_status pi_glue(pi_ctx* ctx, const float* y, const float* center, const void* x_prev, int32_t B, int32_t d,
                  int32_t x_is_f32, void* x_out) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (B < 1 || d < 8 || d % 8) return fail(ctx, PI_ERR_INVALID, "bad shape B=%d d=%d", B, d);
  PI_TRY(check_dev_ptr(ctx, y, "y"));
  PI_TRY(check_dev_ptr(ctx, center, "center", true));
  PI_TRY(check_dev_ptr(ctx, x_prev, "x_prev"));
  PI_TRY(check_dev_ptr(ctx, x_out, "x_out"));
  PI_HIP(ctx, hipSetDevice(ctx->device));
  if (x_is_f32) hipLaunchKernelGGL(k_glue<true>, dim3(B), dim3(BLOCK), 0, ctx->stream, y, center, x_prev, d, x_out);
  else hipLaunchKernelGGL(k_glue<false>, dim3(B), dim3(BLOCK), 0, ctx->stream, y, center, x_prev, d, x_out);
  PI_HIP(ctx, hipGetLastError());
  return PI_OK;
}

pi_status pi_hot_first_order(const double* p, int32_t ffn, int32_t* perm) {
  if (p == nullptr || perm == nullptr || ffn < 1) return PI_ERR_INVALID;
  std::vector<int32_t> order(ffn);
  for (int32_t i = 0; i < ffn; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [p](int32_t a, int32_t b) { return p[a] > p[b]; });
  std::memcpy(perm, order.data(), sizeof(int32_t) * ffn);
  return PI_OK;
}

pi_status pi_permute_rows(pi_ctx* ctx, const void* src, void* dst, const int32_t* perm, int32_t rows,
                          int64_t row_bytes) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (rows < 1 || row_bytes < 4 || row_bytes % 4)
    return fail(ctx, PI_ERR_INVALID, "rows %d / row_bytes %lld invalid", rows, (long long)row_bytes);
  if (src == nullptr || dst == nullptr || perm == nullptr) return fail(ctx, PI_ERR_INVALID, "NULL pointer");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 3u)
    return fail(ctx, PI_ERR_INVALID, "src/dst not 4-byte aligned");
  const uint8_t* s = static_cast<const uint8_t*>(src);
  const uint8_t* d = static_cast<const uint8_t*>(dst);
  const size_t span = (size_t)rows * (size_t)row_bytes;
  if (s < d + span && d < s + span) return fail(ctx, PI_ERR_INVALID, "src and dst overlap");
  PI_HIP(ctx, hipSetDevice(ctx->device));
  const long long rb = row_bytes;
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) && (rb & 15) == 0)
    return fail(ctx, PI_ERR_INVALID, "src/dst must be 16-byte aligned when row_bytes %% 16 == 0");
  hipLaunchKernelGGL(k_permute_rows, dim3(rows), dim3(BLOCK), 0, ctx->stream, static_cast<const uint8_t*>(src),
                     static_cast<uint8_t*>(dst), perm, (int)rows, rb);
  PI_HIP(ctx, hipGetLastError());
  return PI_OK;
}

static pi_status pi_stack_run_impl(pi_ctx* ctx, const pi_ffn* const* layers, int32_t L, const void* x_tokens,
                                   int32_t T, int32_t B, float* y_out, int32_t* n_active_log, int32_t use_graph,
                                   const pi_stack_dump* dump) {
  if (layers == nullptr || L < 1) return fail(ctx, PI_ERR_INVALID, "need at least one layer");
  if (L > NLOG_CAP) return fail(ctx, PI_ERR_INVALID, "at most %d layers", NLOG_CAP);
  if (T < 1 || B < 1 || T % B) return fail(ctx, PI_ERR_INVALID, "T %d must be a positive multiple of B %d", T, B);
  for (int l = 0; l < L; ++l) {
    if (layers[l] == nullptr) return fail(ctx, PI_ERR_INVALID, "layer %d is NULL", l);
    if (layers[l]->ctx != ctx) return fail(ctx, PI_ERR_INVALID, "layer %d belongs to another context", l);
    PI_TRY(check_batch(ctx, layers[l]->desc, B));
    if (layers[l]->desc.d != layers[0]->desc.d || layers[l]->desc.wtype != layers[0]->desc.wtype)
      return fail(ctx, PI_ERR_INVALID, "layer %d: all layers need the same d and weight type", l);
  }
  PI_TRY(check_dev_ptr(ctx, x_tokens, "x_tokens"));
  PI_TRY(check_dev_ptr(ctx, y_out, "y_out"));
  PI_TRY(check_dev_ptr(ctx, n_active_log, "n_active_log", true));
  if (dump != nullptr) {
    PI_TRY(check_dev_ptr(ctx, dump->x, "dump.x", true));
    PI_TRY(check_dev_ptr(ctx, dump->mask, "dump.mask", true));
    PI_TRY(check_dev_ptr(ctx, dump->idx, "dump.idx", true));
    PI_TRY(check_dev_ptr(ctx, dump->n, "dump.n", true));
    PI_TRY(check_dev_ptr(ctx, dump->y, "dump.y", true));
    if (dump->ffn_stride < 64 || dump->ffn_stride % 64)
      return fail(ctx, PI_ERR_INVALID, "dump.ffn_stride %d must be a positive multiple of 64", dump->ffn_stride);
    for (int l = 0; l < L; ++l)
      if (layers[l]->desc.ffn > dump->ffn_stride)
        return fail(ctx, PI_ERR_INVALID, "layer %d: ffn %d above dump.ffn_stride %d", l, layers[l]->desc.ffn,
                    dump->ffn_stride);
    use_graph = 0;
  }
  PI_HIP(ctx, hipSetDevice(ctx->device));
  const int d = layers[0]->desc.d;
  const size_t xe = x_elem(layers[0]->desc.wtype);
  const size_t xbytes = (size_t)B * d * xe, ybytes = (size_t)B * d * 4;
  // the chaining vector that feeds layer l: that of layer l - 1
  auto center_into = [&](int l) -> const float* { return l > 0 ? layers[l - 1]->desc.y_center : nullptr; };

  // dump of step s after layer l: its input, its output (partial sums added) and, through the
  // layer's own output arguments, its mask words, index list and count
  auto dump_slot = [&](int s, int l) -> size_t { return (size_t)s * L + l; };
  auto enqueue_step = [&](int s) -> pi_status {
    for (int l = 0; l < L; ++l) {
      const size_t slot = dump != nullptr ? dump_slot(s, l) : 0;
      uint64_t* mask_out = (dump != nullptr && dump->mask != nullptr)
                               ? dump->mask + slot * (size_t)B * (dump->ffn_stride / 64) : nullptr;
      int32_t* idx_out = (dump != nullptr && dump->idx != nullptr) ? dump->idx + slot * (size_t)dump->ffn_stride
                                                                   : ctx->idx;
      const void* x_cur;
      if (B > 8) {
        // batched layers take x from global memory: the glue runs as its own kernel
        x_cur = ctx->xstage;
        if (l > 0) {
          const void* x_prev = (l == 1) ? (const void*)ctx->xstage : (const void*)ctx->xbuf[(l - 1) & 1];
          PI_HIP(ctx, launch_k(ctx, K_REDUCE, k_glue<false>, dim3(B), 0, ctx->y, center_into(l), x_prev, d,
                               ctx->xbuf[l & 1]));
          x_cur = ctx->xbuf[l & 1];
        }
        PI_TRY(enqueue_batched(ctx, layers[l], x_cur, B, ctx->y, mask_out, idx_out, ctx->nbuf, ctx->nlog + l));
      } else {
        XIn xin;
        if (l == 0) {
          xin = XIn{ctx->xstage, nullptr, nullptr, 1, 0, nullptr};
          x_cur = ctx->xstage;
        } else if (B > 1) {
          // several tokens: every predictor workgroup would re-read B x d partial sums, so the
          // partials are added and the glue applied once, by two small kernels
          const void* x_prev = (l == 1) ? (const void*)ctx->xstage : (const void*)ctx->xbuf[(l - 1) & 1];
          if (glue_parts_ok(ctx, d)) {
            // one workgroup per token straight from the partials: one kernel of 7.6 us
            // instead of k_reduce + k_glue (4.8 + 11.5 us) at the OPT-175B shape, 8 tokens,
            // on MI355X (336 -> 344 tokens/s; OPT-6.7B at 4 tokens 1686 -> 1809 with stage 1
            // above)
            if (xe == 4) PI_TRY(launch_glue_parts<true>(ctx, B, d, center_into(l), x_prev, ctx->xbuf[l & 1]));
            else PI_TRY(launch_glue_parts<false>(ctx, B, d, center_into(l), x_prev, ctx->xbuf[l & 1]));
          } else {
            const int BD = B * d;
            PI_HIP(ctx, launch_k(ctx, K_REDUCE, k_reduce, dim3((BD + WAVE - 1) / WAVE), 0, ctx->part, ctx->down_g,
                                 BD, ctx->y));
            if (xe == 4)
              PI_HIP(ctx, launch_k(ctx, K_REDUCE, k_glue<true>, dim3(B), 0, ctx->y, center_into(l), x_prev, d,
                                   ctx->xbuf[l & 1]));
            else
              PI_HIP(ctx, launch_k(ctx, K_REDUCE, k_glue<false>, dim3(B), 0, ctx->y, center_into(l), x_prev, d,
                                   ctx->xbuf[l & 1]));
          }
          xin = XIn{ctx->xbuf[l & 1], nullptr, nullptr, 1, 0, nullptr};
          x_cur = ctx->xbuf[l & 1];
        } else {
          const void* x_prev = (l == 1) ? (const void*)ctx->xstage : (const void*)ctx->xbuf[(l - 1) & 1];
          if (layers[l]->desc.rank > 0 && glue_split_ok(d, xe) && (ctx->down_g == 8 || ctx->down_g == 16)) {
            // the partial sums are added once (k_glue_sum); the predictor's stage 1 finishes
            // the glue from the centred sum and the slices' sums of squares
            int nsl = 0;
            PI_TRY(launch_glue_sum(ctx, d, center_into(l), &nsl));
            xin = XIn{x_prev, ctx->y, ctx->xbuf[l & 1], 1, B * d, nullptr, ctx->ssq, nsl};
          } else {
            // the glue adds the previous layer's partial sums itself
            xin = XIn{x_prev, ctx->part, ctx->xbuf[l & 1], ctx->down_g, B * d, center_into(l)};
          }
          x_cur = ctx->xbuf[l & 1];
        }
        PI_TRY(enqueue_layer(ctx, layers[l], xin, x_cur, B, l == L - 1 ? ctx->y : nullptr, mask_out, idx_out,
                             ctx->nbuf, ctx->nlog + l));
      }
      if (dump != nullptr) {
        if (dump->x != nullptr)
          PI_HIP(ctx, hipMemcpyAsync(static_cast<uint8_t*>(dump->x) + slot * xbytes, x_cur, xbytes,
                                     hipMemcpyDeviceToDevice, ctx->stream));
        if (dump->n != nullptr)
          PI_HIP(ctx, hipMemcpyAsync(dump->n + slot, ctx->nbuf, 4, hipMemcpyDeviceToDevice, ctx->stream));
        if (dump->y != nullptr) {
          float* yd = dump->y + slot * (size_t)B * d;
          if (B > 8 || l == L - 1) {
            PI_HIP(ctx, hipMemcpyAsync(yd, ctx->y, ybytes, hipMemcpyDeviceToDevice, ctx->stream));
          } else {
            const int BD = B * d;
            PI_HIP(ctx, launch_k(ctx, K_REDUCE, k_reduce, dim3((BD + WAVE - 1) / WAVE), 0, ctx->part, ctx->down_g,
                                 BD, yd));
          }
        }
      }
    }
    return PI_OK;
  };

  bool graph_ok = false;
  if (use_graph) {
    std::vector<uint64_t> key(L);
    for (int l = 0; l < L; ++l) key[l] = layers[l]->serial;
    if (ctx->gexec != nullptr && ctx->g_layers == key && ctx->g_B == B) {
      graph_ok = true;
    } else {
      drop_graph(ctx);
      hipStream_t user = ctx->stream;
      ctx->stream = ctx->cap_stream;
      hipError_t e = hipStreamBeginCapture(ctx->cap_stream, hipStreamCaptureModeThreadLocal);
      if (e != hipSuccess) {
        ctx->stream = user;
        return fail(ctx, PI_ERR_HIP, "graph capture: %s", hipGetErrorString(e));
      }
      pi_status s = enqueue_step(0);
      hipGraph_t graph = nullptr;
      e = hipStreamEndCapture(ctx->cap_stream, &graph);
      ctx->stream = user;
      if (s != PI_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return s;
      }
      if (e != hipSuccess) return fail(ctx, PI_ERR_HIP, "graph capture: %s", hipGetErrorString(e));
      e = hipGraphInstantiate(&ctx->gexec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (e != hipSuccess) {
        ctx->gexec = nullptr;
        return fail(ctx, PI_ERR_HIP, "graph instantiate: %s", hipGetErrorString(e));
      }
      ctx->g_layers = key;
      ctx->g_B = B;
      graph_ok = true;
    }
  }
  const uint8_t* xt = static_cast<const uint8_t*>(x_tokens);
  for (int s = 0; s < T / B; ++s) {
    PI_HIP(ctx, hipMemcpyAsync(ctx->xstage, xt + (size_t)s * xbytes, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
    if (graph_ok) {
      PI_HIP(ctx, hipGraphLaunch(ctx->gexec, ctx->stream));
    } else {
      PI_TRY(enqueue_step(s));
    }
    PI_HIP(ctx, hipMemcpyAsync(reinterpret_cast<uint8_t*>(y_out) + (size_t)s * ybytes, ctx->y, ybytes,
                               hipMemcpyDeviceToDevice, ctx->stream));
    if (n_active_log != nullptr)
      PI_HIP(ctx, hipMemcpyAsync(n_active_log + (size_t)s * L, ctx->nlog, (size_t)L * 4, hipMemcpyDeviceToDevice,
                                 ctx->stream));
  }
  return PI_OK;
}

pi_status pi_stack_run(pi_ctx* ctx, const pi_ffn* const* layers, int32_t L, const void* x_tokens, int32_t T,
                       int32_t B, float* y_out, int32_t* n_active_log, int32_t use_graph) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  return pi_stack_run_impl(ctx, layers, L, x_tokens, T, B, y_out, n_active_log, use_graph, nullptr);
}

pi_status pi_stack_run_dump(pi_ctx* ctx, const pi_ffn* const* layers, int32_t L, const void* x_tokens, int32_t T,
                            int32_t B, float* y_out, int32_t* n_active_log, const pi_stack_dump* dump) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (dump == nullptr) return fail(ctx, PI_ERR_INVALID, "dump is NULL");
  return pi_stack_run_impl(ctx, layers, L, x_tokens, T, B, y_out, n_active_log, 0, dump);
}

pi_status pi_stack_profile(pi_ctx* ctx, const pi_ffn* const* layers, int32_t L, const void* x_tokens, int32_t T,
                           int32_t B, float* y_out, int32_t* n_active_log, double* ms_out, int64_t* launches_out) {
  if (ctx == nullptr) return PI_ERR_INVALID;
  if (ms_out == nullptr || launches_out == nullptr) return fail(ctx, PI_ERR_INVALID, "NULL output array");
  PI_HIP(ctx, hipSetDevice(ctx->device));
  ctx->profiling = true;
  ctx->ev_used = 0;
  pi_status s = pi_stack_run_impl(ctx, layers, L, x_tokens, T, B, y_out, n_active_log, 0, nullptr);
  ctx->profiling = false;
  if (s != PI_OK) return s;
  PI_HIP(ctx, hipStreamSynchronize(ctx->stream));
  for (int k = 0; k < PI_KERNEL_CLASSES; ++k) {
    ms_out[k] = 0.0;
    launches_out[k] = 0;
  }
  for (size_t i = 0; i < ctx->ev_used; ++i) {
    float ms = 0.f;
    PI_HIP(ctx, hipEventElapsedTime(&ms, ctx->ev[2 * i], ctx->ev[2 * i + 1]));
    ms_out[ctx->ev_class[i]] += ms;
    launches_out[ctx->ev_class[i]] += 1;
  }
  return PI_OK;
}

}  // extern "C"
