// HIP kernels (gfx950) of the neuron-aware sparse FFN.
//
// One layer, one batch of B <= 8 tokens, three dependent kernels:
//   k_stage1     z = W1 x                 predictor stage 1; when layers are chained, the
//                                         glue x = fp16(y_prev / rms(y_prev)) is its prologue
//   k_stage2     v = W2 z + b_p           predictor stage 2 and threshold: each wave ballots
//                                         (v > th) over its 8 rows, one byte of the mask word;
//                                         then the workgroup's active neurons' up (and gate)
//                                         rows give a_i = act(row_i . x)      [UP variant]
//   k_truemask   v = W x + b              instead of the two stages when there is no predictor;
//                                         for ReLU, a_i = max(v_i, 0) comes for free
//   k_down_part  y = sum over active i of a_i w_down_t[i]: every workgroup prefix-scans the
//                                         mask words itself (no waiting on other workgroups),
//                                         takes one group of active neurons over one column
//                                         slice into a partial sum; the partials are added
//                                         in a fixed order by k_reduce or the next layer's glue;
//                                         k_down_q4x for Q4_0 rows at 4..8 tokens
// Where the fused activations would make stage 2 slow (x of the batch above 64 KiB, Q4_0
// rows, d >= 8192, 5..8 tokens), stage 2 stops after the threshold and k_up_cols or, for
// Q4_0 rows, k_upq (+ k_act_fin when x is cut into several column slices) computes the
// activations instead. At one token with chained layers, k_glue_sum adds the previous
// layer's partial sums ahead of stage 1.
// Plus k_up (the index-list entry point's gathered GEMV), k_compact, k_threshold, k_glue,
// k_reduce, k_q4_dequant and k_permute_rows.
//
// Pages: P3 = "PowerInfer: Mesin Inferensi LLM Cepat dengan GPU Konsumen" (unite.ai),
// P1 = "Tüketici sınıfı GPU takılı PC'lerde yüksek hızlı büyük dil modeli serving".
#pragma once
#include "pi_device.hpp"

namespace pi {

enum { W_F32 = 0, W_F16 = 1, W_Q4 = 2 };
enum { ACT_RELU = 0, ACT_REGLU = 1, ACT_SQRELU = 2 };

// Activation of a one-row family (ReLU, Squared-ReLU) from its pre-activation h.
template <int ACT>
__device__ __forceinline__ float act_one(float h) {
  const float r = fmaxf(h, 0.f);
  if constexpr (ACT == ACT_SQRELU) return r * r;
  else return r;
}
__device__ __forceinline__ float act_one_rt(int act, float h) {
  const float r = fmaxf(h, 0.f);
  return (act == ACT_SQRELU) ? r * r : r;
}

struct LayerDev {
  int d, ffn, rank, act, wtype;
  int hot_prefix;  // stored neurons [0, hot_prefix) are taken without a prediction (predictor layers)
  float threshold;
  const uint8_t *w_up, *w_gate, *w_down_t;
  const uint16_t *s_up, *s_gate, *s_down;
  const float* b;
  const uint16_t *p_w1, *p_w2;
  const float* p_b;
};

// Where a kernel's input vector x comes from.
//  y == nullptr: x is given ([B][d], fp16 or fp32 storage).
//  y != nullptr: glue between stacked layers. Per token, u = y - c and
//                x = round(u / sqrt(mean(u^2))), or x_prev (= x) unchanged when y (or u) is
//                all zero; workgroup 0 stores it to x_out. c ([d] fp32, the previous layer's
//                expected output) may be NULL (zero). y is the sum of ny partial sums
//                y[g * ystride + t * d + col] (ny >= 1), added in order g = 0, 1, ... (the
//                previous layer's down projection leaves them).
struct XIn {
  const void* x;
  const float* y;
  void* x_out;
  int ny;
  int ystride;
  const float* c;
  // ssq != nullptr (one token, predictor layers): y is already u = y - c, summed and centred
  // by k_glue_sum, whose nsl slices' sums of squares ssq[s] = {sum y^2, sum u^2} give the
  // divisor; stage 1 finishes the glue (k_stage1_g1)
  const float* ssq;
  int nsl;
};

// Element (t, c) of the glue's y, its partial sums added in order.
__device__ __forceinline__ float y_at(const XIn& in, size_t tc) {
  float v = in.y[tc];
  for (int g = 1; g < in.ny; ++g) v += in.y[(size_t)g * in.ystride + tc];
  return v;
}
// Four consecutive elements of y from (t, c), c % 4 == 0.
__device__ __forceinline__ u32x4 y4_at(const XIn& in, size_t tc) {
  constexpr int GU = 8;
  f32x4 v = __builtin_bit_cast(f32x4, ld16(in.y + tc));
  for (int g0 = 1; g0 < in.ny; g0 += GU) {
    u32x4 p[GU];
#pragma unroll
    for (int j = 0; j < GU; ++j)
      p[j] = (g0 + j < in.ny) ? ld16(in.y + (size_t)(g0 + j) * in.ystride + tc) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < GU; ++j)
      if (g0 + j < in.ny) v += __builtin_bit_cast(f32x4, p[j]);
  }
  return __builtin_bit_cast(u32x4, v);
}

template <bool XF32> struct XType { typedef half_t T; };
template <> struct XType<true> { typedef float T; };

// Block-wide sums of two floats per thread (BLOCK threads). Uses `red` [2 * NWAVES] in LDS.
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  __syncthreads();
  if (lane == 0) {
    red[w] = a;
    red[NWAVES + w] = b;
  }
  __syncthreads();
  a = 0.f;
  b = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    a += red[i];
    b += red[NWAVES + i];
  }
}

// The glue's divisor from the sums of squares of y and of u = y - c: sqrt(mean(u^2)), or 0
// (x passes through) when either is zero.
__device__ __forceinline__ float glue_divisor(float ss_y, float ss_u, int d) {
  return (ss_y == 0.f || ss_u == 0.f) ? 0.f : sqrtf(ss_u / (float)d);
}

// Four consecutive elements of the center c from column col (zeros when c is NULL).
__device__ __forceinline__ u32x4 c4_at(const XIn& in, int col) {
  return in.c != nullptr ? ld16(in.c + col) : (u32x4){0, 0, 0, 0};
}

// Per-token divisor of the glue (0: pass x through) into rms_s[NB]. `red` [2 * NWAVES].
template <int NB>
__device__ __forceinline__ void glue_rms(const XIn& in, int B, int d, float* rms_s, float* red) {
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    float ss = 0.f, su = 0.f;
    if (t < B)
      for (int c = threadIdx.x * 4; c < d; c += BLOCK * 4) {
        const u32x4 v = y4_at(in, (size_t)t * d + c);
        const u32x4 cv = c4_at(in, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float yv = u2f(v[e]), uv = yv - u2f(cv[e]);
          ss = fmaf(yv, yv, ss);
          su = fmaf(uv, uv, su);
        }
      }
    block_sum2(ss, su, red);
    if (threadIdx.x == 0) rms_s[t] = glue_divisor(ss, su, d);
  }
  __syncthreads();
}

// The x-staging helpers are forced inline: a device function call starts with a wait for
// every outstanding load, which would make the caller's weight loads issued before the glue
// (k_stage1) complete before the glue issues its own.
// Whole-width glue into LDS: xs[t][c] = round(y[t][c] / rms(y[t])) for c < d (x_prev[t][c]
// when y[t] is all zero), rows t >= B zeroed; also stored to x_out when store_out. Every
// 16-byte load of a token's y is issued before the first is used (d <= 4 * BLOCK * J;
// d % 4 == 0). Same summation order as glue_rms.
constexpr int GLUE_J = 16;
constexpr int GLUE_NY = 8;  // partial sums the whole-width glue takes (more go through y4_at)
// after_issue() runs once, right after the first token's first y loads are issued: the
// caller issues its own x-independent loads there, behind them, since loads complete in
// issue order and the glue should not wait for the caller's.
struct NoHook { __device__ void operator()() const {} };
template <int NB, typename XT, int J = GLUE_J, typename Hook = NoHook>
__device__ __forceinline__ void glue_x(const XIn& in, int B, int d, XT* xs, int ldx, float* red, bool store_out,
                                       Hook after_issue = Hook()) {
  const int n4 = d >> 2;
  // the center's chunks (the same for every token), issued before the first y loads
  u32x4 cv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = threadIdx.x + BLOCK * j;
    cv[j] = (in.c != nullptr) ? ld16_or0(in.c + 4 * min(c, n4 - 1), c < n4) : (u32x4){0, 0, 0, 0};
  }
  for (int t = 0; t < NB; ++t) {
    if (t >= B) {
      for (int c = threadIdx.x; c < d; c += BLOCK) xs[t * ldx + c] = (XT)0.f;
      continue;
    }
    u32x4 v[J];
    if (in.ny == 1) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = threadIdx.x + BLOCK * j;
        v[j] = ld16_or0(in.y + (size_t)t * d + 4 * min(c, n4 - 1), c < n4);
      }
      if (t == 0) after_issue();
    } else {
      // partial sums: four chunks at a time with all of their (up to GLUE_NY) partials in
      // flight, added in partial order
#pragma unroll
      for (int j0 = 0; j0 < J; j0 += 4) {
        if (BLOCK * j0 < n4) {
          u32x4 p[4][GLUE_NY];
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < GLUE_NY; ++g) {
              const int c = threadIdx.x + BLOCK * (j0 + j);
              p[j][g] = ld16_or0(in.y + (size_t)min(g, in.ny - 1) * in.ystride + (size_t)t * d + 4 * min(c, n4 - 1),
                                 c < n4 && g < in.ny);
            }
          if (t == 0 && j0 == 0) after_issue();
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4 acc = __builtin_bit_cast(f32x4, p[j][0]);
#pragma unroll
            for (int g = 1; g < GLUE_NY; ++g)
              if (g < in.ny) acc += __builtin_bit_cast(f32x4, p[j][g]);
            v[j0 + j] = __builtin_bit_cast(u32x4, acc);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j0 + j] = (u32x4){0, 0, 0, 0};
        }
      }
    }
    // sums of squares of y and of u = y - c (v becomes u); chunks past d are zero in both
    float ss = 0.f, su = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float yv = u2f(v[j][e]), uv = yv - u2f(cv[j][e]);
        ss = fmaf(yv, yv, ss);
        su = fmaf(uv, uv, su);
        v[j][e] = __builtin_bit_cast(uint32_t, uv);
      }
    block_sum2(ss, su, red);
    const float r = glue_divisor(ss, su, d);
    const XT* xp = reinterpret_cast<const XT*>(in.x) + (size_t)t * d;
    XT* xo = reinterpret_cast<XT*>(in.x_out) + (size_t)t * d;
    // r is the same in every thread: one branch, so the common case issues no load of x_prev
    if (r != 0.f) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = threadIdx.x + BLOCK * j;
        if (c < n4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const XT o = (XT)(u2f(v[j][e]) / r);
            xs[t * ldx + 4 * c + e] = o;
            if (store_out) xo[4 * c + e] = o;
          }
        }
      }
    } else {
      for (int c = threadIdx.x; c < d; c += BLOCK) {
        const XT o = xp[c];
        xs[t * ldx + c] = o;
        if (store_out) xo[c] = o;
      }
    }
  }
}

// Stage x[:, c0 : c0+cw) of NB tokens into LDS xs[t][0..cw) (zeros for t >= B).
template <int NB, bool XF32>
__device__ __forceinline__ void stage_x(const XIn& in, int B, int d, int c0, int cw, typename XType<XF32>::T* xs, int ldx,
                        const float* rms_s, bool store_out) {
  typedef typename XType<XF32>::T XT;
  for (int t = 0; t < NB; ++t) {
    for (int c = threadIdx.x; c < cw; c += BLOCK) {
      XT v = (XT)0.f;
      if (t < B) {
        const size_t gi = (size_t)t * d + c0 + c;
        if (in.y != nullptr) {
          const float r = rms_s[t];
          if (r == 0.f) v = reinterpret_cast<const XT*>(in.x)[gi];
          else v = (XT)((y_at(in, gi) - (in.c != nullptr ? in.c[c0 + c] : 0.f)) / r);
          if (store_out) reinterpret_cast<XT*>(in.x_out)[gi] = v;
        } else {
          v = reinterpret_cast<const XT*>(in.x)[gi];
        }
      }
      xs[t * ldx + c] = v;
    }
  }
}

// Copy x [NB][d] (fp16 or fp32 storage, rows t >= B zeroed) from global memory into LDS with
// 16-byte accesses (d * sizeof(XT) is a multiple of 16).
template <int NB, typename XT>
__device__ __forceinline__ void load_x(const void* x, int B, int d, XT* xs) {
  constexpr int E = 16 / sizeof(XT);
  const int n16 = d / E;
  for (int t = 0; t < NB; ++t)
    for (int c = threadIdx.x; c < n16; c += BLOCK) {
      u32x4 v = (u32x4){0, 0, 0, 0};
      if (t < B) v = ld16(reinterpret_cast<const XT*>(x) + (size_t)t * d + c * E);
      *reinterpret_cast<u32x4*>(xs + t * d + c * E) = v;
    }
}

// ---------------------------------------------------------------------------------------
// Partial dot products of R weight rows with NB vectors staged in LDS. Lane l handles each
// row's 16-byte chunks l, l+64, l+128, ...; U chunks of all R rows are in flight at a time.
// acc may have more rows (RA) than are used. The caller reduces across lanes.
//   F32: chunk = 4 floats, x fp32.  F16: chunk = 8 halves, x fp16 (dot2).
//   Q4:  chunk = one 32-element block (16 code bytes + an fp16 scale), x fp16.
// ---------------------------------------------------------------------------------------
template <int WT, int NB, int R, int U, typename XT, int RA>
__device__ __forceinline__ void rows_dot(const uint8_t* const (&row)[RA], const uint16_t* const (&srow)[RA],
                                         const XT* xs, int ldx, int d, int lane, float (&acc)[RA][NB]) {
  static_assert(R <= RA, "more rows than accumulators");
  if constexpr (WT == W_F16 || WT == W_F32) {
    constexpr int EPC = (WT == W_F16) ? 8 : 4;  // elements per 16-byte chunk
    const int nch = d / EPC;
    for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
      u32x4 w[R][U];
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + lane + WAVE * u;
          w[q][u] = ld_stream_or0(row[q] + (size_t)min(c, nch - 1) * 16, c < nch);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        if (c < nch) {
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            const u32x4 xv = ld16(xs + t * ldx + c * EPC);
#pragma unroll
            for (int q = 0; q < R; ++q) {
              float s = acc[q][t];
              if constexpr (WT == W_F16) {
                s = dot2(w[q][u][0], xv[0], s);
                s = dot2(w[q][u][1], xv[1], s);
                s = dot2(w[q][u][2], xv[2], s);
                s = dot2(w[q][u][3], xv[3], s);
              } else {
                s = fmaf(u2f(w[q][u][0]), u2f(xv[0]), s);
                s = fmaf(u2f(w[q][u][1]), u2f(xv[1]), s);
                s = fmaf(u2f(w[q][u][2]), u2f(xv[2]), s);
                s = fmaf(u2f(w[q][u][3]), u2f(xv[3]), s);
              }
              acc[q][t] = s;
            }
          }
        }
      }
    }
  } else {  // W_Q4: a lane takes whole blocks, unpacked once for all tokens
    const int nb = d >> 5;
    for (int c0 = 0; c0 < nb; c0 += WAVE * U) {
      u32x4 w[R][U];
      float sc[R][U];
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + lane + WAVE * u;
          const int cc = min(c, nb - 1);
          w[q][u] = ld_stream_or0(row[q] + (size_t)cc * 16, c < nb);
          const float s = half_bits_to_float(srow[q][cc]);
          sc[q][u] = (c < nb) ? s : 0.f;
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        if (c < nb) {
          // (q - 8) of every row's block as fp16 pairs, once for all tokens
          uint32_t wq[R][16];
#pragma unroll
          for (int q = 0; q < R; ++q) q4_block_unpack(w[q][u], wq[q]);
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            const half_t* xb = reinterpret_cast<const half_t*>(xs) + t * ldx + c * 32;
            uint32_t xv[16];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const u32x4 qv = ld16(xb + 8 * m);
              xv[4 * m + 0] = qv[0];
              xv[4 * m + 1] = qv[1];
              xv[4 * m + 2] = qv[2];
              xv[4 * m + 3] = qv[3];
            }
#pragma unroll
            for (int q = 0; q < R; ++q) {
              float s = 0.f;
#pragma unroll
              for (int e = 0; e < 16; ++e) s = dot2(wq[q][e], xv[e], s);
              acc[q][t] = fmaf(sc[q][u], s, acc[q][t]);
            }
          }
        }
      }
    }
  }
}

template <int WT>
__device__ __forceinline__ const uint8_t* row_ptr(const uint8_t* base, int i, int d) {
  if constexpr (WT == W_F32) return base + (size_t)i * d * 4;
  else if constexpr (WT == W_F16) return base + (size_t)i * d * 2;
  else return base + (size_t)i * (d >> 5) * 16;
}
template <int WT>
__device__ __forceinline__ const uint16_t* scale_ptr(const uint16_t* base, int i, int d) {
  return (WT == W_Q4) ? base + (size_t)i * (d >> 5) : nullptr;
}

// ---------------------------------------------------------------------------------------
// Activation rounds. A workgroup computes a_i for a list of `cnt` neurons (item k is neuron
// id_of(k)); item k goes to wave k % 4, and in each round a wave takes up to PW of its items
// (ReLU: PW = 4 up rows; ReGLU: PW = 2 neurons = 4 rows, gate and up) with all their rows in
// flight together. The number of rounds depends only on cnt, so every wave passes the same
// barriers: x may be staged in column windows of width dw (stage(c0, cw) fills xs) when it
// does not fit in LDS whole (dw == d: xs already holds x).
// a_i is computed the same way whichever wave, round or window layout handles it: each lane
// sums its chunks in ascending order, then the wave sums the lanes.
// ---------------------------------------------------------------------------------------
template <int WT>
__device__ __forceinline__ const uint8_t* row_at(const uint8_t* base, int i, int d, int c0) {
  if constexpr (WT == W_F32) return base + ((size_t)i * d + c0) * 4;
  else if constexpr (WT == W_F16) return base + ((size_t)i * d + c0) * 2;
  else return base + ((size_t)i * (d >> 5) + (c0 >> 5)) * 16;
}
template <int WT>
__device__ __forceinline__ const uint16_t* scale_at(const uint16_t* base, int i, int d, int c0) {
  if constexpr (WT == W_Q4) return base + (size_t)i * (d >> 5) + (c0 >> 5);
  else return nullptr;
}

// Chunks per lane in flight per row for R rows in flight: about 128 VGPRs of weights.
template <int WT, int R> struct ActU {
  static constexpr int U = (WT == W_Q4) ? 16 / R : (32 / R > 16 ? 16 : 32 / R);
};

constexpr int ACT_RA = 4;  // rows in flight per wave in a round
template <int ACT> struct ActPW { static constexpr int PW = (ACT == ACT_REGLU) ? 2 : 4; };

// acc[r][t] += row_r[c0, c0+cw) . xs[t][0, cw) for the rows of the first NR ids.
template <int WT, int ACT, int NB, int NR, typename XT>
__device__ __forceinline__ void act_accum(const LayerDev& L, const XT* xs, int ldx, int c0, int cw, int lane,
                                          const int (&ids)[ActPW<ACT>::PW], float (&acc)[ACT_RA][NB]) {
  constexpr int R = (ACT == ACT_REGLU ? 2 : 1) * NR;
  const int d = L.d;
  const uint8_t* rows[ACT_RA] = {nullptr, nullptr, nullptr, nullptr};
  const uint16_t* srows[ACT_RA] = {nullptr, nullptr, nullptr, nullptr};
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    if constexpr (ACT != ACT_REGLU) {
      rows[q] = row_at<WT>(L.w_up, ids[q], d, c0);
      srows[q] = scale_at<WT>(L.s_up, ids[q], d, c0);
    } else {
      rows[2 * q] = row_at<WT>(L.w_gate, ids[q], d, c0);
      srows[2 * q] = scale_at<WT>(L.s_gate, ids[q], d, c0);
      rows[2 * q + 1] = row_at<WT>(L.w_up, ids[q], d, c0);
      srows[2 * q + 1] = scale_at<WT>(L.s_up, ids[q], d, c0);
    }
  }
  rows_dot<WT, NB, R, ActU<WT, R>::U, XT, ACT_RA>(rows, srows, xs, ldx, cw, lane, acc);
}

template <int ACT, int NB>
__device__ __forceinline__ void act_store(const LayerDev& L, int B, int lane, const int (&ids)[ActPW<ACT>::PW], int m,
                                          float (&acc)[ACT_RA][NB], float* __restrict__ a) {
  constexpr int PW = ActPW<ACT>::PW;
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    if (q < m) {
      const float bias = L.b[ids[q]];
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        float v;
        if constexpr (ACT != ACT_REGLU) {
          v = act_one<ACT>(wave_sum(acc[q][t]) + bias);
        } else {
          const float g = wave_sum(acc[2 * q][t]) + bias;
          const float u = wave_sum(acc[2 * q + 1][t]);
          v = fmaxf(g, 0.f) * u;
        }
        if (lane == t && t < B) a[(size_t)ids[q] * NB + t] = v;
      }
    }
  }
}

// Rounds over the columns [cb, ce) of the rows; out(ids, m, acc) takes each round's sums.
template <int WT, int ACT, int NB, typename XT, typename IdOf, typename Stage, typename Out>
__device__ __forceinline__ void act_rounds_cols(const LayerDev& L, int cnt, IdOf id_of, const XT* xs, int ldx, int cb, int ce, int dw,
                                Stage stage, Out out) {
  constexpr int PW = ActPW<ACT>::PW;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int rounds = (cnt + NWAVES * PW - 1) / (NWAVES * PW);
  for (int rho = 0; rho < rounds; ++rho) {
    int ids[PW];
    int m = 0;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int k = wave + NWAVES * (rho * PW + j);
      ids[j] = (k < cnt) ? id_of(k) : 0;
      m += (k < cnt) ? 1 : 0;
    }
    float acc[ACT_RA][NB];
#pragma unroll
    for (int q = 0; q < ACT_RA; ++q)
#pragma unroll
      for (int t = 0; t < NB; ++t) acc[q][t] = 0.f;
    for (int c0 = cb; c0 < ce; c0 += dw) {
      const int cw = min(dw, ce - c0);
      if (dw < ce - cb) {
        __syncthreads();
        stage(c0, cw);
        __syncthreads();
      }
      if constexpr (ACT != ACT_REGLU) {
        switch (m) {
          case 1: act_accum<WT, ACT, NB, 1, XT>(L, xs, ldx, c0, cw, lane, ids, acc); break;
          case 2: act_accum<WT, ACT, NB, 2, XT>(L, xs, ldx, c0, cw, lane, ids, acc); break;
          case 3: act_accum<WT, ACT, NB, 3, XT>(L, xs, ldx, c0, cw, lane, ids, acc); break;
          case 4: act_accum<WT, ACT, NB, 4, XT>(L, xs, ldx, c0, cw, lane, ids, acc); break;
          default: break;
        }
      } else {
        switch (m) {
          case 1: act_accum<WT, ACT, NB, 1, XT>(L, xs, ldx, c0, cw, lane, ids, acc); break;
          case 2: act_accum<WT, ACT, NB, 2, XT>(L, xs, ldx, c0, cw, lane, ids, acc); break;
          default: break;
        }
      }
    }
    out(ids, m, acc);
  }
}

template <int WT, int ACT, int NB, typename XT, typename IdOf, typename Stage>
__device__ __forceinline__ void act_rounds(const LayerDev& L, int B, int cnt, IdOf id_of, const XT* xs, int ldx, int dw, Stage stage,
                           float* __restrict__ a) {
  const int lane = threadIdx.x % WAVE;
  auto out = [&](const int (&ids)[ActPW<ACT>::PW], int m, float (&acc)[ACT_RA][NB]) {
    act_store<ACT, NB>(L, B, lane, ids, m, acc, a);
  };
  act_rounds_cols<WT, ACT, NB, XT>(L, cnt, id_of, xs, ldx, 0, L.d, dw, stage, out);
}

// Copy columns [c0, c0 + cw) of x [NB][d] (rows t >= B zeroed) into xs[t][0, cw) with
// 16-byte accesses (cw * sizeof(XT) % 16 == 0). The NB x cw/E chunks form one flat range:
// each thread issues J loads (over all tokens) before storing any.
template <int NB, typename XT, int NTH = BLOCK>
__device__ __forceinline__ void load_x_cols(const void* x, int B, int d, int c0, int cw, XT* xs, int ldx) {
  constexpr int E = 16 / sizeof(XT);
  constexpr int J = 16 * BLOCK / NTH;
  const int n16 = cw / E, total = NB * n16;
  for (int f0 = 0; f0 < total; f0 += NTH * J) {
    u32x4 v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int f = f0 + threadIdx.x + NTH * j;
      const int t = f / n16, c = f - t * n16;
      const bool ok = f < total && t < B;
      v[j] = ld16_or0(reinterpret_cast<const XT*>(x) + (ok ? (size_t)t * d + c * E : 0) + c0, ok);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int f = f0 + threadIdx.x + NTH * j;
      const int t = f / n16, c = f - t * n16;
      if (f < total) *reinterpret_cast<u32x4*>(xs + t * ldx + c * E) = v[j];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Mask epilogue (wave 0 of a workgroup owning neurons [64*tile, 64*tile + 64)):
// lane j holds v of neuron 64*tile + j for each token; a ballot of (v > threshold) is the
// token's mask word, the OR over tokens the union word (returned, and stored).
// ---------------------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ uint64_t emit_mask(const float (*vs)[WAVE], int tile, int B, float th, int ffn,
                                              uint64_t* mask_tok, uint64_t* mask_union, float* logits) {
  const int lane = threadIdx.x;
  const int W = ffn >> 6;
  uint64_t u = 0;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if (t < B) {
      const float v = vs[t][lane];
      const uint64_t w = __ballot(v > th);
      u |= w;
      if (lane == 0 && mask_tok != nullptr) mask_tok[(size_t)t * W + tile] = w;
      if (logits != nullptr) logits[(size_t)t * ffn + tile * WAVE + lane] = v;
    }
  }
  if (lane == 0) mask_union[tile] = u;
  return u;
}

// ---------------------------------------------------------------------------------------
// k_stage1: z[t][j] = W1[j] . x_t. One wave per row of W1; x staged in LDS in column
// windows of `dc` elements (one window unless NB*d*2 exceeds the LDS budget).
// ---------------------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(BLOCK) void k_stage1(LayerDev L, XIn xin, int B, int dc, float* __restrict__ z) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);
  __shared__ float red[2 * NWAVES];
  __shared__ float rms_s[NB];
  const int d = L.d, r = L.rank;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int row = blockIdx.x * NWAVES + wave;
  // The weights do not depend on x: this wave's first 8 chunks per lane are issued before x
  // is staged, so their latency overlaps. With the whole-width glue they go out right behind
  // the glue's loads of y (loads complete in issue order, so the glue does not wait for them).
  constexpr int PF = 8;
  const int nch0 = min(dc, d) >> 3;
  const uint8_t* wrow0 = reinterpret_cast<const uint8_t*>(L.p_w1) + (size_t)min(row, r - 1) * d * 2;
  u32x4 wp[PF];
  auto issue_w1 = [&]() {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int c = lane + WAVE * u;
      wp[u] = ld_stream_or0(wrow0 + (size_t)min(c, nch0 - 1) * 16, row < r && c < nch0);
    }
  };
  // x fits in LDS (and, for the glue, in one pass of registers): glue or copy it at once
  constexpr int GJ = (NB >= 8) ? 4 : (NB >= 4) ? 8 : GLUE_J;  // x of NB tokens in 64 KB: d <= 4 * BLOCK * GJ
  const bool whole = dc >= d && (xin.y == nullptr || (d <= 4 * BLOCK * GJ && xin.ny <= GLUE_NY));
  if (!(whole && xin.y != nullptr)) issue_w1();
  if (whole) {
    if (xin.y != nullptr) glue_x<NB, half_t, GJ>(xin, B, d, xs, d, red, blockIdx.x == 0, issue_w1);
    else load_x_cols<NB, half_t>(xin.x, B, d, 0, d, xs, d);
  } else if (xin.y != nullptr) {
    glue_rms<NB>(xin, B, d, rms_s, red);
  }
  float acc[1][NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[0][t] = 0.f;
  for (int c0 = 0; c0 < d; c0 += dc) {
    const int cw = min(dc, d - c0);
    __syncthreads();
    if (!whole) {
      if (xin.y != nullptr) stage_x<NB, false>(xin, B, d, c0, cw, xs, dc, rms_s, blockIdx.x == 0);
      else load_x_cols<NB, half_t>(xin.x, B, d, c0, cw, xs, dc);
    }
    __syncthreads();
    if (row < r) {
      int done = 0;  // chunks of this window already accumulated
      if (c0 == 0) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int c = lane + WAVE * u;
          if (c < nch0) {
#pragma unroll
            for (int t = 0; t < NB; ++t) {
              const u32x4 xv = ld16(xs + t * dc + c * 8);
              float s2 = acc[0][t];
              s2 = dot2(wp[u][0], xv[0], s2);
              s2 = dot2(wp[u][1], xv[1], s2);
              s2 = dot2(wp[u][2], xv[2], s2);
              s2 = dot2(wp[u][3], xv[3], s2);
              acc[0][t] = s2;
            }
          }
        }
        done = min(nch0, WAVE * PF);
      }
      if (done * 8 < cw) {
        const uint8_t* const rows[1] = {wrow0 + ((size_t)c0 + done * 8) * 2};
        const uint16_t* const srows[1] = {nullptr};
        rows_dot<W_F16, NB, 1, 8, half_t, 1>(rows, srows, xs + done * 8, dc, cw - done * 8, lane, acc);
      }
    }
  }
  if (row < r) {
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float s = wave_sum(acc[0][t]);
      if (lane == 0 && t < B) z[(size_t)t * r + row] = s;
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_stage1_x: z[t][j] = W1[j] . x_t for 2..8 tokens of given x (fp16, d <= 512 * PF). KS
// waves per row of W1, wave h of a row taking the chunk groups h, h + KS, ... (group g =
// columns 512 g .. 512 g + 511, 16 bytes per lane), all of them in flight from entry; x
// staged in LDS in column windows of dc elements (d, or a multiple of 512), each window's
// chunks taken from registers once the window is staged. The KS shares of a row are added
// in share order.
// ---------------------------------------------------------------------------------------
template <int NB, int PF, int KS>
__global__ __launch_bounds__(BLOCK * KS) void k_stage1_x(LayerDev L, const half_t* __restrict__ x, int B, int dc,
                                                         float* __restrict__ z) {
  constexpr int NTH = BLOCK * KS, PFW = (PF + KS - 1) / KS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);
  __shared__ float s_share[NWAVES * KS * NB];
  const int d = L.d, r = L.rank, nch = d >> 3;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int rw = wave / KS, h = wave % KS;  // row of the workgroup, share of the row
  const int row = blockIdx.x * NWAVES + rw;
  const uint8_t* wrow = reinterpret_cast<const uint8_t*>(L.p_w1) + (size_t)min(row, r - 1) * d * 2;
  u32x4 wv[PFW];
#pragma unroll
  for (int q = 0; q < PFW; ++q) {
    const int g = KS * q + h, c = lane + WAVE * g;
    wv[q] = ld_stream_or0(wrow + (size_t)min(c, nch - 1) * 16, row < r && g < PF && c < nch);
  }
  float acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = 0.f;
  for (int c0 = 0; c0 < d; c0 += dc) {
    const int cw = min(dc, d - c0);
    __syncthreads();
    load_x_cols<NB, half_t, NTH>(x, B, d, c0, cw, xs, dc);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PFW; ++q) {
      const int g = KS * q + h, c = lane + WAVE * g;  // group g's columns lie in this window
      if (g < PF && WAVE * 8 * g >= c0 && WAVE * 8 * g < c0 + cw && c < nch) {
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const u32x4 xv = ld16(xs + t * dc + (c * 8 - c0));
          float s2 = acc[t];
          s2 = dot2(wv[q][0], xv[0], s2);
          s2 = dot2(wv[q][1], xv[1], s2);
          s2 = dot2(wv[q][2], xv[2], s2);
          s2 = dot2(wv[q][3], xv[3], s2);
          acc[t] = s2;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const float s = wave_sum(acc[t]);
    if (lane == 0) s_share[(rw * KS + h) * NB + t] = s;
  }
  __syncthreads();
  if (h == 0 && lane < NB && lane < B && row < r) {
    float v = 0.f;
    for (int k = 0; k < KS; ++k) v += s_share[(rw * KS + k) * NB + lane];
    z[(size_t)lane * r + row] = v;
  }
}

// ---------------------------------------------------------------------------------------
// The glue between stacked layers at one token, in two steps, so that no workgroup of the
// predictor reads the previous layer's G partial sums (G x d floats each).
// k_glue_sum: workgroup s takes columns [4 * BLOCK * s, 4 * BLOCK * (s + 1)): y = the G
// partial sums added in group order (as glue_x adds them), u = y - c, stored to u[col]
// (fp32), and the slice's sums of squares ssq[s] = {sum of y^2, sum of u^2}.
// k_stage1_g1: adds the slices' sums in slice order, x = fp16(u / sqrt(mean(u^2))) (x_prev
// when y or u is all zero), stores x to x_out (workgroup 0) and computes z = W1 x: KS waves
// per row of W1 (alternate 512-column chunk groups, their shares added in order), the row's
// first PRE chunk groups issued at entry (behind the loads of u), the rest once x is formed.
// ---------------------------------------------------------------------------------------
constexpr int GLUE_SLICES_MAX = 16;  // slices of k_glue_sum: d <= 4 * BLOCK * 16

template <int G>
__global__ __launch_bounds__(BLOCK) void k_glue_sum(const float* __restrict__ part, int gstride,
                                                    const float* __restrict__ center, int d, float* __restrict__ u,
                                                    float* __restrict__ ssq) {
  __shared__ float red[2 * NWAVES];
  const int n4 = d >> 2;
  const int c = blockIdx.x * BLOCK + threadIdx.x;
  const bool ok = c < n4;
  const size_t off = 4 * (size_t)min(c, n4 - 1);
  u32x4 p[G];
#pragma unroll
  for (int g = 0; g < G; ++g) p[g] = ld16_or0(part + (size_t)g * gstride + off, ok);
  const u32x4 cv = (center != nullptr) ? ld16_or0(center + off, ok) : (u32x4){0, 0, 0, 0};
  f32x4 y = __builtin_bit_cast(f32x4, p[0]);
#pragma unroll
  for (int g = 1; g < G; ++g) y += __builtin_bit_cast(f32x4, p[g]);
  float ss = 0.f, su = 0.f;
  u32x4 uo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float uv = y[e] - u2f(cv[e]);
    ss = fmaf(y[e], y[e], ss);
    su = fmaf(uv, uv, su);
    uo[e] = __builtin_bit_cast(uint32_t, uv);
  }
  if (ok) *reinterpret_cast<u32x4*>(u + off) = uo;
  block_sum2(ss, su, red);
  if (threadIdx.x == 0) {
    ssq[2 * blockIdx.x] = ss;
    ssq[2 * blockIdx.x + 1] = su;
  }
}

// PF: chunks of 16 bytes per lane in a W1 row (d <= 512 * PF); u is read as PF / 2 chunks
// of 4 floats per thread. PRE <= PF: chunks issued before x is formed.
template <int PF, int PRE, int KS>
__global__ __launch_bounds__(BLOCK * KS) void k_stage1_g1(LayerDev L, const float* __restrict__ u,
                                                          const float* __restrict__ ssq, int nsl,
                                                          const half_t* __restrict__ x_prev,
                                                          half_t* __restrict__ x_out, float* __restrict__ z) {
  constexpr int NTH = BLOCK * KS;
  constexpr int J = (PF / 2 + KS - 1) / KS;     // chunks of 4 floats of u per thread
  constexpr int PFW = (PF + KS - 1) / KS;       // chunk groups of the row per wave
  constexpr int PREW = (PRE + KS - 1) / KS;     // of them issued before x is formed
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);
  __shared__ float s_share[NWAVES * KS];
  const int d = L.d, r = L.rank;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int rw = wave / KS, h = wave % KS;  // row of the workgroup, share of the row
  const int row = blockIdx.x * NWAVES + rw;
  const int n4 = d >> 2, nch = d >> 3;
  // the slices' sums of squares (the same addresses in every thread), then u, then the row
  u32x4 sq[GLUE_SLICES_MAX / 2];
#pragma unroll
  for (int k = 0; k < GLUE_SLICES_MAX / 2; ++k)
    sq[k] = ld16_or0(ssq + 4 * min(k, (nsl - 1) / 2), 2 * k < nsl);
  u32x4 uv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = threadIdx.x + NTH * j;
    uv[j] = ld16_or0(u + 4 * (size_t)min(c, n4 - 1), c < n4);
  }
  const uint8_t* wrow = reinterpret_cast<const uint8_t*>(L.p_w1) + (size_t)min(row, r - 1) * d * 2;
  // chunk group g = KS q + h of the row: columns 512 g .. 512 g + 511, 16 bytes per lane
  u32x4 wv[PFW];
  auto issue = [&](int q) {
    const int g = KS * q + h, c = lane + WAVE * g;
    wv[q] = ld_stream_or0(wrow + (size_t)min(c, nch - 1) * 16, row < r && g < PF && c < nch);
  };
#pragma unroll
  for (int q = 0; q < PREW; ++q) issue(q);
  float sy = 0.f, su = 0.f;
#pragma unroll
  for (int k = 0; k < GLUE_SLICES_MAX / 2; ++k) {
    if (2 * k < nsl) {
      sy += u2f(sq[k][0]);
      su += u2f(sq[k][1]);
    }
    if (2 * k + 1 < nsl) {
      sy += u2f(sq[k][2]);
      su += u2f(sq[k][3]);
    }
  }
  const float rr = glue_divisor(sy, su, d);
  const bool out = blockIdx.x == 0;
  // rr is the same in every thread: one branch, so the common case loads no x_prev
  if (rr != 0.f) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = threadIdx.x + NTH * j;
      if (c < n4) {
        const half2_t h01 = {(half_t)(u2f(uv[j][0]) / rr), (half_t)(u2f(uv[j][1]) / rr)};
        const half2_t h23 = {(half_t)(u2f(uv[j][2]) / rr), (half_t)(u2f(uv[j][3]) / rr)};
        const uint2 o = {__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
        *reinterpret_cast<uint2*>(xs + 4 * c) = o;
        if (out) *reinterpret_cast<uint2*>(x_out + 4 * c) = o;
      }
    }
  } else {
    for (int c = threadIdx.x; c < nch; c += NTH) {
      const u32x4 o = ld16(x_prev + 8 * c);
      *reinterpret_cast<u32x4*>(xs + 8 * c) = o;
      if (out) *reinterpret_cast<u32x4*>(x_out + 8 * c) = o;
    }
  }
  // the rest of the row after x
#pragma unroll
  for (int q = PREW; q < PFW; ++q) issue(q);
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < PFW; ++q) {
    const int g = KS * q + h, c = lane + WAVE * g;
    if (g < PF && c < nch) {
      const u32x4 xv = ld16(xs + 8 * c);
      acc = dot2(wv[q][0], xv[0], acc);
      acc = dot2(wv[q][1], xv[1], acc);
      acc = dot2(wv[q][2], xv[2], acc);
      acc = dot2(wv[q][3], xv[3], acc);
    }
  }
  acc = wave_sum(acc);
  if constexpr (KS == 1) {
    if (lane == 0 && row < r) z[row] = acc;
  } else {
    // the row's shares, added in share order
    if (lane == 0) s_share[rw * KS + h] = acc;
    __syncthreads();
    if (h == 0 && lane == 0 && row < r) {
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k) v += s_share[rw * KS + k];
      z[row] = v;
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_stage2: v = W2 z + b_p and the threshold for 32 neurons per workgroup: wave w owns the 8
// neurons of mask byte w * gridDim.x + blockIdx.x (bytes are dealt out across workgroups, so a
// hot-first layout does not load a few workgroups with every active neuron). Each wave ballots
// (v > th) over its rows and stores that byte of the token's and the batch union's mask words.
// W2 rows are issued before z is read. Lane l keeps z at chunks l + 64j as two fp16 halves
// z = hi + lo (hi = fp16(z), lo = fp16(z - hi), together about 22 significant bits), so
// W2 (fp16) . z runs on dot2 with exact products.
// UP: then the workgroup's active neurons (up to 32) get their activations in balanced rounds
// over its 4 waves; a is dense by neuron id with a neuron's NB tokens contiguous ([ffn][NB],
// NB the batch class 1/2/4/8). x is staged in LDS while the W2 rows
// are in flight (in column windows of width xw after the threshold when it does not fit).
// ---------------------------------------------------------------------------------------
// At 8 tokens without the activations the kernel is held to 4 waves per SIMD (124 instead of
// 136 VGPRs): OPT-175B Q4_0 stage 2 31.3 -> 30.1 us per layer on MI355X.
template <int NB, int CPL, bool UP, int WT, int ACT>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu((NB >= 8 && !UP) ? 4 : 1))) void k_stage2(LayerDev L, const float* __restrict__ z, int B,
                                                  uint64_t* __restrict__ mask_tok, uint64_t* __restrict__ mask_union,
                                                  float* __restrict__ logits, const void* __restrict__ x, int xw,
                                                  float* __restrict__ a) {
  constexpr int RPT = 8;  // rows per wave: one byte of the mask
  typedef typename XType<WT == W_F32>::T XT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ uint32_t s_bits[NWAVES];
  const int r = L.rank, nch = r >> 3;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int byte = wave * gridDim.x + blockIdx.x;  // this wave's byte of the mask
  const int row0 = byte * RPT;                      // its first neuron
  const uint8_t* w2 = reinterpret_cast<const uint8_t*>(L.p_w2);
  // A byte wholly inside the hot prefix reads no predictor rows: its loads all go to the
  // first row's first chunks (one cached line per lane) and are dropped. The loads stay
  // unconditional, so they are all in flight at once.
  const bool all_hot = row0 + RPT <= L.hot_prefix;
  u32x4 w[RPT][CPL];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + WAVE * j;
      const size_t off = all_hot ? (size_t)min(c, nch - 1) * 8 : (size_t)(row0 + i) * r + min(c, nch - 1) * 8;
      w[i][j] = ld_stream_or0(w2 + off * 2, c < nch && !all_hot);
    }
  // z as fp16 pairs hi + lo. At 8 tokens without the fused activations they are staged once
  // per workgroup in LDS ([NB][r/2] words each): in registers they took 128 VGPRs and left
  // room for 2 waves per SIMD. Otherwise each lane keeps its own chunks in registers.
  constexpr bool ZLDS = NB >= 8 && !UP;
  constexpr int ZR = ZLDS ? 1 : NB;
  uint32_t zh[ZR][CPL][4], zl[ZR][CPL][4];
  uint32_t* zsh = reinterpret_cast<uint32_t*>(smem);
  uint32_t* zsl = zsh + NB * (r >> 1);
  auto split = [](float f0, float f1, uint32_t& hi, uint32_t& lo) {
    const half_t h0 = (half_t)f0, h1 = (half_t)f1;
    const half_t l0 = (half_t)(f0 - (float)h0), l1 = (half_t)(f1 - (float)h1);
    hi = __builtin_bit_cast(uint32_t, (half2_t){h0, h1});
    lo = __builtin_bit_cast(uint32_t, (half2_t){l0, l1});
  };
  if constexpr (ZLDS) {
    constexpr int ZJ = 8 * 1024 / 4 / BLOCK;  // float4 groups per thread at the largest rank
    const int r4 = r >> 2, n4 = NB * r4;
    u32x4 v[ZJ];
#pragma unroll
    for (int k = 0; k < ZJ; ++k) {
      const int q = threadIdx.x + BLOCK * k;
      const int t = q / r4, c4 = q - t * r4;
      const bool ok = q < n4 && t < B;
      v[k] = ld16_or0(z + (ok ? (size_t)t * r + 4 * c4 : 0), ok);
    }
#pragma unroll
    for (int k = 0; k < ZJ; ++k) {
      const int q = threadIdx.x + BLOCK * k;
      if (q < n4) {
        const int t = q / r4, c4 = q - t * r4;
        const int o = t * (r >> 1) + 2 * c4;
        split(u2f(v[k][0]), u2f(v[k][1]), zsh[o], zsl[o]);
        split(u2f(v[k][2]), u2f(v[k][3]), zsh[o + 1], zsl[o + 1]);
      }
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int t = 0; t < ZR; ++t)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + WAVE * j;
        const bool ok = t < B && c < nch;
        const float* zp = z + (ok ? (size_t)t * r + c * 8 : 0);
        const u32x4 a0 = ld16_or0(zp, ok), a1 = ld16_or0(zp + 4, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f0 = u2f(e < 2 ? a0[2 * e] : a1[2 * e - 4]);
          const float f1 = u2f(e < 2 ? a0[2 * e + 1] : a1[2 * e - 3]);
          split(f0, f1, zh[t][j][e], zl[t][j][e]);
        }
      }
  }
  if constexpr (UP) {
    if (xw >= L.d) load_x_cols<NB, XT>(x, B, L.d, 0, L.d, xs, L.d);
  }
  const float bias = L.p_b[row0 + (lane & (RPT - 1))];
  uint32_t ubits = 0;
  const int W = L.ffn >> 6;
  uint8_t* mt = reinterpret_cast<uint8_t*>(mask_tok);
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    uint32_t hz[CPL][4], lz[CPL][4];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      if constexpr (ZLDS) {
        const int o = t * (r >> 1) + min(lane + WAVE * j, nch - 1) * 4;  // w is 0 past nch
        const u32x4 h4 = *reinterpret_cast<const u32x4*>(zsh + o);
        const u32x4 l4 = *reinterpret_cast<const u32x4*>(zsl + o);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hz[j][e] = h4[e];
          lz[j][e] = l4[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hz[j][e] = zh[t][j][e];
          lz[j][e] = zl[t][j][e];
        }
      }
    }
    float acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum = dot2(w[i][j][e], hz[j][e], sum);
          sum = dot2(w[i][j][e], lz[j][e], sum);
        }
      acc[i] = sum;
    }
    // hot-prefix neurons are always taken: decision value +inf (the reduction runs in every
    // lane: its shuffles need the whole wave)
    const float vr = transpose_reduce<RPT>(acc, lane) + bias;
    const float v = (row0 + (lane & (RPT - 1)) < L.hot_prefix) ? __builtin_inff() : vr;
    if (t < B) {
      const uint32_t bits = (uint32_t)__ballot(lane < RPT && v > L.threshold) & ((1u << RPT) - 1);
      ubits |= bits;
      if (logits != nullptr && lane < RPT) logits[(size_t)t * L.ffn + row0 + lane] = v;
      if (mask_tok != nullptr && lane == 0) mt[(size_t)t * W * 8 + byte] = (uint8_t)bits;
    }
  }
  if (lane == 0) reinterpret_cast<uint8_t*>(mask_union)[byte] = (uint8_t)ubits;
  if constexpr (UP) {
    if (lane == 0) s_bits[wave] = ubits;
    __syncthreads();
    const uint32_t cm = s_bits[0] | (s_bits[1] << 8) | (s_bits[2] << 16) | (s_bits[3] << 24);
    const int g = blockIdx.x, nwg = gridDim.x;
    auto id_of = [cm, g, nwg](int k) {
      const int j = select_bit((uint64_t)cm, k);
      return ((j >> 3) * nwg + g) * RPT + (j & 7);
    };
    const int xl = (xw >= L.d) ? L.d : xw;
    auto stage = [&](int c0, int cw) { load_x_cols<NB, XT>(x, B, L.d, c0, cw, xs, xl); };
    act_rounds<WT, ACT, NB, XT>(L, B, __popc(cm), id_of, xs, xl, xl, stage, a);
  }
}

// ---------------------------------------------------------------------------------------
// k_truemask: v = W x + b for the 64 neurons of this workgroup (W = up for ReLU, gate for
// ReGLU), then the mask epilogue. Each wave owns 16 rows; x (whole d) in LDS.
// UP: ReLU stores a = max(v, 0) of the active neurons directly; ReGLU reads their up rows.
// ---------------------------------------------------------------------------------------
template <int WT, int NB, bool XF32, bool UP>
__global__ __launch_bounds__(BLOCK) void k_truemask(LayerDev L, XIn xin, int B, uint64_t* __restrict__ mask_tok,
                                                    uint64_t* __restrict__ mask_union, float* __restrict__ logits,
                                                    float* __restrict__ a) {
  typedef typename XType<XF32>::T XT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ float red[2 * NWAVES];
  __shared__ float vs[NB][WAVE];
  __shared__ uint64_t s_union;
  const int d = L.d, ffn = L.ffn;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int tile = blockIdx.x;
  if (xin.y != nullptr) glue_x<NB, XT>(xin, B, d, xs, d, red, blockIdx.x == 0);
  else load_x_cols<NB, XT>(xin.x, B, d, 0, d, xs, d);
  __syncthreads();
  const uint8_t* W = (L.act == ACT_REGLU) ? L.w_gate : L.w_up;
  const uint16_t* S = (L.act == ACT_REGLU) ? L.s_gate : L.s_up;
  // Rows here are d long, so one full wave reduction per row costs little next to its loads.
#pragma unroll 1
  for (int i = 0; i < 16; i += 2) {
    const int row = tile * WAVE + wave * 16 + i;
    const uint8_t* const rows[2] = {row_ptr<WT>(W, row, d), row_ptr<WT>(W, row + 1, d)};
    const uint16_t* const srows[2] = {scale_ptr<WT>(S, row, d), scale_ptr<WT>(S, row + 1, d)};
    float acc[2][NB] = {};
    rows_dot<WT, NB, 2, (WT == W_Q4 ? 2 : 4), XT, 2>(rows, srows, xs, d, d, lane, acc);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float v0 = wave_sum(acc[0][t]) + L.b[row];
      const float v1 = wave_sum(acc[1][t]) + L.b[row + 1];
      if (lane == 0) {
        vs[t][wave * 16 + i] = v0;
        vs[t][wave * 16 + i + 1] = v1;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const uint64_t u = emit_mask<NB>(vs, tile, B, L.threshold, ffn, mask_tok, mask_union, logits);
    if constexpr (UP) {
      if (L.act != ACT_REGLU) {
        // a = act(h) for the union's neurons (a token's inactive neurons give 0)
        if ((u >> lane) & 1ull)
#pragma unroll
          for (int t = 0; t < NB; ++t)
            if (t < B) a[(size_t)(tile * WAVE + lane) * NB + t] = act_one_rt(L.act, vs[t][lane]);
      }
    }
    if (lane == 0) s_union = u;
  }
  if constexpr (UP) {
    if (L.act == ACT_REGLU) {
      __syncthreads();
      const uint64_t u = s_union;
      const int base = tile * WAVE;
      auto id_of = [u, base](int k) { return base + select_bit(u, k); };
      auto stage = [](int, int) {};
      act_rounds<WT, ACT_REGLU, NB, XT>(L, B, __popcll(u), id_of, xs, d, d, stage, a);
    }
  }
}

// k_threshold: mask words from given decision values v [B][ffn] (one wave per 64 neurons).
template <int NB>
__global__ __launch_bounds__(WAVE) void k_threshold(const float* __restrict__ v, int B, int ffn, float th,
                                                    uint64_t* __restrict__ mask_tok,
                                                    uint64_t* __restrict__ mask_union) {
  __shared__ float vs[NB][WAVE];
  const int tile = blockIdx.x, lane = threadIdx.x;
#pragma unroll
  for (int t = 0; t < NB; ++t) vs[t][lane] = (t < B) ? v[(size_t)t * ffn + tile * WAVE + lane] : 0.f;
  (void)emit_mask<NB>(vs, tile, B, th, ffn, mask_tok, mask_union, nullptr);
}

// ---------------------------------------------------------------------------------------
// Prefix scan of the W union words into LDS: wl[w] = word, pre[w] = set bits before word w,
// pre[W] = n. All threads of the block take part.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int scan_words(const uint64_t* __restrict__ words, int W, uint64_t* wl, int* pre,
                                          int* red) {
  int carry = 0;
  for (int w0 = 0; w0 < W; w0 += BLOCK) {
    const int w = w0 + threadIdx.x;
    const uint64_t word = (w < W) ? words[w] : 0ull;
    if (w < W) wl[w] = word;
    int total;
    const int ex = block_exclusive_scan(__popcll(word), red, &total);
    if (w < W) pre[w] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) pre[W] = carry;
  __syncthreads();
  return carry;
}

// The same scan with the first WPT * BLOCK words already loaded by the caller (wv[j] = word
// threadIdx.x + BLOCK * j, 0 past W), so their latency can overlap other loads.
template <int WPT>
__device__ __forceinline__ int scan_words_pre(const uint64_t (&wv)[WPT], const uint64_t* __restrict__ words, int W,
                                              uint64_t* wl, int* pre, int* red) {
  int carry = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    if (j * BLOCK >= W) break;
    const int w = j * BLOCK + threadIdx.x;
    if (w < W) wl[w] = wv[j];
    int total;
    const int ex = block_exclusive_scan(__popcll(wv[j]), red, &total);
    if (w < W) pre[w] = carry + ex;
    carry += total;
  }
  for (int w0 = WPT * BLOCK; w0 < W; w0 += BLOCK) {
    const int w = w0 + threadIdx.x;
    const uint64_t word = (w < W) ? words[w] : 0ull;
    if (w < W) wl[w] = word;
    int total;
    const int ex = block_exclusive_scan(__popcll(word), red, &total);
    if (w < W) pre[w] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) pre[W] = carry;
  __syncthreads();
  return carry;
}

// ---------------------------------------------------------------------------------------
// Compaction: ascending indices of the set bits of W union words. Workgroup g writes the
// indices of words [256g, 256g+256): it counts all earlier set bits itself (no inter-
// workgroup waiting), prefix-scans its own words and expands each word's bits in order.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(BLOCK) void k_compact(const uint64_t* __restrict__ words, int W,
                                                   int32_t* __restrict__ idx, int32_t* __restrict__ n_out,
                                                   int32_t* __restrict__ n_log) {
  __shared__ int red[NWAVES];
  const int g = blockIdx.x, tid = threadIdx.x;
  int before = 0;
  for (int w = tid; w < g * BLOCK; w += BLOCK) before += __popcll(words[w]);
  int total_before;
  (void)block_exclusive_scan(before, red, &total_before);
  const int w = g * BLOCK + tid;
  uint64_t word = (w < W) ? words[w] : 0ull;
  int total;
  int pos = total_before + block_exclusive_scan(__popcll(word), red, &total);
  while (word) {
    const int bit = __ffsll((unsigned long long)word) - 1;
    idx[pos++] = w * WAVE + bit;
    word &= word - 1;
  }
  if (g == (int)gridDim.x - 1 && tid == 0) {
    const int n = total_before + total;
    *n_out = n;
    if (n_log != nullptr) *n_log = n;
  }
}

// ---------------------------------------------------------------------------------------
// k_up (index-list entry point): a[t][i_k] = act(row_{i_k} . x_t) for k < n, with idx and n
// given by the caller (n clamped to [0, ffn], entries outside [0, ffn) skipped). a is dense
// by neuron id. Workgroup g takes the positions [CH*g, CH*g + CH), [CH*(g + grid), ...) in
// activation rounds (CH = 4 waves x PW); x is in LDS whole, or staged in column windows of
// width xw.
// ---------------------------------------------------------------------------------------
template <int WT, int ACT, int NB>
__global__ __launch_bounds__(BLOCK) void k_up(LayerDev L, const void* __restrict__ x, int B, int xw,
                                              const int32_t* __restrict__ idx_in, const int32_t* __restrict__ n_in,
                                              float* __restrict__ a) {
  typedef typename XType<WT == W_F32>::T XT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ int s_ids[NWAVES * ActPW<ACT>::PW];
  __shared__ int s_cnt;
  constexpr int CH = NWAVES * ActPW<ACT>::PW;
  const int ffn = L.ffn, d = L.d;
  const int n = min(max(*n_in, 0), ffn);
  const int xl = (xw >= d) ? d : xw;
  if (xw >= d) load_x_cols<NB, XT>(x, B, d, 0, d, xs, d);
  auto stage = [&](int c0, int cw) { load_x_cols<NB, XT>(x, B, d, c0, cw, xs, xl); };
  for (int k0 = blockIdx.x * CH; k0 < n; k0 += gridDim.x * CH) {
    // this chunk's valid entries, in order
    __syncthreads();
    if (threadIdx.x < WAVE) {
      const int k = k0 + threadIdx.x;
      const int i = (threadIdx.x < CH && k < n) ? idx_in[k] : -1;
      const bool ok = (unsigned)i < (unsigned)ffn;
      const uint64_t bal = __ballot(ok);
      if (ok) s_ids[__popcll(bal & ((1ull << threadIdx.x) - 1))] = i;
      if (threadIdx.x == 0) s_cnt = __popcll(bal);
    }
    __syncthreads();
    const int cnt = s_cnt;
    auto id_of = [](int k) { return s_ids[k]; };
    act_rounds<WT, ACT, NB, XT>(L, B, cnt, id_of, xs, xl, xl, stage, a);
  }
}

// ---------------------------------------------------------------------------------------
// k_up_cols: the gathered up (and gate) GEMV as a kernel of its own, over column slices of
// x when x would leave room for only one workgroup per CU in LDS (every workgroup of the
// fused kernels stages all of it). Workgroup (s, c) stages the columns [s*sw, s*sw + sw) of x once
// and takes the list positions [c*P, c*P + P), P = ceil(n / gridDim.y): for each of those
// neurons i and tokens t, the slice's partial pre-activation row_i[slice] . x_t goes to
// hp[s][r][t][i] (r = 0: the up row, or for ReGLU 0 = gate, 1 = up). k_act_fin adds the
// slices in order and applies the activation; with one slice (gridDim.x == 1) the kernel
// writes a itself, with the same arithmetic. The list is the union words' set bits in
// ascending order (words != nullptr) or the caller's index list (entries outside [0, ffn)
// skipped). Each partial is computed as in the fused kernels: the lane sums of its chunks,
// then the wave sum.
// ---------------------------------------------------------------------------------------
constexpr int UPC_PMAX = 512;  // list positions per workgroup

template <int WT, int ACT, int NB>
__global__ __launch_bounds__(BLOCK) void k_up_cols(LayerDev L, const void* __restrict__ x, int B, int sw,
                                                   const uint64_t* __restrict__ words,
                                                   const int32_t* __restrict__ idx_in,
                                                   const int32_t* __restrict__ n_in, float* __restrict__ hp,
                                                   float* __restrict__ a) {
  typedef typename XType<WT == W_F32>::T XT;
  constexpr int NR = (ACT == ACT_REGLU) ? 2 : 1;
  constexpr int PW = ActPW<ACT>::PW;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* xs = reinterpret_cast<XT*>(smem);                                         // [NB][sw]
  int* il = reinterpret_cast<int*>(smem + (size_t)NB * sw * sizeof(XT));        // [UPC_PMAX]
  __shared__ int red[NWAVES];
  __shared__ int s_cnt;
  const int d = L.d, ffn = L.ffn, W = ffn >> 6;
  const int s = blockIdx.x;
  const int cb = s * sw, cw = min(sw, d - cb);
  // the union words are loaded first, so their latency overlaps the staging of x
  constexpr int WPT = 4;
  uint64_t wv[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = j * BLOCK + threadIdx.x;
    wv[j] = (words != nullptr && w < W) ? words[w] : 0ull;
  }
  load_x_cols<NB, XT>(x, B, d, cb, cw, xs, sw);
  if (words != nullptr) {
    uint64_t* wl = reinterpret_cast<uint64_t*>(il + UPC_PMAX);  // [W]
    int* pre = reinterpret_cast<int*>(wl + W);                  // [W + 1]
    const int n = scan_words_pre<WPT>(wv, words, W, wl, pre, red);
    const int P = (n + gridDim.y - 1) / gridDim.y;
    const int lo = blockIdx.y * P, hi = min(min(n, lo + P), lo + UPC_PMAX);
    for (int w = threadIdx.x; w < W; w += BLOCK) {
      int pos = pre[w];
      if (pos >= hi || pre[w + 1] <= lo) continue;
      uint64_t word = wl[w];
      while (word) {
        if (pos >= lo && pos < hi) il[pos - lo] = w * WAVE + __ffsll((unsigned long long)word) - 1;
        ++pos;
        word &= word - 1;
      }
    }
    if (threadIdx.x == 0) s_cnt = max(0, hi - lo);
  } else {
    const int n = min(max(*n_in, 0), ffn);
    const int P = (n + gridDim.y - 1) / gridDim.y;
    const int lo = blockIdx.y * P, hi = min(min(n, lo + P), lo + UPC_PMAX);
    int carry = 0;
    for (int k0 = lo; k0 < hi; k0 += BLOCK) {
      const int k = k0 + threadIdx.x;
      const int i = (k < hi) ? idx_in[k] : -1;
      const bool ok = (unsigned)i < (unsigned)ffn;
      int total;
      const int ex = block_exclusive_scan(ok ? 1 : 0, red, &total);
      if (ok) il[carry + ex] = i;
      carry += total;
    }
    if (threadIdx.x == 0) s_cnt = carry;
  }
  __syncthreads();
  const int cnt = s_cnt;
  const int lane = threadIdx.x % WAVE;
  auto id_of = [il](int k) { return il[k]; };
  auto stage = [](int, int) {};
  const bool whole = gridDim.x == 1;
  auto out = [&](const int (&ids)[PW], int m, float (&acc)[ACT_RA][NB]) {
    if (whole) {
      act_store<ACT, NB>(L, B, lane, ids, m, acc, a);
      return;
    }
#pragma unroll
    for (int q = 0; q < PW; ++q) {
      if (q >= m) break;
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const float v = wave_sum(acc[NR * q + r][t]);
          if (lane == t && t < B) hp[(((size_t)s * NR + r) * B + t) * ffn + ids[q]] = v;
        }
    }
  };
  act_rounds_cols<WT, ACT, NB, XT>(L, cnt, id_of, xs, sw, cb, cb + cw, cw, stage, out);
}

// ---------------------------------------------------------------------------------------
// k_upq: the gathered up (and gate) GEMV on Q4_0 rows for 1..8 tokens, one workgroup of NTH
// threads per CU, over one column slice of x per workgroup. x is staged once
// per workgroup, each 16-byte piece of a block's 32 columns stored so that the 64 lanes of a
// wave, taking consecutive blocks, read consecutive 16-byte words (no LDS bank conflicts):
// piece m of local block b of token t sits at ((t * 4 + m) * 64 * SB + b) * 8 halves. The
// neurons are dealt out from the union words: at 1..2 tokens without a prefix scan, the
// workgroups of chunk c taking the 16-bit units c, c + NC, c + 2 NC, ... (unit u: bits
// 16 (u % 4) .. 16 (u % 4) + 15 of word u / 4), so the dense words of a hot-first layout
// spread over many workgroups; at 4..8 tokens evenly, every workgroup counting all the words
// (a few KB, from L2) and the workgroups of chunk c taking the active neurons of rank
// [c n / NC, (c + 1) n / NC), n the union's size, so that no workgroup needs a second round
// of rows while others idle (measured on MI355X at the OPT-175B shape: 8 tokens 70.0 ->
// 67.4 us; one token 13.7 -> 15.0 us, where the scan costs more than the balance saves).
// From an index list, positions c, c + NC, ... Lane l takes blocks l, l + 64, ... of the slice (SB
// of them); a wave takes RI neurons per round with every block of their rows in flight. Each
// (row, token) partial is the lane's blocks ascending, then the wave sum: one per (row,
// token) at 1..2 tokens, one transpose_reduce for all the round's sums at 4..8. With
// one slice (gridDim.x == 1) the kernel writes a itself, else the slice's partials go to
// hp[s][r][t][i] for k_act_fin (r = 0: up row; ReGLU: 0 = gate, 1 = up).
// ---------------------------------------------------------------------------------------
constexpr int UPQ_LIST = 1024;  // list entries per workgroup: NTH / 16 units of 16 bits, or NTH positions

// A buffer resource over `bytes` bytes at base (raw 32-bit data format): a load at an offset
// past `bytes` returns zeros and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t BUF_OOB = 0x80000000u;  // an offset past every resource here

template <int ACT, int NB, int SB, int RI, int NTH>
__global__ __launch_bounds__(NTH) void k_upq(LayerDev L, const half_t* __restrict__ x, int B,
                                             const uint64_t* __restrict__ words, int upw,
                                             const int32_t* __restrict__ idx_in, const int32_t* __restrict__ n_in,
                                             float* __restrict__ hp, float* __restrict__ a) {
  constexpr int NRW = (ACT == ACT_REGLU) ? 2 : 1;  // rows per neuron
  constexpr int SLB = WAVE * SB;                    // blocks per slice
  constexpr int NW = NTH / WAVE;
  static_assert(NTH <= UPQ_LIST, "one candidate per thread");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);                                 // [NB][4][SLB][8]
  int* il = reinterpret_cast<int*>(smem + (size_t)NB * 4 * SLB * 16);           // [NTH]
  uint64_t* wl = reinterpret_cast<uint64_t*>(il + NTH);                         // [W] union words
  __shared__ int wcnt[NW];
  const int d = L.d, ffn = L.ffn, W = ffn >> 6, nb = d >> 5;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int s = blockIdx.x, S = gridDim.x, ch = blockIdx.y, NC = gridDim.y;
  const int b0 = s * SLB;  // first block of the slice
  constexpr bool BAL = NB >= 4;  // even shares of the union (else units of 16 bits)
  // even shares: thread t counts the union words [t wpt, (t + 1) wpt)
  const int wpt = (W + NTH - 1) / NTH, w0 = threadIdx.x * wpt;
  int wc = 0;
  if (BAL && words != nullptr)
    for (int j = 0; j < wpt; ++j) {
      const uint64_t word = (w0 + j < W) ? words[w0 + j] : 0ull;
      if (w0 + j < W) wl[w0 + j] = word;
      wc += __popcll(word);
    }
  // units of 16 bits, or the index list: this thread's candidate neuron
  int cand = -1;
  if (!BAL && words != nullptr) {
    const int k = threadIdx.x >> 4, u = ch + NC * k;
    const bool uok = k < upw && u < 4 * W;
    const uint64_t word = uok ? words[u >> 2] : 0ull;
    const int bit = 16 * (u & 3) + (threadIdx.x & 15);
    if (uok && ((word >> bit) & 1ull)) cand = (u >> 2) * WAVE + bit;
  } else if (words == nullptr) {
    const int n = min(max(*n_in, 0), ffn);
    const int p = ch + NC * threadIdx.x;
    const int i = (p < n) ? idx_in[p] : -1;
    if ((unsigned)i < (unsigned)ffn) cand = i;
  }
  // x of the slice, swizzled (zeros past d and for tokens t >= B)
  for (int e = threadIdx.x; e < NB * 4 * SLB; e += NTH) {
    const int bl = e % SLB, m = (e / SLB) % 4, t = e / (4 * SLB);
    const int blk = b0 + bl;
    const bool ok = t < B && blk < nb;
    const u32x4 v = ld16_or0(x + (size_t)min(t, B - 1) * d + (size_t)min(blk, nb - 1) * 32 + 8 * m, ok);
    *reinterpret_cast<u32x4*>(xs + (size_t)((t * 4 + m) * SLB + bl) * 8) = v;
  }
  int cnt;
  if (BAL && words != nullptr) {
    // the union's ranks before this thread's words, and this workgroup's share of them
    int n;
    const int ex = block_exclusive_scan<NW>(wc, wcnt, &n);
    const int lo = (int)((long long)ch * n / NC), hi = (int)((long long)(ch + 1) * n / NC);
    cnt = hi - lo;  // <= ceil(ffn / NC) <= NTH (the launch's NC)
    if (ex < hi && ex + wc > lo) {
      int r = ex;
      for (int j = 0; j < wpt; ++j) {
        const int w = w0 + j;
        if (w >= W || r >= hi) break;
        uint64_t word = wl[w];
        const int pc = __popcll(word);
        if (r + pc <= lo) {
          r += pc;
          continue;
        }
        while (word) {
          if (r >= lo && r < hi) il[r - lo] = w * WAVE + __ffsll((unsigned long long)word) - 1;
          ++r;
          word &= word - 1;
        }
      }
    }
  } else {
    // candidates in thread order: ballot within the wave, wave counts through LDS
    const uint64_t bal = __ballot(cand >= 0);
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    cnt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      base += (w < wave) ? wcnt[w] : 0;
      cnt += wcnt[w];
    }
    if (cand >= 0) il[base + __popcll(bal & ((1ull << lane) - 1))] = cand;
  }
  __syncthreads();
  // the rows: codes and scales through bounds-checked buffer loads (a missing item or block
  // past d loads zeros without touching memory)
  __amdgpu_buffer_rsrc_t rw[NRW], rs[NRW];
#pragma unroll
  for (int r = 0; r < NRW; ++r) {
    const bool gate = ACT == ACT_REGLU && r == 0;
    rw[r] = buf_rsrc(gate ? L.w_gate : L.w_up, (uint32_t)((size_t)ffn * nb * 16));
    rs[r] = buf_rsrc(gate ? L.s_gate : L.s_up, (uint32_t)((size_t)ffn * nb * 2));
  }
  constexpr int STEP = NW * RI;
  auto load = [&](int k0, int (&ids)[RI], u32x4 (&w)[RI][NRW][SB], uint32_t (&sc)[RI][NRW][SB]) {
#pragma unroll
    for (int q = 0; q < RI; ++q) {
      const int k = k0 + NW * q;
      ids[q] = (k < cnt) ? il[k] : -1;
#pragma unroll
      for (int r = 0; r < NRW; ++r)
#pragma unroll
        for (int kb = 0; kb < SB; ++kb) {
          const int blk = b0 + lane + WAVE * kb;
          const bool ok = ids[q] >= 0 && blk < nb && lane + WAVE * kb < SLB;
          const uint32_t e = (uint32_t)ids[q] * (uint32_t)nb + (uint32_t)blk;
          w[q][r][kb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw[r], ok ? e * 16u : BUF_OOB, 0, 2));
          sc[q][r][kb] = __builtin_amdgcn_raw_buffer_load_b16(rs[r], ok ? e * 2u : BUF_OOB, 0, 0);
        }
    }
  };
  auto compute = [&](const int (&ids)[RI], const u32x4 (&w)[RI][NRW][SB], const uint32_t (&sc)[RI][NRW][SB]) {
    // the neurons' biases (wave-uniform loads), issued before the rows are needed
    float bq[RI];
#pragma unroll
    for (int q = 0; q < RI; ++q) bq[q] = (S == 1 && ids[q] >= 0) ? L.b[ids[q]] : 0.f;
    float acc[RI][NRW][NB];
#pragma unroll
    for (int q = 0; q < RI; ++q)
#pragma unroll
      for (int r = 0; r < NRW; ++r)
#pragma unroll
        for (int t = 0; t < NB; ++t) acc[q][r][t] = 0.f;
#pragma unroll
    for (int kb = 0; kb < SB; ++kb) {
      const int bl = lane + WAVE * kb;
      if (b0 + bl < nb) {
        // (q - 8) of every row's block as fp16 pairs, once for all tokens
        uint32_t wq[RI][NRW][16];
        float scf[RI][NRW];
#pragma unroll
        for (int q = 0; q < RI; ++q)
#pragma unroll
          for (int r = 0; r < NRW; ++r) {
            q4_block_unpack(w[q][r][kb], wq[q][r]);
            scf[q][r] = half_bits_to_float((uint16_t)sc[q][r][kb]);
          }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          uint32_t xv[16];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x4 qv = ld16(xs + (size_t)((t * 4 + m) * SLB + bl) * 8);
            xv[4 * m + 0] = qv[0];
            xv[4 * m + 1] = qv[1];
            xv[4 * m + 2] = qv[2];
            xv[4 * m + 3] = qv[3];
          }
#pragma unroll
          for (int q = 0; q < RI; ++q)
#pragma unroll
            for (int r = 0; r < NRW; ++r) {
              float sm = 0.f;
#pragma unroll
              for (int e = 0; e < 16; ++e) sm = dot2(wq[q][r][e], xv[e], sm);
              acc[q][r][t] = fmaf(scf[q][r], sm, acc[q][r][t]);
            }
        }
      }
    }
    if constexpr (NB <= 2) {
      // one wave sum per (row, token): at 1..2 tokens this measured faster than the joint
      // reduction below (OPT-175B shape, one token: 13.8 against 15.2 us per layer)
#pragma unroll
      for (int q = 0; q < RI; ++q) {
        if (ids[q] < 0) break;
        const int i = ids[q];
        if (S == 1) {
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            float o;
            if constexpr (ACT != ACT_REGLU) {
              o = act_one<ACT>(wave_sum(acc[q][0][t]) + bq[q]);
            } else {
              const float g = wave_sum(acc[q][0][t]) + bq[q];
              const float u = wave_sum(acc[q][1][t]);
              o = fmaxf(g, 0.f) * u;
            }
            if (lane == t && t < B) a[(size_t)i * NB + t] = o;
          }
        } else {
#pragma unroll
          for (int r = 0; r < NRW; ++r)
#pragma unroll
            for (int t = 0; t < NB; ++t) {
              const float o = wave_sum(acc[q][r][t]);
              if (lane == t && t < B) hp[(((size_t)s * NRW + r) * B + t) * ffn + i] = o;
            }
        }
      }
      return;
    }
    // the RI x NRW x NB lane sums, reduced over the wave together: afterwards lane k < RR holds
    // value k = (q * NRW + r) * NB + t
    constexpr int RR = RI * NRW * NB;
    float fl[RR];
#pragma unroll
    for (int q = 0; q < RI; ++q)
#pragma unroll
      for (int r = 0; r < NRW; ++r)
#pragma unroll
        for (int t = 0; t < NB; ++t) fl[(q * NRW + r) * NB + t] = acc[q][r][t];
    const float v = transpose_reduce<RR>(fl, lane);
    // ReGLU: the up sum of the same neuron and token sits NB lanes further on
    const float vu = (NRW == 2) ? __shfl(v, min(lane + NB, WAVE - 1), WAVE) : 0.f;
    const int kq = lane / (NRW * NB), kr = (lane / NB) % NRW, kt = lane % NB;
    int iq = -1;
    float bias = 0.f;
#pragma unroll
    for (int q = 0; q < RI; ++q) {
      iq = (q == kq) ? ids[q] : iq;
      bias = (q == kq) ? bq[q] : bias;
    }
    if (lane < RR && iq >= 0 && kt < B) {
      if (S == 1) {
        if (kr == 0) {
          float o;
          if constexpr (ACT != ACT_REGLU) o = act_one<ACT>(v + bias);
          else o = fmaxf(v + bias, 0.f) * vu;
          a[(size_t)iq * NB + kt] = o;
        }
      } else {
        hp[(((size_t)s * NRW + kr) * B + kt) * ffn + iq] = v;
      }
    }
  };
  for (int k0 = wave; k0 < cnt; k0 += STEP) {
    int ids[RI];
    u32x4 w[RI][NRW][SB];
    uint32_t sc[RI][NRW][SB];
    load(k0, ids, w, sc);
    compute(ids, w, sc);
  }
}

// a[t][i] = act(h + b_i) with h = the S slice partials of k_up_cols added in slice order
// (ReGLU: max(h_gate + b_i, 0) * h_up), for the active neurons: the set bits of the union
// words (thread k takes neuron k), or the index list (thread k takes entry k < n).
template <int ACT>
__global__ __launch_bounds__(BLOCK) void k_act_fin(LayerDev L, int B, int S, const float* __restrict__ hp,
                                                   const uint64_t* __restrict__ words,
                                                   const int32_t* __restrict__ idx_in,
                                                   const int32_t* __restrict__ n_in, float* __restrict__ a) {
  constexpr int NR = (ACT == ACT_REGLU) ? 2 : 1;
  const int ffn = L.ffn;
  const int k = blockIdx.x * BLOCK + threadIdx.x;
  int i;
  if (words != nullptr) {
    if (k >= ffn || !((words[k >> 6] >> (k & 63)) & 1ull)) return;
    i = k;
  } else {
    if (k >= min(max(*n_in, 0), ffn)) return;
    i = idx_in[k];
    if ((unsigned)i >= (unsigned)ffn) return;
  }
  const float bias = L.b[i];
  const int nb = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8;  // a's token stride: the batch class
  for (int t = 0; t < B; ++t) {
    float h = 0.f, u = 0.f;
    for (int s = 0; s < S; ++s) {
      h += hp[(((size_t)s * NR) * B + t) * ffn + i];
      if constexpr (NR == 2) u += hp[(((size_t)s * NR + 1) * B + t) * ffn + i];
    }
    float v;
    if constexpr (ACT == ACT_REGLU) v = fmaxf(h + bias, 0.f) * u;
    else v = act_one<ACT>(h + bias);
    a[(size_t)i * nb + t] = v;
  }
}

// ---------------------------------------------------------------------------------------
// k_down_part: part[g][t][c] = sum over the active neurons i of group g of a[t][i] *
// w_down_t[i][c]. Group g holds the neurons of mask words w = g, g + G, g + 2G, ... (words
// dealt out in turn, so a hot-first layout still spreads its hot words over the groups), in
// ascending order. The grid is G groups x S column slices (block = g + G * s); a slice is
// SEG lanes of EPC columns each; the workgroup's 256 threads form 256/SEG neuron slots with
// U rows in flight each, summed in a fixed order. The G partial sums are added later in
// group order (by k_reduce, or by the next layer's glue), so y does not depend on
// scheduling. (Adding them here, in the last workgroup of each slice, needs a device-scope
// release per workgroup: an L2 write-back that costs far more than the separate pass.)
//  SCAN: the group's neurons come from the union words (no workgroup needs the others'
//        counts). One extra workgroup (block 0, dispatched first, so it never waits for a
//        slot behind a full round of the others) prefix-scans all the words and writes the
//        ascending index list idx and n.
//  else: the given index list, filtered to the group's words in list order (an ascending
//        list gives the same group lists, hence the same y, as SCAN).
// tok_mask != nullptr (per-token masking, SCAN only): a[t][i] counts only where bit i of
// token t's mask words tok_mask[t][ffn/64] is set; the scan keeps each listed neuron's token
// bits next to it in LDS.
// Q4_0 rows (1..2 tokens here; 4..8 take k_down_q4x): a lane takes a whole block (16 code
// bytes, 32 columns), SQ lanes a slice.
// ---------------------------------------------------------------------------------------
// v of lane j of this lane's quad (DPP quad permutation; the quad's lanes must be active).
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int j) {
  const int x = (int)v;
  switch (j) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xFF, 0xF, 0xF, false);
  }
}

// SQ: lanes per slice (Q4_0; fp16/fp32 rows take 8 unless SQ asks for more).
template <int WT, int SQ = 4> struct DownGeom {
  static constexpr int EPC = (WT == W_F16) ? 8 : (WT == W_F32) ? 4 : 32;  // columns per lane
  static constexpr int SEG = (WT == W_Q4) ? SQ : (SQ > 8 ? SQ : 8);           // lanes per slice
  static constexpr int SW = SEG * EPC;                                         // slice width (columns)
};

// Capacity of a group's neuron list (ints in LDS): every neuron of its words.
__host__ __device__ constexpr int down_list_cap(int W, int G) { return (W + G - 1) / G * 64; }

// The compaction block of the down kernels: the ascending index list idx and its length n of
// the union words (smem: the words, then their exclusive prefix counts).
__device__ __forceinline__ void down_compact(const uint64_t* __restrict__ words, int W, uint8_t* smem, int* red,
                                             int32_t* __restrict__ idx_out, int32_t* __restrict__ n_out,
                                             int32_t* __restrict__ n_log) {
  uint64_t* wl = reinterpret_cast<uint64_t*>(smem);
  int* pre = reinterpret_cast<int*>(wl + W);
  const int n = scan_words(words, W, wl, pre, red);
  for (int w = threadIdx.x; w < W; w += BLOCK) {
    uint64_t word = wl[w];
    int pos = pre[w];
    while (word) {
      idx_out[pos++] = w * WAVE + __ffsll((unsigned long long)word) - 1;
      word &= word - 1;
    }
  }
  if (threadIdx.x == 0) {
    *n_out = n;
    if (n_log != nullptr) *n_log = n;
  }
}

// Group g's neurons in ascending order into il (per-token masking: each one's token bits into
// tb) and their count, which every thread gets back (a barrier inside).
//  SCAN: from the union words w = g, g + G, ... (a block-wide pass per 256 words).
//  else: the given list, filtered to the group's words, in list order.
template <int NB, bool SCAN, int G>
__device__ __forceinline__ int down_group_list(int g, int B, int W, int ffn, const uint64_t* __restrict__ words,
                                               const int32_t* __restrict__ idx_in, const int32_t* __restrict__ n_in,
                                               const uint64_t* __restrict__ tok_mask, int* il, uint8_t* tb, int* red,
                                               int* s_ng) {
  if constexpr (SCAN) {
    const int nwg = (W - g + G - 1) / G;
    int carry = 0;
    for (int q0 = 0; q0 < nwg; q0 += BLOCK) {
      const int q = q0 + threadIdx.x;
      const int w = g + G * q;
      uint64_t word = (q < nwg) ? words[w] : 0ull;
      uint64_t tw[NB];
#pragma unroll
      for (int t = 0; t < NB; ++t) tw[t] = (tok_mask != nullptr && q < nwg && t < B) ? tok_mask[(size_t)t * W + w] : 0ull;
      int total;
      int pos = carry + block_exclusive_scan(__popcll(word), red, &total);
      while (word) {
        const int bit = __ffsll((unsigned long long)word) - 1;
        if (tok_mask != nullptr) {
          uint32_t bits = 0;
#pragma unroll
          for (int t = 0; t < NB; ++t) bits |= (uint32_t)((tw[t] >> bit) & 1ull) << t;
          tb[pos] = (uint8_t)bits;
        }
        il[pos++] = w * WAVE + bit;
        word &= word - 1;
      }
      carry += total;
    }
    if (threadIdx.x == 0) *s_ng = carry;
  } else {
    const int n = min(max(*n_in, 0), ffn);
    const int cap = down_list_cap(W, G);
    int carry = 0;
    for (int k0 = 0; k0 < n; k0 += BLOCK) {
      const int k = k0 + threadIdx.x;
      const int i = (k < n) ? idx_in[k] : -1;
      const bool mine = (unsigned)i < (unsigned)ffn && ((i >> 6) & (G - 1)) == g;
      int total;
      const int ex = block_exclusive_scan(mine ? 1 : 0, red, &total);
      if (mine && carry + ex < cap) il[carry + ex] = i;
      carry += total;
    }
    if (threadIdx.x == 0) *s_ng = min(carry, cap);
  }
  __syncthreads();
  return *s_ng;
}

// Sum the NSL slots of each of the slice's SW columns in a fixed order and store the group's
// partial part[g][t][col] for the B tokens. col_of(e) is the slice column of this lane's
// element e. The slots' sums [NSL][SW + 1] take the LDS of the neuron list, which no thread
// reads any more after the first barrier.
template <int NB, int EPC, int SW, int NSL, class ColOf>
__device__ __forceinline__ void down_store(uint8_t* smem, const float (&acc)[NB][EPC], ColOf col_of, int B, int g,
                                           int s, int d, int slot, float* __restrict__ part) {
  float (*s_red)[SW + 1] = reinterpret_cast<float (*)[SW + 1]>(smem);
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if (t >= B) break;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPC; ++e) s_red[slot][col_of(e)] = acc[t][e];
    __syncthreads();
    for (int c = threadIdx.x; c < SW; c += BLOCK) {
      const int col = s * SW + c;
      if (col < d) {
        float v = 0.f;
        for (int q = 0; q < NSL; ++q) v += s_red[q][c];
        part[((size_t)g * B + t) * d + col] = v;
      }
    }
  }
}

// k_down_q4x: the down projection of Q4_0 rows at 4..8 tokens, with k_down_part's groups,
// lists, compaction block and partial sums. A slice is 4 blocks (128 columns); the 4 lanes of
// a block's quad take 4 code bytes each (elements 4j..4j+3 and 16+4j..16+4j+3 of the block)
// and NB/4 of the tokens, whose a * s they form and share over the quad (DPP). Neurons are
// taken two at a time: each column's two (q - 8) make an exact fp16 pair, multiplied by the
// fp16 pair of the two a * s with dot2 (fp32 accumulation), one instruction per two weights
// and token. Rounds of U list items per slot are software-pipelined: the loads of the next
// round are issued before the products of this one. All loads are buffer loads: an item past
// the list's end (or a slice past d) reads past its resource and gets zeros, so no load sits
// under a branch.
template <int NB, bool SCAN, int G, int U>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(NB >= 8 ? 3 : 1))) void k_down_q4x(
    LayerDev L, int B, const uint64_t* __restrict__ words, const int32_t* __restrict__ idx_in,
    const int32_t* __restrict__ n_in, const float* __restrict__ a, const uint64_t* __restrict__ tok_mask,
    float* __restrict__ part, int32_t* __restrict__ idx_out, int32_t* __restrict__ n_out, int32_t* __restrict__ n_log) {
  static_assert(NB == 4 || NB == 8, "4 or 8 tokens");
  static_assert(U % 2 == 0, "items are taken in pairs");
  static_assert(G >= 1 && (G & (G - 1)) == 0, "the group count is a power of two");
  constexpr int SEG = 16, EPC = 8, SW = 128, NSL = BLOCK / SEG, TPL = NB / 4, R = NSL * U;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int red[NWAVES];
  __shared__ int s_ng;
  const int d = L.d, ffn = L.ffn, W = ffn >> 6, nbr = d >> 5;
  int* il = reinterpret_cast<int*>(smem);
  uint8_t* tb = reinterpret_cast<uint8_t*>(il + down_list_cap(W, G));
  if constexpr (SCAN) {
    if (blockIdx.x == 0) {  // the compaction block (dispatched first)
      down_compact(words, W, smem, red, idx_out, n_out, n_log);
      return;
    }
  }
  const int bid = SCAN ? (int)blockIdx.x - 1 : (int)blockIdx.x;
  const int g = bid % G, s = bid / G;
  const int slot = threadIdx.x / SEG, sl = threadIdx.x % SEG, qd = sl & 3;
  const int cb = s * (SW / 32) + (sl >> 2);  // this lane's block within a row
  const bool valid = cb < nbr;
  const int ng = down_group_list<NB, SCAN, G>(g, B, W, ffn, words, idx_in, n_in, tok_mask, il, tb, red, &s_ng);
  const auto rw = buf_rsrc(L.w_down_t, (uint32_t)((size_t)ffn * nbr * 16));
  const auto rs = buf_rsrc(L.s_down, (uint32_t)((size_t)ffn * nbr * 2));
  const auto ra = buf_rsrc(a, (uint32_t)((size_t)ffn * NB * 4));
  float acc[NB][EPC];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[t][e] = 0.f;
  // one round's operands: code dword, scale bits, this lane's tokens' a, token bits
  struct Round {
    uint32_t c[U];
    uint32_t sh[U];
    uint32_t av[U][TPL];
    uint32_t tbits[U];
  };
  auto load = [&](int j0, Round& r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + NSL * u;
      const bool in = j < ng;
      const uint32_t i = in ? (uint32_t)il[j] : 0u;
      const uint32_t blk = i * (uint32_t)nbr + (uint32_t)cb;
      const bool ok = in && valid;
      r.c[u] = __builtin_amdgcn_raw_buffer_load_b32(rw, ok ? blk * 16u + qd * 4u : BUF_OOB, 0, 2);
      r.sh[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? blk * 2u : BUF_OOB, 0, 0);
      const uint32_t ao = in ? (i * NB + TPL * qd) * 4u : BUF_OOB;
      if constexpr (TPL == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(ra, ao, 0, 0);
        r.av[u][0] = v[0];
        r.av[u][1] = v[1];
      } else {
        r.av[u][0] = __builtin_amdgcn_raw_buffer_load_b32(ra, ao, 0, 0);
      }
      r.tbits[u] = (SCAN && tok_mask != nullptr && in) ? tb[j] : 0xFFu;
    }
  };
  auto compute = [&](const Round& r) {
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      const uint32_t cu = r.c[u], cv = r.c[u + 1];
      const uint32_t lu = cu & 0x0F0F0F0Fu, lv = cv & 0x0F0F0F0Fu;
      const uint32_t hu = (cu >> 4) & 0x0F0F0F0Fu, hv = (cv >> 4) & 0x0F0F0F0Fu;
      // byte k of u next to byte k of v: elements 4j+k (low nibbles), 16+4j+k (high)
      const uint32_t l01 = __builtin_amdgcn_perm(lv, lu, 0x05010400u), l23 = __builtin_amdgcn_perm(lv, lu, 0x07030602u);
      const uint32_t h01 = __builtin_amdgcn_perm(hv, hu, 0x05010400u), h23 = __builtin_amdgcn_perm(hv, hu, 0x07030602u);
      uint32_t pr[8];
      pr[0] = q4_pair(l01, SEL_B01);
      pr[1] = q4_pair(l01, SEL_B23);
      pr[2] = q4_pair(l23, SEL_B01);
      pr[3] = q4_pair(l23, SEL_B23);
      pr[4] = q4_pair(h01, SEL_B01);
      pr[5] = q4_pair(h01, SEL_B23);
      pr[6] = q4_pair(h23, SEL_B01);
      pr[7] = q4_pair(h23, SEL_B23);
      const float su = half_bits_to_float((uint16_t)r.sh[u]), sv = half_bits_to_float((uint16_t)r.sh[u + 1]);
      // this lane's tokens' fp16 pairs of a * s (a token counts only where its bit is set and
      // it is one of the B), then every token's pair from its quad lane
      uint32_t pp[TPL];
#pragma unroll
      for (int h = 0; h < TPL; ++h) {
        const int t = TPL * qd + h;
        const float au = (t < B && ((r.tbits[u] >> t) & 1u)) ? u2f(r.av[u][h]) : 0.f;
        const float bv = (t < B && ((r.tbits[u + 1] >> t) & 1u)) ? u2f(r.av[u + 1][h]) : 0.f;
        pp[h] = __builtin_bit_cast(uint32_t, (half2_t){(half_t)(au * su), (half_t)(bv * sv)});
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const uint32_t ap = quad_bcast(pp[t % TPL], t / TPL);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = dot2(pr[e], ap, acc[t][e]);
      }
    }
  };
  // two rounds in flight: load the next while forming this one's products
  Round r0, r1;
  int j0 = slot;
  load(j0, r0);
  while (j0 < ng) {
    load(j0 + R, r1);
    compute(r0);
    j0 += R;
    if (j0 >= ng) break;
    load(j0 + R, r0);
    compute(r1);
    j0 += R;
  }
  down_store<NB, EPC, SW, NSL>(smem, acc, [&](int e) { return (sl >> 2) * 32 + 4 * qd + (e < 4 ? e : 12 + e); },
                               B, g, s, d, slot, part);
}

template <int WT, int NB, bool SCAN, int U, int G, int SQ = 4>
__global__ __launch_bounds__(BLOCK) void k_down_part(LayerDev L, int B, const uint64_t* __restrict__ words,
                                                     const int32_t* __restrict__ idx_in,
                                                     const int32_t* __restrict__ n_in, const float* __restrict__ a,
                                                     const uint64_t* __restrict__ tok_mask,
                                                     float* __restrict__ part, int32_t* __restrict__ idx_out,
                                                     int32_t* __restrict__ n_out, int32_t* __restrict__ n_log) {
  static_assert(G >= 1 && (G & (G - 1)) == 0, "the group count is a power of two");
  static_assert(WT != W_Q4 || NB <= 2, "Q4_0 rows at 4..8 tokens take k_down_q4x");
  constexpr int EPC = DownGeom<WT, SQ>::EPC;
  constexpr int SEG = DownGeom<WT, SQ>::SEG;
  constexpr int SW = SEG * EPC;
  constexpr int NSL = BLOCK / SEG;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int red[NWAVES];
  __shared__ int s_ng;
  const int d = L.d, ffn = L.ffn, W = ffn >> 6;
  int* il = reinterpret_cast<int*>(smem);  // the group's neurons [down_list_cap(W, G)]
  // per-token masking: bit t of tb[j] = token t's mask bit of neuron il[j]
  uint8_t* tb = reinterpret_cast<uint8_t*>(il + down_list_cap(W, G));
  if constexpr (SCAN) {
    if (blockIdx.x == 0) {  // the compaction block (dispatched first)
      down_compact(words, W, smem, red, idx_out, n_out, n_log);
      return;
    }
  }
  const int bid = SCAN ? (int)blockIdx.x - 1 : (int)blockIdx.x;  // SCAN: block 0 compacts
  const int g = bid % G, s = bid / G;
  const int slot = threadIdx.x / SEG, sl = threadIdx.x % SEG;
  const int col0 = s * SW + sl * EPC;  // the first column this lane touches
  const bool valid = col0 < d;
  const int ng = down_group_list<NB, SCAN, G>(g, B, W, ffn, words, idx_in, n_in, tok_mask, il, tb, red, &s_ng);
  float acc[NB][EPC];
  float qsum[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    qsum[t] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[t][e] = 0.f;
  }
  // Rounds of U list items per slot, all their row pieces in flight. At 4..8 tokens a missing
  // item (past the list's end) still issues its loads, from item 0's row, and drops them: with
  // the loads under a branch the compiler waits for each one inside it (measured on MI355X
  // when this kernel still took Q4_0 rows at 8 tokens: OPT-175B 77 -> 55 us per layer). At
  // 1..2 tokens the branch is faster.
  constexpr bool FULL = NB >= 4;
  for (int j0 = slot; j0 < ng; j0 += NSL * U) {
    int ii[U];
    uint32_t tbits[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + NSL * u;
      ii[u] = (j < ng) ? il[j] : -1;
      tbits[u] = (SCAN && tok_mask != nullptr && j < ng) ? tb[j] : 0xFFu;
    }
    // activations first (small, likely cached; a neuron's NB tokens are contiguous), then the rows
    float av[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* ap = a + (size_t)(ii[u] >= 0 ? ii[u] : 0) * NB;
      if constexpr (NB >= 4) {
#pragma unroll
        for (int t4 = 0; t4 < NB; t4 += 4) {
          const u32x4 v4 = ld16(ap + t4);  // zeroed below where ii[u] < 0
#pragma unroll
          for (int e = 0; e < 4; ++e) av[u][t4 + e] = u2f(v4[e]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < NB; ++t) av[u][t] = ap[t];  // zeroed below where ii[u] < 0
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        // tokens past B hold no value; per-token masking: token t takes neuron i only if its
        // own mask has it
        const bool on = ii[u] >= 0 && t < B && ((tbits[u] >> t) & 1u);
        av[u][t] = on ? av[u][t] : 0.f;
      }
    }
    u32x4 w[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w[u] = (u32x4){0, 0, 0, 0};
      sc[u] = 0.f;
      const bool ok = ii[u] >= 0 && valid;
      if (FULL || ok) {
        const size_t iu = (size_t)(ii[u] >= 0 ? ii[u] : ii[0]);
        const int cv = valid ? col0 : 0;
        if constexpr (WT == W_F16) w[u] = ld_stream_or0(L.w_down_t + (iu * d + cv) * 2, ok);
        else if constexpr (WT == W_F32) w[u] = ld_stream_or0(L.w_down_t + (iu * d + cv) * 4, ok);
        else {
          const size_t blk = iu * (d >> 5) + (cv >> 5);
          w[u] = ld_stream_or0(L.w_down_t + blk * 16, ok);
          const float sv = half_bits_to_float(L.s_down[blk]);
          sc[u] = ok ? sv : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ii[u] < 0) continue;
      if constexpr (WT == W_F16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = h2f_lo(w[u][e]), hi = h2f_hi(w[u][e]);
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            acc[t][2 * e] = fmaf(av[u][t], lo, acc[t][2 * e]);
            acc[t][2 * e + 1] = fmaf(av[u][t], hi, acc[t][2 * e + 1]);
          }
        }
      } else if constexpr (WT == W_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int t = 0; t < NB; ++t) acc[t][e] = fmaf(av[u][t], u2f(w[u][e]), acc[t][e]);
      } else {
        float q[32];
        q4_block_codes(w[u], q);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const float as = av[u][t] * sc[u];
          qsum[t] += as;
#pragma unroll
          for (int e = 0; e < 32; ++e) acc[t][e] = fmaf(q[e], as, acc[t][e]);
        }
      }
    }
  }
  if constexpr (WT == W_Q4) {
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[t][e] = fmaf(-8.f, qsum[t], acc[t][e]);
  }
  down_store<NB, EPC, SW, NSL>(smem, acc, [&](int e) { return sl * EPC + e; }, B, g, s, d, slot, part);
}

// y[i] = sum_{g < G} part[g][i] over i < BD = B*d, groups summed in order (G <= 64). A
// workgroup covers 64 outputs; its 4 waves each sum every 4th group with all loads in flight,
// then the four wave sums are added in a fixed order.
__global__ __launch_bounds__(BLOCK) void k_reduce(const float* __restrict__ part, int G, int BD, float* __restrict__ y) {
  __shared__ float s4[NWAVES][WAVE];
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int i = blockIdx.x * WAVE + lane;
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int gg = wave + NWAVES * j;
    v[j] = (i < BD && gg < G) ? part[(size_t)gg * BD + i] : 0.f;
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) sum += v[j];
  s4[wave][lane] = sum;
  __syncthreads();
  if (wave == 0 && i < BD) y[i] = (s4[0][lane] + s4[1][lane]) + (s4[2][lane] + s4[3][lane]);
}

// Standalone glue: one workgroup per token, d % 4 == 0: u = y - c (c nullable), x_out =
// round(u / sqrt(mean(u^2))), or x_prev when y or u is all zero. Each thread issues all of
// its 16-byte loads of y and c (up to GLUE_J each) before using them; longer rows take
// further passes.
template <bool XF32>
__global__ __launch_bounds__(BLOCK) void k_glue(const float* __restrict__ y, const float* __restrict__ center,
                                                const void* __restrict__ x_prev, int d, void* __restrict__ x_out) {
  typedef typename XType<XF32>::T XT;
  __shared__ float red[2 * NWAVES];
  const int t = blockIdx.x;
  const float* yt = y + (size_t)t * d;
  const int n4 = d >> 2;
  auto load = [&](int c0, u32x4 (&v)[GLUE_J], u32x4 (&cv)[GLUE_J]) {
#pragma unroll
    for (int j = 0; j < GLUE_J; ++j) {
      const int c = c0 + threadIdx.x + BLOCK * j;
      v[j] = ld16_or0(yt + 4 * min(c, n4 - 1), c < n4);
      cv[j] = center != nullptr ? ld16_or0(center + 4 * min(c, n4 - 1), c < n4) : (u32x4){0, 0, 0, 0};
    }
  };
  float ss = 0.f, su = 0.f;
  for (int c0 = 0; c0 < n4; c0 += BLOCK * GLUE_J) {
    u32x4 v[GLUE_J], cv[GLUE_J];
    load(c0, v, cv);
#pragma unroll
    for (int j = 0; j < GLUE_J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float yv = u2f(v[j][e]), uv = yv - u2f(cv[j][e]);
        ss = fmaf(yv, yv, ss);
        su = fmaf(uv, uv, su);
      }
  }
  block_sum2(ss, su, red);
  const float r = glue_divisor(ss, su, d);
  const XT* xp = reinterpret_cast<const XT*>(x_prev) + (size_t)t * d;
  XT* xo = reinterpret_cast<XT*>(x_out) + (size_t)t * d;
  if (r == 0.f) {  // all-zero y: x passes through (r is the same in every thread)
    for (int c = threadIdx.x; c < d; c += BLOCK) xo[c] = xp[c];
    return;
  }
  for (int c0 = 0; c0 < n4; c0 += BLOCK * GLUE_J) {
    u32x4 v[GLUE_J], cv[GLUE_J];
    load(c0, v, cv);
#pragma unroll
    for (int j = 0; j < GLUE_J; ++j) {
      const int c = c0 + threadIdx.x + BLOCK * j;
      if (c < n4)
#pragma unroll
        for (int e = 0; e < 4; ++e) xo[4 * c + e] = (XT)((u2f(v[j][e]) - u2f(cv[j][e])) / r);
    }
  }
}

// k_glue_parts: the glue between stacked layers at 2..8 tokens, straight from the previous
// layer's G partial sums: workgroup t (GLUE_NTH threads) adds token t's partials in group
// order, u = y - c, and stores x = round(u / sqrt(mean(u^2))) (x_prev where y or u is all
// zero). Each thread keeps its J chunks of 4 columns in registers between the sums of
// squares and the store (d <= 4 * GLUE_NTH * J).
constexpr int GLUE_NTH = 1024;
template <int G, int J, bool XF32>
__global__ __launch_bounds__(GLUE_NTH) void k_glue_parts(const float* __restrict__ part, int gstride,
                                                         const float* __restrict__ center,
                                                         const void* __restrict__ x_prev, int d,
                                                         void* __restrict__ x_out) {
  typedef typename XType<XF32>::T XT;
  constexpr int NW = GLUE_NTH / WAVE;
  // partials in flight per chunk: J * GU <= 16 loads of 16 bytes per thread at a time (more
  // would not fit the 128 registers of a 1024-thread workgroup)
  constexpr int GU = (J >= 3 ? 4 : 8) < G ? (J >= 3 ? 4 : 8) : G;
  __shared__ float red[2 * NW];
  const int t = blockIdx.x, n4 = d >> 2;
  const float* pt = part + (size_t)t * d;
  f32x4 u[J];
  float ss = 0.f, su = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) u[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int g0 = 0; g0 < G; g0 += GU) {
    u32x4 p[J][GU];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = threadIdx.x + GLUE_NTH * j;
      const size_t off = 4 * (size_t)min(c, n4 - 1);
#pragma unroll
      for (int k = 0; k < GU; ++k) p[j][k] = ld16_or0(pt + (size_t)(g0 + k) * gstride + off, c < n4);
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int k = 0; k < GU; ++k) u[j] += __builtin_bit_cast(f32x4, p[j][k]);
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = threadIdx.x + GLUE_NTH * j;
    const u32x4 cv = center != nullptr ? ld16_or0(center + 4 * (size_t)min(c, n4 - 1), c < n4) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float yv = u[j][e];
      u[j][e] = yv - u2f(cv[e]);
      ss = fmaf(yv, yv, ss);
      su = fmaf(u[j][e], u[j][e], su);
    }
  }
  // block sums of both squares (fixed order)
  ss = wave_sum(ss);
  su = wave_sum(su);
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  if (lane == 0) {
    red[w] = ss;
    red[NW + w] = su;
  }
  __syncthreads();
  ss = 0.f;
  su = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    ss += red[i];
    su += red[NW + i];
  }
  const float r = glue_divisor(ss, su, d);
  const XT* xp = reinterpret_cast<const XT*>(x_prev) + (size_t)t * d;
  XT* xo = reinterpret_cast<XT*>(x_out) + (size_t)t * d;
  if (r == 0.f) {  // all-zero y or u: x passes through (r is the same in every thread)
    for (int c = threadIdx.x; c < d; c += GLUE_NTH) xo[c] = xp[c];
    return;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = threadIdx.x + GLUE_NTH * j;
    if (c < n4)
#pragma unroll
      for (int e = 0; e < 4; ++e) xo[4 * c + e] = (XT)(u[j][e] / r);
  }
}

// out[e] = (q - 8) * s for the 32 elements of block e (one block per thread): the (q - 8)
// fp16 pairs of q4_block_unpack, times the block's scale in fp32 (exact).
__global__ __launch_bounds__(BLOCK) void k_q4_dequant(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales, long long nblocks,
                                                      float* __restrict__ out) {
  const long long e = (long long)blockIdx.x * BLOCK + threadIdx.x;
  if (e >= nblocks) return;
  uint32_t wq[16];
  q4_block_unpack(ld16(codes + e * 16), wq);
  const float s = half_bits_to_float(scales[e]);
  float* o = out + e * 32;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const half2_t h = __builtin_bit_cast(half2_t, wq[m]);
    o[2 * m] = (float)h[0] * s;
    o[2 * m + 1] = (float)h[1] * s;
  }
}

// dst row k = src row perm[k]; row_bytes % 4 == 0 (16-byte vectors when row_bytes % 16 == 0).
__global__ __launch_bounds__(BLOCK) void k_permute_rows(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                        const int32_t* __restrict__ perm, int rows,
                                                        long long row_bytes) {
  const int k = blockIdx.x;
  const int from = perm[k];
  if ((unsigned)from >= (unsigned)rows) return;  // not a permutation entry: row left untouched
  const uint8_t* s = src + (size_t)from * row_bytes;
  uint8_t* o = dst + (size_t)k * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (long long c = threadIdx.x; c < row_bytes / 16; c += BLOCK)
      reinterpret_cast<u32x4*>(o)[c] = reinterpret_cast<const u32x4*>(s)[c];
  } else {
    for (long long c = threadIdx.x; c < row_bytes / 4; c += BLOCK)
      reinterpret_cast<uint32_t*>(o)[c] = reinterpret_cast<const uint32_t*>(s)[c];
  }
}

}  // namespace pi
