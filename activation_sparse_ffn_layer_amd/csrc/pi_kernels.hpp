// HIP kernels (gfx950) of the neuron-aware sparse FFN.
//
// One layer, one batch of B <= 8 tokens, three dependent kernels:
//   k_stage1     z = W1 x                 predictor stage 1; when layers are chained, the
//                                         glue x = fp16(y_prev / rms(y_prev)) is its prologue
//   k_stage2     v = W2 z + b_p           predictor stage 2 and threshold: a wavefront ballot of
//                                         (v > th) is the 64-neuron mask word of the workgroup;
//                                         then the workgroup's own active neurons' up (and gate)
//                                         rows give a_i = act(row_i . x)      [UP variant]
//   k_truemask   v = W x + b              instead of the two stages when there is no predictor;
//                                         for ReLU, a_i = max(v_i, 0) comes for free
//   k_down_cols  y[:, cols] = sum over active i of a_i w_down_t[i][cols]: every workgroup
//                                         prefix-scans the mask words itself (no waiting on other
//                                         workgroups), then owns a narrow column slice across
//                                         all active neurons; no partial sums, deterministic
// plus k_up (the index-list entry point's gathered GEMV), k_compact, k_threshold, k_glue and
// k_permute_rows.
//
// Pages: P3 = "PowerInfer: Mesin Inferensi LLM Cepat dengan GPU Konsumen" (unite.ai),
// P1 = "Tüketici sınıfı GPU takılı PC'lerde yüksek hızlı büyük dil modeli serving".
#pragma once
#include "pi_device.hpp"

namespace pi {

enum { W_F32 = 0, W_F16 = 1, W_Q4 = 2 };
enum { ACT_RELU = 0, ACT_REGLU = 1 };

struct LayerDev {
  int d, ffn, rank, act, wtype;
  float threshold;
  const uint8_t *w_up, *w_gate, *w_down_t;
  const uint16_t *s_up, *s_gate, *s_down;
  const float* b;
  const uint16_t *p_w1, *p_w2;
  const float* p_b;
};

// Where a kernel's input vector x comes from.
//  y == nullptr: x is given ([B][d], fp16 or fp32 storage).
//  y != nullptr: glue between stacked layers, x = round(y / sqrt(mean(y^2))) per token, or
//                x_prev (= x) unchanged when y is all zero; workgroup 0 stores it to x_out.
struct XIn {
  const void* x;
  const float* y;
  void* x_out;
};

template <bool XF32> struct XType { typedef half_t T; };
template <> struct XType<true> { typedef float T; };

// Per-token rms of y (0 for an all-zero y) into rms_s[NB].
template <int NB>
__device__ void glue_rms(const float* y, int B, int d, float* rms_s, float* red) {
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    float ss = 0.f;
    if (t < B)
      for (int c = threadIdx.x * 4; c < d; c += BLOCK * 4) {
        const u32x4 v = ld16(y + (size_t)t * d + c);
        ss = fmaf(u2f(v[0]), u2f(v[0]), ss);
        ss = fmaf(u2f(v[1]), u2f(v[1]), ss);
        ss = fmaf(u2f(v[2]), u2f(v[2]), ss);
        ss = fmaf(u2f(v[3]), u2f(v[3]), ss);
      }
    ss = block_sum(ss, red);
    if (threadIdx.x == 0) rms_s[t] = (ss == 0.f) ? 0.f : sqrtf(ss / (float)d);
  }
  __syncthreads();
}

// Stage x[:, c0 : c0+cw) of NB tokens into LDS xs[t][0..cw) (zeros for t >= B).
template <int NB, bool XF32>
__device__ void stage_x(const XIn& in, int B, int d, int c0, int cw, typename XType<XF32>::T* xs, int ldx,
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
          else v = (XT)(in.y[gi] / r);
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
__device__ void load_x(const void* x, int B, int d, XT* xs) {
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
// row's 16-byte chunks l, l+64, l+128, ...; the loads of all R rows are issued together.
// The caller reduces across lanes.
//   F32: chunk = 4 floats, x fp32.  F16: chunk = 8 halves, x fp16 (dot2).
//   Q4:  chunk = one 32-element block (16 code bytes + an fp16 scale), x fp16.
// ---------------------------------------------------------------------------------------
template <int WT, int NB, int R, typename XT>
__device__ __forceinline__ void rows_dot(const uint8_t* const (&row)[R], const uint16_t* const (&srow)[R],
                                         const XT* xs, int ldx, int d, int lane, float (&acc)[R][NB]) {
  if constexpr (WT == W_F16 || WT == W_F32) {
    constexpr int EPC = (WT == W_F16) ? 8 : 4;  // elements per 16-byte chunk
    constexpr int U = (R == 1) ? 8 : 4;
    const int nch = d / EPC;
    for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
      u32x4 w[R][U];
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + lane + WAVE * u;
          w[q][u] = (c < nch) ? ld_stream(row[q] + (size_t)c * 16) : (u32x4){0, 0, 0, 0};
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
  } else {  // W_Q4
    constexpr int U = (R == 1) ? 4 : 2;
    const int nb = d >> 5;
    for (int c0 = 0; c0 < nb; c0 += WAVE * U) {
      u32x4 w[R][U];
      float sc[R][U];
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + lane + WAVE * u;
          w[q][u] = (c < nb) ? ld_stream(row[q] + (size_t)c * 16) : (u32x4){0, 0, 0, 0};
          sc[q][u] = (c < nb) ? half_bits_to_float(srow[q][c]) : 0.f;
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        if (c < nb) {
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
            for (int q = 0; q < R; ++q) acc[q][t] = fmaf(sc[q][u], q4_block_dot(w[q][u], xv, 0.f), acc[q][t]);
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

// a[t][i] = act(...) for the listed neurons of one wave, two rows in flight at a time:
// ReLU pairs two neurons (up rows), ReGLU takes one neuron's gate and up rows together.
template <int WT, int ACT, int NB, typename XT>
__device__ __forceinline__ void act_pair(const LayerDev& L, const XT* xs, int B, int lane, int i0, int i1,
                                         float* __restrict__ a) {
  const int d = L.d, ffn = L.ffn;
  if constexpr (ACT == ACT_RELU) {
    const int j1 = (i1 >= 0) ? i1 : i0;
    const uint8_t* const rows[2] = {row_ptr<WT>(L.w_up, i0, d), row_ptr<WT>(L.w_up, j1, d)};
    const uint16_t* const srows[2] = {scale_ptr<WT>(L.s_up, i0, d), scale_ptr<WT>(L.s_up, j1, d)};
    float acc[2][NB] = {};
    rows_dot<WT, NB, 2, XT>(rows, srows, xs, d, d, lane, acc);
    const float b0 = L.b[i0], b1 = L.b[j1];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float h0 = wave_sum(acc[0][t]) + b0;
      const float h1 = wave_sum(acc[1][t]) + b1;
      if (lane == t && t < B) {
        a[(size_t)t * ffn + i0] = fmaxf(h0, 0.f);
        if (i1 >= 0) a[(size_t)t * ffn + i1] = fmaxf(h1, 0.f);
      }
    }
  } else {
    const uint8_t* const rows[2] = {row_ptr<WT>(L.w_gate, i0, d), row_ptr<WT>(L.w_up, i0, d)};
    const uint16_t* const srows[2] = {scale_ptr<WT>(L.s_gate, i0, d), scale_ptr<WT>(L.s_up, i0, d)};
    float acc[2][NB] = {};
    rows_dot<WT, NB, 2, XT>(rows, srows, xs, d, d, lane, acc);
    const float b0 = L.b[i0];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float g = wave_sum(acc[0][t]) + b0;
      const float u = wave_sum(acc[1][t]);
      if (lane == t && t < B) a[(size_t)t * ffn + i0] = fmaxf(g, 0.f) * u;
    }
  }
}

// The active neurons of a 64-neuron word u (union over the batch), shared out over the 4
// waves of the workgroup: wave w takes set bits w, w+4, ... (ReLU: two per step).
template <int WT, int ACT, int NB, typename XT>
__device__ void word_activations(const LayerDev& L, const XT* xs, int B, int base, uint64_t u, int wave, int lane,
                                 float* __restrict__ a) {
  const int cnt = __popcll(u);
  constexpr int STEP = (ACT == ACT_RELU) ? 2 * NWAVES : NWAVES;
  for (int r = wave; r < cnt; r += STEP) {
    const int i0 = base + select_bit(u, r);
    int i1 = -1;
    if constexpr (ACT == ACT_RELU)
      if (r + NWAVES < cnt) i1 = base + select_bit(u, r + NWAVES);
    act_pair<WT, ACT, NB, XT>(L, xs, B, lane, i0, i1, a);
  }
}

// The active neurons among one wave's rows (bits of `bits`, neuron base + bit), two rows in
// flight at a time.
template <int WT, int ACT, int NB, typename XT>
__device__ void word_activations_wave(const LayerDev& L, const XT* xs, int B, int base, uint32_t bits, int lane,
                                      float* __restrict__ a) {
  while (bits) {
    const int i0 = base + __ffs(bits) - 1;
    bits &= bits - 1;
    int i1 = -1;
    if constexpr (ACT == ACT_RELU) {
      if (bits) {
        i1 = base + __ffs(bits) - 1;
        bits &= bits - 1;
      }
    }
    act_pair<WT, ACT, NB, XT>(L, xs, B, lane, i0, i1, a);
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
  __shared__ float red[NWAVES];
  __shared__ float rms_s[NB];
  const int d = L.d, r = L.rank;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int row = blockIdx.x * NWAVES + wave;
  // The weights do not depend on x: issue this wave's first 8 chunks per lane before the glue
  // and the staging of x, so their latency overlaps.
  constexpr int PF = 8;
  const int nch0 = min(dc, d) >> 3;
  const uint8_t* wrow0 = reinterpret_cast<const uint8_t*>(L.p_w1) + (size_t)row * d * 2;
  u32x4 wp[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int c = lane + WAVE * u;
    wp[u] = (row < r && c < nch0) ? ld_stream(wrow0 + (size_t)c * 16) : (u32x4){0, 0, 0, 0};
  }
  if (xin.y != nullptr) glue_rms<NB>(xin.y, B, d, rms_s, red);
  float acc[1][NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[0][t] = 0.f;
  for (int c0 = 0; c0 < d; c0 += dc) {
    const int cw = min(dc, d - c0);
    __syncthreads();
    stage_x<NB, false>(xin, B, d, c0, cw, xs, dc, rms_s, blockIdx.x == 0);
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
        rows_dot<W_F16, NB, 1, half_t>(rows, srows, xs + done * 8, dc, cw - done * 8, lane, acc);
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
// k_stage2: v = W2 z + b_p for the TILE neurons of this workgroup (TILE/4 rows per wave, at
// most 8 so one wave's rows are one byte of the mask), then the threshold: each wave ballots
// (v > th) over its own rows and stores that byte of the token's and the batch union's 64-bit
// mask word itself. W2 rows are issued before z is read. Lane l keeps z at chunks l + 64j as
// two fp16 halves z = hi + lo (hi = fp16(z), lo = fp16(z - hi), together about 22 significant
// bits), so W2 (fp16) . z runs on dot2 with exact products.
// UP: each wave then goes straight on to the up (and gate) rows of its own active neurons,
// without waiting for the rest of the workgroup; a is dense by neuron id ([B][ffn]). x is
// staged in LDS while the W2 rows are in flight.
// ---------------------------------------------------------------------------------------
template <int NB, int CPL, int TILE, bool UP, int WT, int ACT>
__global__ __launch_bounds__(BLOCK) void k_stage2(LayerDev L, const float* __restrict__ z, int B,
                                                  uint64_t* __restrict__ mask_tok, uint64_t* __restrict__ mask_union,
                                                  float* __restrict__ logits, const void* __restrict__ x,
                                                  float* __restrict__ a) {
  constexpr int RPT = TILE / NWAVES;  // rows per wave
  static_assert(RPT == 8, "a wave owns exactly one byte of the mask");
  typedef typename XType<WT == W_F32>::T XT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  const int r = L.rank, nch = r >> 3;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int row0 = blockIdx.x * TILE + wave * RPT;  // first neuron of this wave
  const uint8_t* w2 = reinterpret_cast<const uint8_t*>(L.p_w2);
  u32x4 w[RPT][CPL];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + WAVE * j;
      w[i][j] = (c < nch) ? ld_stream(w2 + ((size_t)(row0 + i) * r + c * 8) * 2) : (u32x4){0, 0, 0, 0};
    }
  uint32_t zh[NB][CPL][4], zl[NB][CPL][4];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + WAVE * j;
      u32x4 a0 = (u32x4){0, 0, 0, 0}, a1 = (u32x4){0, 0, 0, 0};
      if (t < B && c < nch) {
        a0 = ld16(z + (size_t)t * r + c * 8);
        a1 = ld16(z + (size_t)t * r + c * 8 + 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = u2f(e < 2 ? a0[2 * e] : a1[2 * e - 4]);
        const float f1 = u2f(e < 2 ? a0[2 * e + 1] : a1[2 * e - 3]);
        const half_t h0 = (half_t)f0, h1 = (half_t)f1;
        const half_t l0 = (half_t)(f0 - (float)h0), l1 = (half_t)(f1 - (float)h1);
        zh[t][j][e] = __builtin_bit_cast(uint32_t, (half2_t){h0, h1});
        zl[t][j][e] = __builtin_bit_cast(uint32_t, (half2_t){l0, l1});
      }
    }
  if constexpr (UP) {
    load_x<NB, XT>(x, B, L.d, xs);
    __syncthreads();
  }
  const float bias = L.p_b[row0 + (lane & (RPT - 1))];
  uint32_t ubits = 0;
  const int W = L.ffn >> 6;
  uint8_t* mt = reinterpret_cast<uint8_t*>(mask_tok);
  const int byte = row0 >> 3;  // this wave's byte of the mask
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    float acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum = dot2(w[i][j][e], zh[t][j][e], sum);
          sum = dot2(w[i][j][e], zl[t][j][e], sum);
        }
      acc[i] = sum;
    }
    const float v = transpose_reduce<RPT>(acc, lane) + bias;
    if (t < B) {
      const uint32_t bits = (uint32_t)__ballot(lane < RPT && v > L.threshold) & ((1u << RPT) - 1);
      ubits |= bits;
      if (logits != nullptr && lane < RPT) logits[(size_t)t * L.ffn + row0 + lane] = v;
      if (mask_tok != nullptr && lane == 0) mt[(size_t)t * W * 8 + byte] = (uint8_t)bits;
    }
  }
  if (lane == 0) reinterpret_cast<uint8_t*>(mask_union)[byte] = (uint8_t)ubits;
  if constexpr (UP) word_activations_wave<WT, ACT, NB, XT>(L, xs, B, row0, ubits, lane, a);
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
  __shared__ float red[NWAVES];
  __shared__ float rms_s[NB];
  __shared__ float vs[NB][WAVE];
  __shared__ uint64_t s_union;
  const int d = L.d, ffn = L.ffn;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int tile = blockIdx.x;
  if (xin.y != nullptr) glue_rms<NB>(xin.y, B, d, rms_s, red);
  stage_x<NB, XF32>(xin, B, d, 0, d, xs, d, rms_s, blockIdx.x == 0);
  __syncthreads();
  const uint8_t* W = (L.act == ACT_RELU) ? L.w_up : L.w_gate;
  const uint16_t* S = (L.act == ACT_RELU) ? L.s_up : L.s_gate;
  // Rows here are d long, so one full wave reduction per row costs little next to its loads.
#pragma unroll 1
  for (int i = 0; i < 16; i += 2) {
    const int row = tile * WAVE + wave * 16 + i;
    const uint8_t* const rows[2] = {row_ptr<WT>(W, row, d), row_ptr<WT>(W, row + 1, d)};
    const uint16_t* const srows[2] = {scale_ptr<WT>(S, row, d), scale_ptr<WT>(S, row + 1, d)};
    float acc[2][NB] = {};
    rows_dot<WT, NB, 2, XT>(rows, srows, xs, d, d, lane, acc);
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
      if (L.act == ACT_RELU) {
        // a = max(h, 0) for the union's neurons (a token's inactive neurons give 0)
        if ((u >> lane) & 1ull)
#pragma unroll
          for (int t = 0; t < NB; ++t)
            if (t < B) a[(size_t)t * ffn + tile * WAVE + lane] = fmaxf(vs[t][lane], 0.f);
      }
    }
    if (lane == 0) s_union = u;
  }
  if constexpr (UP) {
    if (L.act == ACT_REGLU) {
      __syncthreads();
      word_activations<WT, ACT_REGLU, NB, XT>(L, xs, B, tile * WAVE, s_union, wave, lane, a);
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

// Neuron id of active position k (< n) from the scanned words.
__device__ __forceinline__ int neuron_at(const uint64_t* wl, const int* pre, int W, int k) {
  int lo = 0, hi = W;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= k) lo = mid;
    else hi = mid;
  }
  return lo * WAVE + select_bit(wl[lo], k - pre[lo]);
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
// by neuron id. Waves take positions k in turn, two neurons (ReLU) or one (ReGLU) at a time.
// ---------------------------------------------------------------------------------------
template <int WT, int ACT, int NB>
__global__ __launch_bounds__(BLOCK) void k_up(LayerDev L, const void* __restrict__ x, int B,
                                              const int32_t* __restrict__ idx_in, const int32_t* __restrict__ n_in,
                                              float* __restrict__ a) {
  typedef typename XType<WT == W_F32>::T XT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  const int ffn = L.ffn;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int n = min(max(*n_in, 0), ffn);
  load_x<NB, XT>(x, B, L.d, xs);
  __syncthreads();
  const int total_waves = gridDim.x * NWAVES;
  constexpr int PER = (ACT == ACT_RELU) ? 2 : 1;
  for (int k = (blockIdx.x * NWAVES + wave) * PER; k < n; k += total_waves * PER) {
    const int i0 = idx_in[k];
    int i1 = (PER == 2 && k + 1 < n) ? idx_in[k + 1] : -1;
    if ((unsigned)i1 >= (unsigned)ffn) i1 = -1;
    if ((unsigned)i0 >= (unsigned)ffn) {  // a caller-supplied entry out of range: skipped
      if (i1 >= 0) act_pair<WT, ACT, NB, XT>(L, xs, B, lane, i1, -1, a);
      continue;
    }
    act_pair<WT, ACT, NB, XT>(L, xs, B, lane, i0, i1, a);
  }
}

// ---------------------------------------------------------------------------------------
// k_down_part: part[g][t][c] = sum over the active positions k of group g of a[t][i_k] *
// w_down_t[i_k][c], for the columns c of slice blockIdx.y. The grid is G groups x S slices;
// group g takes positions k = g, g + G, g + 2G, ... A slice is SEG lanes x 16 bytes of a row
// (fp16: 8*SEG columns, fp32: 4*SEG, Q4_0: 32*SEG); the workgroup's 256 threads form 256/SEG
// neuron slots, each with U rows in flight, and the slots are summed in a fixed order. The G
// partial sums are added later in a fixed order too (by k_reduce, or by the next layer's
// glue), so y does not depend on scheduling.
//  SCAN: positions come from the union words: every workgroup prefix-scans them and expands
//        its own group's positions (k = g + G*j, j < IDX_LDS) into an index list in LDS;
//        beyond that a position is found by binary search. Workgroup (0, 0) also writes
//        idx[k] and n. Otherwise idx and n are given.
// ---------------------------------------------------------------------------------------
constexpr int IDX_LDS = 2048;  // per-group active positions expanded into LDS by the down kernel

template <int WT> struct DownGeom {
  static constexpr int EPC = (WT == W_F16) ? 8 : (WT == W_F32) ? 4 : 32;  // columns per 16-byte chunk
  static constexpr int SEG = (WT == W_Q4) ? 4 : 8;                       // lanes per row segment
  static constexpr int SW = SEG * EPC;                                   // slice width (columns)
};

template <int WT, int NB, bool SCAN, int SEG, int U, int GC = 0, int XMODE = 0>
__global__ __launch_bounds__(BLOCK) void k_down_part(LayerDev L, int B, const uint64_t* __restrict__ words,
                                                     const int32_t* __restrict__ idx_in,
                                                     const int32_t* __restrict__ n_in, const float* __restrict__ a,
                                                     float* __restrict__ part, int G, int32_t* __restrict__ idx_out,
                                                     int32_t* __restrict__ n_out, int32_t* __restrict__ n_log) {
  constexpr int EPC = DownGeom<WT>::EPC;
  constexpr int SW = SEG * EPC;
  constexpr int NSL = BLOCK / SEG;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int red[NWAVES];
  __shared__ float s_red[NSL][SW + 1];
  const int d = L.d, ffn = L.ffn, W = ffn >> 6;
  if constexpr (GC > 0) G = GC;
  const int g = blockIdx.x, s = blockIdx.y;
  const int slot = threadIdx.x / SEG, sl = threadIdx.x % SEG;
  const int col0 = s * SW + sl * EPC;
  const bool valid = col0 < d;
  uint64_t* wl = reinterpret_cast<uint64_t*>(smem);
  int* pre = reinterpret_cast<int*>(wl + W);
  int* il = pre + W + 1;  // [IDX_LDS] expanded index list
  int n;
  if constexpr (SCAN) {
    n = scan_words(words, W, wl, pre, red);
    const bool writer = (XMODE & 1) ? false : (g == 0 && s == 0);
    for (int w = threadIdx.x; w < W; w += BLOCK) {
      uint64_t word = wl[w];
      int pos = pre[w];
      while (word) {
        const int i = w * WAVE + __ffsll((unsigned long long)word) - 1;
        word &= word - 1;
        if (writer) idx_out[pos] = i;
        if (pos % G == g && pos / G < IDX_LDS) il[pos / G] = i;
        ++pos;
      }
    }
    __syncthreads();
    if (writer && threadIdx.x == 0) {
      *n_out = n;
      if (n_log != nullptr) *n_log = n;
    }
  } else {
    n = min(max(*n_in, 0), ffn);
  }
  float acc[NB][EPC];
  float qsum[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    qsum[t] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[t][e] = 0.f;
  }
  for (int j0 = slot; g + G * j0 < n; j0 += NSL * U) {
    int ii[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = g + G * (j0 + NSL * u);
      int i = -1;
      if (k < n) {
        if constexpr (SCAN && (XMODE & 2)) {
          i = idx_in[k];
        } else if constexpr (SCAN) {
          const int j = (k - g) / G;
          i = (j < IDX_LDS) ? il[j] : neuron_at(wl, pre, W, k);
        }
        else i = idx_in[k];
      }
      ii[u] = ((unsigned)i < (unsigned)ffn) ? i : -1;
    }
    u32x4 w[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w[u] = (u32x4){0, 0, 0, 0};
      sc[u] = 0.f;
      if (ii[u] >= 0 && valid) {
        if constexpr (WT == W_F16) w[u] = ld_stream(L.w_down_t + ((size_t)ii[u] * d + col0) * 2);
        else if constexpr (WT == W_F32) w[u] = ld_stream(L.w_down_t + ((size_t)ii[u] * d + col0) * 4);
        else {
          const size_t blk = (size_t)ii[u] * (d >> 5) + (col0 >> 5);
          w[u] = ld_stream(L.w_down_t + blk * 16);
          sc[u] = half_bits_to_float(L.s_down[blk]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ii[u] < 0) continue;
      float av[NB];
#pragma unroll
      for (int t = 0; t < NB; ++t) av[t] = (t < B) ? a[(size_t)t * ffn + ii[u]] : 0.f;
      if constexpr (WT == W_F16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = h2f_lo(w[u][e]), hi = h2f_hi(w[u][e]);
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            acc[t][2 * e] = fmaf(av[t], lo, acc[t][2 * e]);
            acc[t][2 * e + 1] = fmaf(av[t], hi, acc[t][2 * e + 1]);
          }
        }
      } else if constexpr (WT == W_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int t = 0; t < NB; ++t) acc[t][e] = fmaf(av[t], u2f(w[u][e]), acc[t][e]);
      } else {
        float q[32];
        q4_block_codes(w[u], q);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const float as = av[t] * sc[u];
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
  // sum the NSL slots of each column (fixed order) and store this group's partial
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if (t >= B) break;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPC; ++e) s_red[slot][sl * EPC + e] = acc[t][e];
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

// Standalone glue: one workgroup per token.
template <bool XF32>
__global__ __launch_bounds__(BLOCK) void k_glue(const float* __restrict__ y, const void* __restrict__ x_prev, int d,
                                                void* __restrict__ x_out) {
  typedef typename XType<XF32>::T XT;
  __shared__ float red[NWAVES];
  const int t = blockIdx.x;
  const float* yt = y + (size_t)t * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += BLOCK) ss = fmaf(yt[c], yt[c], ss);
  ss = block_sum(ss, red);
  const float r = (ss == 0.f) ? 0.f : sqrtf(ss / (float)d);
  const XT* xp = reinterpret_cast<const XT*>(x_prev) + (size_t)t * d;
  XT* xo = reinterpret_cast<XT*>(x_out) + (size_t)t * d;
  for (int c = threadIdx.x; c < d; c += BLOCK) xo[c] = (r == 0.f) ? xp[c] : (XT)(yt[c] / r);
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
