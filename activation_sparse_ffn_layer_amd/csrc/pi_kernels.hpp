// HIP kernels (gfx950) of the neuron-aware sparse FFN.
//
// Per layer and batch of B <= 8 tokens the path is:
//   k_stage1    z = W1 x                     (predictor, first low-rank stage; glue prologue)
//   k_stage2    v = W2 z + b_p, bits v > th   (second stage + threshold; one 64-neuron word
//                                            per workgroup via a wavefront ballot)
//   k_truemask  v = W x + b, bits v > th      (instead of the two stages when rank == 0)
//   k_up        a_k = act(row_i . x)         (each workgroup prefix-scans the mask words,
//                                            then its waves take active positions k)
//   k_down      partial_g = sum_k a_k w_down_t[i_k] over a column slice
//   k_reduce    y = sum_g partial_g          (fixed order: deterministic)
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
      for (int c = threadIdx.x; c < d; c += BLOCK) {
        const float v = y[(size_t)t * d + c];
        ss = fmaf(v, v, ss);
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

// ---------------------------------------------------------------------------------------
// Partial dot products of one weight row with NB vectors staged in LDS. Lane l handles the
// row's 16-byte chunks l, l+64, l+128, ...; the caller reduces across lanes.
//   F32: chunk = 4 floats, x fp32.  F16: chunk = 8 halves, x fp16 (dot2).
//   Q4:  chunk = one 32-element block (16 code bytes + an fp16 scale), x fp16.
// ---------------------------------------------------------------------------------------
template <int WT, int NB, typename XT>
__device__ __forceinline__ void row_dot(const uint8_t* row, const uint16_t* srow, const XT* xs, int ldx, int d,
                                        int lane, float (&acc)[NB]) {
  if constexpr (WT == W_F16) {
    const int nch = d >> 3;
    constexpr int U = 8;
    for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
      u32x4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        w[u] = (c < nch) ? ld_stream(row + (size_t)c * 16) : (u32x4){0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        if (c < nch) {
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            const u32x4 xv = ld16(reinterpret_cast<const half_t*>(xs) + t * ldx + c * 8);
            float s = acc[t];
            s = dot2(w[u][0], xv[0], s);
            s = dot2(w[u][1], xv[1], s);
            s = dot2(w[u][2], xv[2], s);
            s = dot2(w[u][3], xv[3], s);
            acc[t] = s;
          }
        }
      }
    }
  } else if constexpr (WT == W_F32) {
    const int nch = d >> 2;
    constexpr int U = 8;
    for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
      u32x4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        w[u] = (c < nch) ? ld_stream(row + (size_t)c * 16) : (u32x4){0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        if (c < nch) {
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            const u32x4 xv = ld16(reinterpret_cast<const float*>(xs) + t * ldx + c * 4);
            float s = acc[t];
            s = fmaf(u2f(w[u][0]), u2f(xv[0]), s);
            s = fmaf(u2f(w[u][1]), u2f(xv[1]), s);
            s = fmaf(u2f(w[u][2]), u2f(xv[2]), s);
            s = fmaf(u2f(w[u][3]), u2f(xv[3]), s);
            acc[t] = s;
          }
        }
      }
    }
  } else {  // W_Q4
    const int nb = d >> 5;
    constexpr int U = 4;
    for (int c0 = 0; c0 < nb; c0 += WAVE * U) {
      u32x4 w[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + WAVE * u;
        w[u] = (c < nb) ? ld_stream(row + (size_t)c * 16) : (u32x4){0, 0, 0, 0};
        sc[u] = (c < nb) ? half_bits_to_float(srow[c]) : 0.f;
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
              const u32x4 q = ld16(xb + 8 * m);
              xv[4 * m + 0] = q[0];
              xv[4 * m + 1] = q[1];
              xv[4 * m + 2] = q[2];
              xv[4 * m + 3] = q[3];
            }
            acc[t] = fmaf(sc[u], q4_block_dot(w[u], xv, 0.f), acc[t]);
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

// ---------------------------------------------------------------------------------------
// Mask epilogue (wave 0 of a workgroup owning neurons [64*tile, 64*tile + 64)):
// lane j holds v of neuron 64*tile + j for each token; a ballot of (v > threshold) is the
// token's mask word, the OR over tokens the union word.
// ---------------------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ void emit_mask(const float (*vs)[WAVE], int tile, int B, float th, int ffn,
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
  float acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = 0.f;
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
              float s2 = acc[t];
              s2 = dot2(wp[u][0], xv[0], s2);
              s2 = dot2(wp[u][1], xv[1], s2);
              s2 = dot2(wp[u][2], xv[2], s2);
              s2 = dot2(wp[u][3], xv[3], s2);
              acc[t] = s2;
            }
          }
        }
        done = min(nch0, WAVE * PF);
      }
      if (done * 8 < cw) {
        const uint8_t* wrow = wrow0 + ((size_t)c0 + done * 8) * 2;
        row_dot<W_F16, NB, half_t>(wrow, nullptr, xs + done * 8, dc, cw - done * 8, lane, acc);
      }
    }
  }
  if (row < r) {
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && t < B) z[(size_t)t * r + row] = s;
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_stage2: v = W2 z + b_p for the 64 neurons of this workgroup, then the mask epilogue.
// Lane l keeps z at chunks l + 64j (8 fp32 values each) in registers; each wave reduces
// RPW rows at a time with transpose_reduce.
// ---------------------------------------------------------------------------------------
template <int NB, int CPL, int RPW>
__global__ __launch_bounds__(BLOCK) void k_stage2(LayerDev L, const float* __restrict__ z, int B,
                                                  uint64_t* __restrict__ mask_tok, uint64_t* __restrict__ mask_union,
                                                  float* __restrict__ logits) {
  __shared__ float vs[NB][WAVE];
  const int r = L.rank, nch = r >> 3;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int tile = blockIdx.x;
  const uint8_t* w2 = reinterpret_cast<const uint8_t*>(L.p_w2);
  // W2 rows do not depend on z: issue the first group's loads before reading z.
  u32x4 w[RPW][CPL];
  {
    const int row0 = tile * WAVE + wave * 16;
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + WAVE * j;
        w[i][j] = (c < nch) ? ld_stream(w2 + ((size_t)(row0 + i) * r + c * 8) * 2) : (u32x4){0, 0, 0, 0};
      }
  }
  float zr[NB][CPL][8];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + WAVE * j;
      if (t < B && c < nch) {
        const u32x4 a0 = ld16(z + (size_t)t * r + c * 8);
        const u32x4 a1 = ld16(z + (size_t)t * r + c * 8 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          zr[t][j][e] = u2f(a0[e]);
          zr[t][j][4 + e] = u2f(a1[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) zr[t][j][e] = 0.f;
      }
    }
#pragma unroll 1
  for (int g = 0; g < 16; g += RPW) {
    const int row0 = tile * WAVE + wave * 16 + g;
    if (g > 0) {
#pragma unroll
      for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = lane + WAVE * j;
          w[i][j] = (c < nch) ? ld_stream(w2 + ((size_t)(row0 + i) * r + c * 8) * 2) : (u32x4){0, 0, 0, 0};
        }
    }
    float acc[NB][RPW];
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s = fmaf(h2f_lo(w[i][j][e]), zr[t][j][2 * e], s);
            s = fmaf(h2f_hi(w[i][j][e]), zr[t][j][2 * e + 1], s);
          }
        acc[t][i] = s;
      }
    const float bias = L.p_b[row0 + (lane & (RPW - 1))];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float v = transpose_reduce<RPW>(acc[t], lane) + bias;
      if (lane < RPW) vs[t][wave * 16 + g + lane] = v;
    }
  }
  __syncthreads();
  if (wave == 0) emit_mask<NB>(vs, tile, B, L.threshold, L.ffn, mask_tok, mask_union, logits);
}

// ---------------------------------------------------------------------------------------
// k_truemask: v = W x + b for the 64 neurons of this workgroup (W = up for ReLU, gate for
// ReGLU), then the mask epilogue. Each wave owns 16 rows; x (whole d) in LDS.
// ---------------------------------------------------------------------------------------
template <int WT, int NB, bool XF32>
__global__ __launch_bounds__(BLOCK) void k_truemask(LayerDev L, XIn xin, int B, uint64_t* __restrict__ mask_tok,
                                                    uint64_t* __restrict__ mask_union, float* __restrict__ logits) {
  typedef typename XType<XF32>::T XT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ float red[NWAVES];
  __shared__ float rms_s[NB];
  __shared__ float vs[NB][WAVE];
  const int d = L.d;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int tile = blockIdx.x;
  if (xin.y != nullptr) glue_rms<NB>(xin.y, B, d, rms_s, red);
  stage_x<NB, XF32>(xin, B, d, 0, d, xs, d, rms_s, blockIdx.x == 0);
  __syncthreads();
  const uint8_t* W = (L.act == ACT_RELU) ? L.w_up : L.w_gate;
  const uint16_t* S = (L.act == ACT_RELU) ? L.s_up : L.s_gate;
  // Rows here are d long, so one full wave reduction per row costs little next to its loads.
#pragma unroll 1
  for (int i = 0; i < 16; ++i) {
    const int row = tile * WAVE + wave * 16 + i;
    float a[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) a[t] = 0.f;
    row_dot<WT, NB, XT>(row_ptr<WT>(W, row, d), (WT == W_Q4) ? S + (size_t)row * (d >> 5) : nullptr, xs, d, d,
                        lane, a);
    const float bias = L.b[row];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float v = wave_sum(a[t]) + bias;
      if (lane == 0) vs[t][wave * 16 + i] = v;
    }
  }
  __syncthreads();
  if (wave == 0) emit_mask<NB>(vs, tile, B, L.threshold, L.ffn, mask_tok, mask_union, logits);
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
  emit_mask<NB>(vs, tile, B, th, ffn, mask_tok, mask_union, nullptr);
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
// k_up: a[t][k] = act(row_{i_k} . x_t) for k < n.
//  SCAN: the workgroup loads the union words into LDS and prefix-scans them, then position
//  k maps to neuron i_k = 64w + (the (k - pre[w])-th set bit of word w); the workgroup
//  writes idx[k] = i_k and workgroup 0 writes n. Otherwise idx and n are given.
// ---------------------------------------------------------------------------------------
template <int WT, int ACT, int NB, bool SCAN>
__global__ __launch_bounds__(BLOCK) void k_up(LayerDev L, const void* __restrict__ x, int B,
                                              const uint64_t* __restrict__ words, const int32_t* __restrict__ idx_in,
                                              const int32_t* __restrict__ n_in, int32_t* __restrict__ idx_out,
                                              int32_t* __restrict__ n_out, int32_t* __restrict__ n_log,
                                              float* __restrict__ a) {
  constexpr bool XF32 = (WT == W_F32);
  typedef typename XType<XF32>::T XT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int d = L.d, ffn = L.ffn, W = ffn >> 6;
  XT* xs = reinterpret_cast<XT*>(smem);
  uint64_t* wl = reinterpret_cast<uint64_t*>(smem + (size_t)NB * d * sizeof(XT));
  int* pre = reinterpret_cast<int*>(wl + W);
  __shared__ int red[NWAVES];
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  int n;
  if constexpr (SCAN) {
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
    n = carry;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *n_out = n;
      if (n_log != nullptr) *n_log = n;
    }
  } else {
    n = min(max(*n_in, 0), ffn);
  }
  {
    XIn xin{x, nullptr, nullptr};
    stage_x<NB, XF32>(xin, B, d, 0, d, xs, d, nullptr, false);
  }
  __syncthreads();
  const int total_waves = gridDim.x * NWAVES;
  for (int k = blockIdx.x * NWAVES + wave; k < n; k += total_waves) {
    int i;
    if constexpr (SCAN) {
      int lo = 0, hi = W;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= k) lo = mid;
        else hi = mid;
      }
      i = lo * WAVE + select_bit(wl[lo], k - pre[lo]);
      if (lane == 0) idx_out[k] = i;
    } else {
      i = idx_in[k];
      if ((unsigned)i >= (unsigned)ffn) continue;  // a caller-supplied entry out of range: skipped
    }
    float h[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) h[t] = 0.f;
    if constexpr (ACT == ACT_RELU) {
      row_dot<WT, NB, XT>(row_ptr<WT>(L.w_up, i, d), (WT == W_Q4) ? L.s_up + (size_t)i * (d >> 5) : nullptr, xs, d,
                          d, lane, h);
      const float bias = L.b[i];
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const float v = wave_sum(h[t]) + bias;
        if (lane == t && t < B) a[(size_t)t * ffn + k] = fmaxf(v, 0.f);
      }
    } else {
      float u[NB];
#pragma unroll
      for (int t = 0; t < NB; ++t) u[t] = 0.f;
      row_dot<WT, NB, XT>(row_ptr<WT>(L.w_gate, i, d), (WT == W_Q4) ? L.s_gate + (size_t)i * (d >> 5) : nullptr, xs,
                          d, d, lane, h);
      row_dot<WT, NB, XT>(row_ptr<WT>(L.w_up, i, d), (WT == W_Q4) ? L.s_up + (size_t)i * (d >> 5) : nullptr, xs, d,
                          d, lane, u);
      const float bias = L.b[i];
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const float g = wave_sum(h[t]) + bias;
        const float uu = wave_sum(u[t]);
        if (lane == t && t < B) a[(size_t)t * ffn + k] = fmaxf(g, 0.f) * uu;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_down: partial[g][t][c] = sum over this group's active positions k of a[t][k] *
// w_down_t[i_k][c], for the columns c of slice blockIdx.y. Workgroup = 8 half-waves of 32
// lanes; a half-wave reads one row segment of 32 x 16 bytes per step (256 fp16 / 128 fp32 /
// 1024 Q4 columns), its rows interleaved with the other half-waves and groups.
// ---------------------------------------------------------------------------------------
template <int WT> struct DownGeom {
  static constexpr int EPL = (WT == W_F16) ? 8 : (WT == W_F32) ? 4 : 32;  // columns per lane
  static constexpr int SW = EPL * 32;                                    // slice width
};

template <int WT, int NB>
__global__ __launch_bounds__(BLOCK) void k_down(LayerDev L, int B, const int32_t* __restrict__ idx,
                                                const int32_t* __restrict__ n_in, const float* __restrict__ a,
                                                float* __restrict__ part, int G) {
  constexpr int EPL = DownGeom<WT>::EPL, SW = DownGeom<WT>::SW;
  __shared__ float s_red[8][SW];
  const int d = L.d, ffn = L.ffn;
  const int g = blockIdx.x, s = blockIdx.y;
  const int hw = threadIdx.x >> 5, hl = threadIdx.x & 31;
  const int col0 = s * SW + hl * EPL;
  const bool valid = col0 < d;
  const int n = min(max(*n_in, 0), ffn);
  float acc[NB][EPL];
  float qsum[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    qsum[t] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[t][e] = 0.f;
  }
  constexpr int U = (WT == W_Q4) ? 2 : 4;
  for (int j0 = hw; g + G * j0 < n; j0 += 8 * U) {
    int kk[U];
    int ii[U];
    u32x4 w[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kk[u] = g + G * (j0 + 8 * u);
      ii[u] = (kk[u] < n) ? idx[kk[u]] : -1;
      if ((unsigned)ii[u] >= (unsigned)ffn) ii[u] = -1;
    }
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
      for (int t = 0; t < NB; ++t) av[t] = (t < B) ? a[(size_t)t * ffn + kk[u]] : 0.f;
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
      for (int e = 0; e < EPL; ++e) acc[t][e] = fmaf(-8.f, qsum[t], acc[t][e]);
  }
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if (t >= B) break;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_red[hw][hl * EPL + e] = acc[t][e];
    __syncthreads();
    for (int c = threadIdx.x; c < SW; c += BLOCK) {
      const int col = s * SW + c;
      if (col < d) {
        float v = 0.f;
#pragma unroll
        for (int h = 0; h < 8; ++h) v += s_red[h][c];
        part[((size_t)g * B + t) * d + col] = v;
      }
    }
  }
}

// y[i] = sum_{g < G} part[g][i] over i < BD = B*d (G <= 64). A workgroup covers 64 outputs;
// its 4 waves each sum every 4th group with all loads in flight, then wave 0 adds the four
// wave sums in a fixed order, so the result does not depend on scheduling.
__global__ __launch_bounds__(BLOCK) void k_reduce(const float* __restrict__ part, int G, int BD, float* __restrict__ y) {
  __shared__ float s4[NWAVES][WAVE];
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int i = blockIdx.x * WAVE + lane;
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int g = wave + NWAVES * j;
    v[j] = (i < BD && g < G) ? part[(size_t)g * BD + i] : 0.f;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += v[j];
  s4[wave][lane] = s;
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
