// Batched path (9..64 tokens) on the gfx950 matrix cores (v_mfma_f32_32x32x16_f16).
//
// With many tokens the union of their masks covers most neurons, and every weight row that is
// read is used by every token: the work becomes a dense contraction over gathered rows, which
// is what the matrix cores are for. The same tiling serves four products:
//   predictor stage 1   z = X W1^T           (K = d, split over K into partial sums)
//   predictor stage 2   v = Z W2^T + b_p     (Z = z split into fp16 hi + lo; mask epilogue)
//   gate / up           a = act(X W_gate[idx]^T + b, X W_up[idx]^T)   (gathered rows)
//   down                y = A W_down_t[idx]  (A = the activations, gathered rows, split over K)
// MFMA lane layout (32x32x16 f16, checked on the device): A operand, lane l holds row l%32 and
// k = 8*(l/32)..+7; B operand, lane l holds column l%32 and the same k; accumulator register r
// of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma once
#include "pi_kernels.hpp"

namespace pi {

typedef half_t h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int mfma_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ f16v mfma(h8 a, h8 b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

enum { EPI_PART = 0, EPI_MASK = 1, EPI_ACT = 2 };

// Arguments of the row-tiled product C[t][n] = sum_k X[t][k] W[row(n)][k].
struct MmRows {
  const half_t* x;       // [Bp][K] fp16 (Bp = 32*MT rows, rows >= B ignored)
  const half_t* x_lo;    // HILO: low halves of X
  int B, K, ldx;
  const half_t* w0;      // rows of K halves: W1, W2, or up (ReLU) / gate (ReGLU)
  const half_t* w1;      // ReGLU: up rows
  const int32_t* idx;    // gathered rows: row(n) = idx[n]; NULL: row(n) = n
  const int32_t* n_dev;  // number of columns on the device (gathered), or NULL
  int N;                 // number of columns when n_dev is NULL
  int ks_len;            // K-split chunk length (multiple of the window), K when not split
  // epilogues
  float* part;           // EPI_PART: [KS][B][N] fp32
  const float* bias;     // EPI_MASK: b_p; EPI_ACT: b (by neuron id)
  float threshold;
  uint32_t* mask_tok;    // EPI_MASK: [B][ffn/32] 32-bit mask words (nullable)
  uint32_t* mask_union;  // EPI_MASK: [ffn/32]
  float* logits;         // EPI_MASK: [B][N] (nullable)
  half_t* a16;           // EPI_ACT: [Bp][lda] activations at compacted positions
  int lda;
  int ffn;
};

constexpr int MM_KW = 256;  // K window staged in LDS per step of the workgroup

template <int EPI, int ACT, int MT, bool HILO>
__global__ __launch_bounds__(BLOCK) void k_mm_rows(MmRows p) {
  constexpr int LDR = MM_KW + 8;  // padded LDS row (halves): 16-byte skew between rows
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);         // [32*MT][LDR]
  half_t* xl = xs + 32 * MT * LDR;                      // HILO: low halves
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int N = (p.n_dev != nullptr) ? min(*p.n_dev, p.ffn) : p.N;
  const int n0 = (blockIdx.x * NWAVES + wave) * 32;
  if (blockIdx.x * NWAVES * 32 >= N) return;  // whole workgroup past the end (uniform)
  const int n = n0 + (lane & 31);
  const bool valid = n < N;
  int row = valid ? ((p.idx != nullptr) ? p.idx[n] : n) : 0;
  if ((unsigned)row >= (unsigned)(p.idx != nullptr ? p.ffn : N)) row = 0;
  const int kh = 8 * (lane >> 5);
  const int k_begin = blockIdx.y * p.ks_len, k_end = min(p.K, k_begin + p.ks_len);
  const half_t* r0 = p.w0 + (size_t)row * p.K + kh;
  const half_t* r1 = (ACT == ACT_REGLU && EPI == EPI_ACT) ? p.w1 + (size_t)row * p.K + kh : nullptr;
  f16v acc0[MT], acc1[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    acc0[m] = (f16v){};
    acc1[m] = (f16v){};
  }
  const int rows_x = 32 * MT;
  for (int w0 = k_begin; w0 < k_end; w0 += MM_KW) {
    const int kw = min(MM_KW, k_end - w0);
    __syncthreads();
    // stage X[:, w0 : w0+kw] (16-byte pieces); rows >= B are zeros
    for (int q = threadIdx.x; q < rows_x * (MM_KW / 8); q += BLOCK) {
      const int t = q / (MM_KW / 8), c = (q % (MM_KW / 8)) * 8;
      u32x4 v = (u32x4){0, 0, 0, 0}, vl = (u32x4){0, 0, 0, 0};
      if (t < p.B && c < kw) {
        v = ld16(p.x + (size_t)t * p.ldx + w0 + c);
        if constexpr (HILO) vl = ld16(p.x_lo + (size_t)t * p.ldx + w0 + c);
      }
      *reinterpret_cast<u32x4*>(xs + t * LDR + c) = v;
      if constexpr (HILO) *reinterpret_cast<u32x4*>(xl + t * LDR + c) = vl;
    }
    __syncthreads();
    constexpr int U = 4;
    for (int k = 0; k < kw; k += 16 * U) {
      u32x4 b0[U], b1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = valid && (k + 16 * u < kw);
        b0[u] = in ? ld_stream(r0 + w0 + k + 16 * u) : (u32x4){0, 0, 0, 0};
        if constexpr (ACT == ACT_REGLU && EPI == EPI_ACT) b1[u] = in ? ld_stream(r1 + w0 + k + 16 * u) : (u32x4){0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k + 16 * u >= kw) break;
        const h8 bb0 = __builtin_bit_cast(h8, b0[u]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int xr = (32 * m + (lane & 31)) * LDR + k + 16 * u + kh;
          const h8 a = __builtin_bit_cast(h8, ld16(xs + xr));
          acc0[m] = mfma(a, bb0, acc0[m]);
          if constexpr (HILO) acc0[m] = mfma(__builtin_bit_cast(h8, ld16(xl + xr)), bb0, acc0[m]);
          if constexpr (ACT == ACT_REGLU && EPI == EPI_ACT) acc1[m] = mfma(a, __builtin_bit_cast(h8, b1[u]), acc1[m]);
        }
      }
    }
  }
  // ---- epilogues
  if constexpr (EPI == EPI_PART) {
    if (valid) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * m + mfma_row(r, lane);
          if (t < p.B) p.part[((size_t)blockIdx.y * p.B + t) * N + n] = acc0[m][r];
        }
    }
  } else if constexpr (EPI == EPI_MASK) {
    const float bias = valid ? p.bias[n] : 0.f;
    const int W32 = p.ffn >> 5;
    bool any = false;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * m + mfma_row(r, lane);
        const float v = acc0[m][r] + bias;
        const bool bit = valid && t < p.B && v > p.threshold;
        any |= bit;
        const uint64_t bal = __ballot(bit);
        if (p.mask_tok != nullptr && (lane & 31) == 0 && t < p.B)
          p.mask_tok[(size_t)t * W32 + (n0 >> 5)] = (uint32_t)(bal >> (lane & 32));
        if (p.logits != nullptr && valid && t < p.B) p.logits[(size_t)t * p.N + n] = v;
      }
    const uint64_t u = __ballot(any);
    if (lane == 0) p.mask_union[n0 >> 5] = (uint32_t)u | (uint32_t)(u >> 32);
  } else {  // EPI_ACT: a16[t][n] for compacted position n
    const float bias = valid ? p.bias[row] : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * m + mfma_row(r, lane);
        float a = 0.f;
        if (valid && t < p.B) {
          if constexpr (ACT == ACT_RELU) a = fmaxf(acc0[m][r] + bias, 0.f);
          else a = fmaxf(acc0[m][r] + bias, 0.f) * acc1[m][r];
        }
        if (n < ((N + 15) & ~15)) p.a16[(size_t)t * p.lda + n] = (half_t)a;
      }
  }
}

// Down projection y_part[ks][t][c] = sum over positions k of split ks of a16[t][k] *
// w_down_t[idx[k]][c]. A wave owns 128 columns (4 per lane of a half-wave: one 8-byte load
// per row) and walks its K split 16 positions at a time: lanes of half h load rows
// k + 8h .. k + 8h + 7, so each lane holds the 8 K values of its 4 columns and feeds four
// MFMAs whose output columns are {4*(l%32) + j}.
struct MmDown {
  const half_t* a16;     // [Bp][lda]
  int lda, B;
  const half_t* wd;      // [ffn][d] fp16 rows
  const int32_t* idx;
  const int32_t* n_dev;
  int ffn, d;
  int ks_len;            // positions per K split (multiple of 16)
  float* part;           // [KS][B][d]
};

template <int MT>
__global__ __launch_bounds__(BLOCK) void k_mm_down(MmDown p) {
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int n = min(max(*p.n_dev, 0), p.ffn);
  const int c0 = (blockIdx.x * NWAVES + wave) * 128 + 4 * (lane & 31);
  const bool cvalid = c0 < p.d;
  const int kh = 8 * (lane >> 5);
  const int k_begin = blockIdx.y * p.ks_len, k_end = min(n, k_begin + p.ks_len);
  f16v acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = (f16v){};
  for (int k = k_begin; k < k_end; k += 16) {
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = k + kh + e;
      int i = (kk < k_end) ? p.idx[kk] : -1;
      if ((unsigned)i >= (unsigned)p.ffn) i = -1;
      uint64_t v = 0;
      if (i >= 0 && cvalid) v = *reinterpret_cast<const uint64_t*>(p.wd + (size_t)i * p.d + c0);
      lo[e] = (uint32_t)v;
      hi[e] = (uint32_t)(v >> 32);
    }
    h8 bj[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const half2_t l2 = __builtin_bit_cast(half2_t, lo[e]), h2 = __builtin_bit_cast(half2_t, hi[e]);
      bj[0][e] = l2.x;
      bj[1][e] = l2.y;
      bj[2][e] = h2.x;
      bj[3][e] = h2.y;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = 32 * m + (lane & 31);
      h8 a = __builtin_bit_cast(h8, ld16(p.a16 + (size_t)t * p.lda + k + kh));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + kh + e >= k_end) a[e] = (half_t)0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] = mfma(a, bj[j], acc[m][j]);
    }
  }
  if (!cvalid) return;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * m + mfma_row(r, lane);
      if (t < p.B) {
        float* o = p.part + ((size_t)blockIdx.y * p.B + t) * p.d + c0;
        *reinterpret_cast<f32x4*>(o) = (f32x4){acc[m][0][r], acc[m][1][r], acc[m][2][r], acc[m][3][r]};
      }
    }
}

// z = sum of G partials [G][B][N], written as fp16 hi and lo halves (z = hi + lo to ~22 bits).
__global__ __launch_bounds__(BLOCK) void k_reduce_hilo(const float* __restrict__ part, int G, int BN,
                                                       half_t* __restrict__ hi, half_t* __restrict__ lo) {
  const int i = blockIdx.x * BLOCK + threadIdx.x;
  if (i >= BN) return;
  float s = 0.f;
  for (int g = 0; g < G; ++g) s += part[(size_t)g * BN + i];
  const half_t h = (half_t)s;
  hi[i] = h;
  lo[i] = (half_t)(s - (float)h);
}

}  // namespace pi
