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
  const half_t* x;       // [B][ldx] fp16 token rows
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
  const uint32_t* tok_mask;  // EPI_ACT: [B][ffn/32] mask words; token t keeps only its own
                             // neurons (per-token masking). NULL: the union
  int lda;
  int ffn;
  int hot_prefix;        // EPI_MASK: columns [0, hot_prefix) are taken without a prediction
};

// Whether token t keeps neuron i: always under the union; its own mask bit under per-token
// masking.
__device__ __forceinline__ bool tok_keeps(const MmRows& p, int t, int i) {
  return p.tok_mask == nullptr || ((p.tok_mask[(size_t)t * (p.ffn >> 5) + (i >> 5)] >> (i & 31)) & 1u);
}

// ---------------------------------------------------------------------------------------
// k_mm_gemm: the row-tiled products C[t][n] = sum_k X[t][k] W[row(n)][k], tiled through LDS. A workgroup owns 64
// weight rows (ReGLU activations: 32 neurons' gate rows then their up rows) and all 64 token
// rows of X, and walks K in chunks of MG_KC halves. Every thread loads 16-byte pieces of 4
// weight rows and 4 X rows per chunk (16 lanes cover a row's 256-byte piece: coalesced), the
// next chunk's pieces are loaded while the current chunk, staged in LDS, feeds the MFMAs.
// Wave w computes the 32 x 32 block (tokens 32*(w>>1).., rows 32*(w&1)..).
// K (and every K split) is a multiple of 16; tokens >= B and rows past N are zeros.
// ---------------------------------------------------------------------------------------
constexpr int MG_KC = 128;         // K chunk (halves)
constexpr int MG_P = MG_KC + 8;    // LDS row pitch (halves): 16-byte skew between rows

template <bool HILO>
constexpr size_t mm_gemm_lds() { return (size_t)(HILO ? 3 : 2) * 64 * MG_P * 2; }

template <int EPI, int ACT, bool HILO>
__global__ __launch_bounds__(BLOCK) void k_mm_gemm(MmRows p) {
  constexpr bool GU = (EPI == EPI_ACT && ACT == ACT_REGLU);  // rows = gate rows, then up rows
  constexpr int NPW = GU ? 32 : 64;                          // output columns per workgroup
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* ws = reinterpret_cast<half_t*>(smem);  // [64][MG_P] weight rows
  half_t* xs = ws + 64 * MG_P;                   // [64][MG_P] X rows
  half_t* xls = xs + 64 * MG_P;                  // HILO: low halves of X
  __shared__ uint32_t s_union[2];
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int N = (p.n_dev != nullptr) ? min(max(*p.n_dev, 0), p.ffn) : p.N;
  const int nb = blockIdx.x * NPW;
  if (nb >= N) return;  // uniform over the workgroup
  // load slots: tile rows rr = tid/16 + 16j (j < 4), piece tid%16 of the chunk
  const int piece = threadIdx.x & 15;
  const half_t* wp[4];
  const half_t* xp[4];
  const half_t* xlp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = (threadIdx.x >> 4) + 16 * j;
    const int col = nb + (GU ? (rr & 31) : rr);
    wp[j] = nullptr;
    if (col < N) {
      int row = (p.idx != nullptr) ? p.idx[col] : col;
      if ((unsigned)row >= (unsigned)(p.idx != nullptr ? p.ffn : N)) row = 0;
      const half_t* base = (GU && rr >= 32) ? p.w1 : p.w0;
      wp[j] = base + (size_t)row * p.K + piece * 8;
    }
    xp[j] = (rr < p.B) ? p.x + (size_t)rr * p.ldx + piece * 8 : nullptr;
    xlp[j] = (HILO && rr < p.B) ? p.x_lo + (size_t)rr * p.ldx + piece * 8 : nullptr;
  }
  const int k_begin = blockIdx.y * p.ks_len, k_end = min(p.K, k_begin + p.ks_len);
  u32x4 wr[4], xr[4], xlr[4];
  auto load = [&](int kc) {
    const int off = kc + piece * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = off < k_end;
      wr[j] = (in && wp[j] != nullptr) ? ld_stream(wp[j] + kc) : (u32x4){0, 0, 0, 0};
      xr[j] = (in && xp[j] != nullptr) ? ld16(xp[j] + kc) : (u32x4){0, 0, 0, 0};
      if constexpr (HILO) xlr[j] = (in && xlp[j] != nullptr) ? ld16(xlp[j] + kc) : (u32x4){0, 0, 0, 0};
    }
  };
  f16v acc = (f16v){};
  const int rb = wave & 1, tb = wave >> 1;
  const int kh = 8 * (lane >> 5);
  const half_t* wrd = ws + (32 * rb + (lane & 31)) * MG_P + kh;
  const half_t* xrd = xs + (32 * tb + (lane & 31)) * MG_P + kh;
  const half_t* xlrd = xls + (32 * tb + (lane & 31)) * MG_P + kh;
  if (k_begin < k_end) load(k_begin);
  for (int kc = k_begin; kc < k_end; kc += MG_KC) {
    __syncthreads();  // the previous chunk's reads of LDS are done
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = (threadIdx.x >> 4) + 16 * j;
      *reinterpret_cast<u32x4*>(ws + rr * MG_P + piece * 8) = wr[j];
      *reinterpret_cast<u32x4*>(xs + rr * MG_P + piece * 8) = xr[j];
      if constexpr (HILO) *reinterpret_cast<u32x4*>(xls + rr * MG_P + piece * 8) = xlr[j];
    }
    __syncthreads();
    if (kc + MG_KC < k_end) load(kc + MG_KC);  // next chunk in flight during the MFMAs
    const int kw = min(MG_KC, k_end - kc);
    for (int k = 0; k < kw; k += 16) {
      const h8 b = __builtin_bit_cast(h8, ld16(wrd + k));
      acc = mfma(__builtin_bit_cast(h8, ld16(xrd + k)), b, acc);
      if constexpr (HILO) acc = mfma(__builtin_bit_cast(h8, ld16(xlrd + k)), b, acc);
    }
  }
  // ---- epilogues: acc[r] = C[token 32 tb + mfma_row(r, lane)][tile row 32 rb + lane % 32]
  const int col = nb + (GU ? (lane & 31) : 32 * rb + (lane & 31));
  const bool valid = col < N;
  if constexpr (EPI == EPI_PART) {
    if (valid) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * tb + mfma_row(r, lane);
        if (t < p.B) p.part[((size_t)blockIdx.y * p.B + t) * N + col] = acc[r];
      }
    }
  } else if constexpr (EPI == EPI_MASK) {
    const float bias = valid ? p.bias[col] : 0.f;
    const int W32 = p.ffn >> 5;
    bool any = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * tb + mfma_row(r, lane);
      const float v = (col < p.hot_prefix) ? __builtin_inff() : acc[r] + bias;  // hot prefix: +inf
      const bool bit = valid && t < p.B && v > p.threshold;
      any |= bit;
      const uint64_t bal = __ballot(bit);
      if (p.mask_tok != nullptr && (lane & 31) == 0 && t < p.B)
        p.mask_tok[(size_t)t * W32 + ((nb + 32 * rb) >> 5)] = (uint32_t)(bal >> (lane & 32));
      if (p.logits != nullptr && valid && t < p.B) p.logits[(size_t)t * p.N + col] = v;
    }
    const uint64_t u = __ballot(any);
    const uint32_t u32 = (uint32_t)u | (uint32_t)(u >> 32);
    // the two token halves of a row block: OR through LDS
    if (tb == 1 && lane == 0) s_union[rb] = u32;
    __syncthreads();
    if (tb == 0 && lane == 0) p.mask_union[(nb + 32 * rb) >> 5] = u32 | s_union[rb];
  } else {  // EPI_ACT: a16[t][col] at compacted position col
    const int npad = (N + 15) & ~15;
    if constexpr (GU) {
      // up accumulators (rb = 1) meet the gate ones (rb = 0) through LDS (the tiles are free now)
      __syncthreads();
      float* ex = reinterpret_cast<float*>(smem);  // [2 tb][16 r][64 lanes]
      if (rb == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ex[(tb * 16 + r) * WAVE + lane] = acc[r];
      }
      __syncthreads();
      if (rb == 0 && col < npad) {
        const int nid = valid ? (p.idx != nullptr ? p.idx[col] : col) : 0;
        const float bias = valid ? p.bias[nid] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * tb + mfma_row(r, lane);
          const float up = ex[(tb * 16 + r) * WAVE + lane];
          const float a = (valid && t < p.B && tok_keeps(p, t, nid)) ? fmaxf(acc[r] + bias, 0.f) * up : 0.f;
          if (t < p.B) p.a16[(size_t)t * p.lda + col] = (half_t)a;
        }
      }
    } else if (col < npad) {
      const int nid = valid ? (p.idx != nullptr ? p.idx[col] : col) : 0;
      const float bias = valid ? p.bias[nid] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * tb + mfma_row(r, lane);
        const float a = (valid && t < p.B && tok_keeps(p, t, nid)) ? act_one<ACT>(acc[r] + bias) : 0.f;
        if (t < p.B) p.a16[(size_t)t * p.lda + col] = (half_t)a;
      }
    }
  }
}

// Arguments of the batched down projection part[ks][t][c] = sum over the positions k of split
// ks of a16[t][k] * w_down_t[idx[k]][c].
struct MmDown {
  const half_t* a16;     // [Bp][lda]
  int lda, B;
  const half_t* wd;      // [ffn][d] fp16 rows
  const int32_t* idx;
  const int32_t* n_dev;
  int ffn, d;
  int ks_len;            // positions per K split (multiple of 16, at most MD_SPLIT_MAX)
  float* part;           // [KS][B][d]
};

// ---------------------------------------------------------------------------------------
// k_mm_down: the down projection. A pair of waves owns 128 output columns (4 per lane of a
// half-wave: one 8-byte load per row); wave w takes tokens 32*(w&1).. of them, so each wave
// holds 32 x 128 accumulators. It walks its workgroup's K split 32 positions per step: lanes
// of half h load rows k + 8h .. k + 8h + 7 (and the same of the next 16), so each lane holds
// the 8 K values of its 4 columns and feeds four MFMAs whose output columns are {4*(l%32) + j}.
// Both 16-position steps' rows and activations are in flight together; the split's index
// list is staged in LDS first. (The two waves of a pair read the same rows: the second read
// is served by the caches.)
// ---------------------------------------------------------------------------------------
constexpr int MD_SPLIT_MAX = 4096;  // positions of one K split
constexpr int MD_COLS = 256;        // output columns per workgroup

__global__ __launch_bounds__(BLOCK) void k_mm_down(MmDown p) {
  __shared__ int s_idx[MD_SPLIT_MAX];
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int n = min(max(*p.n_dev, 0), p.ffn);
  const int c0 = blockIdx.x * MD_COLS + (wave >> 1) * 128 + 4 * (lane & 31);
  const int t = 32 * (wave & 1) + (lane & 31);  // this lane's token row of the A operand
  const bool cvalid = c0 < p.d;
  const int kh = 8 * (lane >> 5);
  const int k_begin = blockIdx.y * p.ks_len;
  const int len = max(0, min(n, k_begin + p.ks_len) - k_begin);  // <= ks_len <= MD_SPLIT_MAX
  for (int j = threadIdx.x; j < len; j += BLOCK) {
    const int i = p.idx[k_begin + j];
    s_idx[j] = ((unsigned)i < (unsigned)p.ffn) ? i : -1;
  }
  __syncthreads();
  f16v acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = (f16v){};
  // 32 positions (two 16-position MFMA steps) per block; blocks are ping-ponged between two
  // register sets so the next block's rows are in flight while the current one is used
  auto load = [&](uint64_t (&v)[2][8], h8 (&a)[2], int k) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = k + 16 * st + kh + e;
        const int i = (kk < len) ? s_idx[kk] : -1;
        v[st][e] = (i >= 0 && cvalid) ? *reinterpret_cast<const uint64_t*>(p.wd + (size_t)i * p.d + c0) : 0ull;
      }
      // a step past the split's end loads nothing (its positions would run past lda)
      a[st] = (k + 16 * st < len && t < p.B)
                  ? __builtin_bit_cast(h8, ld16(p.a16 + (size_t)t * p.lda + k_begin + k + 16 * st + kh))
                  : (h8){};
    }
  };
  auto use = [&](const uint64_t (&v)[2][8], const h8 (&a)[2], int k) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (k + 16 * st >= len) break;
      h8 bj[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (uint32_t)v[st][e], hi = (uint32_t)(v[st][e] >> 32);
        bj[0][e] = __builtin_bit_cast(half_t, (uint16_t)(lo & 0xFFFFu));
        bj[1][e] = __builtin_bit_cast(half_t, (uint16_t)(lo >> 16));
        bj[2][e] = __builtin_bit_cast(half_t, (uint16_t)(hi & 0xFFFFu));
        bj[3][e] = __builtin_bit_cast(half_t, (uint16_t)(hi >> 16));
      }
      h8 av = a[st];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + 16 * st + kh + e >= len) av[e] = (half_t)0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma(av, bj[j], acc[j]);
    }
  };
  uint64_t v0[2][8], v1[2][8];
  h8 a0[2], a1[2];
  if (len > 0) load(v0, a0, 0);
  for (int k = 0; k < len; k += 64) {
    if (k + 32 < len) load(v1, a1, k + 32);
    use(v0, a0, k);
    if (k + 64 < len) load(v0, a0, k + 64);
    if (k + 32 < len) use(v1, a1, k + 32);
  }
  if (!cvalid) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tr = 32 * (wave & 1) + mfma_row(r, lane);
    if (tr < p.B) {
      float* o = p.part + ((size_t)blockIdx.y * p.B + tr) * p.d + c0;
      *reinterpret_cast<f32x4*>(o) = (f32x4){acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
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
