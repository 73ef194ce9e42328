// Device helpers for the gfx950 (CDNA4, wave64) kernels of the sparse FFN.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pi {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int BLOCK = 256;  // 4 waves per workgroup everywhere
constexpr int NWAVES = BLOCK / WAVE;

// 16-byte streaming load of weights: each weight byte is used once per call, so the
// nontemporal hint keeps it from displacing x, partial sums and mask words in the caches.
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Loads whose value is replaced by zeros where !ok. The load is always issued, so p must be
// readable either way (callers clamp the index). Written as `ok ? load : 0`, the compiler
// puts a branch around the load and copies its result register inside that branch, and the
// copy waits for the load to arrive: loads meant to be in flight together then go out one
// round trip at a time.
__device__ __forceinline__ u32x4 ld16_or0(const void* p, bool ok) {
  const u32x4 v = ld16(p);
  return ok ? v : (u32x4){0, 0, 0, 0};
}
__device__ __forceinline__ u32x4 ld_stream_or0(const void* p, bool ok) {
  const u32x4 v = ld_stream(p);
  return ok ? v : (u32x4){0, 0, 0, 0};
}

// fp16 x fp16 pair dot product accumulated in fp32 (v_dot2c_f32_f16). Products of two fp16
// values are exact in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ float h2f_lo(uint32_t u) {
  return (float)__builtin_bit_cast(half2_t, u).x;
}
__device__ __forceinline__ float h2f_hi(uint32_t u) {
  return (float)__builtin_bit_cast(half2_t, u).y;
}
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// a where the lane's mask m is all ones, b where it is zero, as bit operations on the
// values. With plain `?:` selects over an array, the compiler turned the exchange steps below
// into indexed reads of the whole array (a compare-and-select chain per value, or scratch):
// about 1300 instructions for one 16-row reduction instead of about 100. (Written as inline
// v_bfi_b32 instead, the instruction escaped the compiler's hazard checks after v_dot2c and
// read a partly accumulated sum.)
__device__ __forceinline__ float bfi_sel(uint32_t m, float a, float b) {
  const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
  return __builtin_bit_cast(float, (ua & m) | (ub & ~m));
}

// Sum R per-lane partial rows over the 64 lanes of a wave with 2R-1+log2(64/R) shuffles:
// each exchange step halves the rows a lane carries. On return every lane holds the full
// sum of row (lane & (R-1)).
template <int R>
__device__ __forceinline__ float transpose_reduce(float (&acc)[R], int lane) {
#pragma unroll
  for (int o = R / 2; o >= 1; o >>= 1) {
    const uint32_t hi = (lane & o) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < o; ++i) {
      const float send = bfi_sel(hi, acc[i], acc[i + o]);
      const float keep = bfi_sel(hi, acc[i + o], acc[i]);
      acc[i] = keep + __shfl_xor(send, o, WAVE);
    }
  }
  float v = acc[0];
#pragma unroll
  for (int o = R; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// transpose_reduce over the lanes that agree in their low S bits: lane groups of 2^S lanes
// carry different columns. On return every lane holds the full sum (over the 64 >> S lanes
// of its group) of value ((lane >> S) & (R-1)).
template <int R, int S>
__device__ __forceinline__ float transpose_reduce_s(float (&acc)[R], int lane) {
#pragma unroll
  for (int o = R / 2; o >= 1; o >>= 1) {
    const uint32_t hi = (lane & (o << S)) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < o; ++i) {
      const float send = bfi_sel(hi, acc[i], acc[i + o]);
      const float keep = bfi_sel(hi, acc[i + o], acc[i]);
      acc[i] = keep + __shfl_xor(send, o << S, WAVE);
    }
  }
  float v = acc[0];
#pragma unroll
  for (int o = R << S; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Block-wide sum of one float per thread (BLOCK threads). Uses `red` [NWAVES] in LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) s += red[i];
  return s;
}

// Exclusive prefix sum of one int per thread over the block (NW waves, BLOCK threads by
// default); returns the thread's exclusive prefix and writes the block total to *total.
// `red` [NW] ints in LDS.
template <int NW = NWAVES>
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  int incl = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    int t = __shfl_up(incl, o, WAVE);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == WAVE - 1) red[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) base += red[i];
    tot += red[i];
  }
  *total = tot;
  return base + incl - v;
}

// Position of the r-th (0-based) set bit of w; r < popcount(w).
__device__ __forceinline__ int select_bit(uint64_t w, int r) {
  int pos = 0;
  uint32_t x = (uint32_t)w;
  int c = __popc(x);
  if (r >= c) { r -= c; pos = 32; x = (uint32_t)(w >> 32); }
  c = __popc(x & 0xFFFFu); if (r >= c) { r -= c; pos += 16; x >>= 16; }
  c = __popc(x & 0xFFu);   if (r >= c) { r -= c; pos += 8;  x >>= 8; }
  c = __popc(x & 0xFu);    if (r >= c) { r -= c; pos += 4;  x >>= 4; }
  c = __popc(x & 0x3u);    if (r >= c) { r -= c; pos += 2;  x >>= 2; }
  c = (int)(x & 1u);       if (r >= c) { pos += 1; }
  return pos;
}

// ---- Q4_0 block arithmetic -------------------------------------------------------------
// A block is 16 code bytes: byte j holds element j (low nibble) and element j+16 (high
// nibble). (q - 8) is rebuilt exactly in fp16 as (0x6400 | q) - 1032 = (1024 + q) - 1032.

// Two fp16 (q-8) values from bytes (sel) of a nibble-masked dword.
__device__ __forceinline__ uint32_t q4_pair(uint32_t nib, uint32_t sel) {
  uint32_t h = __builtin_amdgcn_perm(0x64646464u, nib, sel);
  half2_t v = __builtin_bit_cast(half2_t, h) - (half2_t){(half_t)1032.0f, (half_t)1032.0f};
  return __builtin_bit_cast(uint32_t, v);
}
constexpr uint32_t SEL_B01 = 0x04010400u;  // bytes 0,1 -> halves (lo, hi)
constexpr uint32_t SEL_B23 = 0x04030402u;  // bytes 2,3

// The block's (q_e - 8) as 16 fp16 pairs in element order: dword m holds elements 2m, 2m+1.
// A block's dot product with x is then sum_m dot2(out[m], x pair m), exact products.
__device__ __forceinline__ void q4_block_unpack(u32x4 codes, uint32_t (&out)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = codes[j];
    const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
    out[2 * j] = q4_pair(lo, SEL_B01);
    out[2 * j + 1] = q4_pair(lo, SEL_B23);
    out[8 + 2 * j] = q4_pair(hi, SEL_B01);
    out[8 + 2 * j + 1] = q4_pair(hi, SEL_B23);
  }
}

// Codes of a block as 32 floats in element order (element e = q_e, not yet offset).
__device__ __forceinline__ void q4_block_codes(u32x4 codes, float (&q)[32]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = codes[j];
    const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
    q[4 * j + 0] = (float)((lo >> 0) & 0xFFu);
    q[4 * j + 1] = (float)((lo >> 8) & 0xFFu);
    q[4 * j + 2] = (float)((lo >> 16) & 0xFFu);
    q[4 * j + 3] = (float)((lo >> 24) & 0xFFu);
    q[16 + 4 * j + 0] = (float)((hi >> 0) & 0xFFu);
    q[16 + 4 * j + 1] = (float)((hi >> 8) & 0xFFu);
    q[16 + 4 * j + 2] = (float)((hi >> 16) & 0xFFu);
    q[16 + 4 * j + 3] = (float)((hi >> 24) & 0xFFu);
  }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(half_t, h);
}

}  // namespace pi
