// Shared device helpers (number formats, RoPE angles, reductions) and host
// helpers (validation, error reporting) of the CSA / HCA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "csa.h"

namespace csa {

// ---------------------------------------------------------------------------
// host side: error reporting
// ---------------------------------------------------------------------------
void set_error(const std::string& msg);
int fail(int status, const std::string& msg);
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int dtype_size(int dt) {
  switch (dt) {
    case CSA_F32: return 4;
    case CSA_BF16: return 2;
    case CSA_FP8E4M3: return 1;
    default: return 0;
  }
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// device side: element formats
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// OCP E4M3 byte -> fp32 (the NaN code never occurs in caches we write).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t mt = c & 0x7u;
  float v;
  if (e == 0) {
    v = static_cast<float>(mt) * 0.001953125f;  // m * 2^-9
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (mt << 20));  // (1 + m/8) * 2^(e-7)
  }
  return __uint_as_float(__float_as_uint(v) | s);
}

// fp32 -> OCP E4M3 byte, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(x);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9
    uint32_t q = static_cast<uint32_t>(rintf(a * 512.0f));  // exact scaling, RNE
    return sign | q;                                         // q == 8 is the min normal code
  }
  uint32_t au = __float_as_uint(a);
  int E = static_cast<int>((au >> 23) & 0xFFu) - 127;
  uint32_t m23 = au & 0x7FFFFFu;
  uint32_t r = m23 >> 20;
  uint32_t rem = m23 & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 8u) { r = 0; ++E; }
  uint32_t code = (static_cast<uint32_t>(E + 7) << 3) | r;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// E2M1 code (4 bits, bit 3 = sign) -> fp32, assembled bitwise (no table,
// no branches): magnitudes 0, 0.5 and, for m >= 2, (1 + (m & 1) / 2) *
// 2^((m >> 1) - 1), i.e. 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  const uint32_t mag = m >= 2u ? (((m >> 1) + 126u) << 23) | ((m & 1u) << 22) : (m ? 0x3F000000u : 0u);
  return __uint_as_float(mag | ((c & 8u) << 28));
}

// fp32 (already divided by the block scale) -> E2M1 code, RNE, clamped to 6:
// the magnitude code counts the rounding boundaries at or below |x| (ties
// go to the even code), NaN gives 7.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const float a = fabsf(x);
  const uint32_t n = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                     static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                     static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                     static_cast<uint32_t>(a > 5.0f);
  const uint32_t c = a == a ? n : 7u;
  return (x < 0.0f && c != 0u) ? (c | 8u) : c;
}

// OCP MX shared exponent for E2M1 elements: floor(log2 amax) - 2 in [-127, 127].
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  uint32_t u = __float_as_uint(amax);
  int e = static_cast<int>((u >> 23) & 0xFFu);
  int E = (e == 0) ? -127 : e - 127;  // fp32 subnormal amax: smallest scale
  E -= 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

__device__ __forceinline__ float exp2i(int e) { return ldexpf(1.0f, e); }

// Load one element of a float/bf16 tensor as fp32.
__device__ __forceinline__ float load_elem(const void* p, size_t i, int dt) {
  return dt == CSA_BF16 ? bf16_to_f32(static_cast<const bf16_t*>(p)[i])
                        : static_cast<const float*>(p)[i];
}

// RoPE angle pos * base^(-2p/d_rope) formed in fp64 and turned into fp32
// sine/cosine through fp64 sin/cos.
__device__ __forceinline__ void rope_sincos(int64_t pos, int p, int d_rope, double base,
                                            float* s, float* c) {
  double theta = pow(base, -2.0 * static_cast<double>(p) / static_cast<double>(d_rope));
  double ang = static_cast<double>(pos) * theta;
  double sd, cd;
  sincos(ang, &sd, &cd);
  *s = static_cast<float>(sd);
  *c = static_cast<float>(cd);
}

// ---------------------------------------------------------------------------
// device side: reductions over a workgroup of blockDim.x threads (<= 1024)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// red: __shared__ float[32] scratch.  All threads get the result.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = 0.0f;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}


// ---------------------------------------------------------------------------
// entry placement: contiguous or paged caches
// ---------------------------------------------------------------------------
// Where entry s of sequence b lives.  Contiguous caches keep sequence b at
// rows [b*cap, (b+1)*cap).  Paged caches keep it at row pg*2^shift + s mod
// 2^shift of a pool of `pool` pages, pg = table[b][s >> shift]; a table
// entry outside [0, pool) maps to row -1 (not written; readers clamp it).
struct Pages {
  const int32_t* table;  // [B][tps] when paged, NULL when contiguous
  int shift;             // log2 entries per page
  int64_t tps;           // table entries per sequence (cap >> shift)
  int64_t pool;          // pages in the pool
};

__device__ __forceinline__ int64_t entry_row(const Pages& pg, int64_t cap, int b, int64_t s) {
  if (!pg.table) return static_cast<int64_t>(b) * cap + s;
  const int64_t p = pg.table[static_cast<int64_t>(b) * pg.tps + (s >> pg.shift)];
  if (p < 0 || p >= pg.pool) return -1;
  return (p << pg.shift) | (s & ((int64_t(1) << pg.shift) - 1));
}

// Rows a cache's buffers hold: B*cap contiguous, pool*2^shift paged.
inline int64_t cache_rows(const Pages& pg, int B, int64_t cap) {
  return pg.table ? (pg.pool << pg.shift) : static_cast<int64_t>(B) * cap;
}

// host: checks the paging fields of a descriptor against the cache's block
// table and fills `out`.  page_size 0: contiguous (table must be NULL).
int make_pages(int32_t page_size, int64_t pool_pages, int64_t capacity, const int32_t* table, Pages* out);
// host: the paging fields alone (workspace queries, which see no buffers)
int check_paging(int32_t page_size, int64_t pool_pages, int64_t capacity);

}  // namespace csa
