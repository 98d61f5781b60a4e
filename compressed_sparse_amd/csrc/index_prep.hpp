// Per-row preparation of the lightning indexer (device functions shared by
// the indexer's prep kernel and the fused decode step): the query's MXFP4
// operand for the scaled-MFMA scan, and the decode top-k's cleared row
// state.  [CSA/HCA 混注意力] §1.4 LIGHTNING INDEXER 的 FP4 计 (FP4 QK).
#pragma once

#include "index.hpp"

namespace csa {

constexpr int PREP_HI = 16;  // indexer heads of the MXFP4 scan
constexpr int PREP_DI = 64;  // indexer dims

// One wave rounds query row r to MXFP4 (per head and 32-dim block: the OCP
// MX shared exponent e of the block's largest magnitude, E2M1 codes of
// q / 2^e) and stores it as the A operand of the scaled 32x32x64 MFMA: lane
// l holds head l % 32 (heads 16.. are zero) and dims 32 (l / 32) .. +32, 16
// bytes of codes (low nibble first), and the E8M0 byte e + 127.
__device__ __forceinline__ void mx_prep_row(const IndexParams& P, size_t r) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int h = lane & 31, kb = lane >> 5;
  u32x4_t codes = {0u, 0u, 0u, 0u};
  int e8 = 127;
  if (h < PREP_HI) {
    const u32x4_t* src =
        reinterpret_cast<const u32x4_t*>(static_cast<const bf16_t*>(P.qI) + (r * PREP_HI + h) * PREP_DI + 32 * kb);
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t v = src[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = bf16_to_f32(static_cast<bf16_t>(v[j] & 0xFFFFu));
        x[8 * i + 2 * j + 1] = bf16_to_f32(static_cast<bf16_t>(v[j] >> 16));
      }
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(x[i]));
    const int ex = mx_exponent(am);
    const float inv = exp2i(-ex);
#pragma unroll
    for (int i = 0; i < 32; ++i) codes[i >> 3] |= f32_to_e2m1(x[i] * inv) << (4 * (i & 7));
    e8 = ex + 127;
  }
  uint8_t* dst = P.qpack + r * QPACK_ROW_BYTES;
  reinterpret_cast<u32x4_t*>(dst)[lane] = codes;
  reinterpret_cast<int*>(dst + 64 * 16)[lane] = e8;
}

// The decode top-k state of row r cleared: histogram and candidate count
// (all threads of the workgroup take part).
__device__ __forceinline__ void clear_decode_row(const IndexParams& P, size_t r) {
  for (int i = threadIdx.x; i < HIST_BINS; i += blockDim.x) P.ghist[r * HIST_BINS + i] = 0;
  if (threadIdx.x == 0) P.ccount[r] = 0;
}

}  // namespace csa
