// Entry storage shared by the compressor kernels and the projection's
// finalize pass: the per-channel softmax batch and the lane-parallel RoPE +
// storage-format epilogue of one entry.  [CSA/HCA 混注意力] §1.1 工程细节,
// §1.4 存储格式混 (RoPE dims BF16, the rest FP8).
#pragma once

#include "compress.hpp"

namespace csa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int CW_ROWS = 4;  // window rows per softmax batch

// One batch of a window's softmax for one channel: logits lg (-inf past the
// window) and values vv of CW_ROWS rows folded into the running max mx,
// weight sum sw and weighted sum acc, with one rescale per batch.  Every
// path (prefill kernels, decode) goes through this, in the same row order,
// so they agree bit for bit.
__device__ __forceinline__ void softmax_batch(const float (&lg)[CW_ROWS], const float (&vv)[CW_ROWS], float& mx,
                                              float& sw, float& acc) {
  float bm = lg[0];
#pragma unroll
  for (int u = 1; u < CW_ROWS; ++u) bm = fmaxf(bm, lg[u]);
  const float nm = fmaxf(mx, bm);
  const float sc = __expf(mx - nm);  // 0 on the first batch
  float s = 0.0f, a = 0.0f;
#pragma unroll
  for (int u = 0; u < CW_ROWS; ++u) {
    const float e = __expf(lg[u] - nm);  // 0 past the window
    s += e;
    a = fmaf(e, vv[u], a);
  }
  sw = fmaf(sw, sc, s);
  acc = fmaf(acc, sc, a);
  mx = nm;
}

// Lanes per entry: enough for the 8-channel groups and the RoPE pairs, a
// power of two, so that a wave holds 64 / lanes entries.
__host__ __device__ inline int wave_lanes_per_entry(int ng, int np) {
  const int need = ng > np ? ng : np;
  int l = 1;
  while (l < need) l <<= 1;
  return l;
}

// RoPE and storage of entry i of sequence b by the lpe lanes that hold it:
// lane ll holds channels 8ll .. 8ll+7 in x[0..8) (hg: ll < d_nope / 8) and
// the RoPE pair ll in x[8..10) (hp: ll < d_rope / 2); ok: the entry exists.
// The pair turns at the entry's last position; FP8 / MXFP4 scales reduce over
// the entry's lanes by shuffles, so every lane of the wave must call it.
__device__ __forceinline__ void store_entry_lanes(const CompressParams& P, int b, int64_t i, bool ok, bool hg, bool hp,
                                                  int ll, int lpe, float (&x)[10]) {
  const int jg = 8 * ll;
  // RoPE of the pair at the entry's last position
  if (hp) {
    float sn, co;
    rope_sincos(i * P.m + P.m - 1, ll, P.d_rope, P.base, &sn, &co);
    const double x0 = x[8], x1 = x[9];
    x[8] = static_cast<float>(x0 * co - x1 * sn);
    x[9] = static_cast<float>(x0 * sn + x1 * co);
  }
  // the entry's row; lanes of an entry whose page lies outside the pool store nothing
  const int64_t er = ok ? entry_row(P.pg, P.cap, b, i) : -1;
  const bool sg = hg && er >= 0, sp = hp && er >= 0, so = ok && er >= 0;
  const size_t e = er >= 0 ? static_cast<size_t>(er) : 0;
  switch (P.nope_dt) {
    case CSA_F32:
      if (sg) {
        float* dst = static_cast<float*>(P.nope) + e * P.d_nope + jg;
        *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
      }
      break;
    case CSA_BF16:
      if (sg) {
        u32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          o[c] = static_cast<uint32_t>(f32_to_bf16(x[2 * c])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * c + 1])) << 16);
        *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(P.nope) + e * P.d_nope + jg) = o;
      }
      break;
    case CSA_FP8E4M3: {
      float am = 0.0f;
      if (hg)
#pragma unroll
        for (int c = 0; c < 8; ++c) am = fmaxf(am, fabsf(x[c]));
      for (int o = 1; o < lpe; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));  // over the entry's lanes
      const float s = am > 0.0f ? am / 448.0f : 1.0f;
      if (sg) {
        uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          w0 |= f32_to_e4m3(x[c] / s) << (8 * c);
          w1 |= f32_to_e4m3(x[4 + c] / s) << (8 * c);
        }
        *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(P.nope) + e * P.d_nope + jg) = u32x2{w0, w1};
      }
      if (so && ll == 0) static_cast<float*>(P.scale)[e] = s;
      break;
    }
    case CSA_MXFP4: {
      // block of 32 channels = lanes 4k .. 4k+3
      float am = 0.0f;
      if (hg)
#pragma unroll
        for (int c = 0; c < 8; ++c) am = fmaxf(am, fabsf(x[c]));
      am = fmaxf(am, __shfl_xor(am, 1));
      am = fmaxf(am, __shfl_xor(am, 2));
      const int ex = mx_exponent(am);
      const float inv = exp2i(-ex);
      if (sg) {
        uint32_t wd = 0u;
#pragma unroll
        for (int c = 0; c < 8; ++c) wd |= f32_to_e2m1(x[c] * inv) << (4 * c);
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(P.nope) + e * (P.d_nope / 2) + 4 * ll) = wd;
        if ((ll & 3) == 0) static_cast<uint8_t*>(P.scale)[e * (P.d_nope / 32) + ll / 4] = static_cast<uint8_t>(ex + 127);
      }
      break;
    }
  }
  if (sp) {
    if (P.rope_dt == CSA_F32) {
      *reinterpret_cast<f32x2*>(static_cast<float*>(P.rope) + e * P.d_rope + 2 * ll) = f32x2{x[8], x[9]};
    } else {
      const uint32_t o = static_cast<uint32_t>(f32_to_bf16(x[8])) | (static_cast<uint32_t>(f32_to_bf16(x[9])) << 16);
      *reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(P.rope) + e * P.d_rope + 2 * ll) = o;
    }
  }
}

}  // namespace csa
