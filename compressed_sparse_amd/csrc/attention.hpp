// Attention parameters shared by the generic and the MFMA attention kernels.
#pragma once

#include "common.hpp"

namespace csa {

struct AttnParams {
  int H, d_nope, d_rope, q_dt, o_dt, nope_dt, rope_dt, m;
  double base;
  int64_t cap;
  int T;
  int64_t pos0;
  const int64_t* pos_dev;  // decode: per-sequence positions (T == 1)
  const void* q;
  const void *nope, *scale, *rope;
  const int32_t* idx;      // CSA: [B][T][k]; HCA: NULL
  int k;
  float scale_qk;
  void* o;
  float* lse;
  void* ws;
  size_t ws_bytes;
};

// MFMA path (64 heads, 512 + 64 dims, BF16 q, BF16 / FP8 cache).
bool mfma_attn_supported(const AttnParams& P);
int launch_mfma_attn(const AttnParams& P, int op, int B, hipStream_t s);
size_t mfma_attn_ws_bytes(const csa_attn_desc* d, int op, int B, int T, int64_t pos0, int k);
// BF16-cache kernel of the MFMA path over B sequences (T queries each, or
// `splits` entry ranges of `per` entries when part != NULL, which then
// receives the split partials).
void launch_attn_bf16(const AttnParams& P, bool dense, int B, hipStream_t s, int splits, int64_t per, void* part);

}  // namespace csa
