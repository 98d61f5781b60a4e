// Lightning-indexer parameters shared by the generic and the MFMA kernels.
#pragma once

#include "common.hpp"

namespace csa {

struct IndexParams {
  int H, D, q_dt, qk_dt, key_dt, score_dt, m;
  int64_t cap;
  int T;
  int64_t pos0;
  const int64_t* pos_dev;  // decode: per-sequence positions (T == 1)
  const void* qI;
  const float* w;
  const void* knope;
  const void* kscale;
  int k;
  int32_t* idx;
  float* scores_out;  // optional [B][T][cap]
  float* ws;          // [B][T][n_stride] score rows
  int64_t n_stride;
};

bool index_mfma_supported(const IndexParams& P);
bool index_fused_prefill_ok(const IndexParams& P, int64_t n_max);
int launch_index_fused_prefill(const IndexParams& P, int B, hipStream_t s);
int launch_index_scan(const IndexParams& P, int B, int64_t n_max, hipStream_t s);

}  // namespace csa
