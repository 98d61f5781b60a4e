// Compressor parameters shared by the compressor kernels and the fused
// decode step.
#pragma once

#include "common.hpp"
#include "index.hpp"

namespace csa {

struct CompressParams {
  int m, overlap, d_nope, d_rope, c, in_dt, nope_dt, rope_dt;
  int R, NT;
  double base;
  int64_t cap;
  // prefill: token rows [pos0, pos0 + T) of a/za/b/zb; decode: one row each
  int T;
  int64_t pos0;
  const void *a, *za, *b, *zb;
  const float *Ba, *Bb;
  void *nope, *scale, *rope;
  float* ring;
  Pages pg;  // entry placement (contiguous or paged)
};

enum { RING_A = 0, RING_ZA = 1, RING_B = 2, RING_ZB = 3 };

// host: a cache descriptor and its buffers checked; the compressor
// parameters of a cache (no token inputs; biases Ba, Bb)
int compress_validate_cache(const csa_cache_desc* d, const csa_cache* c);
CompressParams compress_make_params(const csa_cache_desc* d, const csa_cache* c, const float* Ba, const float* Bb);

// host: validation of a decode call's arguments and its parameters
int compress_decode_setup(const csa_cache_desc* d, int B, const int64_t* pos, const void* a, const void* b,
                          const void* za, const void* zb, const float* Ba, const float* Bb, const csa_cache* cache,
                          CompressParams* out);
// host: one decode compressor launch
int launch_compress_decode(const CompressParams& P, int B, const int64_t* pos, hipStream_t s);
// host: the first launch of a fused CSA decode step: both compressors (KV
// entries and indexer keys) and the indexer's per-row preparation (cleared
// histogram and candidate count; MXFP4 query operands when mx_prep).
// Requires both caches to take the same input type.
int launch_decode_step_prep(const CompressParams& kv, const CompressParams& keys, const IndexParams& ip, bool mx_prep,
                            int B, const int64_t* pos, hipStream_t s);

}  // namespace csa
