// Attention parameters shared by the generic and the MFMA attention kernels.
#pragma once

#include "common.hpp"

namespace csa {

struct AttnParams {
  int H, d_nope, d_rope, q_dt, o_dt, nope_dt, rope_dt, m;
  double base;
  int64_t cap;
  int64_t window;          // dense: attend the last `window` visible entries (0: all)
  int qk_mode;             // 0, or CSA_FP8E4M3: the query's non-RoPE dims as MXFP8 against the FP8 codes
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
  Pages pg;           // KV placement (contiguous or paged)
  int64_t span_rows;  // rows one gather descriptor covers: cap from the sequence's first row, or the whole pool
  int64_t seq_stride; // rows from one sequence's first row to the next's: cap, or 0 when paged
  bool list_rows;     // sparse lists already hold pool rows (paged: turned by page_rows_kernel)
};

// MFMA path (64 heads, 512 + 64 dims, BF16 q, BF16 / FP8 cache).
bool mfma_attn_supported(const AttnParams& P);
// false when a sequence's cache rows would need byte offsets of 2^31 or more
bool mfma_attn_capacity_ok(const AttnParams& P);
int launch_mfma_attn(const AttnParams& P, int op, int B, hipStream_t s);
size_t mfma_attn_ws_bytes(const csa_attn_desc* d, int op, int B, int T, int64_t pos0, int k);
// BF16-cache kernel of the MFMA path over B sequences (T queries each, or
// `splits` entry ranges of `per` entries when part != NULL, which then
// receives the split partials).
void launch_attn_bf16(const AttnParams& P, bool dense, int B, hipStream_t s, int splits, int64_t per, void* part);

// host: a sparse decode call's validation and parameters, and the launch of
// any attention op (routes to the MFMA path or the generic kernel)
int sparse_attn_decode_setup(const csa_attn_desc* desc, int B, const int64_t* pos, const void* q, const csa_cache* kv,
                             const int32_t* idx, int k, float softmax_scale, void* o, float* lse, void* ws,
                             size_t ws_bytes, AttnParams* out);
int attn_dispatch(AttnParams& P, int op, int B, void* stream);
size_t attn_ws_bytes(const csa_attn_desc* d, int op, int B, int T, int64_t pos0, int k);
// paged sparse attention on the MFMA path: bytes of the list turned into pool
// rows, and where in P.ws that list goes (NULL when the call needs none or
// the workspace lacks room)
size_t page_list_bytes(const csa_attn_desc* d, int op, int B, int T, int k);
int32_t* page_list_slot(const AttnParams& P, int op, int B);

}  // namespace csa
