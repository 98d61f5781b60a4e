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
  // decode multi-workgroup top-k (NULL otherwise): per-row histogram of the
  // top 11 key bits, candidate count, candidate (key, index) lists and, per
  // CAND_CHUNK-entry chunk, where its index-ordered candidates start and how
  // many there are
  int* ghist;         // [B][HIST_BINS]
  int* ccount;        // [B]
  uint32_t* ckey;     // [B][CAND_CAP]
  int32_t* cidx;      // [B][CAND_CAP]
  int* cbase;         // [B][nch]
  int* ccnt;          // [B][nch]
  int nch;            // chunks per row: ceil(cap / CAND_CHUNK)
  int* csel;          // [B][2]: the histogram bin of the k-th key, keys in higher bins
  // MXFP4 scan: per query row the A operand of the scaled MFMA, 64 lanes x
  // 16 bytes of E2M1 codes, then 64 int32 E8M0 scales (QPACK_ROW_BYTES)
  uint8_t* qpack;
  Pages pg;  // key placement (contiguous or paged)
  // fused decode step over a paged KV cache (NULL otherwise): the final
  // top-k pass also writes each selected entry's row of that cache
  int32_t* rows_out;  // [B][k]
  Pages row_pg;
  int64_t row_cap;
};

constexpr int HIST_BITS = 11;
constexpr int HIST_BINS = 1 << HIST_BITS;
constexpr int CAND_CAP = 8192;    // candidates one row may keep in LDS
constexpr int CAND_CHUNK = 4096;  // entries per candidate workgroup
constexpr int NCH_MAX = 4096;     // chunks per row the final pass can order (cap <= 16M entries)

// First row of a key block that starts at entry s (wave-uniform) of
// sequence b and lies inside one page: contiguous keys are rows b*cap + s;
// paged ones take the page from one scalar table load (a page outside the
// pool reads as page 0).
__device__ __forceinline__ int64_t key_block_row(const IndexParams& P, int b, int64_t s) {
  if (!P.pg.table) return static_cast<int64_t>(b) * P.cap + s;
  typedef const __attribute__((address_space(4))) int32_t ctab_t;
  const int64_t ix = static_cast<int64_t>(b) * P.pg.tps + (s >> P.pg.shift);
  const int64_t pg = reinterpret_cast<ctab_t*>(reinterpret_cast<uintptr_t>(P.pg.table))[ix];
  return ((pg >= 0 && pg < P.pg.pool ? pg : 0) << P.pg.shift) | (s & ((int64_t(1) << P.pg.shift) - 1));
}

// Order-preserving key of a score: larger score -> larger key; -0 == +0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the wave's lanes (row shifts within 16 lanes,
// then the row broadcasts): DPP moves, no LDS round trips
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// LDS histogram increment, aggregated over the lanes of a wave that hit the
// same bin (scores concentrate in a few high-bit bins); after a few rounds
// the remaining lanes (spread bins, little contention) add one by one.
__device__ __forceinline__ void wave_hist_add(int* hist, int bin, bool active) {
  const int lane = threadIdx.x & 63;
  for (int round = 0; round < 4; ++round) {
    const unsigned long long act = __ballot(active);
    if (act == 0ull) return;
    const int leader = __ffsll(static_cast<long long>(act)) - 1;
    const int lb = __builtin_amdgcn_readlane(bin, leader);
    const unsigned long long same = __ballot(active && bin == lb);
    if (lane == leader) atomicAdd(&hist[lb], __popcll(same));
    if (bin == lb) active = false;
  }
  if (active) atomicAdd(&hist[bin], 1);
}

constexpr int QPACK_ROW_BYTES = 64 * 16 + 64 * 4;

bool index_mfma_supported(const IndexParams& P);
// MXFP4 keys and query: the scaled-MFMA scan, which needs
// launch_index_mx_prep (query operands; for decode also the cleared
// histogram and candidate count) before it
bool index_scan_mx(const IndexParams& P);
int launch_index_mx_prep(const IndexParams& P, int rows, hipStream_t s);
bool index_fused_prefill_ok(const IndexParams& P, int64_t n_max);
int launch_index_fused_prefill(const IndexParams& P, int B, hipStream_t s);
// prefill rows of at most FUSED_NMAX entries whose scores a scan kernel
// wrote to the workspace: the fused kernel's select alone
bool index_ws_select_ok(const IndexParams& P, int64_t n_max);
int launch_index_ws_select(const IndexParams& P, int B, hipStream_t s);
int launch_index_scan(const IndexParams& P, int B, int64_t n_max, hipStream_t s);

// host: a decode call's validation and parameters (workspace carved), and
// its launches; with prep_done the per-row preparation is skipped (a fused
// decode step has enqueued it).  index_decode_prep_mx: whether that
// preparation forms MXFP4 query operands.
int index_decode_setup(const csa_index_desc* desc, int B, const int64_t* pos, const void* qI, const float* w,
                       const csa_cache* keys, int k, int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                       IndexParams* out);
bool index_decode_prep_mx(const IndexParams& P);
int launch_index_decode(IndexParams& P, int B, void* stream, bool prep_done);
size_t index_ws_bytes(const csa_index_desc* d, int op, int B, int T, int64_t pos0);

}  // namespace csa
