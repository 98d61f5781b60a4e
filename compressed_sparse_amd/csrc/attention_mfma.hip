// Dispatch of the MFMA attention path (64 query heads sharing one compressed
// entry of 512 non-RoPE + 64 RoPE dims, MQA; BF16 queries and outputs; BF16
// or FP8-with-scale cache) and the log-sum-exp merge of decode splits.
// [CSA/HCA 混注意力] §1.1, §1.2; [读完这篇] §三 CSA 步骤三; §1.4 存储格式混.
//
// Prefill runs one query per work item; decode splits each sequence's entry
// list (CSA) or visible entries (HCA) over several work items, each writing
// a partial (O normalised by its own weights, as BF16, and the log2 of its
// weight sum) that attn_merge_kernel combines.
#include <cmath>

#include "attention.hpp"

namespace csa {
namespace {

constexpr int NH = 64;       // heads
constexpr int DN = 512;      // value / non-RoPE dims
constexpr int DRP = 64;      // RoPE dims
constexpr int TILE = 64;     // entries per tile of the attention kernel
constexpr int MAX_SPLITS = 32;
constexpr int MAX_LIST = 1024;  // list entries one work item handles
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Combines split partials by log-sum-exp: O = sum_s 2^(l_s - M) O_s / sum_s
// 2^(l_s - M), l_s the split's log2 weight sum and M their maximum.  A
// split's partial O is stored in the attention kernel's register order:
// piece (w, mb, nb, jq) of 64 lanes x 8 bytes at 512 ((((w * 4 + mb) * 2 +
// nb) * 4 + jq)) + 8 lane, lane holding head 32nb + lane % 32 and value dims
// 128w + 32mb + 8jq + 4 (lane / 32) .. +4.  Grid (32 blocks (w, mb, nb), B),
// 256 threads: thread (jq, lane) reads one 8-byte piece of every split (2 KB
// contiguous per split and workgroup), the weights of the block's 32 heads
// are formed once in LDS (8 threads per head).  S >= splits is a power of
// two: every thread's S loads (clamped to the last split) are issued before
// the weights are known.
template <int S>
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnParams P, int splits, const void* part, int B) {
  __shared__ float s_f[32][S + 1];
  __shared__ float s_L[32], s_M[32];
  const int blk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int w = blk >> 3, mb = (blk >> 1) & 3, nb = blk & 1;
  const int jq = tid >> 6, lane = tid & 63;
  const int hl = lane & 31, h = 32 * nb + hl;
  const bf16_t* po = static_cast<const bf16_t*>(part) + static_cast<size_t>(b) * splits * (NH * DN) +
                     4 * ((blk * 4 + jq) * 64 + lane);
  uint2 v[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp)
    v[sp] = *reinterpret_cast<const uint2*>(po + static_cast<size_t>(min(sp, splits - 1)) * NH * DN);
  const float* pl = reinterpret_cast<const float*>(static_cast<const bf16_t*>(part) + static_cast<size_t>(B) * splits * (NH * DN)) +
                    static_cast<size_t>(b) * splits * NH;
  // each head's split weights: 8 threads per head (head tid / 8), thread
  // tid % 8 taking splits tid % 8, tid % 8 + 8, ..; maximum and sum over the
  // 8 by lane exchanges
  {
    constexpr int PS = S < 8 ? 1 : S / 8;  // splits per thread
    const int hh = tid >> 3, sub = tid & 7;
    float ls[PS], M = -INFINITY;
#pragma unroll
    for (int u = 0; u < PS; ++u) {
      const int sp = sub + 8 * u;
      ls[u] = sp < splits ? pl[sp * NH + 32 * nb + hh] : -INFINITY;
      M = fmaxf(M, ls[u]);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.0f;
#pragma unroll
    for (int u = 0; u < PS; ++u) {
      const int sp = sub + 8 * u;
      const float f = ls[u] != -INFINITY ? exp2f(ls[u] - M) : 0.0f;  // 0 past the last split and for empty splits
      if (sp < S) s_f[hh][sp] = f;
      L += f;
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) L += __shfl_xor(L, o);
    if (sub == 0) {
      s_L[hh] = L;
      s_M[hh] = M;
    }
  }
  __syncthreads();
  const float L = s_L[hl];
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float f = s_f[hl][sp];
    acc.x = fmaf(__uint_as_float(v[sp].x << 16), f, acc.x);
    acc.y = fmaf(__uint_as_float(v[sp].x & 0xFFFF0000u), f, acc.y);
    acc.z = fmaf(__uint_as_float(v[sp].y << 16), f, acc.z);
    acc.w = fmaf(__uint_as_float(v[sp].y & 0xFFFF0000u), f, acc.w);
  }
  const int d = 128 * w + 32 * mb + 8 * jq + 4 * (lane >> 5);
  bf16_t* out = static_cast<bf16_t*>(P.o) + (static_cast<size_t>(b) * NH + h) * DN + d;
  *reinterpret_cast<uint2*>(out) = make_uint2(pack2_bf16(acc.x * inv, acc.y * inv), pack2_bf16(acc.z * inv, acc.w * inv));
  if (P.lse && w == 0 && mb == 0 && tid < 32) P.lse[static_cast<size_t>(b) * NH + h] = L > 0.0f ? (s_M[hl] + log2f(L)) * LN2 : -INFINITY;
}

// bytes of the split partials of B sequences
size_t part_bytes(int B, int splits) {
  return static_cast<size_t>(B) * splits * NH * (DN * sizeof(bf16_t) + sizeof(float));
}

// Decode splits of one sequence: a function of its entry count alone (the
// list length k, or the capacity for dense), never of the batch size, so a
// sequence's partials, their merge and its output bits are the same in any
// batch.  A sparse split covers two 64-entry tiles (k = 1024: 8 splits); a
// dense split at least DENSE_TILES tiles, at most MAX_SPLITS splits.
constexpr int SPARSE_TILES = 2;
constexpr int DENSE_TILES = 4;
int decode_splits(bool dense, int64_t count) {
  const int64_t ntiles = (count + TILE - 1) / TILE;
  const int64_t per = dense ? DENSE_TILES : SPARSE_TILES;
  int64_t s = (ntiles + per - 1) / per;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  return s < 1 ? 1 : static_cast<int>(s);
}

// Entries a dense decode sequence can attend: the capacity, or the window.
int64_t dense_span(int64_t cap, int64_t window) { return window > 0 && window < cap ? window : cap; }

// Gather offsets of the MFMA kernel are 32-bit byte offsets within one
// sequence's rows, or within the pool of a paged cache (row id times row
// bytes): every cache buffer of a sequence (of the pool) must stay below
// 2^31 bytes.
bool offsets_fit(const AttnParams& P) {
  const int64_t nope_row = P.nope_dt == CSA_FP8E4M3 ? DN : DN * 2;
  const int64_t lim = int64_t(1) << 31;
  return P.span_rows <= lim / nope_row && P.span_rows <= lim / (DRP * 2);
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Paged sparse attention: each listed id turned into its pool row before the
// gather kernel runs, -1 for an id outside [0, n(p)) or on a page outside
// the pool, so that the kernel's tile loop keeps reading rows straight from
// its list.  One thread per list entry.
__global__ void __launch_bounds__(256) page_rows_kernel(AttnParams P, int32_t* rows, int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t bt = i / P.k;
  const int b = static_cast<int>(bt / P.T), t = static_cast<int>(bt % P.T);
  const int64_t pos = P.pos_dev ? P.pos_dev[b] : P.pos0 + t;
  int64_t n = pos < 0 ? 0 : (pos + 1) / P.m;
  if (n > P.cap) n = P.cap;
  const int64_t id = P.idx[i];
  rows[i] = static_cast<int32_t>(id >= 0 && id < n ? entry_row(P.pg, P.cap, b, id) : -1);
}

bool mfma_shape(int H, int d_nope, int d_rope, int q_dt, int o_dt, int nope_dt, int rope_dt) {
  return H == NH && d_nope == DN && d_rope == DRP && q_dt == CSA_BF16 && o_dt == CSA_BF16 &&
         (nope_dt == CSA_BF16 || nope_dt == CSA_FP8E4M3) && rope_dt == CSA_BF16;
}

}  // namespace

bool mfma_attn_supported(const AttnParams& P) {
  const bool shape = mfma_shape(P.H, P.d_nope, P.d_rope, P.q_dt, P.o_dt, P.nope_dt, P.rope_dt);
  // sparse prefill keeps one query's whole list in LDS
  const bool list_fits = P.idx == nullptr || P.pos_dev != nullptr || P.k <= MAX_LIST;
  return shape && list_fits;
}

bool mfma_attn_capacity_ok(const AttnParams& P) { return offsets_fit(P); }

size_t mfma_attn_ws_bytes(const csa_attn_desc* d, int op, int B, int, int64_t, int k) {
  if (op != CSA_OP_SPARSE_ATTN_DECODE && op != CSA_OP_DENSE_ATTN_DECODE) return 0;
  if (!mfma_shape(d->n_heads, d->d_nope, d->d_rope, d->q_dtype, d->o_dtype, d->nope_dtype, d->rope_dtype)) return 0;
  const bool dense = op == CSA_OP_DENSE_ATTN_DECODE;
  return round256(part_bytes(B, decode_splits(dense, dense ? dense_span(d->capacity, d->window) : k)));
}

size_t page_list_bytes(const csa_attn_desc* d, int op, int B, int T, int k) {
  if (d->page_size == 0 || (op != CSA_OP_SPARSE_ATTN_PREFILL && op != CSA_OP_SPARSE_ATTN_DECODE)) return 0;
  if (!mfma_shape(d->n_heads, d->d_nope, d->d_rope, d->q_dtype, d->o_dtype, d->nope_dtype, d->rope_dtype)) return 0;
  const int rows = op == CSA_OP_SPARSE_ATTN_DECODE ? 1 : T;
  return round256(static_cast<size_t>(B) * rows * k * sizeof(int32_t));
}

int32_t* page_list_slot(const AttnParams& P, int op, int B) {
  const bool dense = op == CSA_OP_DENSE_ATTN_PREFILL || op == CSA_OP_DENSE_ATTN_DECODE;
  if (dense || !P.pg.table || !mfma_attn_supported(P)) return nullptr;
  size_t part_room = 0;  // workspace bytes ahead of the list: the decode split partials
  if (op == CSA_OP_SPARSE_ATTN_DECODE) {
    const int splits = decode_splits(false, P.k);
    part_room = splits > 1 ? round256(part_bytes(B, splits)) : 0;
  }
  const size_t need = part_room + static_cast<size_t>(B) * P.T * P.k * sizeof(int32_t);
  if (!P.ws || P.ws_bytes < need) return nullptr;
  return reinterpret_cast<int32_t*>(static_cast<char*>(P.ws) + part_room);
}

int launch_mfma_attn(const AttnParams& P0, int op, int B, hipStream_t s) {
  const bool dense = op == CSA_OP_DENSE_ATTN_PREFILL || op == CSA_OP_DENSE_ATTN_DECODE;
  const bool decode = op == CSA_OP_SPARSE_ATTN_DECODE || op == CSA_OP_DENSE_ATTN_DECODE;
  AttnParams P = P0;
  if (!dense && P.pg.table && !P.list_rows) {
    // paged sparse: the list turned into pool rows in the workspace, after the partials
    const int64_t total = static_cast<int64_t>(B) * P.T * P.k;
    int32_t* rows = page_list_slot(P, op, B);
    if (!rows) return fail(CSA_ERR_WORKSPACE, "workspace too small for the paged list");
    hipLaunchKernelGGL(page_rows_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, P, rows,
                       total);
    int st = check_launch("page_rows_kernel");
    if (st != CSA_OK) return st;
    P.idx = rows;
    P.list_rows = true;
  }
  if (!decode) {
    const int64_t per = dense ? P.cap : P.k;
    launch_attn_bf16(P, dense, B, s, 1, per, nullptr);
    return check_launch("attn_bf16_kernel");
  }
  const int64_t count = dense ? dense_span(P.cap, P.window) : P.k;
  const int64_t ntiles = (count + TILE - 1) / TILE;
  const int splits = decode_splits(dense, count);
  const int64_t tiles_per = (ntiles + splits - 1) / splits;
  const int64_t per = tiles_per * TILE;
  if (splits == 1) {  // one item per sequence writes o and lse itself (the same bits a one-split merge gives)
    launch_attn_bf16(P, dense, B, s, 1, per, nullptr);
    return check_launch("attn_bf16_kernel");
  }
  const size_t need = part_bytes(B, splits);
  if (!P.ws || P.ws_bytes < need) return fail(CSA_ERR_WORKSPACE, "workspace too small for the split partials");
  void* part = P.ws;
  launch_attn_bf16(P, dense, B, s, splits, per, part);
  int st = check_launch("attn_bf16_kernel");
  if (st != CSA_OK) return st;
  const dim3 mg(32, B);  // blocks (w, mb, nb) of the partial layout
  if (splits <= 2) hipLaunchKernelGGL(attn_merge_kernel<2>, mg, dim3(256), 0, s, P, splits, part, B);
  else if (splits <= 4) hipLaunchKernelGGL(attn_merge_kernel<4>, mg, dim3(256), 0, s, P, splits, part, B);
  else if (splits <= 8) hipLaunchKernelGGL(attn_merge_kernel<8>, mg, dim3(256), 0, s, P, splits, part, B);
  else if (splits <= 16) hipLaunchKernelGGL(attn_merge_kernel<16>, mg, dim3(256), 0, s, P, splits, part, B);
  else hipLaunchKernelGGL(attn_merge_kernel<MAX_SPLITS>, mg, dim3(256), 0, s, P, splits, part, B);
  return check_launch("attn_merge_kernel");
}

}  // namespace csa
