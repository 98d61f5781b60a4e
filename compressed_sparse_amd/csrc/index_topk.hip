// Lightning indexer + top-k.  [CSA/HCA 混注意力] §1.1 关键参数 (top-k = 1024),
// §1.4 LIGHTNING INDEXER 的 FP4 计 (QK in FP4, scores FP32 -> BF16);
// [读完这篇] §三 CSA 步骤二 (V3.2 DSA indexer: every query against every
// summary, heads weighted, then top-k).
//
//   I[s] = sum_h w[h] * ReLU(qI[h] . K[s])   for s < n(pos)
//
// Scores land in a workspace row per query; a radix select then finds the
// k-th largest order-preserving key and an ordered compaction writes the
// selected indices in ascending order (ties at the threshold go to the
// lower index).
#include "index.hpp"

namespace csa {



__device__ __forceinline__ int64_t query_pos(const IndexParams& P, int b, int t) {
  return P.pos_dev ? P.pos_dev[b] : P.pos0 + t;
}

__device__ __forceinline__ int64_t visible(int64_t pos, int m, int64_t cap) {
  if (pos < 0) return 0;
  int64_t n = (pos + 1) / m;
  return n < cap ? n : cap;
}

// Key element d of entry s (scale of FP8 entries applied by the caller).
__device__ __forceinline__ float key_elem(const IndexParams& P, size_t e, int d) {
  switch (P.key_dt) {
    case CSA_F32: return static_cast<const float*>(P.knope)[e * P.D + d];
    case CSA_BF16: return bf16_to_f32(static_cast<const bf16_t*>(P.knope)[e * P.D + d]);
    case CSA_FP8E4M3: return e4m3_to_f32(static_cast<const uint8_t*>(P.knope)[e * P.D + d]);
    default: {  // MXFP4
      uint32_t byte = static_cast<const uint8_t*>(P.knope)[e * (P.D / 2) + d / 2];
      uint32_t code = (d & 1) ? (byte >> 4) : (byte & 15u);
      int ex = static_cast<int>(static_cast<const uint8_t*>(P.kscale)[e * (P.D / 32) + d / 32]) - 127;
      return e2m1_to_f32(code) * exp2i(ex);
    }
  }
}

// Loads the query's indexer heads into LDS in the QK format.
__device__ void load_index_query(const IndexParams& P, int b, int t, float* q, float* w) {
  const size_t base = (static_cast<size_t>(b) * P.T + t) * P.H;
  const int tid = threadIdx.x;
  for (int x = tid; x < P.H * P.D; x += blockDim.x) {
    float v = load_elem(P.qI, base * P.D + x, P.q_dt);
    if (P.qk_dt == CSA_BF16) v = round_bf16(v);
    q[x] = v;
  }
  for (int h = tid; h < P.H; h += blockDim.x) w[h] = P.w[base + h];
  __syncthreads();
  if (P.qk_dt == CSA_MXFP4) {
    const int nb = P.D / 32;
    for (int hb = tid; hb < P.H * nb; hb += blockDim.x) {
      float* x = q + (hb / nb) * P.D + (hb % nb) * 32;
      float am = 0.0f;
      for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(x[i]));
      int ex = mx_exponent(am);
      float inv = exp2i(-ex), X = exp2i(ex);
      for (int i = 0; i < 32; ++i) x[i] = e2m1_to_f32(f32_to_e2m1(x[i] * inv)) * X;
    }
    __syncthreads();
  }
}

// Generic scoring: one thread per (query, entry), VALU fp32.
__global__ void __launch_bounds__(256) index_scores_generic(IndexParams P) {
  extern __shared__ float smem[];
  float* w = smem;           // H
  float* q = smem + P.H;     // H * D
  const int b = blockIdx.z, t = blockIdx.y;
  const int64_t pos = query_pos(P, b, t);
  const int64_t n = visible(pos, P.m, P.cap);
  if (static_cast<int64_t>(blockIdx.x) * blockDim.x >= n) return;
  load_index_query(P, b, t, q, w);
  const int64_t s = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (s >= n) return;
  const size_t e = static_cast<size_t>(b) * P.cap + s;
  const float ksc = P.key_dt == CSA_FP8E4M3 ? static_cast<const float*>(P.kscale)[e] : 1.0f;
  float acc = 0.0f;
  for (int h = 0; h < P.H; ++h) {
    float dot = 0.0f;
    const float* qh = q + h * P.D;
    for (int d = 0; d < P.D; ++d) dot = fmaf(qh[d], key_elem(P, e, d), dot);
    dot *= ksc;
    acc = fmaf(w[h], fmaxf(dot, 0.0f), acc);
  }
  if (P.score_dt == CSA_BF16) acc = round_bf16(acc);
  const size_t row = static_cast<size_t>(b) * P.T + t;
  P.ws[row * P.n_stride + s] = acc;
  if (P.scores_out) P.scores_out[row * P.cap + s] = acc;
}

// Order-preserving key of a score: larger score -> larger key; -0 == +0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix count of `flag` over the workgroup, in thread order.
// cnt: __shared__ int[17].  Returns the prefix; *total gets the sum.
__device__ __forceinline__ int block_prefix(bool flag, int* cnt, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  unsigned long long bal = __ballot(flag);
  int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) cnt[wv] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    int c = cnt[i];
    if (i < wv) before += c;
    tot += c;
  }
  *total = tot;
  return before + in_wave;
}

// One workgroup (1024 threads) selects the top-k of one query row.
__global__ void __launch_bounds__(1024) topk_radix_kernel(IndexParams P, int key_bits) {
  __shared__ int hist[256];
  __shared__ int cnt[17];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int b = blockIdx.y, t = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t n = visible(query_pos(P, b, t), P.m, P.cap);
  const size_t row = static_cast<size_t>(b) * P.T + t;
  const float* sc = P.ws + row * P.n_stride;
  int32_t* out = P.idx + row * P.k;
  if (n <= P.k) {
    for (int64_t j = tid; j < P.k; j += nt) out[j] = j < n ? static_cast<int32_t>(j) : -1;
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  int remaining = P.k;
  for (int shift = 24; shift >= 32 - key_bits; shift -= 8) {
    for (int i = tid; i < 256; i += nt) hist[i] = 0;
    __syncthreads();
    for (int64_t s = tid; s < n; s += nt) {
      uint32_t key = score_key(sc[s]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, bin = 255;
      for (; bin > 0; --bin) {
        if (cum + hist[bin] >= remaining) break;
        cum += hist[bin];
      }
      s_prefix = prefix | (static_cast<uint32_t>(bin) << shift);
      s_remaining = remaining - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    pmask |= 255u << shift;
  }
  // keys above the threshold prefix are taken; among keys equal to it (on the
  // examined bits) the `remaining` lowest indices are taken.
  int taken_eq = 0, written = 0;
  for (int64_t base = 0; base < n; base += nt) {
    const int64_t s = base + tid;
    uint32_t key = s < n ? (score_key(sc[s]) & pmask) : 0u;
    bool gt = s < n && key > prefix;
    bool eq = s < n && key == prefix;
    int eq_tot, take_tot;
    int eq_rank = block_prefix(eq, cnt, &eq_tot);
    bool take = gt || (eq && taken_eq + eq_rank < remaining);
    int pos = block_prefix(take, cnt, &take_tot);
    if (take) out[written + pos] = static_cast<int32_t>(s);
    taken_eq += eq_tot;
    written += take_tot;
  }
  for (int j = written + tid; j < P.k; j += nt) out[j] = -1;
}

static int launch_index(IndexParams& P, int B, int64_t n_max, void* stream) {
  hipStream_t s = as_stream(stream);
  if (index_mfma_supported(P)) {
    // scores stay on chip when every row fits the fused kernel's LDS rows
    if (!P.scores_out && index_fused_prefill_ok(P, n_max)) return launch_index_fused_prefill(P, B, s);
    if (n_max > 0) {
      int st = launch_index_scan(P, B, n_max, s);
      if (st != CSA_OK) return st;
    }
    const int bits = P.score_dt == CSA_BF16 ? 16 : 32;
    hipLaunchKernelGGL(topk_radix_kernel, dim3(P.T, B), dim3(1024), 0, s, P, bits);
    return check_launch("topk_radix_kernel");
  }
  const size_t lds = static_cast<size_t>(P.H) * (P.D + 1) * sizeof(float);
  if (n_max > 0) {
    dim3 grid(static_cast<unsigned>((n_max + 255) / 256), P.T, B);
    hipLaunchKernelGGL(index_scores_generic, grid, dim3(256), lds, s, P);
    int st = check_launch("index_scores_generic");
    if (st != CSA_OK) return st;
  }
  const int bits = P.score_dt == CSA_BF16 ? 16 : 32;
  hipLaunchKernelGGL(topk_radix_kernel, dim3(P.T, B), dim3(1024), 0, s, P, bits);
  return check_launch("topk_radix_kernel");
}

static int validate_index_desc(const csa_index_desc* d) {
  if (!d) return fail(CSA_ERR_INVALID_ARG, "index desc is NULL");
  if (d->n_heads < 1 || d->dim < 1 || d->n_heads * d->dim > 8192)
    return fail(CSA_ERR_INVALID_ARG, "n_heads, dim >= 1 and n_heads*dim <= 8192");
  if (d->q_dtype != CSA_F32 && d->q_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "q_dtype must be F32 or BF16");
  if (d->qk_dtype != CSA_F32 && d->qk_dtype != CSA_BF16 && d->qk_dtype != CSA_MXFP4)
    return fail(CSA_ERR_UNSUPPORTED, "qk_dtype must be F32, BF16 or MXFP4");
  if (d->key_dtype < CSA_F32 || d->key_dtype > CSA_MXFP4) return fail(CSA_ERR_UNSUPPORTED, "bad key_dtype");
  if ((d->key_dtype == CSA_MXFP4 || d->qk_dtype == CSA_MXFP4) && d->dim % 32 != 0)
    return fail(CSA_ERR_UNSUPPORTED, "MXFP4 needs dim % 32 == 0");
  if (d->score_dtype != CSA_F32 && d->score_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "score_dtype must be F32 or BF16");
  if (d->m < 1 || d->m > 256) return fail(CSA_ERR_INVALID_ARG, "m must be in 1..256");
  if (d->capacity < 1 || d->capacity > (int64_t(1) << 31) - 1) return fail(CSA_ERR_INVALID_ARG, "capacity must be in 1..2^31-1");
  if (d->reserved != 0) return fail(CSA_ERR_INVALID_ARG, "reserved field must be 0");
  return CSA_OK;
}

static int64_t stride_for(int64_t n) { return ((n + 63) / 64) * 64; }

static int64_t prefill_nmax(const csa_index_desc* d, int T, int64_t pos0) {
  int64_t n = (pos0 + T) / d->m;  // visible to the last query (pos0 + T - 1)
  return n < d->capacity ? n : d->capacity;
}

size_t index_ws_bytes(const csa_index_desc* d, int op, int B, int T, int64_t pos0) {
  if (!d || B < 0 || T < 0) return 0;
  int64_t nmax = op == CSA_OP_INDEX_TOPK_DECODE ? d->capacity : prefill_nmax(d, T, pos0);
  int64_t rows = static_cast<int64_t>(B) * (op == CSA_OP_INDEX_TOPK_DECODE ? 1 : T);
  return static_cast<size_t>(rows * stride_for(nmax) * sizeof(float)) + 256;
}

static int common_index_checks(const csa_index_desc* d, int B, const void* qI, const float* w,
                               const csa_cache* keys, int k, int32_t* idx, float* scores, void* ws) {
  int st;
  if ((st = validate_index_desc(d)) != CSA_OK) return st;
  if (B < 0 || B > 65535) return fail(CSA_ERR_INVALID_ARG, "B must be in 0..65535");
  if (k < 1 || k > 2048) return fail(CSA_ERR_INVALID_ARG, "k must be in 1..2048");
  if (!qI || !w || !keys || !keys->nope || !idx || !ws) return fail(CSA_ERR_INVALID_ARG, "NULL argument");
  if ((d->key_dtype == CSA_FP8E4M3 || d->key_dtype == CSA_MXFP4) && !keys->scale)
    return fail(CSA_ERR_INVALID_ARG, "key scale is NULL");
  if (!aligned16(qI) || !aligned16(w) || !aligned16(keys->nope) || !aligned16(keys->scale) ||
      !aligned16(idx) || !aligned16(scores) || !aligned16(ws))
    return fail(CSA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  return CSA_OK;
}

static IndexParams make_index_params(const csa_index_desc* d, const void* qI, const float* w,
                                     const csa_cache* keys, int k, int32_t* idx, float* scores, void* ws) {
  IndexParams P{};
  P.H = d->n_heads; P.D = d->dim; P.q_dt = d->q_dtype; P.qk_dt = d->qk_dtype;
  P.key_dt = d->key_dtype; P.score_dt = d->score_dtype; P.m = d->m; P.cap = d->capacity;
  P.qI = qI; P.w = w; P.knope = keys->nope; P.kscale = keys->scale;
  P.k = k; P.idx = idx; P.scores_out = scores;
  P.ws = static_cast<float*>(ws);
  return P;
}

}  // namespace csa

using namespace csa;

extern "C" int csa_index_topk_prefill(const csa_index_desc* desc, int B, int T, int64_t pos0,
                                      const void* qI, const float* w, const csa_cache* keys, int k,
                                      int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                                      void* stream) {
  int st = common_index_checks(desc, B, qI, w, keys, k, idx, scores, ws);
  if (st != CSA_OK) return st;
  if (T < 0 || T > 65535 * 16 || pos0 < 0) return fail(CSA_ERR_INVALID_ARG, "T must be in 0..1048560, pos0 >= 0");
  if (T > 65535) return fail(CSA_ERR_UNSUPPORTED, "T > 65535 per call: split the prefill");
  if (ws_bytes < index_ws_bytes(desc, CSA_OP_INDEX_TOPK_PREFILL, B, T, pos0))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  if (B == 0 || T == 0) return CSA_OK;
  IndexParams P = make_index_params(desc, qI, w, keys, k, idx, scores, ws);
  P.T = T;
  P.pos0 = pos0;
  P.pos_dev = nullptr;
  const int64_t nmax = prefill_nmax(desc, T, pos0);
  P.n_stride = stride_for(nmax);
  return launch_index(P, B, nmax, stream);
}

extern "C" int csa_index_topk_decode(const csa_index_desc* desc, int B, const int64_t* pos,
                                     const void* qI, const float* w, const csa_cache* keys, int k,
                                     int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                                     void* stream) {
  int st = common_index_checks(desc, B, qI, w, keys, k, idx, scores, ws);
  if (st != CSA_OK) return st;
  if (!pos || !aligned16(pos)) return fail(pos ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "pos must be an aligned device pointer");
  if (ws_bytes < index_ws_bytes(desc, CSA_OP_INDEX_TOPK_DECODE, B, 1, 0))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  if (B == 0) return CSA_OK;
  IndexParams P = make_index_params(desc, qI, w, keys, k, idx, scores, ws);
  P.T = 1;
  P.pos0 = 0;
  P.pos_dev = pos;
  P.n_stride = stride_for(desc->capacity);
  return launch_index(P, B, desc->capacity, stream);
}
