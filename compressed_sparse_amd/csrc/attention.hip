// Attention over compressed entries: CSA sparse (listed entries) and HCA
// dense (every visible entry).  [CSA/HCA 混注意力] §1.1 (each query attends
// only its selected entries), §1.2 (dense attention over the 128x shorter
// sequence); [读完这篇] §三 CSA 步骤三 (standard attention, KV shared).
//
//   q~ = RoPE_pos(q[h]);  l_s = scale * q~ . K_s;  o[h] = softmax(l) V;
//   lse[h] = log sum exp(l)
//
// This file holds the generic path (any head count / width / format, VALU
// fp32, one workgroup per (query, head), online softmax over chunks of 256
// entries) and the host entry points, which route the MI355X-shaped cases
// (64 heads, 512 + 64 dims, BF16 / FP8 caches) to the MFMA kernels.
#include <mutex>

#include "attention.hpp"

namespace csa {

__device__ __forceinline__ int64_t attn_pos(const AttnParams& P, int b, int t) {
  return P.pos_dev ? P.pos_dev[b] : P.pos0 + t;
}

__device__ __forceinline__ float kv_nope(const AttnParams& P, size_t e, int d) {
  switch (P.nope_dt) {
    case CSA_F32: return static_cast<const float*>(P.nope)[e * P.d_nope + d];
    case CSA_BF16: return bf16_to_f32(static_cast<const bf16_t*>(P.nope)[e * P.d_nope + d]);
    default: return e4m3_to_f32(static_cast<const uint8_t*>(P.nope)[e * P.d_nope + d]) *
                    static_cast<const float*>(P.scale)[e];
  }
}

__device__ __forceinline__ float kv_rope(const AttnParams& P, size_t e, int d) {
  return P.rope_dt == CSA_F32 ? static_cast<const float*>(P.rope)[e * P.d_rope + d]
                              : bf16_to_f32(static_cast<const bf16_t*>(P.rope)[e * P.d_rope + d]);
}

// grid (H, T, B), 256 threads.
__global__ void __launch_bounds__(256) attn_generic_kernel(AttnParams P) {
  extern __shared__ int64_t smem64[];
  const int c = P.d_nope + P.d_rope;
  int64_t* ent = smem64;                               // 256 cache rows (-1: none)
  float* red = reinterpret_cast<float*>(ent + 256);    // 32
  float* q = red + 32;                                 // c
  float* p = q + c;                                    // 256 probabilities of the current chunk
  float* o = p + 256;                                  // d_nope accumulators
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t pos = attn_pos(P, b, t);
  int64_t n = pos < 0 ? 0 : (pos + 1) / P.m;
  if (n > P.cap) n = P.cap;
  const size_t qrow = (static_cast<size_t>(b) * P.T + t) * P.H + h;
  for (int j = tid; j < c; j += nt) q[j] = load_elem(P.q, qrow * c + j, P.q_dt);
  __syncthreads();
  for (int pp = tid; pp < P.d_rope / 2; pp += nt) {
    float s, co;
    rope_sincos(pos, pp, P.d_rope, P.base, &s, &co);
    float x0 = q[P.d_nope + 2 * pp], x1 = q[P.d_nope + 2 * pp + 1];
    q[P.d_nope + 2 * pp] = x0 * co - x1 * s;
    q[P.d_nope + 2 * pp + 1] = x0 * s + x1 * co;
  }
  for (int d = tid; d < P.d_nope; d += nt) o[d] = 0.0f;
  __syncthreads();
  // dense: the visible entries [lo, n), lo > 0 under a sliding window
  const int64_t lo = (!P.idx && P.window > 0 && n > P.window) ? n - P.window : 0;
  const int64_t count = P.idx ? P.k : n - lo;
  const int32_t* list = P.idx ? P.idx + (static_cast<size_t>(b) * P.T + t) * P.k : nullptr;
  float mx = -INFINITY, sum = 0.0f;
  for (int64_t base = 0; base < count; base += nt) {
    const int64_t j = base + tid;
    int64_t s = -1;
    if (j < count) s = list ? static_cast<int64_t>(list[j]) : lo + j;
    if (s >= n) s = -1;
    const int64_t er = s >= 0 ? entry_row(P.pg, P.cap, b, s) : -1;  // -1: page outside the pool
    float l = -INFINITY;
    if (er >= 0) {
      const size_t e = static_cast<size_t>(er);
      float dot = 0.0f;
      for (int d = 0; d < P.d_nope; ++d) dot = fmaf(q[d], kv_nope(P, e, d), dot);
      for (int d = 0; d < P.d_rope; ++d) dot = fmaf(q[P.d_nope + d], kv_rope(P, e, d), dot);
      l = dot * P.scale_qk;
    }
    const float cmax = block_max(l, red);
    const float nmx = fmaxf(mx, cmax);
    float pe = (er >= 0) ? expf(l - nmx) : 0.0f;
    const float csum = block_sum(pe, red);
    const float corr = (nmx == -INFINITY) ? 1.0f : expf(mx - nmx);
    p[tid] = pe;
    ent[tid] = er;
    __syncthreads();
    if (nmx != -INFINITY) {
      const int lim = static_cast<int>((count - base) < nt ? (count - base) : nt);
      for (int d = tid; d < P.d_nope; d += nt) {
        float acc = o[d] * corr;
        for (int i = 0; i < lim; ++i) {
          const int64_t e = ent[i];
          if (e >= 0) acc = fmaf(p[i], kv_nope(P, static_cast<size_t>(e), d), acc);
        }
        o[d] = acc;
      }
      sum = sum * corr + csum;
      mx = nmx;
    }
    __syncthreads();
  }
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  for (int d = tid; d < P.d_nope; d += nt) {
    float v = o[d] * inv;
    if (P.o_dt == CSA_F32) static_cast<float*>(P.o)[qrow * P.d_nope + d] = v;
    else static_cast<bf16_t*>(P.o)[qrow * P.d_nope + d] = f32_to_bf16(v);
  }
  if (P.lse && tid == 0) P.lse[qrow] = sum > 0.0f ? mx + logf(sum) : -INFINITY;
}

static int launch_generic(const AttnParams& P, int B, hipStream_t s) {
  const int c = P.d_nope + P.d_rope;
  const size_t lds = (32 + c + 256 + P.d_nope) * sizeof(float) + 256 * sizeof(int64_t);
  hipLaunchKernelGGL(attn_generic_kernel, dim3(P.H, P.T, B), dim3(256), lds, s, P);
  return check_launch("attn_generic_kernel");
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int validate_attn(const csa_attn_desc* d, int B, const void* q, const csa_cache* kv,
                         void* o, float* lse, float softmax_scale) {
  if (!d) return fail(CSA_ERR_INVALID_ARG, "attn desc is NULL");
  if (!(softmax_scale > 0.0f) || !(softmax_scale < INFINITY))
    return fail(CSA_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  if (d->n_heads < 1 || d->n_heads > 65535) return fail(CSA_ERR_INVALID_ARG, "n_heads must be in 1..65535");
  if (d->d_nope < 1 || d->d_rope < 0 || (d->d_rope & 1) || d->d_nope + d->d_rope > 4096)
    return fail(CSA_ERR_INVALID_ARG, "d_nope >= 1, d_rope even, width <= 4096");
  if (d->q_dtype != CSA_F32 && d->q_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "q_dtype must be F32 or BF16");
  if (d->o_dtype != CSA_F32 && d->o_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "o_dtype must be F32 or BF16");
  if (d->nope_dtype != CSA_F32 && d->nope_dtype != CSA_BF16 && d->nope_dtype != CSA_FP8E4M3)
    return fail(CSA_ERR_UNSUPPORTED, "nope_dtype must be F32, BF16 or FP8E4M3");
  if (d->d_rope > 0 && d->rope_dtype != CSA_F32 && d->rope_dtype != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "rope_dtype must be F32 or BF16");
  if (d->m < 1 || d->m > 256) return fail(CSA_ERR_INVALID_ARG, "m must be in 1..256");
  if (d->capacity < 1 || d->capacity > (int64_t(1) << 31) - 1) return fail(CSA_ERR_INVALID_ARG, "capacity must be in 1..2^31-1");
  if (d->window < 0) return fail(CSA_ERR_INVALID_ARG, "window must be >= 0");
  if (d->qk_mode != 0 && d->qk_mode != CSA_FP8E4M3) return fail(CSA_ERR_INVALID_ARG, "qk_mode must be 0 or FP8E4M3");
  if (d->qk_mode == CSA_FP8E4M3 &&
      (d->nope_dtype != CSA_FP8E4M3 || d->n_heads != 64 || d->d_nope != 512 || d->d_rope != 64 ||
       d->q_dtype != CSA_BF16 || d->o_dtype != CSA_BF16 || d->rope_dtype != CSA_BF16))
    return fail(CSA_ERR_UNSUPPORTED, "qk_mode FP8E4M3 needs 64 BF16 heads over 512 FP8 + 64 BF16 dims, BF16 output");
  if (d->reserved != 0) return fail(CSA_ERR_INVALID_ARG, "reserved field must be 0");
  if (!(d->rope_base > 0.0)) return fail(CSA_ERR_INVALID_ARG, "rope_base must be > 0");
  if (B < 0 || B > 65535) return fail(CSA_ERR_INVALID_ARG, "B must be in 0..65535");
  if (!q || !kv || !kv->nope || !o) return fail(CSA_ERR_INVALID_ARG, "NULL argument");
  if (d->nope_dtype == CSA_FP8E4M3 && !kv->scale) return fail(CSA_ERR_INVALID_ARG, "kv scale is NULL");
  if (d->d_rope > 0 && !kv->rope) return fail(CSA_ERR_INVALID_ARG, "kv rope is NULL");
  if (!aligned16(q) || !aligned16(kv->nope) || !aligned16(kv->scale) || !aligned16(kv->rope) ||
      !aligned16(o) || !aligned16(lse))
    return fail(CSA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  Pages pg;
  return make_pages(d->page_size, d->pool_pages, d->capacity, kv->block_table, &pg);
}

static AttnParams make_attn_params(const csa_attn_desc* d, const void* q, const csa_cache* kv,
                                   const int32_t* idx, int k, float scale, void* o, float* lse,
                                   void* ws, size_t ws_bytes) {
  AttnParams P{};
  P.H = d->n_heads; P.d_nope = d->d_nope; P.d_rope = d->d_rope;
  P.q_dt = d->q_dtype; P.o_dt = d->o_dtype; P.nope_dt = d->nope_dtype; P.rope_dt = d->rope_dtype;
  P.m = d->m; P.base = d->rope_base; P.cap = d->capacity; P.window = d->window; P.qk_mode = d->qk_mode;
  P.q = q; P.nope = kv->nope; P.scale = kv->scale; P.rope = kv->rope;
  P.idx = idx; P.k = k; P.scale_qk = scale; P.o = o; P.lse = lse;
  P.ws = ws; P.ws_bytes = ws_bytes;
  make_pages(d->page_size, d->pool_pages, d->capacity, kv->block_table, &P.pg);  // validated before
  P.span_rows = P.pg.table ? (P.pg.pool << P.pg.shift) : P.cap;
  P.seq_stride = P.pg.table ? 0 : P.cap;
  P.list_rows = false;
  return P;
}

size_t attn_ws_bytes(const csa_attn_desc* d, int op, int B, int T, int64_t pos0, int k) {
  if (!d || B < 0 || T < 0) return 0;
  if (check_paging(d->page_size, d->pool_pages, d->capacity) != CSA_OK) return 0;
  return mfma_attn_ws_bytes(d, op, B, T, pos0, k) + page_list_bytes(d, op, B, T, k);
}

int attn_dispatch(AttnParams& P, int op, int B, void* stream) {
  hipStream_t s = as_stream(stream);
  if (mfma_attn_supported(P)) {
    if (!mfma_attn_capacity_ok(P))
      return fail(CSA_ERR_UNSUPPORTED, "capacity too large: each cache buffer of a sequence (of the pool, when "
                                       "paged) must stay below 2^31 bytes (2^21 BF16 or 2^22 FP8 entries of 512 dims)");
    return launch_mfma_attn(P, op, B, s);
  }
  if (P.qk_mode != 0) return fail(CSA_ERR_UNSUPPORTED, "qk_mode FP8E4M3: sparse prefill lists of at most 1024");
  return launch_generic(P, B, s);
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of two attention results (sliding-window branch + the
// compressed branch): one softmax over the union of their keys
// ---------------------------------------------------------------------------
// grid (rows, H); each thread 4 consecutive value dims.
__global__ void __launch_bounds__(256) lse_merge_kernel(int H, int dv, int o_dt, const void* o1, const float* l1,
                                                        const void* o2, const float* l2, void* o, float* lse) {
  const size_t rh = static_cast<size_t>(blockIdx.x) * H + blockIdx.y;
  const float a = l1[rh], b = l2[rh];
  const float mx = fmaxf(a, b);
  float fa = 0.0f, fb = 0.0f, L = -INFINITY;
  if (mx != -INFINITY) {
    const float wa = expf(a - mx), wb = expf(b - mx);  // exp(-inf) = 0 for an empty side
    const float sw = wa + wb;
    fa = wa / sw;
    fb = wb / sw;
    L = mx + logf(sw);
  }
  for (int d = 4 * threadIdx.x; d < dv; d += 4 * blockDim.x) {
    const size_t e = rh * dv + d;
    float x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = load_elem(o1, e + u, o_dt);
      y[u] = load_elem(o2, e + u, o_dt);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float v = fa * x[u] + fb * y[u];
      if (o_dt == CSA_F32) static_cast<float*>(o)[e + u] = v;
      else static_cast<bf16_t*>(o)[e + u] = f32_to_bf16(v);
    }
  }
  if (lse && threadIdx.x == 0) lse[rh] = L;
}

// ---------------------------------------------------------------------------
// allocation-free decode: split partials in a library-owned device array
// ---------------------------------------------------------------------------
// One copy of this array lives on every GPU the library runs on, for the life
// of the process.  In host code its name is a host-side stand-in: kernels get
// the device address looked up once per device by hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with it current).
static int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CSA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(CSA_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CSA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace csa

using namespace csa;

extern "C" int csa_sparse_attn_prefill(const csa_attn_desc* desc, int B, int T, int64_t pos0,
                                       const void* q, const csa_cache* kv, const int32_t* idx, int k,
                                       float softmax_scale, void* o, float* lse, void* ws,
                                       size_t ws_bytes, void* stream) {
  int st = validate_attn(desc, B, q, kv, o, lse, softmax_scale);
  if (st != CSA_OK) return st;
  if (desc->window != 0) return fail(CSA_ERR_INVALID_ARG, "window must be 0 for sparse attention");
  if (T < 0 || T > 65535 || pos0 < 0) return fail(CSA_ERR_INVALID_ARG, "T must be in 0..65535, pos0 >= 0");
  if (!idx || !aligned16(idx)) return fail(idx ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "idx must be an aligned device pointer");
  if (k < 1 || k > 2048) return fail(CSA_ERR_INVALID_ARG, "k must be in 1..2048");
  if (ws_bytes < attn_ws_bytes(desc, CSA_OP_SPARSE_ATTN_PREFILL, B, T, pos0, k))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  if (B == 0 || T == 0) return CSA_OK;
  AttnParams P = make_attn_params(desc, q, kv, idx, k, softmax_scale, o, lse, ws, ws_bytes);
  P.T = T; P.pos0 = pos0; P.pos_dev = nullptr;
  return attn_dispatch(P, CSA_OP_SPARSE_ATTN_PREFILL, B, stream);
}

namespace csa {

int sparse_attn_decode_setup(const csa_attn_desc* desc, int B, const int64_t* pos, const void* q, const csa_cache* kv,
                             const int32_t* idx, int k, float softmax_scale, void* o, float* lse, void* ws,
                             size_t ws_bytes, AttnParams* out) {
  int st = validate_attn(desc, B, q, kv, o, lse, softmax_scale);
  if (st != CSA_OK) return st;
  if (desc->window != 0) return fail(CSA_ERR_INVALID_ARG, "window must be 0 for sparse attention");
  if (!pos || !aligned16(pos)) return fail(pos ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "pos must be an aligned device pointer");
  if (!idx || !aligned16(idx)) return fail(idx ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "idx must be an aligned device pointer");
  if (k < 1 || k > 2048) return fail(CSA_ERR_INVALID_ARG, "k must be in 1..2048");
  if (ws_bytes < attn_ws_bytes(desc, CSA_OP_SPARSE_ATTN_DECODE, B, 1, 0, k))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  AttnParams P = make_attn_params(desc, q, kv, idx, k, softmax_scale, o, lse, ws, ws_bytes);
  P.T = 1; P.pos0 = 0; P.pos_dev = pos;
  if (mfma_attn_supported(P) && !mfma_attn_capacity_ok(P))
    return fail(CSA_ERR_UNSUPPORTED, "capacity too large: each cache buffer of a sequence (of the pool, when "
                                     "paged) must stay below 2^31 bytes (2^21 BF16 or 2^22 FP8 entries of 512 dims)");
  *out = P;
  return CSA_OK;
}

}  // namespace csa

extern "C" int csa_sparse_attn_decode(const csa_attn_desc* desc, int B, const int64_t* pos,
                                      const void* q, const csa_cache* kv, const int32_t* idx, int k,
                                      float softmax_scale, void* o, float* lse, void* ws,
                                      size_t ws_bytes, void* stream) {
  AttnParams P;
  int st = sparse_attn_decode_setup(desc, B, pos, q, kv, idx, k, softmax_scale, o, lse, ws, ws_bytes, &P);
  if (st != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  return attn_dispatch(P, CSA_OP_SPARSE_ATTN_DECODE, B, stream);
}

// The allocation-free variant of csa_sparse_attn_decode: the split partials
// go to the library's device array instead of a caller workspace.
extern "C" int csa_sparse_attn_decode_noalloc(const csa_attn_desc* desc, int B, const int64_t* pos,
                                              const void* q, const csa_cache* kv, const int32_t* idx, int k,
                                              float softmax_scale, void* o, float* lse, void* stream) {
  int st = validate_attn(desc, B, q, kv, o, lse, softmax_scale);
  if (st != CSA_OK) return st;
  if (desc->window != 0) return fail(CSA_ERR_INVALID_ARG, "window must be 0 for sparse attention");
  if (!pos || !aligned16(pos)) return fail(pos ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "pos must be an aligned device pointer");
  if (!idx || !aligned16(idx)) return fail(idx ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "idx must be an aligned device pointer");
  if (k < 1 || k > 2048) return fail(CSA_ERR_INVALID_ARG, "k must be in 1..2048");
  const size_t need = attn_ws_bytes(desc, CSA_OP_SPARSE_ATTN_DECODE, B, 1, 0, k);
  if (need > CSA_NOALLOC_SCRATCH_BYTES)
    return fail(CSA_ERR_WORKSPACE, "split partials need " + std::to_string(need) + " bytes, above the " +
                                       std::to_string(static_cast<size_t>(CSA_NOALLOC_SCRATCH_BYTES)) +
                                       "-byte library scratch: use csa_sparse_attn_decode with a workspace");
  if (B == 0) return CSA_OK;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != CSA_OK) return st;
  AttnParams P = make_attn_params(desc, q, kv, idx, k, softmax_scale, o, lse, ws, CSA_NOALLOC_SCRATCH_BYTES);
  P.T = 1; P.pos0 = 0; P.pos_dev = pos;
  return attn_dispatch(P, CSA_OP_SPARSE_ATTN_DECODE, B, stream);
}

extern "C" int csa_lse_merge(int rows, int H, int d_v, int o_dtype, const void* o1, const float* lse1,
                             const void* o2, const float* lse2, void* o, float* lse, void* stream) {
  if (rows < 0 || rows > 0x7FFFFFFF / 2) return fail(CSA_ERR_INVALID_ARG, "rows out of range");
  if (H < 1 || H > 65535) return fail(CSA_ERR_INVALID_ARG, "H must be in 1..65535");
  if (d_v < 4 || d_v > 4096 || d_v % 4) return fail(CSA_ERR_INVALID_ARG, "d_v must be a multiple of 4 in 4..4096");
  if (o_dtype != CSA_F32 && o_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "o_dtype must be F32 or BF16");
  if (!o1 || !lse1 || !o2 || !lse2 || !o) return fail(CSA_ERR_INVALID_ARG, "NULL argument");
  if (!aligned16(o1) || !aligned16(o2) || !aligned16(o) || !aligned16(lse1) || !aligned16(lse2) || !aligned16(lse))
    return fail(CSA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (rows == 0) return CSA_OK;
  const int threads = d_v / 4 >= 256 ? 256 : ((d_v / 4 + 63) / 64) * 64;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(rows, H), dim3(threads), 0, as_stream(stream), H, d_v, o_dtype, o1, lse1,
                     o2, lse2, o, lse);
  return check_launch("lse_merge_kernel");
}

extern "C" int hca_dense_attn_prefill(const csa_attn_desc* desc, int B, int T, int64_t pos0,
                                      const void* q, const csa_cache* kv, float softmax_scale, void* o,
                                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = validate_attn(desc, B, q, kv, o, lse, softmax_scale);
  if (st != CSA_OK) return st;
  if (T < 0 || T > 65535 || pos0 < 0) return fail(CSA_ERR_INVALID_ARG, "T must be in 0..65535, pos0 >= 0");
  if (ws_bytes < attn_ws_bytes(desc, CSA_OP_DENSE_ATTN_PREFILL, B, T, pos0, 0))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  if (B == 0 || T == 0) return CSA_OK;
  AttnParams P = make_attn_params(desc, q, kv, nullptr, 0, softmax_scale, o, lse, ws, ws_bytes);
  P.T = T; P.pos0 = pos0; P.pos_dev = nullptr;
  return attn_dispatch(P, CSA_OP_DENSE_ATTN_PREFILL, B, stream);
}

extern "C" int hca_dense_attn_decode(const csa_attn_desc* desc, int B, const int64_t* pos,
                                     const void* q, const csa_cache* kv, float softmax_scale, void* o,
                                     float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = validate_attn(desc, B, q, kv, o, lse, softmax_scale);
  if (st != CSA_OK) return st;
  if (!pos || !aligned16(pos)) return fail(pos ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "pos must be an aligned device pointer");
  if (ws_bytes < attn_ws_bytes(desc, CSA_OP_DENSE_ATTN_DECODE, B, 1, 0, 0))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  if (B == 0) return CSA_OK;
  AttnParams P = make_attn_params(desc, q, kv, nullptr, 0, softmax_scale, o, lse, ws, ws_bytes);
  P.T = 1; P.pos0 = 0; P.pos_dev = pos;
  return attn_dispatch(P, CSA_OP_DENSE_ATTN_DECODE, B, stream);
}
