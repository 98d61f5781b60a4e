// Compressor: every m tokens -> one KV entry, then RoPE and the storage
// format.  [CSA/HCA 混注意力] §1.1 工程细节 (overlapped C^a + C^b, 2m tokens
// per entry), §1.2 (HCA, single window of m' = 128), §1.4 存储格式混 (RoPE
// dims BF16, rest FP8); [读完这篇] §三 压缩机制 (per-dimension weights, 4 W +
// 2 B).
//
// One workgroup builds one entry: each thread owns channels j, j+256, ...,
// runs an online softmax over the 2m (or m) logits of its channel and keeps
// the weighted value; the entry then sits in LDS for the RoPE turn and the
// FP8 / MXFP4 scale reductions.  HBM traffic is the 2m rows in and one entry
// out; the kernel is bandwidth-bound and tiny next to attention.
#include "common.hpp"

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
};

enum { RING_A = 0, RING_ZA = 1, RING_B = 2, RING_ZB = 3 };

__device__ __forceinline__ float* ring_row(const CompressParams& P, int b, int64_t t, int which) {
  int64_t slot = t % P.R;
  return P.ring + ((static_cast<size_t>(b) * P.R + slot) * P.NT + which) * P.c;
}

// Weighted value of channel j of entry i, rows fetched by `get(which, t)`:
// an online softmax over the window's rows (C^a rows of window i, then the
// C^b rows of window i-1).  The rows' loads are issued eight at a time
// (clamped to the last row, so branch-free) before their softmax steps.
template <class Get>
__device__ __forceinline__ float compress_channel(const CompressParams& P, int64_t i, int j, Get get) {
  float mx = -INFINITY, sum = 0.0f, acc = 0.0f;
  auto take = [&](float logit, float v) {
    if (logit > mx) {
      float sc = expf(mx - logit);  // 0 on the first row
      sum = sum * sc + 1.0f;
      acc = acc * sc + v;
      mx = logit;
    } else {
      float e = expf(logit - mx);
      sum += e;
      acc += e * v;
    }
  };
  constexpr int U = 8;
  auto side = [&](int zw, int vw, const float* Bw, int64_t t0) {
    for (int r0 = 0; r0 < P.m; r0 += U) {
      float z[U], v[U], bw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u < P.m ? r0 + u : P.m - 1;
        z[u] = get(zw, t0 + r, j);
        v[u] = get(vw, t0 + r, j);
        bw[u] = Bw[r * P.c + j];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (r0 + u < P.m) take(z[u] + bw[u], v[u]);
    }
  };
  side(RING_ZA, RING_A, P.Ba, i * P.m);
  if (P.overlap && i >= 1) side(RING_ZB, RING_B, P.Bb, (i - 1) * P.m);
  return acc / sum;
}

// RoPE + storage of the entry held in buf[0..c).  All threads call it.
__device__ void finalize_entry(const CompressParams& P, float* buf, float* red, int b, int64_t i) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t pos = i * P.m + P.m - 1;
  for (int p = tid; p < P.d_rope / 2; p += nt) {
    float s, co;
    rope_sincos(pos, p, P.d_rope, P.base, &s, &co);
    double x0 = buf[P.d_nope + 2 * p], x1 = buf[P.d_nope + 2 * p + 1];
    buf[P.d_nope + 2 * p] = static_cast<float>(x0 * co - x1 * s);
    buf[P.d_nope + 2 * p + 1] = static_cast<float>(x0 * s + x1 * co);
  }
  __syncthreads();
  const size_t e = static_cast<size_t>(b) * P.cap + i;
  switch (P.nope_dt) {
    case CSA_F32: {
      float* dst = static_cast<float*>(P.nope) + e * P.d_nope;
      for (int j = tid; j < P.d_nope; j += nt) dst[j] = buf[j];
      break;
    }
    case CSA_BF16: {
      bf16_t* dst = static_cast<bf16_t*>(P.nope) + e * P.d_nope;
      for (int j = tid; j < P.d_nope; j += nt) dst[j] = f32_to_bf16(buf[j]);
      break;
    }
    case CSA_FP8E4M3: {
      float am = 0.0f;
      for (int j = tid; j < P.d_nope; j += nt) am = fmaxf(am, fabsf(buf[j]));
      am = block_max(am, red);
      float s = am > 0.0f ? am / 448.0f : 1.0f;
      uint8_t* dst = static_cast<uint8_t*>(P.nope) + e * P.d_nope;
      for (int j = tid; j < P.d_nope; j += nt) dst[j] = static_cast<uint8_t>(f32_to_e4m3(buf[j] / s));
      if (tid == 0) static_cast<float*>(P.scale)[e] = s;
      break;
    }
    case CSA_MXFP4: {
      const int nb = P.d_nope / 32;
      uint8_t* dst = static_cast<uint8_t*>(P.nope) + e * (P.d_nope / 2);
      uint8_t* sdst = static_cast<uint8_t*>(P.scale) + e * nb;
      for (int blk = tid; blk < nb; blk += nt) {
        const float* x = buf + blk * 32;
        float am = 0.0f;
        for (int q = 0; q < 32; ++q) am = fmaxf(am, fabsf(x[q]));
        int ex = mx_exponent(am);
        float inv = exp2i(-ex);  // exact power of two
        for (int q = 0; q < 32; q += 2) {
          uint32_t lo = f32_to_e2m1(x[q] * inv), hi = f32_to_e2m1(x[q + 1] * inv);
          dst[blk * 16 + q / 2] = static_cast<uint8_t>(lo | (hi << 4));
        }
        sdst[blk] = static_cast<uint8_t>(ex + 127);
      }
      break;
    }
  }
  if (P.d_rope > 0) {
    if (P.rope_dt == CSA_F32) {
      float* dst = static_cast<float*>(P.rope) + e * P.d_rope;
      for (int j = tid; j < P.d_rope; j += nt) dst[j] = buf[P.d_nope + j];
    } else {
      bf16_t* dst = static_cast<bf16_t*>(P.rope) + e * P.d_rope;
      for (int j = tid; j < P.d_rope; j += nt) dst[j] = f32_to_bf16(buf[P.d_nope + j]);
    }
  }
}

__global__ void __launch_bounds__(256) compress_prefill_kernel(CompressParams P, int64_t i_first) {
  extern __shared__ float smem[];
  float* red = smem;       // 32
  float* buf = smem + 32;  // c
  const int b = blockIdx.y;
  const int64_t i = i_first + blockIdx.x;
  auto get = [&](int which, int64_t t, int j) -> float {
    if (t >= P.pos0) {
      const void* src = which == RING_A ? P.a : which == RING_ZA ? P.za : which == RING_B ? P.b : P.zb;
      return load_elem(src, (static_cast<size_t>(b) * P.T + (t - P.pos0)) * P.c + j, P.in_dt);
    }
    return ring_row(P, b, t, which)[j];
  };
  for (int j = threadIdx.x; j < P.c; j += blockDim.x) buf[j] = compress_channel(P, i, j, get);
  __syncthreads();
  finalize_entry(P, buf, red, b, i);
}

// Copies token rows [t_first, pos0 + T) into the ring (after the entries of
// the same call have read the older rows).
__global__ void __launch_bounds__(256) ring_store_kernel(CompressParams P, int64_t t_first) {
  const int b = blockIdx.y;
  const int64_t t = t_first + blockIdx.x;
  const size_t row = (static_cast<size_t>(b) * P.T + (t - P.pos0)) * P.c;
  for (int which = 0; which < P.NT; ++which) {
    const void* src = which == RING_A ? P.a : which == RING_ZA ? P.za : which == RING_B ? P.b : P.zb;
    float* dst = ring_row(P, b, t, which);
    for (int j = threadIdx.x; j < P.c; j += blockDim.x) dst[j] = load_elem(src, row + j, P.in_dt);
  }
}

template <bool IN_BF16>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
  if constexpr (IN_BF16) return bf16_to_f32(static_cast<const bf16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// Decode: one workgroup per sequence, one thread per channel (looping when
// the entry is wider than the workgroup).  The thread loads its channel of
// the new token's rows, stores them into the ring and, when the token
// completes a window, runs the channel's softmax over the window with the
// new row taken from its registers; nothing waits for the ring stores.
template <bool IN_BF16>
__global__ void __launch_bounds__(1024) compress_decode_kernel(CompressParams P, const int64_t* pos_dev) {
  extern __shared__ float smem[];
  float* red = smem;        // 32
  float* buf = smem + 32;   // c: the emitted entry
  const int b = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int64_t pos = pos_dev[b];
  if (pos < 0) return;
  const int64_t i = (pos + 1) / P.m - 1;
  const bool emit = (pos + 1) % P.m == 0 && i < P.cap;
  const size_t row = static_cast<size_t>(b) * P.c;
  for (int j = tid; j < P.c; j += nt) {
    float cur[4];
    cur[RING_A] = load_in<IN_BF16>(P.a, row + j);
    cur[RING_ZA] = load_in<IN_BF16>(P.za, row + j);
    cur[RING_B] = cur[RING_ZB] = 0.0f;
    if (P.NT == 4) {
      cur[RING_B] = load_in<IN_BF16>(P.b, row + j);
      cur[RING_ZB] = load_in<IN_BF16>(P.zb, row + j);
    }
#pragma unroll
    for (int wch = 0; wch < 4; ++wch)
      if (wch < P.NT) ring_row(P, b, pos, wch)[j] = cur[wch];
    if (emit) {
      auto get = [&](int which, int64_t t, int jj) -> float {
        const float v = ring_row(P, b, t, which)[jj];
        return t == pos ? cur[which] : v;
      };
      buf[j] = compress_channel(P, i, j, get);
    }
  }
  if (!emit) return;
  __syncthreads();
  finalize_entry(P, buf, red, b, i);
}

// ---------------------------------------------------------------------------
// host entry points
// ---------------------------------------------------------------------------
static int validate_cache_desc(const csa_cache_desc* d) {
  if (!d) return fail(CSA_ERR_INVALID_ARG, "cache desc is NULL");
  if (d->m < 1 || d->m > 256) return fail(CSA_ERR_INVALID_ARG, "m must be in 1..256");
  if (d->overlap != 0 && d->overlap != 1) return fail(CSA_ERR_INVALID_ARG, "overlap must be 0 or 1");
  if (d->d_nope < 0 || d->d_rope < 0 || (d->d_rope & 1)) return fail(CSA_ERR_INVALID_ARG, "d_nope >= 0, d_rope >= 0 and even");
  if (d->d_nope + d->d_rope < 1 || d->d_nope + d->d_rope > 4096) return fail(CSA_ERR_INVALID_ARG, "entry width must be 1..4096");
  if (d->in_dtype != CSA_F32 && d->in_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "in_dtype must be F32 or BF16");
  if (d->nope_dtype < CSA_F32 || d->nope_dtype > CSA_MXFP4) return fail(CSA_ERR_UNSUPPORTED, "bad nope_dtype");
  if (d->nope_dtype == CSA_MXFP4 && (d->d_nope % 32 != 0 || d->d_rope != 0))
    return fail(CSA_ERR_UNSUPPORTED, "MXFP4 entries need d_nope % 32 == 0 and no RoPE dims");
  if (d->nope_dtype == CSA_FP8E4M3 && d->d_nope < 1) return fail(CSA_ERR_INVALID_ARG, "FP8 entries need d_nope >= 1");
  if (d->d_rope > 0 && d->rope_dtype != CSA_F32 && d->rope_dtype != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "rope_dtype must be F32 or BF16");
  if (d->reserved != 0) return fail(CSA_ERR_INVALID_ARG, "reserved field must be 0");
  if (d->capacity < 1) return fail(CSA_ERR_INVALID_ARG, "capacity must be >= 1");
  if (!(d->rope_base > 0.0)) return fail(CSA_ERR_INVALID_ARG, "rope_base must be > 0");
  return CSA_OK;
}

static int validate_cache(const csa_cache_desc* d, const csa_cache* c) {
  if (!c) return fail(CSA_ERR_INVALID_ARG, "cache is NULL");
  if (!c->nope || !c->ring) return fail(CSA_ERR_INVALID_ARG, "cache nope/ring is NULL");
  if ((d->nope_dtype == CSA_FP8E4M3 || d->nope_dtype == CSA_MXFP4) && !c->scale)
    return fail(CSA_ERR_INVALID_ARG, "cache scale is NULL");
  if (d->d_rope > 0 && !c->rope) return fail(CSA_ERR_INVALID_ARG, "cache rope is NULL");
  if (!aligned16(c->nope) || !aligned16(c->ring) || !aligned16(c->scale) || !aligned16(c->rope))
    return fail(CSA_ERR_ALIGNMENT, "cache buffers must be 16-byte aligned");
  return CSA_OK;
}

static CompressParams make_params(const csa_cache_desc* d, const csa_cache* c, const void* a,
                                  const void* b, const void* za, const void* zb, const float* Ba,
                                  const float* Bb) {
  CompressParams P{};
  P.m = d->m;
  P.overlap = d->overlap;
  P.d_nope = d->d_nope;
  P.d_rope = d->d_rope;
  P.c = d->d_nope + d->d_rope;
  P.in_dt = d->in_dtype;
  P.nope_dt = d->nope_dtype;
  P.rope_dt = d->rope_dtype;
  P.R = d->overlap ? 2 * d->m : d->m;
  P.NT = d->overlap ? 4 : 2;
  P.base = d->rope_base;
  P.cap = d->capacity;
  P.a = a; P.b = b; P.za = za; P.zb = zb; P.Ba = Ba; P.Bb = Bb;
  P.nope = c->nope; P.scale = c->scale; P.rope = c->rope; P.ring = c->ring;
  return P;
}

static int validate_inputs(const csa_cache_desc* d, const void* a, const void* b, const void* za,
                           const void* zb, const float* Ba, const float* Bb) {
  if (!a || !za || !Ba) return fail(CSA_ERR_INVALID_ARG, "a, za, Ba must be non-NULL");
  if (d->overlap && (!b || !zb || !Bb)) return fail(CSA_ERR_INVALID_ARG, "overlap needs b, zb, Bb");
  if (!d->overlap && (b || zb || Bb)) return fail(CSA_ERR_INVALID_ARG, "b, zb, Bb must be NULL without overlap");
  if (!aligned16(a) || !aligned16(b) || !aligned16(za) || !aligned16(zb) || !aligned16(Ba) || !aligned16(Bb))
    return fail(CSA_ERR_ALIGNMENT, "inputs must be 16-byte aligned");
  return CSA_OK;
}

}  // namespace csa

using namespace csa;

extern "C" int csa_compress_prefill(const csa_cache_desc* desc, int B, int T, int64_t pos0,
                                    const void* a, const void* b, const void* za, const void* zb,
                                    const float* Ba, const float* Bb, const csa_cache* cache,
                                    void* stream) {
  int st;
  if ((st = validate_cache_desc(desc)) != CSA_OK) return st;
  if (B < 0 || T < 0 || pos0 < 0) return fail(CSA_ERR_INVALID_ARG, "B, T, pos0 must be >= 0");
  if ((st = validate_cache(desc, cache)) != CSA_OK) return st;
  if ((st = validate_inputs(desc, a, b, za, zb, Ba, Bb)) != CSA_OK) return st;
  if (B == 0 || T == 0) return CSA_OK;
  const int64_t m = desc->m;
  const int64_t i_first = (pos0 + m) / m - 1;  // first entry whose window ends at >= pos0
  const int64_t i_end = (pos0 + T) / m;        // entries [i_first, i_end) complete here
  if (i_end > desc->capacity) return fail(CSA_ERR_CAPACITY, "entries would exceed the cache capacity");
  if (B > 65535) return fail(CSA_ERR_INVALID_ARG, "B too large");
  CompressParams P = make_params(desc, cache, a, b, za, zb, Ba, Bb);
  P.T = T;
  P.pos0 = pos0;
  hipStream_t s = as_stream(stream);
  const size_t lds = (32 + P.c) * sizeof(float);
  if (i_end > i_first) {
    hipLaunchKernelGGL(compress_prefill_kernel, dim3(static_cast<unsigned>(i_end - i_first), B), dim3(256),
                       lds, s, P, i_first);
    if ((st = check_launch("compress_prefill_kernel")) != CSA_OK) return st;
  }
  const int64_t t_first = (pos0 + T - P.R > pos0) ? pos0 + T - P.R : pos0;
  hipLaunchKernelGGL(ring_store_kernel, dim3(static_cast<unsigned>(pos0 + T - t_first), B), dim3(256), 0, s,
                     P, t_first);
  return check_launch("ring_store_kernel");
}

extern "C" int csa_compress_decode(const csa_cache_desc* desc, int B, const int64_t* pos,
                                   const void* a, const void* b, const void* za, const void* zb,
                                   const float* Ba, const float* Bb, const csa_cache* cache,
                                   void* stream) {
  int st;
  if ((st = validate_cache_desc(desc)) != CSA_OK) return st;
  if (B < 0 || B > 65535) return fail(CSA_ERR_INVALID_ARG, "B must be in 0..65535");
  if (!pos || !aligned16(pos)) return fail(pos ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "pos must be a 16-byte aligned device pointer");
  if ((st = validate_cache(desc, cache)) != CSA_OK) return st;
  if ((st = validate_inputs(desc, a, b, za, zb, Ba, Bb)) != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  CompressParams P = make_params(desc, cache, a, b, za, zb, Ba, Bb);
  P.T = 1;
  P.pos0 = 0;
  const size_t lds = (32 + static_cast<size_t>(P.c)) * sizeof(float);
  const int threads = P.c >= 1024 ? 1024 : ((P.c + 63) / 64) * 64;
  if (P.in_dt == CSA_BF16)
    hipLaunchKernelGGL(compress_decode_kernel<true>, dim3(B), dim3(threads), lds, as_stream(stream), P, pos);
  else
    hipLaunchKernelGGL(compress_decode_kernel<false>, dim3(B), dim3(threads), lds, as_stream(stream), P, pos);
  return check_launch("compress_decode_kernel");
}
