// Compressor: every m tokens -> one KV entry, then RoPE and the storage
// format.  [CSA/HCA 混注意力] §1.1 工程细节 (overlapped C^a + C^b, 2m tokens
// per entry), §1.2 (HCA, single window of m' = 128), §1.4 存储格式混 (RoPE
// dims BF16, rest FP8); [读完这篇] §三 压缩机制 (per-dimension weights, 4 W +
// 2 B).
//
// Prefill: compress_prefill_wave_kernel gives each entry a group of lanes (a
// whole wave for 576-wide entries, 8 lanes for 64-wide indexer keys); lane l
// owns 8 consecutive channels and RoPE pair l, folds the 2m (or m) window
// rows into a per-channel online softmax in batches of rows, turns its RoPE
// pair in registers and reduces the FP8 / MXFP4 scales across lanes.
// compress_prefill_kernel (one workgroup per entry, one thread per channel)
// serves entry shapes outside that lane map.  Decode: one workgroup per
// sequence, one thread per channel, the window's older rows from the
// staging ring.  HBM traffic is the window rows in and one entry out; the
// kernels are bandwidth-bound and small next to attention.
#include "compress_store.hpp"
#include "index_prep.hpp"

namespace csa {

__device__ __forceinline__ float* ring_row(const CompressParams& P, int b, int64_t t, int which) {
  int64_t slot = t % P.R;
  return P.ring + ((static_cast<size_t>(b) * P.R + slot) * P.NT + which) * P.c;
}

// Weighted value of channel j of entry i, rows fetched by `get(which, t)`:
// the window's rows (C^a rows of window i, then the C^b rows of window
// i-1) in batches of CW_ROWS (clamped to the last row, so branch-free).
template <class Get>
__device__ __forceinline__ float compress_channel(const CompressParams& P, int64_t i, int j, Get get) {
  const int nrow = P.m + ((P.overlap && i >= 1) ? P.m : 0);
  float mx = -INFINITY, sw = 0.0f, acc = 0.0f;
  for (int r0 = 0; r0 < nrow; r0 += CW_ROWS) {
    float lg[CW_ROWS], vv[CW_ROWS];
#pragma unroll
    for (int u = 0; u < CW_ROWS; ++u) {
      const int rho = min(r0 + u, nrow - 1);
      const bool sa = rho < P.m;
      const int r = sa ? rho : rho - P.m;
      const int64_t t = sa ? i * P.m + r : (i - 1) * P.m + r;
      const float z = get(sa ? RING_ZA : RING_ZB, t, j);
      vv[u] = get(sa ? RING_A : RING_B, t, j);
      const float bw = (sa ? P.Ba : P.Bb)[r * P.c + j];
      lg[u] = r0 + u < nrow ? z + bw : -INFINITY;
    }
    softmax_batch(lg, vv, mx, sw, acc);
  }
  return acc / sw;
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
  const int64_t er = entry_row(P.pg, P.cap, b, i);  // uniform over the workgroup
  if (er < 0) return;                                // page outside the pool: not stored
  const size_t e = static_cast<size_t>(er);
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


// Prefill, a group of lanes per entry (a whole wave for 576-wide entries,
// 8 lanes for 64-wide ones; workgroup: 4 waves).  Lane l of the group owns
// the eight channels 8l .. 8l+7 of the non-RoPE part (l < d_nope / 8) and
// the RoPE pair d_nope + 2l, +1 (l < d_rope / 2), so the rotation stays in
// the lane and every load is a whole 16-byte (8-byte, 4-byte) piece.  A batch
// of CW_ROWS window rows is loaded at once; the softmax of each channel
// then runs over the batch with one rescale per batch (the window's rows:
// C^a rows of window i, then the C^b rows of window i-1).  Scale reductions
// of the storage formats run across lanes.
template <bool IN_BF16>
__global__ void __launch_bounds__(256, 2) compress_prefill_wave_kernel(CompressParams P, int64_t i_first,
                                                                    int64_t i_end) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int ng = P.d_nope / 8, np = P.d_rope / 2;
  const int lpe = wave_lanes_per_entry(ng, np), epw = 64 / lpe, ll = lane & (lpe - 1);
  const int64_t i0 = i_first + (4 * static_cast<int64_t>(blockIdx.x) + (threadIdx.x >> 6)) * epw;
  if (i0 >= i_end) return;
  const int64_t i = i0 + lane / lpe;  // this lane's entry
  const bool ok = i < i_end;
  const bool hg = ok && ll < ng, hp = ok && ll < np;
  const int jg = 8 * ll, jp = P.d_nope + 2 * ll;  // this lane's channels
  const int nrow = P.m + ((P.overlap && i >= 1) ? P.m : 0);
  const int nrow_w = P.overlap ? 2 * P.m : P.m;  // the wave's longest window
  // 8 + 2 channels: running max, sum of weights, weighted sum
  float mx[10], sw[10], acc[10];
#pragma unroll
  for (int c = 0; c < 10; ++c) { mx[c] = -INFINITY; sw[c] = 0.0f; acc[c] = 0.0f; }
  for (int r0 = 0; r0 < nrow_w; r0 += CW_ROWS) {
    float lg[CW_ROWS][10], vv[CW_ROWS][10];
#pragma unroll
    for (int u = 0; u < CW_ROWS; ++u) {
      const int rho = min(r0 + u, nrow - 1);
      const bool sa = rho < P.m;  // side a (C^a of window i) or side b (C^b of window i-1)
      const int r = sa ? rho : rho - P.m;
      const int64_t t = sa ? i * P.m + r : (i - 1) * P.m + r;
      const float* bw = (sa ? P.Ba : P.Bb) + static_cast<size_t>(r) * P.c;
      float z[10], v[10];
      if (t >= P.pos0) {
        const size_t row = (static_cast<size_t>(b) * P.T + (t - P.pos0)) * P.c;
        const void* zs = sa ? P.za : P.zb;
        const void* vs = sa ? P.a : P.b;
        if constexpr (IN_BF16) {
          const bf16_t* zp = static_cast<const bf16_t*>(zs) + row;
          const bf16_t* vp = static_cast<const bf16_t*>(vs) + row;
          u32x4 zq = {0u, 0u, 0u, 0u}, vq = zq;
          uint32_t zr = 0u, vr = 0u;
          if (hg) { zq = *reinterpret_cast<const u32x4*>(zp + jg); vq = *reinterpret_cast<const u32x4*>(vp + jg); }
          if (hp) { zr = *reinterpret_cast<const uint32_t*>(zp + jp); vr = *reinterpret_cast<const uint32_t*>(vp + jp); }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            z[2 * c] = __uint_as_float(zq[c] << 16); z[2 * c + 1] = __uint_as_float(zq[c] & 0xFFFF0000u);
            v[2 * c] = __uint_as_float(vq[c] << 16); v[2 * c + 1] = __uint_as_float(vq[c] & 0xFFFF0000u);
          }
          z[8] = __uint_as_float(zr << 16); z[9] = __uint_as_float(zr & 0xFFFF0000u);
          v[8] = __uint_as_float(vr << 16); v[9] = __uint_as_float(vr & 0xFFFF0000u);
        } else {
          const float* zp = static_cast<const float*>(zs) + row;
          const float* vp = static_cast<const float*>(vs) + row;
          f32x4 z0 = {}, z1 = {}, v0 = {}, v1 = {};
          f32x2 z2 = {}, v2 = {};
          if (hg) {
            z0 = *reinterpret_cast<const f32x4*>(zp + jg); z1 = *reinterpret_cast<const f32x4*>(zp + jg + 4);
            v0 = *reinterpret_cast<const f32x4*>(vp + jg); v1 = *reinterpret_cast<const f32x4*>(vp + jg + 4);
          }
          if (hp) { z2 = *reinterpret_cast<const f32x2*>(zp + jp); v2 = *reinterpret_cast<const f32x2*>(vp + jp); }
#pragma unroll
          for (int c = 0; c < 4; ++c) { z[c] = z0[c]; z[4 + c] = z1[c]; v[c] = v0[c]; v[4 + c] = v1[c]; }
          z[8] = z2[0]; z[9] = z2[1]; v[8] = v2[0]; v[9] = v2[1];
        }
      } else {  // rows before this call: the fp32 ring
        const float* zp = ring_row(P, b, t, sa ? RING_ZA : RING_ZB);
        const float* vp = ring_row(P, b, t, sa ? RING_A : RING_B);
#pragma unroll
        for (int c = 0; c < 10; ++c) { z[c] = 0.0f; v[c] = 0.0f; }
        if (hg)
#pragma unroll
          for (int c = 0; c < 8; ++c) { z[c] = zp[jg + c]; v[c] = vp[jg + c]; }
        if (hp) { z[8] = zp[jp]; z[9] = zp[jp + 1]; v[8] = vp[jp]; v[9] = vp[jp + 1]; }
      }
      float bb[10];
#pragma unroll
      for (int c = 0; c < 10; ++c) bb[c] = 0.0f;
      if (hg) {
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(bw + jg), b1 = *reinterpret_cast<const f32x4*>(bw + jg + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) { bb[c] = b0[c]; bb[4 + c] = b1[c]; }
      }
      if (hp) { bb[8] = bw[jp]; bb[9] = bw[jp + 1]; }
      const bool live = r0 + u < nrow;
#pragma unroll
      for (int c = 0; c < 10; ++c) {
        lg[u][c] = live ? z[c] + bb[c] : -INFINITY;
        vv[u][c] = v[c];
      }
    }
#pragma unroll
    for (int c = 0; c < 10; ++c) {
      float l1[CW_ROWS], v1[CW_ROWS];
#pragma unroll
      for (int u = 0; u < CW_ROWS; ++u) { l1[u] = lg[u][c]; v1[u] = vv[u][c]; }
      softmax_batch(l1, v1, mx[c], sw[c], acc[c]);
    }
  }
  float x[10];
#pragma unroll
  for (int c = 0; c < 10; ++c) x[c] = acc[c] / sw[c];
  store_entry_lanes(P, b, i, ok, hg, hp, ll, lpe, x);
}

// the wave kernel's shapes: one 8-channel group and one RoPE pair per lane
static bool compress_wave_ok(const CompressParams& P) {
  return P.d_nope % 8 == 0 && P.d_nope <= 512 && P.d_rope <= 128 && P.c % 8 == 0;
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
__device__ __forceinline__ void compress_decode_body(const CompressParams& P, const int64_t* pos_dev) {
  extern __shared__ float smem[];
  float* red = smem;        // 32
  float* buf = smem + 32;   // c: the emitted entry
  const int b = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const size_t row = static_cast<size_t>(b) * P.c;
  // the token's projections for this thread's first channel are read beside
  // the position (their addresses do not depend on it), without branches: a
  // compressor without C^b reads a's row in their place and drops it
  const bool has_b = P.NT == 4;
  const void* pb = has_b ? P.b : P.a;
  const void* pzb = has_b ? P.zb : P.za;
  auto load_cur = [&](int j, float (&cur)[4]) {
    cur[RING_A] = load_in<IN_BF16>(P.a, row + j);
    cur[RING_ZA] = load_in<IN_BF16>(P.za, row + j);
    const float vb = load_in<IN_BF16>(pb, row + j), vzb = load_in<IN_BF16>(pzb, row + j);
    cur[RING_B] = has_b ? vb : 0.0f;
    cur[RING_ZB] = has_b ? vzb : 0.0f;
  };
  const int64_t pos = pos_dev[b];
  float cur0[4];
  load_cur(min(tid, P.c - 1), cur0);
#pragma unroll
  for (int x = 0; x < 4; ++x) asm volatile("" : "+v"(cur0[x]));  // loaded here, not sunk past the test below
  if (pos < 0) return;
  const int64_t i = (pos + 1) / P.m - 1;
  const bool emit = (pos + 1) % P.m == 0 && i < P.cap;
  for (int j = tid; j < P.c; j += nt) {
    float cur[4];
    if (j == tid) {
#pragma unroll
      for (int x = 0; x < 4; ++x) cur[x] = cur0[x];
    } else {
      load_cur(j, cur);
    }
#pragma unroll
    for (int wch = 0; wch < 4; ++wch)
      if (wch < P.NT) ring_row(P, b, pos, wch)[j] = cur[wch];
    if (emit) {
      auto get = [&](int which, int64_t t, int jj) -> float {
        const float v = ring_row(P, b, t, which)[jj];
        const float c = which == RING_A ? cur[RING_A] : which == RING_ZA ? cur[RING_ZA]
                      : which == RING_B ? cur[RING_B] : cur[RING_ZB];  // selects, not an indexed array
        return t == pos ? c : v;
      };
      buf[j] = compress_channel(P, i, j, get);
    }
  }
  if (!emit) return;
  __syncthreads();
  finalize_entry(P, buf, red, b, i);
}


template <bool IN_BF16>
__global__ void __launch_bounds__(1024) compress_decode_kernel(CompressParams P, const int64_t* pos_dev) {
  compress_decode_body<IN_BF16>(P, pos_dev);
}

// The first launch of a fused CSA decode step, grid (B, 3): row y = 0
// compresses the new token into the KV cache, y = 1 into the indexer-key
// cache (the same code as compress_decode_kernel, so the entries are the
// same bits), y = 2 prepares the indexer's row b (histogram and candidate
// count cleared; the MXFP4 query operand when mx_prep).
template <bool IN_BF16>
__global__ void __launch_bounds__(1024) decode_step_prep_kernel(CompressParams Pkv, CompressParams Pkey, IndexParams Pi,
                                                                const int64_t* pos_dev, int mx_prep) {
  if (blockIdx.y == 0) {
    compress_decode_body<IN_BF16>(Pkv, pos_dev);
  } else if (blockIdx.y == 1) {
    compress_decode_body<IN_BF16>(Pkey, pos_dev);
  } else {
    const size_t r = blockIdx.x;
    if (mx_prep && threadIdx.x < 64) mx_prep_row(Pi, r);
    if (Pi.ghist) clear_decode_row(Pi, r);
  }
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
  if (d->capacity < 1) return fail(CSA_ERR_INVALID_ARG, "capacity must be >= 1");
  int st;
  if ((st = check_paging(d->page_size, d->pool_pages, d->capacity)) != CSA_OK) return st;
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
  Pages pg;
  return make_pages(d->page_size, d->pool_pages, d->capacity, c->block_table, &pg);
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
  make_pages(d->page_size, d->pool_pages, d->capacity, c->block_table, &P.pg);  // validated before
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

int compress_validate_cache(const csa_cache_desc* d, const csa_cache* c) {
  int st;
  if ((st = validate_cache_desc(d)) != CSA_OK) return st;
  return validate_cache(d, c);
}

CompressParams compress_make_params(const csa_cache_desc* d, const csa_cache* c, const float* Ba, const float* Bb) {
  return make_params(d, c, nullptr, nullptr, nullptr, nullptr, Ba, Bb);
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
    if (compress_wave_ok(P)) {
      const int per_wg = 4 * (64 / wave_lanes_per_entry(P.d_nope / 8, P.d_rope / 2));  // entries
      const dim3 grid(static_cast<unsigned>((i_end - i_first + per_wg - 1) / per_wg), B);
      if (P.in_dt == CSA_BF16)
        hipLaunchKernelGGL(compress_prefill_wave_kernel<true>, grid, dim3(256), 0, s, P, i_first, i_end);
      else
        hipLaunchKernelGGL(compress_prefill_wave_kernel<false>, grid, dim3(256), 0, s, P, i_first, i_end);
      if ((st = check_launch("compress_prefill_wave_kernel")) != CSA_OK) return st;
    } else {
      hipLaunchKernelGGL(compress_prefill_kernel, dim3(static_cast<unsigned>(i_end - i_first), B), dim3(256),
                         lds, s, P, i_first);
      if ((st = check_launch("compress_prefill_kernel")) != CSA_OK) return st;
    }
  }
  const int64_t t_first = (pos0 + T - P.R > pos0) ? pos0 + T - P.R : pos0;
  hipLaunchKernelGGL(ring_store_kernel, dim3(static_cast<unsigned>(pos0 + T - t_first), B), dim3(256), 0, s,
                     P, t_first);
  return check_launch("ring_store_kernel");
}

namespace csa {

int compress_decode_setup(const csa_cache_desc* desc, int B, const int64_t* pos, const void* a, const void* b,
                          const void* za, const void* zb, const float* Ba, const float* Bb, const csa_cache* cache,
                          CompressParams* out) {
  int st;
  if ((st = validate_cache_desc(desc)) != CSA_OK) return st;
  if (B < 0 || B > 65535) return fail(CSA_ERR_INVALID_ARG, "B must be in 0..65535");
  if (!pos || !aligned16(pos)) return fail(pos ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "pos must be a 16-byte aligned device pointer");
  if ((st = validate_cache(desc, cache)) != CSA_OK) return st;
  if ((st = validate_inputs(desc, a, b, za, zb, Ba, Bb)) != CSA_OK) return st;
  *out = make_params(desc, cache, a, b, za, zb, Ba, Bb);
  out->T = 1;
  out->pos0 = 0;
  return CSA_OK;
}

static int decode_threads(int c) { return c >= 1024 ? 1024 : ((c + 63) / 64) * 64; }

int launch_compress_decode(const CompressParams& P, int B, const int64_t* pos, hipStream_t s) {
  const size_t lds = (32 + static_cast<size_t>(P.c)) * sizeof(float);
  const int threads = decode_threads(P.c);
  if (P.in_dt == CSA_BF16)
    hipLaunchKernelGGL(compress_decode_kernel<true>, dim3(B), dim3(threads), lds, s, P, pos);
  else
    hipLaunchKernelGGL(compress_decode_kernel<false>, dim3(B), dim3(threads), lds, s, P, pos);
  return check_launch("compress_decode_kernel");
}

int launch_decode_step_prep(const CompressParams& kv, const CompressParams& keys, const IndexParams& ip, bool mx_prep,
                            int B, const int64_t* pos, hipStream_t s) {
  const int c = kv.c > keys.c ? kv.c : keys.c;
  const size_t lds = (32 + static_cast<size_t>(c)) * sizeof(float);
  int threads = decode_threads(c);
  if (threads < 256) threads = 256;  // the indexer rows clear 2048 histogram bins
  const dim3 grid(B, 3);
  if (kv.in_dt == CSA_BF16)
    hipLaunchKernelGGL(decode_step_prep_kernel<true>, grid, dim3(threads), lds, s, kv, keys, ip, pos, mx_prep ? 1 : 0);
  else
    hipLaunchKernelGGL(decode_step_prep_kernel<false>, grid, dim3(threads), lds, s, kv, keys, ip, pos, mx_prep ? 1 : 0);
  return check_launch("decode_step_prep_kernel");
}

}  // namespace csa

extern "C" int csa_compress_decode(const csa_cache_desc* desc, int B, const int64_t* pos,
                                   const void* a, const void* b, const void* za, const void* zb,
                                   const float* Ba, const float* Bb, const csa_cache* cache,
                                   void* stream) {
  CompressParams P;
  int st = compress_decode_setup(desc, B, pos, a, b, za, zb, Ba, Bb, cache, &P);
  if (st != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  return launch_compress_decode(P, B, pos, as_stream(stream));
}
