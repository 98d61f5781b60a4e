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
  const int64_t er = entry_row(P.pg, P.cap, b, s);
  const size_t e = er >= 0 ? static_cast<size_t>(er) : 0;  // a page outside the pool reads as row 0
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

// Exclusive prefix sums of two per-thread counts over the workgroup, in
// thread order (s_part: __shared__ int[34]); *ta and *tb get the totals.
// Every thread of the workgroup calls it: two barriers inside.
__device__ __forceinline__ void block_scan2(int a, int b, int* s_part, int* pa, int* pb, int* ta, int* tb) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  __syncthreads();  // earlier readers of s_part are done
  if (lane == 63) { s_part[wv] = ia; s_part[17 + wv] = ib; }
  __syncthreads();
  int ba = 0, bb = 0, sa = 0, sb = 0;
  for (int i = 0; i < nw; ++i) {
    const int xa = s_part[i], xb = s_part[17 + i];
    if (i < wv) { ba += xa; bb += xb; }
    sa += xa;
    sb += xb;
  }
  *pa = ba + ia - a;
  *pb = bb + ib - b;
  *ta = sa;
  *tb = sb;
}

// Wave 0's part of one radix-select step: the highest 8-bit digit whose bin
// brings the count of keys taken from the top up to `remaining`.  Lane l
// holds bins 255-4l .. 252-4l; the digit and the count in the bins above it
// go to s_sel[0], s_sel[1].
__device__ __forceinline__ void find_digit(const int* hist, int remaining, int* s_sel) {
  const int lane = threadIdx.x & 63;
  int c[4], tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; tot += c[j]; }
  const int incl = wave_incl_scan(tot);
  const int excl = incl - tot;
  if (excl < remaining && incl >= remaining) {
    int cum = excl;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!found && cum + c[j] >= remaining) {
        s_sel[0] = 255 - 4 * lane - j;
        s_sel[1] = cum;
        found = true;
      }
      cum += c[j];
    }
  } else if (lane == 63 && incl < remaining) {  // fewer keys than asked for: digit 0
    s_sel[0] = 0;
    s_sel[1] = incl - c[3];
  }
}

// Radix select by the whole workgroup over cnt keys key_of(i): 8-bit digits
// over the key's first key_bits bits, below the bits already known (the
// keys matching prefix0 under pmask0 hold the k-th largest; k counts from
// the largest of them; the next digit ends at bit top_shift).  The last
// digit may overlap known bits (it then starts at bit 0).  On return
// *prefix holds the k-th largest key (masked by *pmask) and *rem how many
// keys equal to it belong to the top k.
template <typename KeyOf>
__device__ __forceinline__ void radix_threshold(KeyOf key_of, int64_t cnt, int k, int key_bits, int* hist, int* s_sel,
                                uint32_t* prefix_out, uint32_t* pmask_out, int* rem_out, uint32_t prefix0 = 0u,
                                uint32_t pmask0 = 0u, int top_shift = 24) {
  constexpr int U = 4;  // loads in flight per thread
  const int tid = threadIdx.x, nt = blockDim.x;
  uint32_t prefix = prefix0, pmask = pmask0;
  int remaining = k;
  for (int sd = top_shift;; sd -= 8) {
    const int shift = sd < 0 ? 0 : sd;
    if (shift + 8 <= 32 - key_bits) break;  // only bits below the key's width left
    for (int i = tid; i < 256; i += nt) hist[i] = 0;
    __syncthreads();
    for (int64_t base = 0; base < cnt; base += static_cast<int64_t>(U) * nt) {
      uint32_t key[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * nt + tid;
        key[u] = i < cnt ? key_of(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * nt + tid;
        wave_hist_add(hist, (key[u] >> shift) & 255u, i < cnt && (key[u] & pmask) == prefix);
      }
    }
    __syncthreads();
    if (tid < 64) find_digit(hist, remaining, s_sel);
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_sel[0]) << shift;
    remaining -= s_sel[1];
    pmask |= 255u << shift;
    if (shift == 0) break;
  }
  *prefix_out = prefix;
  *pmask_out = pmask;
  *rem_out = remaining;
}

// Ordered compaction after radix_threshold: the elements whose key is above
// the threshold, and the first `remaining` equal to it, in element order,
// put(j, idx_of(i)) for output slots j = 0, 1, ..  Each thread takes E
// consecutive elements per tile; one workgroup scan per tile (fewer
// elements per thread keep LDS key reads from piling onto the same banks).
template <int E = 8, typename KeyOf, typename IdxOf, typename Put>
__device__ __forceinline__ void ordered_take(KeyOf key_of, IdxOf idx_of, int64_t cnt, uint32_t prefix, uint32_t pmask,
                             int remaining, int* s_part, Put put) {
  const int tid = threadIdx.x, nt = blockDim.x;
  int gt_done = 0, eq_done = 0;
  for (int64_t base = 0; base < cnt; base += static_cast<int64_t>(E) * nt) {
    const int64_t i0 = base + static_cast<int64_t>(tid) * E;
    uint32_t key[E];
    int ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < E; ++u) key[u] = i0 + u < cnt ? key_of(i0 + u) & pmask : 0u;
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const bool ok = i0 + u < cnt;
      ngt += ok && key[u] > prefix;
      neq += ok && key[u] == prefix;
    }
    int pg, pe, tg, te;
    block_scan2(ngt, neq, s_part, &pg, &pe, &tg, &te);
    int eq_before = eq_done + pe;
    int pos = gt_done + pg + min(eq_before, remaining);
#pragma unroll
    for (int u = 0; u < E; ++u) {
      if (i0 + u >= cnt) break;
      if (key[u] > prefix) {
        put(pos++, idx_of(i0 + u));
      } else if (key[u] == prefix) {
        if (eq_before < remaining) put(pos++, idx_of(i0 + u));
        ++eq_before;
      }
    }
    gt_done += tg;
    eq_done += te;
  }
}

// Top-k of sc[0..n) (n > k) by one workgroup, ascending indices, ties to the
// lower index; put(j, index) for slots j < k.
template <typename Put>
__device__ __forceinline__ void row_radix_select(const float* sc, int64_t n, int k, int key_bits, Put put) {
  __shared__ int hist[256];
  __shared__ int s_sel[2];
  __shared__ int s_part[34];
  uint32_t prefix, pmask;
  int remaining;
  auto key_of = [sc](int64_t i) { return score_key(sc[i]); };
  radix_threshold(key_of, n, k, key_bits, hist, s_sel, &prefix, &pmask, &remaining);
  ordered_take(key_of, [](int64_t i) { return static_cast<int32_t>(i); }, n, prefix, pmask, remaining, s_part, put);
}

// One workgroup (1024 threads) selects the top-k of one query row.
__global__ void __launch_bounds__(1024) topk_radix_kernel(IndexParams P, int key_bits) {
  const int b = blockIdx.y, t = blockIdx.x;
  const int64_t n = visible(query_pos(P, b, t), P.m, P.cap);
  const size_t row = static_cast<size_t>(b) * P.T + t;
  int32_t* out = P.idx + row * P.k;
  if (n <= P.k) {
    for (int64_t j = threadIdx.x; j < P.k; j += blockDim.x) out[j] = j < n ? static_cast<int32_t>(j) : -1;
    return;
  }
  row_radix_select(P.ws + row * P.n_stride, n, P.k, key_bits, [out](int64_t j, int32_t id) { out[j] = id; });
}

// ---------------------------------------------------------------------------
// decode top-k across workgroups: the scan kernel has already added every
// score's top-11-bit bin to ghist; here the threshold bin of each row is
// found, each CAND_CHUNK-entry chunk compacts its entries at or above it in
// index order, and one workgroup per row puts the chunks in order and
// selects exactly among the candidates.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) topk_zero_kernel(IndexParams P) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < HIST_BINS; i += blockDim.x) P.ghist[static_cast<size_t>(b) * HIST_BINS + i] = 0;
  if (threadIdx.x == 0) P.ccount[b] = 0;
}

// A 256-thread workgroup's share of row b's histogram: thread t holds the
// counts of bins HIST_BINS-1-(PER t + j) (thread 0 the top bins).
constexpr int HIST_PER = HIST_BINS / 256;
__device__ __forceinline__ void load_hist(const int* gh, int (&c)[HIST_PER]) {
#pragma unroll
  for (int j = 0; j < HIST_PER; ++j) c[j] = gh[HIST_BINS - 1 - (threadIdx.x * HIST_PER + j)];
}

// The bin of the k-th largest key of row b from the loaded histogram (all
// 256 threads get it); the number of keys in higher bins is left in s_part[5].
__device__ int threshold_bin(const int (&c)[HIST_PER], int k, int* s_part) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int PER = HIST_PER;
  int tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) tot += c[j];
  int incl = wave_incl_scan(tot);
  if (lane == 63) s_part[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += s_part[i];
  incl += before;
  const int excl = incl - tot;
  __syncthreads();
  if (excl < k && incl >= k) {
    int cum = excl;
    for (int j = 0; j < PER; ++j) {
      if (cum + c[j] >= k) { s_part[4] = HIST_BINS - 1 - (tid * PER + j); s_part[5] = cum; break; }
      cum += c[j];
    }
  }
  __syncthreads();
  return s_part[4];
}

__global__ void __launch_bounds__(256) topk_cand_kernel(IndexParams P) {
  constexpr int PERW = CAND_CHUNK / 4;  // entries per wave
  constexpr int IT = PERW / 64;
  __shared__ int s_part[8];
  __shared__ uint32_t s_ck[CAND_CHUNK];
  __shared__ int32_t s_ci[CAND_CHUNK];
  __shared__ int s_wc[4];
  __shared__ int s_base;
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t pos = P.pos_dev[b];  // decode: positions on the device
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * CAND_CHUNK;
  const float* sc = P.ws + static_cast<size_t>(b) * P.n_stride;
  const int64_t e0 = c0 + wv * PERW + lane;
  // the chunk's scores (indices kept inside the row's stride; those past the
  // visible entries are not taken) and the row's histogram are read beside
  // the position, not after it
  float v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) v[it] = sc[min(e0 + it * 64, P.n_stride - 1)];
  int hc[HIST_PER];
  load_hist(P.ghist + static_cast<size_t>(b) * HIST_BINS, hc);
#pragma unroll
  for (int it = 0; it < IT; ++it) asm volatile("" : "+v"(v[it]));  // loaded here, not sunk past the test below
#pragma unroll
  for (int j = 0; j < HIST_PER; ++j) asm volatile("" : "+v"(hc[j]));
  const int64_t n = visible(pos, P.m, P.cap);
  if (n <= P.k || c0 >= n) return;
  const int64_t c1 = c0 + CAND_CHUNK < n ? c0 + CAND_CHUNK : n;
  const int bstar = threshold_bin(hc, P.k, s_part);
  if (blockIdx.x == 0 && tid == 0) {  // for the final select: the known top bits
    P.csel[2 * b] = bstar;
    P.csel[2 * b + 1] = s_part[5];
  }
  // each wave compacts its quarter of the chunk, in index order, into its
  // own LDS segment
  const unsigned long long below = (1ull << lane) - 1ull;
  int cnt = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t s = e0 + it * 64;
    const uint32_t key = score_key(v[it]);
    const bool take = s < c1 && static_cast<int>(key >> (32 - HIST_BITS)) >= bstar;
    const unsigned long long m = __ballot(take);
    if (take) {
      const int pos = wv * PERW + cnt + __popcll(m & below);
      s_ck[pos] = key;
      s_ci[pos] = static_cast<int32_t>(s);
    }
    cnt += __popcll(m);
  }
  if (lane == 0) s_wc[wv] = cnt;
  __syncthreads();
  const int p1 = s_wc[0], p2 = p1 + s_wc[1], p3 = p2 + s_wc[2], tot = p3 + s_wc[3];
  const size_t cj = static_cast<size_t>(b) * P.nch + blockIdx.x;
  if (tid == 0) {
    const int base = tot ? atomicAdd(&P.ccount[b], tot) : 0;  // one global atomic per chunk
    s_base = base;
    P.cbase[cj] = base;
    P.ccnt[cj] = tot;
  }
  __syncthreads();
  const int gbase = s_base;
  const size_t cb0 = static_cast<size_t>(b) * CAND_CAP;
  for (int i = tid; i < tot; i += 256) {
    if (gbase + i >= CAND_CAP) break;
    const int w = (i >= p1) + (i >= p2) + (i >= p3);
    const int src = w * PERW + i - (w == 0 ? 0 : w == 1 ? p1 : w == 2 ? p2 : p3);
    P.ckey[cb0 + gbase + i] = s_ck[src];
    P.cidx[cb0 + gbase + i] = s_ci[src];
  }
}

constexpr int ROW_TAB_LDS = 4096;  // block-table entries the final pass stages in LDS

__global__ void __launch_bounds__(1024) topk_final_kernel(IndexParams P, int key_bits) {
  constexpr int CPT = NCH_MAX / 1024;  // chunks per thread
  __shared__ int32_t s_tab[ROW_TAB_LDS];
  __shared__ uint32_t s_key[CAND_CAP];
  __shared__ int32_t s_idx[CAND_CAP];
  __shared__ int s_pre[NCH_MAX];
  __shared__ int s_cb[NCH_MAX];
  __shared__ int hist[256];
  __shared__ int s_sel[2];
  __shared__ int s_part[34];
  const int b = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int64_t pos = P.pos_dev[b];  // decode: positions on the device
  int32_t* out = P.idx + static_cast<size_t>(b) * P.k;
  // the row's chunk counts and bases (every chunk slot of the row; those past
  // the visible entries are dropped below) and its whole candidate list are
  // read beside the position, not after it; slots past the row's candidate
  // count hold older values and are not used
  const size_t rb = static_cast<size_t>(b) * P.nch;
  const size_t cb0 = static_cast<size_t>(b) * CAND_CAP;
  constexpr int CL = CAND_CAP / 1024;
  int32_t cid[CL];
  uint32_t ckv[CL];
  int cc[CPT], cbv[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int j = min(tid * CPT + u, P.nch - 1);
    cc[u] = P.ccnt[rb + j];
    cbv[u] = P.cbase[rb + j];
  }
#pragma unroll
  for (int u = 0; u < CL; ++u) {
    cid[u] = P.cidx[cb0 + tid + 1024 * u];
    ckv[u] = P.ckey[cb0 + tid + 1024 * u];
  }
  // the histogram bin of the k-th key and the count above it (the candidate
  // pass's chunk 0 wrote them)
  uint32_t bstar = static_cast<uint32_t>(P.csel[2 * b]);
  int above = P.csel[2 * b + 1];
#pragma unroll
  for (int u = 0; u < CPT; ++u) asm volatile("" : "+v"(cc[u]), "+v"(cbv[u]));  // loaded here, not sunk past the test below
  asm volatile("" : "+s"(bstar), "+s"(above));
  const int64_t n = visible(pos, P.m, P.cap);
  // a fused decode step over a paged KV cache: each selected entry's pool
  // row as well, the list its sparse attention reads (-1 on a page outside
  // the pool, like the padding).  The sequence's block-table row is staged
  // in LDS first (when it fits), so that no output waits on a table load.
  int32_t* rows = P.rows_out ? P.rows_out + static_cast<size_t>(b) * P.k : nullptr;
  const bool tab_lds = rows && P.row_pg.table && P.row_pg.tps <= ROW_TAB_LDS;
  // the table row's loads are issued now and land in LDS just before the
  // first output (stage_tab; a barrier follows before any put)
  int32_t tr[ROW_TAB_LDS / 1024];
  if (tab_lds) {
#pragma unroll
    for (int u = 0; u < ROW_TAB_LDS / 1024; ++u) {
      const int64_t j = tid + 1024 * u;
      tr[u] = j < P.row_pg.tps ? P.row_pg.table[b * P.row_pg.tps + j] : 0;
    }
  }
  auto stage_tab = [&]() {
    if (tab_lds)
#pragma unroll
      for (int u = 0; u < ROW_TAB_LDS / 1024; ++u) s_tab[tid + 1024 * u] = tr[u];
  };
  auto row_of = [&](int32_t id) -> int32_t {
    if (!tab_lds) return static_cast<int32_t>(entry_row(P.row_pg, P.row_cap, b, id));
    const int64_t pg = s_tab[id >> P.row_pg.shift];
    if (pg < 0 || pg >= P.row_pg.pool) return -1;
    return static_cast<int32_t>((pg << P.row_pg.shift) | (id & ((1 << P.row_pg.shift) - 1)));
  };
  auto put = [&](int64_t j, int32_t id) {
    out[j] = id;
    if (rows) rows[j] = id >= 0 ? row_of(id) : -1;
  };
  if (n <= P.k) {
    stage_tab();
    __syncthreads();
    for (int64_t j = tid; j < P.k; j += nt) put(j, j < n ? static_cast<int32_t>(j) : -1);
    return;
  }
  // where each chunk's candidates go in index order: prefix of the chunk
  // counts (their sum is the row's candidate count)
  const int nch = static_cast<int>((n + CAND_CHUNK - 1) / CAND_CHUNK);
  int loc = 0;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int j = tid * CPT + u;
    if (j < nch) s_cb[j] = cbv[u];
    else cc[u] = 0;
    loc += cc[u];
  }
  int pre, unused, c, unused_tot;
  block_scan2(loc, 0, s_part, &pre, &unused, &c, &unused_tot);
  if (c > CAND_CAP) {  // too many candidates: exact select over the whole row
    stage_tab();          // (the select's barriers precede its first output)
    row_radix_select(P.ws + static_cast<size_t>(b) * P.n_stride, n, P.k, key_bits, put);
    return;
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int j = tid * CPT + u;
    if (j < nch) s_pre[j] = pre;
    pre += cc[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < CL; ++u) {
    const int i = tid + 1024 * u;
    if (i < c) {
      const int j = cid[u] / CAND_CHUNK;
      const int d = s_pre[j] + (i - s_cb[j]);
      s_key[d] = ckv[u];
      s_idx[d] = cid[u];
    }
  }
  __syncthreads();
  // the k-th key lies in the histogram's bin (its top HIST_BITS bits), with
  // `above` candidates in higher bins: the select starts below those bits
  uint32_t prefix, pmask;
  int remaining;
  auto key_of = [](int64_t i) { return s_key[i]; };
  radix_threshold(key_of, c, P.k - above, key_bits, hist, s_sel, &prefix, &pmask, &remaining,
                  bstar << (32 - HIST_BITS), ~0u << (32 - HIST_BITS), 32 - HIST_BITS - 8);
  stage_tab();  // ordered_take's workgroup scan (barriers) precedes its first output
  ordered_take<4>(key_of, [](int64_t i) { return s_idx[i]; }, c, prefix, pmask, remaining, s_part, put);
}

// prep_done: the decode rows' preparation (cleared histogram and count,
// MXFP4 query operands) has already been enqueued by a fused decode step.
static int launch_index(IndexParams& P, int B, int64_t n_max, void* stream, bool prep_done = false) {
  hipStream_t s = as_stream(stream);
  if (index_mfma_supported(P)) {
    // scores stay on chip when every row fits the fused kernel's LDS rows
    if (!P.scores_out && index_fused_prefill_ok(P, n_max)) return launch_index_fused_prefill(P, B, s);
    const int bits = P.score_dt == CSA_BF16 ? 16 : 32;
    if (P.ghist) {  // decode: histogram in the scan, candidates, exact final select
      int st = CSA_OK;
      if (prep_done) {
      } else if (index_scan_mx(P)) {
        st = launch_index_mx_prep(P, B, s);  // clears the histograms too
      } else {
        hipLaunchKernelGGL(topk_zero_kernel, dim3(B), dim3(256), 0, s, P);
        st = check_launch("topk_zero_kernel");
      }
      if (st != CSA_OK) return st;
      if (n_max > 0 && (st = launch_index_scan(P, B, n_max, s)) != CSA_OK) return st;
      hipLaunchKernelGGL(topk_cand_kernel, dim3(static_cast<unsigned>(P.nch), B),
                         dim3(256), 0, s, P);
      if ((st = check_launch("topk_cand_kernel")) != CSA_OK) return st;
      hipLaunchKernelGGL(topk_final_kernel, dim3(B), dim3(1024), 0, s, P, bits);
      return check_launch("topk_final_kernel");
    }
    if (n_max > 0) {
      int st = index_scan_mx(P) ? launch_index_mx_prep(P, B * P.T, s) : CSA_OK;
      if (st != CSA_OK || (st = launch_index_scan(P, B, n_max, s)) != CSA_OK) return st;
    }
    if (index_ws_select_ok(P, n_max)) return launch_index_ws_select(P, B, s);
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
  return check_paging(d->page_size, d->pool_pages, d->capacity);
}

static int64_t stride_for(int64_t n) { return ((n + 63) / 64) * 64; }

static int64_t prefill_nmax(const csa_index_desc* d, int T, int64_t pos0) {
  int64_t n = (pos0 + T) / d->m;  // visible to the last query (pos0 + T - 1)
  return n < d->capacity ? n : d->capacity;
}

static int64_t cand_chunks(int64_t cap) { return (cap + CAND_CHUNK - 1) / CAND_CHUNK; }

// decode workspace after the score rows: histograms, counts, candidates,
// per-chunk candidate bases and counts
static size_t decode_extra_bytes(int B, int64_t cap) {
  return static_cast<size_t>(B) * (HIST_BINS * sizeof(int) + 64 + CAND_CAP * (sizeof(uint32_t) + sizeof(int32_t)) +
                                   2 * cand_chunks(cap) * sizeof(int) + 2 * sizeof(int));
}

size_t index_ws_bytes(const csa_index_desc* d, int op, int B, int T, int64_t pos0) {
  if (!d || B < 0 || T < 0) return 0;
  int64_t nmax = op == CSA_OP_INDEX_TOPK_DECODE ? d->capacity : prefill_nmax(d, T, pos0);
  int64_t rows = static_cast<int64_t>(B) * (op == CSA_OP_INDEX_TOPK_DECODE ? 1 : T);
  size_t bytes = static_cast<size_t>(rows * stride_for(nmax) * sizeof(float)) + 256;
  if (d->qk_dtype == CSA_MXFP4) bytes += static_cast<size_t>(rows) * QPACK_ROW_BYTES + 256;
  if (op == CSA_OP_INDEX_TOPK_DECODE) bytes += decode_extra_bytes(B, d->capacity);
  return bytes;
}

// Workspace after the score rows: the MXFP4 query operands (when the
// scaled-MFMA scan runs), then whatever follows; each part 256-byte aligned.
static char* align256(char* p) { return p + (256 - reinterpret_cast<uintptr_t>(p) % 256) % 256; }

static char* place_qpack(IndexParams& P, int64_t rows) {
  char* p = align256(reinterpret_cast<char*>(P.ws) + static_cast<size_t>(rows) * P.n_stride * sizeof(float));
  if (P.qk_dt != CSA_MXFP4) return p;
  P.qpack = reinterpret_cast<uint8_t*>(p);
  return align256(p + static_cast<size_t>(rows) * QPACK_ROW_BYTES);
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
  Pages pg;
  return make_pages(d->page_size, d->pool_pages, d->capacity, keys->block_table, &pg);
}

static IndexParams make_index_params(const csa_index_desc* d, const void* qI, const float* w,
                                     const csa_cache* keys, int k, int32_t* idx, float* scores, void* ws) {
  IndexParams P{};
  P.H = d->n_heads; P.D = d->dim; P.q_dt = d->q_dtype; P.qk_dt = d->qk_dtype;
  P.key_dt = d->key_dtype; P.score_dt = d->score_dtype; P.m = d->m; P.cap = d->capacity;
  P.qI = qI; P.w = w; P.knope = keys->nope; P.kscale = keys->scale;
  P.k = k; P.idx = idx; P.scores_out = scores;
  P.ws = static_cast<float*>(ws);
  make_pages(d->page_size, d->pool_pages, d->capacity, keys->block_table, &P.pg);  // validated before
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
  if (desc->page_size != 0) return fail(CSA_ERR_UNSUPPORTED, "paged key caches are read by the decode indexer only");
  if (ws_bytes < index_ws_bytes(desc, CSA_OP_INDEX_TOPK_PREFILL, B, T, pos0))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  if (B == 0 || T == 0) return CSA_OK;
  IndexParams P = make_index_params(desc, qI, w, keys, k, idx, scores, ws);
  P.T = T;
  P.pos0 = pos0;
  P.pos_dev = nullptr;
  const int64_t nmax = prefill_nmax(desc, T, pos0);
  P.n_stride = stride_for(nmax);
  place_qpack(P, static_cast<int64_t>(B) * T);
  return launch_index(P, B, nmax, stream);
}

namespace csa {

int index_decode_setup(const csa_index_desc* desc, int B, const int64_t* pos, const void* qI, const float* w,
                       const csa_cache* keys, int k, int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                       IndexParams* out) {
  int st = common_index_checks(desc, B, qI, w, keys, k, idx, scores, ws);
  if (st != CSA_OK) return st;
  if (!pos || !aligned16(pos)) return fail(pos ? CSA_ERR_ALIGNMENT : CSA_ERR_INVALID_ARG, "pos must be an aligned device pointer");
  if (ws_bytes < index_ws_bytes(desc, CSA_OP_INDEX_TOPK_DECODE, B, 1, 0))
    return fail(CSA_ERR_WORKSPACE, "workspace too small");
  IndexParams P = make_index_params(desc, qI, w, keys, k, idx, scores, ws);
  P.T = 1;
  P.pos0 = 0;
  P.pos_dev = pos;
  P.n_stride = stride_for(desc->capacity);
  char* extra = place_qpack(P, B);
  if (index_mfma_supported(P) && cand_chunks(desc->capacity) <= NCH_MAX) {
    P.ghist = reinterpret_cast<int*>(extra);
    P.ccount = P.ghist + static_cast<size_t>(B) * HIST_BINS;
    P.ckey = reinterpret_cast<uint32_t*>(P.ccount + ((B + 15) / 16) * 16);
    P.cidx = reinterpret_cast<int32_t*>(P.ckey + static_cast<size_t>(B) * CAND_CAP);
    P.nch = static_cast<int>(cand_chunks(desc->capacity));
    P.cbase = reinterpret_cast<int*>(P.cidx + static_cast<size_t>(B) * CAND_CAP);
    P.ccnt = P.cbase + static_cast<size_t>(B) * P.nch;
    P.csel = P.ccnt + static_cast<size_t>(B) * P.nch;
  }
  *out = P;
  return CSA_OK;
}

bool index_decode_prep_mx(const IndexParams& P) { return P.ghist != nullptr && index_scan_mx(P); }

int launch_index_decode(IndexParams& P, int B, void* stream, bool prep_done) {
  // rows without the multi-workgroup state need no preparation
  return launch_index(P, B, P.cap, stream, prep_done && P.ghist != nullptr);
}

}  // namespace csa

extern "C" int csa_index_topk_decode(const csa_index_desc* desc, int B, const int64_t* pos,
                                     const void* qI, const float* w, const csa_cache* keys, int k,
                                     int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                                     void* stream) {
  IndexParams P;
  int st = index_decode_setup(desc, B, pos, qI, w, keys, k, idx, scores, ws, ws_bytes, &P);
  if (st != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  return launch_index_decode(P, B, stream, false);
}
