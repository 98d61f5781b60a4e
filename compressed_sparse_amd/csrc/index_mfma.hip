// MFMA lightning indexer for 16 heads x 64 dims (BF16 or MXFP4 QK product;
// BF16, FP8-with-scale or MXFP4 keys).  [CSA/HCA 混注意力] §1.4 LIGHTNING
// INDEXER 的 FP4 计; [读完这篇] §三 CSA 步骤二.
//
//   I[s] = sum_h w[h] * ReLU(qI[h] . K[s])
//
// index_prefill_fused_kernel: 4 consecutive queries per workgroup, i.e. 64
//   MFMA rows (query x head) against 32-entry column blocks
//   (v_mfma_f32_32x32x16_bf16, keys loaded straight from L2 as the B
//   operand).  The 4 score rows stay in LDS (4 x 8192 fp32) and each wave
//   then radix-selects one row's top-k, so scores never reach HBM.
// index_scan_kernel: one query row against a 1024-entry chunk per
//   workgroup (v_mfma_f32_16x16x32_bf16, rows = the 16 heads); the decode
//   scan and the fallback for long prefill rows.  FP8 and E2M1 codes widen
//   to BF16 exactly in registers; the per-entry FP8 scale multiplies the dot
//   product, the E8M0 block scales are folded into the widened values.
//
// Both kernels reduce heads in a fixed order (4 or 8 heads inside a lane,
// then fixed cross-lane shuffles), so scores are run-to-run deterministic.
#include "index.hpp"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int HI = 16;
constexpr int DI = 64;
constexpr int QG = 4;          // queries per fused workgroup
constexpr int FUSED_NMAX = 8192;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Hardware widening of FP8 E4M3 / E2M1 codes to BF16 (the scaled
// conversions with scale 1: exact for every code).  fp8x8: two words, first
// byte first; e2m1x8: one word, low nibble first.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI));
}

__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
               fp8x2_to_bf16x2<true>(w1)};
}

template <int BYTE>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, BYTE));
}

__device__ __forceinline__ u32x4 e2m1x8_to_bf16(uint32_t word) {
  return u32x4{e2m1x2_to_bf16x2<0>(word), e2m1x2_to_bf16x2<1>(word), e2m1x2_to_bf16x2<2>(word),
               e2m1x2_to_bf16x2<3>(word)};
}

// Orders this wave's LDS accesses before the ones that follow.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// fused prefill: scores of 4 queries in LDS, then one wave per row selects
// ---------------------------------------------------------------------------

// Wave-level radix select of the top-k of row[0..n) (n > k) and ordered
// compaction of the selected indices into out[0..k).
__device__ void wave_radix_select(const float* row, int n, int k, int key_bits, int* hist, int32_t* out) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  for (int shift = 24; shift >= 32 - key_bits; shift -= 8) {
    for (int i = lane; i < 256; i += 64) hist[i] = 0;
    wave_lds_sync();
    for (int s = lane; s < n; s += 64) {
      const uint32_t key = order_key(row[s]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    wave_lds_sync();
    // lane i owns bins 255-4i .. 252-4i (descending); inclusive scan from the top
    int c[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; tot += c[j]; }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int excl = incl - tot;  // count in bins above this lane's bins
    int bin = -1, above = 0;
    if (excl < remaining && incl >= remaining) {
      int cum = excl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (bin < 0 && cum + c[j] >= remaining) { bin = 255 - 4 * lane - j; above = cum; }
        cum += c[j];
      }
    }
    const unsigned long long who = __ballot(bin >= 0);
    const int src = __ffsll(static_cast<long long>(who)) - 1;
    bin = __shfl(bin, src);
    above = __shfl(above, src);
    prefix |= static_cast<uint32_t>(bin) << shift;
    pmask |= 255u << shift;
    remaining -= above;
    wave_lds_sync();
  }
  int taken_eq = 0, written = 0;
  for (int base = 0; base < n; base += 64) {
    const int s = base + lane;
    const uint32_t key = s < n ? (order_key(row[s]) & pmask) : 0u;
    const bool gt = s < n && key > prefix;
    const bool eq = s < n && key == prefix;
    const unsigned long long below = (1ull << lane) - 1ull;
    const unsigned long long eqm = __ballot(eq);
    const bool take = gt || (eq && taken_eq + __popcll(eqm & below) < remaining);
    const unsigned long long tm = __ballot(take);
    if (take) out[written + __popcll(tm & below)] = s;
    taken_eq += __popcll(eqm);
    written += __popcll(tm);
  }
  for (int j = written + lane; j < k; j += 64) out[j] = -1;
}

constexpr int SEL_BINS = 1024;  // value-range bins of the fused select
constexpr int SEL_CB = 256;     // threshold-bin entries ranked directly

// Exact top-k of row[0..n) (n > k) by one wave, ascending indices, ties to
// the lower index.  The row's scores fall into SEL_BINS equal-width bins
// between its min and max (a monotone map, so a bin holds a contiguous key
// range and equal scores share a bin); the histogram finds the bin B that
// holds the k-th largest score.  Bins above B are taken whole; the entries
// of B are ranked by (key descending, index ascending) against each other
// and the best k - |bins above B| taken; one last pass writes the indices
// in order.  A threshold bin with more than SEL_CB entries (heavy ties)
// falls back to the radix select.
__device__ void wave_select(const float* row, int n, int k, int key_bits, int* hist, int* cidx, uint32_t* ckey,
                            int* crank, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  // lane l reads entries 4(base + l) .. +3 of each 256-entry step (the row
  // is 16-byte aligned and padded past n)
  auto quad = [&](int base) { return *reinterpret_cast<const float4*>(row + 4 * (base + lane)); };
  float mn = INFINITY, mx = -INFINITY;
  for (int base = 0; 4 * base < n; base += 64) {
    const float4 v = quad(base);
    const int s = 4 * (base + lane);
    if (s < n) { mn = fminf(mn, v.x); mx = fmaxf(mx, v.x); }
    if (s + 1 < n) { mn = fminf(mn, v.y); mx = fmaxf(mx, v.y); }
    if (s + 2 < n) { mn = fminf(mn, v.z); mx = fmaxf(mx, v.z); }
    if (s + 3 < n) { mn = fminf(mn, v.w); mx = fmaxf(mx, v.w); }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  const float span = mx - mn;
  float scale = span > 0.0f ? static_cast<float>(SEL_BINS) / span : 0.0f;
  if (!(scale < 3.0e38f)) scale = 0.0f;  // degenerate range: one bin, radix fallback
  auto bin_of = [&](float v) { return min(SEL_BINS - 1, static_cast<int>((v - mn) * scale)); };
  for (int i = lane; i < SEL_BINS; i += 64) hist[i] = 0;
  wave_lds_sync();
  for (int base = 0; 4 * base < n; base += 64) {
    const float4 v = quad(base);
    const int s = 4 * (base + lane);
    if (s < n) atomicAdd(&hist[bin_of(v.x)], 1);
    if (s + 1 < n) atomicAdd(&hist[bin_of(v.y)], 1);
    if (s + 2 < n) atomicAdd(&hist[bin_of(v.z)], 1);
    if (s + 3 < n) atomicAdd(&hist[bin_of(v.w)], 1);
  }
  wave_lds_sync();
  // lane l owns bins SEL_BINS-1-16l .. SEL_BINS-16-16l (descending)
  constexpr int PER = SEL_BINS / 64;
  int c[PER], tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { c[j] = hist[SEL_BINS - 1 - PER * lane - j]; tot += c[j]; }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  int bsel = -1, above = 0;
  if (incl - tot < k && incl >= k) {
    int cum = incl - tot;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (bsel < 0 && cum + c[j] >= k) { bsel = SEL_BINS - 1 - PER * lane - j; above = cum; }
      cum += c[j];
    }
  }
  const unsigned long long who = __ballot(bsel >= 0);
  const int src = __ffsll(static_cast<long long>(who)) - 1;
  const int B = __builtin_amdgcn_readlane(bsel, src);
  const int rem = k - __builtin_amdgcn_readlane(above, src);  // entries of bin B to take
  // the entries of bin B in index order: lanes before this one, then this
  // lane's earlier elements
  int cnt = 0;
  for (int base = 0; 4 * base < n; base += 64) {
    const float4 v = quad(base);
    const int s = 4 * (base + lane);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    bool in[4];
    int mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) { in[u] = s + u < n && bin_of(vv[u]) == B; mine += in[u]; }
    int before = 0, total = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned long long m = __ballot(in[u]);
      before += __popcll(m & below);
      total += __popcll(m);
    }
    int pos = cnt + before;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (in[u]) {
        if (pos < SEL_CB) { cidx[pos] = s + u; ckey[pos] = order_key(vv[u]); }
        ++pos;
      }
    }
    cnt += total;
  }
  if (cnt > SEL_CB) {
    wave_lds_sync();
    wave_radix_select(row, n, k, key_bits, hist, out);
    return;
  }
  wave_lds_sync();
  // rank of entry e among bin B: entries with a larger key, or an equal key
  // and a lower index (cidx is ascending, so the lower position)
  for (int e = lane; e < cnt; e += 64) {
    const uint32_t ke = ckey[e];
    int r = 0;
    for (int f = 0; f < cnt; ++f) {
      const uint32_t kf = ckey[f];
      r += (kf > ke || (kf == ke && f < e)) ? 1 : 0;
    }
    crank[e] = r;
  }
  wave_lds_sync();
  // ordered output: bins above B, and the entries of B ranked below rem
  int written = 0, seen = 0;
  for (int base = 0; 4 * base < n; base += 64) {
    const float4 v = quad(base);
    const int s = 4 * (base + lane);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    int bn[4];
    bool inb[4];
    int bbefore = 0, btotal = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bn[u] = s + u < n ? bin_of(vv[u]) : -1;
      inb[u] = bn[u] == B;
      const unsigned long long m = __ballot(inb[u]);
      bbefore += __popcll(m & below);
      btotal += __popcll(m);
    }
    int jb = seen + bbefore;
    bool take[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      take[u] = bn[u] > B;
      if (inb[u]) { take[u] = crank[jb] < rem; ++jb; }
    }
    int tbefore = 0, ttotal = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned long long m = __ballot(take[u]);
      tbefore += __popcll(m & below);
      ttotal += __popcll(m);
    }
    int pos = written + tbefore;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (take[u]) out[pos++] = s + u;
    written += ttotal;
    seen += btotal;
  }
}

template <bool KFP8>
__global__ void __launch_bounds__(256, 1) index_prefill_fused_kernel(IndexParams P) {
  __shared__ float srow[QG][FUSED_NMAX];
  __shared__ int hist[QG][SEL_BINS];
  __shared__ int cidx[QG][SEL_CB];
  __shared__ uint32_t ckey[QG][SEL_CB];
  __shared__ int crank[QG][SEL_CB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * QG;
  // visible entries of query t0 + q (0 past the end of the rows)
  auto nvis = [&](int q) -> int {
    if (t0 + q >= P.T) return 0;
    int64_t n = (P.pos0 + t0 + q + 1) / P.m;
    return static_cast<int>(n < P.cap ? n : P.cap);
  };
  int nmax = 0;
  for (int q = 0; q < QG; ++q) nmax = nvis(q) > nmax ? nvis(q) : nmax;
  // rows that keep every visible entry need no scores
  const bool need = nmax > P.k;
  const size_t row0 = static_cast<size_t>(b) * P.T + t0;

  if (need) {
    // A operands: rows r = 32*rb + (lane & 31) -> query 2rb + r/16, head r%16;
    // k-step ks covers dims (lane>>5)*32 + ks*8 .. +8 (same map for B)
    bf16x8 qa[2][4];
    float wv[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = lane & 31;
      const int q = 2 * rb + (r >> 4);
      const bool live = t0 + q < P.T;
      const bf16_t* qp = static_cast<const bf16_t*>(P.qI) + ((row0 + q) * HI + (r & 15)) * DI + (lane >> 5) * 32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        qa[rb][ks] = as_bf16x8(live ? *reinterpret_cast<const u32x4*>(qp + ks * 8) : z);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int qq = 2 * rb + (rr >> 4);
        wv[rb][v] = (t0 + qq < P.T) ? P.w[(row0 + qq) * HI + (rr & 15)] : 0.0f;
      }
    }
    const size_t seq = static_cast<size_t>(b) * P.cap;
    const int nblocks = (nmax + 31) / 32;
    // raw key rows of one 32-entry block (lane: entry lane%32, dims
    // (lane/32)*32 .. +32), clamped to the last visible entry: branch-free
    auto loadk = [&](int cb, u32x4 (&kr)[4], float& ksc) {
      const int s = min(cb * 32 + (lane & 31), nmax - 1);
      if (KFP8) {
        const uint8_t* kp = static_cast<const uint8_t*>(P.knope) + (seq + s) * DI + (lane >> 5) * 32;
        kr[0] = *reinterpret_cast<const u32x4*>(kp);
        kr[1] = *reinterpret_cast<const u32x4*>(kp + 16);
        ksc = static_cast<const float*>(P.kscale)[seq + s];
      } else {
        const bf16_t* kp = static_cast<const bf16_t*>(P.knope) + (seq + s) * DI + (lane >> 5) * 32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kr[ks] = *reinterpret_cast<const u32x4*>(kp + ks * 8);
        ksc = 1.0f;
      }
    };
    auto compute = [&](int cb, const u32x4 (&raw)[4], float ksc) {
      const int s = cb * 32 + (lane & 31);
      u32x4 kr[4];
      if (KFP8) {
        kr[0] = fp8x8_to_bf16(raw[0][0], raw[0][1]);
        kr[1] = fp8x8_to_bf16(raw[0][2], raw[0][3]);
        kr[2] = fp8x8_to_bf16(raw[1][0], raw[1][1]);
        kr[3] = fp8x8_to_bf16(raw[1][2], raw[1][3]);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kr[ks] = raw[ks];
      }
      f32x16 acc[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        acc[rb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][ks], as_bf16x8(kr[ks]), acc[rb], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float s0 = 0.0f, s1 = 0.0f;  // queries 2rb, 2rb+1 (8 heads of each in this lane)
#pragma unroll
        for (int v = 0; v < 8; ++v) s0 = fmaf(wv[rb][v], fmaxf(acc[rb][v] * ksc, 0.0f), s0);
#pragma unroll
        for (int v = 8; v < 16; ++v) s1 = fmaf(wv[rb][v], fmaxf(acc[rb][v] * ksc, 0.0f), s1);
        const float o0 = __shfl_xor(s0, 32), o1 = __shfl_xor(s1, 32);
        // lanes 0-31 hold head groups {0-3, 8-11}, lanes 32-63 {4-7, 12-15}:
        // add in a fixed order (lower half first)
        const float t0s = (lane < 32) ? s0 + o0 : o0 + s0;
        const float t1s = (lane < 32) ? s1 + o1 : o1 + s1;
        const int q = 2 * rb + (lane >> 5);
        float val = (lane < 32) ? t0s : t1s;
        if (P.score_dt == CSA_BF16) val = round_bf16(val);
        if (s < nvis(q)) srow[q][s] = val;
      }
    };
    // the next block's rows load while this block is multiplied (a block
    // past the end re-reads the last one; no load sits under a branch)
    u32x4 ka[4], kb[4];
    float sa, sb;
    int cb = w;
    if (cb < nblocks) {
      loadk(cb, ka, sa);
      while (true) {
        loadk(min(cb + 4, nblocks - 1), kb, sb);
        compute(cb, ka, sa);
        cb += 4;
        if (cb >= nblocks) break;
        loadk(min(cb + 4, nblocks - 1), ka, sa);
        compute(cb, kb, sb);
        cb += 4;
        if (cb >= nblocks) break;
      }
    }
  }
  __syncthreads();
  // one wave per query row
  const int q = w;
  if (t0 + q >= P.T) return;
  int32_t* out = P.idx + (row0 + q) * P.k;
  const int n = nvis(q);
  if (n <= P.k) {
    for (int j = lane; j < P.k; j += 64) out[j] = j < n ? j : -1;
    return;
  }
  wave_select(srow[q], n, P.k, P.score_dt == CSA_BF16 ? 16 : 32, hist[q], cidx[q], ckey[q], crank[q], out);
}

// ---------------------------------------------------------------------------
// streaming scan: one query row x 1024 entries per workgroup
// ---------------------------------------------------------------------------
constexpr int SCAN_CHUNK = 2048;

template <int KFMT, bool QMX>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KFMT == CSA_FP8E4M3 ? 3 : 4))) index_scan_kernel(IndexParams P) {
  // this chunk's top-11-bit key histogram (decode top-k), one per wave so
  // that no barrier separates the clearing from the counting
  __shared__ int lhist_w[4][HIST_BINS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.z, t = blockIdx.y;
  const int64_t pos = P.pos_dev ? P.pos_dev[b] : P.pos0 + t;
  int64_t n = pos < 0 ? 0 : (pos + 1) / P.m;
  if (n > P.cap) n = P.cap;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * SCAN_CHUNK;
  if (c0 >= n) return;
  const size_t row = static_cast<size_t>(b) * P.T + t;
  // A operand (16x16x32): head = lane & 15, g = lane >> 4.  BF16 / FP8 keys:
  // k-step ks covers dims g*16 + ks*8 .. +8.  MXFP4 keys: k-step ks is the
  // 32-dim scale block ks, dims ks*32 + g*8 .. +8, so that the block scale
  // multiplies that MFMA's result.
  const int g = lane >> 4, h = lane & 15;
  bf16x8 qa[2];
  {
    const bf16_t* qrow = static_cast<const bf16_t*>(P.qI) + (row * HI + h) * DI;
    u32x4 r[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      r[ks] = *reinterpret_cast<const u32x4*>(qrow + (KFMT == CSA_MXFP4 ? ks * 32 + g * 8 : g * 16 + ks * 8));
    if (QMX) {  // the query's own MXFP4 rounding, per 32-dim block
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf16_to_f32(static_cast<bf16_t>(r[ks][i] & 0xFFFFu));
          x[2 * i + 1] = bf16_to_f32(static_cast<bf16_t>(r[ks][i] >> 16));
        }
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
        am = fmaxf(am, __shfl_xor(am, 16));  // the block's other three groups
        am = fmaxf(am, __shfl_xor(am, 32));
        const int ex = mx_exponent(am);
        const float inv = exp2i(-ex), X = exp2i(ex);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = e2m1_to_f32(f32_to_e2m1(x[i] * inv)) * X;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[ks][i] = pack_bf16(x[2 * i], x[2 * i + 1]);
      }
    }
    qa[0] = as_bf16x8(r[0]);
    qa[1] = as_bf16x8(r[1]);
  }
  float wv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) wv[v] = P.w[row * HI + g * 4 + v];
  const size_t seq = static_cast<size_t>(b) * P.cap;
  const int cn = static_cast<int>(n - c0 < SCAN_CHUNK ? n - c0 : SCAN_CHUNK);  // entries of this chunk
  // wave-uniform bases of this chunk; per-lane offsets are 32-bit
  float* wsb = P.ws + row * P.n_stride + c0;
  float* sob = P.scores_out ? P.scores_out + row * P.cap + c0 : nullptr;
  const uint8_t* kb = static_cast<const uint8_t*>(P.knope) +
                      (seq + c0) * (KFMT == CSA_BF16 ? 2 * DI : KFMT == CSA_FP8E4M3 ? DI : DI / 2);
  const uint8_t* sb = static_cast<const uint8_t*>(P.kscale) + (seq + c0) * (KFMT == CSA_MXFP4 ? DI / 32 : 4);
  int* lhist = lhist_w[w];
  if (P.ghist)
    for (int i = lane; i < HIST_BINS; i += 64) lhist[i] = 0;
  // each wave: 16-entry column blocks w, w+4, ...  A batch of NB blocks is
  // loaded (clamped to the last entry, so branch-free) while the previous
  // batch is widened, multiplied and reduced over heads (two register sets,
  // used in turn).
  constexpr int NB = KFMT == CSA_BF16 ? 4 : 8;
  auto load = [&](int e0, u32x4 (&ra)[NB], u32x4 (&rb)[NB], uint32_t (&rs)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int s = min(e0 + 64 * j + (lane & 15), cn - 1);
      if constexpr (KFMT == CSA_BF16) {
        ra[j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * 2 * DI + g * 32));
        rb[j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * 2 * DI + g * 32 + 16));
      } else if constexpr (KFMT == CSA_FP8E4M3) {
        ra[j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * DI + g * 16));
        rs[j] = *reinterpret_cast<const uint32_t*>(sb + static_cast<uint32_t>(s * 4));
      } else {  // MXFP4: 8 codes of block 0 and of block 1 at dims ks*32 + g*8, both block scales
        ra[j][0] = *reinterpret_cast<const uint32_t*>(kb + static_cast<uint32_t>(s * (DI / 2) + g * 4));
        ra[j][1] = *reinterpret_cast<const uint32_t*>(kb + static_cast<uint32_t>(s * (DI / 2) + g * 4 + 16));
        rs[j] = *reinterpret_cast<const uint16_t*>(sb + static_cast<uint32_t>(s * (DI / 32)));
      }
    }
  };
  auto compute = [&](int e0, const u32x4 (&ra)[NB], const u32x4 (&rb)[NB], const uint32_t (&rs)[NB]) {
    f32x4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (KFMT == CSA_MXFP4) {  // dot = X0 * (block 0 codes . q) + X1 * (block 1 codes . q)
        const f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0], as_bf16x8(e2m1x8_to_bf16(ra[j][0])), f32x4{}, 0, 0, 0);
        const f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1], as_bf16x8(e2m1x8_to_bf16(ra[j][1])), f32x4{}, 0, 0, 0);
        const float X0 = exp2i(static_cast<int>(rs[j] & 0xFFu) - 127);
        const float X1 = exp2i(static_cast<int>(rs[j] >> 8) - 127);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[j][v] = fmaf(a1[v], X1, a0[v] * X0);
      } else {
        const u32x4 k0 = KFMT == CSA_FP8E4M3 ? fp8x8_to_bf16(ra[j][0], ra[j][1]) : ra[j];
        const u32x4 k1 = KFMT == CSA_FP8E4M3 ? fp8x8_to_bf16(ra[j][2], ra[j][3]) : rb[j];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0], as_bf16x8(k0), f32x4{}, 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1], as_bf16x8(k1), acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) {
      // lane (entry e = lane & 15, group g): partial score of block 4q + i
      // over heads 4g .. 4g+3 (the positive FP8 scale commutes with ReLU;
      // ReLU as an integer max: every negative float, -0 included, becomes +0)
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 c = acc[4 * q + i];
        float sc = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) sc = fmaf(wv[v], __int_as_float(max(__float_as_int(c[v]), 0)), sc);
        if constexpr (KFMT == CSA_FP8E4M3) sc *= __uint_as_float(rs[4 * q + i]);
        p[i] = sc;
      }
      // butterfly over the four groups: after it, group g holds the full
      // score of block 4q + g (groups g, g^2 first, then g, g^1)
      const bool hi = g >= 2, odd = g & 1;
      const float ka = hi ? p[2] : p[0], kb2 = hi ? p[3] : p[1];
      const float ra2 = __shfl_xor(hi ? p[0] : p[2], 32), rb2 = __shfl_xor(hi ? p[1] : p[3], 32);
      const float x = hi ? ra2 + ka : ka + ra2;    // block 2*hi: groups 0 + 2, 1 + 3
      const float y = hi ? rb2 + kb2 : kb2 + rb2;  // block 2*hi + 1
      const float r = __shfl_xor(odd ? x : y, 16);
      float tot = odd ? r + y : x + r;             // block 2*hi + odd = g: (g0 + g2) + (g1 + g3)
      if (P.score_dt == CSA_BF16) tot = round_bf16(tot);
      const int s = e0 + 64 * (4 * q + g) + (lane & 15);
      const bool ok = s < cn;
      if (ok) {
        wsb[s] = tot;
        if (sob) sob[s] = tot;
      }
      if (P.ghist) wave_hist_add(lhist, static_cast<int>(score_key(tot) >> (32 - HIST_BITS)), ok);
    }
  };
  u32x4 xa[NB], xb[NB], ya[NB], yb[NB];
  uint32_t xs[NB], ys[NB];
  // The loads are unconditional (a batch past the end re-reads the last
  // entry): a load under a branch would make the compiler wait for every
  // outstanding load before the next batch's arithmetic.
  int e0 = w * 16;
  load(e0, xa, xb, xs);
  while (e0 < cn) {
    load(e0 + 64 * NB, ya, yb, ys);
    compute(e0, xa, xb, xs);
    e0 += 64 * NB;
    if (e0 >= cn) break;
    load(e0 + 64 * NB, xa, xb, xs);
    compute(e0, ya, yb, ys);
    e0 += 64 * NB;
  }
  if (P.ghist) {
    __syncthreads();
    int* gh = P.ghist + static_cast<size_t>(b) * HIST_BINS;
    for (int i = tid; i < HIST_BINS; i += 256) {
      const int c = lhist_w[0][i] + lhist_w[1][i] + lhist_w[2][i] + lhist_w[3][i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

}  // namespace

bool index_mfma_supported(const IndexParams& P) {
  return P.H == HI && P.D == DI && P.q_dt == CSA_BF16 &&
         ((P.qk_dt == CSA_BF16 && (P.key_dt == CSA_BF16 || P.key_dt == CSA_FP8E4M3)) ||
          (P.qk_dt == CSA_MXFP4 && P.key_dt == CSA_MXFP4));
}

bool index_fused_prefill_ok(const IndexParams& P, int64_t n_max) {
  return index_mfma_supported(P) && P.qk_dt == CSA_BF16 && P.pos_dev == nullptr && n_max <= FUSED_NMAX;
}

int launch_index_fused_prefill(const IndexParams& P, int B, hipStream_t s) {
  dim3 grid((P.T + QG - 1) / QG, B);
  if (P.key_dt == CSA_FP8E4M3) hipLaunchKernelGGL(index_prefill_fused_kernel<true>, grid, dim3(256), 0, s, P);
  else hipLaunchKernelGGL(index_prefill_fused_kernel<false>, grid, dim3(256), 0, s, P);
  return check_launch("index_prefill_fused_kernel");
}

int launch_index_scan(const IndexParams& P, int B, int64_t n_max, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((n_max + SCAN_CHUNK - 1) / SCAN_CHUNK), P.T, B);
  if (P.qk_dt == CSA_MXFP4) hipLaunchKernelGGL((index_scan_kernel<CSA_MXFP4, true>), grid, dim3(256), 0, s, P);
  else if (P.key_dt == CSA_FP8E4M3) hipLaunchKernelGGL((index_scan_kernel<CSA_FP8E4M3, false>), grid, dim3(256), 0, s, P);
  else hipLaunchKernelGGL((index_scan_kernel<CSA_BF16, false>), grid, dim3(256), 0, s, P);
  return check_launch("index_scan_kernel");
}

}  // namespace csa
