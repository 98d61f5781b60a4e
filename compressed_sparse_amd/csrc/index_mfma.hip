// MFMA lightning indexer for 16 heads x 64 dims (BF16 or MXFP4 QK product;
// BF16, FP8-with-scale or MXFP4 keys).  [CSA/HCA 混注意力] §1.4 LIGHTNING
// INDEXER 的 FP4 计; [读完这篇] §三 CSA 步骤二.
//
//   I[s] = sum_h w[h] * ReLU(qI[h] . K[s])
//
// index_prefill_fused_kernel: 4 consecutive queries per workgroup, i.e. 64
//   MFMA rows (query x head) against 16-entry column blocks
//   (v_mfma_f32_16x16x32_bf16; keys read by coalesced loads and passed
//   through a per-wave LDS stage into the B operand's layout; MXFP4: 32-entry
//   blocks on the scaled FP4 MFMA).  The 4 score rows stay in LDS (4 x 8192
//   fp32) and two waves per row then select its top-k (binned threshold,
//   exact ranking inside the threshold bin), so scores never reach HBM.
// index_scan_kernel: one query row against a 1024-entry chunk per
//   workgroup (v_mfma_f32_16x16x32_bf16, rows = the 16 heads); the decode
//   scan and the fallback for long prefill rows, BF16 or FP8 keys.  FP8
//   codes widen to BF16 exactly in registers; the per-entry FP8 scale
//   multiplies the dot product.
// index_scan_mx_kernel: the same for MXFP4 keys and query, on the scaled
//   FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4): codes go in as they are
//   stored and the hardware applies both operands' E8M0 block scales.  The
//   query's MXFP4 operand is formed once per row by index_mx_prep_kernel.
//
// All kernels reduce heads in a fixed order (4 or 8 heads inside a lane,
// then fixed cross-lane shuffles), so scores are run-to-run deterministic.
#include "index.hpp"
#include "index_prep.hpp"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int HI = 16;
constexpr int DI = 64;
constexpr int QG = 4;          // queries per fused workgroup
constexpr int FUSED_NMAX = 8192;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Hardware widening of FP8 E4M3 codes to BF16 (the scaled conversion with
// scale 1: exact for every code); two words, first byte first.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI));
}

__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
               fp8x2_to_bf16x2<true>(w1)};
}

// Orders this wave's LDS accesses before the ones that follow.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Buffer descriptor of `bytes` bytes from `base` (wave-uniform; read back
// from lane 0 so that it is built in scalar registers); loads past the range
// return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t key_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  const int nb = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0), nb, 0x00020000);
}

// ReLU as an integer max: every negative float, -0 included, becomes +0
// (one instruction; the float max would first quiet NaNs)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// fused prefill: scores of 4 queries in LDS, then two waves per row select
// ---------------------------------------------------------------------------

constexpr int FW = 8;           // waves per fused workgroup (two per SIMD; two per row in the select)
constexpr int SEL_BINS = 2048;  // value-range bins of the fused select (16-bit counts, two per word)
constexpr int SEL_HW = SEL_BINS / 2;  // histogram words per row
constexpr int SEL_CBH = 128;    // threshold-bin entries ranked directly, per half row
constexpr int KD = 4;           // key blocks in flight per wave (scoring)
constexpr int HSTEPS = FUSED_NMAX / 512;  // 256-entry steps in half a row, at most

__device__ __forceinline__ int mbcnt(unsigned long long m) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

// Wave-level radix select of the top-k of row[0..n) (n > k) and ordered
// compaction of the selected indices into out[0..k).
__device__ __forceinline__ void wave_radix_select(const float* row, int n, int k, int key_bits, int* hist,
                                                  int32_t* out) {
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
    const int incl = wave_incl_scan(tot);
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
    bin = __builtin_amdgcn_readlane(bin, src);
    above = __builtin_amdgcn_readlane(above, src);
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

// index_prefill_fused_kernel: queries t0 .. t0+3 of sequence b.
//
// Scoring: 8 waves take 16-entry key blocks in turn (two waves per SIMD, so
// one multiplies while the other reduces), each for all 64 (query, head)
// rows; every lane ends with the weighted ReLU sum of one query and entry,
// and the row's extremes are kept on the way.
//
// Select, exact top-k of each row with n > k (ascending indices, ties to the
// lower index), by the row's two waves, one per half of its 256-entry
// steps.  Scores map monotonically onto t = (s - min) * (BINS-2) / (max -
// min) + 1, bin floor(t) in 1 .. BINS-1; the row's tail up to a whole step
// holds -inf (bin 0).  A shared histogram gives the bin B of the k-th
// largest score; entries with t >= B+1 are taken, those of bin B are ranked
// by (score descending, index ascending) and the best k - |above B| taken.
// Each half compacts its taken indices, in order, into the front of its own
// part of the row (a position never passes an entry still to be read), and
// the two runs are copied out back to back.  A row whose scores are all
// equal keeps its first k entries; a range too narrow for the bins, or a
// threshold bin of more than SEL_CBH entries in a half (heavy ties), takes
// the radix select.
// FROM_WS: no scoring; the 4 rows' scores come from the workspace rows a
// scan kernel wrote (rows the LDS does not hold, or scores requested), then
// the same select.
// MX: MXFP4 keys and query (operands formed by index_mx_prep_kernel): waves
// take 32-entry key blocks in turn; per block two scaled FP4 MFMAs, the A
// rows of the first carrying queries 0 and 1 (16 heads each), of the second
// queries 2 and 3, as in the two-query scan; after the ReLU-weighted head
// sums and one cross-half swap per MFMA, lanes 0..31 hold queries 0 and 2,
// lanes 32..63 queries 1 and 3.
template <bool KFP8, bool FROM_WS, bool MX = false>
__global__ void __launch_bounds__(64 * FW, 1) index_prefill_fused_kernel(IndexParams P) {
  __shared__ __align__(16) float srow[QG][FUSED_NMAX];
  // select state (histograms, bin-B candidates, ranks); while scoring, the
  // same bytes stage each wave's key block
  __shared__ __align__(16) int sel_mem[QG * SEL_HW + 3 * QG * 2 * SEL_CBH];
  static_assert(sizeof(sel_mem) >= FW * 2048, "key stage");
  int (*hist)[SEL_HW] = reinterpret_cast<int (*)[SEL_HW]>(sel_mem);
  int (*cidx)[2][SEL_CBH] = reinterpret_cast<int (*)[2][SEL_CBH]>(sel_mem + QG * SEL_HW);
  uint32_t (*ckey)[2][SEL_CBH] = reinterpret_cast<uint32_t (*)[2][SEL_CBH]>(sel_mem + QG * SEL_HW + QG * 2 * SEL_CBH);
  int (*crank)[2][SEL_CBH] = reinterpret_cast<int (*)[2][SEL_CBH]>(sel_mem + QG * SEL_HW + 2 * QG * 2 * SEL_CBH);
  __shared__ float s_mm[FW][QG][2];  // per wave and row: min, max of the scores it wrote
  __shared__ int s_cnt[QG][2][2];    // per row and half: bin-B entries, entries above B
  __shared__ int s_sink[FW][64];     // stores of lanes with nothing to store
  // the wave index is uniform: saying so keeps the loops below scalar
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  // longest rows first (a query's visible entries grow with t): the last
  // workgroups to start are the short ones, so the launch ends on a short tail
  const int t0 = (gridDim.x - 1 - blockIdx.x) * QG;
  // visible entries of query t0 + q (0 past the end of the rows): one 64-bit
  // division per workgroup, (pos0 + t0 + 1) = qb m + rb
  const int64_t base = P.pos0 + t0 + 1;
  const int64_t qb = base / P.m;
  const int rb0 = static_cast<int>(base - qb * P.m);
  auto nvis = [&](int q) -> int {
    if (t0 + q >= P.T) return 0;
    const int64_t n = qb + (rb0 + q) / P.m;
    return static_cast<int>(n < P.cap ? n : P.cap);
  };
  int nmax = 0;
  for (int q = 0; q < QG; ++q) nmax = nvis(q) > nmax ? nvis(q) : nmax;
  // rows that keep every visible entry need no scores
  const bool need = nmax > P.k;
  const size_t row0 = static_cast<size_t>(b) * P.T + t0;

  if (need) {
   if constexpr (FROM_WS) {
    // lane l of wave w reads entries 4(64w + l) + 2048i .. +3 of each row
    // (FUSED_NMAX/2048 16-byte loads per row, all issued before any is
    // used; the rows are n_stride >= n long, so a load past n stays in the
    // row and its values are dropped), keeping the wave's extremes
    constexpr int NL = FUSED_NMAX / (4 * 64 * FW);
    float4 v[QG][NL];
#pragma unroll
    for (int qq = 0; qq < QG; ++qq)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int e = 4 * (64 * w + lane) + 4 * 64 * FW * i;
        const int ec = min(e, static_cast<int>(P.n_stride) - 4);
        v[qq][i] = nvis(qq) > e ? *reinterpret_cast<const float4*>(P.ws + (row0 + qq) * P.n_stride + ec)
                                : float4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      const int nv = nvis(qq);
      float mnv = INFINITY, mxv = -INFINITY;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int e = 4 * (64 * w + lane) + 4 * 64 * FW * i;
        const float x[4] = {v[qq][i].x, v[qq][i].y, v[qq][i].z, v[qq][i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (e + c < nv) {
            srow[qq][e + c] = x[c];
            mnv = fminf(mnv, x[c]);
            mxv = fmaxf(mxv, x[c]);
          }
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        mnv = fminf(mnv, __shfl_xor(mnv, o));
        mxv = fmaxf(mxv, __shfl_xor(mxv, o));
      }
      if (lane == 0) {
        s_mm[w][qq][0] = mnv;
        s_mm[w][qq][1] = mxv;
      }
    }
   } else if constexpr (MX) {
    const int qsel = (lane >> 4) & 1, mine = lane >> 5;
    i32x8 qa[2];
    int qs[2];
    float wv[2][2][8];  // pair p, query 2p + i, head of accumulator v
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool lq = t0 + 2 * p + qsel < P.T;
      u32x4 qc = {0u, 0u, 0u, 0u};
      qs[p] = 127;
      if (lq) {
        const uint8_t* qp = P.qpack + (row0 + 2 * p + qsel) * QPACK_ROW_BYTES;
        const int ql = (lane & 15) + 32 * (lane >> 5);
        qc = reinterpret_cast<const u32x4*>(qp)[ql];
        qs[p] = reinterpret_cast<const int*>(qp + 64 * 16)[ql];
      }
      qa[p] = i32x8{static_cast<int>(qc[0]), static_cast<int>(qc[1]), static_cast<int>(qc[2]),
                    static_cast<int>(qc[3]), 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int h = (v & 4 ? 8 : 0) + 4 * (lane >> 5) + (v & 3);
          wv[p][i][v] = t0 + 2 * p + i < P.T ? P.w[(row0 + 2 * p + i) * HI + h] : 0.0f;
        }
    }
    // this lane's rows: queries mine (pair 0) and 2 + mine (pair 1)
    const int nvr[2] = {nvis(mine), nvis(2 + mine)};
    float mnr[2] = {INFINITY, INFINITY}, mxr[2] = {-INFINITY, -INFINITY};
    const size_t seq = static_cast<size_t>(b) * P.cap;
    const uint8_t* kb = static_cast<const uint8_t*>(P.knope) + seq * (DI / 2);
    const uint8_t* sb = static_cast<const uint8_t*>(P.kscale) + seq * (DI / 32);
    const int nb32 = (nmax + 31) / 32;
    // lane l loads entry 32 c + l % 32, half l / 32 (a block past the end
    // re-reads the last entry); MXD blocks in flight per wave
    constexpr int MXD = 8;
    auto loadk = [&](int c, u32x4& kc, uint32_t& ks) {
      const int e = min(32 * c + (lane & 31), nmax - 1);
      kc = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(e * (DI / 2) + 16 * (lane >> 5)));
      ks = sb[static_cast<uint32_t>(e * (DI / 32) + (lane >> 5))];
    };
    u32x4 kr[MXD];
    uint32_t kss[MXD];
#pragma unroll
    for (int i = 0; i < MXD; ++i) loadk(min(w + FW * i, nb32 - 1), kr[i], kss[i]);
    for (int cb = w; cb < nb32; cb += FW * MXD) {
#pragma unroll
      for (int i = 0; i < MXD; ++i) {
        const int c = cb + FW * i;
        const i32x8 kv = {static_cast<int>(kr[i][0]), static_cast<int>(kr[i][1]), static_cast<int>(kr[i][2]),
                          static_cast<int>(kr[i][3]), 0, 0, 0, 0};
        const int ksc = static_cast<int>(kss[i]);
        loadk(min(c + FW * MXD, nb32 - 1), kr[i], kss[i]);
        if (c < nb32) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            // formats 4, 4: E2M1 A and B; scale bytes in bits 0..7
            const f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[p], kv, f32x16{}, 4, 4, 0, qs[p], 0,
                                                                               ksc);
            float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              p0 = fmaf(wv[p][0][v], relu(acc[v]), p0);
              p1 = fmaf(wv[p][1][v], relu(acc[v + 8]), p1);
            }
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
            float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if (P.score_dt == CSA_BF16) tot = round_bf16(tot);
            const int e = 32 * c + (lane & 31);
            if (e < nvr[p]) {
              srow[2 * p + mine][e] = tot;
              mnr[p] = fminf(mnr[p], tot);
              mxr[p] = fmaxf(mxr[p], tot);
            }
          }
        }
      }
    }
    // per-row extremes of this wave's scores (the 32 lanes of each row)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        mnr[p] = fminf(mnr[p], __shfl_xor(mnr[p], o));
        mxr[p] = fmaxf(mxr[p], __shfl_xor(mxr[p], o));
      }
      if ((lane & 31) == 0) {
        s_mm[w][2 * p + mine][0] = mnr[p];
        s_mm[w][2 * p + mine][1] = mxr[p];
      }
    }
   } else {
    // 16x16x32 MFMAs over 16-entry key blocks.  Row r of head block j holds
    // query r/4, head 4j + r%4, so that lane l's four accumulators are the
    // 16 heads (head 4j + i in element i of block j) of query l/16 against
    // entry l%16.  K-step ks, lane group g = l/16 covers dims 32ks + 8g
    // (BF16 keys: one k-step reads 64 contiguous bytes of each of 16 rows)
    // or 16g + 8ks (FP8 keys: one 16-byte read covers both k-steps); the
    // query follows the same map.
    const int g = lane >> 4, e16 = lane & 15;
    bf16x8 qa[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qq = e16 >> 2, hh = 4 * j + (e16 & 3);
      const bool live = t0 + qq < P.T;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int d0 = KFP8 ? 16 * g + 8 * ks : 32 * ks + 8 * g;
        const bf16_t* qp = static_cast<const bf16_t*>(P.qI) + ((row0 + qq) * HI + hh) * DI + d0;
        const u32x4 z = {0u, 0u, 0u, 0u};
        qa[j][ks] = as_bf16x8(live ? *reinterpret_cast<const u32x4*>(qp) : z);
      }
    }
    float wv[16];  // weights of this lane's query g
#pragma unroll
    for (int v = 0; v < 16; ++v) wv[v] = (t0 + g < P.T) ? P.w[(row0 + g) * HI + v] : 0.0f;
    const int nv = nvis(g);
    float mnv = INFINITY, mxv = -INFINITY;
    const size_t seq = static_cast<size_t>(b) * P.cap;
    const int nblocks = (nmax + 15) / 16;
    // Key blocks arrive by coalesced reads (BF16: lane l reads 16 bytes of
    // row 8i + l/8 at chunk l%8, i = 0, 1; FP8: row l/4, chunk l%4), pass
    // through this wave's 2 KB LDS stage and are read back in the MFMA's
    // layout.  Stage chunk c of row r sits at chunk c ^ ((r/2)%8) (BF16,
    // 128-byte rows) or c ^ ((r/4)%4) (FP8, 64-byte rows): both the writes
    // and the reads of 16 lanes then cover distinct bank groups.
    uint8_t* stage = reinterpret_cast<uint8_t*>(sel_mem) + 2048 * w;
    // the sequence's first nmax key rows as a buffer (rows past them read as
    // zero; their scores are dropped): each load is a fixed lane offset plus
    // the block's start (nmax <= FUSED_NMAX rows, so 32-bit offsets)
    constexpr int KROW = KFP8 ? DI : 2 * DI;  // bytes per key row
    const __amdgpu_buffer_rsrc_t krs =
        key_rsrc(static_cast<const uint8_t*>(P.knope) + seq * KROW, static_cast<uint32_t>(nmax) * KROW);
    const __amdgpu_buffer_rsrc_t srs =
        key_rsrc(KFP8 ? static_cast<const float*>(P.kscale) + seq : nullptr, KFP8 ? static_cast<uint32_t>(nmax) * 4 : 0);
    // BF16: lane l reads row 8i + l/8, chunk l%8; FP8: row l/4, chunk l%4
    const uint32_t lo0 = KFP8 ? (lane >> 2) * DI + 16 * (lane & 3) : (lane >> 3) * KROW + 16 * (lane & 7);
    auto loadk = [&](int cb, u32x4 (&kr)[2], float& ksc) {
      const uint32_t b0 = static_cast<uint32_t>(cb) * 16 * KROW;
      kr[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, lo0 + b0, 0, 0));
      if (KFP8) {
        kr[1] = kr[0];
        ksc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, 4 * (cb * 16 + e16), 0, 0));
      } else {
        kr[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, lo0 + b0 + 8 * KROW, 0, 0));
        ksc = 1.0f;
      }
    };
    // block registers -> stage -> B operands (k-steps 0, 1)
    auto restage = [&](const u32x4 (&kr)[2], u32x4 (&kb)[2]) {
      wave_lds_sync();  // the previous block's reads are done
      if (KFP8) {
        const int r = lane >> 2;
        *reinterpret_cast<u32x4*>(stage + 64 * r + 16 * ((lane & 3) ^ ((r >> 2) & 3))) = kr[0];
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 8 * i + (lane >> 3);
          *reinterpret_cast<u32x4*>(stage + 128 * r + 16 * ((lane & 7) ^ ((r >> 1) & 7))) = kr[i];
        }
      }
      wave_lds_sync();
      if (KFP8) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(stage + 64 * e16 + 16 * (g ^ ((e16 >> 2) & 3)));
        kb[0] = fp8x8_to_bf16(raw[0], raw[1]);
        kb[1] = fp8x8_to_bf16(raw[2], raw[3]);
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          kb[ks] = *reinterpret_cast<const u32x4*>(stage + 128 * e16 + 16 * ((4 * ks + g) ^ ((e16 >> 1) & 7)));
      }
    };
    // the extremes are kept of the unrounded scores and rounded once at the
    // end (RNE is monotonic, so they are the BF16 scores' extremes); the
    // fp32 results of the sums need no canonicalising for fminf / fmaxf
    const bool rb = P.score_dt == CSA_BF16;
    auto compute = [&](int cb, const u32x4 (&kb)[2], float ksc) {
      f32x4 acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j][0], as_bf16x8(kb[0]), f32x4{}, 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j][1], as_bf16x8(kb[1]), acc[j], 0, 0, 0);
      }
      // heads 0..15 in order; the positive FP8 entry scale commutes with the
      // ReLU and multiplies the head sum (one product instead of sixteen)
      float val = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) val = fmaf(wv[4 * j + i], relu(acc[j][i]), val);
      if (KFP8) val *= ksc;
      const int s = cb * 16 + e16;
      if (s < nv) {
        srow[g][s] = rb ? round_bf16(val) : val;
        mnv = fminf(mnv, val);
        mxv = fmaxf(mxv, val);
      }
    };
    // KD blocks of keys in flight per wave: block c + FW KD loads into the
    // registers block c has just staged (a block past the end re-reads the
    // last one, so no load sits under a branch)
    {
      u32x4 kr[KD][2];
      float ks[KD];
      const int lastb = nblocks - 1;
      // issued in block order (the scheduler would otherwise reorder them, and
      // the loop's first wait would then have to drain them all)
#pragma unroll
      for (int i = 0; i < KD; ++i) {
        loadk(min(w + FW * i, lastb), kr[i], ks[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int cb = w; cb < nblocks; cb += FW * KD) {
#pragma unroll
        for (int i = 0; i < KD; ++i) {
          const int c = cb + FW * i;
          // every load and stage step is unconditional (past the last block
          // they repeat it), so the loads keep their issue order and each
          // block waits for its own loads only; the uniform branch holds no
          // memory load
          u32x4 kb[2];
          restage(kr[i], kb);
          const float ksc = ks[i];
          loadk(min(c + FW * KD, lastb), kr[i], ks[i]);
          if (c < nblocks) compute(c, kb, ksc);
        }
      }
      if (rb) {
        mnv = round_bf16(mnv);
        mxv = round_bf16(mxv);
      }
    }
    // per-row extremes of this wave's scores (the 16 lanes of query g)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      mnv = fminf(mnv, __shfl_xor(mnv, o));
      mxv = fmaxf(mxv, __shfl_xor(mxv, o));
    }
    if (e16 == 0) {
      s_mm[w][g][0] = mnv;
      s_mm[w][g][1] = mxv;
    }
   }
  }
  __syncthreads();

  // ---- select: row q, half hf; every wave passes the same barriers ----
  const int q = w & 3, hf = w >> 2;
  const bool live = t0 + q < P.T;
  const int k = P.k;
  const int n = live ? __builtin_amdgcn_readfirstlane(nvis(q)) : 0;
  int32_t* out = P.idx + (row0 + q) * k;
  float* row = srow[q];
  float mn = INFINITY, mx = -INFINITY;
  if (n > k) {
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      mn = fminf(mn, s_mm[j][q][0]);
      mx = fmaxf(mx, s_mm[j][q][1]);
    }
  }
  const float span = mx - mn;
  const float scale = static_cast<float>(SEL_BINS - 2) / span;
  // 0: no row, 1: every entry kept, 2: every score equal, 3: radix select,
  // 4: binned select
  int mode = !live ? 0 : n <= k ? 1 : !(span > 0.0f) ? 2 : !(scale < 3.0e38f) ? 3 : 4;
  const int nq = (n + 255) >> 8, nqh = (nq + 1) >> 1;
  const int c0 = hf * nqh, nc = min(nq, c0 + nqh) - c0;  // this half's steps: c0 .. c0 + nc
  const unsigned long long below = (1ull << lane) - 1ull;
  // this half's scores as t = (s - min) * (BINS-2) / (max - min) + 1, read
  // once; entries past n get -inf
  float4 tq[HSTEPS];
  if (mode == 4) {
    for (int i = lane + 64 * hf; i < SEL_HW; i += 128) hist[q][i] = 0;
#pragma unroll
    for (int i = 0; i < HSTEPS; ++i) {
      if (i < nc) {
        const float4 v = *reinterpret_cast<const float4*>(row + 4 * (64 * (c0 + i) + lane));
        tq[i] = float4{fmaf(v.x - mn, scale, 1.0f), fmaf(v.y - mn, scale, 1.0f), fmaf(v.z - mn, scale, 1.0f),
                       fmaf(v.w - mn, scale, 1.0f)};
        if (c0 + i == nq - 1) {
          const int s = 4 * (64 * (c0 + i) + lane);
          if (s >= n) tq[i].x = -INFINITY;
          if (s + 1 >= n) tq[i].y = -INFINITY;
          if (s + 2 >= n) tq[i].z = -INFINITY;
          if (s + 3 >= n) tq[i].w = -INFINITY;
        }
      }
    }
  }
  __syncthreads();
  auto binof = [](float t) {
    return static_cast<int>(__builtin_amdgcn_fmed3f(t, 0.0f, static_cast<float>(SEL_BINS - 1)));
  };
  if (mode == 4) {
#pragma unroll
    for (int i = 0; i < HSTEPS; ++i) {
      if (i < nc) {
        const float tt[4] = {tq[i].x, tq[i].y, tq[i].z, tq[i].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int bn = binof(tt[u]);  // bin 2w + h counts in bits 16h .. 16h+15 of word w
          atomicAdd(&hist[q][bn >> 1], 1 << (16 * (bn & 1)));
        }
      }
    }
  }
  __syncthreads();
  // the bin B of the k-th largest score (both waves of the row): lane l owns
  // bins BINS-1-PER*l .. BINS-PER-PER*l (descending; words HW-16(l+1) ..
  // HW-16l-1); the k largest scores lie in bins >= 1, so the search never
  // reaches bin 0
  int B = 1, rem = 0;
  if (mode == 4) {
    constexpr int PER = SEL_BINS / 64;
    int cnts[PER], tot = 0;
#pragma unroll
    for (int j = 0; j < PER / 2; j += 4) {
      const int4 h4 = *reinterpret_cast<const int4*>(&hist[q][SEL_HW - (PER / 2) * (lane + 1) + j]);
      const int hw[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // word (PER/2)(HW/(PER/2) - l - 1) + j + u: bins 2(..) (low), +1 (high)
        const int jj = PER - 2 * (j + u);  // descending position of the word's high bin, plus 2
        cnts[jj - 2] = static_cast<int>(static_cast<uint32_t>(hw[u]) >> 16);
        cnts[jj - 1] = hw[u] & 0xFFFF;
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) tot += cnts[j];
    const int incl = wave_incl_scan(tot);
    int bsel = -1, above = 0;
    if (incl - tot < k && incl >= k) {
      int cum = incl - tot;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (bsel < 0 && cum + cnts[j] >= k) { bsel = SEL_BINS - 1 - PER * lane - j; above = cum; }
        cum += cnts[j];
      }
    }
    const unsigned long long who = __ballot(bsel >= 0);
    const int src = __ffsll(static_cast<long long>(who)) - 1;
    B = __builtin_amdgcn_readlane(bsel, src);
    rem = k - __builtin_amdgcn_readlane(above, src);  // entries of bin B to take
  }
  // bin > B  <=>  t >= B+1;  bin == B  <=>  B <= t < B+1 (t stays below BINS)
  const float tb = static_cast<float>(B), tb1 = static_cast<float>(B + 1);
  // this half's entries of bin B, in index order; hasb marks the steps
  // that hold one (uniform)
  uint32_t hasb = 0;
  if (mode == 4) {
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < HSTEPS; ++i) {
      if (i < nc) {
        const float tt[4] = {tq[i].x, tq[i].y, tq[i].z, tq[i].w};
        bool in[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) in[u] = tt[u] >= tb && tt[u] < tb1;
        if (__ballot(in[0] || in[1] || in[2] || in[3])) {
          hasb |= 1u << i;
          const int s = 4 * (64 * (c0 + i) + lane);
          int pos = cnt, total = 0;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const unsigned long long m = __ballot(in[u]);
            pos += mbcnt(m);
            total += __popcll(m);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (in[u]) {
              if (pos < SEL_CBH) { cidx[q][hf][pos] = s + u; ckey[q][hf][pos] = order_key(row[s + u]); }
              ++pos;
            }
          }
          cnt += total;
        }
      }
    }
    if (lane == 0) s_cnt[q][hf][0] = cnt;
  }
  __syncthreads();
  const int cnt0 = s_cnt[q][0][0], cnt1 = s_cnt[q][1][0];
  if (mode == 4 && (cnt0 > SEL_CBH || cnt1 > SEL_CBH)) mode = 3;
  // rank of each bin-B entry among both halves' (half 0 first: index order):
  // entries with a larger key, or an equal key and a lower index.  The
  // candidates' keys sit in lanes (two per lane and half) and are read back
  // one by one with readlane.
  if (mode == 4) {
    uint32_t kk[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ch = hh ? cnt1 : cnt0;
      kk[hh][0] = lane < ch ? ckey[q][hh][lane] : 0u;
      kk[hh][1] = lane + 64 < ch ? ckey[q][hh][lane + 64] : 0u;
    }
    const int cnth = hf ? cnt1 : cnt0, g0 = hf ? cnt0 : 0;
    const uint32_t ke0 = hf ? kk[1][0] : kk[0][0], ke1 = hf ? kk[1][1] : kk[0][1];
    const int ge0 = g0 + lane, ge1 = g0 + lane + 64;
    int r0 = 0, r1 = 0;
    for (int f = 0; f < cnt0 + cnt1; ++f) {
      const int hh = f < cnt0 ? 0 : 1, e = hh ? f - cnt0 : f;
      const uint32_t kf = __builtin_amdgcn_readlane(e < 64 ? kk[hh][0] : kk[hh][1], e & 63);
      r0 += (kf > ke0 || (kf == ke0 && f < ge0)) ? 1 : 0;
      r1 += (kf > ke1 || (kf == ke1 && f < ge1)) ? 1 : 0;
    }
    if (lane < cnth) crank[q][hf][lane] = r0;
    if (lane + 64 < cnth) crank[q][hf][lane + 64] = r1;
  }
  __syncthreads();
  // ordered output of each half: entries above B and the chosen entries of
  // bin B, compacted (every score is in registers by now) into the row:
  // half 0 from element 0, half 1 from element FUSED_NMAX/2 (k is at most
  // 2048); positions from a prefix sum of each lane's take count
  if (mode == 4) {
    int* outl = reinterpret_cast<int*>(row) + (hf ? FUSED_NMAX / 2 : 0);
    int* sink = &s_sink[w][lane];
    int written = 0, seen = 0;
#pragma unroll
    for (int i = 0; i < HSTEPS; ++i) {
      if (i < nc) {
        const int s = 4 * (64 * (c0 + i) + lane);
        const float tt[4] = {tq[i].x, tq[i].y, tq[i].z, tq[i].w};
        bool take[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) take[u] = tt[u] >= tb1;
        if (hasb & (1u << i)) {
          bool inb[4];
          int jb = seen, btotal = 0;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            inb[u] = tt[u] >= tb && !take[u];
            const unsigned long long m = __ballot(inb[u]);
            jb += mbcnt(m);
            btotal += __popcll(m);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (inb[u]) { take[u] = crank[q][hf][jb] < rem; ++jb; }
          seen += btotal;
        }
        const int tk = (take[0] ? 1 : 0) + (take[1] ? 1 : 0) + (take[2] ? 1 : 0) + (take[3] ? 1 : 0);
        const int incl = wave_incl_scan(tk);
        int pos = written + incl - tk;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          *(take[u] ? outl + pos : sink) = s + u;
          pos += take[u] ? 1 : 0;
        }
        written += __builtin_amdgcn_readlane(incl, 63);
      }
    }
    if (hf == 0 && lane == 0) s_cnt[q][0][1] = written;
  }
  __syncthreads();
  if (mode == 4) {
    const int* o = reinterpret_cast<const int*>(row);
    const int base1 = s_cnt[q][0][1];  // half 0's run
    for (int j = lane + 64 * hf; j < k; j += 128) out[j] = j < base1 ? o[j] : o[FUSED_NMAX / 2 + j - base1];
  } else if (mode == 3) {
    if (hf == 0) wave_radix_select(row, n, k, P.score_dt == CSA_BF16 ? 16 : 32, hist[q], out);
  } else if (mode == 2) {
    for (int j = lane + 64 * hf; j < k; j += 128) out[j] = j;
  } else if (mode == 1) {
    for (int j = lane + 64 * hf; j < k; j += 128) out[j] = j < n ? j : -1;
  }
}

// ---------------------------------------------------------------------------
// streaming scan: one query row x 1024 entries per workgroup
// ---------------------------------------------------------------------------
constexpr int SCAN_CHUNK = 1024;

// Clears a wave's LDS histogram (four bins per store).
__device__ __forceinline__ void clear_hist(int* hist, int lane) {
#pragma unroll
  for (int i = 0; i < HIST_BINS / 256; ++i) reinterpret_cast<u32x4*>(hist)[lane + 64 * i] = u32x4{0u, 0u, 0u, 0u};
}

// Adds a workgroup's four wave histograms to the row's global histogram.
__device__ __forceinline__ void flush_hist(const int (*lhist_w)[HIST_BINS], int* gh, int tid) {
  for (int i = tid; i < HIST_BINS; i += 256) {
    const int c = lhist_w[0][i] + lhist_w[1][i] + lhist_w[2][i] + lhist_w[3][i];
    if (c) atomicAdd(&gh[i], c);
  }
}

template <int KFMT, bool PAGED>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KFMT == CSA_FP8E4M3 ? 3 : 4))) index_scan_kernel(IndexParams P) {
  // this chunk's top-11-bit key histogram (decode top-k), one per wave so
  // that no barrier separates the clearing from the counting
  __shared__ int lhist_w[4][HIST_BINS];
  // the wave index as a scalar where paged key blocks need it for their table loads
  const int tid = threadIdx.x, lane = tid & 63, w = PAGED ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int b = blockIdx.z, t = blockIdx.y;
  const int64_t pos = P.pos_dev ? P.pos_dev[b] : P.pos0 + t;
  int64_t n = pos < 0 ? 0 : (pos + 1) / P.m;
  if (n > P.cap) n = P.cap;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * SCAN_CHUNK;
  if (c0 >= n) return;
  const size_t row = static_cast<size_t>(b) * P.T + t;
  const int cn = static_cast<int>(n - c0 < SCAN_CHUNK ? n - c0 : SCAN_CHUNK);  // entries of this chunk
  int page_of_block = 0;  // paged: lane l holds the page of the wave's block l
  if constexpr (PAGED) {
    const int64_t blk = min(16 * w + 64 * lane, (cn - 1) & ~15);
    const int64_t pg = P.pg.table[static_cast<int64_t>(b) * P.pg.tps + ((c0 + blk) >> P.pg.shift)];
    page_of_block = pg >= 0 && pg < P.pg.pool ? static_cast<int>(pg) : 0;  // outside the pool: page 0
  }
  // A operand (16x16x32): head = lane & 15, g = lane >> 4; k-step ks covers
  // dims g*16 + ks*8 .. +8
  const int g = lane >> 4, h = lane & 15;
  bf16x8 qa[2];
  {
    const bf16_t* qrow = static_cast<const bf16_t*>(P.qI) + (row * HI + h) * DI;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qa[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + g * 16 + ks * 8));
  }
  float wv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) wv[v] = P.w[row * HI + g * 4 + v];
  // wave-uniform bases of this chunk (of each key block); per-lane offsets are 32-bit
  float* wsb = P.ws + row * P.n_stride + c0;
  float* sob = P.scores_out ? P.scores_out + row * P.cap + c0 : nullptr;
  constexpr int KROW = KFMT == CSA_BF16 ? 2 * DI : DI;  // bytes per key row
  const uint8_t* knope = static_cast<const uint8_t*>(P.knope);
  const uint8_t* kscale = static_cast<const uint8_t*>(P.kscale);
  // contiguous keys: the chunk's rows from one base
  const size_t seq = static_cast<size_t>(b) * P.cap;
  const uint8_t* kbc = knope + (seq + c0) * KROW;
  const uint8_t* sbc = kscale + (seq + c0) * 4;
  int* lhist = lhist_w[w];
  if (P.ghist) clear_hist(lhist, lane);
  // each wave: 16-entry column blocks w, w+4, ...  A batch of NB blocks is
  // loaded (clamped to the last entry, so branch-free) while the previous
  // batch is widened, multiplied and reduced over heads (two register sets,
  // used in turn).
  constexpr int NB = 4;
  // Block j of a batch: the 16 entries from e0 + 64 j (entries past the
  // chunk's end re-read its last entry; those scores are dropped).  Paged:
  // the block's rows from its page (a block never crosses one; a block past
  // the end re-reads the chunk's last block).
  // Paged: the wave's blocks are 16w + 64 l (l = 0, 1, ..; past the chunk's
  // end its last block); lane l fetched block l's page once, at the start,
  // and a block takes it with a lane read, so no key load waits on the table.
  auto load = [&](int e0, u32x4 (&ra)[NB], u32x4 (&rb)[NB], uint32_t (&rs)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint8_t* kb = kbc;
      const uint8_t* sb = sbc;
      int s;
      if constexpr (PAGED) {
        const int blk = min(e0 + 64 * j, (cn - 1) & ~15);
        const int64_t pg = __builtin_amdgcn_readlane(page_of_block, (e0 - 16 * w) / 64 + j);
        const int64_t r0 = (pg << P.pg.shift) | ((c0 + blk) & ((int64_t(1) << P.pg.shift) - 1));
        kb = knope + r0 * KROW;
        sb = kscale + r0 * 4;
        s = min(blk + (lane & 15), cn - 1) - blk;
      } else {
        s = min(e0 + 64 * j + (lane & 15), cn - 1);
      }
      if constexpr (KFMT == CSA_BF16) {
        ra[j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * 2 * DI + g * 32));
        rb[j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * 2 * DI + g * 32 + 16));
      } else {
        ra[j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * DI + g * 16));
        rs[j] = *reinterpret_cast<const uint32_t*>(sb + static_cast<uint32_t>(s * 4));
      }
    }
  };
  auto compute = [&](int e0, const u32x4 (&ra)[NB], const u32x4 (&rb)[NB], const uint32_t (&rs)[NB]) {
    f32x4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const u32x4 k0 = KFMT == CSA_FP8E4M3 ? fp8x8_to_bf16(ra[j][0], ra[j][1]) : ra[j];
      const u32x4 k1 = KFMT == CSA_FP8E4M3 ? fp8x8_to_bf16(ra[j][2], ra[j][3]) : rb[j];
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0], as_bf16x8(k0), f32x4{}, 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1], as_bf16x8(k1), acc[j], 0, 0, 0);
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
    flush_hist(lhist_w, P.ghist + static_cast<size_t>(b) * HIST_BINS, tid);
  }
}

// ---------------------------------------------------------------------------
// MXFP4 keys and query
// ---------------------------------------------------------------------------

// One wave per query row (decode: one row per workgroup, whose other waves
// clear the row's histogram).  The wave rounds the row's query to MXFP4 (per
// head and 32-dim block: the OCP MX shared exponent e of the block's largest
// magnitude, E2M1 codes of q / 2^e) and stores it as the A operand of the
// scaled 32x32x64 MFMA: lane l holds head l % 32 (heads 16.. are zero) and
// dims 32 (l / 32) .. +32, 16 bytes of codes (low nibble first), and the
// E8M0 byte e + 127.  Decode: the row's histogram and candidate count are
// cleared too.
__global__ void __launch_bounds__(256) index_mx_prep_kernel(IndexParams P, int rows) {
  // decode: one row per workgroup (its waves then clear the histogram);
  // prefill: one row per wave
  const int tid = threadIdx.x;
  const size_t r = P.ghist ? blockIdx.x : static_cast<size_t>(blockIdx.x) * 4 + (tid >> 6);
  if ((P.ghist ? tid < 64 : true) && r < static_cast<size_t>(rows)) mx_prep_row(P, r);
  if (P.ghist) clear_decode_row(P, r);  // decode: one row per sequence
}

// Per 32-entry block one scaled MFMA: 32 (16 real) heads x 32 entries x 64
// dims, E2M1 codes of both operands with both E8M0 block scales applied in
// the MFMA (exact products, fp32 sum).  Accumulator lane l holds entry l % 32
// and heads 4 (l / 32) + v, 8 + 4 (l / 32) + v (v < 4); its ReLU-weighted
// partial sum and that of lane l ^ 32 make the score, combined for two blocks
// at once by one cross-half lane swap (lanes 0..31: block A, 32..63: block
// B).  Wave w takes the 64-entry block pairs w, w + 4, ..; all its key loads
// are issued before the first MFMA.
constexpr int MX_PAIRS = SCAN_CHUNK / 256;  // block pairs per wave

template <bool PAGED>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) index_scan_mx_kernel(IndexParams P) {
  __shared__ int lhist_w[4][HIST_BINS];
  // the wave index as a scalar where paged key blocks need it for their table loads
  const int tid = threadIdx.x, lane = tid & 63, w = PAGED ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int b = blockIdx.z, t = blockIdx.y;
  const int64_t pos = P.pos_dev ? P.pos_dev[b] : P.pos0 + t;
  int64_t n = pos < 0 ? 0 : (pos + 1) / P.m;
  if (n > P.cap) n = P.cap;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * SCAN_CHUNK;
  if (c0 >= n) return;
  const size_t row = static_cast<size_t>(b) * P.T + t;
  const int cn = static_cast<int>(n - c0 < SCAN_CHUNK ? n - c0 : SCAN_CHUNK);
  // every key load first (entries past the chunk's end re-read its last
  // entry, branch-free; those scores are dropped).  Paged: each 64-entry
  // block pair from its page (a pair never crosses one; a pair past the end
  // re-reads the chunk's last pair).
  const size_t seq = static_cast<size_t>(b) * P.cap;
  const uint8_t* kbc = static_cast<const uint8_t*>(P.knope) + (seq + c0) * (DI / 2);
  const uint8_t* sbc = static_cast<const uint8_t*>(P.kscale) + (seq + c0) * (DI / 32);
  u32x4 kc[MX_PAIRS][2];
  uint32_t ks[MX_PAIRS][2];
#pragma unroll
  for (int p = 0; p < MX_PAIRS; ++p) {
    int blk = 64 * (w + 4 * p), s0 = 0;  // entry s of the chunk at kb + (s - s0) rows
    const uint8_t* kb = kbc;
    const uint8_t* sb = sbc;
    if constexpr (PAGED) {
      blk = min(blk, (cn - 1) & ~63);
      const int64_t r0 = key_block_row(P, b, c0 + blk);
      kb = static_cast<const uint8_t*>(P.knope) + r0 * (DI / 2);
      sb = static_cast<const uint8_t*>(P.kscale) + r0 * (DI / 32);
      s0 = blk;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int s = min(blk + 32 * j + (lane & 31), cn - 1) - s0;
      kc[p][j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * (DI / 2) + 16 * (lane >> 5)));
      ks[p][j] = sb[static_cast<uint32_t>(s * (DI / 32) + (lane >> 5))];
    }
  }
  const uint8_t* qp = P.qpack + row * QPACK_ROW_BYTES;
  const u32x4 qc = reinterpret_cast<const u32x4*>(qp)[lane];
  const int qs = reinterpret_cast<const int*>(qp + 64 * 16)[lane];
  const i32x8 qa = {static_cast<int>(qc[0]), static_cast<int>(qc[1]), static_cast<int>(qc[2]), static_cast<int>(qc[3]),
                    0, 0, 0, 0};
  float wv[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) wv[v] = P.w[row * HI + (v & 4 ? 8 : 0) + 4 * (lane >> 5) + (v & 3)];
  float* wsb = P.ws + row * P.n_stride + c0;
  float* sob = P.scores_out ? P.scores_out + row * P.cap + c0 : nullptr;
  int* lhist = lhist_w[w];
  if (P.ghist) clear_hist(lhist, lane);
#pragma unroll
  for (int p = 0; p < MX_PAIRS; ++p) {
    float part[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const i32x8 kv = {static_cast<int>(kc[p][j][0]), static_cast<int>(kc[p][j][1]), static_cast<int>(kc[p][j][2]),
                        static_cast<int>(kc[p][j][3]), 0, 0, 0, 0};
      // formats 4, 4: E2M1 A and B; scale bytes in bits 0..7 of qs and ks
      const f32x16 acc =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kv, f32x16{}, 4, 4, 0, qs, 0, static_cast<int>(ks[p][j]));
      float sc = 0.0f;
#pragma unroll
      for (int v = 0; v < 8; ++v) sc = fmaf(wv[v], relu(acc[v]), sc);
      part[j] = sc;
    }
    // lanes 0..31: part A of lanes l and l + 32; lanes 32..63: part B of l - 32 and l
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
    float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (P.score_dt == CSA_BF16) tot = round_bf16(tot);
    const int s = 64 * (w + 4 * p) + lane;
    const bool ok = s < cn;
    if (ok) {
      wsb[s] = tot;
      if (sob) sob[s] = tot;
    }
    if (P.ghist) wave_hist_add(lhist, static_cast<int>(score_key(tot) >> (32 - HIST_BITS)), ok);
  }
  if (P.ghist) {
    __syncthreads();
    flush_hist(lhist_w, P.ghist + static_cast<size_t>(b) * HIST_BINS, tid);
  }
}

// Prefill form: the A operand's rows 16..31 carry the next query's heads,
// so one scaled MFMA scores 32 entries against two consecutive queries
// (t0, t0 + 1).  Lane l's accumulators 0..7 are query t0's partial sums,
// 8..15 query t0 + 1's (same heads); one cross-half swap leaves lanes
// 0..31 with query t0's scores of the block's entries and lanes 32..63 with
// query t0 + 1's.  Wave w takes the blocks w, w + 4, .. of the chunk.
constexpr int MX2_BLOCKS = SCAN_CHUNK / 128;  // 32-entry blocks per wave

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) index_scan_mx2_kernel(IndexParams P) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.z, t0 = 2 * blockIdx.y;
  const bool two = t0 + 1 < P.T;
  auto vis = [&](int t) -> int64_t {
    const int64_t pos = P.pos0 + t;
    const int64_t n = pos < 0 ? 0 : (pos + 1) / P.m;
    return n < P.cap ? n : P.cap;
  };
  const int64_t n0 = vis(t0), n1 = two ? vis(t0 + 1) : n0;  // n1 >= n0
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * SCAN_CHUNK;
  if (c0 >= n1) return;
  const size_t row0 = static_cast<size_t>(b) * P.T + t0;
  const int cn = static_cast<int>(n1 - c0 < SCAN_CHUNK ? n1 - c0 : SCAN_CHUNK);
  const int cn0 = static_cast<int>(n0 - c0 < 0 ? 0 : (n0 - c0 < SCAN_CHUNK ? n0 - c0 : SCAN_CHUNK));
  const size_t seq = static_cast<size_t>(b) * P.cap;
  const uint8_t* kb = static_cast<const uint8_t*>(P.knope) + (seq + c0) * (DI / 2);
  const uint8_t* sb = static_cast<const uint8_t*>(P.kscale) + (seq + c0) * (DI / 32);
  u32x4 kc[MX2_BLOCKS];
  uint32_t ks[MX2_BLOCKS];
#pragma unroll
  for (int j = 0; j < MX2_BLOCKS; ++j) {
    const int s = min(32 * (w + 4 * j) + (lane & 31), cn - 1);
    kc[j] = *reinterpret_cast<const u32x4*>(kb + static_cast<uint32_t>(s * (DI / 2) + 16 * (lane >> 5)));
    ks[j] = sb[static_cast<uint32_t>(s * (DI / 32) + (lane >> 5))];
  }
  // A operand: row l % 32 = (query (l % 32) / 16, head l % 16), block l / 32
  const int qsel = (lane >> 4) & 1;
  u32x4 qc = {0u, 0u, 0u, 0u};
  int qs = 127;
  if (!qsel || two) {
    const uint8_t* qp = P.qpack + (row0 + qsel) * QPACK_ROW_BYTES;
    const int ql = (lane & 15) + 32 * (lane >> 5);
    qc = reinterpret_cast<const u32x4*>(qp)[ql];
    qs = reinterpret_cast<const int*>(qp + 64 * 16)[ql];
  }
  const i32x8 qa = {static_cast<int>(qc[0]), static_cast<int>(qc[1]), static_cast<int>(qc[2]), static_cast<int>(qc[3]),
                    0, 0, 0, 0};
  float wv0[8], wv1[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int h = (v & 4 ? 8 : 0) + 4 * (lane >> 5) + (v & 3);
    wv0[v] = P.w[row0 * HI + h];
    wv1[v] = two ? P.w[(row0 + 1) * HI + h] : 0.0f;
  }
  const int mine = lane >> 5;  // 0: query t0, 1: query t0 + 1
  float* wsb = P.ws + (row0 + mine) * P.n_stride + c0;
  float* sob = P.scores_out ? P.scores_out + (row0 + mine) * P.cap + c0 : nullptr;
  const int lim = mine ? (two ? cn : 0) : cn0;
#pragma unroll
  for (int j = 0; j < MX2_BLOCKS; ++j) {
    const i32x8 kv = {static_cast<int>(kc[j][0]), static_cast<int>(kc[j][1]), static_cast<int>(kc[j][2]),
                      static_cast<int>(kc[j][3]), 0, 0, 0, 0};
    const f32x16 acc =
        __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kv, f32x16{}, 4, 4, 0, qs, 0, static_cast<int>(ks[j]));
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      p0 = fmaf(wv0[v], relu(acc[v]), p0);
      p1 = fmaf(wv1[v], relu(acc[v + 8]), p1);
    }
    // lanes 0..31: query t0, heads of lanes l and l + 32; lanes 32..63: query t0 + 1
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (P.score_dt == CSA_BF16) tot = round_bf16(tot);
    const int s = 32 * (w + 4 * j) + (lane & 31);
    if (s < lim) {
      wsb[s] = tot;
      if (sob) sob[s] = tot;
    }
  }
}

}  // namespace

bool index_mfma_supported(const IndexParams& P) {
  return P.H == HI && P.D == DI && P.q_dt == CSA_BF16 &&
         ((P.qk_dt == CSA_BF16 && (P.key_dt == CSA_BF16 || P.key_dt == CSA_FP8E4M3)) ||
          (P.qk_dt == CSA_MXFP4 && P.key_dt == CSA_MXFP4));
}

bool index_scan_mx(const IndexParams& P) {
  return index_mfma_supported(P) && P.qk_dt == CSA_MXFP4;
}

int launch_index_mx_prep(const IndexParams& P, int rows, hipStream_t s) {
  hipLaunchKernelGGL(index_mx_prep_kernel, dim3(P.ghist ? rows : (rows + 3) / 4), dim3(256), 0, s, P, rows);
  return check_launch("index_mx_prep_kernel");
}

bool index_fused_prefill_ok(const IndexParams& P, int64_t n_max) {
  return index_mfma_supported(P) && P.pos_dev == nullptr && P.pg.table == nullptr && n_max <= FUSED_NMAX;
}

// MXFP4: the query operands are formed first (index_mx_prep_kernel)
int launch_index_fused_prefill(const IndexParams& P, int B, hipStream_t s) {
  dim3 grid((P.T + QG - 1) / QG, B);
  if (P.qk_dt == CSA_MXFP4) {
    const int st = launch_index_mx_prep(P, B * P.T, s);
    if (st != CSA_OK) return st;
    hipLaunchKernelGGL((index_prefill_fused_kernel<false, false, true>), grid, dim3(64 * FW), 0, s, P);
  } else if (P.key_dt == CSA_FP8E4M3) {
    hipLaunchKernelGGL((index_prefill_fused_kernel<true, false>), grid, dim3(64 * FW), 0, s, P);
  } else {
    hipLaunchKernelGGL((index_prefill_fused_kernel<false, false>), grid, dim3(64 * FW), 0, s, P);
  }
  return check_launch("index_prefill_fused_kernel");
}

bool index_ws_select_ok(const IndexParams& P, int64_t n_max) {
  return index_mfma_supported(P) && P.pos_dev == nullptr && n_max <= FUSED_NMAX;
}

int launch_index_ws_select(const IndexParams& P, int B, hipStream_t s) {
  dim3 grid((P.T + QG - 1) / QG, B);
  hipLaunchKernelGGL((index_prefill_fused_kernel<false, true>), grid, dim3(64 * FW), 0, s, P);
  return check_launch("index_prefill_fused_kernel (select)");
}

int launch_index_scan(const IndexParams& P, int B, int64_t n_max, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((n_max + SCAN_CHUNK - 1) / SCAN_CHUNK), P.T, B);
  if (P.qk_dt == CSA_MXFP4 && !P.ghist && !P.pos_dev) {  // prefill: two queries per workgroup
    hipLaunchKernelGGL(index_scan_mx2_kernel, dim3(grid.x, (P.T + 1) / 2, B), dim3(256), 0, s, P);
    return check_launch("index_scan_mx2_kernel");
  }
  const bool paged = P.pg.table != nullptr;
  if (P.qk_dt == CSA_MXFP4) {
    if (paged) hipLaunchKernelGGL(index_scan_mx_kernel<true>, grid, dim3(256), 0, s, P);
    else hipLaunchKernelGGL(index_scan_mx_kernel<false>, grid, dim3(256), 0, s, P);
  } else if (P.key_dt == CSA_FP8E4M3) {
    if (paged) hipLaunchKernelGGL((index_scan_kernel<CSA_FP8E4M3, true>), grid, dim3(256), 0, s, P);
    else hipLaunchKernelGGL((index_scan_kernel<CSA_FP8E4M3, false>), grid, dim3(256), 0, s, P);
  } else {
    if (paged) hipLaunchKernelGGL((index_scan_kernel<CSA_BF16, true>), grid, dim3(256), 0, s, P);
    else hipLaunchKernelGGL((index_scan_kernel<CSA_BF16, false>), grid, dim3(256), 0, s, P);
  }
  return check_launch("index_scan_kernel");
}

}  // namespace csa
