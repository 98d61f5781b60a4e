// MFMA attention for the MI355X-shaped cases: 64 query heads sharing one
// compressed entry of 512 non-RoPE + 64 RoPE dims (MQA), BF16 queries and
// outputs, BF16 or FP8-with-scale cache.  [CSA/HCA 混注意力] §1.1, §1.2;
// [读完这篇] §三 CSA 步骤三 (standard attention over the selected entries, KV
// shared across heads); §1.4 存储格式混 (FP8 non-RoPE dims, BF16 RoPE dims).
//
// One workgroup (4 waves) owns one query (all 64 heads) and a range of its
// entry list.  The query's 64 heads sit in LDS (RoPE applied once); entries
// are gathered 64 at a time into an LDS tile (rows padded to 1168 B so the
// 32 rows an MFMA operand touches fall on distinct bank groups), the next
// tile's rows riding in registers while the current one is multiplied.  FP8
// codes widen to BF16 exactly on the way in; the per-entry scale multiplies
// the non-RoPE part of the logit and is folded into P for the values.
//
// Wave w owns heads 32*(w/2).. and, for the logits, entries 32*(w%2).. of a
// tile; for P.V it owns value dims 256*(w%2)...  Both products run
// transposed so that one lane holds one head:
//
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = entry rows, B = head rows
//   softmax          per lane: max / sum over its 16 entries, one cross-lane
//                    step, one LDS exchange with the partner wave
//   O^T += V^T P^T   A = V read column-wise from the K tile with
//                    ds_read_b64_tr_b16, B = P^T rows through LDS
//
// LDS operand reads are software-pipelined one group of MFMAs ahead.
// Decode splits the entry list over several workgroups per sequence; each
// writes an unnormalised partial (O, max, sum) and attn_merge_kernel
// combines them by log-sum-exp.
#include <cmath>
#include <utility>

#include "attention.hpp"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int NH = 64;       // heads
constexpr int DN = 512;      // value / non-RoPE dims
constexpr int DRP = 64;      // RoPE dims
constexpr int CW = DN + DRP; // entry width
constexpr int TILE = 64;     // entries per LDS tile
constexpr int KROW = CW + 8; // padded LDS row (bf16 elements), 1168 B
constexpr int PROW = TILE + 8;  // padded P row, 144 B
constexpr int MAX_SPLITS = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Theta {
  double t[DRP / 2];  // base^(-2p/d_rope)
};

// Registers of one prefetched tile: wave w holds entries w*16 .. w*16+15, one
// entry per load (lane l: dims 8l .. 8l+7, 16 B of BF16 or 8 B of FP8), plus
// two 16-byte RoPE chunks per thread.
template <bool FP8>
struct Prefetch;
template <>
struct Prefetch<false> {
  u32x4 nope[16];
  u32x4 rope[2];
  float scale;
};
template <>
struct Prefetch<true> {
  u32x2 nope[16];
  u32x4 rope[2];
  float scale;  // thread tid < TILE: the FP8 scale of entry tid
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// FP8 E4M3 code -> BF16 bits (exact: 3 mantissa bits fit in 7).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  return __float_as_uint(e4m3_to_f32(c)) >> 16;
}

__device__ __forceinline__ bf16x8 lds_b128(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// acc += A B over NSTEP k-steps of 16, A and B rows read from LDS (16 B per
// lane per step, step s at +16s); loads of the next group of 4 steps are
// issued before the MFMAs of the current group.
template <int NSTEP>
__device__ __forceinline__ void mm_lds(const bf16_t* a, const bf16_t* b, f32x16& acc) {
  constexpr int GS = 2;  // k-steps per group
  static_assert(NSTEP % GS == 0, "whole groups");
  bf16x8 ra[2][GS], rb[2][GS];
#pragma unroll
  for (int i = 0; i < GS; ++i) { ra[0][i] = lds_b128(a + 16 * i); rb[0][i] = lds_b128(b + 16 * i); }
#pragma unroll
  for (int g = 0; g < NSTEP / GS; ++g) {
    const int cur = g & 1;
    if (g + 1 < NSTEP / GS) {
#pragma unroll
      for (int i = 0; i < GS; ++i) {
        ra[cur ^ 1][i] = lds_b128(a + 16 * (GS * (g + 1) + i));
        rb[cur ^ 1][i] = lds_b128(b + 16 * (GS * (g + 1) + i));
      }
    }
#pragma unroll
    for (int i = 0; i < GS; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[cur][i], rb[cur][i], acc, 0, 0, 0);
  }
}

// Stages the query's 64 heads in LDS (row = head), the last 64 dims turned
// by RoPE at `pos` (angles reduced in fp64), rounded back to BF16.  Every
// thread issues all of its loads (16 non-RoPE and 2 RoPE chunks of 8 dims)
// before the first LDS store.
__device__ __forceinline__ void stage_query(bf16_t* qtile, const bf16_t* q, int64_t pos, const Theta& th) {
  const int tid = threadIdx.x;
  constexpr int NN = NH * (DN / 8) / 256, NR = NH * (DRP / 8) / 256;
  u32x4 rn[NN], rr[NR];
#pragma unroll
  for (int it = 0; it < NN; ++it) {
    const int c = it * 256 + tid, h = c / (DN / 8), d0 = (c % (DN / 8)) * 8;
    rn[it] = *reinterpret_cast<const u32x4*>(q + static_cast<size_t>(h) * CW + d0);
  }
#pragma unroll
  for (int it = 0; it < NR; ++it) {
    const int c = it * 256 + tid, h = c / (DRP / 8), d0 = DN + (c % (DRP / 8)) * 8;
    rr[it] = *reinterpret_cast<const u32x4*>(q + static_cast<size_t>(h) * CW + d0);
  }
#pragma unroll
  for (int it = 0; it < NN; ++it) {
    const int c = it * 256 + tid, h = c / (DN / 8), d0 = (c % (DN / 8)) * 8;
    *reinterpret_cast<u32x4*>(qtile + h * KROW + d0) = rn[it];
  }
#pragma unroll
  for (int it = 0; it < NR; ++it) {
    const int c = it * 256 + tid, h = c / (DRP / 8), p0 = (c % (DRP / 8)) * 4;
    u32x4 raw = rr[it];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double ang = static_cast<double>(pos) * th.t[p0 + i];
      const float red = static_cast<float>(ang - rint(ang * 0.15915494309189535) * 6.283185307179586);
      const float sn = __sinf(red), cs = __cosf(red);
      const float x0 = bf16_to_f32(static_cast<bf16_t>(raw[i] & 0xFFFFu));
      const float x1 = bf16_to_f32(static_cast<bf16_t>(raw[i] >> 16));
      raw[i] = static_cast<uint32_t>(f32_to_bf16(x0 * cs - x1 * sn)) |
               (static_cast<uint32_t>(f32_to_bf16(x0 * sn + x1 * cs)) << 16);
    }
    *reinterpret_cast<u32x4*>(qtile + h * KROW + DN + 2 * p0) = raw;
  }
}

// Workgroup barrier ordering LDS accesses only: global loads in flight (the
// next tile's prefetch) stay in flight across it, where __syncthreads()
// would wait for them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two fp32 -> packed BF16 pair (hardware RNE conversion).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// 4 FP8 E4M3 codes -> 4 BF16 values (exact: 3 mantissa bits fit in 7).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return u32x2{pack2_bf16(lo[0], lo[1]), pack2_bf16(hi[0], hi[1])};
}

// Id of list slot r of this workgroup (its valid ids are compacted to the
// front of s_list; slots past `nvalid` repeat slot 0, whose row is a real
// entry, and are masked out of the softmax).
template <bool DENSE>
__device__ __forceinline__ int slot_id(const int* s_list, int64_t r, int64_t r0, int64_t nvalid) {
  const int64_t rr = r < nvalid ? r : 0;
  return DENSE ? static_cast<int>(r0 + rr) : s_list[rr];
}

// Issues the global loads of one 64-entry tile starting at slot rl.  Lane i
// < 16 of wave w reads the id of the wave's row i from LDS once; the rows'
// ids then come from v_readlane (wave-uniform, so the row addresses are
// scalar) without a dependent LDS read per row.
template <bool FP8, bool DENSE>
__device__ __forceinline__ void load_tile(Prefetch<FP8>& pf, const AttnParams& P, const int* s_list, int64_t rl,
                                          int64_t r0, int64_t nvalid, size_t seq) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int my_id = slot_id<DENSE>(s_list, rl + w * 16 + (lane & 15), r0, nvalid);
  int rid[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) rid[it] = slot_id<DENSE>(s_list, rl + (it * 256 + tid) / 8, r0, nvalid);
  int sid = 0;
  if constexpr (FP8) sid = slot_id<DENSE>(s_list, rl + lane, r0, nvalid);
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int id = __builtin_amdgcn_readlane(my_id, it);
    if constexpr (!FP8) {
      const bf16_t* row = static_cast<const bf16_t*>(P.nope) + (seq + id) * DN;
      pf.nope[it] = *reinterpret_cast<const u32x4*>(row + lane * 8);
    } else {
      const uint8_t* row = static_cast<const uint8_t*>(P.nope) + (seq + id) * DN;
      pf.nope[it] = *reinterpret_cast<const u32x2*>(row + lane * 8);
    }
  }
  const bf16_t* rbase = static_cast<const bf16_t*>(P.rope);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = it * 256 + tid;
    pf.rope[it] = *reinterpret_cast<const u32x4*>(rbase + (seq + rid[it]) * DRP + (q % 8) * 8);
  }
  if constexpr (FP8) {
    if (tid < TILE) pf.scale = static_cast<const float*>(P.scale)[seq + sid];
  }
}

template <bool FP8>
__device__ __forceinline__ void store_tile(const Prefetch<FP8>& pf, bf16_t* ktile, float* s_scale) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    u32x4 v;
    if constexpr (!FP8) {
      v = pf.nope[it];
    } else {
      const u32x2 lo = fp8x4_to_bf16x4(pf.nope[it][0]), hi = fp8x4_to_bf16x4(pf.nope[it][1]);
      v = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    *reinterpret_cast<u32x4*>(ktile + (w * 16 + it) * KROW + lane * 8) = v;
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = it * 256 + tid;
    *reinterpret_cast<u32x4*>(ktile + (q / 8) * KROW + DN + (q % 8) * 8) = pf.rope[it];
  }
  if (FP8 && tid < TILE) s_scale[tid] = pf.scale;
}

// Entry (row of S^T within the wave's 32) held in register v of a 32x32
// MFMA result; the lane's column is its head.
__device__ __forceinline__ int acc_row(int v, int lane) { return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); }

typedef short v4s __attribute__((ext_vector_type(4)));

// V^T operand (A of O^T += V^T P^T) for value dims [dv0, dv0 + 32) and
// entries [k0, k0 + 16) from the row-major tile, via two transposing LDS
// reads: within a 16-lane group, result lane i slot s is element i%4 of the
// 8 bytes addressed by lane 4s + i/4; lane L = 16G + 4s + q therefore points
// at entry k0 + 8(G/2) + s (+4 for the second read), dims dv0 + 16(G%2) + 4q,
// which gives lane l the dims dv0 + l%32 of entries k0 + 8(l/32) .. +8.
__device__ __forceinline__ bf16x8 v_operand(const bf16_t* ktile, int k0, int dv0, int lane) {
  const int G = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
  const bf16_t* p = ktile + (k0 + 8 * (G >> 1) + s) * KROW + dv0 + 16 * (G & 1) + 4 * q;
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * KROW));
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s all = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, all);
}

constexpr int MAX_LIST = 1024;  // list entries one workgroup handles

template <bool FP8, bool DENSE, bool SPLIT>
__global__ void __launch_bounds__(256, 1)
attn_mfma_kernel(AttnParams P, Theta th, int splits, int64_t per_split, float* part) {
  __shared__ __attribute__((aligned(16))) bf16_t ktile[TILE * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t qtile[NH * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t pbuf[NH * PROW];
  __shared__ float s_scale[TILE];
  __shared__ float s_xchg[2][NH];
  __shared__ int s_list[DENSE ? 1 : MAX_LIST];
  __shared__ int s_cnt[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hp = w >> 1, ep = w & 1;
  const int b = blockIdx.z;
  const int t = SPLIT ? 0 : blockIdx.x;
  const int split = SPLIT ? blockIdx.x : 0;
  const int64_t pos = P.pos_dev ? P.pos_dev[b] : P.pos0 + t;
  int64_t n = pos < 0 ? 0 : (pos + 1) / P.m;
  if (n > P.cap) n = P.cap;
  const int64_t count = DENSE ? n : P.k;
  const int64_t r0 = static_cast<int64_t>(split) * per_split;
  int64_t r1 = r0 + per_split;
  if (r1 > count) r1 = count;
  const size_t qrow = (static_cast<size_t>(b) * P.T + t) * NH;
  const size_t seq = static_cast<size_t>(b) * P.cap;
  const int head = 32 * hp + (lane & 31);  // this lane's head

  // the valid ids of this workgroup's list range, compacted into s_list
  int64_t nvalid;
  if (DENSE) {
    nvalid = r1 > r0 ? r1 - r0 : 0;
  } else {
    const int32_t* list = P.idx + (static_cast<size_t>(b) * P.T + t) * P.k;
    int base = 0;
    for (int64_t c0 = 0; c0 < r1 - r0; c0 += 256) {
      const int64_t r = c0 + tid;
      int64_t sid = r < r1 - r0 ? static_cast<int64_t>(list[r0 + r]) : -1;
      const bool ok = sid >= 0 && sid < n;
      const unsigned long long bal = __ballot(ok);
      if (lane == 0) s_cnt[w] = __popcll(bal);
      lds_barrier();
      int before = 0, tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { before += i < w ? s_cnt[i] : 0; tot += s_cnt[i]; }
      if (ok) s_list[base + before + __popcll(bal & ((1ull << lane) - 1ull))] = static_cast<int>(sid);
      base += tot;
      lds_barrier();
    }
    nvalid = base;
  }
  stage_query(qtile, static_cast<const bf16_t*>(P.q) + qrow * CW, pos, th);
  const bf16_t* qop = qtile + head * KROW + (lane >> 5) * 8;                       // B of S^T
  const bf16_t* kop = ktile + (ep * 32 + (lane & 31)) * KROW + (lane >> 5) * 8;    // A of S^T
  const bf16_t* pop = pbuf + head * PROW + (lane >> 5) * 8;                        // B of O^T

  const float lscale = P.scale_qk * LOG2E;
  f32x16 oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = f32x16{};
  // running max (log2 domain) and this lane's partial denominator; the max
  // only moves when a tile's max exceeds it by more than 2^8, so P stays
  // below 256 and the accumulators are rarely rescaled
  float m_run = -INFINITY, l_part = 0.0f;

  lds_barrier();  // s_list and the query tile ready
  const int64_t ntiles = (nvalid + TILE - 1) / TILE;
  Prefetch<FP8> pf;
  if (ntiles > 0) load_tile<FP8, DENSE>(pf, P, s_list, 0, r0, nvalid, seq);
  for (int64_t j = 0; j < ntiles; ++j) {
    lds_barrier();  // previous tile's O^T finished with ktile / pbuf
    store_tile<FP8>(pf, ktile, s_scale);
    lds_barrier();
    if (j + 1 < ntiles) load_tile<FP8, DENSE>(pf, P, s_list, (j + 1) * TILE, r0, nvalid, seq);

    // --- S^T = K Q^T: entries 32ep.. x heads 32hp.. --------------------------
    f32x16 sn = f32x16{}, sr = f32x16{};
    if (FP8) {
      mm_lds<DN / 16>(kop, qop, sn);
      mm_lds<DRP / 16>(kop + DN, qop + DN, sr);
    } else {
      mm_lds<CW / 16>(kop, qop, sn);
    }
    const int64_t valid_end = nvalid - j * TILE;  // entries of this tile below it are real
    float lg[16], esc[16];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int e = ep * 32 + acc_row(v, lane);
      esc[v] = FP8 ? s_scale[e] : 1.0f;
      lg[v] = e < valid_end ? (FP8 ? sn[v] * esc[v] + sr[v] : sn[v]) * lscale : -INFINITY;
      mx = fmaxf(mx, lg[v]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));  // the other 16 entries of this head
    if (lane < 32) s_xchg[ep][head] = mx;
    lds_barrier();
    mx = fmaxf(mx, s_xchg[ep ^ 1][head]);
    const bool move = mx > m_run + 8.0f;
    if (__ballot(move)) {
      // accumulators are still zero while m_run is -inf: no rescale needed
      const float alpha = move ? (m_run == -INFINITY ? 0.0f : exp2f(m_run - mx)) : 1.0f;
      if (__ballot(move && m_run != -INFINITY)) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) oacc[nb] *= alpha;
      }
      l_part *= alpha;
      m_run = move ? mx : m_run;
    }
    float psum = 0.0f;
    uint32_t pk[8];
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = exp2f(lg[v] - m_run), p1 = exp2f(lg[v + 1] - m_run);
      psum += p0 + p1;
      // V rows in the tile are unscaled FP8 codes: the entry scale goes into P
      pk[v >> 1] = FP8 ? pack2_bf16(p0 * esc[v], p1 * esc[v + 1]) : pack2_bf16(p0, p1);
    }
    l_part += psum;
    // P^T rows: 4 consecutive entries per register quad -> one 8-byte store each
#pragma unroll
    for (int jq = 0; jq < 4; ++jq)
      *reinterpret_cast<uint2*>(pbuf + head * PROW + ep * 32 + jq * 8 + (lane >> 5) * 4) =
          make_uint2(pk[2 * jq], pk[2 * jq + 1]);
    lds_barrier();

    // --- O^T += V^T P^T: value dims 256ep.. x heads 32hp.. --------------------
    bf16x8 pb[TILE / 16];
#pragma unroll
    for (int ks = 0; ks < TILE / 16; ++ks) pb[ks] = lds_b128(pop + ks * 16);
    bf16x8 va[3];
    va[0] = v_operand(ktile, 0, ep * 256, lane);
    va[1] = v_operand(ktile, 16, ep * 256, lane);
#pragma unroll
    for (int i = 0; i < 8 * (TILE / 16); ++i) {
      if (i + 2 < 8 * (TILE / 16))
        va[(i + 2) % 3] = v_operand(ktile, ((i + 2) % 4) * 16, ep * 256 + ((i + 2) / 4) * 32, lane);
      oacc[i / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], pb[i % 4], oacc[i / 4], 0, 0, 0);
    }
  }

  // --- finish: softmax denominators -------------------------------------
  l_part += __shfl_xor(l_part, 32);
  lds_barrier();
  if (lane < 32) s_xchg[ep][head] = l_part;
  lds_barrier();
  const float ltot = l_part + s_xchg[ep ^ 1][head];

  // O^T layout: lane = head, register (nb, v) = value dim ep*256 + nb*32 + acc_row(v)
  if (!SPLIT) {
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    bf16_t* out = static_cast<bf16_t*>(P.o) + (qrow + head) * DN + ep * 256;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const uint32_t lo = pack2_bf16(oacc[nb][4 * jq] * inv, oacc[nb][4 * jq + 1] * inv);
        const uint32_t hi = pack2_bf16(oacc[nb][4 * jq + 2] * inv, oacc[nb][4 * jq + 3] * inv);
        *reinterpret_cast<uint2*>(out + nb * 32 + jq * 8 + (lane >> 5) * 4) = make_uint2(lo, hi);
      }
    if (P.lse && ep == 0 && lane < 32) P.lse[qrow + head] = ltot > 0.0f ? (m_run + log2f(ltot)) * LN2 : -INFINITY;
  } else {
    // partial: [B][splits][NH][DN] O, then [B][splits][NH][2] (max, sum)
    const size_t slot = static_cast<size_t>(b) * splits + split;
    float* po = part + slot * (NH * DN) + head * DN + ep * 256;
    float* pml = part + static_cast<size_t>(gridDim.z) * splits * (NH * DN) + slot * (2 * NH);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<float4*>(po + nb * 32 + jq * 8 + (lane >> 5) * 4) =
            make_float4(oacc[nb][4 * jq], oacc[nb][4 * jq + 1], oacc[nb][4 * jq + 2], oacc[nb][4 * jq + 3]);
    if (ep == 0 && lane < 32) {
      pml[2 * head] = m_run;
      pml[2 * head + 1] = ltot;
    }
  }
}

// Combines split partials by log-sum-exp; grid (NH, B), one thread per 4
// value dims (128 threads), the head's split weights computed once in LDS.
// S >= splits is a power of two: every thread's S partial loads (clamped to
// the last split) are issued before the weights are known.
template <int S>
__global__ void __launch_bounds__(128) attn_merge_kernel(AttnParams P, int splits, const float* part, int B) {
  __shared__ float s_f[S];
  __shared__ float s_L, s_M;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* po = part + static_cast<size_t>(b) * splits * (NH * DN) + static_cast<size_t>(h) * DN + 4 * tid;
  float4 v[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp)
    v[sp] = *reinterpret_cast<const float4*>(po + static_cast<size_t>(min(sp, splits - 1)) * NH * DN);
  const float* pml = part + static_cast<size_t>(B) * splits * (NH * DN) + static_cast<size_t>(b) * splits * (2 * NH);
  if (tid < 64) {
    const float ms = tid < splits ? pml[(tid * NH + h) * 2] : -INFINITY;
    const float ls = tid < splits ? pml[(tid * NH + h) * 2 + 1] : 0.0f;
    float M = ms;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = (tid < splits && ms != -INFINITY) ? exp2f(ms - M) : 0.0f;
    float L = ls * f;
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    if (tid < S) s_f[tid] = f;
    if (tid == 0) { s_L = L; s_M = M; }
  }
  __syncthreads();
  const float L = s_L;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float f = s_f[sp];  // 0 past the last split and for empty splits
    acc.x += v[sp].x * f; acc.y += v[sp].y * f; acc.z += v[sp].z * f; acc.w += v[sp].w * f;
  }
  bf16_t* out = static_cast<bf16_t*>(P.o) + (static_cast<size_t>(b) * NH + h) * DN + 4 * tid;
  *reinterpret_cast<uint2*>(out) = make_uint2(pack2_bf16(acc.x * inv, acc.y * inv), pack2_bf16(acc.z * inv, acc.w * inv));
  if (P.lse && tid == 0) P.lse[static_cast<size_t>(b) * NH + h] = L > 0.0f ? (s_M + log2f(L)) * LN2 : -INFINITY;
}

Theta make_theta(double base) {
  Theta th;
  for (int p = 0; p < DRP / 2; ++p) th.t[p] = std::pow(base, -2.0 * p / DRP);
  return th;
}

int decode_splits(int B, int64_t ntiles) {
  int64_t s = (256 + B - 1) / B;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  if (s > ntiles) s = ntiles;
  return s < 1 ? 1 : static_cast<int>(s);
}

}  // namespace

bool mfma_attn_supported(const AttnParams& P) {
  const bool shape = P.H == NH && P.d_nope == DN && P.d_rope == DRP && P.q_dt == CSA_BF16 && P.o_dt == CSA_BF16 &&
                     (P.nope_dt == CSA_BF16 || P.nope_dt == CSA_FP8E4M3) && P.rope_dt == CSA_BF16;
  // sparse prefill keeps one query's whole list in LDS
  const bool list_fits = P.idx == nullptr || P.pos_dev != nullptr || P.k <= MAX_LIST;
  return shape && list_fits;
}

size_t mfma_attn_ws_bytes(const csa_attn_desc* d, int op, int B, int, int64_t, int) {
  if (op != CSA_OP_SPARSE_ATTN_DECODE && op != CSA_OP_DENSE_ATTN_DECODE) return 0;
  if (d->n_heads != NH || d->d_nope != DN || d->d_rope != DRP) return 0;
  return static_cast<size_t>(B) * MAX_SPLITS * (NH * DN + 2 * NH) * sizeof(float);
}

template <bool FP8, bool DENSE, bool SPLIT>
static void launch_one(const AttnParams& P, dim3 grid, hipStream_t s, int splits, int64_t per, float* part) {
  hipLaunchKernelGGL((attn_mfma_kernel<FP8, DENSE, SPLIT>), grid, dim3(256), 0, s, P, make_theta(P.base), splits,
                     per, part);
}

int launch_mfma_attn(const AttnParams& P, int op, int B, hipStream_t s) {
  const bool fp8 = P.nope_dt == CSA_FP8E4M3;
  const bool dense = op == CSA_OP_DENSE_ATTN_PREFILL || op == CSA_OP_DENSE_ATTN_DECODE;
  const bool decode = op == CSA_OP_SPARSE_ATTN_DECODE || op == CSA_OP_DENSE_ATTN_DECODE;
  if (!decode) {
    const int64_t per = dense ? P.cap : P.k;
    dim3 grid(P.T, 1, B);
    if (fp8) dense ? launch_one<true, true, false>(P, grid, s, 1, per, nullptr) : launch_one<true, false, false>(P, grid, s, 1, per, nullptr);
    else launch_attn_bf16(P, dense, B, s, 1, per, nullptr);
    return check_launch("attn_mfma_kernel");
  }
  const int64_t count = dense ? P.cap : P.k;
  const int64_t ntiles = (count + TILE - 1) / TILE;
  int splits = decode_splits(B, ntiles);
  if (!dense) {  // each workgroup's list range must fit its LDS copy
    const int min_s = static_cast<int>((ntiles * TILE + MAX_LIST - 1) / MAX_LIST);
    if (splits < min_s) splits = min_s;
  }
  const int64_t tiles_per = (ntiles + splits - 1) / splits;
  const int64_t per = tiles_per * TILE;
  const size_t need = static_cast<size_t>(B) * splits * (NH * DN + 2 * NH) * sizeof(float);
  if (!P.ws || P.ws_bytes < need) return fail(CSA_ERR_WORKSPACE, "workspace too small for the split partials");
  float* part = static_cast<float*>(P.ws);
  dim3 grid(splits, 1, B);
  if (fp8) dense ? launch_one<true, true, true>(P, grid, s, splits, per, part) : launch_one<true, false, true>(P, grid, s, splits, per, part);
  else launch_attn_bf16(P, dense, B, s, splits, per, part);
  int st = check_launch("attn_mfma_kernel");
  if (st != CSA_OK) return st;
  const dim3 mg(NH, B);
  if (splits <= 1) hipLaunchKernelGGL(attn_merge_kernel<1>, mg, dim3(128), 0, s, P, splits, part, B);
  else if (splits <= 2) hipLaunchKernelGGL(attn_merge_kernel<2>, mg, dim3(128), 0, s, P, splits, part, B);
  else if (splits <= 4) hipLaunchKernelGGL(attn_merge_kernel<4>, mg, dim3(128), 0, s, P, splits, part, B);
  else if (splits <= 8) hipLaunchKernelGGL(attn_merge_kernel<8>, mg, dim3(128), 0, s, P, splits, part, B);
  else if (splits <= 16) hipLaunchKernelGGL(attn_merge_kernel<16>, mg, dim3(128), 0, s, P, splits, part, B);
  else hipLaunchKernelGGL(attn_merge_kernel<MAX_SPLITS>, mg, dim3(128), 0, s, P, splits, part, B);
  return check_launch("attn_merge_kernel");
}

}  // namespace csa
