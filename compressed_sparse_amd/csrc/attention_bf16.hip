// MFMA attention over a BF16 cache (64 query heads sharing one entry of 512
// non-RoPE + 64 RoPE dims, MQA): the CSA prefill shape.  [CSA/HCA 混注意力]
// §1.1, §1.2; [读完这篇] §三 CSA 步骤三 (standard attention over the selected
// entries, one KV shared by all heads).
//
// One workgroup (8 waves, two per SIMD so that one wave's softmax and LDS
// waits overlap the other's MFMAs) owns one query and a range of its entry
// list, 64 entries per tile.  Per tile the work is S^T = K Q^T (64 x 64 x
// 576) and O^T += V^T P^T (512 x 64 x 64):
//
//  * entry rows go HBM/L2 -> LDS by direct loads (global_load_lds_dwordx4),
//    no VGPR staging, into two tile buffers used in turn: tile j+1 loads
//    while tile j is multiplied.  Rows are unpadded; the 16-byte chunks of a
//    row are XOR-swizzled by row so that the MFMA operand reads of 16
//    consecutive rows (and the transposing V reads) hit distinct banks;
//  * wave w = (ep, hq) computes S^T for entries 32ep.. x heads 16hq..
//    (v_mfma_f32_16x16x32_bf16) with the query's B fragments (its 16 heads,
//    all 576 dims, RoPE applied) held in registers, then that block's
//    softmax; P^T goes through LDS;
//  * for O^T (v_mfma_f32_32x32x16_bf16) wave w owns value dims 64w.. for all
//    64 heads, so each V element is read from LDS once per tile.
//
// The softmax running max moves only when a tile's max exceeds it by more
// than 2^8 (P stays below 256); the waves that own a head's O^T columns
// rescale them by the factor the softmax waves publish in LDS.
#include <cmath>
#include <utility>

#include "attention.hpp"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

constexpr int NH = 64;
constexpr int DN = 512;
constexpr int DRP = 64;
constexpr int CW = DN + DRP;
constexpr int TILE = 64;
constexpr int NROW = DN * 2;               // bytes of one non-RoPE row in LDS
constexpr int RROW = DRP * 2;              // bytes of one RoPE row
constexpr int ROPE_OFF = TILE * NROW;      // the RoPE rows follow the 64 non-RoPE rows
constexpr int KBUF = TILE * (NROW + RROW); // 73,728 B per tile buffer
constexpr int PROW = TILE + 8;             // padded P^T row (bf16 elements)
constexpr int MAX_LIST = 1024;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Theta {
  double t[DRP / 2];  // base^(-2p/d_rope)
};

// 16-byte chunk c of row r sits at chunk c ^ swz(r).  LDS serves 128 B (32
// banks) per cycle: 8 consecutive rows read at one chunk (an MFMA A operand)
// and the 4 rows x 2 chunks of a transposing V read then fall on distinct
// 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return 2 * (r & 3) + ((r >> 2) & 1); }
__device__ __forceinline__ int swz_rope(int r) { return swz(r); }

// Workgroup barrier for LDS data: this wave's LDS accesses complete, then
// s_barrier.  Loads in flight (the next tile) are not waited for.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits until this wave's direct-to-LDS tile loads (its only vector memory
// operations in the tile loop) have landed.
__device__ __forceinline__ void wait_tile_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ bf16x8 lds_b128(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Row of S^T within a wave's 32 held in register v of a 32x32 MFMA result.
__device__ __forceinline__ int acc_row(int v, int lane) { return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); }

template <bool DENSE>
__device__ __forceinline__ int slot_id(const int* s_list, int64_t r, int64_t r0, int64_t nvalid) {
  const int64_t rr = r < nvalid ? r : 0;  // slots past the valid ones repeat slot 0 (masked later)
  return DENSE ? static_cast<int>(r0 + rr) : s_list[rr];
}

constexpr int NW = 8;              // waves per workgroup
constexpr int ROWS_W = TILE / NW;  // tile rows each wave loads

// Issues the direct-to-LDS loads of the 64-entry tile at list slot rl into
// buf: wave w loads rows 8w .. 8w+7 (one 1 KB instruction per non-RoPE row,
// lane L fetching the chunk that belongs at slot L) and their RoPE rows (one
// instruction of 8 rows x 8 chunks).
template <bool DENSE>
__device__ __forceinline__ void issue_tile(uint8_t* buf, const AttnParams& P, const int* s_list, int64_t rl,
                                           int64_t r0, int64_t nvalid, size_t seq) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int my_id = slot_id<DENSE>(s_list, rl + w * ROWS_W + (lane & (ROWS_W - 1)), r0, nvalid);
  const uint8_t* nope = static_cast<const uint8_t*>(P.nope);
  const bf16_t* rope = static_cast<const bf16_t*>(P.rope);
#pragma unroll
  for (int it = 0; it < ROWS_W; ++it) {
    const int id = __builtin_amdgcn_readlane(my_id, it);
    const int r = w * ROWS_W + it;
    // scalar row base + 32-bit lane offset (swz(r) depends on `it` only)
    const uint8_t* row = nope + (seq + static_cast<size_t>(id)) * NROW;
    __builtin_amdgcn_global_load_lds(row + static_cast<uint32_t>(16 * (lane ^ swz(r))), buf + r * NROW, 16, 0, 0);
  }
  const int r = w * ROWS_W + (lane >> 3);
  const int idr = __shfl(my_id, lane >> 3);
  const bf16_t* src = rope + (seq + idr) * DRP + 8 * ((lane & 7) ^ swz_rope(r));
  __builtin_amdgcn_global_load_lds(src, buf + ROPE_OFF + w * ROWS_W * RROW, 16, 0, 0);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool DENSE, bool SPLIT>
__global__ void __launch_bounds__(512, 1)
attn_bf16_kernel(AttnParams P, Theta th, int splits, int64_t per_split, float* part) {
  __shared__ __attribute__((aligned(16))) uint8_t kb0[KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[KBUF];
  __shared__ __attribute__((aligned(16))) bf16_t pbuf[NH * PROW];
  __shared__ int s_list[DENSE ? 1 : MAX_LIST];
  __shared__ float s_xchg[2][NH];
  __shared__ float s_alpha[NH];
  __shared__ float s_m[NH];
  __shared__ int s_cnt[NW];
  __shared__ int s_mv[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ep = w & 1, hq = w >> 1;  // S^T role: entries 32ep.., heads 16hq..
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
  const int head = 16 * hq + (lane & 15);  // this lane's head in the S^T role
  const int g4 = lane >> 4;                // k-slice / row group of the 16x16 MFMA

  // the valid ids of this workgroup's list range, compacted into s_list
  int64_t nvalid;
  if (DENSE) {
    nvalid = r1 > r0 ? r1 - r0 : 0;
  } else {
    const int32_t* list = P.idx + (static_cast<size_t>(b) * P.T + t) * P.k;
    int base = 0;
    for (int64_t c0 = 0; c0 < r1 - r0; c0 += 64 * NW) {
      const int64_t r = c0 + tid;
      const int64_t sid = r < r1 - r0 ? static_cast<int64_t>(list[r0 + r]) : -1;
      const bool ok = sid >= 0 && sid < n;
      const unsigned long long bal = __ballot(ok);
      if (lane == 0) s_cnt[w] = __popcll(bal);
      lds_sync();
      int before = 0, tot = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) { before += i < w ? s_cnt[i] : 0; tot += s_cnt[i]; }
      if (ok) s_list[base + before + __popcll(bal & ((1ull << lane) - 1ull))] = static_cast<int>(sid);
      base += tot;
      lds_sync();
    }
    nvalid = base;
  }
  const int ntiles = static_cast<int>((nvalid + TILE - 1) / TILE);
  const int nval = static_cast<int>(nvalid);
  if (ntiles > 0) issue_tile<DENSE>(kb0, P, s_list, 0, r0, nvalid, seq);

  // B fragments of S^T (16x16x32): lane = head 16hq + lane%16, k-step s holds
  // dims 32s + 8(lane/16) .. +8; the RoPE steps turned at `pos`
  constexpr int QS = CW / 32;
  bf16x8 qf[QS];
  {
    const bf16_t* qh = static_cast<const bf16_t*>(P.q) + (qrow + head) * CW + 8 * g4;
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qh + 32 * s);
#pragma unroll
    for (int s = DN / 32; s < QS; ++s) {
      u32x4 raw = __builtin_bit_cast(u32x4, qf[s]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 16 * (s - DN / 32) + 4 * g4 + i;
        const double ang = static_cast<double>(pos) * th.t[p];
        const float red = static_cast<float>(ang - rint(ang * 0.15915494309189535) * 6.283185307179586);
        const float sn = __sinf(red), cs = __cosf(red);
        const float x0 = bf16_to_f32(static_cast<bf16_t>(raw[i] & 0xFFFFu));
        const float x1 = bf16_to_f32(static_cast<bf16_t>(raw[i] >> 16));
        raw[i] = pack2_bf16(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
      }
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // LDS byte offsets of the S^T A operand (16x16x32): M-block mb rows
  // 32ep + 16mb + lane%16, k-step s chunk 4s + lane/16
  int offA[2][4], offR[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int r = 32 * ep + 16 * mb + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) offA[mb][i] = r * NROW + 16 * ((4 * i + g4) ^ swz(r));
#pragma unroll
    for (int i = 0; i < 2; ++i) offR[mb][i] = ROPE_OFF + r * RROW + 16 * ((4 * i + g4) ^ swz_rope(r));
  }
  // V^T operand (transposing reads): within a 16-lane group, result lane i
  // slot s is element i%4 of the 8 bytes addressed by lane 4s + i/4.  Lane
  // L = 16G + 4s + q reads entry 8(G/2) + s (+4 for the second read) of the
  // k-step, value dims 64w + 32mb + 16(G%2) + 4q .. +4.
  const int G = lane >> 4, sq = (lane >> 2) & 3, q4 = lane & 3;
  const int rowA = 8 * (G >> 1) + sq, rowB = rowA + 4;
  int offV[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    // 16-byte chunk 8w + 4mb + 2(G%2) + q/2: high bits w/2, low four bits swizzled
    const int c = 8 * (w & 1) + 4 * mb + 2 * (G & 1) + (q4 >> 1);
    offV[mb][0] = rowA * NROW + 16 * (16 * (w >> 1) + (c ^ swz(rowA))) + 8 * (q4 & 1);
    offV[mb][1] = rowB * NROW + 16 * (16 * (w >> 1) + (c ^ swz(rowB))) + 8 * (q4 & 1);
  }
  const bf16_t* pop = pbuf + (lane & 31) * PROW + 8 * (lane >> 5);  // + 32 nb rows: heads 32nb..

  const float lscale = P.scale_qk * LOG2E;
  f32x16 oacc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) oacc[mb][nb] = f32x16{};
  float m_run = -INFINITY, l_part = 0.0f;

  auto tile = [&](auto parity, int j) {
    constexpr int PAR = decltype(parity)::value;
    const uint8_t* cur = PAR ? kb1 : kb0;
    uint8_t* nxt = PAR ? kb0 : kb1;
    wait_tile_loads();
    lds_sync();  // tile j in LDS; every wave done with tile j-1 (its buffer, pbuf, s_alpha)
    if (j + 1 < ntiles) issue_tile<DENSE>(nxt, P, s_list, static_cast<int64_t>(j + 1) * TILE, r0, nvalid, seq);

    // --- S^T = K Q^T: entries 32ep + 16mb.. x heads 16hq.. ------------------
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int s = 0; s < QS; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 a = s < DN / 32 ? lds_b128(cur + offA[mb][s & 3] + 256 * (s >> 2))
                                     : lds_b128(cur + offR[mb][s - DN / 32]);
        sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[mb], 0, 0, 0);
      }
    }
    // --- softmax: lane holds entries 32ep + 16mb + 4(lane/16) + v of its head
    const int vend = nval - j * TILE;  // entries of this tile below it are real
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e = 32 * ep + 16 * mb + 4 * g4 + v;
        sacc[mb][v] = e < vend ? sacc[mb][v] * lscale : -INFINITY;
        mx = fmaxf(mx, sacc[mb][v]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lane < 16) s_xchg[ep][head] = mx;
    lds_sync();
    mx = fmaxf(mx, s_xchg[ep ^ 1][head]);
    const bool move = mx > m_run + 8.0f;
    const bool rescale = move && m_run != -INFINITY;
    const float alpha = rescale ? exp2f(m_run - mx) : 1.0f;
    if (move) m_run = mx;
    l_part *= alpha;
    if (ep == 0) {
      if (lane < 16) s_alpha[head] = alpha;
      const bool any = __ballot(rescale) != 0ull;
      if (lane == 0) s_mv[hq] = any ? 1 : 0;
    }
    float psum = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float p0 = __builtin_amdgcn_exp2f(sacc[mb][0] - m_run), p1 = __builtin_amdgcn_exp2f(sacc[mb][1] - m_run);
      const float p2 = __builtin_amdgcn_exp2f(sacc[mb][2] - m_run), p3 = __builtin_amdgcn_exp2f(sacc[mb][3] - m_run);
      psum += (p0 + p1) + (p2 + p3);
      *reinterpret_cast<uint2*>(pbuf + head * PROW + 32 * ep + 16 * mb + 4 * g4) =
          make_uint2(pack2_bf16(p0, p1), pack2_bf16(p2, p3));
    }
    l_part += psum;
    lds_sync();

    // --- O^T += V^T P^T: value dims 64w.. x all 64 heads ----------------------
    if (s_mv[0] | s_mv[1] | s_mv[2] | s_mv[3]) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float a = s_alpha[32 * nb + (lane & 31)];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) oacc[mb][nb] *= a;
      }
    }
#pragma unroll
    for (int ks = 0; ks < TILE / 16; ++ks) {
      bf16x8 pb[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) pb[nb] = *reinterpret_cast<const bf16x8*>(pop + 32 * nb * PROW + 16 * ks);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        typedef __attribute__((address_space(3))) v4s lds_v4s;
        const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(cur + offV[mb][0] + 16 * ks * NROW));
        const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(cur + offV[mb][1] + 16 * ks * NROW));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          oacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[nb], oacc[mb][nb], 0, 0, 0);
      }
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) tile(std::integral_constant<int, 1>{}, j + 1);
  }

  // --- finish: denominators and maxima to LDS, then each wave its O^T ----
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
  lds_sync();
  if (lane < 16) s_xchg[ep][head] = l_part;
  if (ep == 0 && lane < 16) s_m[head] = m_run;
  lds_sync();
  // O^T block (mb, nb): lane = head 32nb + lane%32, register v = value dim
  // 64w + 32mb + acc_row(v)
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int h = 32 * nb + (lane & 31);
    const float ltot = s_xchg[0][h] + s_xchg[1][h];
    if (!SPLIT) {
      const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
      bf16_t* out = static_cast<bf16_t*>(P.o) + (qrow + h) * DN + 64 * w;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x16& o = oacc[mb][nb];
          const uint32_t lo = pack2_bf16(o[4 * jq] * inv, o[4 * jq + 1] * inv);
          const uint32_t hi2 = pack2_bf16(o[4 * jq + 2] * inv, o[4 * jq + 3] * inv);
          *reinterpret_cast<uint2*>(out + 32 * mb + jq * 8 + (lane >> 5) * 4) = make_uint2(lo, hi2);
        }
      if (P.lse && w == 0 && lane < 32)
        P.lse[qrow + h] = ltot > 0.0f ? (s_m[h] + log2f(ltot)) * LN2 : -INFINITY;
    } else {
      // partial: [B][splits][NH][DN] O, then [B][splits][NH][2] (max, sum)
      const size_t slot = static_cast<size_t>(b) * splits + split;
      float* po = part + slot * (NH * DN) + static_cast<size_t>(h) * DN + 64 * w;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x16& o = oacc[mb][nb];
          *reinterpret_cast<float4*>(po + 32 * mb + jq * 8 + (lane >> 5) * 4) =
              make_float4(o[4 * jq], o[4 * jq + 1], o[4 * jq + 2], o[4 * jq + 3]);
        }
      if (w == 0 && lane < 32) {
        float* pml = part + static_cast<size_t>(gridDim.z) * splits * (NH * DN) + slot * (2 * NH);
        pml[2 * h] = s_m[h];
        pml[2 * h + 1] = ltot;
      }
    }
  }
}

}  // namespace

void launch_attn_bf16(const AttnParams& P, bool dense, dim3 grid, hipStream_t s, int splits, int64_t per,
                      float* part) {
  Theta th;
  for (int p = 0; p < DRP / 2; ++p) th.t[p] = std::pow(P.base, -2.0 * p / DRP);
  const bool split = part != nullptr;
  if (dense) {
    if (split) hipLaunchKernelGGL((attn_bf16_kernel<true, true>), grid, dim3(512), 0, s, P, th, splits, per, part);
    else hipLaunchKernelGGL((attn_bf16_kernel<true, false>), grid, dim3(512), 0, s, P, th, splits, per, part);
  } else {
    if (split) hipLaunchKernelGGL((attn_bf16_kernel<false, true>), grid, dim3(512), 0, s, P, th, splits, per, part);
    else hipLaunchKernelGGL((attn_bf16_kernel<false, false>), grid, dim3(512), 0, s, P, th, splits, per, part);
  }
}

}  // namespace csa
