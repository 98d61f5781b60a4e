// MFMA attention over a BF16 cache (64 query heads sharing one entry of 512
// non-RoPE + 64 RoPE dims, MQA): the CSA prefill shape.  [CSA/HCA 混注意力]
// §1.1, §1.2; [读完这篇] §三 CSA 步骤三 (standard attention over the selected
// entries, one KV shared by all heads).
//
// A work item is one query (prefill) or one range of a sequence's entries
// (split decode).  The grid is persistent, one 4-wave workgroup per compute
// unit, one wave per SIMD with the whole 512-register file, so that each
// wave keeps its query fragments, its output accumulators and a queue of
// LDS operand reads in flight.  Items run 64 entries per tile; per tile the
// work is S^T = K Q^T (64 x 64 x 576) and O^T += V^T P^T (512 x 64 x 64):
//
//  * entry rows go HBM/L2 -> LDS by direct loads (buffer_load_dwordx4 ...
//    lds), no VGPR staging, into two tile buffers used in turn: tile j+1
//    loads while tile j is multiplied, its loads spread over tile j's MFMAs.  Rows are unpadded; their 16-byte chunks
//    are XOR-swizzled by row so that MFMA operand reads and transposing V
//    reads hit distinct banks;
//  * wave w = (eh, hh) computes the 32 x 32 block of S^T for entries 32eh..
//    and heads 32hh.. (v_mfma_f32_32x32x16_bf16) with the query's B
//    fragments (its 32 heads, all 576 dims, RoPE applied) in registers, so
//    each entry row is read from LDS by two waves only; the two entry halves
//    of a head agree on the softmax maximum through LDS; P^T goes through
//    LDS;
//  * for O^T (v_mfma_f32_32x32x16_bf16) wave w owns value dims 128w.. for
//    all 64 heads, so each V element is read from LDS once per tile.
//
// The softmax running max moves only when a tile's max exceeds it by more
// than 2^8 (P stays below 256); only then do the two entry halves of a head
// exchange maxima, and the waves that own a head's O^T columns rescale them
// by the factor the softmax waves publish in LDS.
//
// While a workgroup finishes an item it already holds the next item's index
// list, has the next item's first tile in flight and reloads its query
// fragments behind the last S^T MFMAs.  The finished
// item's output is staged in the free tile buffer and stored, as whole 1 KB
// rows, once the next item's first tile has landed, so the stores drain
// while that tile is multiplied.
#include <atomic>
#include <cmath>

#include "attention.hpp"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int NH = 64;
constexpr int DN = 512;
constexpr int DRP = 64;
constexpr int CW = DN + DRP;
constexpr int TILE = 64;
constexpr int NROW = DN * 2;               // bytes of one BF16 non-RoPE row (and of a staged output row)
constexpr int RROW = DRP * 2;              // bytes of one RoPE row
constexpr int PROW = TILE + 8;             // padded P^T row (bf16 elements)

// Tile buffer layout: 64 non-RoPE rows (BF16 1 KB, or FP8 codes 512 B),
// then 64 RoPE rows, then (FP8) the 64 entry scales.  An FP8 buffer is
// padded to 64 KB so that an item's output (64 rows of 1 KB) can be staged
// in it.
template <bool FP8>
struct Lay {
  static constexpr int NROWB = FP8 ? DN : DN * 2;
  static constexpr int ROPE_OFF = TILE * NROWB;
  static constexpr int SC_OFF = ROPE_OFF + TILE * RROW;
  static constexpr int BYTES = SC_OFF + (FP8 ? TILE * 4 : 0);
  static constexpr int KBUF = BYTES > TILE * NROW ? BYTES : TILE * NROW;
  static constexpr int NLOAD = FP8 ? 11 : 18;  // loads per wave per tile
};
constexpr int MAX_LIST = 1024;
constexpr int NW = 4;                      // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int QS = CW / 16;                // k-steps of S^T (16 dims each)
constexpr int SPF = 6;                     // S^T A operands in flight
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// RoPE frequencies theta_p = base^(-2p/d_rope) = r^p, r = base^(-2/d_rope):
// the uniform powers a lane needs to form its own 16 (held in scalar
// registers; a per-lane table here would be read with lane-dependent
// offsets and kept live in vector registers across the item loop)
struct Theta {
  double r1, r2, r3, r4, r8;
};

// 16-byte chunk c of row r sits at chunk c ^ swz(r).  The LDS has 64 banks
// (256 B); a 128-bit read is served in four passes of 16 lanes (lanes with
// equal bit 5 and equal parity of bits 2..4), a 64-bit read (also the
// transposing one) in two passes of 32 lanes (equal bit 5).  With these
// swizzles the 16 rows of one pass of an S^T A-operand read (rows that
// differ in bits 0, 1, 2 and 4) and the 4 rows x 4 half-chunks of one pass
// of a transposing V read land on distinct banks.  RoPE rows are 128 B
// (8 chunks), two rows per bank line.
__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + 2 * ((r >> 2) & 1) + ((r >> 4) & 1); }
__device__ __forceinline__ int swz_rope(int r) { return 4 * ((r >> 1) & 1) + 2 * ((r >> 2) & 1) + ((r >> 4) & 1); }
// FP8 rows (512 B, 32 chunks): an S^T A-operand pass reads one chunk of 16
// rows differing in bits 0, 1, 2 and 4; a transposing 8-bit V read pass
// reads 8 consecutive rows x 2 chunks x 2 halves.
__device__ __forceinline__ int swzf(int r) { return 2 * (r & 7) + ((r >> 4) & 1); }

// 8 FP8 E4M3 codes (low byte first) widened to BF16, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI));
}
__device__ __forceinline__ bf16x8 fp8x8_bf16(uint32_t w0, uint32_t w1) {
  return __builtin_bit_cast(bf16x8, u32x4{fp8x2_bf16x2<false>(w0), fp8x2_bf16x2<true>(w0), fp8x2_bf16x2<false>(w1),
                                          fp8x2_bf16x2<true>(w1)});
}

// Workgroup barrier for LDS data: this wave's LDS accesses complete, then
// s_barrier.  Global loads in flight (the next tile) are not waited for.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits until all of this wave's vector memory operations have completed
// (its direct-to-LDS tile loads, query loads and earlier stores).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// Waits until at most N of this wave's vector memory operations are in flight
// (the N issued last may still be; vmcnt counts them in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ bf16x8 lds_b128(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// x of lanes l and l ^ 32 combined in both (v_permlane32_swap: lanes 0..31
// receive the upper half's values and give theirs, no LDS round trip as a
// ds_bpermute shuffle takes).
__device__ __forceinline__ float max_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Row of a 32x32 MFMA result held in register v of this lane.
__device__ __forceinline__ int acc_row(int v, int lane) { return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); }

template <bool DENSE>
__device__ __forceinline__ int slot_id(const int* s_list, int64_t r, int64_t r0, int64_t nvalid) {
  const int64_t rr = r < nvalid ? r : 0;  // slots past the valid ones repeat slot 0 (masked later)
  return DENSE ? static_cast<int>(r0 + rr) : s_list[rr];
}

// Direct-to-LDS loads of one 64-entry tile into buf: wave w loads rows
// 16w .. 16w+15.  Load it < 16 is non-RoPE row 16w + it (one 1 KB
// instruction, lane L fetching the chunk that belongs at slot L); loads 16
// and 17 are RoPE rows 16w .. 16w+7 and 16w+8 .. 16w+15 (8 rows x 8 chunks
// each).  my_id: lane i < 16 holds the entry id of row 16w + i.
// Dense attention over a paged cache: the rows are consecutive entries of
// sequence b (slots past the valid ones repeat the last valid entry), so the
// 16 rows of a wave lie in at most two pages (a page holds at least 64
// entries), whose table entries arrive by two scalar loads; the lane's id
// becomes its pool row.  A page outside the pool reads as page 0.
__device__ __forceinline__ int64_t page_base(const AttnParams& P, int b, int id) {
  typedef const __attribute__((address_space(4))) int32_t ctab_t;
  const int64_t ix = static_cast<int64_t>(b) * P.pg.tps + (id >> P.pg.shift);
  const int64_t pg = reinterpret_cast<ctab_t*>(reinterpret_cast<uintptr_t>(P.pg.table))[ix];
  return (pg >= 0 && pg < P.pg.pool ? pg : 0) << P.pg.shift;
}

template <bool DENSE, bool PAGED>
__device__ __forceinline__ int tile_ids(const AttnParams& P, int b, const int* s_list, int64_t rl, int64_t r0,
                                        int64_t nvalid) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t r = rl + 16 * w + (lane & 15);
  if constexpr (!DENSE || !PAGED) return slot_id<DENSE>(s_list, r, r0, nvalid);
  const int id = static_cast<int>(r0 + (r < nvalid ? r : nvalid - 1));
  const int f = __builtin_amdgcn_readlane(id, 0), l = __builtin_amdgcn_readlane(id, 15);
  const int64_t bf = page_base(P, b, f), bl = page_base(P, b, l);
  const int mask = (1 << P.pg.shift) - 1;
  return static_cast<int>(((id >> P.pg.shift) == (f >> P.pg.shift) ? bf : bl) + (id & mask));
}

// Buffer descriptor (raw, byte-addressed, 32-bit data format) over
// [base, base + bytes).  The loads go through the buffer path so that the
// compiler keeps counting LDS reads in order around them.
__device__ __forceinline__ uint32_t span(uint64_t b) { return b < 0xFFFFFFFFull ? static_cast<uint32_t>(b) : 0xFFFFFFFFu; }
// Base and size are wave-uniform; they are read back from lane 0 so that the
// descriptor is built in scalar registers even where the compiler has moved
// their arithmetic to vector registers (a descriptor it takes for divergent
// gets a loop over its distinct values around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  const int nb = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0), nb, 0x00020000);
}

// Load `it` of this wave's share of one tile.  BF16: it < 16 is non-RoPE row
// 16w + it (one 1 KB instruction, lane L fetching the chunk that belongs at
// slot L).  FP8: it < 8 is rows 16w + 2it (lanes 0..31) and 16w + 2it + 1
// (lanes 32..63), it == 10 the scales of rows 16w .. 16w+15.  Then the
// RoPE rows 16w .. 16w+7 and 16w+8 .. 16w+15 (8 rows x 8 chunks each).
template <bool FP8>
__device__ __forceinline__ void issue_load(uint8_t* buf, const AttnParams& P, int my_id, size_t seq, int it) {
  typedef __attribute__((address_space(3))) void lds_void;
  typedef Lay<FP8> L;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // rows, LDS addresses: scalar
  const uint64_t cap = static_cast<uint64_t>(P.span_rows);  // rows the descriptors cover
  if (!FP8 && it < 16) {
    const int id = __builtin_amdgcn_readlane(my_id, it);
    const int r = 16 * w + it;
    // one descriptor for the sequence's rows; the row as the scalar offset,
    // the lane's chunk (the one that belongs at slot `lane`) as the vector
    // one: 16 lane ^ 16 swz(r), the swizzle passed through a scalar so that
    // each load forms its offset with one XOR instead of keeping 16 live
    int sw = 16 * swz(r);
    asm volatile("" : "+s"(sw));
    const uint8_t* base = static_cast<const uint8_t*>(P.nope) + seq * NROW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(base, span(cap * NROW)), (lds_void*)(buf + r * NROW), 16,
                                             (16 * static_cast<int>(threadIdx.x & 63)) ^ sw, id * NROW, 0, 0);
    return;
  }
  if (FP8 && it < 8) {
    // rows 16w + 2it (lanes 0..31) and 16w + 2it + 1 (lanes 32..63).  Their
    // swizzle swzf(16w + 2it + h) = 4 (it & 3) + 2h + (w & 1), disjoint bits:
    // the chunk offset is a per-lane constant XOR a scalar
    const int ida = __builtin_amdgcn_readlane(my_id, 2 * it), idb = __builtin_amdgcn_readlane(my_id, 2 * it + 1);
    const int ln = threadIdx.x & 63;
    int sw = 64 * (it & 3);
    asm volatile("" : "+s"(sw));
    const int lf = 16 * ((ln & 31) ^ (2 * (ln >> 5)) ^ (w & 1));
    const uint8_t* base = static_cast<const uint8_t*>(P.nope) + seq * DN;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(base, span(cap * DN)), (lds_void*)(buf + (16 * w + 2 * it) * DN), 16,
                                             (ln < 32 ? ida : idb) * DN + (lf ^ sw), 0, 0, 0);
    return;
  }
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // lane offsets are recomputed per load, not kept live
  if (FP8 && it == 10) {
    const uint8_t* base = static_cast<const uint8_t*>(P.scale) + seq * 4;
    if (lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(base, span(cap * 4)), (lds_void*)(buf + L::SC_OFF + 64 * w), 4,
                                               my_id * 4, 0, 0, 0);
  } else {
    const int h = it - (FP8 ? 8 : 16);
    const int r = 16 * w + 8 * h + (lane >> 3);
    const int idr = __shfl(my_id, 8 * h + (lane >> 3));
    const uint8_t* base = static_cast<const uint8_t*>(P.rope) + seq * RROW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(base, span(cap * RROW)),
                                             (lds_void*)(buf + L::ROPE_OFF + (16 * w + 8 * h) * RROW), 16,
                                             idr * RROW + 16 * ((lane & 7) ^ swz_rope(r)), 0, 0, 0);
  }
}

// All loads of the tile at list slot rl, back to back.
template <bool FP8, bool DENSE, bool PAGED>
__device__ __forceinline__ void issue_tile(uint8_t* buf, const AttnParams& P, const int* s_list, int64_t rl,
                                           int64_t r0, int64_t nvalid, size_t seq, int b) {
  const int my_id = tile_ids<DENSE, PAGED>(P, b, s_list, rl, r0, nvalid);
#pragma unroll
  for (int it = 0; it < Lay<FP8>::NLOAD; ++it) issue_load<FP8>(buf, P, my_id, seq, it);
}

// A wave-uniform 64-bit value read back from lane 0: keeps it (and what is
// computed from it) in scalar registers where its arithmetic went through
// vector registers (the 64-bit division by m has no scalar form).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One work item: query t of sequence b, entries [r0, r1) of its list (or of
// the cache, dense) among the n visible ones.
struct Item {
  int b, t, split;
  int64_t pos, n, r0, r1;
  size_t qrow, seq;
};

template <bool DENSE, bool SPLIT>
__device__ __forceinline__ Item make_item(const AttnParams& P, int64_t it, int splits, int64_t per_split) {
  Item I;
  I.split = SPLIT ? static_cast<int>(it % splits) : 0;
  const int64_t bt = SPLIT ? it / splits : it;
  I.t = SPLIT ? 0 : static_cast<int>(bt % P.T);
  I.b = static_cast<int>(SPLIT ? bt : bt / P.T);
  // decode items take the sequence's position, prefill ones pos0 + t; kept
  // in scalar registers
  if (SPLIT || P.pos_dev) {
    // a scalar load (constant address space, uniform index): a vector load
    // here would make its wait drain every load and gather in flight
    typedef const __attribute__((address_space(4))) int64_t cpos_t;
    const int bb = __builtin_amdgcn_readfirstlane(I.b);
    I.pos = reinterpret_cast<cpos_t*>(reinterpret_cast<uintptr_t>(P.pos_dev))[bb];
  } else {
    I.pos = P.pos0 + I.t;
  }
  int64_t n = I.pos < 0 ? 0 : (I.pos + 1) / P.m;
  I.n = uniform64(n > P.cap ? P.cap : n);
  // dense: the visible entries [lo, n), lo > 0 under a sliding window; the
  // splits of a decode sequence cover them from lo on
  const int64_t lo = (DENSE && P.window > 0 && I.n > P.window) ? I.n - P.window : 0;
  const int64_t end = DENSE ? I.n : P.k;
  I.r0 = uniform64(lo + static_cast<int64_t>(I.split) * per_split);
  I.r1 = uniform64(I.r0 + per_split < end ? I.r0 + per_split : end);
  I.qrow = (static_cast<size_t>(I.b) * P.T + I.t) * NH;
  I.seq = static_cast<size_t>(I.b) * P.seq_stride;  // paged: 0 (rows are pool rows)
  return I;
}

// Item processed by workgroup g of nwg in round r.  Workgroup g runs on XCD
// g % 8; when nwg is a multiple of 8 each XCD takes nwg / 8 consecutive
// items per round, so neighbouring queries (whose lists overlap) share an L2.
__device__ __forceinline__ int64_t item_of(int g, int64_t r, int nwg) {
  if (nwg % 8) return r * nwg + g;
  return r * nwg + static_cast<int64_t>(g % 8) * (nwg / 8) + g / 8;
}

// The item's list entries r0 + tid + 256u, u < 4 (-1 past r1).
__device__ __forceinline__ void load_list(const AttnParams& P, const Item& I, int tid, int32_t (&lr)[4]) {
  const int32_t* list = P.idx + (static_cast<size_t>(I.b) * P.T + I.t) * P.k;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t r = u * NT + tid;
    lr[u] = r < I.r1 - I.r0 ? list[I.r0 + r] : -1;
  }
}

// Compacts the valid ids (0 <= id < n) of lr into s_list in list order and
// returns their count.  Two workgroup barriers.
__device__ __forceinline__ int compact_list(const int32_t (&lr)[4], int64_t n, int* s_list, int (&s_cnt)[4][NW]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  bool ok[4];
  unsigned long long bal[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ok[u] = lr[u] >= 0 && lr[u] < n;
    bal[u] = __ballot(ok[u]);
    if (lane == 0) s_cnt[u][w] = __popcll(bal[u]);
  }
  lds_sync();
  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      before += i < w ? s_cnt[u][i] : 0;
      tot += s_cnt[u][i];
    }
    if (ok[u]) s_list[base + before + __popcll(bal[u] & below)] = lr[u];
    base += tot;
  }
  lds_sync();
  return __builtin_amdgcn_readfirstlane(base);
}

// B fragment k-step s of S^T (32x32x16) for this lane: head 32hh + lane%32,
// dims 16s + 8(lane/32) .. +8.  FP8 non-RoPE k-steps come in pairs that
// share one 16-byte A read per lane: k-step s then holds dims
// 32(s/2) + 16(lane/32) + 8(s%2) .. +8 (the same permutation of k on both
// operands).
template <bool FP8>
__device__ __forceinline__ bf16x8 load_qs(const AttnParams& P, size_t qrow, int hh, int s) {
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const bf16_t* qh = static_cast<const bf16_t*>(P.q) + (qrow + 32 * hh + (lane & 31)) * CW;
  const int d = FP8 && s < DN / 16 ? 32 * (s >> 1) + 16 * half + 8 * (s & 1) : 16 * s + 8 * half;
  return *reinterpret_cast<const bf16x8*>(qh + d);
}

// The first item's query (64 heads x 576 BF16 dims, one contiguous 72 KB
// block) is staged in LDS by 72 direct loads of 1 KB, 18 per wave, each
// covering 8 head rows x 128 contiguous bytes.  Chunk group cg (dims 64cg ..
// 64cg + 63) of head row h sits at byte 8192 cg + 128 h of the free tile
// buffer (cg < 8) or at byte 128 h of the P^T buffer (cg = 8, the RoPE dims),
// its 16-byte chunk b at slot b ^ ((h >> 1) & 7): the 16 lanes of one pass
// of a fragment read (16 head rows, one chunk) then hit distinct banks.
// Loading the fragments straight from global memory instead reads 32 bytes
// of each of 32 rows per instruction, and moved four times the bytes used
// from L2 at the start of a decode item.
__device__ __forceinline__ void stage_query(const AttnParams& P, size_t qrow, uint8_t* qb, uint8_t* qr) {
  typedef __attribute__((address_space(3))) void lds_void;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint8_t* base = static_cast<const uint8_t*>(P.q) + qrow * (CW * 2);
  const auto rs = rsrc(base, NH * CW * 2);
#pragma unroll
  for (int j = 0; j < NH * CW * 2 / 1024 / NW; ++j) {
    const int blk = (NH * CW * 2 / 1024 / NW) * w + j;  // chunk group blk / 8, rows 8 (blk % 8) ..
    const int cg = blk >> 3, h = 8 * (blk & 7) + (lane >> 3);
    uint8_t* dst = cg < 8 ? qb + 8192 * cg + 1024 * (blk & 7) : qr + 1024 * (blk & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16,
                                             h * (CW * 2) + 16 * (8 * cg + ((lane & 7) ^ ((h >> 1) & 7))), 0, 0, 0);
  }
}

// B fragment k-step s (as load_qs) read from the staged query.
template <bool FP8>
__device__ __forceinline__ bf16x8 read_qs(const uint8_t* qb, const uint8_t* qr, int hh, int s) {
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int h = 32 * hh + (lane & 31);
  const int c = (FP8 && s < DN / 16 ? 32 * (s >> 1) + 16 * half + 8 * (s & 1) : 16 * s + 8 * half) >> 3;
  const int cg = c >> 3;  // the same for both lane halves
  const uint8_t* p = (cg < 8 ? qb + 8192 * cg : qr) + 128 * h + 16 * ((c & 7) ^ ((h >> 1) & 7));
  return *reinterpret_cast<const bf16x8*>(p);
}

// FP8 QK product: the query's non-RoPE dims as B operands of
// v_mfma_scale_f32_32x32x64_f8f6f4.  With 8-bit operands that MFMA's k-block
// b (b < 2, 32 k values, one E8M0 scale from lane 32b + column) is held as
// bytes 16b .. 16b+15 of both lane halves: half h holds its elements
// 16h .. 16h+15.  MFMA u (u < 8) covers dims 64u .. 64u+63 of head
// 32hh + lane%32, k-block b being MX block 2u + b.  Lane half h first rounds
// the whole MX block 2u + h to MXFP8 (OCP MX: shared exponent
// e = floor(log2 amax) - 8, elements RNE(x / 2^e) on the E4M3 grid
// saturating to +-448), then trades 16 codes with lane l ^ 32 (one
// v_permlane32_swap per dword pair): q8[u] ends as the MFMA operand, qsc[u]
// the lane's own block's E8M0 byte sb = e + 127.  amax comes from the BF16 bit patterns (|x| as
// 16-bit integers orders like the values); its exponent field E gives
// sb = E - 8, at least 0 (smaller block maxima, zero included, all take
// 2^-127).  The hardware conversion divides the BF16 pair by the fp32 scale
// 2^e exactly and rounds RNE on the OCP E4M3 grid, giving the NaN code above
// 464; NaN bytes become +-448 (0x7E / 0xFE), the saturated value.  A wave
// with a block of sb = 0 (2^-127 is not a normal fp32) takes the general
// form for that block instead: each lane multiplies by its 2^-e, clamps to
// +-448 and converts unscaled (the branch is uniform over the wave).
__device__ __forceinline__ uint32_t fp8x4_scaled(uint32_t d0, uint32_t d1, float s) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s{0, 0}, __builtin_bit_cast(bf16x2, d0), s, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, d1), s, true);
  const uint32_t w = __builtin_bit_cast(uint32_t, r);
  // bytes 0x7F / 0xFF (NaN) lose one: (w & 0x7F..) + 0x01.. sets bit 7 of
  // exactly those bytes, with no carry between bytes
  return w - ((((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) >> 7);
}
__device__ __forceinline__ uint32_t fp8x4_general(uint32_t d0, uint32_t d1, float f) {
  const float y0 = __builtin_amdgcn_fmed3f(__uint_as_float(d0 << 16) * f, -448.0f, 448.0f);
  const float y1 = __builtin_amdgcn_fmed3f(__uint_as_float(d0 & 0xFFFF0000u) * f, -448.0f, 448.0f);
  const float y2 = __builtin_amdgcn_fmed3f(__uint_as_float(d1 << 16) * f, -448.0f, 448.0f);
  const float y3 = __builtin_amdgcn_fmed3f(__uint_as_float(d1 & 0xFFFF0000u) * f, -448.0f, 448.0f);
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true));
}
__device__ __forceinline__ void load_q8(const AttnParams& P, size_t qrow, int hh, i32x8 (&q8)[8], int (&qsc)[8]) {
  const int lane = threadIdx.x & 63, half = lane >> 5;
  // 16-byte chunk 8u + 4h + c (c < 4) of the row holds block 2u + h
  const u32x4* qh =
      reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(P.q) + (qrow + 32 * hh + (lane & 31)) * CW) + 4 * half;
  u32x4 raw[8][4];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[u][c] = qh[8 * u + c];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    u16x2 mx = u16x2{0, 0};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, raw[u][c][i] & 0x7FFF7FFFu));
    const int E = static_cast<int>((mx[0] > mx[1] ? mx[0] : mx[1]) >> 7);
    const int sb = E > 8 ? E - 8 : 0;
    qsc[u] = sb;
    uint32_t c[8];  // codes of dims 4j .. 4j+3 of the lane's block: input dwords 2j, 2j + 1
    if (__builtin_amdgcn_ballot_w64(sb == 0) == 0) {
      const float sc = __uint_as_float(static_cast<uint32_t>(sb) << 23);  // 2^e
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = fp8x4_scaled(raw[u][j >> 1][2 * (j & 1)], raw[u][j >> 1][2 * (j & 1) + 1], sc);
    } else {
      const float f = __uint_as_float(static_cast<uint32_t>(254 - sb) << 23);  // 2^-e
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = fp8x4_general(raw[u][j >> 1][2 * (j & 1)], raw[u][j >> 1][2 * (j & 1) + 1], f);
    }
    // lanes < 32 (block 2u) keep codes 0..15 and take block 2u + 1's codes
    // 0..15 from lane l + 32, which keeps its codes 16..31 and takes block
    // 2u's codes 16..31
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto sw = __builtin_amdgcn_permlane32_swap(c[j], c[4 + j], false, false);
      q8[u][j] = static_cast<int>(sw[0]);
      q8[u][4 + j] = static_cast<int>(sw[1]);
    }
  }
}

// Turns the RoPE k-steps (dims 512..575, pairs (2p, 2p+1)) by position pos.
// Lane pair p = 8(s - DN/16) + 4 half + i: theta_p = r^(4 half) r^(8(s -
// DN/16)) r^i, a few fp64 products (relative error ~1e-15).
__device__ __forceinline__ void rope_q(const Theta& th, int64_t pos, bf16x8 (&qf)[QS]) {
  int half = (threadIdx.x & 63) >> 5;
  asm volatile("" : "+v"(half));  // formed per call: kept out of registers between items
  double tj = half ? th.r4 : 1.0;
#pragma unroll
  for (int s = DN / 16; s < QS; ++s) {
    u32x4 raw = __builtin_bit_cast(u32x4, qf[s]);
    if (s > DN / 16) tj *= th.r8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double theta = i == 0 ? tj : i == 1 ? tj * th.r1 : i == 2 ? tj * th.r2 : tj * th.r3;
      const double ang = static_cast<double>(pos) * theta;
      const float red = static_cast<float>(ang - rint(ang * 0.15915494309189535) * 6.283185307179586);
      const float sn = __sinf(red), cs = __cosf(red);
      const float x0 = bf16_to_f32(static_cast<bf16_t>(raw[i] & 0xFFFFu));
      const float x1 = bf16_to_f32(static_cast<bf16_t>(raw[i] >> 16));
      raw[i] = pack2_bf16(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
    }
    qf[s] = __builtin_bit_cast(bf16x8, raw);
  }
}

template <bool FP8, bool DENSE, bool SPLIT, bool PAGED, bool QK8>
__global__ void __launch_bounds__(NT, 1)
attn_bf16_kernel(AttnParams P, Theta th, int splits, int64_t per_split, void* part, int64_t nitems, int nbatch) {
  typedef Lay<FP8> L;
  __shared__ __attribute__((aligned(16))) uint8_t kb0[L::KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[L::KBUF];
  __shared__ __attribute__((aligned(16))) bf16_t pbuf[NH * PROW];
  __shared__ int s_list[DENSE ? 1 : MAX_LIST];
  __shared__ float s_xchg[2][NH];
  __shared__ float s_alpha[NH];
  __shared__ float s_m[NH];
  __shared__ int s_cnt[4][NW];
  __shared__ int s_flag[NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int eh = w & 1, hh = w >> 1;       // S^T role: entries 32eh.., heads 32hh..
  const int head = 32 * hh + (lane & 31);  // this lane's head in the S^T role
  const int half = lane >> 5;
  const int g = blockIdx.x, nwg = gridDim.x;

  int64_t round = 0;
  int64_t it = item_of(g, 0, nwg);
  if (it >= nitems) return;
  Item I = make_item<DENSE, SPLIT>(P, it, splits, per_split);
  static_assert(L::KBUF >= 8 * 8192 && sizeof(pbuf) >= NH * 128, "query staging: 64 KB + 8 KB");
  uint8_t* const qst = reinterpret_cast<uint8_t*>(pbuf);
  // split decode: the first item's query staged in LDS (kb1 and pbuf are
  // free until its first tile; sparse: its loads overlap the list's).  A
  // workgroup runs one or two such items, and this start is a large part of
  // each; prefill workgroups run many items and keep the direct loads.
  constexpr bool STAGE_Q = SPLIT && !QK8;
  int nvalid;
  if (DENSE) {
    if constexpr (STAGE_Q) stage_query(P, I.qrow, kb1, qst);
    nvalid = static_cast<int>(I.r1 > I.r0 ? I.r1 - I.r0 : 0);
  } else {
    int32_t lr[4];
    load_list(P, I, tid, lr);
    // the list's loads first: its compaction waits for them only, while the
    // query's loads (issued after them) are still landing
    if constexpr (STAGE_Q) stage_query(P, I.qrow, kb1, qst);
    nvalid = compact_list(lr, P.list_rows ? P.span_rows : I.n, s_list, s_cnt);
  }
  // the tile count is wave-uniform; read back from lane 0 so that the tile
  // loop's exit (and what it carries: buffer parity, prefetch ids) stays
  // scalar control flow
  int ntiles = __builtin_amdgcn_readfirstlane((nvalid + TILE - 1) / TILE);
  int par = 0;  // buffer of the next tile: kb0 / kb1
  // BF16 query fragments (QK8: the RoPE k-steps only, loaded directly).
  // Staged: the first tile's loads follow the query's, and the wait covers
  // the query's only (loads complete in issue order), so the tile's latency
  // runs on under the fragment reads and the RoPE turn
  constexpr int Q0 = QK8 ? DN / 16 : 0;
  bf16x8 qf[QS];
  if constexpr (STAGE_Q) __builtin_amdgcn_sched_barrier(0);
  if (ntiles > 0) issue_tile<FP8, DENSE, PAGED>(kb0, P, s_list, 0, I.r0, nvalid, I.seq, I.b);
  if constexpr (STAGE_Q) __builtin_amdgcn_sched_barrier(0);
  if constexpr (!STAGE_Q) {
#pragma unroll
    for (int s = Q0; s < QS; ++s) qf[s] = load_qs<FP8>(P, I.qrow, hh, s);
  } else {
    if (ntiles > 0) wait_vmem_but<L::NLOAD>();  // this wave's query blocks have landed
    else wait_vmem();
    lds_sync();  // and every wave's
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = read_qs<FP8>(kb1, qst, hh, s);
  }
  i32x8 q8[8];  // QK8: the non-RoPE dims as MXFP8 codes and scales (else unused)
  int qsc[8];

  // LDS byte offsets of the S^T A operand (32x32x16): row 32eh + lane%32,
  // chunk 2i + lane/32 of the non-RoPE row (BF16: k-step i, FP8: k-steps 2i
  // and 2i + 1) and of the RoPE row.  The swizzle touches the low four chunk
  // bits, so reads 8 apart differ by a constant 256 B.
  int offA[8], offR[4];
  {
    const int r = 32 * eh + (lane & 31);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // QK8: reads 2i' and 2i' + 1 of scaled MFMA i' take chunks
      // 4i' + half and 4i' + 2 + half (dims 64i' + 16half .. +16 and
      // 64i' + 32 + 16half .. +16, the lane's share of both k-blocks)
      const int c = QK8 ? 4 * (i >> 1) + half + 2 * (i & 1) : 2 * i + half;
      offA[i] = r * L::NROWB + 16 * (c ^ (FP8 ? swzf(r) : swz(r)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) offR[i] = L::ROPE_OFF + r * RROW + 16 * ((2 * i + half) ^ swz_rope(r));
  }
  // V^T operand (transposing reads): within a 16-lane group, result lane i
  // slot s is element i%4 of the 8 bytes addressed by lane 4s + i/4.  Lane
  // L = 16G + 4s + q reads entry 8(G/2) + s (+4 for the second read) of the
  // 16-entry k-step, value dims 128w + 32mb + 16(G%2) + 4q .. +4.  Rows of
  // odd k-steps (bit 4 set) have chunk bit 0 flipped: byte offset ^ 16.
  const int G = lane >> 4, sq = (lane >> 2) & 3, q4 = lane & 3;
  const int rowA = 8 * (G >> 1) + sq, rowB = rowA + 4;
  // FP8 (8-bit transposing reads): within a 16-lane group, result lane i
  // byte k is byte i%8 of the 8 bytes addressed by lane 2k + i/8.  Lane
  // L = 16G + 2k + h reads entry 8(G/2) + k of the k-step, value dims
  // 128w + 32mb + 16(G%2) + 8h .. +8: chunk 8w + 2mb + G%2, byte 8h.
  int offV[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (FP8) {
      const int k8 = (lane & 15) >> 1, h8 = lane & 1;
      const int row = 8 * (G >> 1) + k8;
      const int c = 8 * (w & 1) + 2 * mb + (G & 1);
      offV[mb][0] = row * DN + 16 * (16 * (w >> 1) + (c ^ swzf(row))) + 8 * h8;
      offV[mb][1] = 0;
    } else {
      // 16-byte chunk 16w + 4mb + 2(G%2) + q/2: high bits w, low four bits swizzled
      const int c = 4 * mb + 2 * (G & 1) + (q4 >> 1);
      offV[mb][0] = rowA * NROW + 16 * (16 * w + (c ^ swz(rowA))) + 8 * (q4 & 1);
      offV[mb][1] = rowB * NROW + 16 * (16 * w + (c ^ swz(rowB))) + 8 * (q4 & 1);
    }
  }
  const int pop = (lane & 31) * PROW + 8 * half;  // P^T B operand (elements); + 32 nb rows: heads 32nb..
  const float lscale = P.scale_qk * LOG2E;
  bool staged = false;  // an output waits in the free tile buffer
  size_t staged_qrow = 0;

  // Stores the staged output rows (16 per wave) from `buf` to rows dst +
  // h * DN: row h chunk c sits at chunk c ^ (h & 15).
  auto store_staged = [&](const uint8_t* buf, bf16_t* dst) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // lane offsets recomputed per call
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = 16 * w + i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(buf + h * NROW + 16 * (ln ^ (h & 15)));
      *reinterpret_cast<u32x4*>(dst + static_cast<size_t>(h) * DN + 8 * ln) = v;
    }
  };

  while (true) {
    // the next item: its list is read now, compacted and its first tile
    // issued at the start of this item's last tile, its query loaded behind
    // this item's last S^T MFMAs
    const int64_t itn = item_of(g, round + 1, nwg);
    const bool has_next = itn < nitems;
    const Item In = make_item<DENSE, SPLIT>(P, has_next ? itn : it, splits, per_split);
    int32_t lrn[4] = {-1, -1, -1, -1};
    if (!DENSE && has_next) load_list(P, In, tid, lrn);
    int nvalid_n = 0;
    bool next_started = false;

    if (QK8) load_q8(P, I.qrow, hh, q8, qsc);
    rope_q(th, I.pos, qf);
    // entry ids of the tile whose loads the current tile issues (read ahead)
    int my_id_pf = ntiles > 1 ? tile_ids<DENSE, PAGED>(P, I.b, s_list, TILE, I.r0, nvalid) : 0;
    f32x16 oacc[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) oacc[mb][nb] = f32x16{};
    float m_run = -INFINITY, l_part = 0.0f;

    // next item's list compacted into s_list, its first tile issued into buf
    auto start_next = [&](uint8_t* buf) {
      nvalid_n = DENSE ? static_cast<int>(In.r1 > In.r0 ? In.r1 - In.r0 : 0) : compact_list(lrn, P.list_rows ? P.span_rows : In.n, s_list, s_cnt);
      if (nvalid_n > 0) issue_tile<FP8, DENSE, PAGED>(buf, P, s_list, 0, In.r0, nvalid_n, In.seq, In.b);
      next_started = true;
    };

    // one tile.  The buffers come in as restrict pointers: the tile read,
    // the tile being loaded and P^T never overlap, and saying so lets the
    // compiler keep LDS reads (the transposing ones included) from waiting on
    // the direct-to-LDS loads in flight.
    auto tile = [&](const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt, bf16_t* __restrict__ pbuf_r,
                    int j) {
      const bool last = j + 1 == ntiles;
      // the buffer's base folded into the operand lane offsets once per tile
      // (28 adds; the reads then take the fixed base kb0 and immediates, where
      // each read would otherwise add the base itself)
      const int cb = __builtin_amdgcn_readfirstlane(static_cast<int>(cur - kb0));
      int tA[8], tR[4], tV[4][2][2];
#pragma unroll
      for (int i = 0; i < 8; ++i) { tA[i] = offA[i] + cb; asm volatile("" : "+v"(tA[i])); }
#pragma unroll
      for (int i = 0; i < 4; ++i) { tR[i] = offR[i] + cb; asm volatile("" : "+v"(tR[i])); }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int k = 0; k < (FP8 ? 1 : 2); ++k) {
          tV[mb][k][0] = offV[mb][k] + cb;
          tV[mb][k][1] = (offV[mb][k] ^ 16) + cb;
          asm volatile("" : "+v"(tV[mb][k][0]));
          asm volatile("" : "+v"(tV[mb][k][1]));
        }
      wait_vmem();
      lds_sync();  // tile j in LDS; every wave done with tile j-1 (its buffer, pbuf, s_alpha)
      if (staged) {  // the previous item's output, staged in nxt
        store_staged(nxt, static_cast<bf16_t*>(P.o) + staged_qrow * DN);
        lds_sync();
        staged = false;
      }
      // The next tile's loads (this item's tile j+1, or the next item's first
      // tile) are spread over this tile's MFMAs (a wave that issues them back
      // to back stalls until the memory pipeline takes them), none in the
      // softmax, whose VALU work would wait behind them: most in the S^T
      // MFMAs, the rest early in PV (the split measured best per format).
      // Every tile issues all of them, without branches in the MFMA loops;
      // with no next tile they re-read the current item's first entry into
      // the free buffer.
      int my_id = 0;
      size_t lseq = I.seq;
      if (!last) {
        my_id = my_id_pf;
      } else if (has_next) {
        nvalid_n = DENSE ? static_cast<int>(In.r1 > In.r0 ? In.r1 - In.r0 : 0) : compact_list(lrn, P.list_rows ? P.span_rows : In.n, s_list, s_cnt);
        next_started = true;
        if (nvalid_n > 0) {
          my_id = tile_ids<DENSE, PAGED>(P, In.b, s_list, 0, In.r0, nvalid_n);
          lseq = In.seq;
        }
      }

      // --- S^T = K Q^T: entries 32eh.. x heads 32hh.. ------------------------
      // A operands run SPF k-steps ahead of the MFMAs (scheduling barriers
      // keep that order); in the item's last tile the query fragments are
      // reloaded for the next item right after their last use
      // one A read per unit: BF16 36 units of one k-step; FP8 16 units of two
      // non-RoPE k-steps (16 codes widened in registers) and 4 RoPE k-steps
      constexpr int NU = FP8 ? DN / 32 + DRP / 16 : QS;
      constexpr int NUN = FP8 ? DN / 32 : DN / 16;  // non-RoPE units
      auto aop = [&](int u) -> u32x4 {
        return u < NUN ? *reinterpret_cast<const u32x4*>(kb0 + tA[u & 7] + 256 * (u >> 3))
                       : *reinterpret_cast<const u32x4*>(kb0 + tR[u - NUN]);
      };
      f32x16 sacc = f32x16{};
      f32x16 sacr = f32x16{};  // FP8: the RoPE part, unscaled
      {
        u32x4 ring[SPF];
        u32x4 a_lo = u32x4{};  // QK8: the first half of a scaled MFMA's A operand
#pragma unroll
        for (int u = 0; u < SPF; ++u) ring[u] = aop(u);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const u32x4 a = ring[u % SPF];
          if (u + SPF < NU) ring[u % SPF] = aop(u + SPF);
          if (QK8 && u < NUN) {
            // codes in as stored (scale 2^0), the query's block scale from
            // its E8M0 byte; the entry's fp32 scale follows on the sum
            if (u & 1) {
              const i32x8 a8 = __builtin_bit_cast(i32x8, __builtin_shufflevector(a_lo, a, 0, 1, 2, 3, 4, 5, 6, 7));
              sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, q8[u >> 1], sacc, 0, 0, 0, 127, 0,
                                                                     qsc[u >> 1]);
              // keeps the compiler from sinking the scaled MFMAs to the
              // end of the loop, away from the loads they hide
              asm volatile("" : "+v"(sacc));
            } else {
              a_lo = a;
            }
          } else if (FP8 && u < NUN) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_bf16(a[0], a[1]), qf[2 * u], sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_bf16(a[2], a[3]), qf[2 * u + 1], sacc, 0, 0, 0);
          } else if (FP8) {
            sacr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[DN / 16 + u - NUN], sacr, 0,
                                                           0, 0);
          } else {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[u], sacc, 0, 0, 0);
          }
          // loads 0..11 (BF16), 0..9 (FP8), 0..6 (QK8)
          if (QK8 ? u % 3 == 1 : FP8 ? u % 2 == 1 : u % 3 == 1)
            issue_load<FP8>(nxt, P, my_id, lseq, QK8 ? u / 3 : FP8 ? u / 2 : u / 3);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (last && has_next) {
#pragma unroll
        for (int s = Q0; s < QS; ++s) qf[s] = load_qs<FP8>(P, In.qrow, hh, s);
      }
      // FP8: S = scale_e (q . codes_e) + (q_rope . k_rope_e); P^T carries the
      // scale into O (the V rows in LDS are unscaled codes)
      float esc[16];
      if (FP8) {
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const float4 sc = *reinterpret_cast<const float4*>(cur + L::SC_OFF + 4 * (32 * eh + 8 * jq + 4 * half));
          esc[4 * jq] = sc.x;
          esc[4 * jq + 1] = sc.y;
          esc[4 * jq + 2] = sc.z;
          esc[4 * jq + 3] = sc.w;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[v] = sacc[v] * esc[v] + sacr[v];
      }

      // --- softmax: lane holds entries 32eh + acc_row(v) of its head ---------
      // P = exp2(S - m_run) with the running reference m_run of the head,
      // which both entry halves hold alike.  While no score of the tile
      // exceeds m_run + 8 (P < 256) no wave needs the other half's maximum,
      // so one barrier (P^T written) serves the tile.  Otherwise (the first
      // tile of an item, or a jump of the maximum) a wave flags it, and after
      // that barrier all waves agree on the new reference from the maxima
      // they published, rewrite P^T, rescale l and O^T, and meet once more.
      // the scores stay unscaled: the positive scale commutes with the max,
      // and exp2 takes fma(s, scale, -m)
      const int vend = nvalid - j * TILE;  // entries of this tile below it are real
      if (vend < TILE) {  // an item's last tile: entries past the list are masked
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int e = 32 * eh + acc_row(v, lane);
          sacc[v] = e < vend ? sacc[v] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
      mx = max_xor32(mx) * lscale;
      if (lane < 32) s_xchg[eh][head] = mx;
      const bool bad = m_run == -INFINITY || !(mx <= m_run + 8.0f);
      const bool wave_bad = __ballot(bad) != 0ull;
      if (lane == 0) s_flag[w] = wave_bad ? 1 : 0;
      auto write_p = [&]() -> float {
        float ps = 0.0f;
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[4 * jq], lscale, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[4 * jq + 1], lscale, -m_run));
          const float p2 = __builtin_amdgcn_exp2f(fmaf(sacc[4 * jq + 2], lscale, -m_run));
          const float p3 = __builtin_amdgcn_exp2f(fmaf(sacc[4 * jq + 3], lscale, -m_run));
          ps += (p0 + p1) + (p2 + p3);
          const float f0 = FP8 ? esc[4 * jq] : 1.0f, f1 = FP8 ? esc[4 * jq + 1] : 1.0f;
          const float f2 = FP8 ? esc[4 * jq + 2] : 1.0f, f3 = FP8 ? esc[4 * jq + 3] : 1.0f;
          *reinterpret_cast<uint2*>(pbuf_r + head * PROW + 32 * eh + 8 * jq + 4 * half) =
              make_uint2(pack2_bf16(p0 * f0, p1 * f1), pack2_bf16(p2 * f2, p3 * f3));
        }
        return ps;
      };
      float psum = 0.0f;
      if (!wave_bad) psum = write_p();
      lds_sync();
      if (s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) {
        const float mall = fmaxf(mx, s_xchg[eh ^ 1][head]);
        const bool move = m_run == -INFINITY || mall > m_run + 8.0f;
        const float alpha = move && m_run != -INFINITY ? exp2f(m_run - mall) : 1.0f;
        if (move) m_run = mall;
        l_part *= alpha;
        if (eh == 0 && lane < 32) s_alpha[head] = alpha;
        psum = write_p();
        lds_sync();
        if (j > 0) {  // an item's first tile starts from m_run = -inf: alpha = 1, O^T = 0
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const float a = s_alpha[32 * nb + (lane & 31)];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) oacc[mb][nb] *= a;
          }
        }
      }
      l_part += psum;

      // --- O^T += V^T P^T: value dims 128w.. x all 64 heads ---------------------
      // 16 steps (ks, mb): V^T operands run PPF steps ahead of the MFMAs,
      // P^T operands one k-step ahead
      {
        typedef __attribute__((address_space(3))) v4s lds_v4s;
        constexpr int PPF = 4;
        // one V^T operand per step: BF16 two 16-bit transposing reads, FP8
        // one 8-bit transposing read widened in registers
        typedef int v2i __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) v2i lds_v2i;
        struct VOp {
          v4s x, y;
        };
        auto vop = [&](int t) -> VOp {
          const int ks = t >> 2, mb = t & 3;
          VOp r;
          if (FP8) {
            const v2i c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(kb0 + tV[mb][0][ks & 1] + 16 * ks * DN));
            r.x = __builtin_bit_cast(v4s, c);
            r.y = r.x;
          } else {
            r.x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(kb0 + tV[mb][0][ks & 1] + 16 * ks * NROW));
            r.y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(kb0 + tV[mb][1][ks & 1] + 16 * ks * NROW));
          }
          return r;
        };
        auto vval = [&](const VOp& o) -> bf16x8 {
          if (FP8) {
            const v2i c = __builtin_bit_cast(v2i, o.x);
            return fp8x8_bf16(static_cast<uint32_t>(c[0]), static_cast<uint32_t>(c[1]));
          }
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(o.x, o.y, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        auto pop_ks = [&](int ks, int nb) -> bf16x8 {
          return *reinterpret_cast<const bf16x8*>(pbuf_r + pop + 32 * nb * PROW + 16 * ks);
        };
        VOp vr[PPF];
        bf16x8 pbr[2][2];
        pbr[0][0] = pop_ks(0, 0);
        pbr[0][1] = pop_ks(0, 1);
#pragma unroll
        for (int t = 0; t < PPF; ++t) vr[t] = vop(t);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int ks = t >> 2;
          const bf16x8 va = vval(vr[t % PPF]);
          if (t + PPF < 16) vr[t % PPF] = vop(t + PPF);
          if ((t & 3) == 0 && ks + 1 < 4) {
            pbr[(ks + 1) & 1][0] = pop_ks(ks + 1, 0);
            pbr[(ks + 1) & 1][1] = pop_ks(ks + 1, 1);
          }
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            oacc[t & 3][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pbr[ks & 1][nb], oacc[t & 3][nb], 0, 0, 0);
          // loads 12..17 (BF16), 10 (FP8), 7..10 (QK8)
          if (QK8 ? t % 4 == 1 : FP8 ? t == 1 : t % 2 == 1 && t < 12)
            issue_load<FP8>(nxt, P, my_id, lseq, QK8 ? 7 + t / 4 : FP8 ? 10 : 12 + t / 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    for (int j = 0; j < ntiles; ++j) {
      tile(par ? kb1 : kb0, par ? kb0 : kb1, pbuf, j);
      if (j + 2 < ntiles) my_id_pf = tile_ids<DENSE, PAGED>(P, I.b, s_list, static_cast<int64_t>(j + 2) * TILE, I.r0, nvalid);
      par ^= 1;
    }

    // --- finish: denominators and maxima to LDS, then each wave its O^T ----
    l_part = sum_xor32(l_part);
    lds_sync();  // every wave done with the last tile: its buffer is free
    if (lane < 32) s_xchg[eh][head] = l_part;
    if (eh == 0 && lane < 32) s_m[head] = m_run;
    lds_sync();
    uint8_t* stage = par ? kb0 : kb1;  // not the buffer of the next item's first tile
    // O^T block (mb, nb): lane = head 32nb + lane%32, register v = value dim
    // 128w + 32mb + acc_row(v)
    // partials of a decode split: normalised BF16 rows [B][splits][NH][DN],
    // then the log2-sum-exp per head, fp32 [B][splits][NH]
    // partials of a split sequence go straight from registers in
    // their own layout: piece (w, mb, nb, jq) of 64 lanes x 8 bytes at
    // 512 ((((w * 4 + mb) * 2 + nb) * 4 + jq)) + 8 lane, lane holding head
    // 32nb + lane % 32, dims 128w + 32mb + 8jq + 4 (lane / 32) .. +4; the merge
    // reads them in that order.  No LDS staging, no barrier before the stores.
    const size_t slot = static_cast<size_t>(I.b) * splits + I.split;
    bf16_t* part_o = static_cast<bf16_t*>(part);
    float* part_lse = reinterpret_cast<float*>(part_o + static_cast<size_t>(nbatch) * splits * (NH * DN));
    constexpr bool native = SPLIT;  // a split launch always has splits > 1
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int h = 32 * nb + (lane & 31);
      const float ltot = s_xchg[0][h] + s_xchg[1][h];
      const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x16& o = oacc[mb][nb];
          const uint32_t lo = pack2_bf16(o[4 * jq] * inv, o[4 * jq + 1] * inv);
          const uint32_t hi2 = pack2_bf16(o[4 * jq + 2] * inv, o[4 * jq + 3] * inv);
          if constexpr (native) {
            *reinterpret_cast<uint2*>(part_o + slot * (NH * DN) + 4 * ((((w * 4 + mb) * 2 + nb) * 4 + jq) * 64 + lane)) =
                make_uint2(lo, hi2);
          } else {
            // dims 128w + 32mb + 8jq + 4half: chunk 16w + 4mb + jq, byte 8half
            const int c = 16 * w + 4 * mb + jq;
            *reinterpret_cast<uint2*>(stage + h * NROW + 16 * (c ^ (h & 15)) + 8 * half) = make_uint2(lo, hi2);
          }
        }
      if (w == 0 && lane < 32) {
        const float l2 = ltot > 0.0f ? s_m[h] + log2f(ltot) : -INFINITY;
        if (SPLIT) part_lse[slot * NH + h] = l2;
        else if (P.lse) P.lse[I.qrow + h] = l2 * LN2;
      }
    }
    // the output stays staged until the next item's first tile has landed,
    // when there is one; else (and for split partials) it is stored now
    const bool defer = !SPLIT && has_next && next_started && nvalid_n > 0;
    staged_qrow = I.qrow;
    if (!defer && !native) {
      lds_sync();  // every wave's part of the rows written
      store_staged(stage, static_cast<bf16_t*>(P.o) + staged_qrow * DN);
    }
    if (!has_next) break;
    if (!next_started) {  // this item had no tile: start the next one now
      wait_vmem();  // earlier loads into the free buffers have landed
      if (par == 0) start_next(kb0);
      else start_next(kb1);
#pragma unroll
      for (int s = Q0; s < QS; ++s) qf[s] = load_qs<FP8>(P, In.qrow, hh, s);
    }
    staged = defer;
    I = In;
    it = itn;
    nvalid = __builtin_amdgcn_readfirstlane(nvalid_n);
    ntiles = __builtin_amdgcn_readfirstlane((nvalid + TILE - 1) / TILE);
    ++round;
  }
  wait_vmem();  // no load into this workgroup's LDS outlives it
}

}  // namespace

// One persistent workgroup per compute unit (at most one item each when the
// items are fewer).
void launch_attn_bf16(const AttnParams& P, bool dense, int B, hipStream_t s, int splits, int64_t per, void* part) {
  // compute units per device, looked up once; concurrent first calls store
  // the same value
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int cu = cus[dev & 63].load(std::memory_order_relaxed);
  if (cu == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cu = v;
    cus[dev & 63].store(cu, std::memory_order_relaxed);
  }
  Theta th;
  th.r1 = std::pow(P.base, -2.0 / DRP);
  th.r2 = std::pow(P.base, -4.0 / DRP);
  th.r3 = std::pow(P.base, -6.0 / DRP);
  th.r4 = std::pow(P.base, -8.0 / DRP);
  th.r8 = std::pow(P.base, -16.0 / DRP);
  const bool split = part != nullptr;
  const int64_t nitems = static_cast<int64_t>(B) * (split ? splits : P.T);
  if (nitems <= 0) return;
  const dim3 grid(static_cast<unsigned>(nitems < cu ? nitems : cu));
  const bool fp8 = P.nope_dt == CSA_FP8E4M3;
  // paged caches need a kernel of their own only for dense attention (sparse
  // lists arrive as pool rows)
  const bool paged = dense && P.pg.table != nullptr;
#define CSA_ATTN_LAUNCH(F, D, S, G) \
  hipLaunchKernelGGL((attn_bf16_kernel<F, D, S, G, false>), grid, dim3(NT), 0, s, P, th, splits, per, part, nitems, B)
#define CSA_ATTN_LAUNCH8(D, S, G) \
  hipLaunchKernelGGL((attn_bf16_kernel<true, D, S, G, true>), grid, dim3(NT), 0, s, P, th, splits, per, part, nitems, B)
  if (fp8 && P.qk_mode == CSA_FP8E4M3) {
    if (dense) {
      if (paged) {
        if (split) CSA_ATTN_LAUNCH8(true, true, true);
        else CSA_ATTN_LAUNCH8(true, false, true);
      } else {
        if (split) CSA_ATTN_LAUNCH8(true, true, false);
        else CSA_ATTN_LAUNCH8(true, false, false);
      }
    } else {
      if (split) CSA_ATTN_LAUNCH8(false, true, false);
      else CSA_ATTN_LAUNCH8(false, false, false);
    }
  } else if (fp8) {
    if (dense) {
      if (paged) {
        if (split) CSA_ATTN_LAUNCH(true, true, true, true);
        else CSA_ATTN_LAUNCH(true, true, false, true);
      } else {
        if (split) CSA_ATTN_LAUNCH(true, true, true, false);
        else CSA_ATTN_LAUNCH(true, true, false, false);
      }
    } else {
      if (split) CSA_ATTN_LAUNCH(true, false, true, false);
      else CSA_ATTN_LAUNCH(true, false, false, false);
    }
  } else {
    if (dense) {
      if (paged) {
        if (split) CSA_ATTN_LAUNCH(false, true, true, true);
        else CSA_ATTN_LAUNCH(false, true, false, true);
      } else {
        if (split) CSA_ATTN_LAUNCH(false, true, true, false);
        else CSA_ATTN_LAUNCH(false, true, false, false);
      }
    } else {
      if (split) CSA_ATTN_LAUNCH(false, false, true, false);
      else CSA_ATTN_LAUNCH(false, false, false, false);
    }
  }
#undef CSA_ATTN_LAUNCH
#undef CSA_ATTN_LAUNCH8
}

}  // namespace csa
