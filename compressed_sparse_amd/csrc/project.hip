// Compressor inputs projected from hidden states and compressed in one
// kernel.  [读完这篇] §三 压缩机制: the compressor's learnable parameters are
// four projection matrices W^{aKV}, W^{bKV}, W^{aZ}, W^{bZ} and two biases
// B^a, B^b; [CSA/HCA 混注意力] §1.1 工程细节 (entry i mixes window i's C^a rows
// and window i-1's C^b rows), §1.2 (HCA: one window of m' tokens).
//
//   Y[t][j*NT + u] = sum_k X[t][k] W[j*NT + u][k]      (u: a, za, b, zb)
//   entry i, channel j = the compressor's softmax over the window rows of Y
//
// project_gemm_kernel: one workgroup computes a 256-token x 256-column tile of
// Y (128 columns when the projected width needs it) with
// v_mfma_f32_32x32x16_bf16, 4 waves of 128 x 128 (x 64); both operands are
// read by 16-byte buffer loads into registers two K steps ahead and written
// to one of two LDS buffers one step ahead (64-wide K steps, the loads and
// writes spread over the MFMA stream), the 16-byte chunks of each 128-byte
// row XOR-swizzled by the row.  Columns of a
// tile are the NT projections of consecutive channels, so the
// epilogue finds every input of its entries' channels in the tile: Y goes to
// LDS in 64-column passes (fp32, never rounded) and each (entry, channel) runs the compressor's
// softmax over its window rows (overlapped tiles start one window early, so
// window i-1 is in the tile; the call's first window reads it from the
// staging ring).  Entry values (fp32, before RoPE) go to the workspace, with
// the rows of the call's last tokens; project_finalize_kernel turns and
// stores the entries like the compressor, project_ring_kernel refreshes the
// ring.  The GEMM dominates: 2 * d_model flop per token and column.
#include <type_traits>

#include "compress_store.hpp"

namespace csa {
namespace {

constexpr int PT_M = 256;  // tokens per tile
constexpr int PT_K = 64;   // K per LDS stage
constexpr int PT_G = 64;   // columns per epilogue pass
constexpr int PNT = 256;   // threads

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct ProjParams {
  CompressParams C;   // cache, formats, m, NT, c, biases (C.Ba, C.Bb), ring
  const bf16_t* X;    // [B][T][d] hidden states
  const bf16_t* W;    // [NT * c][d] projection rows
  int d, T;
  int64_t pos0;
  int64_t E0;         // first entry of the call (pos0 / m)
  int64_t n_ent;      // entries the call completes
  int wpt;            // entries per token tile
  int ovl;            // overlapped: tiles start one window early
  int n_mt, n_nt;     // token tiles, column tiles
  int64_t t_first;    // first token whose row the ring keeps
  float* went;        // [B][n_ent][c] entry values before RoPE
  float* wring;       // [B][R][NT][c] rows of tokens t_first ..
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t prsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// Row of a 32x32 MFMA result held in register v of this lane.
__device__ __forceinline__ int acc_row(int v, int lane) { return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); }

// Tile: 256 tokens x TN columns; wave (wm, wn) owns rows 128 wm .. and
// columns (TN / 2) wn .., 4 x TN/64 MFMA blocks of 32 x 32 (accumulators in
// AGPRs).  K runs in 64-wide stages through two LDS buffers: a stage's rows
// (128 bytes each) are read from memory into registers one stage ahead (16
// bytes per lane, 8 lanes per row, so each load instruction reads 8 whole
// cache lines; rows outside the sequence read as zero through the buffer
// descriptor's range), then written to LDS while the previous stage's MFMAs
// are done.  Chunk c of row r sits in slot c ^ ((r / 2) % 8): two 128-byte
// rows share a line of the 64 banks, so the 16 lanes of a 16-byte access
// (16 consecutive rows, or two rows' 8 chunks) hit distinct banks.  (Direct-to-LDS loads of these 8-row pieces ran at about a
// third of this rate.)
constexpr int PK = 64;  // K per stage

// Workgroup barrier for LDS data: this wave's LDS accesses complete, then
// s_barrier.  Unlike __syncthreads() it does not wait for the wave's global
// loads in flight (the next stage's rows).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

template <int TN>
__device__ __forceinline__ void project_gemm_body(const ProjParams& P) {
  constexpr int STA = PT_M * PK * 2, STB = TN * PK * 2;  // stage bytes
  constexpr int MB = 4, NB = TN / 64;                     // blocks per wave
  constexpr int LA = 8, LB = TN / 32;                     // row loads per lane and stage (8 rows per instruction)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (STA + STB)];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.z;
  // tiles in N-fastest order; each XCD (workgroup g runs on XCD g % 8)
  // takes a contiguous run of them, so the column tiles of one token tile
  // share its hidden rows in one L2 (the grid is padded to a multiple of 8;
  // padding workgroups exit)
  const int total = P.n_mt * P.n_nt;
  const int g = blockIdx.x;
  const int tile = (g % 8) * ((total + 7) / 8) + g / 8;
  if (tile >= total) return;
  const int mt = tile / P.n_nt, nt = tile % P.n_nt;
  const int m = P.C.m, NT = P.C.NT, c = P.C.c;
  const int64_t win0 = P.E0 + static_cast<int64_t>(mt) * P.wpt - P.ovl;  // window of the tile's row 0
  const int64_t t0 = win0 * m;                                             // token of row 0
  const int n0 = nt * TN;

  const auto rx = prsrc(P.X + static_cast<size_t>(b) * P.T * P.d, static_cast<uint32_t>(static_cast<size_t>(P.T) * P.d * 2));
  const auto rw = prsrc(P.W, static_cast<uint32_t>(static_cast<size_t>(NT) * c * P.d * 2));
  uint8_t* const sA0 = smem;
  uint8_t* const sB0 = smem + 2 * STA;

  // load i of this wave: rows 64w + 8i + lane / 8 (A) and (TN / 4) w + 8i +
  // lane / 8 (B), chunk lane % 8; stored at slot (lane % 8) ^ (row / 2 % 8)
  const int ch = lane & 7;
  // slot of this lane's chunk in the rows of load i (8i + lane / 8 modulo 16)
  auto slotw = [&](int i) { return 16 * (ch ^ (((8 * i + (lane >> 3)) >> 1) & 7)); };
  uint32_t voA[LA], voB[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int row = 64 * w + 8 * i + (lane >> 3);
    const int64_t tr = t0 + row - P.pos0;
    voA[i] = (tr >= 0 && tr < P.T) ? static_cast<uint32_t>((tr * P.d + ch * 8) * 2) : 0x80000000u;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int row = (TN / 4) * w + 8 * i + (lane >> 3);
    voB[i] = static_cast<uint32_t>((static_cast<int64_t>(n0 + row) * P.d + ch * 8) * 2);
  }
  u32x4v ra[LA], rb[LB];
  auto gload = [&](int ks) {
    const int soff = ks * PK * 2;
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rx, voA[i], soff, 0));
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rw, voB[i], soff, 0));
  };
  auto swrite = [&](int p) {
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *reinterpret_cast<u32x4v*>(sA0 + p * STA + (64 * w + 8 * i + (lane >> 3)) * 128 + slotw(i)) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<u32x4v*>(sB0 + p * STB + ((TN / 4) * w + 8 * i + (lane >> 3)) * 128 + slotw(i)) = rb[i];
  };

  // Operand reads: row r = base + 32 blk + lane % 32 (r / 2 % 8 = lane % 32
  // / 2 % 8), k step s: chunk 2s + lane / 32 at slot chunk ^ (r / 2 % 8)
  const int wm = w >> 1, wn = w & 1, half = lane >> 5, sx = ((lane & 31) >> 1) & 7;
  const int rowA = 128 * wm + (lane & 31), rowB = (TN / 2) * wn + (lane & 31);
  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  const int S = P.d / PK;
  gload(0);
  swrite(0);
  if (S > 1) gload(1);
  lds_sync();
  // per stage: LA + LB pieces, each the LDS write of one register of the
  // next stage's rows (loaded during the previous stage) followed by that
  // register's load for the stage after next, spread evenly over the stage's
  // MFMAs so that neither the writes nor the load issue hold up the MFMA
  // stream; the other buffer is free, every wave having finished its
  // previous stage before the last barrier
  constexpr int NPC = LA + LB;                      // pieces per stage
  constexpr int NMF = (PK / 16) * MB * NB;          // MFMAs per stage
  constexpr int EVERY = NMF / NPC;                  // MFMAs between pieces
  static_assert(EVERY >= 1, "a piece per MFMA at most");
  // one stage; WR: write the next stage's rows, LD: load the stage after
  // next (compile-time, so that no branch splits the MFMA stream)
  auto stage = [&](int ks, auto wr_tag, auto ld_tag) {
    constexpr bool WR = decltype(wr_tag)::value, LD = decltype(ld_tag)::value;
    const uint8_t* a = sA0 + (ks & 1) * STA + rowA * 128;
    const uint8_t* bb = sB0 + (ks & 1) * STB + rowB * 128;
    const int pw = (ks + 1) & 1, soff2 = (ks + 2) * PK * 2;
    auto piece = [&](int q) {
      if (q < LA) {
        *reinterpret_cast<u32x4v*>(sA0 + pw * STA + (64 * w + 8 * q + (lane >> 3)) * 128 + slotw(q)) = ra[q];
        if (LD) ra[q] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rx, voA[q], soff2, 0));
      } else {
        const int i = q - LA;
        *reinterpret_cast<u32x4v*>(sB0 + pw * STB + ((TN / 4) * w + 8 * i + (lane >> 3)) * 128 + slotw(i)) = rb[i];
        if (LD) rb[i] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rw, voB[i], soff2, 0));
      }
    };
    // k step s + 1's operands are read before k step s's MFMAs (scheduling
    // barriers keep that order), hiding the reads behind MFMAs
    bf16x8 fa[2][MB], fb[2][NB];
    auto read = [&](int s) {
      const int slot = 16 * ((2 * s + half) ^ sx);
#pragma unroll
      for (int i = 0; i < MB; ++i) fa[s & 1][i] = *reinterpret_cast<const bf16x8*>(a + i * 32 * 128 + slot);
#pragma unroll
      for (int j = 0; j < NB; ++j) fb[s & 1][j] = *reinterpret_cast<const bf16x8*>(bb + j * 32 * 128 + slot);
    };
    read(0);
#pragma unroll
    for (int s = 0; s < PK / 16; ++s) {
      if (s + 1 < PK / 16) read(s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][i], fb[s & 1][j], acc[i][j], 0, 0, 0);
          const int f = (s * MB + i) * NB + j;  // MFMA index within the stage
          if (WR && f % EVERY == EVERY - 1 && f / EVERY < NPC) {
            piece(f / EVERY);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (WR) lds_sync();  // the writes are visible and every wave is done with stage ks
  };
  typedef std::integral_constant<bool, true> yes;
  typedef std::integral_constant<bool, false> no;
  for (int ks = 0; ks + 2 < S; ++ks) stage(ks, yes(), yes());
  if (S >= 2) stage(S - 2, yes(), no());
  stage(S - 1, no(), no());
  __syncthreads();  // every wave done with the stage buffers

  // ---- epilogue, in passes of 64 columns (16 or 32 channels) ------------
  // Pass q: the waves owning columns 64q .. write them to LDS as fp32 [256]
  // [64]; then every (entry, channel) of those columns runs the compressor's
  // softmax over its window rows, and the ring's rows are staged.
  float* sY = reinterpret_cast<float*>(smem);
  // the pass's biases, [m][channels] each, after the Y columns
  float* sBa = sY + PT_M * PT_G;
  float* sBb = sBa + 128 * (PT_G / 2);
  const int nwin = PT_M / m, own = nwin - P.ovl;
  const int64_t t_end = P.pos0 + P.T;
  const int own0 = P.ovl * m;
  // the ring keeps rows of this tile (its last token tile) or not at all
  const bool ring_rows = t0 + PT_M > P.t_first && t0 + own0 < t_end;
#pragma unroll
  for (int q = 0; q < TN / PT_G; ++q) {
    if (wn == (q * PT_G) / (TN / 2)) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int col = (TN / 2) * wn + 32 * j - q * PT_G;  // column of block j within the pass
        if (col < 0 || col >= PT_G) continue;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            sY[(128 * wm + 32 * i + acc_row(v, lane)) * PT_G + col + (lane & 31)] = acc[i][j][v];
      }
    }
    const int chans = PT_G / NT, j0 = (n0 + q * PT_G) / NT;
    for (int x = tid; x < m * chans; x += PNT) {
      const int r = x / chans, jj = x % chans;
      sBa[x] = P.C.Ba[r * c + j0 + jj];
      if (P.ovl) sBb[x] = P.C.Bb[r * c + j0 + jj];
    }
    __syncthreads();
    for (int task = tid; task < own * chans; task += PNT) {
      const int lw = P.ovl + task / chans, jj = task % chans, j = j0 + jj;
      const int64_t e = win0 + lw;  // the entry of local window lw
      if (e - P.E0 >= P.n_ent) continue;
      // window rows in the compressor's order: C^a rows of window e, then the
      // C^b rows of window e-1 (tile rows, or ring rows when that window
      // precedes the call), in batches of CW_ROWS
      const bool prev = P.ovl && e >= 1;
      const bool prev_ring = prev && (e - 1) * m < P.pos0;
      const int nrow = m + (prev ? m : 0);
      float mx = -INFINITY, sw = 0.0f, ac = 0.0f;
      for (int r0 = 0; r0 < nrow; r0 += CW_ROWS) {
        float lg[CW_ROWS], vv[CW_ROWS];
#pragma unroll
        for (int u = 0; u < CW_ROWS; ++u) {
          const int rho = min(r0 + u, nrow - 1);
          const bool sa = rho < m;
          const int r = sa ? rho : rho - m;
          float z, x;
          if (sa) {
            const float* yr = sY + (lw * m + r) * PT_G + jj * NT;
            z = yr[RING_ZA] + sBa[r * chans + jj];
            x = yr[RING_A];
          } else if (prev_ring) {
            const int64_t t = (e - 1) * m + r;
            const float* rr = P.C.ring + ((static_cast<size_t>(b) * P.C.R + t % P.C.R) * NT) * c;
            z = rr[RING_ZB * c + j] + sBb[r * chans + jj];
            x = rr[RING_B * c + j];
          } else {
            const float* yr = sY + ((lw - 1) * m + r) * PT_G + jj * NT;
            z = yr[RING_ZB] + sBb[r * chans + jj];
            x = yr[RING_B];
          }
          lg[u] = r0 + u < nrow ? z : -INFINITY;
          vv[u] = x;
        }
        softmax_batch(lg, vv, mx, sw, ac);
      }
      P.went[(static_cast<size_t>(b) * P.n_ent + (e - P.E0)) * c + j] = ac / sw;
    }
    // rows of the tokens the ring keeps (the tile's own rows only)
    for (int qq = tid; ring_rows && qq < (PT_M - own0) * PT_G; qq += PNT) {
      const int row = own0 + qq / PT_G, col = qq % PT_G;
      const int64_t t = t0 + row;
      if (t < P.t_first || t >= t_end) continue;
      const int n = n0 + q * PT_G + col;
      P.wring[((static_cast<size_t>(b) * P.C.R + (t - P.t_first)) * NT + n % NT) * c + n / NT] = sY[row * PT_G + col];
    }
    __syncthreads();
  }
}

template <int TN>
__global__ void __launch_bounds__(PNT) __attribute__((amdgpu_waves_per_eu(1))) project_gemm_kernel(ProjParams P) {
  project_gemm_body<TN>(P);
}

// RoPE and storage of the call's entries from their fp32 values, with the
// compressor's own lane map and epilogue (so the codes follow the same
// rules): a group of lanes per entry, lane l holding channels 8l .. 8l+7 and
// RoPE pair l.
__global__ void __launch_bounds__(256) project_finalize_kernel(ProjParams P) {
  const CompressParams& C = P.C;
  const int lane = threadIdx.x & 63, b = blockIdx.y;
  const int ng = C.d_nope / 8, np = C.d_rope / 2;
  const int lpe = wave_lanes_per_entry(ng, np), epw = 64 / lpe, ll = lane & (lpe - 1);
  const int64_t e0 = (4 * static_cast<int64_t>(blockIdx.x) + (threadIdx.x >> 6)) * epw;
  if (e0 >= P.n_ent) return;
  const int64_t e = e0 + lane / lpe;
  const bool ok = e < P.n_ent;
  const bool hg = ok && ll < ng, hp = ok && ll < np;
  const float* src = P.went + (static_cast<size_t>(b) * P.n_ent + (ok ? e : 0)) * C.c;
  float x[10];
#pragma unroll
  for (int q = 0; q < 10; ++q) x[q] = 0.0f;
  if (hg) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(src + 8 * ll);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 8 * ll + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) { x[q] = v0[q]; x[4 + q] = v1[q]; }
  }
  if (hp) { x[8] = src[C.d_nope + 2 * ll]; x[9] = src[C.d_nope + 2 * ll + 1]; }
  store_entry_lanes(C, b, P.E0 + e, ok, hg, hp, ll, lpe, x);
}

// The ring's rows of tokens t_first .. pos0 + T - 1 (slot t mod R).
__global__ void __launch_bounds__(256) project_ring_kernel(ProjParams P) {
  const int b = blockIdx.y;
  const int64_t t = P.t_first + blockIdx.x;
  const int n = P.C.NT * P.C.c;
  const float* src = P.wring + (static_cast<size_t>(b) * P.C.R + (t - P.t_first)) * n;
  float* dst = P.C.ring + (static_cast<size_t>(b) * P.C.R + t % P.C.R) * n;
  for (int q = threadIdx.x; q < n; q += blockDim.x) dst[q] = src[q];
}

void launch_project_gemm(const ProjParams& P, int TN, dim3 grid, hipStream_t s) {
  if (TN == 256) hipLaunchKernelGGL(project_gemm_kernel<256>, grid, dim3(PNT), 0, s, P);
  else hipLaunchKernelGGL(project_gemm_kernel<128>, grid, dim3(PNT), 0, s, P);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace parts: entry values, then ring rows.
void ws_parts(const csa_cache_desc* d, int B, int T, int64_t pos0, size_t* ent, size_t* ring) {
  const int64_t m = d->m, c = d->d_nope + d->d_rope;
  const int64_t R = d->overlap ? 2 * m : m, NT = d->overlap ? 4 : 2;
  const int64_t n_ent = (pos0 + T) / m - pos0 / m;
  *ent = align256(static_cast<size_t>(B) * (n_ent > 0 ? n_ent : 0) * c * sizeof(float));
  *ring = align256(static_cast<size_t>(B) * R * NT * c * sizeof(float));
}

}  // namespace
}  // namespace csa

using namespace csa;

extern "C" size_t csa_compress_project_workspace_bytes(const csa_cache_desc* desc, int B, int T, int64_t pos0) {
  if (!desc || B <= 0 || T <= 0 || pos0 < 0 || desc->m < 1) return 0;
  size_t ent, ring;
  ws_parts(desc, B, T, pos0, &ent, &ring);
  return ent + ring;
}

extern "C" int csa_compress_project_prefill(const csa_cache_desc* desc, int B, int T, int64_t pos0, const void* X,
                                            int d_model, const void* W, const float* Ba, const float* Bb,
                                            const csa_cache* cache, void* ws, size_t ws_bytes, void* stream) {
  int st;
  if ((st = compress_validate_cache(desc, cache)) != CSA_OK) return st;
  if (B < 0 || B > 65535 || T < 0 || pos0 < 0) return fail(CSA_ERR_INVALID_ARG, "B in 0..65535, T >= 0, pos0 >= 0");
  if (!X || !W || !Ba) return fail(CSA_ERR_INVALID_ARG, "X, W, Ba must be non-NULL");
  if (desc->overlap && !Bb) return fail(CSA_ERR_INVALID_ARG, "overlap needs Bb");
  if (!desc->overlap && Bb) return fail(CSA_ERR_INVALID_ARG, "Bb must be NULL without overlap");
  if (!aligned16(X) || !aligned16(W) || !aligned16(Ba) || !aligned16(Bb) || !aligned16(ws))
    return fail(CSA_ERR_ALIGNMENT, "X, W, Ba, Bb, ws must be 16-byte aligned");
  const int m = desc->m, c = desc->d_nope + desc->d_rope, NT = desc->overlap ? 4 : 2;
  if (desc->in_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "hidden states and weights must be BF16 (in_dtype)");
  if (128 % m || (desc->overlap && m > 64))
    return fail(CSA_ERR_UNSUPPORTED, "m must divide 128 (and be at most 64 when overlapped)");
  if (pos0 % m) return fail(CSA_ERR_UNSUPPORTED, "pos0 must be a multiple of m");
  if ((static_cast<int64_t>(NT) * c) % 128)
    return fail(CSA_ERR_UNSUPPORTED, "NT * c must be a multiple of 128 (c a multiple of 128 / NT)");
  if (desc->d_nope % 8 || desc->d_nope > 512 || desc->d_rope > 128)
    return fail(CSA_ERR_UNSUPPORTED, "d_nope a multiple of 8 up to 512, d_rope up to 128");
  if (d_model < PT_K || d_model % PT_K) return fail(CSA_ERR_INVALID_ARG, "d_model must be a positive multiple of 64");
  if (static_cast<int64_t>(T) * d_model * 2 >= (int64_t(1) << 31) ||
      static_cast<int64_t>(NT) * c * d_model * 2 >= (int64_t(1) << 31))
    return fail(CSA_ERR_UNSUPPORTED, "a sequence's hidden rows and the weights must each stay below 2^31 bytes");
  const int64_t E0 = pos0 / m, i_end = (pos0 + T) / m;
  if (i_end > desc->capacity) return fail(CSA_ERR_CAPACITY, "entries would exceed the cache capacity");
  if (B == 0 || T == 0) return CSA_OK;
  if (!ws || ws_bytes < csa_compress_project_workspace_bytes(desc, B, T, pos0))
    return fail(CSA_ERR_WORKSPACE, "workspace smaller than csa_compress_project_workspace_bytes()");

  ProjParams P{};
  P.C = compress_make_params(desc, cache, Ba, Bb);
  P.X = static_cast<const bf16_t*>(X);
  P.W = static_cast<const bf16_t*>(W);
  P.d = d_model;
  P.T = T;
  P.pos0 = pos0;
  P.E0 = E0;
  P.n_ent = i_end - E0;
  P.ovl = desc->overlap ? 1 : 0;
  P.wpt = PT_M / m - P.ovl;
  const int64_t windows = (pos0 + T - 1) / m - E0 + 1;  // every window the call's tokens touch
  P.n_mt = static_cast<int>((windows + P.wpt - 1) / P.wpt);
  const int TN = (NT * c) % 256 ? 128 : 256;  // column tile
  P.n_nt = NT * c / TN;
  P.t_first = pos0 + T - P.C.R > pos0 ? pos0 + T - P.C.R : pos0;
  size_t ent, ring;
  ws_parts(desc, B, T, pos0, &ent, &ring);
  P.went = static_cast<float*>(ws);
  P.wring = reinterpret_cast<float*>(static_cast<char*>(ws) + ent);
  hipStream_t s = as_stream(stream);
  const dim3 grid(static_cast<unsigned>((P.n_mt * P.n_nt + 7) / 8 * 8), 1, B);
  launch_project_gemm(P, TN, grid, s);
  if ((st = check_launch("project_gemm_kernel")) != CSA_OK) return st;
  if (P.n_ent > 0) {
    const int epw = 64 / wave_lanes_per_entry(desc->d_nope / 8, desc->d_rope / 2);
    const dim3 grid(static_cast<unsigned>((P.n_ent + 4 * epw - 1) / (4 * epw)), B);
    hipLaunchKernelGGL(project_finalize_kernel, grid, dim3(256), 0, s, P);
    if ((st = check_launch("project_finalize_kernel")) != CSA_OK) return st;
  }
  hipLaunchKernelGGL(project_ring_kernel, dim3(static_cast<unsigned>(pos0 + T - P.t_first), B), dim3(256), 0, s, P);
  return check_launch("project_ring_kernel");
}
