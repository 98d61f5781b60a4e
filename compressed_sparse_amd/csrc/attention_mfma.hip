// Dispatch of the MFMA attention path (64 query heads sharing one compressed
// entry of 512 non-RoPE + 64 RoPE dims, MQA; BF16 queries and outputs; BF16
// or FP8-with-scale cache) and the log-sum-exp merge of decode splits.
// [CSA/HCA 混注意力] §1.1, §1.2; [读完这篇] §三 CSA 步骤三; §1.4 存储格式混.
//
// Prefill runs one query per work item; decode splits each sequence's entry
// list (CSA) or visible entries (HCA) over several work items, each writing
// a partial (O normalised by its own weights, as BF16, and the log2 of its
// weight sum) that attn_merge_kernel combines.
#include <cmath>

#include "attention.hpp"

namespace csa {
namespace {

constexpr int NH = 64;       // heads
constexpr int DN = 512;      // value / non-RoPE dims
constexpr int DRP = 64;      // RoPE dims
constexpr int TILE = 64;     // entries per tile of the attention kernel
constexpr int MAX_SPLITS = 32;
constexpr int MAX_LIST = 1024;  // list entries one work item handles
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Combines split partials by log-sum-exp: O = sum_s 2^(l_s - M) O_s / sum_s
// 2^(l_s - M), l_s the split's log2 weight sum and M their maximum; grid
// (NH, B), one thread per 4 value dims (128 threads), the head's split
// weights computed once in LDS.  S >= splits is a power of two: every
// thread's S partial loads (clamped to the last split) are issued before
// the weights are known.
template <int S>
__global__ void __launch_bounds__(128) attn_merge_kernel(AttnParams P, int splits, const void* part, int B) {
  __shared__ float s_f[S];
  __shared__ float s_L, s_M;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const bf16_t* po = static_cast<const bf16_t*>(part) + static_cast<size_t>(b) * splits * (NH * DN) +
                     static_cast<size_t>(h) * DN + 4 * tid;
  uint2 v[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp)
    v[sp] = *reinterpret_cast<const uint2*>(po + static_cast<size_t>(min(sp, splits - 1)) * NH * DN);
  const float* pl = reinterpret_cast<const float*>(static_cast<const bf16_t*>(part) + static_cast<size_t>(B) * splits * (NH * DN)) +
                    static_cast<size_t>(b) * splits * NH;
  if (tid < 64) {
    const float ls = tid < splits ? pl[tid * NH + h] : -INFINITY;
    float M = ls;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = ls != -INFINITY ? exp2f(ls - M) : 0.0f;
    float L = f;
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
    acc.x = fmaf(__uint_as_float(v[sp].x << 16), f, acc.x);
    acc.y = fmaf(__uint_as_float(v[sp].x & 0xFFFF0000u), f, acc.y);
    acc.z = fmaf(__uint_as_float(v[sp].y << 16), f, acc.z);
    acc.w = fmaf(__uint_as_float(v[sp].y & 0xFFFF0000u), f, acc.w);
  }
  bf16_t* out = static_cast<bf16_t*>(P.o) + (static_cast<size_t>(b) * NH + h) * DN + 4 * tid;
  *reinterpret_cast<uint2*>(out) = make_uint2(pack2_bf16(acc.x * inv, acc.y * inv), pack2_bf16(acc.z * inv, acc.w * inv));
  if (P.lse && tid == 0) P.lse[static_cast<size_t>(b) * NH + h] = L > 0.0f ? (s_M + log2f(L)) * LN2 : -INFINITY;
}

// bytes of the split partials of B sequences
size_t part_bytes(int B, int splits) {
  return static_cast<size_t>(B) * splits * NH * (DN * sizeof(bf16_t) + sizeof(float));
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
  return part_bytes(B, MAX_SPLITS);
}

int launch_mfma_attn(const AttnParams& P, int op, int B, hipStream_t s) {
  const bool dense = op == CSA_OP_DENSE_ATTN_PREFILL || op == CSA_OP_DENSE_ATTN_DECODE;
  const bool decode = op == CSA_OP_SPARSE_ATTN_DECODE || op == CSA_OP_DENSE_ATTN_DECODE;
  if (!decode) {
    const int64_t per = dense ? P.cap : P.k;
    launch_attn_bf16(P, dense, B, s, 1, per, nullptr);
    return check_launch("attn_bf16_kernel");
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
  const size_t need = part_bytes(B, splits);
  if (!P.ws || P.ws_bytes < need) return fail(CSA_ERR_WORKSPACE, "workspace too small for the split partials");
  void* part = P.ws;
  launch_attn_bf16(P, dense, B, s, splits, per, part);
  int st = check_launch("attn_bf16_kernel");
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
