/*
 * csa.h - C ABI of the CSA / HCA hybrid-attention hot path for MI355X (gfx950).
 *
 * The library computes the three steps of compressed sparse attention (CSA)
 * and heavily compressed attention (HCA) over a compressed KV cache:
 *
 *   compress   every m tokens -> one KV entry (overlapped for CSA, m = 4;
 *              single window for HCA, m' = 128), then RoPE + storage format;
 *   index_topk lightning-indexer scores of each query against every visible
 *              entry, and the k best entries (k = 1024);
 *   attention  softmax attention of all query heads over the selected entries
 *              (CSA, sparse) or over every visible entry (HCA, dense).
 *
 * Page citations (titles shortened):
 *   [CSA/HCA 混注意力]  "从论文出发，逐层剖析 CSA / HCA 混注意力、mHC 残差连接与 Muon 优化器"
 *   [三大核心架构创新]  "DeepSeek-V4 技术解析：三大核心架构创新如何突破百万Token上下文瓶颈"
 *   [读完这篇]          "读完这篇你就搞懂 DeepSeek v4 了"
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device pointers; "host" ones are read
 *     on the host before the call returns.  Buffers are owned by the caller;
 *     the library keeps no pointer after a call returns and never allocates
 *     or frees device memory.  Scratch memory comes only through `ws`.
 *   - Tensors are row-major with the last dimension contiguous.  Device base
 *     pointers must be 16-byte aligned.  Indices are int32, positions int64.
 *   - `stream` is a hipStream_t (NULL = the default stream).  On CSA_OK the
 *     work has been enqueued on that stream; faults during execution surface
 *     as HIP errors on the stream.  Every argument is validated on the host
 *     first: on any error nothing is launched, outputs are untouched, and
 *     csa_last_error() (thread-local) describes the problem.
 *   - Results are deterministic: the same inputs give bitwise-equal outputs,
 *     and a sequence's results do not depend on the other sequences in the
 *     batch.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 1

/* Status codes. */
enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent descriptor */
  CSA_ERR_ALIGNMENT = 2,   /* a device pointer is not 16-byte aligned */
  CSA_ERR_UNSUPPORTED = 3, /* valid but not implemented (dtype/shape combination) */
  CSA_ERR_WORKSPACE = 4,   /* ws_bytes smaller than csa_workspace_bytes() */
  CSA_ERR_CAPACITY = 5,    /* entries would be written past the cache capacity */
  CSA_ERR_HIP = 6          /* a HIP runtime call failed while enqueueing */
};

/* Element formats. */
enum {
  CSA_F32 = 0,     /* IEEE binary32 */
  CSA_BF16 = 1,    /* bfloat16, RNE conversions */
  CSA_FP8E4M3 = 2, /* OCP OFP8 E4M3 bytes with one fp32 scale per entry */
  CSA_MXFP4 = 3    /* OCP MX v1.0: packed E2M1 pairs (low nibble = even element)
                      + one E8M0 byte per 32 elements */
};

/* Compressed-cache layout and compressor parameters.
 * [CSA/HCA 混注意力] §1.1 工程细节 (overlap of C^a and C^b, m = 4), §1.2 (HCA,
 * m' = 128), §1.4 存储格式混 (RoPE dims BF16, the rest FP8). */
typedef struct csa_cache_desc {
  int32_t m;          /* tokens per entry, 1..256 */
  int32_t overlap;    /* 1: entry i mixes window i (C^a) and window i-1 (C^b); 0: window i only */
  int32_t d_nope;     /* dims stored in nope_dtype (the value part of a KV entry) */
  int32_t d_rope;     /* RoPE dims, the last d_rope of an entry; even; 0 for indexer keys */
  int32_t in_dtype;   /* a, b, za, zb element type: CSA_F32 or CSA_BF16 */
  int32_t nope_dtype; /* CSA_F32, CSA_BF16, CSA_FP8E4M3, or CSA_MXFP4 (indexer keys only) */
  int32_t rope_dtype; /* CSA_F32 or CSA_BF16 */
  int32_t reserved;   /* must be 0 */
  double rope_base;   /* RoPE base (10000) */
  int64_t capacity;   /* entries per sequence */
} csa_cache_desc;

/* Device buffers of a compressed cache for B sequences (sequence stride =
 * capacity entries).  c = d_nope + d_rope.
 *   nope : [B][capacity][d_nope] elements; MXFP4: [B][capacity][d_nope/2] bytes
 *   scale: FP8E4M3: float [B][capacity]; MXFP4: uint8 [B][capacity][d_nope/32];
 *          otherwise unused (may be NULL)
 *   rope : [B][capacity][d_rope] elements of rope_dtype (NULL when d_rope = 0)
 *   ring : float [B][R][NT][c] staging rows of the most recent tokens,
 *          R = overlap ? 2m : m, NT = overlap ? 4 (a, za, b, zb) : 2 (a, za);
 *          token p lives in slot p mod R.  The compressor reads it for entries
 *          that need tokens before the current call and refreshes it. */
typedef struct csa_cache {
  void* nope;
  void* scale;
  void* rope;
  float* ring;
} csa_cache;

/* Lightning-indexer configuration.  [CSA/HCA 混注意力] §1.4 LIGHTNING INDEXER
 * 的 FP4 计 (FP4 QK, scores FP32 -> BF16); [读完这篇] §三 CSA 步骤二 (V3.2
 * DSA form, heads weighted before top-k). */
typedef struct csa_index_desc {
  int32_t n_heads;     /* H_I */
  int32_t dim;         /* d_I (a multiple of 32 for MXFP4) */
  int32_t q_dtype;     /* qI element type: CSA_F32 or CSA_BF16 */
  int32_t qk_dtype;    /* format of the QK product: CSA_F32, CSA_BF16, or CSA_MXFP4
                          (qI is quantised to MXFP4 inside the call) */
  int32_t key_dtype;   /* key cache format: CSA_F32, CSA_BF16, CSA_FP8E4M3, CSA_MXFP4 */
  int32_t score_dtype; /* CSA_F32, or CSA_BF16 (scores rounded FP32 -> BF16 before selection) */
  int32_t m;           /* tokens per key entry (visibility) */
  int32_t reserved;    /* must be 0 */
  int64_t capacity;    /* key entries per sequence */
} csa_index_desc;

/* Attention configuration (CSA sparse and HCA dense). */
typedef struct csa_attn_desc {
  int32_t n_heads;    /* H query heads sharing one KV entry (MQA) */
  int32_t d_nope;     /* value dim d_v (the non-RoPE part of an entry) */
  int32_t d_rope;     /* RoPE dims of q and of each entry (last d_rope dims) */
  int32_t q_dtype;    /* CSA_F32 or CSA_BF16 */
  int32_t o_dtype;    /* CSA_F32 or CSA_BF16 */
  int32_t nope_dtype; /* cache: CSA_F32, CSA_BF16, CSA_FP8E4M3 */
  int32_t rope_dtype; /* cache: CSA_F32, CSA_BF16 */
  int32_t m;          /* tokens per entry (visibility) */
  double rope_base;
  int64_t capacity;   /* entries per sequence */
} csa_attn_desc;

/* ---- compressor ---------------------------------------------------------
 * Entry i of channel j ([CSA/HCA 混注意力] §1.1 工程细节; [三大核心架构创新]
 * §2.2 第一步; [读完这篇] §三 压缩机制 (4 W + 2 B, per-dimension weights)):
 *   one softmax over the logits za[im+r][j] + Ba[r][j] and, when overlapped
 *   and i >= 1, zb[(i-1)m+r][j] + Bb[r][j] (r < m); the entry is the
 *   softmax-weighted sum of the matching a and b values.  Entry 0 has no C^b.
 * Then the last d_rope dims turn by RoPE at position im + m - 1 (adjacent
 * pairs, theta_p = base^(-2p/d_rope)), and the entry is stored in the cache
 * format (FP8: scale = amax/448 of the d_nope part, codes RNE saturating).
 */

/* Prefill: tokens [pos0, pos0 + T) of each of B sequences (same pos0 for all).
 *   a, za, b, zb : device [B][T][c] of desc->in_dtype (b, zb NULL iff !overlap)
 *   Ba, Bb       : device float [m][c] (Bb NULL iff !overlap)
 * Writes every entry whose window ends inside [pos0, pos0 + T); tokens before
 * pos0 that such an entry needs are read from the ring, which must then hold
 * them (a previous call on the same cache).  The ring is left holding the
 * last R tokens.  CSA_ERR_CAPACITY if an entry index reaches capacity. */
int csa_compress_prefill(const csa_cache_desc* desc, int B, int T, int64_t pos0,
                         const void* a, const void* b, const void* za, const void* zb,
                         const float* Ba, const float* Bb, const csa_cache* cache,
                         void* stream);

/* Decode: one new token per sequence at device position pos[b] (int64 [B]).
 *   a, za, b, zb : device [B][c].  The token enters the ring; when
 * (pos[b] + 1) mod m == 0 the entry pos[b]/m is completed and stored (if it
 * is below capacity; otherwise it is dropped). */
int csa_compress_decode(const csa_cache_desc* desc, int B, const int64_t* pos,
                        const void* a, const void* b, const void* za, const void* zb,
                        const float* Ba, const float* Bb, const csa_cache* cache,
                        void* stream);

/* ---- lightning indexer + top-k ------------------------------------------
 * For the query at absolute position p, n(p) = floor((p + 1) / m) entries are
 * visible (an entry becomes visible once its window is complete), capped at
 * capacity.  Score ([CSA/HCA 混注意力] §1.4; [读完这篇] §三 CSA 步骤二):
 *   I[s] = sum_h w[h] * max(0, qI[h] . K[s]),  s < n(p)
 * with K decoded from the key cache (FP8: code * scale) and, in MXFP4 mode,
 * qI quantised to MXFP4 per head.  BF16 score mode rounds I to BF16 (RNE).
 * Selection ([CSA/HCA 混注意力] §1.1 关键参数, top-k = 1024): the min(k, n)
 * entries with the largest I, equal scores going to the lower index, listed
 * in ascending index order and padded with -1.  k in 1..2048.
 *   qI    : device [B][T][H_I][d_I] of q_dtype
 *   w     : device float [B][T][H_I]
 *   keys  : cache buffers (nope/scale) of the key cache
 *   idx   : device int32 [B][T][k]
 *   scores: device float [B][T][capacity] or NULL; when given, receives I
 *           (as used for selection) for s < n, the rest untouched
 *   ws    : device workspace of csa_workspace_bytes(CSA_OP_INDEX_TOPK_*) bytes */
int csa_index_topk_prefill(const csa_index_desc* desc, int B, int T, int64_t pos0,
                           const void* qI, const float* w, const csa_cache* keys, int k,
                           int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                           void* stream);

/* Decode: one query per sequence at device position pos[b]; qI [B][H_I][d_I],
 * w [B][H_I], idx [B][k], scores [B][capacity] or NULL. */
int csa_index_topk_decode(const csa_index_desc* desc, int B, const int64_t* pos,
                          const void* qI, const float* w, const csa_cache* keys, int k,
                          int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                          void* stream);

/* ---- attention ------------------------------------------------------------
 * For the query at absolute position p and each head h ([CSA/HCA 混注意力]
 * §1.1 (CSA attends only the selected entries), §1.2 (HCA dense over the
 * 128x shorter sequence); [读完这篇] §三 CSA 步骤三 (standard attention, KV
 * shared by all heads)):
 *   q~ = q[h] with its last d_rope dims turned by RoPE at position p
 *   l_s = softmax_scale * q~ . K_s      (K_s: the whole decoded entry)
 *   o[h] = sum_s softmax(l)_s * V_s     (V_s: the d_nope part of the entry)
 *   lse[h] = log sum_s exp(l_s)
 * over S = the listed entries (CSA) or all s < n(p) (HCA).  Listed indices
 * outside [0, n(p)) are skipped.  An empty S gives o = 0 and lse = -inf.
 *   q   : device [B][T][H][d_nope + d_rope] of q_dtype
 *   idx : device int32 [B][T][k] (CSA only)
 *   o   : device [B][T][H][d_nope] of o_dtype
 *   lse : device float [B][T][H] or NULL
 *   ws  : device workspace of csa_workspace_bytes(...) bytes (may be 0)
 * In all four attention calls softmax_scale must be positive and finite
 * (CSA_ERR_INVALID_ARG otherwise). */
int csa_sparse_attn_prefill(const csa_attn_desc* desc, int B, int T, int64_t pos0,
                            const void* q, const csa_cache* kv, const int32_t* idx, int k,
                            float softmax_scale, void* o, float* lse, void* ws,
                            size_t ws_bytes, void* stream);

/* Decode: q [B][H][c], idx [B][k], o [B][H][d_nope], lse [B][H]; positions
 * device int64 pos[B]. */
int csa_sparse_attn_decode(const csa_attn_desc* desc, int B, const int64_t* pos,
                           const void* q, const csa_cache* kv, const int32_t* idx, int k,
                           float softmax_scale, void* o, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

int hca_dense_attn_prefill(const csa_attn_desc* desc, int B, int T, int64_t pos0,
                           const void* q, const csa_cache* kv, float softmax_scale, void* o,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

int hca_dense_attn_decode(const csa_attn_desc* desc, int B, const int64_t* pos,
                          const void* q, const csa_cache* kv, float softmax_scale, void* o,
                          float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---- workspace and diagnostics ------------------------------------------ */
enum {
  CSA_OP_INDEX_TOPK_PREFILL = 1,  /* desc: csa_index_desc */
  CSA_OP_INDEX_TOPK_DECODE = 2,   /* desc: csa_index_desc */
  CSA_OP_SPARSE_ATTN_PREFILL = 3, /* desc: csa_attn_desc */
  CSA_OP_SPARSE_ATTN_DECODE = 4,  /* desc: csa_attn_desc */
  CSA_OP_DENSE_ATTN_PREFILL = 5,  /* desc: csa_attn_desc */
  CSA_OP_DENSE_ATTN_DECODE = 6    /* desc: csa_attn_desc */
};

/* Workspace bytes `op` needs for B sequences of T queries (T = 1 for decode)
 * starting at pos0 (prefill; ignored for decode, which sizes for capacity),
 * with k selected entries.  Pure host function; returns 0 for a bad op. */
size_t csa_workspace_bytes(int op, const void* desc, int B, int T, int64_t pos0, int k);

const char* csa_status_string(int status);
const char* csa_last_error(void);
int csa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
