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
 *     and, for the same descriptor, a sequence's results do not depend on
 *     the other sequences in the batch or on the batch size (work is split
 *     per sequence by its own entry count only).
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 3

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
  int32_t page_size;  /* 0: contiguous caches (sequence b owns rows [b*capacity, (b+1)*capacity));
                         else entries per page, a power of two in 64..65536, and the cache is
                         paged (csa_cache.block_table) */
  double rope_base;   /* RoPE base (10000) */
  int64_t capacity;   /* entries per sequence (logical; a multiple of page_size when paged) */
  int64_t pool_pages; /* paged: physical pages in the pool; 0 when contiguous */
} csa_cache_desc;

/* Device buffers of a compressed cache for B sequences.  c = d_nope + d_rope.
 * Rows: contiguous caches hold entry s of sequence b in row b*capacity + s
 * (ROWS = B*capacity); paged caches hold it in row
 * block_table[b][s / page_size] * page_size + s % page_size of a pool shared
 * by the batch (ROWS = pool_pages*page_size).  [百万令牌的智慧觉醒] §🏗️
 * (heterogeneous KV cache of the serving framework), [CSA/HCA 混注意力]
 * 共享前缀场景的理复用 (compressed entries reused on a shared prefix: two
 * sequences' tables may name the same pages for a common, complete prefix).
 *   nope : [ROWS][d_nope] elements; MXFP4: [ROWS][d_nope/2] bytes
 *   scale: FP8E4M3: float [ROWS]; MXFP4: uint8 [ROWS][d_nope/32];
 *          otherwise unused (may be NULL)
 *   rope : [ROWS][d_rope] elements of rope_dtype (NULL when d_rope = 0)
 *   ring : float [B][R][NT][c] staging rows of the most recent tokens,
 *          R = overlap ? 2m : m, NT = overlap ? 4 (a, za, b, zb) : 2 (a, za);
 *          token p lives in slot p mod R.  The compressor reads it for entries
 *          that need tokens before the current call and refreshes it.  Never
 *          paged.
 *   block_table: device int32 [B][capacity/page_size] when paged, NULL when
 *          contiguous.  Entries must lie in [0, pool_pages); the kernels
 *          never touch memory outside the pool: an entry whose page is out of
 *          range is not written and reads as some row of the pool (its
 *          results are then unspecified).  Pages written in one call (the
 *          compressor's) must not be shared with another sequence of it. */
typedef struct csa_cache {
  void* nope;
  void* scale;
  void* rope;
  float* ring;
  const int32_t* block_table;
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
  int32_t page_size;   /* key cache paging, as csa_cache_desc.page_size (decode only) */
  int64_t capacity;    /* key entries per sequence */
  int64_t pool_pages;  /* paged: pages in the key pool; 0 when contiguous */
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
  int32_t window;     /* dense attention only: attend the last `window` visible entries
                         (a sliding window; with m = 1 over per-token entries, the
                         sliding-window branch); 0 = every visible entry.  Must be 0
                         for sparse attention. */
  int32_t qk_mode;    /* 0: QK in the query's own format.  CSA_FP8E4M3 (FP8 cache,
                         64 BF16 heads over 512 + 64 dims, BF16 output): each head's
                         512 non-RoPE query dims are rounded to MXFP8 inside the call
                         (OCP MX: blocks of 32 dims, E4M3 elements RNE saturating at
                         448, one E8M0 scale 2^(floor(log2 amax) - 8)) and multiplied
                         with the cache's FP8 codes in FP8 (exact products, fp32 sums,
                         the entry scale applied to the sum); the RoPE dims stay BF16.
                         A reading of [CSA/HCA 混注意力] §1.4 存储格式混 (non-RoPE dims
                         in FP8, RoPE dims in BF16).  CSA_ERR_UNSUPPORTED for other
                         shapes, and for sparse prefill lists longer than 1024. */
  double rope_base;
  int64_t capacity;   /* entries per sequence */
  int32_t page_size;  /* KV cache paging, as csa_cache_desc.page_size */
  int32_t reserved;   /* must be 0 */
  int64_t pool_pages; /* paged: pages in the KV pool; 0 when contiguous */
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

/* Prefill from hidden states: the compressor's four input projections
 * ([读完这篇] §三 压缩机制: learnable W^{aKV}, W^{bKV}, W^{aZ}, W^{bZ} and the
 * biases B^a, B^b) fused with the compression, so that a, za, b, zb never
 * reach memory:
 *   a = X W^{aKV}, za = X W^{aZ}, b = X W^{bKV}, zb = X W^{bZ}
 * (fp32 accumulation, not rounded), then exactly the entries, RoPE, storage
 * and ring update of csa_compress_prefill on those rows.
 *   X  : device BF16 [B][T][d_model] hidden states of tokens [pos0, pos0 + T)
 *   W  : device BF16 [NT * c][d_model]: row j*NT + u is column j of projection
 *        u, u = 0: W^{aKV}, 1: W^{aZ}, 2: W^{bKV}, 3: W^{bZ} (NT = 4 when
 *        overlapped, else NT = 2: W^{aKV}, W^{aZ}); c = d_nope + d_rope
 *   Ba, Bb : device float [m][c] (Bb NULL iff !overlap)
 *   ws : device workspace of csa_compress_project_workspace_bytes() bytes
 * desc->in_dtype must be CSA_BF16 (the type of X and W).  Supported shapes
 * (CSA_ERR_UNSUPPORTED otherwise): m divides 128 (at most 64 when
 * overlapped), pos0 a multiple of m, NT * c a multiple of 128, d_nope a
 * multiple of 8 up to 512, d_rope up to 128, d_model a multiple of 64, and
 * T * d_model * 2 and NT * c * d_model * 2 below 2^31 bytes.
 * CSA_ERR_CAPACITY if an entry index reaches capacity. */
int csa_compress_project_prefill(const csa_cache_desc* desc, int B, int T, int64_t pos0, const void* X,
                                 int d_model, const void* W, const float* Ba, const float* Bb,
                                 const csa_cache* cache, void* ws, size_t ws_bytes, void* stream);
size_t csa_compress_project_workspace_bytes(const csa_cache_desc* desc, int B, int T, int64_t pos0);

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
 *   ws    : device workspace of csa_workspace_bytes(CSA_OP_INDEX_TOPK_*) bytes
 * Paged key caches (desc->page_size > 0) are read by csa_index_topk_decode;
 * csa_index_topk_prefill returns CSA_ERR_UNSUPPORTED for them.  A key block
 * of the scan (16 entries, 64 for MXFP4) never crosses a page. */
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
 * over S = the listed entries (CSA) or all s < n(p) (HCA; with window w > 0
 * only max(0, n(p) - w) <= s < n(p)).  Listed indices outside [0, n(p)) are
 * skipped.  An empty S gives o = 0 and lse = -inf.
 *   q   : device [B][T][H][d_nope + d_rope] of q_dtype
 *   idx : device int32 [B][T][k] (CSA only)
 *   o   : device [B][T][H][d_nope] of o_dtype
 *   lse : device float [B][T][H] or NULL
 *   ws  : device workspace of csa_workspace_bytes(...) bytes (may be 0)
 * In all four attention calls softmax_scale must be positive and finite
 * (CSA_ERR_INVALID_ARG otherwise).  With 64 BF16 heads over 512 + 64 BF16
 * or FP8 dims (the matrix-core path) each cache buffer of one sequence must
 * stay below 2^31 bytes: capacity <= 2^21 (BF16 non-RoPE rows) or 2^22 (FP8
 * rows), CSA_ERR_UNSUPPORTED otherwise.  Decode workspaces hold per-sequence
 * split partials: csa_workspace_bytes grows linearly with B.
 * Paged KV caches (desc->page_size > 0, kv->block_table): the same results
 * as the contiguous layout holding the same entries.  The 2^31-byte limit
 * then applies to the pool (pool_pages*page_size rows), and the sparse calls
 * first turn their lists into pool rows inside the workspace
 * (csa_workspace_bytes includes B*T*k int32 for it). */
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

/* Allocation-free variant of csa_sparse_attn_decode, for callers that cannot
 * allocate device memory or hand the library a workspace (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments and results as csa_sparse_attn_decode without ws/ws_bytes:
 * the decode split partials go to one library-owned device array of
 * CSA_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds until the process ends.  CSA_ERR_WORKSPACE when the call needs more
 * than that (csa_workspace_bytes(CSA_OP_SPARSE_ATTN_DECODE, ...) bytes: about
 * 0.5 MiB per sequence at k = 1024, so B <= 127).  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  No part of the array
 * needs to start at zero: every call writes each partial it reads. */
#define CSA_NOALLOC_SCRATCH_BYTES (64u << 20)
int csa_sparse_attn_decode_noalloc(const csa_attn_desc* desc, int B, const int64_t* pos,
                                   const void* q, const csa_cache* kv, const int32_t* idx, int k,
                                   float softmax_scale, void* o, float* lse, void* stream);

int hca_dense_attn_prefill(const csa_attn_desc* desc, int B, int T, int64_t pos0,
                           const void* q, const csa_cache* kv, float softmax_scale, void* o,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

int hca_dense_attn_decode(const csa_attn_desc* desc, int B, const int64_t* pos,
                          const void* q, const csa_cache* kv, float softmax_scale, void* o,
                          float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---- log-sum-exp merge of two attention results --------------------------
 * The sliding-window branch of a CSA / HCA layer ([CSA/HCA 混注意力] §1.3:
 * V4-Flash's sliding-window layers; the uncompressed SWA KV of the prefix-cache
 * paragraph) attends the most recent uncompressed tokens; its result and the
 * compressed branch's are one softmax over the union of their keys, formed
 * from the two partial results: per (row, head)
 *   l = log(exp(lse1) + exp(lse2)),  o = exp(lse1 - l) o1 + exp(lse2 - l) o2
 * (both -inf: o = 0, lse = -inf).
 *   o1, o2, o : device [rows][H][d_v] of o_dtype (CSA_F32 or CSA_BF16); o may
 *               alias o1 or o2
 *   lse1, lse2: device float [rows][H]; lse: device float [rows][H] or NULL
 * rows = B*T (prefill) or B (decode).  d_v a multiple of 4, at most 4096. */
int csa_lse_merge(int rows, int H, int d_v, int o_dtype, const void* o1, const float* lse1, const void* o2,
                  const float* lse2, void* o, float* lse, void* stream);

/* ---- fused CSA decode step -------------------------------------------------
 * One decode step of a CSA layer ([CSA/HCA 混注意力] §1.1: compress, index,
 * select the top k, attend; §1.3: one CSA layer of the interleaved stack)
 * in one call: exactly
 *   csa_compress_decode(kv_desc, B, pos, a, b, za, zb, Ba, Bb, kv)
 *   csa_compress_decode(key_desc, B, pos, ka, kb, kza, kzb, kBa, kBb, keys)
 *   csa_index_topk_decode(idesc, B, pos, qI, w, keys, k, idx, scores, ...)
 *   csa_sparse_attn_decode(adesc, B, pos, q, kv, idx, k, softmax_scale, o, lse, ...)
 * with the same results bit for bit, in fewer launches (both compressors and
 * the indexer's per-row preparation run in one; they need the same in_dtype,
 * else they launch apart).  The descriptors must agree (m, capacities, the
 * KV layout with the attention's, the key layout with the indexer's), else
 * CSA_ERR_INVALID_ARG.  Every argument of the four calls is validated first;
 * on any error nothing is launched.
 *   in : the new token's compressor rows and queries, device pointers:
 *        a, b, za, zb [B][c]; Ba, Bb [m][c] (b, zb, Bb NULL without
 *        overlap); ka, kb, kza, kzb [B][d_I]; kBa, kBb [m][d_I]; q [B][H][c];
 *        qI [B][H_I][d_I]; w float [B][H_I]
 *   idx: device int32 [B][k] (receives the selection); scores as in
 *        csa_index_topk_decode; o, lse as in csa_sparse_attn_decode
 *   ws : device workspace of csa_decode_step_workspace_bytes(idesc, adesc, B, k) */
typedef struct csa_decode_inputs {
  const void* a;
  const void* b;
  const void* za;
  const void* zb;
  const float* Ba;
  const float* Bb;
  const void* ka;
  const void* kb;
  const void* kza;
  const void* kzb;
  const float* kBa;
  const float* kBb;
  const void* q;
  const void* qI;
  const float* w;
} csa_decode_inputs;

int csa_decode_step(const csa_cache_desc* kv_desc, const csa_cache* kv, const csa_cache_desc* key_desc,
                    const csa_cache* keys, const csa_index_desc* idesc, const csa_attn_desc* adesc, int B,
                    const int64_t* pos, const csa_decode_inputs* in, int k, float softmax_scale, int32_t* idx,
                    float* scores, void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of csa_decode_step for B sequences and k selected entries
 * (pure host function; 0 for NULL descriptors). */
size_t csa_decode_step_workspace_bytes(const csa_index_desc* idesc, const csa_attn_desc* adesc, int B, int k);

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
