// Fused CSA decode step: the four decode calls of one CSA layer (compress
// the new token into the KV cache and into the indexer-key cache, indexer +
// top-k, sparse attention) behind one entry point, so that the small
// per-sequence launches merge: one launch runs both compressors and the
// indexer's per-row preparation, where the separate calls take three or
// four.  [CSA/HCA 混注意力] §1.1 (compress, index, top-k, attend), §1.3 (one
// CSA layer of the interleaved stack).  Results are the same bits as the
// separate calls: the same device code runs, only its launches are merged.
#include "attention.hpp"
#include "compress.hpp"
#include "index.hpp"

namespace csa {
namespace {

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

int check_consistent(const csa_cache_desc* kvd, const csa_cache_desc* kd, const csa_index_desc* id,
                     const csa_attn_desc* ad) {
  if (!kvd || !kd || !id || !ad) return fail(CSA_ERR_INVALID_ARG, "descriptor is NULL");
  if (kvd->m != ad->m || kd->m != id->m || kvd->m != kd->m)
    return fail(CSA_ERR_INVALID_ARG, "the caches, indexer and attention must share m");
  if (kvd->capacity != ad->capacity || kd->capacity != id->capacity)
    return fail(CSA_ERR_INVALID_ARG, "cache and reader capacities differ");
  if (kvd->d_nope != ad->d_nope || kvd->d_rope != ad->d_rope || kvd->nope_dtype != ad->nope_dtype ||
      (kvd->d_rope > 0 && kvd->rope_dtype != ad->rope_dtype))
    return fail(CSA_ERR_INVALID_ARG, "KV cache and attention descriptors disagree");
  if (kd->d_nope != id->dim || kd->d_rope != 0 || kd->nope_dtype != id->key_dtype)
    return fail(CSA_ERR_INVALID_ARG, "indexer-key cache and indexer descriptors disagree");
  if (kvd->page_size != ad->page_size || kvd->pool_pages != ad->pool_pages || kd->page_size != id->page_size ||
      kd->pool_pages != id->pool_pages)
    return fail(CSA_ERR_INVALID_ARG, "cache and reader paging (page_size, pool_pages) differ");
  return CSA_OK;
}

size_t index_part(const csa_index_desc* id, int B) {
  return round256(index_ws_bytes(id, CSA_OP_INDEX_TOPK_DECODE, B, 1, 0));
}

}  // namespace
}  // namespace csa

using namespace csa;

extern "C" size_t csa_decode_step_workspace_bytes(const csa_index_desc* idesc, const csa_attn_desc* adesc, int B,
                                                  int k) {
  if (!idesc || !adesc || B < 0) return 0;
  return index_part(idesc, B) + attn_ws_bytes(adesc, CSA_OP_SPARSE_ATTN_DECODE, B, 1, 0, k);
}

extern "C" int csa_decode_step(const csa_cache_desc* kv_desc, const csa_cache* kv, const csa_cache_desc* key_desc,
                               const csa_cache* keys, const csa_index_desc* idesc, const csa_attn_desc* adesc, int B,
                               const int64_t* pos, const csa_decode_inputs* in, int k, float softmax_scale,
                               int32_t* idx, float* scores, void* o, float* lse, void* ws, size_t ws_bytes,
                               void* stream) {
  int st;
  if (!in) return fail(CSA_ERR_INVALID_ARG, "inputs are NULL");
  if ((st = check_consistent(kv_desc, key_desc, idesc, adesc)) != CSA_OK) return st;
  CompressParams Pkv, Pkey;
  IndexParams Pi;
  AttnParams Pa;
  if ((st = compress_decode_setup(kv_desc, B, pos, in->a, in->b, in->za, in->zb, in->Ba, in->Bb, kv, &Pkv)) != CSA_OK)
    return st;
  if ((st = compress_decode_setup(key_desc, B, pos, in->ka, in->kb, in->kza, in->kzb, in->kBa, in->kBb, keys, &Pkey)) !=
      CSA_OK)
    return st;
  const size_t ipart = index_part(idesc, B);
  if (!ws || ws_bytes < csa_decode_step_workspace_bytes(idesc, adesc, B, k))
    return fail(CSA_ERR_WORKSPACE, "workspace smaller than csa_decode_step_workspace_bytes()");
  if ((st = index_decode_setup(idesc, B, pos, in->qI, in->w, keys, k, idx, scores, ws, ipart, &Pi)) != CSA_OK)
    return st;
  void* aws = static_cast<char*>(ws) + ipart;
  if ((st = sparse_attn_decode_setup(adesc, B, pos, in->q, kv, idx, k, softmax_scale, o, lse, aws, ws_bytes - ipart,
                                     &Pa)) != CSA_OK)
    return st;
  if (B == 0) return CSA_OK;
  // paged KV cache: the final top-k pass writes the selected entries' pool
  // rows where the attention reads its list (no separate translation launch)
  if (Pi.ghist) {
    if (int32_t* rows = page_list_slot(Pa, CSA_OP_SPARSE_ATTN_DECODE, B)) {
      Pi.rows_out = rows;
      Pi.row_pg = Pa.pg;
      Pi.row_cap = Pa.cap;
      Pa.idx = rows;
      Pa.list_rows = true;
    }
  }
  hipStream_t s = as_stream(stream);
  const bool fused = Pkv.in_dt == Pkey.in_dt;
  if (fused) {
    st = launch_decode_step_prep(Pkv, Pkey, Pi, index_decode_prep_mx(Pi), B, pos, s);
  } else {
    st = launch_compress_decode(Pkv, B, pos, s);
    if (st == CSA_OK) st = launch_compress_decode(Pkey, B, pos, s);
  }
  if (st != CSA_OK) return st;
  if ((st = launch_index_decode(Pi, B, stream, fused)) != CSA_OK) return st;
  return attn_dispatch(Pa, CSA_OP_SPARSE_ATTN_DECODE, B, stream);
}
