// Library-wide host functions: error state, status strings, workspace query.
#include <hip/hip_runtime.h>

#include <string>

#include "common.hpp"

namespace csa {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return CSA_OK;
}

int check_paging(int32_t page_size, int64_t pool_pages, int64_t capacity) {
  if (page_size == 0) {
    if (pool_pages != 0) return fail(CSA_ERR_INVALID_ARG, "pool_pages must be 0 for a contiguous cache");
    return CSA_OK;
  }
  if (page_size < 64 || page_size > 65536 || (page_size & (page_size - 1)))
    return fail(CSA_ERR_INVALID_ARG, "page_size must be 0 or a power of two in 64..65536");
  if (capacity % page_size) return fail(CSA_ERR_INVALID_ARG, "capacity must be a multiple of page_size");
  if (pool_pages < 1 || pool_pages > (int64_t(1) << 31) / page_size)
    return fail(CSA_ERR_INVALID_ARG, "pool_pages must be in 1..2^31/page_size");
  return CSA_OK;
}

int make_pages(int32_t page_size, int64_t pool_pages, int64_t capacity, const int32_t* table, Pages* out) {
  int st;
  if ((st = check_paging(page_size, pool_pages, capacity)) != CSA_OK) return st;
  *out = Pages{};
  if (page_size == 0) {
    if (table) return fail(CSA_ERR_INVALID_ARG, "block_table must be NULL for a contiguous cache");
    return CSA_OK;
  }
  if (!table) return fail(CSA_ERR_INVALID_ARG, "a paged cache needs a block_table");
  if (reinterpret_cast<uintptr_t>(table) & 3u) return fail(CSA_ERR_ALIGNMENT, "block_table must be 4-byte aligned");
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  out->table = table;
  out->shift = shift;
  out->tps = capacity >> shift;
  out->pool = pool_pages;
  return CSA_OK;
}

size_t index_ws_bytes(const csa_index_desc* d, int op, int B, int T, int64_t pos0);
size_t attn_ws_bytes(const csa_attn_desc* d, int op, int B, int T, int64_t pos0, int k);

}  // namespace csa

extern "C" size_t csa_workspace_bytes(int op, const void* desc, int B, int T, int64_t pos0, int k) {
  switch (op) {
    case CSA_OP_INDEX_TOPK_PREFILL:
    case CSA_OP_INDEX_TOPK_DECODE:
      return csa::index_ws_bytes(static_cast<const csa_index_desc*>(desc), op, B, T, pos0);
    case CSA_OP_SPARSE_ATTN_PREFILL:
    case CSA_OP_SPARSE_ATTN_DECODE:
    case CSA_OP_DENSE_ATTN_PREFILL:
    case CSA_OP_DENSE_ATTN_DECODE:
      return csa::attn_ws_bytes(static_cast<const csa_attn_desc*>(desc), op, B, T, pos0, k);
    default:
      return 0;
  }
}

extern "C" const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARG: return "CSA_ERR_INVALID_ARG";
    case CSA_ERR_ALIGNMENT: return "CSA_ERR_ALIGNMENT";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
    case CSA_ERR_CAPACITY: return "CSA_ERR_CAPACITY";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
    default: return "unknown status";
  }
}

extern "C" const char* csa_last_error(void) { return csa::g_last_error.c_str(); }

extern "C" int csa_version(void) { return CSA_ABI_VERSION; }
