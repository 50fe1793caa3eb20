// KV commit of the accepted slice and promotion of the hit branch, on gfx950.
//
// What is computed ([D3D] 前置知识: 异步起草与缓存命中 and 方法步骤详情 step 4): after the target
// verifies the current block, the verified prefix grows by the anchor and the accepted drafts
// (a0, d_1 .. d_{n_acc}); their drafter keys / values were computed by this round's packed forward as
// rows 0 .. n_acc of the request's block 0, whose in-block mask is causal, so they are exactly the
// prefix keys / values the next round needs. They are appended to the paged drafter cache and the
// prefix length advances by n_acc + 1. A cache hit reuses the hit branch's remaining draft: its
// packed tokens become the next round's current block.
//
// One workgroup per (request, slice row) copies the row's H_kv * d keys and values (16-byte pieces)
// to its page slot. The prefix length and the promoted block are written by a second pass, one
// workgroup per request, so that every copy reads the prefix length before it changes. A slice row
// without a cache slot (its page index past max_pages, or a page id outside [0, num_pages)) is
// skipped; the prefix then grows only by the rows before the first such row, and status reports it.
#include <limits.h>

#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kThreads = 256;

struct CommitArgs {
  const void *k_new, *v_new;
  void *k_cache, *v_cache;
  const int32_t *page_table;
  const int32_t *req_block_off;
  const int32_t *n_accepted;
  int32_t *prefix_len;
  const int32_t *hit;
  const int32_t *packed_tokens;
  int32_t *next_block;
  int32_t *status;
  int page_size, max_pages, num_pages;
  int n_req, B, row_bytes;  // row_bytes = H_kv * d * element size (multiple of 16)
};

__device__ __forceinline__ int slice_rows(const CommitArgs &a, int i) {
  return min(max(a.n_accepted[i], 0), a.B - 1) + 1;
}

// Whether slice row j of request i has a cache slot; its byte offset in the cache when it does.
__device__ __forceinline__ bool slot_of(const CommitArgs &a, int i, int j, size_t *off) {
  const int t = a.prefix_len[i] + j;
  if (t < 0 || t / a.page_size >= a.max_pages) return false;
  const int page = a.page_table[static_cast<size_t>(i) * a.max_pages + t / a.page_size];
  if (page < 0 || page >= a.num_pages) return false;
  *off = (static_cast<size_t>(page) * a.page_size + t % a.page_size) * a.row_bytes;
  return true;
}

__global__ __launch_bounds__(kThreads) void commit_copy_kernel(const CommitArgs a) {
  const int i = blockIdx.y, j = blockIdx.x;
  if (j >= slice_rows(a, i)) return;
  size_t dst;
  if (!slot_of(a, i, j, &dst)) return;
  const size_t src = static_cast<size_t>(a.req_block_off[i] * a.B + j) * a.row_bytes;
  const char *ks = static_cast<const char *>(a.k_new) + src;
  const char *vs = static_cast<const char *>(a.v_new) + src;
  char *kd = static_cast<char *>(a.k_cache) + dst;
  char *vd = static_cast<char *>(a.v_cache) + dst;
  for (int b = threadIdx.x * 16; b < a.row_bytes; b += kThreads * 16) {
    *reinterpret_cast<u32x4 *>(kd + b) = *reinterpret_cast<const u32x4 *>(ks + b);
    *reinterpret_cast<u32x4 *>(vd + b) = *reinterpret_cast<const u32x4 *>(vs + b);
  }
}

// One workgroup per request: status (0 = every slice row committed, 1 = a row had no cache slot),
// the new prefix length (grown by the rows before the first row without a slot), and the promoted
// block (-1 tokens on a miss).
__global__ __launch_bounds__(kThreads) void commit_finish_kernel(const CommitArgs a) {
  __shared__ int sh_first;
  const int i = blockIdx.x;
  const int n = slice_rows(a, i);
  if (threadIdx.x == 0) sh_first = n;
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < n) {
    size_t off;
    if (!slot_of(a, i, threadIdx.x, &off)) atomicMin(&sh_first, static_cast<int>(threadIdx.x));
  }
  __syncthreads();
  const int h = a.hit ? a.hit[i] : -1;
  if (a.next_block && static_cast<int>(threadIdx.x) < a.B) {
    const int blocks = a.req_block_off[i + 1] - a.req_block_off[i];
    const bool ok = h >= 1 && h < blocks && a.packed_tokens;
    a.next_block[static_cast<size_t>(i) * a.B + threadIdx.x] =
        ok ? a.packed_tokens[static_cast<size_t>(a.req_block_off[i] + h) * a.B + threadIdx.x] : -1;
  }
  if (threadIdx.x == 0) {
    const int first = sh_first;
    if (a.status) a.status[i] = first < n ? 1 : 0;
    a.prefix_len[i] += first;
  }
}

}  // namespace
}  // namespace d3d

extern "C" int kv_commit(d3d_dtype dtype, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                         const int32_t *page_table, int page_size, int max_pages, int num_pages,
                         const int32_t *req_block_off, int32_t *prefix_len, const int32_t *n_accepted, int n_req,
                         int block_size, int n_heads_kv, int head_dim, const int32_t *hit,
                         const int32_t *packed_tokens, int32_t *next_block, int32_t *status, hipStream_t stream) {
  using namespace d3d;
  if (dtype != D3D_BF16 && dtype != D3D_F32) return D3D_EINVAL;
  if (!k_new || !v_new || !k_cache || !v_cache || !page_table || !req_block_off || !prefix_len || !n_accepted)
    return D3D_EINVAL;
  if (n_req < 1 || block_size < 1 || block_size > kThreads || page_size < 1 || max_pages < 1 || num_pages < 1 ||
      n_heads_kv < 1 || head_dim < 1)
    return D3D_EINVAL;
  if (n_heads_kv > (1 << 16) || head_dim > (1 << 16)) return D3D_EUNSUPPORTED;  // keeps the row size below in range
  const long long row_bytes = static_cast<long long>(n_heads_kv) * head_dim * (dtype == D3D_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0 || row_bytes > (1ll << 30)) return D3D_EUNSUPPORTED;
  CommitArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.req_block_off = req_block_off;
  a.n_accepted = n_accepted;
  a.prefix_len = prefix_len;
  a.hit = hit;
  a.packed_tokens = packed_tokens;
  a.next_block = next_block;
  a.status = status;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.n_req = n_req;
  a.B = block_size;
  a.row_bytes = static_cast<int>(row_bytes);
  commit_copy_kernel<<<dim3(block_size, n_req), kThreads, 0, stream>>>(a);
  commit_finish_kernel<<<n_req, kThreads, 0, stream>>>(a);
  return launch_status();
}
