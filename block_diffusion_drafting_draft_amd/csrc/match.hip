// Branch-cache match, descriptor builder and status strings.
//
// [D3D] 前置知识: 异步起草与缓存命中: after verification, a branch drafted during the previous
// round is reused when the verified prefix equals its start. With the accepted slice a0, y_1..y_n
// and the resampled or bonus token t, the branch of rejection position r with anchor a reproduces
// that prefix exactly when r = n + 1 and a = t. The first such block in pack order is returned.
#include <algorithm>

#include "d3d_internal.h"

namespace d3d {
namespace {

// One wavefront per request.
__global__ __launch_bounds__(256) void match_kernel(const d3d_block_desc *descs, int total_blocks,
                                                    const int32_t *off, int n_req,
                                                    const int32_t *n_acc, const int32_t *next,
                                                    int32_t *hit) {
  const int i = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= n_req) return;
  const int b0 = min(max(off[i], 0), total_blocks);
  const int b1 = min(max(off[i + 1], b0), total_blocks);
  const int found = match_request(descs, b0, b1, n_acc[i] + 1, next[i]);
  if (lane == 0) hit[i] = found;
}

// One thread per descriptor: request i = t / per, block b = t mod per, in the pack order of the
// host builder ([D3D] 方法步骤详情 step 4: the current block, then the F anchors of rejection
// positions k = 1..C-1, k-major, then the full-accept block).
__global__ __launch_bounds__(256) void build_descs_kernel(int n_req, int B, int C, int F, const int32_t *prefix_len,
                                                          const int32_t *cur_anchor, const int32_t *alt_anchors,
                                                          d3d_block_desc *out, int32_t *req_block_off) {
  const int per = (C - 1) * F + 2;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (req_block_off && t <= n_req) req_block_off[t] = t * per;
  if (t >= n_req * per) return;
  const int i = t / per, b = t - i * per;
  const int32_t *alt = alt_anchors + static_cast<size_t>(i) * (per - 1);
  d3d_block_desc d;
  d.prefix_len = prefix_len[i];
  if (b == 0) {
    d.rej_pos = 0;
    d.anchor = cur_anchor[i];
    d.flags = static_cast<int32_t>(D3D_BLOCK_CAUSAL);
  } else if (b < per - 1) {
    d.rej_pos = (b - 1) / F + 1;
    d.anchor = alt[b - 1];  // (k - 1) F + f
    d.flags = 0;
  } else {
    d.rej_pos = B;
    d.anchor = alt[(C - 1) * F];
    d.flags = 0;
  }
  out[t] = d;
}

}  // namespace
}  // namespace d3d

extern "C" int d3d_build_branch_descs_device(int n_req, int block_size, int coverage, int fanout,
                                             const int32_t *prefix_len, const int32_t *cur_anchor,
                                             const int32_t *alt_anchors, d3d_block_desc *out,
                                             int32_t *req_block_off, hipStream_t stream) {
  if (n_req < 1 || !prefix_len || !cur_anchor || !alt_anchors || !out) return D3D_EINVAL;
  if (block_size < 1 || block_size > 64 || coverage < 2 || coverage > block_size || fanout < 1) return D3D_EINVAL;
  const long long per = static_cast<long long>(coverage - 1) * fanout + 2;
  if (n_req > ((1ll << 31) - 257) / per) return D3D_EINVAL;  // n_req * per < 2^31 - 256: an int32 index per thread
  const int total = static_cast<int>(per * n_req);
  const int grid = (std::max(total, n_req + 1) + 255) / 256;
  d3d::build_descs_kernel<<<grid, 256, 0, stream>>>(n_req, block_size, coverage, fanout, prefix_len, cur_anchor,
                                                    alt_anchors, out, req_block_off);
  return d3d::launch_status();
}

extern "C" int branch_cache_match(const d3d_block_desc *descs, int total_blocks,
                                  const int32_t *req_block_off, int n_req,
                                  const int32_t *n_accepted, const int32_t *next_token,
                                  int32_t *hit_branch, hipStream_t stream) {
  if (!descs || !req_block_off || !n_accepted || !next_token || !hit_branch) return D3D_EINVAL;
  if (n_req < 1 || total_blocks < 1) return D3D_EINVAL;
  const int per_block = 4;  // requests (wavefronts) per workgroup
  d3d::match_kernel<<<n_req / per_block + (n_req % per_block != 0), 64 * per_block, 0, stream>>>(
      descs, total_blocks, req_block_off, n_req, n_accepted, next_token, hit_branch);
  return d3d::launch_status();
}

extern "C" int d3d_build_branch_descs(int block_size, int coverage, int fanout, int prefix_len,
                                      int32_t cur_anchor, const int32_t *alt_anchors,
                                      d3d_block_desc *out, int cap, int *n_out) {
  if (block_size < 1 || block_size > 64 || coverage < 2 || coverage > block_size || fanout < 1 ||
      prefix_len < 0 || !alt_anchors || !out || !n_out)
    return D3D_EINVAL;
  const long long n = static_cast<long long>(coverage - 1) * fanout + 2;
  if (n > cap) return D3D_EINVAL;
  int w = 0;
  out[w++] = d3d_block_desc{prefix_len, 0, cur_anchor, static_cast<int32_t>(D3D_BLOCK_CAUSAL)};
  for (int k = 1; k < coverage; ++k)
    for (int f = 0; f < fanout; ++f)
      out[w++] = d3d_block_desc{prefix_len, k, alt_anchors[(k - 1) * fanout + f], 0};
  out[w++] = d3d_block_desc{prefix_len, block_size, alt_anchors[(coverage - 1) * fanout], 0};
  *n_out = w;
  return D3D_OK;
}

extern "C" int d3d_build_branch_descs_batch(int n_req, int block_size, int coverage, int fanout,
                                            const int32_t *prefix_len, const int32_t *cur_anchor,
                                            const int32_t *alt_anchors, d3d_block_desc *out, int cap,
                                            int32_t *req_block_off) {
  if (n_req < 1 || !prefix_len || !cur_anchor || !alt_anchors || !out || !req_block_off) return D3D_EINVAL;
  if (block_size < 1 || block_size > 64 || coverage < 2 || coverage > block_size || fanout < 1) return D3D_EINVAL;
  const long long per = static_cast<long long>(coverage - 1) * fanout + 2;
  if (cap < 1 || per > cap || n_req > cap / per) return D3D_EINVAL;  // per * n_req > cap, without overflow
  for (int i = 0; i < n_req; ++i)
    if (prefix_len[i] < 0) return D3D_EINVAL;
  const int na = static_cast<int>(per - 1);  // anchors per request
  req_block_off[0] = 0;
  for (int i = 0; i < n_req; ++i) {
    int n = 0;
    const int st = d3d_build_branch_descs(block_size, coverage, fanout, prefix_len[i], cur_anchor[i],
                                          alt_anchors + static_cast<size_t>(i) * na, out + per * i,
                                          static_cast<int>(per), &n);
    if (st != D3D_OK) return st;
    req_block_off[i + 1] = req_block_off[i] + n;
  }
  return D3D_OK;
}

extern "C" const char *d3d_status_string(int status) {
  switch (status) {
    case D3D_OK: return "ok";
    case D3D_EINVAL: return "invalid argument or shape";
    case D3D_EUNSUPPORTED: return "unsupported configuration";
    case D3D_EHIP: return "HIP launch error";
    case D3D_EWORKSPACE: return "workspace missing or too small";
    case D3D_ESCRATCH: return "the call needs more workspace than the allocation-free entry point's static scratch";
    default: return "unknown status";
  }
}
