// Top-k token selection over drafter logit rows on gfx950.
//
// What is computed ([D3D] 方法步骤详情 step 4 and 前置知识: 异步起草与缓存命中): the packed draft
// forward yields logits for every masked position of every branch block; greedy drafting keeps the
// most likely token of each (k = 1). Each of the first C-1 rejection positions gets F alternative
// anchors: the F most likely tokens of the draft distribution at that position other than the
// rejected draft token (its residual mass is zero, so it can never be the replacement), and the
// full-accept block's anchor is the most likely token of the position after the block.
// Order: larger logit first, ties to the lower token id (a strict total order, so the result is
// unique); NaN logits count as -inf.
//
// Design (HBM-bound for the drafted tokens: every logit of every row is read once):
//   1. topk_chunk  grid (chunk, row): 16-byte vector reads of a slice of one row; each thread keeps
//                  its K best (value, id) in registers, then k rounds of a workgroup argmax over the
//                  heads of the threads' lists. Partial k-list per (row, chunk).
//   2. topk_merge  one workgroup per row: the same rounds over the chunks' candidates (one per
//                  thread); writes the k ids.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kThreads = 256;
constexpr int kSelSlots = 2048;  // chunk workgroups resident at once: 8 per CU on 256 CUs
constexpr int kSelMinChunk = 1024;
constexpr int kSelMaxChunks = 32;
constexpr int kSelMaxK = 8;

struct Cand {
  float v;
  int32_t id;  // INT_MAX: empty slot (loses to every token, -inf logits included)
};

__device__ __forceinline__ bool beats(float v, int id, float w, int jd) { return v > w || (v == w && id < jd); }

struct SelArgs {
  const void *logits;
  const int32_t *rows;     // row r reads logits row rows[r] (NULL: row r)
  const int32_t *exclude;  // token skipped in row r (NULL or < 0: none)
  int32_t *out;
  const int32_t *out_off;  // row r's k ids start at out[out_off[r]] (NULL: r * k)
  int vocab, n_rows, k;
  int chunks, chunk_len;
  Cand *part;  // [n_rows][chunks][k]
};

// The K best elements seen so far, best first.
template <int K>
struct TopK {
  float v[K];
  int id[K];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      v[i] = -INFINITY;
      id[i] = INT_MAX;
    }
  }
  __device__ __forceinline__ void push(float z, int t) {
    if (!beats(z, t, v[K - 1], id[K - 1])) return;
    bool placed = false;
#pragma unroll
    for (int i = K - 1; i >= 0; --i) {
      const bool above = i > 0 && beats(z, t, v[i - 1], id[i - 1]);  // z goes above slot i-1
      if (!placed) {
        if (above) {
          v[i] = v[i - 1];
          id[i] = id[i - 1];
        } else {
          v[i] = z;
          id[i] = t;
          placed = true;
        }
      }
    }
  }
};

__device__ __forceinline__ float clean(float z) { return z != z ? -INFINITY : z; }

template <typename T, int W>
__device__ __forceinline__ void unpack_w(const u32x4 &w, float (&z)[W]);
template <>
__device__ __forceinline__ void unpack_w<__bf16, 8>(const u32x4 &w, float (&z)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    z[2 * k] = bf16_lo(w[k]);
    z[2 * k + 1] = bf16_hi(w[k]);
  }
}
template <>
__device__ __forceinline__ void unpack_w<float, 4>(const u32x4 &w, float (&z)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) z[k] = __uint_as_float(w[k]);
}

// The workgroup's k best of the threads' lists (each best first): k rounds in which every thread
// offers the head of its list, a workgroup argmax picks the best offer (ids are unique, so exactly
// one thread wins) and the winner pops it. Round j's winner is written by `emit(j, v, id)` (thread 0).
template <int K, typename EMIT>
__device__ __forceinline__ void select_rounds(TopK<K> &l, int k, float *sh_v, int *sh_id, EMIT emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = 0; j < k; ++j) {
    float bv = l.v[0];
    int bi = l.id[0];
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sh_v[wave] = bv;
      sh_id[wave] = bi;
    }
    __syncthreads();
    bv = sh_v[0];
    bi = sh_id[0];
    for (int w = 1; w < kThreads / 64; ++w)
      if (beats(sh_v[w], sh_id[w], bv, bi)) {
        bv = sh_v[w];
        bi = sh_id[w];
      }
    __syncthreads();
    if (threadIdx.x == 0) emit(j, bv, bi);
    if (l.id[0] == bi && bi != INT_MAX) {  // the winner pops its head
#pragma unroll
      for (int i = 0; i + 1 < K; ++i) {
        l.v[i] = l.v[i + 1];
        l.id[i] = l.id[i + 1];
      }
      l.v[K - 1] = -INFINITY;
      l.id[K - 1] = INT_MAX;
    }
  }
}

template <typename T, bool VEC, int K>
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(const SelArgs a) {
  __shared__ float sh_v[kThreads / 64];
  __shared__ int sh_id[kThreads / 64];
  const int r = blockIdx.y, chunk = blockIdx.x;
  const int row = a.rows ? a.rows[r] : r;
  const int ex = a.exclude ? a.exclude[r] : -1;
  const T *base = static_cast<const T *>(a.logits) + static_cast<size_t>(row) * a.vocab;
  const int begin = chunk * a.chunk_len;
  const int end = min(begin + a.chunk_len, a.vocab);
  TopK<K> acc;
  acc.init();
  if constexpr (VEC) {
    constexpr int W = 16 / sizeof(T);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(base + begin);
    const int nvec = (end - begin) / W;
    constexpr int U = 4;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += kThreads * U) {
      u32x4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = min(v0 + u * kThreads, nvec - 1);  // unconditional (clamped), used only if in range
        buf[u] = vp[v];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kThreads;
        if (v < nvec) {
          float z[W];
          unpack_w<T, W>(buf[u], z);
          const int id0 = begin + v * W;
          if constexpr (K == 1) {
            // argmax: the vector's maximum first (v_max ignores NaN; an all-NaN vector gives -inf),
            // and the first index holding it only when it beats the running best. Ids grow within a
            // thread, so an equal maximum loses unless the best is still the empty slot.
            const bool has_ex = static_cast<unsigned>(ex - id0) < static_cast<unsigned>(W);
            if (has_ex) {
#pragma unroll
              for (int e = 0; e < W; ++e) z[e] = id0 + e == ex ? NAN : z[e];
            }
            float vm = z[0];
#pragma unroll
            for (int e = 1; e < W; ++e) vm = fmaxf(vm, z[e]);
            vm = clean(vm);
            if (vm > acc.v[0] || (vm == acc.v[0] && acc.id[0] == INT_MAX)) {
              int first = INT_MAX;
#pragma unroll
              for (int e = W - 1; e >= 0; --e)
                if (clean(z[e]) == vm && id0 + e != ex) first = id0 + e;
              if (first != INT_MAX) {
                acc.v[0] = vm;
                acc.id[0] = first;
              }
            }
          } else {
#pragma unroll
            for (int e = 0; e < W; ++e) {
              if (id0 + e != ex) acc.push(clean(z[e]), id0 + e);
            }
          }
        }
      }
    }
  } else {
    for (int t = begin + threadIdx.x; t < end; t += kThreads)
      if (t != ex) acc.push(clean(load_elem(base + t)), t);
  }
  Cand *dst = a.part + (static_cast<size_t>(r) * a.chunks + chunk) * a.k;
  select_rounds<K>(acc, a.k, sh_v, sh_id, [&](int j, float v, int id) {
    Cand c;
    c.v = v;
    c.id = id;
    dst[j] = c;
  });
}

template <int K>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const SelArgs a) {
  __shared__ float sh_v[kThreads / 64];
  __shared__ int sh_id[kThreads / 64];
  const int r = blockIdx.x;
  const int n = a.chunks * a.k;  // <= kSelMaxChunks * kSelMaxK = kThreads candidates, one per thread
  TopK<K> l;
  l.init();
  const Cand c = a.part[static_cast<size_t>(r) * n + min(static_cast<int>(threadIdx.x), n - 1)];
  if (static_cast<int>(threadIdx.x) < n) {
    l.v[0] = c.v;
    l.id[0] = c.id;
  }
  const size_t o = a.out_off ? static_cast<size_t>(a.out_off[r]) : static_cast<size_t>(r) * a.k;
  select_rounds<K>(l, a.k, sh_v, sh_id, [&](int j, float, int id) { a.out[o + j] = id == INT_MAX ? -1 : id; });
}

struct SelPlan {
  int chunks, chunk_len;
  size_t total;
};

int plan_select(int n_rows, int vocab, int k, SelPlan *p) {
  if (n_rows < 1 || vocab < 1 || k < 1 || k > kSelMaxK) return D3D_EINVAL;
  int chunks = std::max(1, kSelSlots / n_rows);
  chunks = std::min(chunks, (vocab + kSelMinChunk - 1) / kSelMinChunk);
  chunks = std::min(chunks, kSelMaxChunks);
  int len = (vocab + chunks - 1) / chunks;
  len = (len + 63) / 64 * 64;
  p->chunk_len = len;
  p->chunks = (vocab + len - 1) / len;
  p->total = align_up(sizeof(Cand) * static_cast<size_t>(n_rows) * p->chunks * k, 256);
  return D3D_OK;
}

template <typename T, bool VEC>
void launch_select(const SelArgs &a, hipStream_t stream) {
  // per-thread lists just deep enough for k (a thread's share of the k best is at most k elements)
  const dim3 grid(a.chunks, a.n_rows);
  if (a.k == 1) {
    topk_chunk_kernel<T, VEC, 1><<<grid, kThreads, 0, stream>>>(a);
    topk_merge_kernel<1><<<a.n_rows, kThreads, 0, stream>>>(a);
  } else if (a.k == 2) {
    topk_chunk_kernel<T, VEC, 2><<<grid, kThreads, 0, stream>>>(a);
    topk_merge_kernel<2><<<a.n_rows, kThreads, 0, stream>>>(a);
  } else if (a.k <= 4) {
    topk_chunk_kernel<T, VEC, 4><<<grid, kThreads, 0, stream>>>(a);
    topk_merge_kernel<4><<<a.n_rows, kThreads, 0, stream>>>(a);
  } else {
    topk_chunk_kernel<T, VEC, kSelMaxK><<<grid, kThreads, 0, stream>>>(a);
    topk_merge_kernel<kSelMaxK><<<a.n_rows, kThreads, 0, stream>>>(a);
  }
}

}  // namespace
}  // namespace d3d

extern "C" size_t draft_topk_workspace(int n_rows, int vocab, int k) {
  d3d::SelPlan p;
  if (d3d::plan_select(n_rows, vocab, k, &p) != D3D_OK) return 0;
  return p.total;
}

extern "C" int draft_topk(d3d_dtype dtype, const void *logits, int vocab, int n_rows, const int32_t *rows,
                          const int32_t *exclude, int k, int32_t *out, const int32_t *out_off, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  using namespace d3d;
  if (dtype != D3D_BF16 && dtype != D3D_F32) return D3D_EINVAL;
  if (!logits || !out) return D3D_EINVAL;
  SelPlan p;
  if (plan_select(n_rows, vocab, k, &p) != D3D_OK) return D3D_EINVAL;
  if (!ws || ws_bytes < p.total) return D3D_EWORKSPACE;
  SelArgs a;
  a.logits = logits;
  a.rows = rows;
  a.exclude = exclude;
  a.out = out;
  a.out_off = out_off;
  a.vocab = vocab;
  a.n_rows = n_rows;
  a.k = k;
  a.chunks = p.chunks;
  a.chunk_len = p.chunk_len;
  a.part = static_cast<Cand *>(ws);
  const size_t esize = dtype == D3D_BF16 ? 2 : 4;
  const bool vec = reinterpret_cast<uintptr_t>(logits) % 16 == 0 && (static_cast<size_t>(vocab) * esize) % 16 == 0;
  if (dtype == D3D_BF16) {
    if (vec)
      launch_select<__bf16, true>(a, stream);
    else
      launch_select<__bf16, false>(a, stream);
  } else {
    if (vec)
      launch_select<float, true>(a, stream);
    else
      launch_select<float, false>(a, stream);
  }
  return launch_status();
}
