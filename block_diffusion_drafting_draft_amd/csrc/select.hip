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
//
// Sampled drafting at temperature T > 0 ([DScout] 实验结果 decodes at temperature 1): the token of a
// row is a draw from softmax(z / T), taken as the token with the largest score z_v / T + G_v where
// G_v = -ln(-ln u_v) is Gumbel noise (the Gumbel-max rule), ties to the lower id. u_v is a 24-bit
// uniform ((w >> 8) + 1/2) / 2^24 of word (v mod 4) of Philox4x32-10 at counter (v div 4, logits row,
// round, 2) under the 64-bit seed, so that any implementation of the same generator draws the same
// token. The winner is decided in fp64; a cheap fp32 score is a filter in front of it:
//   1. sample_chunk  grid (chunk, row), ALU-bound (one Philox block per 4 tokens, two base-2 logs
//                    per token, no per-token branch): each thread keeps its two best fp32 scores;
//                    when they lie more than a margin apart (the margin exceeds twice the fp32
//                    error) the best token is the thread's fp64 winner and only its fp64 score is
//                    computed, otherwise the thread re-scores its tokens within the margin in fp64.
//                    A 16-byte vector of tokens whose largest logit cannot reach the thread's second
//                    score even with the largest Gumbel value drawn (17.33) is skipped whole.
//   2. sample_merge  one workgroup per row: the best (fp64 score, id) of the chunks.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kThreads = 256;
// Chunk workgroups per call: two rounds of 8 per CU on 256 CUs. Against one round (2048), at 360 rows
// of 151936: top-k 31.1 -> 29.6 us, sampling 105 -> 89 us; at 5760 rows both unchanged; 8192 slower.
constexpr int kSelSlots = 4096;
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
  if (n_rows < 1 || vocab < 1 || vocab > kMaxVocab || k < 1 || k > kSelMaxK) return D3D_EINVAL;
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

// ------------------------------------------------------------------------------------------------
// Sampled drafting (Gumbel-max over counter-based uniforms)

struct SampCand {
  double s;    // fp64 score, -inf: nothing finite seen
  int32_t id;  // INT_MAX: empty
  int32_t pad;
};

struct SampArgs {
  const void *logits;
  const int32_t *rows;  // row r reads logits row rows[r] (NULL: row r); the row index is the counter word
  int32_t *out;         // [n_rows]
  int vocab, n_rows, chunks, chunk_len;
  float c2;     // fl(log2(e) / T): the filter's scale
  double t;     // T: the fp64 score divides by it
  uint32_t k0, k1, round;
  SampCand *part;  // [n_rows][chunks]
};

// The fp32 filter works in log2 units: z log2(e) / T - log2(-log2 u) orders the tokens exactly as the
// score z / T - ln(-ln u) does (a positive factor and a dropped constant, log2(ln 2)), and needs only
// the hardware base-2 logarithm (every argument here is a normal float).
constexpr float kGumbelCap2 = 25.5f;  // > 25.0, the largest Gumbel value drawn, in log2 units

// -log2 u for u = (m + 1/2) / 2^24, m = w >> 8, in fp32 with relative error below 1e-6: close to 1
// (where u itself is not representable in fp32) the series -log2(1 - t) = (t + t^2/2 + ...) / ln 2 in
// the exact complement t = (2^24 - 1 - m + 1/2) / 2^24 < 2^-4; elsewhere -log2 of the rounded u
// (|log2 u| > 0.093). Both forms, then a select: nearly every wavefront has lanes on both sides.
__device__ __forceinline__ float neg_log2_u32(uint32_t w) {
  const uint32_t m = w >> 8;
  const uint32_t n = 0xFFFFFFu - m;
  const float t = (static_cast<float>(n) + 0.5f) * 0x1p-24f;
  float p = 1.0f / 6.0f;
  p = fmaf(p, t, 0.2f);
  p = fmaf(p, t, 0.25f);
  p = fmaf(p, t, 1.0f / 3.0f);
  p = fmaf(p, t, 0.5f);
  p = fmaf(p, t, 1.0f);
  const float lg = -__builtin_amdgcn_logf((static_cast<float>(m) + 0.5f) * 0x1p-24f);
  return n < (1u << 20) ? p * t * 1.44269504f : lg;
}

// Filter margin, in log2 units: well above twice the fp32 score error (about 6e-6 + 3e-7 |score|).
__device__ __forceinline__ float samp_margin(float s) { return 1e-4f + 1e-6f * fabsf(s); }

// fp32 filter score of one token (z already cleaned: NaN -> -inf), in log2 units.
__device__ __forceinline__ float score32(const SampArgs &a, float z, uint32_t w) {
  return fmaf(z, a.c2, -__builtin_amdgcn_logf(neg_log2_u32(w)));
}

// fp64 score: z / T - ln(-ln u) with the exact uniform; this decides the token. Out of line: it
// runs for one token per thread and for the rare ambiguous re-walk.
__device__ __noinline__ double score64(const SampArgs &a, float z, uint32_t w) {
  const double u = (static_cast<double>(w >> 8) + 0.5) * 0x1p-24;
  return static_cast<double>(z) / a.t - log(-log(u));
}

__device__ __forceinline__ bool samp_better(double s, int id, double bs, int bi) {
  return id != INT_MAX && (bi == INT_MAX || s > bs || (s == bs && id < bi));
}

// The Philox word of token t of a row (word t mod 4 of block t div 4).
__device__ __forceinline__ uint32_t samp_word(const SampArgs &a, uint32_t ctr_row, int t) {
  const Philox4 ph = philox4x32_10(static_cast<uint32_t>(t / 4), ctr_row, a.round, 2u, a.k0, a.k1);
  const int e = t & 3;
  return e == 0 ? ph.x[0] : e == 1 ? ph.x[1] : e == 2 ? ph.x[2] : ph.x[3];
}

// A thread's two best fp32 scores and the token of the best. When the second lies more than the margin
// below the best, no other token of the thread can have a higher fp64 score than the best token (each
// fp32 score is within half the margin of the fp64 one); otherwise the thread is ambiguous and
// re-walks its tokens in fp64. Ids grow within a thread, so an equal score keeps the earlier token
// and lands in s2 (ambiguous). No per-token branch: a max, a min and one select.
struct SampTop2 {
  float s1, s2;
  int id1;
  __device__ __forceinline__ void init() {
    s1 = -INFINITY;
    s2 = -INFINITY;
    id1 = INT_MAX;
  }
  __device__ __forceinline__ void push(float s, int id) {
    id1 = s > s1 ? id : id1;
    s2 = fmaxf(s2, fminf(s, s1));
    s1 = fmaxf(s1, s);
  }
};

// Visits the thread's tokens of one chunk: f(z, id, word) for every token, or, where a whole
// 16-byte vector's largest logit cannot reach floor_of() even with the largest Gumbel value, none of
// the vector (its noise is not generated). floor_of() is re-read per vector: it rises as tokens pass.
template <typename T, bool VEC, typename F, typename FLOOR>
__device__ __forceinline__ void samp_walk(const SampArgs &a, const T *base, int begin, int end, uint32_t ctr_row,
                                          F &&f, FLOOR &&floor_of) {
  if constexpr (VEC) {
    constexpr int W = 16 / sizeof(T);  // tokens per vector: 8 (bf16) or 4 (fp32), W-aligned ids
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(base + begin);
    const int nvec = (end - begin) / W;
    constexpr int U = 4;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += kThreads * U) {
      u32x4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) buf[u] = vp[min(v0 + u * kThreads, nvec - 1)];  // clamped, in bounds
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kThreads;
        if (v < nvec) {
          float z[W];
          unpack_w<T, W>(buf[u], z);
          float zmax = -INFINITY;
#pragma unroll
          for (int e = 0; e < W; ++e) {
            z[e] = clean(z[e]);
            zmax = fmaxf(zmax, z[e]);
          }
          if (fmaf(zmax, a.c2, kGumbelCap2) < floor_of()) continue;
          const int id0 = begin + v * W;
#pragma unroll
          for (int q = 0; q < W / 4; ++q) {
            const Philox4 ph = philox4x32_10(static_cast<uint32_t>(id0 / 4 + q), ctr_row, a.round, 2u, a.k0, a.k1);
#pragma unroll
            for (int e = 0; e < 4; ++e) f(z[4 * q + e], id0 + 4 * q + e, ph.x[e]);
          }
        }
      }
    }
  } else {
    // scalar path: each thread takes the 4 consecutive tokens of one Philox block at a time
    for (int t0 = (begin & ~3) + 4 * static_cast<int>(threadIdx.x); t0 < end; t0 += 4 * kThreads) {
      const Philox4 ph = philox4x32_10(static_cast<uint32_t>(t0 / 4), ctr_row, a.round, 2u, a.k0, a.k1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
        if (t >= begin && t < end) f(clean(load_elem(base + t)), t, ph.x[e]);
      }
    }
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_chunk_kernel(const SampArgs a) {
  __shared__ double sh_s[kThreads / 64];
  __shared__ int sh_id[kThreads / 64];
  const int r = blockIdx.y, chunk = blockIdx.x;
  const int row = a.rows ? a.rows[r] : r;
  const T *base = static_cast<const T *>(a.logits) + static_cast<size_t>(row) * a.vocab;
  const int begin = chunk * a.chunk_len;
  const int end = min(begin + a.chunk_len, a.vocab);
  const uint32_t ctr_row = static_cast<uint32_t>(row);
  SampTop2 t2;
  t2.init();
  samp_walk<T, VEC>(
      a, base, begin, end, ctr_row, [&](float z, int id, uint32_t w) { t2.push(score32(a, z, w), id); },
      [&] { return t2.s2 - samp_margin(t2.s2); });
  // The skip test uses the second score: a skipped vector's fp32 scores lie below it, so none of its
  // tokens can be the best or change the second score.
  double bs = -INFINITY;
  int bi = INT_MAX;
  if (t2.id1 != INT_MAX && t2.s1 > -INFINITY) {
    if (t2.s2 < t2.s1 - samp_margin(t2.s1)) {
      const int t = t2.id1;
      bs = score64(a, clean(load_elem(base + t)), samp_word(a, ctr_row, t));
      bi = t;
    } else {
      // ambiguous (rare): every token of the thread within the margin of the best, in fp64, one
      // Philox block at a time (kept compact: this path is cold)
      const float lim = t2.s1 - samp_margin(t2.s1);
      const auto visit = [&](int t, uint32_t w) {
        if (t < begin || t >= end) return;
        const float z = clean(load_elem(base + t));
        if (!(score32(a, z, w) < lim)) {  // NaN limit (an infinite best): every token
          const double sd = score64(a, z, w);
          if (samp_better(sd, t, bs, bi)) {
            bs = sd;
            bi = t;
          }
        }
      };
      // the same tokens as the main walk: whole W-token vectors v = tid, tid + NT, ... (vector path)
      // or Philox blocks of 4 tokens (scalar path)
      constexpr int W = VEC ? 16 / static_cast<int>(sizeof(T)) : 4;
      const int first = VEC ? begin : (begin & ~3);
#pragma unroll 1
      for (int t0 = first + W * static_cast<int>(threadIdx.x); t0 < end; t0 += W * kThreads) {
#pragma unroll 1
        for (int q = 0; q < W / 4; ++q) {
          const Philox4 ph = philox4x32_10(static_cast<uint32_t>(t0 / 4 + q), ctr_row, a.round, 2u, a.k0, a.k1);
#pragma unroll 1
          for (int e = 0; e < 4; ++e) visit(t0 + 4 * q + e, ph.x[e]);
        }
      }
    }
  }
  // workgroup argmax of (fp64 score, id), ties to the lower id; an empty slot loses to everything
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    const double os = __shfl_xor(bs, o);
    const int oi = __shfl_xor(bi, o);
    if (samp_better(os, oi, bs, bi)) {
      bs = os;
      bi = oi;
    }
  }
  if (lane == 0) {
    sh_s[wave] = bs;
    sh_id[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) {
      if (samp_better(sh_s[w], sh_id[w], bs, bi)) {
        bs = sh_s[w];
        bi = sh_id[w];
      }
    }
    SampCand c;
    c.s = bs;
    c.id = bi;
    c.pad = 0;
    a.part[static_cast<size_t>(r) * a.chunks + chunk] = c;
  }
}

// One wavefront per row: the best chunk candidate (chunks are in id order; ties to the lower id). A
// row whose best score is -inf (every logit -inf or NaN) gets -1.
__global__ __launch_bounds__(64) void sample_merge_kernel(const SampArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  double bs = -INFINITY;
  int bi = INT_MAX;
  for (int c = lane; c < a.chunks; c += 64) {
    const SampCand x = a.part[static_cast<size_t>(r) * a.chunks + c];
    if (samp_better(x.s, x.id, bs, bi)) {
      bs = x.s;
      bi = x.id;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const double os = __shfl_xor(bs, o);
    const int oi = __shfl_xor(bi, o);
    if (samp_better(os, oi, bs, bi)) {
      bs = os;
      bi = oi;
    }
  }
  if (lane == 0) a.out[r] = bi == INT_MAX ? -1 : bi;
}

template <typename T, bool VEC>
void launch_sample(const SampArgs &a, hipStream_t stream) {
  sample_chunk_kernel<T, VEC><<<dim3(a.chunks, a.n_rows), kThreads, 0, stream>>>(a);
  sample_merge_kernel<<<a.n_rows, 64, 0, stream>>>(a);
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

extern "C" size_t draft_sample_workspace(int n_rows, int vocab) {
  d3d::SelPlan p;
  if (d3d::plan_select(n_rows, vocab, 1, &p) != D3D_OK) return 0;
  return d3d::align_up(sizeof(d3d::SampCand) * static_cast<size_t>(n_rows) * p.chunks, 256);
}

extern "C" int draft_sample(d3d_dtype dtype, const void *logits, int vocab, int n_rows, const int32_t *rows,
                            float temperature, uint64_t seed, uint32_t round, int32_t *out, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
  using namespace d3d;
  if (dtype != D3D_BF16 && dtype != D3D_F32) return D3D_EINVAL;
  if (!logits || !out) return D3D_EINVAL;
  if (!(temperature > 0.0f) || !(temperature < INFINITY)) return D3D_EINVAL;
  SelPlan p;
  if (plan_select(n_rows, vocab, 1, &p) != D3D_OK) return D3D_EINVAL;
  const size_t need = align_up(sizeof(SampCand) * static_cast<size_t>(n_rows) * p.chunks, 256);
  if (!ws || ws_bytes < need) return D3D_EWORKSPACE;
  SampArgs a;
  a.logits = logits;
  a.rows = rows;
  a.out = out;
  a.vocab = vocab;
  a.n_rows = n_rows;
  a.chunks = p.chunks;
  a.chunk_len = p.chunk_len;
  a.c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  a.t = static_cast<double>(temperature);
  a.k0 = static_cast<uint32_t>(seed);
  a.k1 = static_cast<uint32_t>(seed >> 32);
  a.round = round;
  a.part = static_cast<SampCand *>(ws);
  const size_t esize = dtype == D3D_BF16 ? 2 : 4;
  const bool vec = reinterpret_cast<uintptr_t>(logits) % 16 == 0 && (static_cast<size_t>(vocab) * esize) % 16 == 0;
  if (dtype == D3D_BF16) {
    if (vec)
      launch_sample<__bf16, true>(a, stream);
    else
      launch_sample<__bf16, false>(a, stream);
  } else {
    if (vec)
      launch_sample<float, true>(a, stream);
    else
      launch_sample<float, false>(a, stream);
  }
  return launch_status();
}
