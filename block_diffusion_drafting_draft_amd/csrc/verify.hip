// Speculative-sampling verification on gfx950.
//
// What is computed ([D3D] 前置知识: 投机解码; [DScout] 前置知识: 推测解码, 平均接受长度 MAT,
// 接受加权损失 AWL 与推测采样接受规则): per request, alpha_j = min(1, P_j(y_j)/Q_j(y_j)) for every
// draft, the first rejection against Philox uniforms, the residual max(0, P - Q) or bonus draw,
// the prefix-survival products S(k) and tau = 1 + sum_k S(k).
//
// Design (HBM-bound: the whole vocabulary of every row is read once; everything after that pass
// touches one or two rows per request and is latency-bound, so it is built from few dependent
// memory round trips):
//   1. stats   grid (chunk, row), one round of resident workgroups: one coalesced 16-byte-vector
//              pass over a slice of one logit row: sum of exp((z - ref)/T) against a reference
//              logit of the slice with fp32 exp2 per element and fp64 accumulation per thread (the
//              maximum and first argmax when greedy), and the logit at the row's draft token when
//              the slice holds it. Partial per (row, chunk).
//   2. sample  grid (sample chunk, request): every workgroup stages its request's partials in
//              LDS, merges each row in fp64, forms alpha_j from fp64 scalars, draws the Philox
//              uniforms, finds the first rejection, S(k) and tau (the chunk-0 workgroup stores
//              them). Then, over its 2048-token slice of the one or two rows the draw needs
//              (target row j*, and draft row j* after a rejection), in fp64: the slice's shares of
//              the row sums Sp = sum exp(ap), Sq = sum exp(aq) (ap = (z^P - ref)/T, likewise aq)
//              and the sums A, B of exp(ap), exp(aq) over the tokens with P > Q. Which tokens those
//              are is read off ap - aq against an estimate of log(Sp/Sq) from the statistics pass;
//              tokens within a band of it are only counted. Since Sp and Sq are common factors,
//              the slice's residual mass is exactly A/Sp - B/Sq, so no pass has to wait for the
//              row sums before it can weigh its tokens.
//   3. pick    the request's last workgroup to finish its slice (an atomic count per request,
//              zeroed by the statistics pass) forms Sp, Sq and every slice mass (a slice with
//              tokens in the band, or every slice if the estimate missed the band, is weighed
//              again token by token), takes the prefix over the slice masses and scans the slice
//              that holds u'Z, returning the smallest token whose inclusive cumulative mass
//              exceeds u'Z.
// The sample pass reads 8 consecutive tokens per thread with one 16-byte load per row.
// Nothing returns to the host; the sample pass is stream-ordered after the statistics pass.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Statistics workgroups per call (upper bound; the chunk count per row follows from it). Per-workgroup
// start stamps of the serving batch's 496 rows show that 1984 workgroups (4 per row) do not all start
// at once: the last ones wait ~15 us for early ones to finish, a second partial round. At 992 (2 per
// row) every workgroup starts within 1 us, and the call measured 70.6 -> 68.1 us cold, 62.7 -> 61.7
// warm (1488 workgroups: 69.4 / 60.8).
constexpr int kStatSlots = 1024;
// Threads per statistics workgroup: 512 against 256 took the async verify from 21.0 to 20.2 us
// in-graph (twice the threads per chunk of its 248 workgroups); the serving batch did not move.
constexpr int kStatThreads = 512;
constexpr int kStatMinChunk = 1024;
// Per row: more chunks only lengthen decide's staging and row merge. At a single request's 31 rows
// (the async round) 8 chunks measured ~1 us faster in the round than 32, and no slower alone.
constexpr int kStatMaxChunks = 8;
constexpr int kSampleElems = 8;                        // tokens per thread in the sample passes
constexpr int kSampleChunk = kThreads * kSampleElems;  // tokens per sample workgroup
constexpr int kMaxSampleChunks = 1024;
constexpr int kMaxReqPartials = 2048;  // stats partials of one request staged in LDS by decide
constexpr double kNear = 1e-6;
// Half-width of the band around the estimate of log(Sp/Sq) inside which a token's side (P > Q or
// not) is left to the exact row sums. The estimate comes from fp32 exp2 terms (per-term relative
// error below 1.3e-6, from the argument's rounding at |x| <= 8 and the exp2 itself), so it is
// within 2.6e-6 of the exact value; the pick checks that it is within half the band.
constexpr double kRhoBand = 0x1p-16;

struct StatPartial {
  float max;    // greedy: the chunk maximum; sampling: the chunk's reference logit (see RowAcc)
  int32_t aux;  // greedy: first argmax; sampling: bits of the logit at the row's draft token when
                // this chunk holds that token, else 0
  double sum;   // sum of exp((z - max) / T) over the chunk
};

enum SampleMode : int32_t { kDone = 0, kResidual = 1, kBonus = 2 };

struct SampleState {
  int32_t mode;
  int32_t tgt_row;  // global target row index (request * (n_draft + 1) + j)
  int32_t drf_row;  // global draft row index (request * n_draft + j)
  float max_p;
  float max_q;
  uint32_t near;  // flags bit 0 of the acceptance decisions
  double u;
  double rho;  // residual draw: log(Sp/Sq) estimated from the statistics partials
};

// One (request, sample chunk) of the sample pass: the slice's shares of Sp and Sq; A and B over its
// tokens with ap - aq above the band (A only, = sp, for the bonus draw); the count of tokens in it.
struct SampleRec {
  double sp, sq, a, b, amb;
};
constexpr int kRecFields = 5;
// Per-request counters sit 256 bytes apart: 75 workgroups of each request increment theirs at
// about the same time, and counters sharing a cache line serialise every request's increments.
constexpr int kCounterStride = 64;

struct VerifyArgs {
  const void *target;
  const void *draft;
  const int32_t *tokens;
  int n_req, n_draft, vocab, n_tgt_rows;
  int chunks, chunk_len;
  int s_chunks;
  float c_log2;    // log2(e) / T
  double inv_t;    // 1 / T (fp64)
  uint64_t seed;
  uint32_t round;
  int greedy;
  int32_t *n_acc;
  int32_t *next_token;
  float *alpha;
  float *survival;
  float *tau;
  uint32_t *flags;
  StatPartial *stats;
  SampleRec *rec;     // [n_req][s_chunks]
  uint32_t *counter;  // [n_req * kCounterStride] sample workgroups done; zeroed by the statistics pass
  // optional cache match of the verified outcome against the round's branch descriptors
  const d3d_block_desc *descs;
  const int32_t *req_block_off;
  int total_blocks;
  int32_t *hit;
};

// The cache match of request i once its outcome is known (one whole wavefront).
__device__ __forceinline__ void match_outcome(const VerifyArgs &a, int i, int n_acc, int tok) {
  const int b0 = min(max(a.req_block_off[i], 0), a.total_blocks);
  const int b1 = min(max(a.req_block_off[i + 1], b0), a.total_blocks);
  const int found = match_request(a.descs, b0, b1, n_acc + 1, tok);
  if ((threadIdx.x & 63) == 0) a.hit[i] = found;
}

// ------------------------------------------------------------------------------------------------
// block reductions (256 threads = 4 wavefronts)
// ------------------------------------------------------------------------------------------------
template <int NW = kWaves>
__device__ __forceinline__ float block_max(float v, float *sh) {
  v = wave::reduce(v, 64, wave::Max{});
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < NW; ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}

template <int NW = kWaves>
__device__ __forceinline__ double block_sum(double v, double *sh) {
  v = wave::reduce(v, 64, wave::Add{});
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
  for (int i = 1; i < NW; ++i) r += sh[i];
  __syncthreads();
  return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_min_int(int v, int *sh) {
  v = wave::reduce(v, 64, wave::Min{});
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
  for (int i = 1; i < NW; ++i) r = min(r, sh[i]);
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------------------------------------
// 1. stats
// ------------------------------------------------------------------------------------------------
// Per-thread accumulator of one row slice. Greedy: the running maximum and its first index.
// Sampling: a reference value m (an element of the slice) and s = sum of exp((z - m)/T) relative to
// it. The reference is not kept at the running maximum element by element: a later logit above it
// simply contributes a term above 1. It moves up to a group's maximum once a group's fp32 sum
// reaches 2^8, so every term that is kept satisfies (z - m) log2(e)/T < 8. That bound is what keeps
// the sum accurate: the fp32 rounding of the exponent argument x is relative, an error of about
// |x| 2^-24 ln 2 in the term, and the terms that carry the row's mass are the ones near the top.
// (Letting x grow to ~120 before moving, at T = 0.25 on a 151936-token row, put 3e-6 into alpha.)
// Consumers only need some reference, not the maximum.
struct GreedyAcc {
  float m = -INFINITY;
  int arg = INT_MAX;

  // Fold N consecutive elements starting at token index `idx` (z in fp32, exact for bf16).
  template <int N>
  __device__ __forceinline__ void fold(const float (&z)[N], int idx, float, double) {
    float vm = z[0];
#pragma unroll
    for (int k = 1; k < N; ++k) vm = fmaxf(vm, z[k]);
    if (vm > m) {
      m = vm;
      int first = N - 1;
#pragma unroll
      for (int k = N - 1; k >= 0; --k)
        if (z[k] == vm) first = k;
      arg = idx + first;
    }
  }
};

struct SumAcc {
  float m = -INFINITY;
  double s = 0.0;

  template <int N>
  __device__ __forceinline__ float group_sum(const float (&z)[N], float c) const {
    float part = __builtin_amdgcn_exp2f((z[0] - m) * c);
#pragma unroll
    for (int k = 1; k < N; ++k) part += __builtin_amdgcn_exp2f((z[k] - m) * c);
    return part;
  }

  // With no finite logit seen yet m = -inf, and a group holding one makes the sum +inf or NaN, so
  // the one test below also sets the first reference. (The argument is formed as (z - m) * c rather
  // than z * c - m * c: with m * c the reference itself would overflow fp32 at tiny temperatures.)
  template <int N>
  __device__ __forceinline__ void fold(const float (&z)[N], int, float c, double inv_t) {
    float part = group_sum(z, c);
    if (!(part < 0x1p8f)) {
      float vm = z[0];
#pragma unroll
      for (int k = 1; k < N; ++k) vm = fmaxf(vm, z[k]);
      if (vm == -INFINITY) return;  // no finite logit in the group, none before it either
      s = m == -INFINITY ? 0.0 : s * exp_fp64((static_cast<double>(m) - vm) * inv_t);
      m = vm;
      part = group_sum(z, c);
    }
    s += static_cast<double>(part);
  }
};

template <bool GREEDY>
using RowAcc = typename std::conditional<GREEDY, GreedyAcc, SumAcc>::type;

__device__ __forceinline__ void unpack(const u32x4 &w, float (&z)[8], const __bf16 *) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    z[2 * k] = bf16_lo(w[k]);
    z[2 * k + 1] = bf16_hi(w[k]);
  }
}
__device__ __forceinline__ void unpack(const u32x4 &w, float (&z)[4], const float *) {
#pragma unroll
  for (int k = 0; k < 4; ++k) z[k] = __uint_as_float(w[k]);
}

// The draft token a row judges (target row j < n_draft or draft row j), or -1 for the bonus row.
__device__ __forceinline__ int row_token(const VerifyArgs &a, int row) {
  int i, j;
  if (row < a.n_tgt_rows) {
    i = row / (a.n_draft + 1);
    j = row - i * (a.n_draft + 1);
    if (j == a.n_draft) return -1;
  } else {
    const int r = row - a.n_tgt_rows;
    i = r / a.n_draft;
    j = r - i * a.n_draft;
  }
  return min(max(a.tokens[static_cast<size_t>(i) * a.n_draft + j], 0), a.vocab - 1);
}

template <typename T, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kStatThreads) void stats_kernel(const VerifyArgs a) {
  constexpr int NW = kStatThreads / 64;
  __shared__ float sh_f[NW];
  __shared__ double sh_d[NW];
  __shared__ int sh_i[NW];
  const int row = blockIdx.y;
  const int chunk = blockIdx.x;
  const T *base = row < a.n_tgt_rows
                      ? static_cast<const T *>(a.target) + static_cast<size_t>(row) * a.vocab
                      : static_cast<const T *>(a.draft) +
                            static_cast<size_t>(row - a.n_tgt_rows) * a.vocab;
  const int begin = chunk * a.chunk_len;
  const int end = min(begin + a.chunk_len, a.vocab);
  // the logit at the row's draft token, read up front (a wave-uniform load) when this chunk holds it
  const int y = GREEDY ? -1 : row_token(a, row);
  const bool has_y = y >= begin && y < end;
  float zy = 0.f;
  if (has_y) zy = load_elem(base + y);
  RowAcc<GREEDY> acc;
  if constexpr (VEC) {
    constexpr int W = 16 / sizeof(T);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(base + begin);
    const int nvec = (end - begin) / W;
    constexpr int U = 4;
    // steps of U vectors per thread with every load in range (no per-load test), then the rest
    int v = threadIdx.x;
    for (; v + (U - 1) * kStatThreads < nvec; v += U * kStatThreads) {
      u32x4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) buf[u] = vp[v + u * kStatThreads];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float z[W];
        unpack(buf[u], z, static_cast<const T *>(nullptr));
        acc.fold(z, begin + (v + u * kStatThreads) * W, a.c_log2, a.inv_t);
      }
    }
    for (; v < nvec; v += kStatThreads) {
      float z[W];
      unpack(vp[v], z, static_cast<const T *>(nullptr));
      acc.fold(z, begin + v * W, a.c_log2, a.inv_t);
    }
  } else {
    for (int idx = begin + threadIdx.x; idx < end; idx += kStatThreads) {
      float z[1] = {load_elem(base + idx)};
      acc.fold(z, idx, a.c_log2, a.inv_t);
    }
  }
  const float m = block_max<NW>(acc.m, sh_f);
  StatPartial out;
  out.max = m;
  if constexpr (GREEDY) {
    out.aux = block_min_int<NW>(acc.m == m ? acc.arg : INT_MAX, sh_i);
    out.sum = 0.0;
  } else {
    const double mine =
        acc.m == -INFINITY ? 0.0 : acc.s * exp_fp64((static_cast<double>(acc.m) - m) * a.inv_t);
    out.sum = block_sum<NW>(mine, sh_d);
    out.aux = has_y ? __float_as_int(zy) : 0;
  }
  if (threadIdx.x == 0) {
    a.stats[static_cast<size_t>(row) * a.chunks + chunk] = out;
    // the sample pass counts its finished workgroups per request from zero
    if (!GREEDY && chunk == 0 && row < a.n_req) a.counter[static_cast<size_t>(row) * kCounterStride] = 0u;
  }
}

// ------------------------------------------------------------------------------------------------
// 2. decide (run by every workgroup of the lse pass for its request)
// ------------------------------------------------------------------------------------------------
// Local rows 0..nd are the request's target rows, nd+1..2nd its draft rows (greedy: target only).
struct ReqRows {
  float max[127];
  double logsum[127];  // log of the row's sum of exp((z - max) / T)
  double lp[127];      // log-probability of the row's draft token (rows with one)
  int arg[127];
  int tok[63];
  double u[64];        // the request's uniforms: u_j (j < n_draft), u' (j = n_draft)
};

// Loads the request's stats partials into LDS (one round trip), merges every row with a group of
// g lanes (g a power of two, so a group never straddles a wavefront; lanes stride over chunks in
// increasing order, which keeps the first argmax), then wavefront 0 takes the decisions. The
// results are identical in every workgroup of the request; only `store` writes them out.
__device__ __forceinline__ void decide_request(const VerifyArgs &a, int i, StatPartial *part, ReqRows &rr,
                               SampleState *sh_state, bool store) {
  const int nd = a.n_draft;
  const int C = a.chunks;
  const int n_rows = a.greedy ? nd + 1 : 2 * nd + 1;
  const int n_tp = (nd + 1) * C;
  const int n_all = n_rows * C;
  const StatPartial *tgt = a.stats + static_cast<size_t>(i) * n_tp;
  const StatPartial *drf = a.stats + static_cast<size_t>(a.n_tgt_rows) * C + static_cast<size_t>(i) * nd * C;
  {
    // every load is issued (indexes clamped) before any LDS store, so this is one round trip
    constexpr int K = kMaxReqPartials / kThreads;
    static_assert(sizeof(StatPartial) == sizeof(u32x4), "a partial moves as one 16-byte vector");
    u32x4 tmp[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int t = min(static_cast<int>(threadIdx.x) + k * kThreads, n_all - 1);
      const StatPartial *src = t < n_tp ? tgt + t : drf + (t - n_tp);
      tmp[k] = *reinterpret_cast<const u32x4 *>(src);
    }
    if (threadIdx.x < nd)
      rr.tok[threadIdx.x] = min(max(a.tokens[static_cast<size_t>(i) * nd + threadIdx.x], 0), a.vocab - 1);
    // the request's Philox uniforms, drawn while the partials are in flight (they depend on no
    // logit): lane j < n_draft draws u_j, lane n_draft draws u'
    if (!a.greedy && threadIdx.x <= nd)
      rr.u[threadIdx.x] = threadIdx.x < nd ? philox_uniform(a.seed, threadIdx.x, static_cast<uint32_t>(i), a.round, 0u)
                                           : philox_uniform(a.seed, 0u, static_cast<uint32_t>(i), a.round, 1u);
    u32x4 *dst = reinterpret_cast<u32x4 *>(part);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int t = static_cast<int>(threadIdx.x) + k * kThreads;
      if (t < n_all) dst[t] = tmp[k];
    }
  }
  __syncthreads();
  int g = 64;
  while (g > 1 && n_rows * g > kThreads) g >>= 1;
  const int r = threadIdx.x / g, sub = threadIdx.x % g;
  // the row's maximum reference (and, greedy, the first argmax: chunks are visited in increasing
  // order per lane and ties go to the lowest index), then one independent exp per chunk
  float m = -INFINITY;
  int arg = INT_MAX;
  if (r < n_rows) {
    for (int c = sub; c < C; c += g) {
      const StatPartial q = part[r * C + c];
      if (q.max > m) {
        m = q.max;
        arg = q.aux;
      }
    }
  }
  const float wm = wave::reduce(m, g, wave::Max{});
  const int warg = wave::reduce(m == wm ? arg : INT_MAX, g, wave::Min{});
  double ws = 0.0;
  if (!a.greedy && r < n_rows && wm != -INFINITY) {
    for (int c = sub; c < C; c += g) {
      const StatPartial q = part[r * C + c];
      if (q.max != -INFINITY) ws += q.sum * exp_fp64((static_cast<double>(q.max) - wm) * a.inv_t);
    }
  }
  ws = wave::reduce(ws, g, wave::Add{});
  if (sub == 0 && r < n_rows) {
    rr.max[r] = wm;
    rr.arg[r] = warg;
    if (!a.greedy) {
      // per row, in parallel: the log of the row sum and the draft token's log-probability
      // log P_j(y) = (z_y - ref)/T - log sum_j, so the decision needs no exp, division or log
      const double ls = log(ws);
      rr.logsum[r] = ls;
      const int j = r <= nd ? r : r - nd - 1;
      if (j < nd) {
        const float zy = __int_as_float(part[r * C + rr.tok[j] / a.chunk_len].aux);
        rr.lp[r] = wm == -INFINITY ? -INFINITY : (static_cast<double>(zy) - wm) * a.inv_t - ls;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // lane j judges draft j
  const int lane = threadIdx.x;
  const int j = lane;
  double alpha = 1.0, u = 1.0;
  if (j < nd) {
    if (a.greedy) {
      // a row of -inf logits has no argmax (INT_MAX): its draft is rejected
      alpha = (rr.tok[j] == rr.arg[j]) ? 1.0 : 0.0;
    } else {
      // alpha = min(1, P/Q) = min(1, exp(log P - log Q)); 1 when Q(y) is zero in fp64 (its
      // log-probability below ln 2^-1075, where exp rounds to zero)
      const double lq = rr.lp[nd + 1 + j];
      alpha = lq > -745.1332191019412 ? fmin(1.0, exp_fp64(rr.lp[j] - lq)) : 1.0;
    }
    u = a.greedy ? 0.5 : rr.u[j];  // greedy: alpha is 0 or 1, any u in (0, 1) decides it
  }
  // first rejection: lowest lane with !(u < alpha)
  const unsigned long long rej = __ballot(j < nd && !(u < alpha));
  const int n_acc = rej ? __ffsll(static_cast<long long>(rej)) - 1 : nd;
  const unsigned long long near = __ballot(!a.greedy && j < nd && j <= n_acc && fabs(u - alpha) < kNear);
  // S(k) = prod_{j<k} alpha_j: inclusive prefix product over lanes
  const double surv = wave::incl_scan(alpha, 1.0, wave::Mul{});  // lanes >= nd hold 1
  const double tsum = wave::reduce(j < nd ? surv : 0.0, 64, wave::Add{});
  if (store && j < nd) {
    if (a.alpha) a.alpha[static_cast<size_t>(i) * nd + j] = static_cast<float>(alpha);
    if (a.survival) a.survival[static_cast<size_t>(i) * nd + j] = static_cast<float>(surv);
  }
  if (lane == 0) {
    SampleState st;
    st.tgt_row = i * (nd + 1) + n_acc;
    st.drf_row = i * nd + min(n_acc, nd - 1);  // a valid row in every mode; its values unused for the bonus
    st.max_p = rr.max[n_acc];
    st.max_q = (!a.greedy && n_acc < nd) ? rr.max[nd + 1 + n_acc] : 0.f;
    st.u = a.greedy ? 0.0 : rr.u[nd];
    st.mode = a.greedy ? kDone : (n_acc < nd ? kResidual : kBonus);
    st.near = near ? 1u : 0u;
    // sums relative to the same references as the draw's ap and aq
    st.rho = st.mode == kResidual ? rr.logsum[n_acc] - rr.logsum[nd + 1 + n_acc] : 0.0;
    *sh_state = st;
    if (store) {
      a.n_acc[i] = n_acc;
      if (a.tau) a.tau[i] = static_cast<float>(1.0 + tsum);
      if (a.greedy) {
        if (a.flags) a.flags[i] = 0u;
        a.next_token[i] = rr.arg[n_acc] == INT_MAX ? -1 : rr.arg[n_acc];  // -1: every logit is -inf
      }
    }
  }
  // greedy: the outcome is final here (sampling matches after its draw)
  if (store && a.greedy && a.hit) match_outcome(a, i, n_acc, rr.arg[n_acc] == INT_MAX ? -1 : rr.arg[n_acc]);
}

// ------------------------------------------------------------------------------------------------
// 2.-4. fp64 sample of the one row the next token is drawn from
// ------------------------------------------------------------------------------------------------
// Eight consecutive logits from token v0 on; tokens past the vocabulary read as -inf (zero mass).
// The loads are unconditional (from a clamped, in-bounds position) and the masking is a select
// afterwards, so a caller's loads of several rows all issue before the first wait. Vector mode
// needs V >= 8 and V a multiple of the vector width (16 B); then a partial group can only occur for
// fp32 (4 per vector) with v0 = V - 4, where the clamped load starts 4 tokens early.
template <typename T, bool VEC>
__device__ __forceinline__ void load8(const T *row, int v0, int V, float (&z)[kSampleElems]) {
  if constexpr (VEC) {
    constexpr int W = 16 / sizeof(T);
    const int vc = min(v0, V - kSampleElems);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(row + vc);
    float t[kSampleElems];
#pragma unroll
    for (int h = 0; h < kSampleElems / W; ++h) {
      float u[W];
      unpack(vp[h], u, static_cast<const T *>(nullptr));
#pragma unroll
      for (int k = 0; k < W; ++k) t[h * W + k] = u[k];
    }
    const bool shifted = vc != v0;
#pragma unroll
    for (int k = 0; k < kSampleElems; ++k)
      z[k] = v0 + k < V ? (shifted ? t[(k + 4) & (kSampleElems - 1)] : t[k]) : -INFINITY;
  } else {
#pragma unroll
    for (int k = 0; k < kSampleElems; ++k) {
      const float t = load_elem(row + min(v0 + k, V - 1));
      z[k] = v0 + k < V ? t : -INFINITY;
    }
  }
}

// 2^(j/32), j = 0..31, rounded to fp64 (computed to 60 digits and rounded once).
__device__ constexpr double kExp2Frac[32] = {
    0x1.0000000000000p+0, 0x1.059b0d3158574p+0, 0x1.0b5586cf9890fp+0, 0x1.11301d0125b51p+0,
    0x1.172b83c7d517bp+0, 0x1.1d4873168b9aap+0, 0x1.2387a6e756238p+0, 0x1.29e9df51fdee1p+0,
    0x1.306fe0a31b715p+0, 0x1.371a7373aa9cbp+0, 0x1.3dea64c123422p+0, 0x1.44e086061892dp+0,
    0x1.4bfdad5362a27p+0, 0x1.5342b569d4f82p+0, 0x1.5ab07dd485429p+0, 0x1.6247eb03a5585p+0,
    0x1.6a09e667f3bcdp+0, 0x1.71f75e8ec5f74p+0, 0x1.7a11473eb0187p+0, 0x1.82589994cce13p+0,
    0x1.8ace5422aa0dbp+0, 0x1.93737b0cdc5e5p+0, 0x1.9c49182a3f090p+0, 0x1.a5503b23e255dp+0,
    0x1.ae89f995ad3adp+0, 0x1.b7f76f2fb5e47p+0, 0x1.c199bdd85529cp+0, 0x1.cb720dcef9069p+0,
    0x1.d5818dcfba487p+0, 0x1.dfc97337b9b5fp+0, 0x1.ea4afa2a490dap+0, 0x1.f50765b6e4540p+0,
};

// exp(x) in fp64, table-driven (P. T. P. Tang, "Table-driven implementation of the exponential function
// in IEEE floating-point arithmetic", ACM TOMS 15(2), 1989): x = (32 k + j) ln2/32 + r with |r| <= ln2/64
// (Cody-Waite: ln2/32 split into a head whose products with the integer are exact and a tail), e^r by
// its Taylor series to degree 6 (truncation below 2e-18 relative), times 2^(j/32) from `tab` (the table
// above, staged in LDS) and 2^k. About 12 fp64 operations and one LDS read against exp_fp64's 18. NaN and
// arguments below the smallest subnormal give 0.
__device__ __forceinline__ double exp_fp64_tab(double x, const double *tab) {
  constexpr double kInvStep = 46.16624130844683;      // 32 / ln 2
  constexpr double kStepHi = 0.021660834550857544;    // (ln 2 with its low 32 mantissa bits cleared) / 32
  constexpr double kStepLo = 1.4841640746973977e-08;  // ln 2 / 32 - kStepHi
  if (!(x > -745.5)) return 0.0;
  const double n = rint(x * kInvStep);
  double r = fma(-n, kStepHi, x);
  r = fma(-n, kStepLo, r);
  double p = 1.0 / 720.0;
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = static_cast<int>(n);
  return ldexp(p * tab[ni & 31], ni >> 5);
}

template <typename T>
struct DrawRows {
  const T *p;
  const T *q;
  float mp, mq;
  double inv_t, log_sp, log_sq;
  int mode;
  const double *tab;  // kExp2Frac in LDS
  // Mass of a token with target logit zp and draft logit zq in the law being drawn from:
  // max(0, P - Q) after a rejection, P for the bonus draw or the zero-mass fallback.
  __device__ __forceinline__ double mass(float zp, float zq) const {
    const double ap = (static_cast<double>(zp) - mp) * inv_t - log_sp;
    if (mode != kResidual) return exp_fp64_tab(ap, tab);
    const double aq = (static_cast<double>(zq) - mq) * inv_t - log_sq;
    if (!(ap > aq)) return 0.0;  // P(v) <= Q(v): no residual mass, no exp needed
    return fmax(0.0, exp_fp64_tab(ap, tab) - exp_fp64_tab(aq, tab));
  }
};

template <typename T>
__device__ __forceinline__ DrawRows<T> draw_rows_base(const VerifyArgs &a, const SampleState &st) {
  DrawRows<T> d;
  d.p = static_cast<const T *>(a.target) + static_cast<size_t>(st.tgt_row) * a.vocab;
  d.q = static_cast<const T *>(a.draft) + static_cast<size_t>(st.drf_row) * a.vocab;
  d.mp = st.max_p;
  d.mq = st.max_q;
  d.inv_t = a.inv_t;
  d.log_sp = 0.0;
  d.log_sq = 0.0;
  d.mode = st.mode;
  return d;
}

// The 8 masses of this thread's tokens in sample chunk c.
template <typename T, bool VEC>
__device__ __forceinline__ void chunk_masses(const DrawRows<T> &d, int c, int V, double (&mass)[kSampleElems]) {
  const int v0 = c * kSampleChunk + static_cast<int>(threadIdx.x) * kSampleElems;
  float zp[kSampleElems], zq[kSampleElems];
  load8<T, VEC>(d.p, v0, V, zp);
  load8<T, VEC>(d.q, v0, V, zq);  // unconditional: both loads issue before the first wait
#pragma unroll
  for (int k = 0; k < kSampleElems; ++k) mass[k] = d.mass(zp[k], d.mode == kResidual ? zq[k] : 0.f);
}

// Block-wide sums of N doubles per thread; every thread gets the totals.
template <int N>
__device__ __forceinline__ void block_sums(double (&v)[N], double *sh) {
#pragma unroll
  for (int f = 0; f < N; ++f) v[f] = wave::reduce(v[f], 64, wave::Add{});
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int f = 0; f < N; ++f) sh[w * N + f] = v[f];
  __syncthreads();
#pragma unroll
  for (int f = 0; f < N; ++f) {
    double r = sh[f];
    for (int k = 1; k < kWaves; ++k) r += sh[k * N + f];
    v[f] = r;
  }
  __syncthreads();
}

// A workgroup-uniform copy of the state read from LDS, held in scalar registers.
__device__ __forceinline__ int32_t sgpr(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float sgpr(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
__device__ __forceinline__ double sgpr(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readfirstlane(static_cast<int>(b));
  const int hi = __builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}
__device__ __forceinline__ SampleState uniform_state(const SampleState &s) {
  SampleState u;
  u.mode = sgpr(s.mode);
  u.tgt_row = sgpr(s.tgt_row);
  u.drf_row = sgpr(s.drf_row);
  u.max_p = sgpr(s.max_p);
  u.max_q = sgpr(s.max_q);
  u.near = static_cast<uint32_t>(sgpr(static_cast<int32_t>(s.near)));
  u.u = sgpr(s.u);
  u.rho = sgpr(s.rho);
  return u;
}

// Block-wide exclusive prefix sum of one double per thread (256 threads); also returns the total.
__device__ __forceinline__ double block_excl_scan(double v, double *sh, double *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const double incl = wave::incl_scan(v, 0.0, wave::Add{});
  if (lane == 63) sh[wv] = incl;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wv) off += sh[w];
    tot += sh[w];
  }
  __syncthreads();
  *total = tot;
  return off + wave::shift_up(incl, 0.0);
}

// Block-wide exclusive prefix sum of one double per thread with one barrier (the same arithmetic as
// block_excl_scan); `sh` (kWaves doubles) must not be written again before the next barrier.
__device__ __forceinline__ double block_excl_scan1(double v, double *sh, double *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const double incl = wave::incl_scan(v, 0.0, wave::Add{});
  if (lane == 63) sh[wv] = incl;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wv) off += sh[w];
    tot += sh[w];
  }
  *total = tot;
  return off + wave::shift_up(incl, 0.0);
}

// Per wavefront, the first lane with `hit` and the last lane with `pos` publish (index, value) into
// LDS slot [wave]; after one barrier every thread takes the first hit over the wavefronts, else the
// last positive entry. Index INT_MAX / -1: none.
struct Pick {
  int hit_i, last_i;
  double hit_v, last_v;
};
__device__ __forceinline__ Pick block_pick(bool hit, int hit_i, double hit_v, bool pos, int last_i, double last_v,
                                           int *sh_i, double *sh_v) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const unsigned long long hb = __ballot(hit), pb = __ballot(pos);
  const int hl = hb ? __ffsll(static_cast<long long>(hb)) - 1 : 0;
  const int pl = pb ? 63 - __clzll(static_cast<long long>(pb)) : 0;
  if (lane == hl) {
    sh_i[2 * wv] = hb ? hit_i : INT_MAX;
    sh_v[2 * wv] = hit_v;
  }
  if (lane == pl) {
    sh_i[2 * wv + 1] = pb ? last_i : -1;
    sh_v[2 * wv + 1] = last_v;
  }
  __syncthreads();
  Pick r{INT_MAX, -1, 0.0, 0.0};
  for (int w = 0; w < kWaves; ++w) {
    if (r.hit_i == INT_MAX && sh_i[2 * w] != INT_MAX) {
      r.hit_i = sh_i[2 * w];
      r.hit_v = sh_v[2 * w];
    }
    if (sh_i[2 * w + 1] >= 0) {
      r.last_i = sh_i[2 * w + 1];
      r.last_v = sh_v[2 * w + 1];
    }
  }
  return r;
}

// Inside sample chunk c, whose tokens start at cumulative mass `offset`: the smallest v with
// offset + C(v) > target. Thread t owns tokens 8t..8t+7 of the chunk; the owner is the first
// thread whose inclusive prefix exceeds the target, and it walks its 8 masses. If rounding leaves
// no crossing, the last token with positive mass is returned. The thread that settles the token
// writes next_token and flags (bit 1 when target is within kNear * z of the token's cumulative
// bounds) and returns it in sh_tok (-1: no token has mass).
template <typename T, bool VEC>
__device__ __forceinline__ void chunk_find(const VerifyArgs &a, int i, const DrawRows<T> &d, int c, double offset,
                                           double target, double z, uint32_t fl, double *sh_scan, int *sh_pi,
                                           double *sh_pv, int *sh_tok) {
  double m[kSampleElems];
  chunk_masses<T, VEC>(d, c, a.vocab, m);
  double local = 0.0;
#pragma unroll
  for (int k = 0; k < kSampleElems; ++k) local += m[k];
  double total;
  const double start = offset + block_excl_scan1(local, sh_scan, &total);
  const int me = static_cast<int>(threadIdx.x);
  const Pick pk = block_pick(start + local > target, me, 0.0, local > 0.0, me, 0.0, sh_pi, sh_pv);
  const int owner = pk.hit_i, last = pk.last_i;
  const bool is_owner = me == owner;
  if (is_owner || (owner == INT_MAX && me == last) || (owner == INT_MAX && last < 0 && me == 0)) {
    const int v0 = c * kSampleChunk + me * kSampleElems;
    double cum = start;
    int last_v = -1, hit_v = -1;
    double last_c = offset, last_p = offset, hit_c = cum, hit_p = cum;
    if (owner != INT_MAX || last >= 0) {
      last_c = cum;
      last_p = cum;
#pragma unroll
      for (int k = 0; k < kSampleElems; ++k) {
        const double prev = cum;
        cum += m[k];
        if (m[k] > 0.0) {
          last_v = v0 + k;
          last_c = cum;
          last_p = prev;
        }
        if (is_owner && hit_v < 0 && cum > target) {
          hit_v = v0 + k;
          hit_c = cum;
          hit_p = prev;
        }
      }
    }
    const bool h = hit_v >= 0;
    const int v = h ? hit_v : last_v;
    const double c_v = h ? hit_c : last_c, c_prev = h ? hit_p : last_p;
    if (fabs(target - c_v) < kNear * z || fabs(target - c_prev) < kNear * z) fl |= 2u;
    a.next_token[i] = v;
    if (a.flags) a.flags[i] = fl;
    *sh_tok = v;
  }
}

// The draw of request i from its chunk masses (thread t holds chunks 4t..4t+3): chunk prefix, the
// chunk holding u'Z, then the in-chunk scan. Three barriers on the common path: the chunk prefix,
// the choice of the chunk (first chunk whose inclusive prefix exceeds u'Z), the in-chunk prefix and
// the choice of the owner thread (together with the chunk's, one each). Returns the token in every
// thread when `uniform` (one more barrier).
template <typename T, bool VEC>
__device__ __forceinline__ int draw_token(const VerifyArgs &a, int i, const SampleState &st, DrawRows<T> d,
                                           const double (&mine)[kMaxSampleChunks / kThreads], double *sh_d,
                                           int *sh_i, double *sh_cum, double *sh_s1, double *sh_s2, int *sh_pi,
                                           double *sh_pv, int *sh_pi2, double *sh_pv2, int *sh_tok, bool uniform) {
  constexpr int CPT = kMaxSampleChunks / kThreads;
  const int c0 = threadIdx.x * CPT;
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) run += mine[k];
  double z;
  const double base = block_excl_scan1(run, sh_s1, &z);
  z = sgpr(z);
  uint32_t fl = st.near;
  int c;
  double offset, target;
  if (z > 0.0) {
    target = sgpr(st.u * z);
    // this thread's chunks: the first whose inclusive prefix exceeds the target, the last with mass
    int hit_c = INT_MAX, last_c = -1;
    double hit_o = 0.0, last_o = 0.0, cum = base;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const double prev = cum;
      cum += mine[k];
      if (c0 + k < a.s_chunks) {
        if (hit_c == INT_MAX && cum > target) {
          hit_c = c0 + k;
          hit_o = prev;
        }
        if (cum > prev) {
          last_c = c0 + k;
          last_o = prev;
        }
      }
    }
    const Pick pk = block_pick(hit_c != INT_MAX, hit_c, hit_o, last_c >= 0, last_c, last_o, sh_pi, sh_pv);
    c = pk.hit_i != INT_MAX ? pk.hit_i : max(pk.last_i, 0);
    offset = pk.hit_i != INT_MAX ? pk.hit_v : (pk.last_i >= 0 ? pk.last_v : 0.0);
  } else {
    // zero residual mass (not reachable in exact arithmetic): draw from P instead, chunk by chunk
    fl |= 4u;
    d.mode = kBonus;
    double zp_tot = 0.0;
    for (int cc = 0; cc < a.s_chunks; ++cc) {
      double m[kSampleElems];
      chunk_masses<T, VEC>(d, cc, a.vocab, m);
      double t = 0.0;
#pragma unroll
      for (int k = 0; k < kSampleElems; ++k) t += m[k];
      const double cs = block_sum(t, sh_d);
      if (threadIdx.x == 0) sh_cum[cc] = zp_tot + cs;  // inclusive prefix
      zp_tot += cs;
    }
    z = zp_tot;
    __syncthreads();
    target = sgpr(st.u * z);
    int cand = INT_MAX, lastpos = -1;
    for (int cc = threadIdx.x; cc < a.s_chunks; cc += kThreads) {
      const double below = cc > 0 ? sh_cum[cc - 1] : 0.0;
      if (cand == INT_MAX && sh_cum[cc] > target) cand = cc;
      if (sh_cum[cc] > below) lastpos = cc;
    }
    const int c_star = block_min_int(cand, sh_i);
    const int c_last = -block_min_int(lastpos >= 0 ? -lastpos : INT_MAX, sh_i);
    c = c_star != INT_MAX ? c_star : max(c_last, 0);
    offset = c > 0 ? sh_cum[c - 1] : 0.0;
  }
  c = sgpr(c);
  offset = sgpr(offset);
  chunk_find<T, VEC>(a, i, d, c, offset, target, z, fl, sh_s2, sh_pi2, sh_pv2, sh_tok);
  if (!uniform) return -1;
  __syncthreads();
  return *sh_tok;
}

// The slice sums of one (request, sample chunk), then, in the request's last workgroup to finish,
// the draw.
// At most 80 VGPRs (6 waves per SIMD): the draft attention kernel that runs beside verify in a round
// leaves 80 per SIMD on each of its compute units, so a sample workgroup fits next to it instead of
// holding a compute unit that an attention workgroup then waits for.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void sample_kernel(const VerifyArgs a) {
  constexpr int CPT = kMaxSampleChunks / kThreads;
  extern __shared__ __align__(16) unsigned char dyn_lds[];  // decide's partials, then the pick's prefix
  __shared__ ReqRows rr;
  __shared__ SampleState sh_state;
  __shared__ double sh_d[kWaves * kRecFields];
  __shared__ int sh_i[kWaves];
  __shared__ double sh_s1[kWaves], sh_s2[kWaves], sh_pv[2 * kWaves], sh_pv2[2 * kWaves];
  __shared__ int sh_pi[2 * kWaves], sh_pi2[2 * kWaves], sh_tok;
  __shared__ uint32_t sh_last;
  const int i = blockIdx.y;
  __shared__ double sh_exp2[32];
  if (threadIdx.x < 32) sh_exp2[threadIdx.x] = kExp2Frac[threadIdx.x];
  decide_request(a, i, reinterpret_cast<StatPartial *>(dyn_lds), rr, &sh_state, blockIdx.x == 0);
  __syncthreads();
  const SampleState st = uniform_state(sh_state);  // in scalar registers: the budget is 80 VGPRs
  if (st.mode == kDone) return;
  DrawRows<T> d = draw_rows_base<T>(a, st);
  d.tab = sh_exp2;
  const bool residual = st.mode == kResidual;
  {
    const int v0 = blockIdx.x * kSampleChunk + static_cast<int>(threadIdx.x) * kSampleElems;
    float zp[kSampleElems], zq[kSampleElems];
    load8<T, VEC>(d.p, v0, a.vocab, zp);
    load8<T, VEC>(d.q, v0, a.vocab, zq);  // the draft row is valid in every mode
    double s[kRecFields] = {0.0, 0.0, 0.0, 0.0, 0.0};
    // the references as fp64 in scalar registers (converted per use they took vector registers)
    const double ref_p = sgpr(static_cast<double>(st.max_p)), ref_q = sgpr(static_cast<double>(st.max_q));
#pragma unroll
    for (int k = 0; k < kSampleElems; ++k) {
      const double ap = (static_cast<double>(zp[k]) - ref_p) * a.inv_t;
      const double ep = exp_fp64_tab(ap, sh_exp2);
      s[0] += ep;
      if (residual) {
        const double aq = (static_cast<double>(zq[k]) - ref_q) * a.inv_t;
        const double eq = exp_fp64_tab(aq, sh_exp2);
        s[1] += eq;
        if (ep > 0.0) {  // a token without target mass has no residual mass
          const double t = (ap - aq) - st.rho;
          if (t > kRhoBand) {
            s[2] += ep;
            s[3] += eq;
          } else if (!(t < -kRhoBand)) {
            s[4] += 1.0;
          }
        }
      }
    }
    if (!residual) s[2] = s[0];
    block_sums(s, sh_d);
    // Publication of the record. Its fields are written with device-scope atomic stores, which
    // write through to the memory every XCD shares, and the wait makes them complete before the
    // count is incremented; the last workgroup reads them with device-scope atomic loads, which do
    // not hit lines another XCD's L2 may hold stale. That is the ordering a release / acquire pair
    // gives, without its writeback and invalidation of the whole L2, which only plain accesses
    // need and which cost ~17 us over the 1200 workgroups of a 16-request serving batch.
    if (threadIdx.x == 0) {
      double *dst = reinterpret_cast<double *>(a.rec + static_cast<size_t>(i) * a.s_chunks + blockIdx.x);
#pragma unroll
      for (int f = 0; f < kRecFields; ++f) __hip_atomic_store(dst + f, s[f], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t done = __hip_atomic_fetch_add(a.counter + static_cast<size_t>(i) * kCounterStride, 1u,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh_last = done + 1 == static_cast<uint32_t>(a.s_chunks) ? 1u : 0u;
    }
    __syncthreads();
    if (!sh_last) return;
  }
  // the request's last workgroup: every record of the request is published
  const SampleRec *rec = a.rec + static_cast<size_t>(i) * a.s_chunks;
  const int c0 = threadIdx.x * CPT;
  // the row sums first, then (second pass, few registers live across the reduction) each chunk's mass
  const auto field = [&](int k, int f) {
    const double *src = reinterpret_cast<const double *>(rec + min(c0 + k, a.s_chunks - 1));
    return __hip_atomic_load(src + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  double tot[2] = {0.0, 0.0};
#pragma unroll
  for (int k = 0; k < CPT; ++k) {  // unconditional loads (clamped), then selects
    const double sp = field(k, 0), sq = field(k, 1);
    tot[0] += c0 + k < a.s_chunks ? sp : 0.0;
    tot[1] += c0 + k < a.s_chunks ? sq : 0.0;
  }
  block_sums(tot, sh_d);
  d.log_sp = sgpr(log(tot[0]));
  d.log_sq = sgpr(residual ? log(tot[1]) : 0.0);
  const double inv_sp = sgpr(1.0 / tot[0]), inv_sq = sgpr(residual ? 1.0 / tot[1] : 0.0);
  // the estimate must be within half the band for the split sums to hold
  const bool split_ok = !residual || fabs((d.log_sp - d.log_sq) - st.rho) <= 0.5 * kRhoBand;
  double mine[CPT];
  bool redo[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const double ra = field(k, 2), rb = field(k, 3), ramb = field(k, 4);
    const bool in = c0 + k < a.s_chunks;
    mine[k] = !in ? 0.0 : residual ? fmax(0.0, ra * inv_sp - rb * inv_sq) : ra * inv_sp;
    redo[k] = in && residual && (!split_ok || ramb > 0.0);
  }
  // slices whose split is not settled: weighed token by token, one slice at a time
  for (;;) {
    int cand = INT_MAX;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (redo[k]) cand = min(cand, c0 + k);
    const int cf = block_min_int(cand, sh_i);
    if (cf == INT_MAX) break;
    double m[kSampleElems];
    chunk_masses<T, VEC>(d, cf, a.vocab, m);
    double t[1] = {0.0};
#pragma unroll
    for (int k = 0; k < kSampleElems; ++k) t[0] += m[k];
    block_sums(t, sh_d);
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (c0 + k == cf) {
        mine[k] = t[0];
        redo[k] = false;
      }
  }
  const int tok = draw_token<T, VEC>(a, i, st, d, mine, sh_d, sh_i, reinterpret_cast<double *>(dyn_lds), sh_s1, sh_s2,
                                     sh_pi, sh_pv, sh_pi2, sh_pv2, &sh_tok, a.hit != nullptr);
  if (a.hit && threadIdx.x < 64) match_outcome(a, i, st.tgt_row - i * (a.n_draft + 1), tok);
}

// ------------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------------
struct VerifyPlan {
  int chunks, chunk_len, s_chunks;
  size_t off_stats, off_rec, off_cnt, total;
};

int plan_verify(int n_req, int n_draft, int vocab, VerifyPlan *p) {
  if (n_req < 1 || n_draft < 1 || n_draft > 63 || vocab < 1 || vocab > kMaxVocab) return D3D_EINVAL;
  const int rows_req = 2 * n_draft + 1;
  const long long rows = static_cast<long long>(n_req) * rows_req;
  if (rows > INT_MAX) return D3D_EINVAL;
  const int s_chunks = (vocab + kSampleChunk - 1) / kSampleChunk;
  if (s_chunks > kMaxSampleChunks) return D3D_EINVAL;
  // One round of resident stats workgroups when the rows allow it; whole 64-token chunks; the
  // request's partials must fit decide's LDS stage.
  int chunks = static_cast<int>(std::max<long long>(1, kStatSlots / rows));
  chunks = std::min(chunks, (vocab + kStatMinChunk - 1) / kStatMinChunk);
  chunks = std::min(chunks, kMaxReqPartials / rows_req);
  chunks = std::min(chunks, kStatMaxChunks);
  int len = (vocab + chunks - 1) / chunks;
  len = (len + 63) / 64 * 64;
  p->chunk_len = len;
  p->chunks = (vocab + len - 1) / len;
  p->s_chunks = s_chunks;
  size_t off = 0;
  p->off_stats = off;
  off = align_up(off + sizeof(StatPartial) * static_cast<size_t>(rows) * p->chunks, 256);
  p->off_rec = off;
  off = align_up(off + sizeof(SampleRec) * static_cast<size_t>(n_req) * s_chunks, 256);
  p->off_cnt = off;
  off = align_up(off + sizeof(uint32_t) * kCounterStride * static_cast<size_t>(n_req), 256);
  p->total = off;
  return D3D_OK;
}

template <typename T, bool VEC>
int launch_verify(const VerifyArgs &a, hipStream_t stream) {
  // greedy verify reads no draft rows
  const int stat_rows = a.greedy ? a.n_tgt_rows : a.n_req * (2 * a.n_draft + 1);
  const dim3 stat_grid(a.chunks, stat_rows);
  if (a.greedy)
    stats_kernel<T, VEC, true><<<stat_grid, kStatThreads, 0, stream>>>(a);
  else
    stats_kernel<T, VEC, false><<<stat_grid, kStatThreads, 0, stream>>>(a);
  const int rows_req = a.greedy ? a.n_draft + 1 : 2 * a.n_draft + 1;
  // the dynamic stage holds decide's partials, then (last workgroup) the pick's chunk prefix
  const size_t lds = std::max(sizeof(StatPartial) * static_cast<size_t>(rows_req) * a.chunks,
                              sizeof(double) * static_cast<size_t>(a.s_chunks));
  const dim3 grid(a.greedy ? 1 : a.s_chunks, a.n_req);
  sample_kernel<T, VEC><<<grid, kThreads, lds, stream>>>(a);
  return launch_status();
}

}  // namespace
}  // namespace d3d

extern "C" size_t spec_verify_workspace(int n_req, int n_draft, int vocab) {
  d3d::VerifyPlan p;
  if (d3d::plan_verify(n_req, n_draft, vocab, &p) != D3D_OK) return 0;
  return p.total;
}

namespace d3d {
namespace {
// Every argument check of a verify call, before anything touches the device; fills the plan.
int check_verify(d3d_dtype dtype, const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                 int n_req, int n_draft, int vocab, float temperature, const int32_t *n_accepted,
                 const int32_t *next_token, VerifyPlan *p) {
  if (dtype != D3D_BF16 && dtype != D3D_F32) return D3D_EINVAL;
  if (!target_logits || !draft_tokens || !n_accepted || !next_token) return D3D_EINVAL;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return D3D_EINVAL;
  if (temperature != 0.f && !draft_logits) return D3D_EINVAL;
  return plan_verify(n_req, n_draft, vocab, p);
}

int verify_impl(d3d_dtype dtype, const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                int n_req, int n_draft, int vocab, float temperature, uint64_t seed, uint32_t round,
                int32_t *n_accepted, int32_t *next_token, float *alpha, float *survival, float *tau, uint32_t *flags,
                void *ws, size_t ws_bytes, const d3d_block_desc *descs, int total_blocks,
                const int32_t *req_block_off, int32_t *hit, hipStream_t stream) {
  VerifyPlan p;
  if (check_verify(dtype, target_logits, draft_logits, draft_tokens, n_req, n_draft, vocab, temperature, n_accepted,
                   next_token, &p) != D3D_OK)
    return D3D_EINVAL;
  const bool greedy = temperature == 0.f;
  if (!ws || ws_bytes < p.total) return D3D_EWORKSPACE;
  char *w = static_cast<char *>(ws);
  VerifyArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.n_req = n_req;
  a.n_draft = n_draft;
  a.vocab = vocab;
  a.n_tgt_rows = n_req * (n_draft + 1);
  a.chunks = p.chunks;
  a.chunk_len = p.chunk_len;
  a.s_chunks = p.s_chunks;
  a.c_log2 = greedy ? 0.f : static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  a.inv_t = greedy ? 0.0 : 1.0 / static_cast<double>(temperature);
  a.seed = seed;
  a.round = round;
  a.greedy = greedy ? 1 : 0;
  a.n_acc = n_accepted;
  a.next_token = next_token;
  a.alpha = alpha;
  a.survival = survival;
  a.tau = tau;
  a.flags = flags;
  a.stats = reinterpret_cast<StatPartial *>(w + p.off_stats);
  a.rec = reinterpret_cast<SampleRec *>(w + p.off_rec);
  a.counter = reinterpret_cast<uint32_t *>(w + p.off_cnt);
  a.descs = descs;
  a.req_block_off = req_block_off;
  a.total_blocks = total_blocks;
  a.hit = hit;
  const size_t esize = dtype == D3D_BF16 ? 2 : 4;
  const size_t width = 16 / esize;
  const bool aligned = (reinterpret_cast<uintptr_t>(target_logits) % 16 == 0) &&
                       (greedy || reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0);
  const bool vec = aligned && (static_cast<size_t>(vocab) % width == 0) && vocab >= kSampleElems;
  if (dtype == D3D_BF16)
    return vec ? launch_verify<__bf16, true>(a, stream) : launch_verify<__bf16, false>(a, stream);
  return vec ? launch_verify<float, true>(a, stream) : launch_verify<float, false>(a, stream);
}
}  // namespace
}  // namespace d3d

extern "C" int spec_verify(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
                           const int32_t *draft_tokens, int n_req, int n_draft, int vocab,
                           float temperature, uint64_t seed, uint32_t round, int32_t *n_accepted,
                           int32_t *next_token, float *alpha, float *survival, float *tau,
                           uint32_t *flags, void *ws, size_t ws_bytes, hipStream_t stream) {
  return d3d::verify_impl(dtype, target_logits, draft_logits, draft_tokens, n_req, n_draft, vocab, temperature, seed,
                          round, n_accepted, next_token, alpha, survival, tau, flags, ws, ws_bytes, nullptr, 0,
                          nullptr, nullptr, stream);
}

extern "C" int spec_verify_match(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
                                 const int32_t *draft_tokens, int n_req, int n_draft, int vocab, float temperature,
                                 uint64_t seed, uint32_t round, int32_t *n_accepted, int32_t *next_token,
                                 float *alpha, float *survival, float *tau, uint32_t *flags, void *ws,
                                 size_t ws_bytes, const d3d_block_desc *descs, int total_blocks,
                                 const int32_t *req_block_off, int32_t *hit_branch, hipStream_t stream) {
  if (!descs || !req_block_off || !hit_branch || total_blocks < 1) return D3D_EINVAL;
  return d3d::verify_impl(dtype, target_logits, draft_logits, draft_tokens, n_req, n_draft, vocab, temperature, seed,
                          round, n_accepted, next_token, alpha, survival, tau, flags, ws, ws_bytes, descs,
                          total_blocks, req_block_off, hit_branch, stream);
}

// ------------------------------------------------------------------------------------------------
// allocation-free variant: the workspace lives in a file-scope device array
// ------------------------------------------------------------------------------------------------
// One copy per GPU (held until the process ends). Its host-side name is only a stand-in for the
// device address: host code uses the address hipGetSymbolAddress returns on each device, never the
// name. Nothing in the verify workspace needs initial contents, so no call clears it.
static __device__ __align__(256) unsigned char scratch[D3D_VERIFY_SCRATCH_BYTES];

namespace d3d {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, looked up once per device.
int scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return D3D_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return D3D_EUNSUPPORTED;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return D3D_EHIP;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return D3D_OK;
}
}  // namespace
}  // namespace d3d

extern "C" int spec_verify_noalloc(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
                                   const int32_t *draft_tokens, int n_req, int n_draft, int vocab,
                                   float temperature, uint64_t seed, uint32_t round, int32_t *n_accepted,
                                   int32_t *next_token, float *alpha, float *survival, float *tau,
                                   uint32_t *flags, hipStream_t stream) {
  d3d::VerifyPlan p;
  if (d3d::check_verify(dtype, target_logits, draft_logits, draft_tokens, n_req, n_draft, vocab, temperature,
                        n_accepted, next_token, &p) != D3D_OK)
    return D3D_EINVAL;
  if (p.total > D3D_VERIFY_SCRATCH_BYTES) return D3D_ESCRATCH;  // before the scratch address is looked up
  void *ws = nullptr;
  const int st = d3d::scratch_ptr(&ws);
  if (st != D3D_OK) return st;
  return d3d::verify_impl(dtype, target_logits, draft_logits, draft_tokens, n_req, n_draft, vocab, temperature,
                          seed, round, n_accepted, next_token, alpha, survival, tau, flags, ws,
                          D3D_VERIFY_SCRATCH_BYTES, nullptr, 0, nullptr, nullptr, stream);
}
