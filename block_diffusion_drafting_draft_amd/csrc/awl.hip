// Acceptance-weighted loss (AWL) of drafter training and its gradient, on gfx950.
//
// What is computed ([DScout] 前置知识: 接受加权损失 AWL 与推测采样接受规则; 方法步骤详情 step 4): for
// block r and future position k (k = 0..n_pos-1), alpha_{r,k} = min(1, P_{r,k}(y_{r,k}) / Q_{r,k}(y_{r,k}))
// with P / Q the softmaxes of the target / draft logits and y the draft token; the position weight is
// the stop-gradient product of the earlier scores, w_{r,k} = prod_{j<k} alpha_{r,j} (w_{r,0} = 1);
// L = sum I w CE(Q, y*) / (sum I w + eps), CE(Q, y*) = -log Q(y*), I the inclusion mask. The gradient
// reaches the draft logits only: dL/dz = I w / (sum I w + eps) * (Q - onehot(y*)).
//
// Passes (HBM-bound: the target and draft logits are read once for the statistics, the draft logits
// once more and the gradient written once):
//   1. stats  grid (chunk, row) over the target rows then the draft rows: one 16-byte-vector pass,
//             sum of exp(z - ref) against a reference logit of the slice (fp32 exp, fp64 accumulation,
//             as in the verify statistics), and the logits at the draft token and the label.
//   2. block  one workgroup per block: merges each row (fp64), alpha, the weights (a wave prefix
//             product), -log Q(y*), the row's log-sum-exp, and the block's sums of I w CE and I w.
//   3. final  one workgroup: the loss and 1 / (sum I w + eps).
//   4. grad   grid (chunk, draft row): I w / (sum I w + eps) * (Q - onehot(y*)), stored in the logits'
//             element type (skipped when no gradient is requested).
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kAwlSlots = 16384;  // target workgroups of the statistics pass (many rounds per CU: a short last round)
constexpr int kAwlMinChunk = 1024;
constexpr int kAwlMaxChunks = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453;

struct AwlPartial {
  float ref;    // reference logit of the slice
  float z_tok;  // logit at the draft token when the slice holds it
  float z_lab;  // logit at the label when the slice holds it (draft rows)
  float pad;
  double sum;   // sum of exp(z - ref) over the slice
};

struct AwlArgs {
  const void *target, *draft;
  const int32_t *tokens, *labels, *include;
  int n_blocks, n_pos, vocab, n_rows;  // n_rows = n_blocks * n_pos
  int chunks, chunk_len;
  double eps;
  float *weights, *ce;
  double *loss;
  void *grad;
  AwlPartial *part;  // [2 n_rows][chunks]: target rows then draft rows
  double *lse;       // [n_rows] draft rows' log-sum-exp
  double *block_sums;  // [n_blocks][2]: sum I w CE, sum I w
  double *scale;       // [1]: 1 / (sum I w + eps)
};

template <int W>
__device__ __forceinline__ void unpack(const u32x4 &w, float (&z)[W]);
template <>
__device__ __forceinline__ void unpack<8>(const u32x4 &w, float (&z)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    z[2 * k] = bf16_lo(w[k]);
    z[2 * k + 1] = bf16_hi(w[k]);
  }
}
template <>
__device__ __forceinline__ void unpack<4>(const u32x4 &w, float (&z)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) z[k] = __uint_as_float(w[k]);
}

__device__ __forceinline__ double block_sum(double v, double *sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < kWaves; ++i) r += sh[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float v, float *sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}

// s 2^(mc - nmc), out of line: it runs only when the reference moves, and inlined, its constants
// would hold registers for the whole streaming loop
__device__ __attribute__((noinline)) double rescale(double s, float mc, float nmc) {
  return s * exp_fp64((static_cast<double>(mc) - nmc) * kLn2);
}

struct RefSum {
  float m = -INFINITY, mc = -INFINITY;
  double s = 0.0;

  template <int N>
  __device__ __forceinline__ float group_sum(const float (&z)[N]) const {
    float part = __builtin_amdgcn_exp2f(__builtin_fmaf(z[0], kLog2e, -mc));
#pragma unroll
    for (int k = 1; k < N; ++k) part += __builtin_amdgcn_exp2f(__builtin_fmaf(z[k], kLog2e, -mc));
    return part;
  }

  template <int N>
  __device__ __forceinline__ void fold(const float (&z)[N]) {
    float part = group_sum(z);
    // the reference moves once a group's sum reaches 2^8: a kept term has an exponent argument
    // below 8, whose relative fp32 rounding (|x| 2^-24) stays far below the weights' 1e-6 budget
    if (!(part < 0x1p8f)) {
      float vm = z[0];
#pragma unroll
      for (int k = 1; k < N; ++k) vm = fmaxf(vm, z[k]);
      if (vm == -INFINITY) return;  // no finite logit yet
      const float nmc = vm * kLog2e;
      s = m == -INFINITY ? 0.0 : rescale(s, mc, nmc);
      m = vm;
      mc = nmc;
      part = group_sum(z);
    }
    s += static_cast<double>(part);
  }

  // the reference r the terms are taken against (-inf when no finite logit was seen)
  __device__ __forceinline__ double ref() const {
    if (m == -INFINITY) return -INFINITY;
    const float rho = __builtin_fmaf(m, kLog2e, -mc);
    return static_cast<double>(m) - static_cast<double>(rho) / static_cast<double>(kLog2e);
  }
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void awl_stats_kernel(const AwlArgs a) {
  __shared__ float sh_f[kWaves];
  __shared__ double sh_d[kWaves];
  const int row = blockIdx.y, chunk = blockIdx.x;
  const bool is_draft = row >= a.n_rows;
  const int r = is_draft ? row - a.n_rows : row;
  const T *base = static_cast<const T *>(is_draft ? a.draft : a.target) + static_cast<size_t>(r) * a.vocab;
  const int begin = chunk * a.chunk_len;
  const int end = min(begin + a.chunk_len, a.vocab);
  const int tok = min(max(a.tokens[r], 0), a.vocab - 1);
  const int lab = min(max(a.labels[r], 0), a.vocab - 1);
  const bool has_tok = tok >= begin && tok < end;
  const bool has_lab = is_draft && lab >= begin && lab < end;
  RefSum acc;
  if constexpr (VEC) {
    constexpr int W = 16 / sizeof(T);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(base + begin);
    const int nvec = (end - begin) / W;
    stream_vecs<kThreads, 4>(
        vp, nvec,
        [&](const u32x4 &w, int) {
          float z[W];
          unpack<W>(w, z);
          acc.fold(z);
        },
        [] {});
  } else {
    for (int t = begin + threadIdx.x; t < end; t += kThreads) {
      float z[1] = {load_elem(base + t)};
      acc.fold(z);
    }
  }
  // the captured logits (wave-uniform loads of lines the pass has just read), issued before the
  // reductions so that their latency overlaps them
  float z_tok = -INFINITY, z_lab = -INFINITY;
  if (threadIdx.x == 0) {
    if (has_tok) z_tok = load_elem(base + tok);
    if (has_lab) z_lab = load_elem(base + lab);
  }
  const float m = block_max(acc.m, sh_f);
  const double mine = acc.m == -INFINITY ? 0.0 : acc.s * exp_fp64(acc.ref() - m);
  const double s = block_sum(mine, sh_d);
  if (threadIdx.x == 0) {
    AwlPartial p;
    p.ref = m;
    p.z_tok = z_tok;
    p.z_lab = z_lab;
    p.pad = 0.f;
    p.sum = s;
    a.part[static_cast<size_t>(row) * a.chunks + chunk] = p;
  }
}

// One workgroup per block. Local rows 0..n_pos-1 are the block's target rows, n_pos..2n_pos-1 its
// draft rows; each is merged by a power-of-two group of g lanes (a group never straddles a
// wavefront).
__global__ __launch_bounds__(kThreads) void awl_block_kernel(const AwlArgs a) {
  __shared__ double sh_lse[128];
  __shared__ float sh_tok[128], sh_lab[128];
  const int b = blockIdx.x;
  const int n_local = 2 * a.n_pos;
  int g = 64;
  while (g > 1 && n_local * g > kThreads) g >>= 1;
  const int lr = threadIdx.x / g, sub = threadIdx.x % g;
  const bool active = lr < n_local;
  const bool is_draft = lr >= a.n_pos;
  const int r = b * a.n_pos + (is_draft ? lr - a.n_pos : lr);
  const int grow = active ? (is_draft ? a.n_rows + r : r) : 0;
  const AwlPartial *p = a.part + static_cast<size_t>(grow) * a.chunks;
  float m = -INFINITY, zt = -INFINITY, zl = -INFINITY;
  if (active) {
    for (int c = sub; c < a.chunks; c += g) {
      const AwlPartial q = p[c];
      m = fmaxf(m, q.ref);
      zt = fmaxf(zt, q.z_tok);  // exactly one chunk holds the token: the others carry -inf
      zl = fmaxf(zl, q.z_lab);
    }
  }
  for (int o = g >> 1; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o));
    zt = fmaxf(zt, __shfl_xor(zt, o));
    zl = fmaxf(zl, __shfl_xor(zl, o));
  }
  double s = 0.0;
  if (active && m != -INFINITY) {
    for (int c = sub; c < a.chunks; c += g) {
      const AwlPartial q = p[c];
      if (q.ref != -INFINITY) s += q.sum * exp_fp64(static_cast<double>(q.ref) - m);
    }
  }
  for (int o = g >> 1; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (active && sub == 0) {
    sh_lse[lr] = static_cast<double>(m) + log(s);
    sh_tok[lr] = zt;
    sh_lab[lr] = zl;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // lane k: position k of the block
  const int k = threadIdx.x;
  const bool pos = k < a.n_pos;
  double alpha = 1.0, ce = 0.0;
  if (pos) {
    const double py = exp_fp64(static_cast<double>(sh_tok[k]) - sh_lse[k]);
    const double qy = exp_fp64(static_cast<double>(sh_tok[a.n_pos + k]) - sh_lse[a.n_pos + k]);
    alpha = qy > 0.0 ? fmin(1.0, py / qy) : 1.0;
    ce = sh_lse[a.n_pos + k] - static_cast<double>(sh_lab[a.n_pos + k]);
  }
  // w_k = prod_{j<k} alpha_j: exclusive prefix product over lanes
  double incl = alpha;
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(incl, o);
    if (k >= o) incl *= t;
  }
  double w = __shfl_up(incl, 1);
  if (k == 0) w = 1.0;
  const int rk = b * a.n_pos + k;
  const double inc = pos && (!a.include || a.include[rk] != 0) ? 1.0 : 0.0;
  double num = inc * w * ce, den = inc * w;
  for (int o = 32; o > 0; o >>= 1) {
    num += __shfl_xor(num, o);
    den += __shfl_xor(den, o);
  }
  if (pos) {
    a.weights[rk] = static_cast<float>(w);
    if (a.ce) a.ce[rk] = static_cast<float>(ce);
    a.lse[rk] = sh_lse[a.n_pos + k];
  }
  if (k == 0) {
    a.block_sums[2 * b] = num;
    a.block_sums[2 * b + 1] = den;
  }
}

__global__ __launch_bounds__(kThreads) void awl_final_kernel(const AwlArgs a) {
  __shared__ double sh_d[kWaves];
  double num = 0.0, den = 0.0;
  for (int b = threadIdx.x; b < a.n_blocks; b += kThreads) {
    num += a.block_sums[2 * b];
    den += a.block_sums[2 * b + 1];
  }
  num = block_sum(num, sh_d);
  den = block_sum(den, sh_d);
  if (threadIdx.x == 0) {
    a.loss[0] = num / (den + a.eps);
    a.scale[0] = 1.0 / (den + a.eps);
  }
}

// g = coef * Q(v) - coef [v = y*] with coef * Q(v) = 2^(z log2(e) - lse log2(e) + log2(coef)): one fma
// and one exp per element (coef = 0 gives 2^-inf = 0). The label's element is rewritten afterwards by
// the thread that stored its vector, so the two stores to it are ordered.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void awl_grad_kernel(const AwlArgs a) {
  const int r = blockIdx.y, chunk = blockIdx.x;
  const int lab = min(max(a.labels[r], 0), a.vocab - 1);
  const T *src = static_cast<const T *>(a.draft) + static_cast<size_t>(r) * a.vocab;
  T *dst = static_cast<T *>(a.grad) + static_cast<size_t>(r) * a.vocab;
  const int begin = chunk * a.chunk_len;
  const int end = min(begin + a.chunk_len, a.vocab);
  // the row's coefficient and exponent shift, from the earlier passes' outputs
  float coef = 0.f, shift = 0.f;
  const auto setup = [&] {
    const bool inc = !a.include || a.include[r] != 0;
    coef = inc ? static_cast<float>(static_cast<double>(a.weights[r]) * a.scale[0]) : 0.f;
    shift = static_cast<float>(-a.lse[r] * static_cast<double>(kLog2e) + log2(static_cast<double>(coef)));
  };
  const auto q_of = [&](float z) { return __builtin_amdgcn_exp2f(__builtin_fmaf(z, kLog2e, shift)); };
  if constexpr (VEC) {
    constexpr int W = 16 / sizeof(T);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(src + begin);
    u32x4 *wp = reinterpret_cast<u32x4 *>(dst + begin);
    const int nvec = (end - begin) / W;  // chunks hold whole vectors on this path
    const int lab_v = lab >= begin && lab < end ? (lab - begin) / W : -1;
    stream_vecs<kThreads, 4>(
        vp, nvec,
        [&](const u32x4 &w, int v) {
          float z[W];
          unpack<W>(w, z);
          float g[W];
#pragma unroll
          for (int k = 0; k < W; ++k) g[k] = q_of(z[k]);
          u32x4 o;
          if constexpr (W == 8) {
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(g[2 * k], g[2 * k + 1]);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = __float_as_uint(g[k]);
          }
          // non-temporal, like the loads: the gradient is not read back here (about 8 % faster for
          // the whole call than cached accesses when calls run back to back)
          __builtin_nontemporal_store(o, wp + v);
        },
        setup);
    if (lab_v >= 0 && static_cast<int>(threadIdx.x) == lab_v % kThreads)
      dst[lab] = static_cast<T>(q_of(load_elem(src + lab)) - coef);
  } else {
    setup();
    for (int v = begin + threadIdx.x; v < end; v += kThreads) {
      const float g = q_of(load_elem(src + v)) - (v == lab ? coef : 0.f);
      dst[v] = static_cast<T>(g);
    }
  }
}

struct AwlPlan {
  int chunks, chunk_len;
  size_t off_part, off_lse, off_sums, off_scale, total;
};

int plan_awl(int n_blocks, int n_pos, int vocab, AwlPlan *p) {
  if (n_blocks < 1 || n_pos < 1 || n_pos > 63 || vocab < 1 || vocab > kMaxVocab) return D3D_EINVAL;
  const long long rows = 2ll * n_blocks * n_pos;
  if (rows > INT_MAX) return D3D_EINVAL;
  int chunks = static_cast<int>(std::max<long long>(1, kAwlSlots / rows));
  chunks = std::min(chunks, (vocab + kAwlMinChunk - 1) / kAwlMinChunk);
  chunks = std::min(chunks, kAwlMaxChunks);
  int len = (vocab + chunks - 1) / chunks;
  len = (len + 63) / 64 * 64;
  p->chunk_len = len;
  p->chunks = (vocab + len - 1) / len;
  size_t off = 0;
  p->off_part = off;
  off = align_up(off + sizeof(AwlPartial) * static_cast<size_t>(rows) * p->chunks, 256);
  p->off_lse = off;
  off = align_up(off + sizeof(double) * static_cast<size_t>(n_blocks) * n_pos, 256);
  p->off_sums = off;
  off = align_up(off + sizeof(double) * 2 * static_cast<size_t>(n_blocks), 256);
  p->off_scale = off;
  off = align_up(off + sizeof(double), 256);
  p->total = off;
  return D3D_OK;
}

template <typename T, bool VEC>
void launch_awl(const AwlArgs &a, hipStream_t stream) {
  awl_stats_kernel<T, VEC><<<dim3(a.chunks, 2 * a.n_rows), kThreads, 0, stream>>>(a);
  awl_block_kernel<<<a.n_blocks, kThreads, 0, stream>>>(a);
  awl_final_kernel<<<1, kThreads, 0, stream>>>(a);
  if (a.grad) awl_grad_kernel<T, VEC><<<dim3(a.chunks, a.n_rows), kThreads, 0, stream>>>(a);
}

}  // namespace
}  // namespace d3d

extern "C" size_t awl_loss_workspace(int n_blocks, int n_pos, int vocab) {
  d3d::AwlPlan p;
  if (d3d::plan_awl(n_blocks, n_pos, vocab, &p) != D3D_OK) return 0;
  return p.total;
}

extern "C" int awl_loss(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
                        const int32_t *draft_tokens, const int32_t *labels, const int32_t *include, int n_blocks,
                        int n_pos, int vocab, double eps, float *weights, float *ce, double *loss, void *grad,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
  using namespace d3d;
  if (dtype != D3D_BF16 && dtype != D3D_F32) return D3D_EINVAL;
  if (!target_logits || !draft_logits || !draft_tokens || !labels || !weights || !loss) return D3D_EINVAL;
  if (!(eps >= 0.0) || !isfinite(eps)) return D3D_EINVAL;
  AwlPlan p;
  if (plan_awl(n_blocks, n_pos, vocab, &p) != D3D_OK) return D3D_EINVAL;
  if (!ws || ws_bytes < p.total) return D3D_EWORKSPACE;
  char *w = static_cast<char *>(ws);
  AwlArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.labels = labels;
  a.include = include;
  a.n_blocks = n_blocks;
  a.n_pos = n_pos;
  a.vocab = vocab;
  a.n_rows = n_blocks * n_pos;
  a.chunks = p.chunks;
  a.chunk_len = p.chunk_len;
  a.eps = eps;
  a.weights = weights;
  a.ce = ce;
  a.loss = loss;
  a.grad = grad;
  a.part = reinterpret_cast<AwlPartial *>(w + p.off_part);
  a.lse = reinterpret_cast<double *>(w + p.off_lse);
  a.block_sums = reinterpret_cast<double *>(w + p.off_sums);
  a.scale = reinterpret_cast<double *>(w + p.off_scale);
  const size_t esize = dtype == D3D_BF16 ? 2 : 4;
  const auto al = [](const void *q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  const bool vec = al(target_logits) && al(draft_logits) && (!grad || al(grad)) &&
                   (static_cast<size_t>(vocab) * esize) % 16 == 0;
  if (dtype == D3D_BF16) {
    if (vec)
      launch_awl<__bf16, true>(a, stream);
    else
      launch_awl<__bf16, false>(a, stream);
  } else {
    if (vec)
      launch_awl<float, true>(a, stream);
    else
      launch_awl<float, false>(a, stream);
  }
  return launch_status();
}
