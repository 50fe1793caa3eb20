// Internal definitions shared by the gfx950 kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "d3d.h"

namespace d3d {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// Largest vocabulary a logit row may have: the planners' chunk arithmetic stays inside int.
constexpr int kMaxVocab = 1 << 28;
// Longest request prefix draft attention takes: key positions and split lengths stay inside int.
constexpr int kMaxPrefix = 1 << 30;

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies; workgroups round-robin across them

// bf16 <-> f32 (bf16 is the upper half of an IEEE binary32 value).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// two fp32 values rounded to nearest-even bf16, packed low / high
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ float load_elem(const __bf16 *p) {
  return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t *>(p)) << 16);
}
__device__ __forceinline__ float load_elem(const float *p) { return *p; }

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11, section 3): per round, words 0 and 2 are multiplied by the round constants; the high
// halves are mixed with words 1 and 3 and the round key; the key advances by the Weyl constants.
struct Philox4 {
  uint32_t x[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32 x 32 -> 64-bit product per word (v_mad_u64_u32) instead of separate high and low halves
    const uint64_t pa = static_cast<uint64_t>(kMulA) * c0, pb = static_cast<uint64_t>(kMulB) * c2;
    const uint32_t hi_a = static_cast<uint32_t>(pa >> 32), lo_a = static_cast<uint32_t>(pa);
    const uint32_t hi_b = static_cast<uint32_t>(pb >> 32), lo_b = static_cast<uint32_t>(pb);
    const uint32_t n0 = hi_b ^ c1 ^ k0, n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  Philox4 out;
  out.x[0] = c0;
  out.x[1] = c1;
  out.x[2] = c2;
  out.x[3] = c3;
  return out;
}

// Uniform double on the 53-bit grid of [0, 1): top 27 bits of word 0, top 26 bits of word 1.
__device__ __forceinline__ double philox_uniform(uint64_t seed, uint32_t pos, uint32_t req,
                                                 uint32_t round, uint32_t purpose) {
  const Philox4 r = philox4x32_10(pos, req, round, purpose, static_cast<uint32_t>(seed),
                                  static_cast<uint32_t>(seed >> 32));
  const double hi = static_cast<double>(r.x[0] >> 5);
  const double lo = static_cast<double>(r.x[1] >> 6);
  return (hi * 67108864.0 + lo) * 0x1.0p-53;
}

// exp(x) in fp64 for x < 709 (the arguments here are differences from a row reference, at most
// about 84, or log-probabilities). Cody-Waite argument reduction (W. J. Cody and W. Waite, "Software
// Manual for the Elementary Functions", 1980): x = k ln2 + r with |r| <= ln2/2, ln2 split into a
// 21-bit head (k * head is exact) and a tail; then the Taylor series of e^r to degree 12
// (truncation below 2e-16 relative) and a scaling by 2^k. About 18 fp64 operations. NaN (from
// -inf - -inf) and arguments below the smallest subnormal give 0.
__device__ __forceinline__ double exp_fp64(double x) {
  constexpr double kInvLn2 = 1.4426950408889634;
  constexpr double kLn2Hi = 0.6931467056274414;      // ln 2 with its low 32 mantissa bits cleared
  constexpr double kLn2Lo = 4.7493250390316726e-07;  // ln 2 - kLn2Hi
  if (!(x > -745.5)) return 0.0;
  const double k = rint(x * kInvLn2);
  double r = fma(-k, kLn2Hi, x);
  r = fma(-k, kLn2Lo, r);
  double p = 2.08767569878681e-09;  // 1/12!
  p = fma(p, r, 2.505210838544172e-08);
  p = fma(p, r, 2.755731922398589e-07);
  p = fma(p, r, 2.7557319223985893e-06);
  p = fma(p, r, 2.48015873015873e-05);
  p = fma(p, r, 0.0001984126984126984);
  p = fma(p, r, 0.001388888888888889);
  p = fma(p, r, 0.008333333333333333);
  p = fma(p, r, 0.041666666666666664);
  p = fma(p, r, 0.16666666666666666);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, static_cast<int>(k));
}

// Cache match of one request ([D3D] 前置知识: 异步起草与缓存命中), run by one whole wavefront (every
// lane gets the result): the first branch block b of [b0 + 1, b1) in pack order whose rejection
// position is n_acc + 1 and whose anchor is the verified next token, as b - b0, or -1. Lanes test 64
// consecutive blocks at a time; the lowest matching lane of the first window with one wins.
__device__ __forceinline__ int match_request(const d3d_block_desc *descs, int b0, int b1, int want_r, int tok) {
  const int lane = threadIdx.x & 63;
  for (int base = b0 + 1; base < b1; base += 64) {
    const int b = base + lane;
    bool m = false;
    if (b < b1) {
      const d3d_block_desc d = descs[b];
      m = d.rej_pos == want_r && d.anchor == tok;
    }
    const unsigned long long bal = __ballot(m);
    if (bal) return base + (__ffsll(static_cast<long long>(bal)) - 1) - b0;
  }
  return -1;
}

// Streams the nvec 16-byte vectors of a slice through f(vector, index) with NT threads, thread t
// taking vectors t, t + NT, ... The full steps (U vectors for every lane) run with a uniform trip count and no
// per-lane predicate, in two register sets used in turn: the next step's loads are issued before the
// current step's vectors are consumed, so every wave keeps loads in flight while it computes (two
// sets rather than a copy, which would wait for the loads). The data are read once per pass:
// non-temporal loads. A prefetch past the full steps reads
// clamped, in-bounds positions and is not consumed; the remaining vectors follow one per lane.
template <int NT, int U, typename F, typename P>
__device__ __forceinline__ void stream_vecs(const u32x4 *vp, int nvec, F &&f, P &&after_first_loads) {
  constexpr int S = NT * U;
  const int full = nvec / S;
  const int t = threadIdx.x;
  const auto fetch = [&](u32x4 (&b)[U], int v0) {
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = __builtin_nontemporal_load(vp + min(v0 + u * NT, nvec - 1));
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the consumption that follows
  };
  const auto consume = [&](const u32x4 (&b)[U], int v0) {
#pragma unroll
    for (int u = 0; u < U; ++u) f(b[u], v0 + u * NT);
  };
  if (nvec <= 0) {
    after_first_loads();
    return;
  }
  u32x4 a[U], b[U];
  fetch(a, t);
  after_first_loads();
  if (full > 0) {
    int s = 0;
    for (; s + 2 <= full; s += 2) {
      fetch(b, t + (s + 1) * S);
      consume(a, t + s * S);
      fetch(a, t + (s + 2) * S);
      consume(b, t + (s + 1) * S);
    }
    if (s < full) consume(a, t + s * S);
  }
  for (int v = full * S + t; v < nvec; v += NT) f(vp[v], v);
}

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? D3D_OK : D3D_EHIP;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------------------------------------------
// Wavefront collectives without LDS traffic: DPP moves inside rows of 16 lanes and gfx950's
// permlane swaps between rows. (A lane shuffle goes through ds_bpermute, an LDS round trip per
// step; these are VALU moves.) A reduction leaves its result in every lane of the group; its
// operation must be commutative and associative, since inside a row the partner is a mirror lane,
// not the xor lane.
// ------------------------------------------------------------------------------------------------
namespace wave {

// DPP controls (GFX9 encoding)
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15 - i within 16
constexpr int kRowShr = 0x110;        // + k: lane i takes lane i - k of its row
constexpr int kRowBcast15 = 0x142;    // lane 15 of a row to every lane of the next row
constexpr int kRowBcast31 = 0x143;    // lane 31 to every lane of rows 2 and 3
constexpr int kWaveShr1 = 0x138;      // lane i takes lane i - 1 of the wavefront

template <typename T>
struct Words;
template <>
struct Words<float> {
  static constexpr int N = 1;
  __device__ static void split(float v, uint32_t (&w)[1]) { w[0] = __float_as_uint(v); }
  __device__ static float join(const uint32_t (&w)[1]) { return __uint_as_float(w[0]); }
};
template <>
struct Words<int> {
  static constexpr int N = 1;
  __device__ static void split(int v, uint32_t (&w)[1]) { w[0] = static_cast<uint32_t>(v); }
  __device__ static int join(const uint32_t (&w)[1]) { return static_cast<int>(w[0]); }
};
template <>
struct Words<double> {
  static constexpr int N = 2;
  __device__ static void split(double v, uint32_t (&w)[2]) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    w[0] = static_cast<uint32_t>(b);
    w[1] = static_cast<uint32_t>(b >> 32);
  }
  __device__ static double join(const uint32_t (&w)[2]) {
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(w[1]) << 32) | w[0]));
  }
};

// The DPP move CTRL of v; lanes without a source (or outside ROW_MASK) get `old`.
template <int CTRL, int ROW_MASK = 0xF, typename T>
__device__ __forceinline__ T move(T old, T v) {
  using W = Words<T>;
  uint32_t o[W::N], x[W::N];
  W::split(old, o);
  W::split(v, x);
#pragma unroll
  for (int k = 0; k < W::N; ++k)
    x[k] = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(o[k]), static_cast<int>(x[k]), CTRL, ROW_MASK, 0xF, false));
  return W::join(x);
}

// op of v over the lane pairs (i, i ^ 16) (ROWS = 16) or (i, i ^ 32) (ROWS = 32), in every lane.
template <int ROWS, typename T, typename Op>
__device__ __forceinline__ T swap_combine(T v, Op op) {
  using W = Words<T>;
  uint32_t x[W::N], a[W::N], b[W::N];
  W::split(v, x);
#pragma unroll
  for (int k = 0; k < W::N; ++k) {
    if constexpr (ROWS == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(x[k], x[k], false, false);
      a[k] = r[0];
      b[k] = r[1];
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(x[k], x[k], false, false);
      a[k] = r[0];
      b[k] = r[1];
    }
  }
  return op(W::join(a), W::join(b));
}

// op over each group of G consecutive lanes (G a power of two, 1..64; uniform across the wave).
template <typename T, typename Op>
__device__ __forceinline__ T reduce(T v, int G, Op op) {
  if (G > 1) v = op(v, move<kQuadXor1>(v, v));
  if (G > 2) v = op(v, move<kQuadXor2>(v, v));
  if (G > 4) v = op(v, move<kRowHalfMirror>(v, v));
  if (G > 8) v = op(v, move<kRowMirror>(v, v));
  if (G > 16) v = swap_combine<16>(v, op);
  if (G > 32) v = swap_combine<32>(v, op);
  return v;
}

// Inclusive scan over the 64 lanes in lane order; `id` is op's identity.
template <typename T, typename Op>
__device__ __forceinline__ T incl_scan(T v, T id, Op op) {
  v = op(v, move<kRowShr + 1>(id, v));
  v = op(v, move<kRowShr + 2>(id, v));
  v = op(v, move<kRowShr + 4>(id, v));
  v = op(v, move<kRowShr + 8>(id, v));
  v = op(v, move<kRowBcast15, 0xA>(id, v));
  v = op(v, move<kRowBcast31, 0xC>(id, v));
  return v;
}

// The previous lane's value (lane 0: id): an inclusive scan made exclusive.
template <typename T>
__device__ __forceinline__ T shift_up(T v, T id) {
  return move<kWaveShr1>(id, v);
}

struct Add {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct Mul {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a * b; }
};
struct Max {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct Min {
  __device__ int operator()(int a, int b) const { return a < b ? a : b; }
};

}  // namespace wave

}  // namespace d3d
