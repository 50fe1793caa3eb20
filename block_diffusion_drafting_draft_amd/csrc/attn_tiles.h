// Shared pieces of the bf16 attention walks (the packed draft attention and the training-time
// attention): LDS tile geometry and swizzle, fragment addresses, LDS-DMA copies, waits and barriers,
// and the one-tile online-softmax step.
#pragma once

#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kKeys = 64;  // keys per tile

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_PTR(type, p) ((__attribute__((address_space(3))) type *)(p))

// ------------------------------------------------------------------------------------------------
// bf16: two wavefronts of 64 rows, LDS-DMA tiles, swizzled rows, transposing V reads
// ------------------------------------------------------------------------------------------------
// A workgroup is eight wavefronts, one per CU; each wavefront owns 32 of the item's 256 rows (two
// wavefronts per SIMD, whose MFMA and VALU phases interleave). Every K/V tile in LDS serves all 256
// rows, and a ring of four tiles keeps three copies in flight ahead of the one being computed.
constexpr int kBfThreads = 512;
constexpr int kStages = 4;
// Lazy rescale: a row's softmax reference moves only when a tile's maximum exceeds it by more than
// kSlack (log2 units), so stored probabilities stay below 2^kSlack and the O rescale is rare.
constexpr float kSlack = 8.f;

// XOR swizzle of the 16-byte chunks of LDS row r. 256-byte rows (d = 128): chunk c of row r lives at
// c ^ f(r) with f(r) = ((r & 3) << 2) | ((r >> 2) & 3) -- a bijection over any 16 aligned rows (the K
// fragment reads: 16 rows, same chunk) that also puts the 4 aligned chunks of 4 consecutive rows in
// distinct bank groups (the transposing V reads). 128-byte rows (d = 64) share a bank line in pairs:
// f(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3) has the same two properties there. f depends on
// r mod 16 only.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
struct DmaTile {
  static constexpr int RB = D * 2;                      // bytes per LDS row (one key, one head)
  static constexpr int CH = D / 8;                      // 16-byte chunks per row
  static constexpr int BYTES = kKeys * RB;              // one K or V tile
  static constexpr int NI = BYTES / (kBfThreads * 16);  // DMA instructions per wavefront per operand
  static constexpr int RPI = 64 / CH;                   // rows per DMA instruction
};

// LDS byte offsets of this lane's fragments inside a tile, fixed for the whole walk.
//  K (A operand of S^T = K Q^T), k-step kk: row col (+32 for the second 32-key half), chunk 2kk + hh.
//  V^T (A operand of O^T = V^T P^T), k-step t, column block b: lane l gets column 32b + l%32 of keys
//  16t + 4hh + {0..3} (first transposing read) and 16t + 8 + 4hh + {0..3} (second); inside its
//  16-lane group, lane j points at row 16t + 4hh + j/4 (+8), columns 32b + 16((l>>4)&1) + 4(j%4).
// Row bases are multiples of the row size and the swizzle acts on the chunk bits only, so the offset
// of k-step kk is k ^ (kk << 5) and that of column block b is v ^ (b << 6); t moves by 16 rows, an
// immediate. Three registers instead of one per fragment.
template <int D>
struct FragAddr {
  uint32_t k, vlo, vhi;
  __device__ __forceinline__ uint32_t kof(int kk) const { return k ^ static_cast<uint32_t>(kk << 5); }
  __device__ __forceinline__ uint32_t vlof(int b) const { return vlo ^ static_cast<uint32_t>(b << 6); }
  __device__ __forceinline__ uint32_t vhif(int b) const { return vhi ^ static_cast<uint32_t>(b << 6); }
};

template <int D>
__device__ __forceinline__ FragAddr<D> frag_addr() {
  using TT = DmaTile<D>;
  const int lane = threadIdx.x & 63, col = lane & 31, hh = lane >> 5;
  const int j = lane & 15, dd = (lane >> 4) & 1;
  FragAddr<D> f;
  f.k = col * TT::RB + ((hh ^ swz<D>(col)) << 4);
  const int r1 = 4 * hh + (j >> 2), r2 = r1 + 8;
  const int ch = 2 * dd + ((j & 3) >> 1), byte = (j & 1) * 8;
  f.vlo = r1 * TT::RB + ((ch ^ swz<D>(r1)) << 4) + byte;
  f.vhi = r2 * TT::RB + ((ch ^ swz<D>(r2)) << 4) + byte;
  return f;
}

// DMA geometry of this lane: instruction i of wavefront w fills LDS bytes [(w*NI + i)*1024, +1024),
// lane l the 16 bytes at l*16: row (w*NI + i)*RPI + l/CH, physical chunk l % CH, which holds the
// row's logical chunk (l % CH) ^ swz(row). Recomputed where used (a few integer operations) rather
// than held in registers for the whole walk.
template <int D>
__device__ __forceinline__ int dma_row(int i) {
  using TT = DmaTile<D>;
  return ((threadIdx.x >> 6) * TT::NI + i) * TT::RPI + (threadIdx.x & 63) / TT::CH;
}

template <int D>
__device__ __forceinline__ uint32_t dma_chunk(int i) {
  return static_cast<uint32_t>((((threadIdx.x & 63) % DmaTile<D>::CH) ^ swz<D>(dma_row<D>(i))) << 4);
}

// The copies into LDS are issued as inline assembly: the compiler then does not see them as LDS
// writes, so it neither tracks nor waits for them before LDS reads (its tracking is per LDS object
// and limited, and a lost track costs a wait for every copy in flight). Completion is handled
// explicitly: wait_vm before the barrier that publishes a stage, and a full wait before reuse.
// Vector-memory operations complete in issue order, so extra younger operations only make the
// compiler's own vmcnt waits stricter. m0 holds the wavefront's LDS destination (an asm input).
template <int D>
__device__ __forceinline__ uint32_t lds_dst(char *lds, int i) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(char, lds))) + (wave * DmaTile<D>::NI + i) * 1024;
}

// 16 bytes per lane from a 64-bit per-lane address.
template <int D>
__device__ __forceinline__ void dma16(const char *src, char *lds, int i) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_dst<D>(lds, i)) : "memory");
}

// 16 bytes per lane from a wave-uniform base plus a 32-bit lane offset.
template <int D>
__device__ __forceinline__ void dma16_s(const char *base, uint32_t voff, char *lds, int i) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_dst<D>(lds, i)) : "memory");
}

// The same through a buffer resource (base and byte range in SGPRs): the tile position is a scalar
// offset, and bytes outside the range read as zero.
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data format

template <int D>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, char *lds, int i, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
               "{m0}"(lds_dst<D>(lds, i))
               : "memory");
}

// Wait until at most N vector-memory operations of this wavefront are outstanding (the copies of
// later tiles may stay in flight). Other counters are not waited on.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence: __syncthreads() releases at workgroup scope, which waits
// for every outstanding vector-memory operation (vmcnt(0)) and would drain the copies of later
// tiles. The copy the next step reads has been waited for explicitly (wait_vm), this wavefront's LDS
// reads are complete (lgkmcnt(0)), and the memory clobber keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void barrier_keep_copies() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D>
struct Rows1 {
  f32x16 o[D / 32];
  float m;  // softmax reference (scaled log2 units), -inf until a key is visible
  float l;  // this lane's half of the running sum
};

// One 64-key tile: S^T = K Q^T, mask (MASK only), tile maximum and (rarely) the O rescale, then
// P = 2^(c*S - m) as the bf16 B operand of O^T += V^T P^T. The lane holds the keys
// kappa = mb*32 + 8*(r/4) + 4*hh + r%4 of its query column; visible(kappa - 4*hh) decides the mask
// (the lane's 4*hh is folded into the caller's limit or table pointer, so the argument is a
// compile-time constant). The row sum adds the bf16 values the PV product uses.
template <int D, bool MASK, typename VIS>
__device__ __forceinline__ void tile1(const char *kst, const char *vst, const FragAddr<D> &fa,
                                      const bf16x8 (&q)[D / 16], Rows1<D> &st, float c, VIS visible) {
  using TT = DmaTile<D>;
  // The fragment reads are fenced into halves (scheduling barriers) so that at most half a tile of
  // K or V fragments is in flight: the other wavefront of the SIMD covers the LDS latency.
  // Each k-step's two K fragments are read one step ahead of their MFMAs (scheduling groups: the
  // reads of steps 0 and 1, then per step two MFMAs and the next step's reads).
  f32x16 s[2] = {};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int kk = h * D / 32; kk < (h + 1) * D / 32; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kst + fa.kof(kk) + 32 * mb * TT::RB);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q[kk], s[mb], 0, 0, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);  // reads of the first two k-steps
#pragma unroll
    for (int kk = 0; kk < D / 32 - 2; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);  // MFMAs of step kk
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);  // reads of step kk + 2
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 2);  // MFMAs of the last two steps
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (MASK) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[mb][r] = visible(mb * 32 + 8 * (r >> 2) + (r & 3)) ? s[mb][r] : -INFINITY;
      }
  }
  // row maximum: a max3 tree over the lane's 32 keys, then the other half of the column (lane ^ 32)
  // through the half swap, which leaves the lane's own value in one result and its partner's in the
  // other
  float m1[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int x = 3 * i, y = 3 * i + 1, z = 3 * i + 2;
    m1[i] = fmaxf(fmaxf(s[x >> 4][x & 15], s[y >> 4][y & 15]), s[z >> 4][z & 15]);
  }
  m1[10] = fmaxf(s[1][14], s[1][15]);
  float mx = fmaxf(fmaxf(fmaxf(fmaxf(m1[0], m1[1]), m1[2]), fmaxf(fmaxf(m1[3], m1[4]), m1[5])),
                   fmaxf(fmaxf(fmaxf(m1[6], m1[7]), m1[8]), fmaxf(m1[9], m1[10])));
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const float mt = mx * c;
  const bool up = mt > st.m + kSlack;  // m = -inf: any finite maximum moves it
  if (__ballot(up)) {
    const float mn = up ? mt : st.m;
    const float al = up ? __builtin_amdgcn_exp2f(st.m - mn) : 1.f;
    st.l *= al;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[b][r] *= al;
    st.m = mn;
  }
  const float mu = st.m == -INFINITY ? 0.f : st.m;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  bf16x8 p[4];
  float part[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains for the row sum
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      p[t][i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + i], c, -mu)));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16x2 pr = {p[t][2 * u], p[t][2 * u + 1]};
      part[u] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, part[u], false);
    }
  }
  st.l += (part[0] + part[1]) + (part[2] + part[3]);
  // V^T fragments likewise one MFMA ahead (two transposing reads each).
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 2 * h; t < 2 * h + 2; ++t)
#pragma unroll
      for (int b = 0; b < D / 32; ++b) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vst + fa.vlof(b) + 16 * t * TT::RB));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vst + fa.vhif(b) + 16 * t * TT::RB));
        const v4i16 both[2] = {lo, hi};
        st.o[b] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(both), p[t], st.o[b], 0, 0, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 3);  // fragments of the first two MFMAs
#pragma unroll
    for (int i = 0; i < D / 16 - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 3);
  }
}

// Key / value source of the bf16 walk: a contiguous per-request cache, a paged cache whose page size
// is a multiple of the rows one DMA instruction covers (page id wave-uniform), or any paged cache.

}  // namespace
}  // namespace d3d
