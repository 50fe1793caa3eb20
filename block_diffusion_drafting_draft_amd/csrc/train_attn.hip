// Training-time packed attention, forward and backward, on gfx950.
//
// What is computed ([D3D] 方法步骤详情 step 2 and 核心方法; [DScout] 方法步骤详情 step 2 for the
// horizons B in {8, 16, 24, 32}): one training response of L tokens is followed in the packed
// sequence by n_blocks diffusion blocks of B rows, block i starting at the anchor a_i of the
// response. A response row p attends to response keys j <= p (causal, shared as every block's
// prefix); a row of block i attends to the response keys j < a_i and to every row of block i
// (bidirectional inside the block); no row sees another block. Grouped-query heads: query head h
// uses key / value head h / (H_q / H_kv).
//   forward:  o = softmax(scale q k^T) v per visible set, lse = log sum exp(scale q k^T)
//   backward: D = rowsum(do * o), dS = P (do v^T - D), dq = scale dS k, dk = scale dS^T q, dv = P^T do
//
// Query-centric passes (forward, dq): a workgroup of 8 wavefronts owns 256 query-head rows of one
// key / value head -- 256 / G positions x the G heads of the group, each wavefront 32 rows -- and
// walks two key ranges through the four-stage LDS-DMA ring of the draft attention: the response keys
// below the largest limit of its rows (each wavefront skips the tiles past its own rows' limits and
// masks only the tiles that cut through them), then the rows of the blocks its rows belong to.
// S^T = K Q^T with Q in registers (the B operand), so every lane holds one row's column.
//   forward: the online-softmax step of the draft attention, then o and lse.
//   dq:      P^T = 2^(c S^T - lse2) with the stored lse, dP^T = V dO^T (dO in registers like Q),
//            dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (transposing reads of the K tile); it also
//            writes D for the key-centric pass.
// Key-centric pass (dk, dv): a workgroup of 4 wavefronts owns 128 keys of one key / value head, each
// wavefront 32 keys (K and V in registers as B operands), and walks the query tiles (64 rows) that
// can see them: S = Q K^T, P = 2^(c S - lse2), dP = dO V^T, dS = P (dP - D), then
// dV^T += dO^T P and dK^T += Q^T dS with transposing reads of the dO and Q tiles.
#include <float.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "attn_tiles.h"
#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kTD = 128;          // head dimension
constexpr int kQRows = 256;       // query-head rows per query-centric workgroup
constexpr int kKThreads = 256;    // key-centric workgroup: 4 wavefronts
constexpr int kKKeys = 128;       // keys per key-centric workgroup
constexpr int kMaxAnchors = 2048;  // blocks per call (the key-centric pass keeps them in LDS)
constexpr float kLog2eF = 1.4426950408889634f;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
constexpr float kLn2F = 0.6931471805599453f;

struct TrainArgs {
  const void *q, *k, *v;
  const void *o, *dout;  // backward inputs
  void *out;             // forward output / dq
  float *lse;            // [N, H_q], natural log of the partition of scale q k^T
  float *delta;          // [N, H_q], rowsum(do * o) (written by the dq pass)
  void *dk, *dv;
  const int32_t *anchors;
  int L, n_blocks, B, N, Hq, Hkv, G;
  int n_qitems;  // query-centric items per key / value head
  int n_kitems;  // key-centric items per key / value head
  float scale, c;  // c = scale * log2(e)
};

// Row geometry of a packed position: the response keys it sees ([0, lim)) and its own block's key
// rows ([blo, bhi), empty for response rows and rows past N).
struct RowSeg {
  int lim, blo, bhi;
};

__device__ __forceinline__ RowSeg row_seg(const TrainArgs &a, int pos) {
  RowSeg s;
  if (pos < a.L) {
    s.lim = pos + 1;
    s.blo = s.bhi = 0;
  } else if (pos < a.N) {
    const int b = (pos - a.L) / a.B;
    s.lim = min(max(a.anchors[b], 0), a.L);
    s.blo = a.L + b * a.B;
    s.bhi = s.blo + a.B;
  } else {
    s.lim = 0;
    s.blo = s.bhi = 0;
  }
  return s;
}

// Workgroup id -> (item, kv head): the key / value head varies fastest, so with H_kv = 8 every item
// of one head runs on one XCD (workgroup w runs on XCD w % 8) and its L2 holds that head's keys.
// Items are taken from the end of the packed sequence: the block region first, then the response
// from its end down, so the longer response walks start before the shorter ones.
__device__ __forceinline__ void item_of(int n_items, int Hkv, int &item, int &g) {
  const int w = blockIdx.x;
  g = w % Hkv;
  item = n_items - 1 - w / Hkv;
}

__device__ __forceinline__ int wave_min(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// The four-stage ring over key rows [k0, k1) of one key / value head: tile i is copied three tiles
// ahead into stage i % 4; compute(kst, vst, kt) runs on every tile (kt = the tile's first key row),
// after_first() once after the first copies are issued (it must end with a full wait). Rows past N
// read as zero (the buffer's range check, applied to the lane offset that carries the tile offset);
// rows past k1 are the caller's to mask.
template <typename Compute, typename First>
__device__ __forceinline__ void ring_walk(char *const (&stk)[kStages], char *const (&stv)[kStages],
                                          __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                          const uint32_t (&off)[DmaTile<kTD>::NI], uint32_t row_bytes, int k0, int k1,
                                          Compute &&compute, First &&after_first) {
  using TT = DmaTile<kTD>;
  const int n_tiles = (k1 - k0 + kKeys - 1) / kKeys;
  auto issue = [&](int s, int kt) __attribute__((always_inline)) {
    // the tile offset goes into the lane offset, which the buffer's range check covers
    const uint32_t toff = static_cast<uint32_t>(kt) * row_bytes;
#pragma unroll
    for (int i = 0; i < TT::NI; ++i) {
      dma16_buf<kTD>(krs, stk[s], i, off[i] + toff, 0);
      dma16_buf<kTD>(vrs, stv[s], i, off[i] + toff, 0);
    }
  };
  if (n_tiles <= 0) {
    after_first();
    return;
  }
  issue(0, k0);
  if (n_tiles > 1) issue(1, k0 + kKeys);
  if (n_tiles > 2) issue(2, k0 + 2 * kKeys);
  after_first();
  barrier_keep_copies();
  auto wait_next = [&](int i) __attribute__((always_inline)) {
    const int later = n_tiles - i - 2;  // tiles issued after tile i + 1 (at most two)
    if (later >= 2)
      wait_vm<4 * TT::NI>();
    else if (later == 1)
      wait_vm<2 * TT::NI>();
    else
      wait_vm<0>();
    barrier_keep_copies();
  };
  for (int i = 0; i < n_tiles; i += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      if (i + u < n_tiles) {
        if (i + u + 3 < n_tiles) issue((u + 3) % kStages, k0 + (i + u + 3) * kKeys);
        compute(stk[u], stv[u], k0 + (i + u) * kKeys);
        wait_next(i + u);
      }
    }
  }
}

// One dq tile: S^T = K Q^T, P^T = 2^(c S^T - lse2) (0 where masked), dP^T = V dO^T,
// dS^T = P^T (dP^T - D), dQ^T += K^T dS^T, one 32-key half at a time (register pressure). The lane
// holds keys kappa = mb*32 + 8*(r/4) + 4*hh + r%4 of its row column; visible(kappa - 4*hh) as in the
// forward step.
template <bool MASK, typename VIS>
__device__ __forceinline__ void dq_tile(const char *kst, const char *vst, const FragAddr<kTD> &fa,
                                        const bf16x8 (&q)[kTD / 16], const bf16x8 (&dof)[kTD / 16], f32x16 (&acc)[kTD / 32],
                                        float c, float lse2, float dlt, VIS visible) {
  using TT = DmaTile<kTD>;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int kk = 0; kk < kTD / 16; ++kk) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kst + fa.kof(kk) + 32 * mb * TT::RB);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q[kk], s, 0, 0, 0);
      const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vst + fa.kof(kk) + 32 * mb * TT::RB);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[kk], dp, 0, 0, 0);
    }
    bf16x8 ds[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * t2 + i;
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
        if constexpr (MASK) p = visible(mb * 32 + 8 * (r >> 2) + (r & 3)) ? p : 0.f;
        ds[t2][i] = static_cast<__bf16>(p * (dp[r] - dlt));
      }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int t = 2 * mb + t2;
#pragma unroll
      for (int b = 0; b < kTD / 32; ++b) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, kst + fa.vlof(b) + 16 * t * TT::RB));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, kst + fa.vhif(b) + 16 * t * TT::RB));
        const v4i16 both[2] = {lo, hi};
        acc[b] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(both), ds[t2], acc[b], 0, 0, 0);
      }
    }
  }
}

// Query-centric pass: BWD = false is the forward (o, lse), BWD = true the dq pass (dq, D).
template <bool BWD>
__global__ __launch_bounds__(kBfThreads, 1) void train_q_kernel(const TrainArgs a) {
  using TT = DmaTile<kTD>;
  __shared__ __attribute__((aligned(1024))) char lds_s0[2 * TT::BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s1[2 * TT::BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s2[2 * TT::BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s3[2 * TT::BYTES];
  __shared__ int sh_red[4][kBfThreads / 64];
  char *const stk[kStages] = {lds_s0, lds_s1, lds_s2, lds_s3};
  char *const stv[kStages] = {lds_s0 + TT::BYTES, lds_s1 + TT::BYTES, lds_s2 + TT::BYTES, lds_s3 + TT::BYTES};
  int item, g;
  item_of(a.n_qitems, a.Hkv, item, g);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5;
  const int P = 32 / a.G;  // positions per wavefront
  const int col = lane & 31;
  const int pos = item * (kQRows / a.G) + wave * P + col / a.G;
  const int h = g * a.G + col % a.G;
  const bool valid = pos < a.N;
  const RowSeg seg = row_seg(a, pos);
  // wavefront and workgroup extents of the two key ranges
  const int w_lim_max = wave_max(seg.lim), w_lim_min = wave_min(valid ? seg.lim : INT_MAX);
  const bool has_blk = seg.bhi > seg.blo;
  const int w_blo = wave_min(has_blk ? seg.blo : INT_MAX), w_bhi = wave_max(has_blk ? seg.bhi : 0);
  if (lane == 0) {
    sh_red[0][wave] = w_lim_max;
    sh_red[1][wave] = w_blo;
    sh_red[2][wave] = w_bhi;
  }
  __syncthreads();
  int g_lim = 0, g_blo = INT_MAX, g_bhi = 0;
#pragma unroll
  for (int w = 0; w < kBfThreads / 64; ++w) {
    g_lim = max(g_lim, sh_red[0][w]);
    g_blo = min(g_blo, sh_red[1][w]);
    g_bhi = max(g_bhi, sh_red[2][w]);
  }
  const size_t row_q = static_cast<size_t>(valid ? pos : 0) * a.Hq + h;  // (position, head) row
  bf16x8 qf[kTD / 16], dof[kTD / 16];
  float lse2 = 0.f, dlt = 0.f;
  auto load_rows = [&]() __attribute__((always_inline)) {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + row_q * kTD;
#pragma unroll
    for (int kk = 0; kk < kTD / 16; ++kk)
      qf[kk] = valid ? *reinterpret_cast<const bf16x8 *>(qrow + kk * 16 + hh * 8) : bf16x8{};
    if constexpr (BWD) {
      const __bf16 *drow = static_cast<const __bf16 *>(a.dout) + row_q * kTD;
      const __bf16 *orow = static_cast<const __bf16 *>(a.o) + row_q * kTD;
      float part = 0.f;
#pragma unroll
      for (int kk = 0; kk < kTD / 16; ++kk) {
        dof[kk] = valid ? *reinterpret_cast<const bf16x8 *>(drow + kk * 16 + hh * 8) : bf16x8{};
        const bf16x8 of = valid ? *reinterpret_cast<const bf16x8 *>(orow + kk * 16 + hh * 8) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) part += static_cast<float>(dof[kk][e]) * static_cast<float>(of[e]);
      }
      dlt = part + __shfl_xor(part, 32);
      lse2 = valid ? a.lse[row_q] * kLog2eF : 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);
  };
  const FragAddr<kTD> fa = frag_addr<kTD>();
  const uint32_t row_bytes = static_cast<uint32_t>(a.Hkv * kTD * 2);
  uint32_t off[TT::NI];
#pragma unroll
  for (int i = 0; i < TT::NI; ++i) off[i] = static_cast<uint32_t>(dma_row<kTD>(i)) * row_bytes + dma_chunk<kTD>(i);
  const size_t gb = static_cast<size_t>(g) * kTD * 2;
  const int range = static_cast<int>(static_cast<size_t>(a.N) * row_bytes - gb);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.k) + gb), 0, range, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.v) + gb), 0, range, kBufWord3);
  const float c = a.c;

  Rows1<kTD> st;  // forward: online softmax state; dq: st.o is the dQ^T accumulator
#pragma unroll
  for (int b = 0; b < kTD / 32; ++b) st.o[b] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  auto step = [&](const char *kst, const char *vst, auto masked, auto vis) __attribute__((always_inline)) {
    if constexpr (BWD)
      dq_tile<decltype(masked)::value>(kst, vst, fa, qf, dof, st.o, c, lse2, dlt, vis);
    else
      tile1<kTD, decltype(masked)::value>(kst, vst, fa, qf, st, c, vis);
  };
  using No = std::integral_constant<bool, false>;
  using Yes = std::integral_constant<bool, true>;
  // response keys [0, g_lim): unmasked below the wavefront's smallest limit
  bool loaded = false;
  ring_walk(
      stk, stv, krs, vrs, off, row_bytes, 0, g_lim,
      [&](const char *kst, const char *vst, int kt) __attribute__((always_inline)) {
        if (kt >= w_lim_max) return;
        if (kt + kKeys <= w_lim_min) {
          step(kst, vst, No{}, [](int) { return true; });
        } else {
          const int lim_hh = seg.lim - kt - 4 * hh;
          step(kst, vst, Yes{}, [&](int kc) { return kc < lim_hh; });
        }
      },
      [&]() __attribute__((always_inline)) {
        load_rows();
        loaded = true;
      });
  if (!loaded) load_rows();
  // rows of the workgroup's blocks [g_blo, g_bhi): each row sees its own block's rows
  if (g_bhi > g_blo) {
    __syncthreads();
    ring_walk(
        stk, stv, krs, vrs, off, row_bytes, g_blo, g_bhi,
        [&](const char *kst, const char *vst, int kt) __attribute__((always_inline)) {
          if (kt >= w_bhi || kt + kKeys <= w_blo) return;
          const int lo = seg.blo - kt - 4 * hh, hi = seg.bhi - kt - 4 * hh;
          step(kst, vst, Yes{}, [&](int kc) { return (static_cast<int>(kc >= lo) & static_cast<int>(kc < hi)) != 0; });
        },
        [] { wait_vm<0>(); });  // the first tile's copy has landed before the first step
  }
  if (!valid) return;
  float mul;
  if constexpr (BWD) {
    mul = a.scale;
    if (hh == 0) a.delta[row_q] = dlt;
  } else {
    const float l_tot = st.l + __shfl_xor(st.l, 32);
    mul = 1.f / l_tot;
    if (hh == 0) a.lse[row_q] = (st.m + __log2f(l_tot)) * kLn2F;
  }
  __bf16 *orow = static_cast<__bf16 *>(a.out) + row_q * kTD;
#pragma unroll
  for (int b = 0; b < kTD / 32; ++b)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = b * 32 + 8 * r4 + 4 * hh;
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = static_cast<__bf16>(st.o[b][4 * r4 + e] * mul);
      *reinterpret_cast<bf16x4 *>(orow + d0) = v4;
    }
}

// ------------------------------------------------------------------------------------------------
// key-centric pass: dk, dv
// ------------------------------------------------------------------------------------------------
constexpr int kQTRows = 64;                                    // query-head rows per query tile
constexpr int kMaxList = 4096;                                 // listed query tiles of the block region
constexpr int kKvNI = kQTRows * kTD * 2 / (kKThreads * 16);   // 16-byte copies per wavefront per operand
constexpr int kKvOps = 2 * kKvNI + 2;                          // copies per wavefront per tile (+ 2 tables)
// query tiles per workgroup: at L 4096 + 128 x 16, 32/8 heads the backward measured 1066-1099 us with
// 96, 1023-1048 with 112 or 128, 1064-1073 with 144 or 160
constexpr int kWalkChunk = 128;

struct KStage {
  char q[kQTRows * kTD * 2];
  char d[kQTRows * kTD * 2];
  float lse[kKThreads / 64][kQTRows];  // each wavefront copies its own rows' tables
  float dlt[kKThreads / 64][kQTRows];
};

// LDS-DMA copies of the key-centric ring (4 wavefronts): copy i of this wavefront fills bytes
// [(wave*4 + i)*1024, +1024) of a 16 KB operand tile, 16 bytes a lane; the table copies put one
// dword a lane at dst + lane*4.
__device__ __forceinline__ uint32_t kv_dst(const char *lds, int i) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(const char, lds))) + (wave * kKvNI + i) * 1024;
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(const char, p)));
}
__device__ __forceinline__ void kv_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t dst, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(dst) : "memory");
}
__device__ __forceinline__ void kv_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t dst, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(dst) : "memory");
}

// Visible response keys [0, lim) and own-block keys [blo, bhi) of a packed position (anchors in LDS).
__device__ __forceinline__ RowSeg row_seg_lds(const TrainArgs &a, const int *anc, int pos) {
  RowSeg s;
  s.lim = 0;
  s.blo = s.bhi = 0;
  if (pos < a.L) {
    s.lim = pos + 1;
  } else if (pos < a.N) {
    const int b = (pos - a.L) / a.B;
    s.lim = anc[b];
    s.blo = a.L + b * a.B;
    s.bhi = s.blo + a.B;
  }
  return s;
}

// Workgroup = (kv head g, key item, walk chunk). The walk of a key item lists the query tiles whose
// rows may see one of its 128 keys: the response tiles from the one holding k0, then the tiles of
// the block region with a block whose anchor lies past k0 or whose own rows meet the keys. A
// workgroup takes kWalkChunk consecutive tiles of that walk and stores its partial dK, dV (fp32) in
// its chunk's slab, with a flag saying whether the chunk had any tile; the finish pass sums the
// flagged partials (a fixed order: no atomics, deterministic).
__global__ __launch_bounds__(kKThreads, 1) void train_kv_kernel(const TrainArgs a, float *slab_k, float *slab_v,
                                                                int32_t *flags) {
  __shared__ __attribute__((aligned(1024))) KStage stage[kStages];
  __shared__ int anc[kMaxAnchors];
  __shared__ short list[kMaxList];
  __shared__ int sh_cnt[kKThreads / 64];
  __shared__ __attribute__((aligned(16))) int sg_lim[kKThreads / 64][kQTRows];
  __shared__ __attribute__((aligned(16))) int sg_blo[kKThreads / 64][kQTRows];
  __shared__ __attribute__((aligned(16))) int sg_bhi[kKThreads / 64][kQTRows];
  const int w = blockIdx.x;
  const int g = w % a.Hkv;
  const int rest = w / a.Hkv;
  const int chunk = rest / a.n_kitems, item = rest % a.n_kitems;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5;
  const int TP = kQTRows / a.G;  // positions per query tile
  const int k0 = item * kKKeys, k1 = min(k0 + kKKeys, a.N);
  const int kw0 = k0 + wave * 32, kw1 = min(kw0 + 32, a.N);
  const int kj = kw0 + (lane & 31);  // this lane's key
  const bool kvalid = kj < a.N;
  for (int b = threadIdx.x; b < a.n_blocks; b += kKThreads) anc[b] = min(max(a.anchors[b], 0), a.L);
  __syncthreads();
  const int n_ptiles = (a.N + TP - 1) / TP;
  const int t_resp_end = a.L > 0 ? (a.L - 1) / TP + 1 : 0;  // tiles holding a response position
  const int t_c0 = k0 < a.L ? k0 / TP : t_resp_end;
  const int n_clean = t_resp_end - t_c0;
  int n_list = 0;
  for (int base = t_resp_end; base < n_ptiles; base += kKThreads) {
    const int t = base + threadIdx.x;
    bool need = false;
    if (t < n_ptiles) {
      const int p0 = t * TP, p1 = min(p0 + TP, a.N);
      const int b0 = (p0 - a.L) / a.B, b1 = (p1 - 1 - a.L) / a.B;
      for (int b = b0; b <= b1; ++b) {
        const int lo = a.L + b * a.B;
        need |= anc[b] > k0 || (lo < k1 && lo + a.B > k0);
      }
    }
    const unsigned long long m = __ballot(need);
    if (lane == 0) sh_cnt[wave] = __popcll(m);
    __syncthreads();
    int before = n_list, total = n_list;
    for (int v = 0; v < kKThreads / 64; ++v) {
      if (v < wave) before += sh_cnt[v];
      total += sh_cnt[v];
    }
    if (need) {
      const int idx = before + __popcll(m & ((1ull << lane) - 1ull));
      if (idx < kMaxList) list[idx] = static_cast<short>(t - t_resp_end);
    }
    n_list = total;
    __syncthreads();
  }
  n_list = min(n_list, kMaxList);
  const int j0 = chunk * kWalkChunk;
  const int n_tiles = min(n_clean + n_list, j0 + kWalkChunk) - j0;
  const size_t flag = (static_cast<size_t>(chunk) * a.n_kitems + item) * a.Hkv + g;
  if (threadIdx.x == 0) flags[flag] = n_tiles > 0 ? 1 : 0;
  if (n_tiles <= 0) return;  // workgroup-uniform
  auto tile_pos0 = [&](int j) __attribute__((always_inline)) {
    return (j < n_clean ? t_c0 + j : t_resp_end + list[j - n_clean]) * TP;
  };
  // copy geometry: LDS row r of a tile is query row (position p0 + r / G, head g*G + r % G)
  const uint32_t hrow = static_cast<uint32_t>(a.Hq) * kTD * 2;  // bytes per position
  uint32_t voff[kKvNI];
#pragma unroll
  for (int i = 0; i < kKvNI; ++i) {
    const int r = (wave * kKvNI + i) * 4 + lane / 16;
    voff[i] = static_cast<uint32_t>(r / a.G) * hrow + static_cast<uint32_t>(r % a.G) * kTD * 2 +
              (static_cast<uint32_t>((lane % 16) ^ swz<kTD>(r)) << 4);
  }
  const uint32_t toff = static_cast<uint32_t>(lane / a.G) * a.Hq * 4 + static_cast<uint32_t>(lane % a.G) * 4;
  const size_t hb = static_cast<size_t>(g) * a.G * kTD * 2;
  const int qrange = static_cast<int>(static_cast<size_t>(a.N) * hrow - hb);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.q) + hb), 0, qrange, kBufWord3);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.dout) + hb), 0, qrange, kBufWord3);
  const size_t tb = static_cast<size_t>(g) * a.G * 4;
  const int trange = static_cast<int>(static_cast<size_t>(a.N) * a.Hq * 4 - tb);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char *>(a.lse) + tb, 0, trange, kBufWord3);
  const __amdgpu_buffer_rsrc_t ers =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char *>(a.delta) + tb, 0, trange, kBufWord3);
  auto issue = [&](int s, int j) __attribute__((always_inline)) {
    // the tile offset goes into the lane offsets, which the buffers' range checks cover: rows past N
    // read as zero
    const int p0 = __builtin_amdgcn_readfirstlane(tile_pos0(j0 + j));  // uniform (the list is in LDS)
    const uint32_t qo = static_cast<uint32_t>(p0) * hrow;
#pragma unroll
    for (int i = 0; i < kKvNI; ++i) {
      kv_dma16(qrs, kv_dst(stage[s].q, i), voff[i] + qo, 0);
      kv_dma16(drs, kv_dst(stage[s].d, i), voff[i] + qo, 0);
    }
    const uint32_t to = toff + static_cast<uint32_t>(p0) * a.Hq * 4;
    kv_dma4(lrs, lds_addr(&stage[s].lse[wave][0]), to, 0);
    kv_dma4(ers, lds_addr(&stage[s].dlt[wave][0]), to, 0);
  };
  // K, V of this lane's key as B operands (rows past N read as zero)
  bf16x8 kf[kTD / 16], vf[kTD / 16];
  auto load_kv = [&]() __attribute__((always_inline)) {
    const size_t krow = (static_cast<size_t>(kvalid ? kj : 0) * a.Hkv + g) * kTD;
    const __bf16 *kr = static_cast<const __bf16 *>(a.k) + krow;
    const __bf16 *vr = static_cast<const __bf16 *>(a.v) + krow;
#pragma unroll
    for (int kk = 0; kk < kTD / 16; ++kk) {
      kf[kk] = kvalid ? *reinterpret_cast<const bf16x8 *>(kr + kk * 16 + hh * 8) : bf16x8{};
      vf[kk] = kvalid ? *reinterpret_cast<const bf16x8 *>(vr + kk * 16 + hh * 8) : bf16x8{};
    }
    __builtin_amdgcn_s_waitcnt(0);
  };
  f32x16 dv_acc[kTD / 32], dk_acc[kTD / 32];
#pragma unroll
  for (int b = 0; b < kTD / 32; ++b) dv_acc[b] = dk_acc[b] = f32x16{};
  const FragAddr<kTD> fa = frag_addr<kTD>();
  const float c = a.c;
  using TT = DmaTile<kTD>;
  auto compute = [&](const KStage &S, int j) __attribute__((always_inline)) {
    // this tile's row segments (lane l: row l), and how the wavefront's keys meet them
    const int p0 = tile_pos0(j0 + j);
    const RowSeg sg = row_seg_lds(a, anc, p0 + lane / a.G);
    sg_lim[wave][lane] = sg.lim;
    sg_blo[wave][lane] = sg.blo;
    sg_bhi[wave][lane] = sg.bhi;
    const bool meets = sg.lim > kw0 || (sg.blo < kw1 && sg.bhi > kw0);
    if (!__ballot(meets)) return;  // no row sees a key of this wavefront
    const bool all = kw1 == kw0 + 32 && !__ballot(sg.lim < kw1);  // every row sees every key
    const float *lse = S.lse[wave];
    const float *dlt = S.dlt[wave];
    const int *tl = sg_lim[wave], *tlo = sg_blo[wave], *thi = sg_bhi[wave];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // the lane's 16 rows of this half are 4 runs of 4 consecutive rows (8i + 4hh + 32mb ..):
      // their tables come in as 16-byte reads, issued ahead of the matrix work
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l4[i] = *reinterpret_cast<const f32x4 *>(lse + 32 * mb + 8 * i + 4 * hh);
        d4[i] = *reinterpret_cast<const f32x4 *>(dlt + 32 * mb + 8 * i + 4 * hh);
      }
      // one wavefront per SIMD: the fragment reads are scheduled two steps ahead of their MFMAs
      // (scheduling groups), so the LDS latency hides behind the matrix work
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < kTD / 16; ++kk) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(S.q + fa.kof(kk) + 32 * mb * TT::RB);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
        const bf16x8 da = *reinterpret_cast<const bf16x8 *>(S.d + fa.kof(kk) + 32 * mb * TT::RB);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[kk], dp, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int kk = 0; kk < kTD / 16 - 2; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
      __builtin_amdgcn_sched_barrier(0);
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l4[r >> 2][r & 3] * kLog2eF));
      if (!all) {  // wavefront-uniform: a tile that cuts through the wavefront's keys
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row0 = 32 * mb + 8 * i + 4 * hh;
          const i32x4 lim = *reinterpret_cast<const i32x4 *>(tl + row0);
          const i32x4 lo = *reinterpret_cast<const i32x4 *>(tlo + row0);
          const i32x4 hi = *reinterpret_cast<const i32x4 *>(thi + row0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int vis = static_cast<int>(kvalid) &
                            (static_cast<int>(kj < lim[e]) | (static_cast<int>(kj >= lo[e]) & static_cast<int>(kj < hi[e])));
            pr[4 * i + e] = vis ? pr[4 * i + e] : 0.f;
          }
        }
      }
      bf16x8 pb[2], db[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * t2 + i;
          pb[t2][i] = static_cast<__bf16>(pr[r]);
          db[t2][i] = static_cast<__bf16>(pr[r] * (dp[r] - d4[r >> 2][r & 3]));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int t = 2 * mb + t2;
#pragma unroll
        for (int b = 0; b < kTD / 32; ++b) {
          const v4i16 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, S.d + fa.vlof(b) + 16 * t * TT::RB));
          const v4i16 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, S.d + fa.vhif(b) + 16 * t * TT::RB));
          const v4i16 d2[2] = {dlo, dhi};
          dv_acc[b] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(d2), pb[t2], dv_acc[b], 0, 0, 0);
          const v4i16 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, S.q + fa.vlof(b) + 16 * t * TT::RB));
          const v4i16 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, S.q + fa.vhif(b) + 16 * t * TT::RB));
          const v4i16 q2[2] = {qlo, qhi};
          dk_acc[b] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(q2), db[t2], dk_acc[b], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 2);  // reads of the first two (t, b) steps
#pragma unroll
      for (int i = 0; i < 2 * kTD / 32 - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // four-stage ring: tile j is copied three tiles ahead into stage j % 4
  issue(0, 0);
  if (n_tiles > 1) issue(1, 1);
  if (n_tiles > 2) issue(2, 2);
  load_kv();  // its full wait covers the copies issued so far
  barrier_keep_copies();
  auto wait_next = [&](int j) __attribute__((always_inline)) {
    const int later = n_tiles - j - 2;
    if (later >= 2)
      wait_vm<2 * kKvOps>();
    else if (later == 1)
      wait_vm<kKvOps>();
    else
      wait_vm<0>();
    barrier_keep_copies();
  };
  for (int j = 0; j < n_tiles; j += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      if (j + u < n_tiles) {
        if (j + u + 3 < n_tiles) issue((u + 3) % kStages, j + u + 3);
        compute(stage[u], j + u);
        wait_next(j + u);
      }
    }
  }
  if (!kvalid) return;
  const size_t orow = (static_cast<size_t>(chunk) * a.N * a.Hkv + static_cast<size_t>(kj) * a.Hkv + g) * kTD;
#pragma unroll
  for (int b = 0; b < kTD / 32; ++b)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = b * 32 + 8 * r4 + 4 * hh;
      f32x4 k4, v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = dk_acc[b][4 * r4 + e] * a.scale;
        v4[e] = dv_acc[b][4 * r4 + e];
      }
      *reinterpret_cast<f32x4 *>(slab_k + orow + d0) = k4;
      *reinterpret_cast<f32x4 *>(slab_v + orow + d0) = v4;
    }
}

// dk, dv (bf16): the sum of the flagged chunk partials of each key, in chunk order. Every key has at
// least chunk 0 (its own row sees it).
__global__ __launch_bounds__(256) void train_kv_finish_kernel(const TrainArgs a, const float *slab_k,
                                                              const float *slab_v, const int32_t *flags, int n_chunks,
                                                              __bf16 *dk, __bf16 *dv) {
  const size_t per_chunk = static_cast<size_t>(a.N) * a.Hkv * kTD;
  const size_t n8 = per_chunk / 8;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n8; i += static_cast<size_t>(gridDim.x) * 256) {
    const size_t e = i * 8;
    const int row = static_cast<int>(e / kTD);  // key * Hkv + g
    const int key = row / a.Hkv, g = row % a.Hkv;
    const int item = key / kKKeys;
    f32x4 ka = {}, kb = {}, va = {}, vb = {};
    for (int c = 0; c < n_chunks; ++c) {
      if (!flags[(static_cast<size_t>(c) * a.n_kitems + item) * a.Hkv + g]) continue;
      const f32x4 *k4 = reinterpret_cast<const f32x4 *>(slab_k + c * per_chunk + e);
      const f32x4 *v4 = reinterpret_cast<const f32x4 *>(slab_v + c * per_chunk + e);
      ka += k4[0];
      kb += k4[1];
      va += v4[0];
      vb += v4[1];
    }
    u32x4 ko, vo;
    ko[0] = pack_bf16x2(ka[0], ka[1]);
    ko[1] = pack_bf16x2(ka[2], ka[3]);
    ko[2] = pack_bf16x2(kb[0], kb[1]);
    ko[3] = pack_bf16x2(kb[2], kb[3]);
    vo[0] = pack_bf16x2(va[0], va[1]);
    vo[1] = pack_bf16x2(va[2], va[3]);
    vo[2] = pack_bf16x2(vb[0], vb[1]);
    vo[3] = pack_bf16x2(vb[2], vb[3]);
    reinterpret_cast<u32x4 *>(dk)[i] = ko;
    reinterpret_cast<u32x4 *>(dv)[i] = vo;
  }
}

struct TrainShape {
  int N, G, n_qitems, n_kitems;
};

int check_train(d3d_dtype dtype, int L, int n_blocks, int B, int Hq, int Hkv, int head_dim, TrainShape *sh) {
  if (dtype != D3D_BF16 || head_dim != kTD) return D3D_EUNSUPPORTED;
  if (L < 0 || n_blocks < 0 || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return D3D_EINVAL;
  const int G = Hq / Hkv;
  if (32 % G != 0 || n_blocks > kMaxAnchors) return D3D_EUNSUPPORTED;
  if ((static_cast<long long>(n_blocks) * B + kQTRows / G) / (kQTRows / G) + 1 > kMaxList) return D3D_EUNSUPPORTED;
  const long long N = static_cast<long long>(L) + static_cast<long long>(n_blocks) * B;
  if (N < 1) return D3D_EINVAL;
  if (N >= (1ll << 31) || Hq >= (1 << 16) || N * Hq * kTD * 2 >= (1ll << 31)) return D3D_EUNSUPPORTED;  // 32-bit buffer offsets
  sh->N = static_cast<int>(N);
  sh->G = G;
  sh->n_qitems = static_cast<int>((N + kQRows / G - 1) / (kQRows / G));
  sh->n_kitems = static_cast<int>((N + kKKeys - 1) / kKKeys);
  return D3D_OK;
}

TrainArgs train_args(const TrainShape &sh, const void *q, const void *k, const void *v, const int32_t *anchors, int L,
                     int n_blocks, int B, int Hq, int Hkv, float scale) {
  TrainArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.anchors = anchors;
  a.L = L;
  a.n_blocks = n_blocks;
  a.B = B;
  a.N = sh.N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = sh.G;
  a.n_qitems = sh.n_qitems;
  a.n_kitems = sh.n_kitems;
  a.scale = scale;
  a.c = scale * kLog2eF;
  return a;
}

}  // namespace
}  // namespace d3d

namespace d3d {
namespace {
struct TrainWs {
  size_t delta, flags, slab_k, slab_v, total;
  int n_chunks;
};
TrainWs train_ws(long long N, int n_kitems, int G, int Hq, int Hkv) {
  const int TP = kQTRows / G;
  const long long n_ptiles = (N + TP - 1) / TP;
  TrainWs w;
  w.n_chunks = static_cast<int>((n_ptiles + kWalkChunk - 1) / kWalkChunk);
  const size_t slab = static_cast<size_t>(w.n_chunks) * N * Hkv * kTD * sizeof(float);
  w.delta = 0;
  w.flags = align_up(static_cast<size_t>(N) * Hq * sizeof(float), 256);
  w.slab_k = align_up(w.flags + static_cast<size_t>(w.n_chunks) * n_kitems * Hkv * sizeof(int32_t), 256);
  w.slab_v = align_up(w.slab_k + slab, 256);
  w.total = align_up(w.slab_v + slab, 256);
  return w;
}
}  // namespace
}  // namespace d3d

extern "C" size_t train_attn_workspace(int L, int n_blocks, int block_size, int n_heads_q, int n_heads_kv) {
  using namespace d3d;
  TrainShape sh;
  if (check_train(D3D_BF16, L, n_blocks, block_size, n_heads_q, n_heads_kv, kTD, &sh) != D3D_OK) return 0;
  return train_ws(sh.N, sh.n_kitems, sh.G, n_heads_q, n_heads_kv).total;
}

extern "C" int train_attn_fwd(d3d_dtype dtype, const void *q, const void *k, const void *v, const int32_t *anchors,
                              int L, int n_blocks, int block_size, int n_heads_q, int n_heads_kv, int head_dim,
                              float scale, void *out, float *lse, hipStream_t stream) {
  using namespace d3d;
  TrainShape sh;
  const int st = check_train(dtype, L, n_blocks, block_size, n_heads_q, n_heads_kv, head_dim, &sh);
  if (st != D3D_OK) return st;
  if (!q || !k || !v || !out || !lse || (n_blocks > 0 && !anchors) || !(scale > 0.f)) return D3D_EINVAL;
  TrainArgs a = train_args(sh, q, k, v, anchors, L, n_blocks, block_size, n_heads_q, n_heads_kv, scale);
  a.out = out;
  a.lse = lse;
  train_q_kernel<false><<<sh.n_qitems * n_heads_kv, kBfThreads, 0, stream>>>(a);
  return launch_status();
}

extern "C" int train_attn_bwd(d3d_dtype dtype, const void *q, const void *k, const void *v, const void *out,
                              const void *dout, const float *lse, const int32_t *anchors, int L, int n_blocks,
                              int block_size, int n_heads_q, int n_heads_kv, int head_dim, float scale, void *dq,
                              void *dk, void *dv, void *ws, size_t ws_bytes, hipStream_t stream) {
  using namespace d3d;
  TrainShape sh;
  const int st = check_train(dtype, L, n_blocks, block_size, n_heads_q, n_heads_kv, head_dim, &sh);
  if (st != D3D_OK) return st;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || (n_blocks > 0 && !anchors) || !(scale > 0.f))
    return D3D_EINVAL;
  const TrainWs tw = train_ws(sh.N, sh.n_kitems, sh.G, n_heads_q, n_heads_kv);
  if (!ws || ws_bytes < tw.total) return D3D_EWORKSPACE;
  TrainArgs a = train_args(sh, q, k, v, anchors, L, n_blocks, block_size, n_heads_q, n_heads_kv, scale);
  a.o = out;
  a.dout = dout;
  a.lse = const_cast<float *>(lse);
  char *w = static_cast<char *>(ws);
  a.delta = reinterpret_cast<float *>(w + tw.delta);
  int32_t *flags = reinterpret_cast<int32_t *>(w + tw.flags);
  float *slab_k = reinterpret_cast<float *>(w + tw.slab_k);
  float *slab_v = reinterpret_cast<float *>(w + tw.slab_v);
  a.out = dq;
  a.dk = dk;
  a.dv = dv;
  train_q_kernel<true><<<sh.n_qitems * n_heads_kv, kBfThreads, 0, stream>>>(a);
  train_kv_kernel<<<sh.n_kitems * n_heads_kv * tw.n_chunks, kKThreads, 0, stream>>>(a, slab_k, slab_v, flags);
  const size_t n8 = static_cast<size_t>(sh.N) * n_heads_kv * kTD / 8;
  const int blocks = static_cast<int>(std::min<size_t>((n8 + 255) / 256, 4096));
  train_kv_finish_kernel<<<blocks, 256, 0, stream>>>(a, slab_k, slab_v, flags, tw.n_chunks, static_cast<__bf16 *>(dk),
                                                     static_cast<__bf16 *>(dv));
  return launch_status();
}
