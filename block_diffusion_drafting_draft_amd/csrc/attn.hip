// Packed draft attention on gfx950 (one drafter attention layer of the packed async forward).
//
// What is computed ([D3D] 核心方法: the prefix is shared and causally encoded, attention is
// bidirectional inside a block; 方法步骤详情 step 4: one packed forward drafts every branch):
// each packed query row attends to the whole request prefix, to the first r_b rows of its
// request's current block (the accepted slice its branch assumes), and to its own block (all rows,
// or rows up to itself for a causal block), with grouped-query heads.
//
// Design:
//  * A bf16 workgroup (8 wavefronts, one workgroup per compute unit) owns 256 query-head rows that
//    share one key/value head: with group size G = H_q / H_kv, 256/G queries x G heads. Each
//    wavefront owns 32 rows; two wavefronts share a SIMD. (fp32: 4 wavefronts, 128 rows.)
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: Q stays in registers (the B operand)
//    for the whole key walk, K and V come from LDS. The S^T accumulator leaves every lane holding one
//    query column, so the softmax row max / sum are per-lane scalars (one cross-half exchange), and
//    the accumulator registers are already the B operand of the PV product.
//  * bf16 tiles of 64 keys are copied global -> LDS by the LDS-DMA loads (global_load_lds, 16 bytes a
//    lane, 1 KB a wavefront instruction): no register staging and no LDS store instructions. Rows are
//    kept in natural [key][d] order with an XOR swizzle of the 16-byte chunks that keeps both read
//    patterns below conflict-free. K fragments are plain 16-byte reads; V^T fragments come from the
//    transposing LDS read ds_read_b64_tr_b16, which hands each lane 4 consecutive keys of one column
//    -- exactly the key order the S^T accumulator holds, so no data is permuted anywhere.
//  * Prefix phase: a four-stage ring of LDS tiles over the request's prefix (three copies in flight
//    ahead of the tile being computed, one barrier per tile), no mask except the ragged end; every
//    packed query of the request shares this one walk.
//  * In-pack tail: the rows of the request's current block and of the blocks the tile's queries
//    belong to are gathered into 64-key tiles with a per-(row, key) visibility test from the block
//    descriptors.
//  * Split-KV: a request's prefix is cut into equal key ranges; each (request, split, kv head) is a
//    "group" whose tiles share one key/value slice. Groups are dealt round-robin to the 8 XCDs so that
//    all tiles of a group run on one XCD (its L2 serves the slice to all of them), longest first.
//    Split partials (unnormalised O, running max, sum) are merged by a second kernel.
//  * fp32 inputs take a register-staged variant of the same walk on v_mfma_f32_32x32x2f32.
#include <float.h>
#include <math.h>

#include <algorithm>
#include <vector>

#include "attn_tiles.h"
#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kThreads = 256;  // fp32 kernel and the split combine
constexpr int kRows = 128;     // query-head rows per fp32 work item
constexpr int kBfRows = 256;   // query-head rows per bf16 work item
constexpr int kMinSplit = 256;
constexpr int kMaxSplits = 32;

struct ReqInfo {
  int32_t q_begin;      // global packed row of the request's first query
  int32_t n_q;          // packed query rows of the request
  int32_t prefix;       // prefix length
  int32_t split_len;    // keys per split after the first (multiple of 64), 0 when the prefix is empty
  int32_t split0_len;   // keys of the first split, which also walks the in-pack tail
  int32_t n_splits;
  int32_t group_begin;  // first (split, kv head) group of the request in dispatch order
  int32_t block_begin;  // global index of the request's current block
  int32_t req;          // request index (page-table row / contiguous cache slot)
  int32_t part_begin;   // first split-partial slot, when n_splits > 1
  int32_t comb_begin;   // first combine row, when n_splits > 1
};

struct AttnArgs {
  const void *q;
  const void *k_new;
  const void *v_new;
  const void *k_cache;
  const void *v_cache;
  const int32_t *page_table;
  const d3d_block_desc *descs;
  void *out;
  float *part_o;   // [slots][D] unnormalised split outputs
  float *part_ml;  // [slots][2] (running max in scaled log2 units, sum)
  int page_size, max_pages, num_pages, kv_stride;
  int B, Hq, Hkv, G, Qt;
  float scale_log2;
  int n_entries, n_groups, t_max, comb_rows;
  int n_new;  // packed rows of k_new / v_new (all requests)
  ReqInfo req[D3D_ATTN_MAX_REQ];
};

template <typename T>
struct Cfg;
template <>
struct Cfg<__bf16> {
  static constexpr bool kBf16 = true;
};
template <>
struct Cfg<float> {
  static constexpr bool kBf16 = false;
};


// ------------------------------------------------------------------------------------------------
// work item, lane rows, softmax, output (shared by both element types)
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ int find_entry(const AttnArgs &a, int gamma) {
  int e = 0;
  while (e + 1 < a.n_entries && a.req[e + 1].group_begin <= gamma) ++e;
  return e;
}

struct Item {
  ReqInfo R;
  int split, g, tile, k0, k1;
};

// XCD-aware mapping of the workgroup id: workgroup w runs on XCD w % 8; consecutive groups are
// dealt round-robin to the XCDs and every tile of one group stays on the same XCD.
__device__ __forceinline__ bool decode_item(const AttnArgs &a, Item &it) {
  const int w = blockIdx.x;
  const int x = w % kXcds, k = w / kXcds;
  const int j = k / a.t_max;
  it.tile = k - j * a.t_max;
  const int gamma = j * kXcds + x;
  if (gamma >= a.n_groups) return false;
  it.R = a.req[find_entry(a, gamma)];
  const int gl = gamma - it.R.group_begin;
  it.split = gl / a.Hkv;
  it.g = gl - it.split * a.Hkv;
  if (it.tile >= (it.R.n_q + a.Qt - 1) / a.Qt) return false;
  it.k0 = it.split == 0 ? 0 : it.R.split0_len + (it.split - 1) * it.R.split_len;
  it.k1 = min(it.R.prefix, it.split == 0 ? it.R.split0_len : it.k0 + it.R.split_len);
  return true;
}

struct LaneRow {
  int q_local, h, blk, pos, r;
  bool valid, causal;
};

// Query row `row` of the work item's G * Qt query-head rows: rows are query-major, the G heads of one
// query on consecutive rows (consecutive in memory too). An item with fewer than Qt queries -- a
// synchronous draft's few queries -- so fills its first wavefronts, and wavefronts without a valid
// row skip the tile work.
__device__ __forceinline__ LaneRow lane_row(const AttnArgs &a, const Item &it, int row) {
  const int qi = row / a.G, head_local = row - qi * a.G;
  LaneRow L;
  L.q_local = it.tile * a.Qt + qi;
  L.valid = L.q_local < it.R.n_q;
  L.h = it.g * a.G + head_local;
  L.blk = L.valid ? L.q_local / a.B : -1;
  L.pos = L.valid ? L.q_local - L.blk * a.B : 0;
  L.r = 0;
  L.causal = false;
  if (L.valid) {
    const d3d_block_desc dsc = a.descs[it.R.block_begin + L.blk];
    L.r = L.blk == 0 ? 0 : min(max(dsc.rej_pos, 0), a.B);
    L.causal = (dsc.flags & D3D_BLOCK_CAUSAL) != 0;
  }
  return L;
}

// The output row of query-head row `row` only (no descriptor read): what the final write needs.
__device__ __forceinline__ LaneRow out_row(const AttnArgs &a, const Item &it, int row) {
  const int qi = row / a.G, head_local = row - qi * a.G;
  LaneRow L;
  L.q_local = it.tile * a.Qt + qi;
  L.valid = L.q_local < it.R.n_q;
  L.h = it.g * a.G + head_local;
  L.blk = -1;
  L.pos = 0;
  L.r = 0;
  L.causal = false;
  return L;
}

// Per-wavefront online-softmax state for 32 query columns.
template <int D>
struct RowState {
  f32x16 o[D / 32];
  float m;  // running max of scale*log2(e)*s
  float l;  // this lane's half of the running sum
};

// Mask, online-softmax update of (m, l, O) and S -> P in place. The lane holds the keys
// kappa = mb*32 + 8*(r/4) + 4*hh + r%4 of its query column.
template <int D, typename VIS>
__device__ __forceinline__ void softmax_update(f32x16 (&s)[2], RowState<D> &st, float c, bool need_mask,
                                               VIS visible) {
  const int hh = (threadIdx.x & 63) >> 5;
  if (need_mask) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = mb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        s[mb][r] = visible(key) ? s[mb][r] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx * c);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  // The running max only moves for some lanes on some tiles; when it moves for no lane of the
  // wavefront the rescale factor is exactly 1 and the O rescale is skipped.
  if (__ballot(m_new > st.m)) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
    st.l *= alpha;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[b][r] *= alpha;
  }
  float psum = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][r], c, -m_use));
      s[mb][r] = p;
      psum += p;
    }
  st.l += psum;
  st.m = m_new;
}

// Final write: the normalised output (single split) or the split partial (unnormalised O, m, l).
template <typename T, int D>
__device__ __forceinline__ void write_result(const AttnArgs &a, const Item &it, const LaneRow &L,
                                             const f32x16 (&o)[D / 32], float m, float l) {
  const int hh = (threadIdx.x & 63) >> 5;
  const float l_tot = l + __shfl_xor(l, 32);
  if (!L.valid) return;
  const ReqInfo &R = it.R;
  const size_t orow = static_cast<size_t>(R.q_begin + L.q_local) * a.Hq + L.h;
  if (R.n_splits == 1) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = b * 32 + 8 * r4 + 4 * hh;
        if constexpr (Cfg<T>::kBf16) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = static_cast<__bf16>(o[b][4 * r4 + e] * inv);
          *reinterpret_cast<bf16x4 *>(static_cast<T *>(a.out) + orow * D + d0) = v4;
        } else {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o[b][4 * r4 + e] * inv;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + orow * D + d0) = v4;
        }
      }
  } else {
    const size_t slot = static_cast<size_t>(R.part_begin) +
                        (static_cast<size_t>(it.split) * R.n_q + L.q_local) * a.Hq + L.h;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = b * 32 + 8 * r4 + 4 * hh;
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[b][4 * r4 + e];
        *reinterpret_cast<f32x4 *>(a.part_o + slot * D + d0) = v4;
      }
    if (hh == 0) {
      a.part_ml[slot * 2] = m;
      a.part_ml[slot * 2 + 1] = l_tot;
    }
  }
}

// In-pack tail of a tile: the list of packed rows (relative to the request) its queries may see --
// the current block's B rows, then the rows of the tile's own blocks other than the current block.
struct TailList {
  int first, n;
};

__device__ __forceinline__ TailList tail_list(const AttnArgs &a, const Item &it) {
  const int tq0 = it.tile * a.Qt;
  const int tq1 = min(it.R.n_q, tq0 + a.Qt);
  const int bf = tq0 / a.B, bl = (tq1 - 1) / a.B;
  TailList t;
  t.first = max(bf, 1);
  t.n = a.B + max(0, bl - t.first + 1) * a.B;
  return t;
}

// Fill the per-key tables of tail tile kt (threads 0..63): packed row, block and position of each
// list slot (-1 block for slots past the list).
__device__ __forceinline__ void tail_tables(const AttnArgs &a, const TailList &tl, int kt, int *sh_row,
                                            int *sh_blk, int *sh_pos) {
  if (threadIdx.x < kKeys) {
    const int kappa = kt + threadIdx.x;
    int rr = -1, blk = -1, pos = 0;
    if (kappa < tl.n) {
      rr = kappa < a.B ? kappa : tl.first * a.B + (kappa - a.B);
      blk = rr / a.B;
      pos = rr - blk * a.B;
    }
    sh_row[threadIdx.x] = rr;
    sh_blk[threadIdx.x] = blk;
    sh_pos[threadIdx.x] = pos;
  }
}

// Visibility of tail key `key` for this lane's query row, evaluated without branches: the mask is
// applied per accumulator register under divergent lanes, and a select chain keeps every lane on one
// straight path (short-circuit branches here let the masked copy of S be lost on some lanes).
__device__ __forceinline__ bool tail_visible(const LaneRow &L, const int *sh_blk, const int *sh_pos, int key) {
  const int blk = sh_blk[key], pos = sh_pos[key];
  const int own = static_cast<int>(blk == L.blk) & (static_cast<int>(!L.causal) | static_cast<int>(pos <= L.pos));
  const int cur = static_cast<int>(blk == 0) & static_cast<int>(pos < L.r);
  return (static_cast<int>(blk >= 0) & (own | cur)) != 0;
}

enum KvMode { kContig = 0, kPagedWave = 1, kPagedLane = 2 };

template <int D, int KV>
__global__ __launch_bounds__(kBfThreads, 2) void attn_kernel_bf16(const AttnArgs a) {
  using TT = DmaTile<D>;
  // one LDS object per stage and operand, so that the DMA into one stage is provably independent of
  // the reads of the others (no conservative wait between them)
  // (K tile then V tile per stage: four objects, few enough for the compiler to track each stage's
  // copies separately)
  __shared__ __attribute__((aligned(1024))) char lds_s0[2 * TT::BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s1[2 * TT::BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s2[2 * TT::BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_s3[2 * TT::BYTES];
  char *const lds_k0 = lds_s0, *const lds_v0 = lds_s0 + TT::BYTES;
  char *const lds_k1 = lds_s1, *const lds_v1 = lds_s1 + TT::BYTES;
  char *const lds_k2 = lds_s2, *const lds_v2 = lds_s2 + TT::BYTES;
  char *const lds_k3 = lds_s3, *const lds_v3 = lds_s3 + TT::BYTES;
  __shared__ int sh_row[kKeys];
  __shared__ int sh_blk[kKeys];
  __shared__ int sh_pos[kKeys];
  Item it;
  if (!decode_item(a, it)) return;
  const ReqInfo &R = it.R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5;
  // this lane's query row (recomputed after the walk instead of held in registers)
  auto row_of = [&]() __attribute__((always_inline)) { return lane_row(a, it, wave * 32 + (lane & 31)); };
  // a wavefront without a valid row (an item with fewer queries than Qt) only copies and waits
  const bool live = __ballot(out_row(a, it, wave * 32 + (lane & 31)).valid) != 0;
  bf16x8 qf[D / 16];
  // Q fragments of this lane's row. They are loaded after the first tile copies are issued, and one
  // full wait (which the compiler sees: otherwise it keeps Q pending into the loop and waits there
  // for every copy in flight) then covers both, so the two latencies overlap.
  auto load_q = [&]() __attribute__((always_inline)) {
    const LaneRow L = row_of();
    const __bf16 *qrow =
        static_cast<const __bf16 *>(a.q) + (static_cast<size_t>(R.q_begin + L.q_local) * a.Hq + L.h) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = L.valid ? *reinterpret_cast<const bf16x8 *>(qrow + kk * 16 + hh * 8) : bf16x8{};
    __builtin_amdgcn_s_waitcnt(0);
  };
  Rows1<D> st;
#pragma unroll
  for (int b = 0; b < D / 32; ++b) st.o[b] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;
  const FragAddr<D> fa = frag_addr<D>();
  const size_t row_bytes = static_cast<size_t>(a.Hkv) * D * 2;  // bytes between consecutive tokens

  // ---- prefix phase: 64-key tiles through a four-stage ring, one barrier per tile ----
  if (it.k1 > it.k0) {
    const int k1 = it.k1;
    const char *kc = static_cast<const char *>(a.k_cache);
    const char *vc = static_cast<const char *>(a.v_cache);
    // Paged caches: with page_size a multiple of RPI every DMA instruction reads RPI consecutive
    // tokens of one page, so its page id is wave-uniform (a scalar load, one tile ahead) and the
    // address is a scalar page base plus a 32-bit lane offset. Other page sizes take a per-lane path.
    constexpr bool PAGED = KV != kContig;
    constexpr bool page_uniform = KV == kPagedWave;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int pg[TT::NI];  // page ids of the tile whose DMA is issued next
    auto load_pages = [&](int kt) __attribute__((always_inline)) {
      if constexpr (PAGED) {
        const int32_t *pt = a.page_table + static_cast<size_t>(R.req) * a.max_pages;
        if constexpr (page_uniform) {
          // the page table is read-only during the kernel: constant-space loads with a wave-uniform
          // index become scalar loads
          const __attribute__((address_space(4))) int32_t *ptc = (const __attribute__((address_space(4))) int32_t *)pt;
#pragma unroll
          for (int i = 0; i < TT::NI; ++i)
            pg[i] = ptc[min(kt + (wave_u * TT::NI + i) * TT::RPI, k1 - 1) / a.page_size];
        } else {
#pragma unroll
          for (int i = 0; i < TT::NI; ++i) pg[i] = pt[min(kt + dma_row<D>(i), k1 - 1) / a.page_size];
        }
      }
    };
    // contiguous cache: this request's key / value rows of head g as buffers; rows of the last tile
    // past the split's end are masked, and past the request's rows they read as zero
    uint32_t off[TT::NI];  // byte offsets of this lane's 16-byte pieces in a tile
    __amdgpu_buffer_rsrc_t krs, vrs;
    if constexpr (!PAGED) {
#pragma unroll
      for (int i = 0; i < TT::NI; ++i) off[i] = static_cast<uint32_t>(dma_row<D>(i) * row_bytes) + dma_chunk<D>(i);
      const size_t base = (static_cast<size_t>(R.req) * a.kv_stride * a.Hkv + it.g) * D * 2;
      const int range = static_cast<int>(static_cast<size_t>(a.kv_stride) * row_bytes - static_cast<size_t>(it.g) * D * 2);
      krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kc + base), 0, range, kBufWord3);
      vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vc + base), 0, range, kBufWord3);
    }
    // DMA of the K and V tile at prefix token kt into kd / vd
    auto issue = [&](char *kd, char *vd, int kt) __attribute__((always_inline)) {
      if constexpr (PAGED) {
        const size_t page_bytes = static_cast<size_t>(a.page_size) * row_bytes;
        if constexpr (page_uniform) {
          const int lr = (lane & 63) / TT::CH;  // row inside the instruction's RPI rows
#pragma unroll
          for (int i = 0; i < TT::NI; ++i) {
            const int jj0 = min(kt + (wave_u * TT::NI + i) * TT::RPI, k1 - 1);
            const int page = min(max(pg[i], 0), a.num_pages - 1);
            const int rip = min(jj0 % a.page_size + lr, a.page_size - 1);  // stays in the page; masked past k1
            const size_t pbase = static_cast<size_t>(page) * page_bytes + static_cast<size_t>(it.g) * D * 2;
            const uint32_t lo = static_cast<uint32_t>(rip * row_bytes) + dma_chunk<D>(i);
            dma16_s<D>(kc + pbase, lo, kd, i);
            dma16_s<D>(vc + pbase, lo, vd, i);
          }
        } else {
#pragma unroll
          for (int i = 0; i < TT::NI; ++i) {
            const int jj = min(kt + dma_row<D>(i), k1 - 1);
            const int page = min(max(pg[i], 0), a.num_pages - 1);
            const size_t o = ((static_cast<size_t>(page) * a.page_size + (jj % a.page_size)) * a.Hkv + it.g) * D * 2 +
                             dma_chunk<D>(i);
            dma16<D>(kc + o, kd, i);
            dma16<D>(vc + o, vd, i);
          }
        }
      } else {
        const uint32_t soff = static_cast<uint32_t>(kt * row_bytes);
#pragma unroll
        for (int i = 0; i < TT::NI; ++i) {
          dma16_buf<D>(krs, kd, i, off[i], soff);
          dma16_buf<D>(vrs, vd, i, off[i], soff);
        }
      }
    };
    // Full tiles in a loop unrolled over the four stages; the ragged last tile (if any) after it, so
    // that no tile variant joins the loop's accumulators. Step i prefetches tile i+3 into the stage
    // read at step i-1, computes tile i, then waits for its own copy of tile i+1 (the copies of
    // tiles i+2, i+3 may stay in flight) and for every wavefront.
    const int n_full = (k1 - it.k0) / kKeys;
    const int n_tiles = (k1 - it.k0 + kKeys - 1) / kKeys;
    auto wait_next = [&](int i) __attribute__((always_inline)) {
      const int later = n_tiles - i - 2;  // tiles issued after tile i+1 (at most two)
      if (later >= 2)
        wait_vm<4 * TT::NI>();
      else if (later == 1)
        wait_vm<2 * TT::NI>();
      else
        wait_vm<0>();
      barrier_keep_copies();
    };
    auto body = [&](const char *kcur, const char *vcur, char *kpre, char *vpre, int i) __attribute__((always_inline)) {
      if (i + 3 < n_tiles) {
        issue(kpre, vpre, it.k0 + (i + 3) * kKeys);
        if (i + 4 < n_tiles) load_pages(it.k0 + (i + 4) * kKeys);
      }
      if (live) tile1<D, false>(kcur, vcur, fa, qf, st, c, [](int) { return true; });
      wait_next(i);
    };
    load_pages(it.k0);
    issue(lds_k0, lds_v0, it.k0);
    if (n_tiles > 1) {
      load_pages(it.k0 + kKeys);
      issue(lds_k1, lds_v1, it.k0 + kKeys);
    }
    if (n_tiles > 2) {
      load_pages(it.k0 + 2 * kKeys);
      issue(lds_k2, lds_v2, it.k0 + 2 * kKeys);
    }
    if (n_tiles > 3) load_pages(it.k0 + 3 * kKeys);
    load_q();  // every copy issued so far has landed too
    barrier_keep_copies();
    for (int i = 0; i < n_full; i += kStages) {
      body(lds_k0, lds_v0, lds_k3, lds_v3, i);
      if (i + 1 < n_full) body(lds_k1, lds_v1, lds_k0, lds_v0, i + 1);
      if (i + 2 < n_full) body(lds_k2, lds_v2, lds_k1, lds_v1, i + 2);
      if (i + 3 < n_full) body(lds_k3, lds_v3, lds_k2, lds_v2, i + 3);
    }
    if (n_full < n_tiles) {  // ragged last tile: keys past the split's end are masked
      const int lim_hh = k1 - (it.k0 + n_full * kKeys) - 4 * hh;
      auto vis = [&](int kc) { return kc < lim_hh; };
      if (live) switch (n_full % kStages) {
        case 0: tile1<D, true>(lds_k0, lds_v0, fa, qf, st, c, vis); break;
        case 1: tile1<D, true>(lds_k1, lds_v1, fa, qf, st, c, vis); break;
        case 2: tile1<D, true>(lds_k2, lds_v2, fa, qf, st, c, vis); break;
        default: tile1<D, true>(lds_k3, lds_v3, fa, qf, st, c, vis); break;
      }
      __syncthreads();
    }
  } else {
    load_q();
  }

  // ---- in-pack tail (first split only) ----
  if (it.split == 0) {
    const LaneRow L = row_of();
    const TailList tl = tail_list(a, it);
    const size_t gb = static_cast<size_t>(it.g) * D * 2;
    const int range = static_cast<int>(static_cast<size_t>(a.n_new) * row_bytes - gb);
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.k_new) + gb), 0, range, kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.v_new) + gb), 0, range, kBufWord3);
    for (int kt = 0; kt < tl.n; kt += kKeys) {
      __syncthreads();
      tail_tables(a, tl, kt, sh_row, sh_blk, sh_pos);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TT::NI; ++i) {
        const int rr = max(sh_row[dma_row<D>(i)], 0);  // unused slots read row 0 of the request; masked
        const uint32_t o = static_cast<uint32_t>((R.q_begin + rr) * row_bytes) + dma_chunk<D>(i);
        dma16_buf<D>(krs, lds_k0, i, o, 0);
        dma16_buf<D>(vrs, lds_v0, i, o, 0);
      }
      wait_vm<0>();
      __syncthreads();
      if (live)
        tile1<D, true>(lds_k0, lds_v0, fa, qf, st, c,
                       [&](int kc) { return tail_visible(L, sh_blk + 4 * hh, sh_pos + 4 * hh, kc); });
    }
  }
  write_result<__bf16, D>(a, it, out_row(a, it, wave * 32 + (lane & 31)), st.o, st.m, st.l);
}

// ------------------------------------------------------------------------------------------------
// fp32: register-staged tiles, padded LDS rows, v_mfma_f32_32x32x2f32
// ------------------------------------------------------------------------------------------------
template <int D>
struct F32Tile {
  static constexpr int KS = D + 2;  // padded K row (floats): 2-way-free bank pattern for the reads
  static constexpr int VS = D + 8;  // padded V row (floats)
  static constexpr int CH = D / 4;  // 16-byte chunks per row
  static constexpr int NK = kKeys * CH / kThreads;
};

template <int D, typename RF>
__device__ __forceinline__ void f32_load(u32x4 (&k)[F32Tile<D>::NK], u32x4 (&v)[F32Tile<D>::NK], RF key_row,
                                         RF val_row) {
  using TT = F32Tile<D>;
#pragma unroll
  for (int i = 0; i < TT::NK; ++i) {
    const int cidx = threadIdx.x + kThreads * i;
    const int key = cidx / TT::CH, part = cidx % TT::CH;
    k[i] = *reinterpret_cast<const u32x4 *>(key_row(key) + part * 4);
    v[i] = *reinterpret_cast<const u32x4 *>(val_row(key) + part * 4);
  }
}

template <int D>
__device__ __forceinline__ void f32_store(const u32x4 (&k)[F32Tile<D>::NK], const u32x4 (&v)[F32Tile<D>::NK],
                                          float *ks, float *vs) {
  using TT = F32Tile<D>;
#pragma unroll
  for (int i = 0; i < TT::NK; ++i) {
    const int cidx = threadIdx.x + kThreads * i;
    const int key = cidx / TT::CH, part = cidx % TT::CH;
#pragma unroll
    for (int e = 0; e < 4; ++e) ks[key * TT::KS + part * 4 + e] = __uint_as_float(k[i][e]);
    *reinterpret_cast<u32x4 *>(vs + key * TT::VS + part * 4) = v[i];
  }
}

template <int D, typename VIS>
__device__ __forceinline__ void tile_step_f32(const float *ks, const float *vs, const float (&qf)[D / 2],
                                              RowState<D> &st, float c, bool need_mask, VIS visible) {
  using TT = F32Tile<D>;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  f32x16 s[2] = {};
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(mb * 32 + col) * TT::KS + 2 * kk + hh], qf[kk], s[mb], 0, 0, 0);
  softmax_update<D>(s, st, c, need_mask, visible);
  // k-step (mb, r): lane half hh supplies key mb*32 + 8(r/4) + 4hh + r%4 -- the key its own
  // accumulator register r holds
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = mb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
        st.o[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * TT::VS + b * 32 + col], s[mb][r], st.o[b], 0, 0, 0);
    }
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel_f32(const AttnArgs a) {
  using TT = F32Tile<D>;
  __shared__ __attribute__((aligned(16))) float ks[kKeys * TT::KS];
  __shared__ __attribute__((aligned(16))) float vs[kKeys * TT::VS];
  __shared__ int sh_row[kKeys];
  __shared__ int sh_blk[kKeys];
  __shared__ int sh_pos[kKeys];
  Item it;
  if (!decode_item(a, it)) return;
  const ReqInfo &R = it.R;
  const LaneRow L = lane_row(a, it, (threadIdx.x >> 6) * 32 + (threadIdx.x & 31));
  const int hh = (threadIdx.x & 63) >> 5;
  float qf[D / 2];
  {
    const float *qrow = static_cast<const float *>(a.q) + (static_cast<size_t>(R.q_begin + L.q_local) * a.Hq + L.h) * D;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qf[kk] = L.valid ? qrow[2 * kk + hh] : 0.f;
  }
  RowState<D> st;
#pragma unroll
  for (int b = 0; b < D / 32; ++b) st.o[b] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;
  u32x4 kr[TT::NK], vr[TT::NK];
  if (it.k1 > it.k0) {
    const size_t rs = static_cast<size_t>(a.Hkv) * D;
    const float *kc = static_cast<const float *>(a.k_cache);
    const float *vc = static_cast<const float *>(a.v_cache);
    const float *kb = kc + (static_cast<size_t>(R.req) * a.kv_stride * a.Hkv + it.g) * D;
    const float *vb = vc + (static_cast<size_t>(R.req) * a.kv_stride * a.Hkv + it.g) * D;
    const int k1 = it.k1;
    for (int kt = it.k0; kt < k1; kt += kKeys) {
      auto row_at = [&](const float *flat, const float *cache) {
        return [&, flat, cache](int key) -> const float * {
          const int jj = min(kt + key, k1 - 1);
          if (!PAGED) return flat + jj * rs;
          int page = a.page_table[static_cast<size_t>(R.req) * a.max_pages + jj / a.page_size];
          page = min(max(page, 0), a.num_pages - 1);
          return cache + ((static_cast<size_t>(page) * a.page_size + (jj % a.page_size)) * a.Hkv + it.g) * D;
        };
      };
      f32_load<D>(kr, vr, row_at(kb, kc), row_at(vb, vc));
      __syncthreads();
      f32_store<D>(kr, vr, ks, vs);
      __syncthreads();
      const int lim = k1 - kt;
      tile_step_f32<D>(ks, vs, qf, st, c, lim < kKeys, [&](int key) { return key < lim; });
    }
  }
  if (it.split == 0) {
    const TailList tl = tail_list(a, it);
    const float *kn = static_cast<const float *>(a.k_new);
    const float *vn = static_cast<const float *>(a.v_new);
    for (int kt = 0; kt < tl.n; kt += kKeys) {
      __syncthreads();
      tail_tables(a, tl, kt, sh_row, sh_blk, sh_pos);
      __syncthreads();
      auto src = [&](const float *base) {
        return [&, base](int r) -> const float * {
          return base + (static_cast<size_t>(R.q_begin + max(sh_row[r], 0)) * a.Hkv + it.g) * D;
        };
      };
      f32_load<D>(kr, vr, src(kn), src(vn));
      f32_store<D>(kr, vr, ks, vs);
      __syncthreads();
      tile_step_f32<D>(ks, vs, qf, st, c, true, [&](int key) { return tail_visible(L, sh_blk, sh_pos, key); });
    }
  }
  write_result<float, D>(a, it, L, st.o, st.m, st.l);
}

// Merge split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s. Each thread owns four
// consecutive elements of one row (16-byte loads); D/4 threads per row. MS bounds the split count
// (its load arrays are unrolled to MS): 8 keeps the kernel near 60 registers, so the whole grid of a
// 384-query pack is resident at once; 16 serves plans with more splits.
template <typename T, int D, int MS>
__global__ __launch_bounds__(kThreads) void combine_kernel(const AttnArgs a) {
  constexpr int TPR = D / 4;  // threads per row
  const int row = blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * 4;
  if (row >= a.comb_rows) return;
  int e = 0;
  for (int i = 0; i < a.n_entries; ++i) {
    const ReqInfo &R = a.req[i];
    if (R.n_splits > 1 && row >= R.comb_begin && row < R.comb_begin + R.n_q * a.Hq) e = i;
  }
  // The request's fields first, all of them waited for before the partials are loaded: the partial
  // loads sit under per-lane conditions, and with an older load still pending the compiler waits for
  // every load issued so far after the first of them (an extra round trip).
  const ReqInfo &R = a.req[e];
  const int comb_begin = R.comb_begin, n_q = R.n_q, part_begin = R.part_begin, q_begin = R.q_begin;
  const int ns = R.n_splits;
  __builtin_amdgcn_s_waitcnt(0);
  const int local = row - comb_begin;
  const int q_local = local / a.Hq, h = local - q_local * a.Hq;
  const size_t stride = static_cast<size_t>(n_q) * a.Hq;  // slots between consecutive splits
  const size_t slot0 = static_cast<size_t>(part_begin) + static_cast<size_t>(q_local) * a.Hq + h;
  // every partial is loaded up front (one round trip), then merged in split order
  float pm[MS], pl[MS];
  f32x4 po[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    pm[s] = -INFINITY;
    pl[s] = 0.f;
    po[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s < ns) {
      const size_t slot = slot0 + s * stride;
      pm[s] = a.part_ml[slot * 2];
      pl[s] = a.part_ml[slot * 2 + 1];
      po[s] = *reinterpret_cast<const f32x4 *>(a.part_o + slot * D + d0);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s) M = fmaxf(M, pm[s]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const float wgt = s < ns ? __builtin_amdgcn_exp2f(pm[s] - M) : 0.f;
    lsum += wgt * pl[s];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += wgt * po[s][k];
  }
  const float inv = 1.f / lsum;
  const size_t orow = static_cast<size_t>(q_begin + q_local) * a.Hq + h;
  if constexpr (Cfg<T>::kBf16) {
    bf16x4 v4;
#pragma unroll
    for (int k = 0; k < 4; ++k) v4[k] = static_cast<__bf16>(acc[k] * inv);
    *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(a.out) + orow * D + d0) = v4;
  } else {
    f32x4 v4;
#pragma unroll
    for (int k = 0; k < 4; ++k) v4[k] = acc[k] * inv;
    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + orow * D + d0) = v4;
  }
}

// ------------------------------------------------------------------------------------------------
// host-side planning
// ------------------------------------------------------------------------------------------------
struct AttnPlan {
  AttnArgs args;
  int grid;
  int comb_grid;
  size_t part_slots;
  size_t ws_bytes;
  int max_splits;  // largest split count of any request
};

// Compute units of the current device (one bf16 / fp32 workgroup each); 256 when no device answers.
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

// Work items are (request, row tile of `rows` query-head rows, key/value head); a request's prefix
// may be cut into s equal key ranges ("splits") so that there are enough items for every compute
// unit, at the price of partial results that a second pass merges. The split count is the one that
// minimises a simple estimate, in microseconds, of
//   makespan: max(longest item, ceil(items / slots) * mean item), items of 64-key tiles at an
//             assumed ~50 % of the MFMA rate, and
//   merge:    the partial rows written and read back once at an assumed ~5 TB/s.
int plan_attn(const int32_t *off, const int32_t *pre, int n_req, int B, int Hq, int Hkv, int D, int rows,
              int slots, AttnPlan *P) {
  if (!off || !pre || n_req < 1 || n_req > D3D_ATTN_MAX_REQ) return D3D_EINVAL;
  if (B < 1 || B > 64 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return D3D_EINVAL;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return D3D_EUNSUPPORTED;
  if (D != 64 && D != 128) return D3D_EUNSUPPORTED;
  if (off[0] != 0) return D3D_EINVAL;
  for (int i = 0; i < n_req; ++i) {
    if (off[i + 1] < off[i] || pre[i] < 0 || pre[i] > kMaxPrefix) return D3D_EINVAL;
  }
  const long long total_q = static_cast<long long>(off[n_req]) * B;
  // packed rows are addressed with 32-bit byte offsets (buffer loads)
  if (total_q >= (1ll << 31) || Hkv >= (1 << 16) || total_q * Hkv * D * 2 >= (1ll << 31)) return D3D_EUNSUPPORTED;
  const int Qt = rows / G;
  AttnArgs &a = P->args;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.Qt = Qt;
  a.n_new = static_cast<int>(total_q);

  std::vector<int> n_q(n_req), tiles(n_req), splits(n_req), len(n_req), len0(n_req);
  for (int i = 0; i < n_req; ++i) {
    n_q[i] = (off[i + 1] - off[i]) * B;
    tiles[i] = (n_q[i] + Qt - 1) / Qt;
  }
  const double tile_us = kKeys * static_cast<double>(rows) * D * 4 / 4.9e12 * 1e6;
  const double row_us = (D * 4.0 + 8.0) * 2 / 5e12 * 1e6;
  auto split_of = [&](int i, int s) {
    return pre[i] == 0 ? 1 : std::max(1, std::min(s, (pre[i] + kMinSplit - 1) / kMinSplit));
  };
  int best_s = 1;
  double best_t = 0;
  for (int s = 1; s <= kMaxSplits; ++s) {
    double items = 0, work = 0, longest = 0, merge = 0;
    for (int i = 0; i < n_req; ++i) {
      if (n_q[i] == 0) continue;
      const int si = split_of(i, s);
      const int ti = (pre[i] + si * kKeys - 1) / (si * kKeys) + 1;  // tiles per item (+1 for the tail)
      const double ni = static_cast<double>(tiles[i]) * Hkv * si;
      items += ni;
      work += ni * ti;
      longest = std::max(longest, static_cast<double>(ti));
      if (si > 1) merge += static_cast<double>(si) * n_q[i] * Hq;
    }
    if (items == 0) break;
    const double t = std::max(longest, std::ceil(items / slots) * (work / items)) * tile_us + merge * row_us;
    if (s == 1 || t < best_t * 0.98) {  // more splits only for a clear gain
      best_s = s;
      best_t = t;
    }
  }
  // The first split also walks the in-pack tail (at most ceil((B + Qt) / 64) tiles), so it gets fewer
  // prefix keys and every split takes about the same time. A tail tile costs about 1.75 prefix tiles
  // (measured per workgroup: its rows are gathered through per-key tables, its copy is not
  // pipelined and its softmax is masked), so the first split gives up that many prefix keys per tail
  // tile, rounded down to whole tiles of its own.
  const int tail_keys = (B + Qt + kKeys - 1) / kKeys * kKeys * 7 / 4;
  // A call this small (a synchronous draft: a few row items per key/value head) leaves most compute
  // units idle at any split count the estimate above weighs, and each workgroup's fixed fill and
  // write dominate its few tiles: cut every prefix into the shortest splits the merge takes (one
  // tile, or more when that would exceed kMaxSplits) and give the first split only the in-pack tail.
  double items1 = 0;
  for (int i = 0; i < n_req; ++i) items1 += static_cast<double>(tiles[i]) * Hkv;
  if (items1 * 8 <= slots) {
    for (int i = 0; i < n_req; ++i) {
      if (pre[i] == 0) {
        splits[i] = 1;
        len[i] = len0[i] = 0;
        continue;
      }
      int l = kKeys;
      if (1 + (pre[i] + l - 1) / l > kMaxSplits) l = ((pre[i] + kMaxSplits - 2) / (kMaxSplits - 1) + kKeys - 1) / kKeys * kKeys;
      len0[i] = 0;
      len[i] = l;
      splits[i] = 1 + (pre[i] + l - 1) / l;
    }
  } else
  for (int i = 0; i < n_req; ++i) {
    if (pre[i] == 0) {
      splits[i] = 1;
      len[i] = len0[i] = 0;
      continue;
    }
    const int si = split_of(i, best_s);
    if (si == 1) {
      splits[i] = 1;
      len[i] = len0[i] = pre[i];
      continue;
    }
    const int share = ((pre[i] + tail_keys + si - 1) / si + kKeys - 1) / kKeys * kKeys;
    const int l0 = std::max(kKeys, std::min(pre[i], (share - tail_keys) / kKeys * kKeys));
    const int rest = pre[i] - l0;
    if (rest <= 0) {
      splits[i] = 1;
      len[i] = len0[i] = pre[i];
      continue;
    }
    int l = ((rest + si - 2) / (si - 1) + kKeys - 1) / kKeys * kKeys;
    len0[i] = l0;
    len[i] = l;
    splits[i] = 1 + (rest + l - 1) / l;
  }
  // longest work item first (per-item keys; ties keep request order)
  std::vector<int> order;
  for (int i = 0; i < n_req; ++i)
    if (n_q[i] > 0) order.push_back(i);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    const int kx = std::min(len[x], pre[x]), ky = std::min(len[y], pre[y]);
    return kx > ky;
  });
  int groups = 0, t_max = 1;
  size_t part = 0;
  int comb = 0;
  a.n_entries = static_cast<int>(order.size());
  for (size_t e = 0; e < order.size(); ++e) {
    const int i = order[e];
    ReqInfo &R = a.req[e];
    R.q_begin = off[i] * B;
    R.n_q = n_q[i];
    R.prefix = pre[i];
    R.split_len = len[i];
    R.split0_len = len0[i];
    R.n_splits = splits[i];
    R.group_begin = groups;
    R.block_begin = off[i];
    R.req = i;
    R.part_begin = -1;
    R.comb_begin = -1;
    if (splits[i] > 1) {
      R.part_begin = static_cast<int32_t>(part);
      part += static_cast<size_t>(splits[i]) * n_q[i] * Hq;
      R.comb_begin = comb;
      comb += n_q[i] * Hq;
    }
    groups += splits[i] * Hkv;
    t_max = std::max(t_max, tiles[i]);
  }
  if (part >= (1ull << 31)) return D3D_EUNSUPPORTED;
  P->max_splits = 1;
  for (int i = 0; i < n_req; ++i) P->max_splits = std::max(P->max_splits, splits[i]);
  a.n_groups = groups;
  a.t_max = t_max;
  a.comb_rows = comb;
  P->grid = kXcds * ((groups + kXcds - 1) / kXcds) * t_max;
  const int rows_per_block = kThreads / (D / 4);
  P->comb_grid = (comb + rows_per_block - 1) / rows_per_block;
  P->part_slots = part;
  P->ws_bytes = part ? align_up(part * D * sizeof(float), 256) + align_up(part * 2 * sizeof(float), 256) : 0;
  return D3D_OK;
}

template <typename T, int D>
void launch(const AttnPlan &P, bool paged, hipEvent_t join, hipStream_t stream) {
  if (P.args.n_groups > 0) {
    if constexpr (Cfg<T>::kBf16) {
      // rows one DMA instruction covers: 64 / (D / 8)
      if (!paged)
        attn_kernel_bf16<D, kContig><<<P.grid, kBfThreads, 0, stream>>>(P.args);
      else if (P.args.page_size % (512 / D) == 0)
        attn_kernel_bf16<D, kPagedWave><<<P.grid, kBfThreads, 0, stream>>>(P.args);
      else
        attn_kernel_bf16<D, kPagedLane><<<P.grid, kBfThreads, 0, stream>>>(P.args);
    } else {
      if (paged)
        attn_kernel_f32<D, true><<<P.grid, kThreads, 0, stream>>>(P.args);
      else
        attn_kernel_f32<D, false><<<P.grid, kThreads, 0, stream>>>(P.args);
    }
  }
  if (join) (void)hipStreamWaitEvent(stream, join, 0);  // the caller's other stream joins here
  if (P.args.comb_rows > 0) {
    if (P.max_splits <= 8)
      combine_kernel<T, D, 8><<<P.comb_grid, kThreads, 0, stream>>>(P.args);
    else
      combine_kernel<T, D, kMaxSplits><<<P.comb_grid, kThreads, 0, stream>>>(P.args);
  }
}

}  // namespace
}  // namespace d3d

extern "C" size_t draft_attn_packed_workspace(d3d_dtype dtype, const int32_t *req_block_off,
                                              const int32_t *req_prefix_len, int n_req, int block_size,
                                              int n_heads_q, int n_heads_kv, int head_dim) {
  if (dtype != D3D_BF16 && dtype != D3D_F32) return 0;
  d3d::AttnPlan P;
  if (d3d::plan_attn(req_block_off, req_prefix_len, n_req, block_size, n_heads_q, n_heads_kv, head_dim,
                     dtype == D3D_BF16 ? d3d::kBfRows : d3d::kRows, d3d::device_cus(), &P) != D3D_OK)
    return 0;
  return P.ws_bytes;
}

extern "C" int draft_attn_packed_join(d3d_dtype dtype, const void *q, const void *k_new, const void *v_new,
                                      const void *k_cache, const void *v_cache, const int32_t *page_table,
                                      int page_size, int max_pages, int num_pages, int kv_stride,
                                      const d3d_block_desc *descs, const int32_t *req_block_off,
                                      const int32_t *req_prefix_len, int n_req, int block_size, int n_heads_q,
                                      int n_heads_kv, int head_dim, float scale, void *out, void *ws,
                                      size_t ws_bytes, hipEvent_t join, hipStream_t stream) {
  using namespace d3d;
  if (dtype != D3D_BF16 && dtype != D3D_F32) return D3D_EINVAL;
  AttnPlan P;
  const int st = plan_attn(req_block_off, req_prefix_len, n_req, block_size, n_heads_q, n_heads_kv, head_dim,
                           dtype == D3D_BF16 ? kBfRows : kRows, device_cus(), &P);
  if (st != D3D_OK) return st;
  if (!q || !k_new || !v_new || !descs || !out) return D3D_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return D3D_EINVAL;
  int max_pre = 0;
  for (int i = 0; i < n_req; ++i) max_pre = std::max(max_pre, req_prefix_len[i]);
  const bool paged = page_table != nullptr;
  if (max_pre > 0 && (!k_cache || !v_cache)) return D3D_EINVAL;
  if (paged) {
    if (page_size < 1 || max_pages < 1 || num_pages < 1) return D3D_EINVAL;
    if (static_cast<long long>(max_pages) * page_size < max_pre) return D3D_EINVAL;
  } else if (max_pre > 0) {
    if (kv_stride < max_pre) return D3D_EINVAL;
    // one request's rows of the contiguous cache are addressed with 32-bit byte offsets
    if (static_cast<long long>(kv_stride) * n_heads_kv * head_dim * 2 >= (1ll << 31)) return D3D_EUNSUPPORTED;
  }
  if (P.ws_bytes && (!ws || ws_bytes < P.ws_bytes)) return D3D_EWORKSPACE;
  for (const void *ptr : {q, k_new, v_new, static_cast<const void *>(out)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return D3D_EINVAL;
  if (max_pre > 0)
    for (const void *ptr : {k_cache, v_cache})
      if (reinterpret_cast<uintptr_t>(ptr) % 16) return D3D_EINVAL;
  AttnArgs &a = P.args;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.descs = descs;
  a.out = out;
  a.part_o = static_cast<float *>(ws);
  a.part_ml = P.part_slots ? reinterpret_cast<float *>(static_cast<char *>(ws) +
                                                        align_up(P.part_slots * head_dim * sizeof(float), 256))
                           : nullptr;
  a.page_size = paged ? page_size : 1;
  a.max_pages = paged ? max_pages : 0;
  a.num_pages = paged ? num_pages : 0;
  a.kv_stride = paged ? 0 : kv_stride;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  if (dtype == D3D_BF16) {
    if (head_dim == 128)
      launch<__bf16, 128>(P, paged, join, stream);
    else
      launch<__bf16, 64>(P, paged, join, stream);
  } else {
    if (head_dim == 128)
      launch<float, 128>(P, paged, join, stream);
    else
      launch<float, 64>(P, paged, join, stream);
  }
  return launch_status();
}

extern "C" int draft_attn_packed(d3d_dtype dtype, const void *q, const void *k_new, const void *v_new,
                                 const void *k_cache, const void *v_cache, const int32_t *page_table,
                                 int page_size, int max_pages, int num_pages, int kv_stride,
                                 const d3d_block_desc *descs, const int32_t *req_block_off,
                                 const int32_t *req_prefix_len, int n_req, int block_size, int n_heads_q,
                                 int n_heads_kv, int head_dim, float scale, void *out, void *ws,
                                 size_t ws_bytes, hipStream_t stream) {
  return draft_attn_packed_join(dtype, q, k_new, v_new, k_cache, v_cache, page_table, page_size, max_pages, num_pages,
                                kv_stride, descs, req_block_off, req_prefix_len, n_req, block_size, n_heads_q,
                                n_heads_kv, head_dim, scale, out, ws, ws_bytes, nullptr, stream);
}
