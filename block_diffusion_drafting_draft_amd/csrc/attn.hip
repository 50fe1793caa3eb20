// Packed draft attention on gfx950 (one drafter attention layer of the packed async forward).
//
// What is computed ([D3D] 核心方法: the prefix is shared and causally encoded, attention is
// bidirectional inside a block; 方法步骤详情 step 4: one packed forward drafts every branch):
// each packed query row attends to the whole request prefix, to the first r_b rows of its
// request's current block (the accepted slice its branch assumes), and to its own block (all rows,
// or rows up to itself for a causal block), with grouped-query heads.
//
// Design:
//  * A workgroup (4 wavefronts) owns 128 query-head rows that share one key/value head: with group
//    size G = H_q / H_kv, 128/G queries x G heads. Each wavefront owns 32 rows.
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: Q stays in registers (the B operand)
//    for the whole key walk, K and V come from LDS. The S^T accumulator leaves every lane holding one
//    query column, so the softmax row max / sum are per-lane scalars (one cross-half exchange), and
//    the accumulator registers are already the B operand of the PV product once the keys are
//    permuted consistently: V is stored transposed in LDS with each 16-key group reordered so that
//    the 8 keys a lane's accumulator holds are 8 contiguous bf16 (one 16-byte LDS read).
//  * Prefix phase: 64-key tiles over the request's prefix, no mask except the ragged end; every
//    packed query of the request shares this one walk (no per-branch prefix re-read).
//  * In-pack tail: the keys of the request's current block and of the blocks the tile's queries
//    belong to are gathered into 64-key tiles with a per-(row, key) visibility test from the block
//    descriptors.
//  * Split-KV: a request's prefix is cut into equal key ranges; each (request, split, kv head) is a
//    "group" whose tiles share one key/value slice. Groups are dealt round-robin to the 8 XCDs so that
//    all tiles of a group run on one XCD (its L2 serves the slice to all of them), longest first.
//    Split partials (unnormalised O, running max, sum) are merged by a second kernel.
#include <float.h>
#include <math.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "d3d_internal.h"

namespace d3d {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;  // query-head rows per workgroup
constexpr int kKeys = 64;   // keys per tile
constexpr int kTargetItems = 768;
constexpr int kMinSplit = 256;
constexpr int kMaxSplits = 16;

struct ReqInfo {
  int32_t q_begin;      // global packed row of the request's first query
  int32_t n_q;          // packed query rows of the request
  int32_t prefix;       // prefix length
  int32_t split_len;    // keys per split (multiple of 64), 0 when the prefix is empty
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

// LDS row strides (elements). bf16: K [64][D+8], V^T [D][64+8]. f32: K [64][D+2], V [64][D+8].
template <typename T, int D>
struct Lds {
  static constexpr bool kBf16 = Cfg<T>::kBf16;
  static constexpr int KS = kBf16 ? D + 8 : D + 2;
  static constexpr int VS = kBf16 ? kKeys + 8 : D + 8;
  static constexpr int VROWS = kBf16 ? D : kKeys;
  static constexpr int K_ELEMS = kKeys * KS;
  static constexpr int V_ELEMS = VROWS * VS;
};

// Column of key kappa (0..63) inside the transposed V tile: within each 16-key group, keys
// {0-3, 8-11} -> columns 0-7 and {4-7, 12-15} -> columns 8-15, matching the keys one lane half of
// the S^T accumulator holds.
__device__ __forceinline__ int vt_col(int kappa) {
  const int w = kappa & 15;
  return (kappa & ~15) + 8 * ((w >> 2) & 1) + 4 * (w >> 3) + (w & 3);
}

template <typename T, int D>
struct TileRegs {
  static constexpr int CH = D * static_cast<int>(sizeof(T)) / 16;  // 16-byte chunks per row
  static constexpr int NK = kKeys * CH / kThreads;                  // K chunks per thread
  // bf16 V is loaded as (4-key group, 8-element d group) units, 4-key group index fastest so that
  // the transposed LDS stores of a wavefront half hit distinct banks; f32 V is loaded like K.
  static constexpr int NVU = Cfg<T>::kBf16 ? (16 * (D / 8) + kThreads - 1) / kThreads : NK;
  u32x4 k[NK];
  u32x4 v[Cfg<T>::kBf16 ? NVU * 4 : NK];
};

// Keys (0..63 within a tile) this thread loads: K chunk i covers key kkey(i), bytes part*16..+16 of
// its row; bf16 V covers keys 4*kg..4*kg+3 at elements 8*dg..8*dg+7 (kg fastest across lanes).
template <typename T, int D>
struct TileMap {
  static constexpr int CH = TileRegs<T, D>::CH;
  __device__ static int kkey(int i) { return (static_cast<int>(threadIdx.x) + kThreads * i) / CH; }
  __device__ static int kpart() { return static_cast<int>(threadIdx.x) % CH; }
  __device__ static int vkey(int e) { return Cfg<T>::kBf16 ? 4 * (static_cast<int>(threadIdx.x) % 16) + e : 0; }
  __device__ static int vdg() { return static_cast<int>(threadIdx.x) / 16; }
  __device__ static bool von() { return static_cast<int>(threadIdx.x) < 16 * (D / 8); }
};

// Load one 64-key tile into registers. row(kappa) returns the row of key kappa (0..63 within the tile)
// of the K (or V) cache; it must always be a valid address (callers clamp out-of-range keys to the
// last valid key -- those keys are masked, so their contents never reach the result).
template <typename T, int D, typename KF, typename VF>
__device__ __forceinline__ void load_tile(TileRegs<T, D> &r, KF key_row, VF val_row) {
  using M = TileMap<T, D>;
  constexpr int E = 16 / sizeof(T);
#pragma unroll
  for (int i = 0; i < TileRegs<T, D>::NK; ++i)
    r.k[i] = *reinterpret_cast<const u32x4 *>(key_row(M::kkey(i)) + M::kpart() * E);
  if constexpr (Cfg<T>::kBf16) {
    static_assert(TileRegs<T, D>::NVU == 1, "one V unit per thread");
    if (M::von()) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r.v[e] = *reinterpret_cast<const u32x4 *>(val_row(M::vkey(e)) + M::vdg() * 8);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TileRegs<T, D>::NK; ++i)
      r.v[i] = *reinterpret_cast<const u32x4 *>(val_row(M::kkey(i)) + M::kpart() * E);
  }
}

template <typename T, int D>
__device__ __forceinline__ void store_tile(const TileRegs<T, D> &r, T *ks, T *vs) {
  using L = Lds<T, D>;
  constexpr int CH = TileRegs<T, D>::CH;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TileRegs<T, D>::NK; ++i) {
    const int c = tid + kThreads * i;
    const int key = c / CH, part = c % CH;
    if constexpr (Cfg<T>::kBf16) {
      *reinterpret_cast<u32x4 *>(ks + key * L::KS + part * 8) = r.k[i];
    } else {
      float *dst = reinterpret_cast<float *>(ks) + key * L::KS + part * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(r.k[i][e]);
    }
  }
  if constexpr (Cfg<T>::kBf16) {
#pragma unroll
    for (int i = 0; i < TileRegs<T, D>::NVU; ++i) {
      const int u = tid + kThreads * i;
      if (u >= 16 * (D / 8)) break;
      const int kg = u % 16, dg = u / 16;
      const int col = vt_col(4 * kg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of keys 4kg..4kg+3 -> four consecutive bf16 in row d = 8dg + e: one byte permute
        // per output word picks the matching 16-bit halves of two keys' words
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 pk = {__builtin_amdgcn_perm(r.v[4 * i + 1][w], r.v[4 * i + 0][w], sel),
                    __builtin_amdgcn_perm(r.v[4 * i + 3][w], r.v[4 * i + 2][w], sel)};
        *reinterpret_cast<u32x2 *>(vs + (8 * dg + e) * L::VS + col) = pk;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TileRegs<T, D>::NK; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / CH, part = c % CH;
      *reinterpret_cast<u32x4 *>(reinterpret_cast<float *>(vs) + key * L::VS + part * 4) = r.v[i];
    }
  }
}

// Per-wavefront online-softmax state for 32 query columns.
template <int D>
struct RowState {
  f32x16 o[D / 32];
  float m;  // running max of scale*log2(e)*s
  float l;  // this lane's half of the running sum
};

// One 64-key tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
// visible(key) -> bool decides masking for this lane's query column (key = 0..63 within tile).
template <typename T, int D, typename QF, typename VIS>
__device__ __forceinline__ void tile_step(const T *ks, const T *vs, const QF &qf, RowState<D> &st,
                                          float c, bool need_mask, VIS visible) {
  using L = Lds<T, D>;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  f32x16 s[2] = {};
  if constexpr (Cfg<T>::kBf16) {
    bf16x8 kfr[2][D / 16];  // all K fragments of the tile read before the MFMA chain
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        kfr[mb][kk] = *reinterpret_cast<const bf16x8 *>(ks + (mb * 32 + col) * L::KS + kk * 16 + hh * 8);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[mb][kk], qf[kk], s[mb], 0, 0, 0);
  } else {
    const float *kf = reinterpret_cast<const float *>(ks);
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const float a = kf[(mb * 32 + col) * L::KS + 2 * kk + hh];
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[kk], s[mb], 0, 0, 0);
      }
    }
  }
  if (need_mask) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = mb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (!visible(key)) s[mb][r] = -INFINITY;
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
  if constexpr (Cfg<T>::kBf16) {
    bf16x8 vfr[4][D / 32];  // all V^T fragments of the tile
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
        vfr[t][b] = *reinterpret_cast<const bf16x8 *>(vs + (b * 32 + col) * L::VS + t * 16 + hh * 8);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = static_cast<__bf16>(s[t >> 1][8 * (t & 1) + i]);
#pragma unroll
      for (int b = 0; b < D / 32; ++b) st.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[t][b], pb, st.o[b], 0, 0, 0);
    }
  } else {
    const float *vf = reinterpret_cast<const float *>(vs);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = mb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
          st.o[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[key * L::VS + b * 32 + col], s[mb][r], st.o[b], 0, 0, 0);
      }
  }
}

__device__ __forceinline__ int find_entry(const AttnArgs &a, int gamma) {
  int e = 0;
  while (e + 1 < a.n_entries && a.req[e + 1].group_begin <= gamma) ++e;
  return e;
}

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(const AttnArgs a) {
  using L = Lds<T, D>;
  __shared__ __attribute__((aligned(16))) T ks2[2][L::K_ELEMS];
  __shared__ __attribute__((aligned(16))) T vs2[2][L::V_ELEMS];
  T *ks = ks2[0];
  T *vs = vs2[0];
  __shared__ int sh_row[kKeys];
  __shared__ int sh_blk[kKeys];
  __shared__ int sh_pos[kKeys];

  // ---- work item: XCD-aware mapping of the workgroup id onto (group, tile) ----
  const int w = blockIdx.x;
  const int x = w % kXcds, k = w / kXcds;
  const int j = k / a.t_max, tile = k - j * a.t_max;
  const int gamma = j * kXcds + x;
  if (gamma >= a.n_groups) return;
  const ReqInfo R = a.req[find_entry(a, gamma)];
  const int gl = gamma - R.group_begin;
  const int split = gl / a.Hkv, g = gl - split * a.Hkv;
  const int n_tiles = (R.n_q + a.Qt - 1) / a.Qt;
  if (tile >= n_tiles) return;
  const int k0 = split * R.split_len;
  const int k1 = min(R.prefix, k0 + R.split_len);

  // ---- this lane's query row ----
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int row = wave * 32 + col;
  const int head_local = row / a.Qt, qi = row - head_local * a.Qt;
  const int q_local = tile * a.Qt + qi;
  const bool valid = q_local < R.n_q;
  const int h = g * a.G + head_local;
  const int b_lane = valid ? q_local / a.B : -1;
  const int pos_lane = valid ? q_local - b_lane * a.B : 0;
  int r_lane = 0;
  bool causal_lane = false;
  if (valid) {
    const d3d_block_desc dsc = a.descs[R.block_begin + b_lane];
    r_lane = b_lane == 0 ? 0 : min(max(dsc.rej_pos, 0), a.B);
    causal_lane = (dsc.flags & D3D_BLOCK_CAUSAL) != 0;
  }

  // ---- Q fragment (B operand), resident for the whole walk ----
  using QFrag = typename std::conditional<Cfg<T>::kBf16, bf16x8, float>::type;
  constexpr int NQ = Cfg<T>::kBf16 ? D / 16 : D / 2;
  QFrag qf[NQ];
  {
    const T *qrow = static_cast<const T *>(a.q) + (static_cast<size_t>(R.q_begin + q_local) * a.Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
      if constexpr (Cfg<T>::kBf16) {
        qf[kk] = valid ? *reinterpret_cast<const bf16x8 *>(qrow + kk * 16 + hh * 8) : bf16x8{};
      } else {
        qf[kk] = valid ? qrow[2 * kk + hh] : 0.f;
      }
    }
  }

  RowState<D> st;
#pragma unroll
  for (int b = 0; b < D / 32; ++b) st.o[b] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;
  const T *kc = static_cast<const T *>(a.k_cache);
  const T *vc = static_cast<const T *>(a.v_cache);

  // ---- prefix phase: double-buffered 64-key tiles, one barrier per tile ----
  if (k1 > k0) {
    const size_t rs = static_cast<size_t>(a.Hkv) * D;  // elements between consecutive tokens
    const T *kb = kc + (static_cast<size_t>(R.req) * a.kv_stride * a.Hkv + g) * D;
    const T *vb = vc + (static_cast<size_t>(R.req) * a.kv_stride * a.Hkv + g) * D;
    // row of prefix token jj (clamped to the last token of this split's range)
    auto row_at = [&](const T *flat, const T *cache, int jj) -> const T * {
      jj = min(jj, k1 - 1);
      if (!PAGED) return flat + jj * rs;
      int page = a.page_table[static_cast<size_t>(R.req) * a.max_pages + jj / a.page_size];
      page = min(max(page, 0), a.num_pages - 1);
      return cache + ((static_cast<size_t>(page) * a.page_size + (jj % a.page_size)) * a.Hkv + g) * D;
    };
    TileRegs<T, D> regs;
    load_tile<T, D>(regs, [&](int kappa) { return row_at(kb, kc, k0 + kappa); },
                    [&](int kappa) { return row_at(vb, vc, k0 + kappa); });
    store_tile<T, D>(regs, ks2[0], vs2[0]);
    __syncthreads();
    int stage = 0;
    for (int kt = k0; kt < k1; kt += kKeys) {
      const int nk = kt + kKeys;
      if (nk < k1)
        load_tile<T, D>(regs, [&](int kappa) { return row_at(kb, kc, nk + kappa); },
                        [&](int kappa) { return row_at(vb, vc, nk + kappa); });
      const int lim = k1 - kt;
      tile_step<T, D>(ks2[stage], vs2[stage], qf, st, c, lim < kKeys, [&](int key) { return key < lim; });
      if (nk < k1) store_tile<T, D>(regs, ks2[stage ^ 1], vs2[stage ^ 1]);
      __syncthreads();
      stage ^= 1;
    }
  }

  // ---- in-pack tail (first split only) ----
  if (split == 0) {
    const int tq0 = tile * a.Qt;
    const int tq1 = min(R.n_q, tq0 + a.Qt);
    const int bf = tq0 / a.B, bl = (tq1 - 1) / a.B;
    const int first = max(bf, 1);
    const int n_list = a.B + max(0, bl - first + 1) * a.B;
    const T *kn = static_cast<const T *>(a.k_new);
    const T *vn = static_cast<const T *>(a.v_new);
    for (int kt = 0; kt < n_list; kt += kKeys) {
      __syncthreads();
      if (threadIdx.x < kKeys) {
        const int kappa = kt + threadIdx.x;
        int rr = -1, blk = -1, pos = 0;
        if (kappa < n_list) {
          rr = kappa < a.B ? kappa : first * a.B + (kappa - a.B);
          blk = rr / a.B;
          pos = rr - blk * a.B;
        }
        sh_row[threadIdx.x] = rr;
        sh_blk[threadIdx.x] = blk;
        sh_pos[threadIdx.x] = pos;
      }
      __syncthreads();
      TileRegs<T, D> regs;
      auto src = [&](const T *base) {
        return [&, base](int kappa) -> const T * {
          const int rr = max(sh_row[kappa], 0);  // unused slots read row 0 of the request; masked
          return base + (static_cast<size_t>(R.q_begin + rr) * a.Hkv + g) * D;
        };
      };
      load_tile<T, D>(regs, src(kn), src(vn));
      store_tile<T, D>(regs, ks, vs);
      __syncthreads();
      tile_step<T, D>(ks, vs, qf, st, c, true, [&](int key) {
        const int blk = sh_blk[key];
        if (blk < 0) return false;
        if (blk == b_lane) return !causal_lane || sh_pos[key] <= pos_lane;
        return blk == 0 && sh_pos[key] < r_lane;
      });
    }
  }

  // ---- write ----
  const float l_tot = st.l + __shfl_xor(st.l, 32);
  if (!valid) return;
  const size_t orow = static_cast<size_t>(R.q_begin + q_local) * a.Hq + h;
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
          for (int e = 0; e < 4; ++e) v4[e] = static_cast<__bf16>(st.o[b][4 * r4 + e] * inv);
          *reinterpret_cast<bf16x4 *>(static_cast<T *>(a.out) + orow * D + d0) = v4;
        } else {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = st.o[b][4 * r4 + e] * inv;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + orow * D + d0) = v4;
        }
      }
  } else {
    const size_t slot = static_cast<size_t>(R.part_begin) +
                        (static_cast<size_t>(split) * R.n_q + q_local) * a.Hq + h;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = b * 32 + 8 * r4 + 4 * hh;
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = st.o[b][4 * r4 + e];
        *reinterpret_cast<f32x4 *>(a.part_o + slot * D + d0) = v4;
      }
    if (hh == 0) {
      a.part_ml[slot * 2] = st.m;
      a.part_ml[slot * 2 + 1] = l_tot;
    }
  }
}

// Merge split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s. Each thread owns four
// consecutive elements of one row (16-byte loads); D/4 threads per row.
template <typename T, int D>
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
  const ReqInfo &R = a.req[e];
  const int local = row - R.comb_begin;
  const int q_local = local / a.Hq, h = local - q_local * a.Hq;
  const size_t stride = static_cast<size_t>(R.n_q) * a.Hq;  // slots between consecutive splits
  const size_t slot0 = static_cast<size_t>(R.part_begin) + static_cast<size_t>(q_local) * a.Hq + h;
  float M = -INFINITY;
  for (int s = 0; s < R.n_splits; ++s) M = fmaxf(M, a.part_ml[(slot0 + s * stride) * 2]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll 4
  for (int s = 0; s < R.n_splits; ++s) {
    const size_t slot = slot0 + s * stride;
    const float wgt = __builtin_amdgcn_exp2f(a.part_ml[slot * 2] - M);
    lsum += wgt * a.part_ml[slot * 2 + 1];
    const f32x4 o = *reinterpret_cast<const f32x4 *>(a.part_o + slot * D + d0);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += wgt * o[k];
  }
  const float inv = 1.f / lsum;
  const size_t orow = static_cast<size_t>(R.q_begin + q_local) * a.Hq + h;
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
};

int plan_attn(const int32_t *off, const int32_t *pre, int n_req, int B, int Hq, int Hkv, int D,
              AttnPlan *P) {
  if (!off || !pre || n_req < 1 || n_req > D3D_ATTN_MAX_REQ) return D3D_EINVAL;
  if (B < 1 || B > 64 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return D3D_EINVAL;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return D3D_EUNSUPPORTED;
  if (D != 64 && D != 128) return D3D_EUNSUPPORTED;
  if (off[0] != 0) return D3D_EINVAL;
  for (int i = 0; i < n_req; ++i) {
    if (off[i + 1] < off[i] || pre[i] < 0) return D3D_EINVAL;
  }
  const long long total_q = static_cast<long long>(off[n_req]) * B;
  if (total_q >= (1ll << 31)) return D3D_EUNSUPPORTED;
  const int Qt = kRows / G;
  AttnArgs &a = P->args;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.Qt = Qt;

  std::vector<int> n_q(n_req), tiles(n_req), splits(n_req), len(n_req);
  long long base_items = 0;
  for (int i = 0; i < n_req; ++i) {
    n_q[i] = (off[i + 1] - off[i]) * B;
    tiles[i] = (n_q[i] + Qt - 1) / Qt;
    base_items += static_cast<long long>(tiles[i]) * Hkv;
  }
  const long long factor = base_items >= kTargetItems || base_items == 0
                               ? 1
                               : (kTargetItems + base_items - 1) / base_items;
  for (int i = 0; i < n_req; ++i) {
    if (pre[i] == 0) {
      splits[i] = 1;
      len[i] = 0;
      continue;
    }
    long long s = std::min<long long>(std::min<long long>(factor, kMaxSplits), std::max(1, pre[i] / kMinSplit));
    int l = static_cast<int>((pre[i] + s - 1) / s);
    l = (l + kKeys - 1) / kKeys * kKeys;
    len[i] = l;
    splits[i] = (pre[i] + l - 1) / l;
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
void launch(const AttnPlan &P, bool paged, hipStream_t stream) {
  if (P.args.n_groups > 0) {
    if (paged)
      attn_kernel<T, D, true><<<P.grid, kThreads, 0, stream>>>(P.args);
    else
      attn_kernel<T, D, false><<<P.grid, kThreads, 0, stream>>>(P.args);
  }
  if (P.args.comb_rows > 0) combine_kernel<T, D><<<P.comb_grid, kThreads, 0, stream>>>(P.args);
}

}  // namespace
}  // namespace d3d

extern "C" size_t draft_attn_packed_workspace(const int32_t *req_block_off, const int32_t *req_prefix_len,
                                              int n_req, int block_size, int n_heads_q, int n_heads_kv,
                                              int head_dim) {
  d3d::AttnPlan P;
  if (d3d::plan_attn(req_block_off, req_prefix_len, n_req, block_size, n_heads_q, n_heads_kv, head_dim, &P) !=
      D3D_OK)
    return 0;
  return P.ws_bytes;
}

extern "C" int draft_attn_packed(d3d_dtype dtype, const void *q, const void *k_new, const void *v_new,
                                 const void *k_cache, const void *v_cache, const int32_t *page_table,
                                 int page_size, int max_pages, int num_pages, int kv_stride,
                                 const d3d_block_desc *descs, const int32_t *req_block_off,
                                 const int32_t *req_prefix_len, int n_req, int block_size, int n_heads_q,
                                 int n_heads_kv, int head_dim, float scale, void *out, void *ws,
                                 size_t ws_bytes, hipStream_t stream) {
  using namespace d3d;
  if (dtype != D3D_BF16 && dtype != D3D_F32) return D3D_EINVAL;
  AttnPlan P;
  const int st = plan_attn(req_block_off, req_prefix_len, n_req, block_size, n_heads_q, n_heads_kv, head_dim, &P);
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
  } else if (max_pre > 0 && kv_stride < max_pre) {
    return D3D_EINVAL;
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
      launch<__bf16, 128>(P, paged, stream);
    else
      launch<__bf16, 64>(P, paged, stream);
  } else {
    if (head_dim == 128)
      launch<float, 128>(P, paged, stream);
    else
      launch<float, 64>(P, paged, stream);
  }
  return launch_status();
}
