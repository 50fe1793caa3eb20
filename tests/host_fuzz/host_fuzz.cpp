// Host-side fuzz of libd3d's C ABI: argument checks, planners, workspace sizes and the host
// descriptor builders, driven with random and extreme arguments. Built together with the
// library's sources compiled for the host only (no device code object is embedded, so no kernel
// is registered) and run where no GPU is visible: an entry point that accepts its arguments
// reaches a launch that the HIP runtime refuses, and nothing touches the fake device pointers.
// Meant to run under AddressSanitizer and UndefinedBehaviorSanitizer; the statuses returned are
// checked against the rules the header states.
//
//   host_fuzz <iterations> <seed>     fuzz; exit 0 when every check held
//   host_fuzz --plant-overflow        read one element past a heap array (the sanitizer must stop it)
//   host_fuzz --plant-signed-overflow add 1 to INT_MAX (the sanitizer must stop it)

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "d3d.h"

namespace {

uint64_t g_state = 1;
long g_checks = 0;
long g_accepted = 0;  // calls whose arguments were valid and reached the launch

uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int uniform(int lo, int hi) {  // inclusive
  const uint64_t span = static_cast<uint64_t>(static_cast<int64_t>(hi) - lo) + 1;
  return static_cast<int>(lo + static_cast<int64_t>(next_u64() % span));
}

bool coin(int percent) { return uniform(0, 99) < percent; }

int mul_sat(int a, int b) {  // a * b clamped to the int range
  const long long p = static_cast<long long>(a) * b;
  return static_cast<int>(p > INT_MAX ? INT_MAX : (p < INT_MIN ? INT_MIN : p));
}

// A size argument: mostly small and plausible, sometimes at a limit or far past one.
int size_arg(int lo, int hi) {
  static const int edge[] = {INT_MIN, INT_MIN + 1, -65536, -2, -1, 0, 1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33,
                             62, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1023, 1024, 65535, 65536,
                             151936, 1 << 20, 1 << 24, 1 << 30, INT_MAX / 2, INT_MAX - 64, INT_MAX - 1, INT_MAX};
  if (coin(25)) return edge[uniform(0, static_cast<int>(sizeof(edge) / sizeof(edge[0])) - 1)];
  return uniform(lo, hi);
}

d3d_dtype bad_dtype() {  // any 32-bit value but the two valid ones
  int v;
  do v = coin(50) ? uniform(-3, 9) : static_cast<int>(next_u64());
  while (v == D3D_BF16 || v == D3D_F32);
  return static_cast<d3d_dtype>(v);
}

float temperature_arg() {
  static const float t[] = {0.f, -0.f, 1.f, 0.7f, 0.25f, 1e-30f, 1e30f, -1.f, -1e-30f, INFINITY, -INFINITY, NAN};
  return t[uniform(0, static_cast<int>(sizeof(t) / sizeof(t[0])) - 1)];
}

#define CHECK(cond, ...)                                                     \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s -- ", __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                                     \
      std::fprintf(stderr, "\n");                                            \
      std::exit(1);                                                          \
    }                                                                        \
  } while (0)

// Fake, 256-byte-aligned device addresses: never dereferenced on the host, and no kernel runs.
void *fake(int i) { return reinterpret_cast<void *>(static_cast<uintptr_t>(0x7f0000000000ull + 0x100000ull * i)); }
template <typename T>
T *fake_t(int i) { return static_cast<T *>(fake(i)); }

// An accepted call ends at a launch the runtime refuses (no kernel is registered, no device is
// visible): D3D_EHIP, or D3D_OK when the call had nothing to launch.
bool launched(int st) { return st == D3D_EHIP || st == D3D_OK; }

// ------------------------------------------------------------------ descriptor builders (host)
void fuzz_build_descs() {
  const int B = coin(80) ? uniform(1, 64) : size_arg(-4, 80);
  const int C = coin(80) ? uniform(2, B > 2 ? B : 2) : size_arg(-2, 70);
  const int F = coin(80) ? uniform(1, 6) : size_arg(-2, 12);
  const int L = coin(85) ? uniform(0, 1 << 20) : size_arg(-8, 100);
  const bool valid_shape = B >= 1 && B <= 64 && C >= 2 && C <= B && F >= 1 && L >= 0;
  const long long need = valid_shape ? static_cast<long long>(C - 1) * F + 2 : 0;
  const bool huge = need > (1 << 20);  // then only a capacity too small is tried
  int cap = valid_shape && !huge && coin(70) ? static_cast<int>(need) + uniform(-1, 2) : uniform(0, 40);
  if (cap < 0) cap = 0;
  // anchors exactly as many as the call may read; descriptors exactly `cap`
  std::vector<int32_t> anchors(valid_shape && !huge ? static_cast<size_t>(need - 1) : 1);
  for (auto &a : anchors) a = static_cast<int32_t>(next_u64());
  std::vector<d3d_block_desc> out(cap > 0 ? cap : 1);
  const int cur = static_cast<int32_t>(next_u64());
  int n_out = -7;
  const bool null_anchor = coin(3), null_out = coin(3), null_n = coin(3);
  const int st = d3d_build_branch_descs(B, C, F, L, cur, null_anchor ? nullptr : anchors.data(),
                                        null_out ? nullptr : (cap > 0 ? out.data() : nullptr), cap,
                                        null_n ? nullptr : &n_out);
  const bool valid = valid_shape && !null_anchor && !null_out && !null_n && cap > 0 && need <= cap;
  CHECK(valid ? st == D3D_OK : st == D3D_EINVAL, "B=%d C=%d F=%d L=%d cap=%d st=%d", B, C, F, L, cap, st);
  if (!valid) return;
  CHECK(n_out == need, "n_out %d need %lld", n_out, need);
  CHECK(out[0].rej_pos == 0 && out[0].anchor == cur && out[0].flags == D3D_BLOCK_CAUSAL && out[0].prefix_len == L,
        "current block");
  int w = 1;
  for (int k = 1; k < C; ++k)
    for (int f = 0; f < F; ++f, ++w)
      CHECK(out[w].rej_pos == k && out[w].anchor == anchors[(k - 1) * F + f] && out[w].flags == 0 &&
                out[w].prefix_len == L,
            "branch k=%d f=%d", k, f);
  CHECK(out[w].rej_pos == B && out[w].anchor == anchors[(C - 1) * F] && out[w].flags == 0, "full-accept block");
}

void fuzz_build_descs_batch() {
  const int n = coin(85) ? uniform(1, 40) : size_arg(-2, 50);
  const int B = coin(85) ? uniform(1, 64) : size_arg(-2, 80);
  const int C = coin(85) ? uniform(2, B > 2 ? B : 2) : size_arg(-2, 70);
  const int F = coin(85) ? uniform(1, 4) : size_arg(-2, 8);
  const bool valid_shape = n >= 1 && n <= 4096 && B >= 1 && B <= 64 && C >= 2 && C <= B && F >= 1;
  const long long per = valid_shape ? static_cast<long long>(C - 1) * F + 2 : 0;
  if (valid_shape && per * n > (1 << 22)) return;  // keep host arrays small
  int cap = valid_shape && coin(75) ? static_cast<int>(per * n) + uniform(-1, 1) : uniform(0, 64);
  if (cap < 0) cap = 0;
  const size_t nn = n >= 1 && n <= 4096 ? static_cast<size_t>(n) : 1;
  std::vector<int32_t> pre(nn), cur(nn), anchors(valid_shape ? nn * static_cast<size_t>(per - 1) : 1);
  std::vector<int32_t> off(nn + 1, -9);
  bool pre_ok = true;
  for (auto &p : pre) {
    p = coin(97) ? uniform(0, 1 << 20) : uniform(-5, -1);
    pre_ok = pre_ok && p >= 0;
  }
  for (auto &c : cur) c = static_cast<int32_t>(next_u64());
  for (auto &a : anchors) a = static_cast<int32_t>(next_u64());
  std::vector<d3d_block_desc> out(cap > 0 ? cap : 1);
  const int st = d3d_build_branch_descs_batch(n, B, C, F, pre.data(), cur.data(), anchors.data(),
                                              cap > 0 ? out.data() : nullptr, cap, off.data());
  const bool valid = valid_shape && cap > 0 && per * n <= cap && pre_ok;
  CHECK(valid ? st == D3D_OK : st == D3D_EINVAL, "n=%d B=%d C=%d F=%d cap=%d st=%d", n, B, C, F, cap, st);
  if (!valid) return;
  for (int i = 0; i <= n; ++i) CHECK(off[i] == per * i, "offset %d", i);
  for (int i = 0; i < n; ++i) {
    const d3d_block_desc *d = out.data() + per * i;
    CHECK(d[0].anchor == cur[i] && d[0].prefix_len == pre[i] && d[0].rej_pos == 0, "request %d current block", i);
    CHECK(d[per - 1].anchor == anchors[static_cast<size_t>(i) * (per - 1) + per - 2] && d[per - 1].rej_pos == B,
          "request %d full-accept block", i);
  }
}

void fuzz_build_descs_device() {
  const int n = coin(85) ? uniform(1, 4096) : size_arg(-2, 50);
  const int B = coin(85) ? uniform(1, 64) : size_arg(-2, 80);
  const int C = coin(85) ? uniform(2, B > 2 ? B : 2) : size_arg(-2, 70);
  const int F = coin(85) ? uniform(1, 8) : size_arg(-2, 8);
  const bool n1 = coin(4), n2 = coin(4), n3 = coin(4), n4 = coin(4);
  const int st = d3d_build_branch_descs_device(n, B, C, F, n1 ? nullptr : fake_t<int32_t>(1),
                                               n2 ? nullptr : fake_t<int32_t>(2), n3 ? nullptr : fake_t<int32_t>(3),
                                               n4 ? nullptr : fake_t<d3d_block_desc>(4),
                                               coin(50) ? fake_t<int32_t>(5) : nullptr, nullptr);
  bool valid = n >= 1 && B >= 1 && B <= 64 && C >= 2 && C <= B && F >= 1 && !n1 && !n2 && !n3 && !n4;
  if (valid) valid = static_cast<double>(static_cast<long long>(C - 1) * F + 2) * n < 2147483392.0;
  CHECK(valid ? launched(st) : st == D3D_EINVAL, "device descs n=%d B=%d C=%d F=%d gave %d", n, B, C, F, st);
  if (valid) ++g_accepted;
}

// ------------------------------------------------------------------ packed draft attention
void fuzz_attention() {
  const int n_req = coin(85) ? uniform(1, 64) : size_arg(-2, 70);
  const int nn = n_req >= 1 && n_req <= 80 ? n_req : 1;  // host arrays as long as the call may read
  std::vector<int32_t> off(nn + 1), pre(nn);
  const int B = coin(85) ? uniform(1, 64) : size_arg(-2, 70);
  const int Hkv = coin(85) ? (1 << uniform(0, 3)) : size_arg(-1, 9);
  const int Hq = coin(85) ? mul_sat(Hkv, 1 << uniform(0, 4)) : size_arg(-1, 40);
  const int D = coin(85) ? (coin(50) ? 64 : 128) : size_arg(-1, 300);
  bool arrays_ok = true;
  off[0] = coin(97) ? 0 : uniform(-3, 3);
  arrays_ok = off[0] == 0;
  for (int i = 0; i < nn; ++i) {
    const int blocks = coin(95) ? uniform(0, coin(20) ? 40 : 6) : uniform(-2, -1);
    const long long next = static_cast<long long>(off[i]) + blocks;
    off[i + 1] = coin(1) ? size_arg(-10, 10) : static_cast<int32_t>(next > INT_MAX ? INT_MAX : next);
    if (off[i + 1] < off[i]) arrays_ok = false;
    pre[i] = coin(90) ? (coin(10) ? 0 : uniform(1, 40000)) : size_arg(-5, 1 << 20);
    if (pre[i] < 0 || pre[i] > (1 << 30)) arrays_ok = false;
  }
  const d3d_dtype dt = coin(90) ? (coin(50) ? D3D_BF16 : D3D_F32) : bad_dtype();
  const size_t ws = draft_attn_packed_workspace(dt, off.data(), pre.data(), n_req, B, Hq, Hkv, D);
  const bool shape_ok = (dt == D3D_BF16 || dt == D3D_F32) && n_req >= 1 && n_req <= D3D_ATTN_MAX_REQ &&
                        B >= 1 && B <= 64 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && arrays_ok;
  const int G = shape_ok ? Hq / Hkv : 0;
  const bool supported = shape_ok && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) && (D == 64 || D == 128);
  if (!supported) CHECK(ws == 0, "workspace %zu for an invalid shape", ws);

  const bool paged = coin(50);
  int max_pre = 0;
  for (int i = 0; i < nn && supported; ++i) max_pre = pre[i] > max_pre ? pre[i] : max_pre;
  const int page_size = paged ? (coin(85) ? (1 << uniform(0, 8)) : size_arg(-1, 300)) : 0;
  const int max_pages = paged ? (coin(85) && page_size > 0 ? static_cast<int>((static_cast<long long>(max_pre) + page_size - 1) / page_size) +
                                                                 uniform(0, 2)
                                                           : size_arg(-1, 1 << 16))
                              : 0;
  const int num_pages = paged ? (coin(90) ? uniform(1, 1 << 20) : size_arg(-1, 10)) : 0;
  const int kv_stride = paged ? 0 : (coin(85) ? max_pre + uniform(0, 64) : size_arg(-1, 1 << 16));  // max_pre <= 2^30
  const float scale = coin(90) ? 0.125f : temperature_arg();
  const bool give_ws = coin(90);
  const size_t ws_bytes = give_ws ? (coin(85) ? ws : (ws > 0 ? ws - 1 : 0)) : 0;
  const bool misalign = coin(5);
  const void *q = coin(2) ? nullptr : static_cast<const char *>(fake(1)) + (misalign ? 8 : 0);
  const int st = draft_attn_packed(dt, q, fake(2), fake(3), fake(4), fake(5), paged ? fake_t<int32_t>(6) : nullptr,
                                   page_size, max_pages, num_pages, kv_stride, fake_t<d3d_block_desc>(7),
                                   off.data(), pre.data(), n_req, B, Hq, Hkv, D, scale, fake(8),
                                   give_ws ? fake(9) : nullptr, ws_bytes, nullptr);
  bool valid = supported && q && !misalign && scale > 0.f && std::isfinite(scale);
  if (valid && paged)
    valid = page_size >= 1 && max_pages >= 1 && num_pages >= 1 && static_cast<long long>(max_pages) * page_size >= max_pre;
  if (valid && !paged && max_pre > 0) valid = kv_stride >= max_pre;
  const bool too_big = valid && !paged && max_pre > 0 && static_cast<double>(kv_stride) * Hkv * D * 2 >= 2147483648.0;
  if (!valid) {
    CHECK(st == D3D_EINVAL || st == D3D_EUNSUPPORTED || st == D3D_EWORKSPACE, "invalid attention call gave %d", st);
    return;
  }
  if (ws > 0 && (!give_ws || ws_bytes < ws)) {
    CHECK(st == D3D_EWORKSPACE || (too_big && st == D3D_EUNSUPPORTED), "short workspace gave %d", st);
    return;
  }
  // the remaining refusals are documented size limits (32-bit offsets of one request's cache rows
  // or of the packed rows)
  CHECK(launched(st) || st == D3D_EUNSUPPORTED, "valid attention call gave %d", st);
  if (launched(st)) ++g_accepted;
}

// ------------------------------------------------------------------ verify (and its variants)
void fuzz_verify() {
  const int n_req = coin(80) ? uniform(1, 64) : size_arg(-2, 5000);
  const int n_draft = coin(80) ? uniform(1, 63) : size_arg(-2, 70);
  const int vocab = coin(80) ? (coin(50) ? uniform(1, 2000) : 151936) : size_arg(-2, 1 << 20);
  const float T = coin(60) ? (coin(50) ? 1.f : 0.f) : temperature_arg();
  const d3d_dtype dt = coin(95) ? (coin(50) ? D3D_BF16 : D3D_F32) : bad_dtype();
  const size_t ws = spec_verify_workspace(n_req, n_draft, vocab);
  const bool shape_ok = n_req >= 1 && n_draft >= 1 && n_draft <= 63 && vocab >= 1 && vocab <= (1 << 28) &&
                        static_cast<long long>(n_req) * (2 * n_draft + 1) <= INT_MAX;
  if (!shape_ok) CHECK(ws == 0, "verify workspace %zu for an invalid shape", ws);
  if (shape_ok && ws == 0) return;  // a vocabulary past the sampling pass's limit
  if (shape_ok) CHECK(ws % 256 == 0, "verify workspace %zu not 256-aligned", ws);
  const bool greedy = T == 0.f;
  const bool null_draft = coin(5), null_tok = coin(3), null_acc = coin(3), null_next = coin(3);
  const bool give_ws = coin(92);
  const size_t ws_bytes = give_ws ? (coin(85) ? ws : ws - 1) : 0;
  const int mode = uniform(0, 2);  // 0 spec_verify, 1 spec_verify_match, 2 spec_verify_noalloc
  const int total_blocks = coin(90) ? uniform(1, 1 << 12) : size_arg(-2, 4);
  const bool null_descs = coin(4), null_off = coin(4), null_hit = coin(4);
  int st;
  if (mode == 0)
    st = spec_verify(dt, fake(1), null_draft ? nullptr : fake(2), null_tok ? nullptr : fake_t<int32_t>(3), n_req,
                     n_draft, vocab, T, next_u64(), static_cast<uint32_t>(next_u64()),
                     null_acc ? nullptr : fake_t<int32_t>(4), null_next ? nullptr : fake_t<int32_t>(5),
                     coin(50) ? fake_t<float>(6) : nullptr, coin(50) ? fake_t<float>(7) : nullptr,
                     coin(50) ? fake_t<float>(8) : nullptr, coin(50) ? fake_t<uint32_t>(9) : nullptr,
                     give_ws ? fake(10) : nullptr, ws_bytes, nullptr);
  else if (mode == 1)
    st = spec_verify_match(dt, fake(1), null_draft ? nullptr : fake(2), null_tok ? nullptr : fake_t<int32_t>(3),
                           n_req, n_draft, vocab, T, next_u64(), 7u, null_acc ? nullptr : fake_t<int32_t>(4),
                           null_next ? nullptr : fake_t<int32_t>(5), fake_t<float>(6), fake_t<float>(7),
                           fake_t<float>(8), fake_t<uint32_t>(9), give_ws ? fake(10) : nullptr, ws_bytes,
                           null_descs ? nullptr : fake_t<d3d_block_desc>(11), total_blocks,
                           null_off ? nullptr : fake_t<int32_t>(12), null_hit ? nullptr : fake_t<int32_t>(13),
                           nullptr);
  else
    st = spec_verify_noalloc(dt, fake(1), null_draft ? nullptr : fake(2), null_tok ? nullptr : fake_t<int32_t>(3),
                             n_req, n_draft, vocab, T, next_u64(), 3u, null_acc ? nullptr : fake_t<int32_t>(4),
                             null_next ? nullptr : fake_t<int32_t>(5), nullptr, nullptr, nullptr, nullptr, nullptr);
  bool valid = shape_ok && (dt == D3D_BF16 || dt == D3D_F32) && !null_tok && !null_acc && !null_next &&
               T >= 0.f && std::isfinite(T) && (greedy || !null_draft);
  if (mode == 1) valid = valid && !null_descs && !null_off && !null_hit && total_blocks >= 1;
  if (!valid) {
    CHECK(st == D3D_EINVAL || (mode == 2 && st == D3D_ESCRATCH), "invalid verify call (mode %d) gave %d", mode, st);
    return;
  }
  if (mode == 2) {
    if (ws > D3D_VERIFY_SCRATCH_BYTES) {
      CHECK(st == D3D_ESCRATCH, "noalloc past its scratch gave %d", st);
      return;
    }
    // without a device the scratch address cannot be obtained
    CHECK(st == D3D_EHIP, "noalloc without a device gave %d", st);
    return;
  }
  if (!give_ws || ws_bytes < ws) {
    CHECK(st == D3D_EWORKSPACE, "short verify workspace gave %d", st);
    return;
  }
  CHECK(launched(st), "valid verify call (mode %d) gave %d", mode, st);
  ++g_accepted;
}

void fuzz_match() {
  const int n_req = coin(90) ? uniform(1, 4096) : size_arg(-2, 10);
  const int total = coin(90) ? uniform(1, 1 << 16) : size_arg(-2, 10);
  const bool n1 = coin(4), n2 = coin(4), n3 = coin(4), n4 = coin(4), n5 = coin(4);
  const int st = branch_cache_match(n1 ? nullptr : fake_t<d3d_block_desc>(1), total, n2 ? nullptr : fake_t<int32_t>(2),
                                    n_req, n3 ? nullptr : fake_t<int32_t>(3), n4 ? nullptr : fake_t<int32_t>(4),
                                    n5 ? nullptr : fake_t<int32_t>(5), nullptr);
  const bool valid = !n1 && !n2 && !n3 && !n4 && !n5 && n_req >= 1 && total >= 1;
  CHECK(valid ? launched(st) : st == D3D_EINVAL, "match n_req=%d total=%d gave %d", n_req, total, st);
  if (valid) ++g_accepted;
}

// ------------------------------------------------------------------ drafter token selection
void fuzz_select() {
  const int n_rows = coin(85) ? uniform(1, 4096) : size_arg(-2, 10);
  const int vocab = coin(85) ? (coin(50) ? uniform(1, 5000) : 151936) : size_arg(-2, 1 << 20);
  const int k = coin(85) ? uniform(1, 8) : size_arg(-2, 12);
  const d3d_dtype dt = coin(95) ? (coin(50) ? D3D_BF16 : D3D_F32) : bad_dtype();
  const bool sample = coin(50);
  const size_t ws = sample ? draft_sample_workspace(n_rows, vocab) : draft_topk_workspace(n_rows, vocab, k);
  const bool shape_ok = n_rows >= 1 && vocab >= 1 && vocab <= (1 << 28) && (sample || (k >= 1 && k <= 8));
  if (!shape_ok) CHECK(ws == 0, "select workspace %zu for an invalid shape", ws);
  if (shape_ok) CHECK(ws > 0 && ws % 256 == 0, "select workspace %zu", ws);
  const bool null_logits = coin(3), null_out = coin(3), give_ws = coin(92);
  const size_t ws_bytes = give_ws ? (coin(85) ? ws : (ws ? ws - 1 : 0)) : 0;
  const float T = coin(70) ? 1.f : temperature_arg();
  int st;
  if (sample)
    st = draft_sample(dt, null_logits ? nullptr : fake(1), vocab, n_rows, coin(50) ? fake_t<int32_t>(2) : nullptr, T,
                      next_u64(), 1u, null_out ? nullptr : fake_t<int32_t>(3), give_ws ? fake(4) : nullptr, ws_bytes,
                      nullptr);
  else
    st = draft_topk(dt, null_logits ? nullptr : fake(1), vocab, n_rows, coin(50) ? fake_t<int32_t>(2) : nullptr,
                    coin(50) ? fake_t<int32_t>(3) : nullptr, k, null_out ? nullptr : fake_t<int32_t>(4),
                    coin(50) ? fake_t<int32_t>(5) : nullptr, give_ws ? fake(6) : nullptr, ws_bytes, nullptr);
  bool valid = shape_ok && (dt == D3D_BF16 || dt == D3D_F32) && !null_logits && !null_out;
  if (sample) valid = valid && T > 0.f && std::isfinite(T);
  if (!valid) {
    CHECK(st == D3D_EINVAL, "invalid select call gave %d", st);
    return;
  }
  if (!give_ws || ws_bytes < ws) {
    CHECK(st == D3D_EWORKSPACE, "short select workspace gave %d", st);
    return;
  }
  CHECK(launched(st), "valid select call gave %d", st);
  ++g_accepted;
}

// ------------------------------------------------------------------ KV commit
void fuzz_commit() {
  const d3d_dtype dt = coin(95) ? (coin(50) ? D3D_BF16 : D3D_F32) : bad_dtype();
  const int n_req = coin(90) ? uniform(1, 512) : size_arg(-2, 10);
  const int B = coin(90) ? uniform(1, 64) : size_arg(-2, 300);
  const int page_size = coin(90) ? (1 << uniform(0, 8)) : size_arg(-2, 10);
  const int max_pages = coin(90) ? uniform(1, 4096) : size_arg(-2, 10);
  const int num_pages = coin(90) ? uniform(1, 1 << 20) : size_arg(-2, 10);
  const int Hkv = coin(90) ? (1 << uniform(0, 3)) : size_arg(-2, 10);
  const int D = coin(90) ? (coin(50) ? 64 : 128) : size_arg(-2, 300);
  const bool nulls = coin(5);
  const bool with_hit = coin(50);
  const int st = kv_commit(dt, fake(1), fake(2), fake(3), fake(4), nulls ? nullptr : fake_t<int32_t>(5), page_size,
                           max_pages, num_pages, fake_t<int32_t>(6), fake_t<int32_t>(7), fake_t<int32_t>(8), n_req, B,
                           Hkv, D, with_hit ? fake_t<int32_t>(9) : nullptr, with_hit ? fake_t<int32_t>(10) : nullptr,
                           with_hit ? fake_t<int32_t>(11) : nullptr, coin(50) ? fake_t<int32_t>(12) : nullptr, nullptr);
  const bool shape_ok = (dt == D3D_BF16 || dt == D3D_F32) && !nulls && n_req >= 1 && B >= 1 && B <= 256 &&
                        page_size >= 1 && max_pages >= 1 && num_pages >= 1 && Hkv >= 1 && D >= 1;
  if (!shape_ok) {
    CHECK(st == D3D_EINVAL, "invalid commit call gave %d", st);
    return;
  }
  if (Hkv > (1 << 16) || D > (1 << 16)) {
    CHECK(st == D3D_EUNSUPPORTED, "commit with %d heads of %d gave %d", Hkv, D, st);
    return;
  }
  const long long row = static_cast<long long>(Hkv) * D * (dt == D3D_BF16 ? 2 : 4);
  if (row % 16 != 0) {
    CHECK(st == D3D_EUNSUPPORTED, "commit row of %lld bytes gave %d", row, st);
    return;
  }
  CHECK(launched(st) || st == D3D_EUNSUPPORTED, "valid commit call gave %d", st);
  if (launched(st)) ++g_accepted;
}

// ------------------------------------------------------------------ acceptance-weighted loss
void fuzz_awl() {
  const d3d_dtype dt = coin(95) ? (coin(50) ? D3D_BF16 : D3D_F32) : bad_dtype();
  const int n_blocks = coin(85) ? uniform(1, 4096) : size_arg(-2, 10);
  const int n_pos = coin(85) ? uniform(1, 63) : size_arg(-2, 70);
  const int vocab = coin(85) ? (coin(50) ? uniform(1, 5000) : 151936) : size_arg(-2, 1 << 20);
  const double eps = coin(85) ? 1e-6 : static_cast<double>(temperature_arg());
  const size_t ws = awl_loss_workspace(n_blocks, n_pos, vocab);
  const bool shape_ok = n_blocks >= 1 && n_pos >= 1 && n_pos <= 63 && vocab >= 1 && vocab <= (1 << 28) &&
                        2ll * n_blocks * n_pos <= INT_MAX;
  if (!shape_ok) CHECK(ws == 0, "awl workspace %zu for an invalid shape", ws);
  if (shape_ok) CHECK(ws > 0 && ws % 256 == 0, "awl workspace %zu", ws);
  const bool nulls = coin(5), give_ws = coin(92);
  const size_t ws_bytes = give_ws ? (coin(85) ? ws : (ws ? ws - 1 : 0)) : 0;
  const int st = awl_loss(dt, fake(1), fake(2), fake_t<int32_t>(3), nulls ? nullptr : fake_t<int32_t>(4),
                          coin(50) ? fake_t<int32_t>(5) : nullptr, n_blocks, n_pos, vocab, eps, fake_t<float>(6),
                          coin(50) ? fake_t<float>(7) : nullptr, fake_t<double>(8), coin(50) ? fake(9) : nullptr,
                          give_ws ? fake(10) : nullptr, ws_bytes, nullptr);
  const bool valid = shape_ok && (dt == D3D_BF16 || dt == D3D_F32) && !nulls && eps >= 0.0 && std::isfinite(eps);
  if (!valid) {
    CHECK(st == D3D_EINVAL, "invalid awl call gave %d", st);
    return;
  }
  if (!give_ws || ws_bytes < ws) {
    CHECK(st == D3D_EWORKSPACE, "short awl workspace gave %d", st);
    return;
  }
  CHECK(launched(st), "valid awl call gave %d", st);
  ++g_accepted;
}

// ------------------------------------------------------------------ training attention
void fuzz_train_attn() {
  const d3d_dtype dt = coin(90) ? D3D_BF16 : (coin(50) ? D3D_F32 : bad_dtype());
  const int L = coin(85) ? uniform(0, 8192) : size_arg(-2, 10);
  const int nb = coin(85) ? uniform(0, 2048) : size_arg(-2, 4000);
  const int B = coin(85) ? uniform(1, 64) : size_arg(-2, 100);
  const int Hkv = coin(85) ? (1 << uniform(0, 3)) : size_arg(-2, 10);
  const int Hq = coin(85) ? mul_sat(Hkv, 1 << uniform(0, 5)) : size_arg(-2, 70);
  const int D = coin(90) ? 128 : size_arg(-2, 300);
  const float scale = coin(90) ? 0.0883883f : temperature_arg();
  const size_t ws = train_attn_workspace(L, nb, B, Hq, Hkv);
  const bool bwd = coin(50);
  const bool nulls = coin(5), give_ws = coin(92);
  const size_t ws_bytes = give_ws ? (coin(85) ? ws : (ws ? ws - 1 : 0)) : 0;
  int st;
  if (bwd)
    st = train_attn_bwd(dt, fake(1), fake(2), fake(3), fake(4), nulls ? nullptr : fake(5), fake_t<float>(6),
                        fake_t<int32_t>(7), L, nb, B, Hq, Hkv, D, scale, fake(8), fake(9), fake(10),
                        give_ws ? fake(11) : nullptr, ws_bytes, nullptr);
  else
    st = train_attn_fwd(dt, fake(1), fake(2), fake(3), nulls ? nullptr : fake_t<int32_t>(7), L, nb, B, Hq, Hkv, D,
                        scale, fake(4), fake_t<float>(6), nullptr);
  // EUNSUPPORTED and EINVAL both appear for shape problems (dtype / head_dim / group / sizes)
  const bool basic = dt == D3D_BF16 && D == 128 && L >= 0 && nb >= 0 && B >= 1 && Hq >= 1 && Hkv >= 1 &&
                     Hq % Hkv == 0 && 32 % (Hq / Hkv) == 0 && nb <= 2048 && static_cast<long long>(L) + 1ll * nb * B >= 1;
  if (!basic) {
    CHECK(st == D3D_EINVAL || st == D3D_EUNSUPPORTED, "invalid train attention call gave %d", st);
    return;
  }
  if (st == D3D_EUNSUPPORTED) {  // the documented size limits
    const long long n_rows = static_cast<long long>(L) + 1ll * nb * B;
    CHECK(n_rows >= (1ll << 31) || Hq >= (1 << 16) || n_rows * Hq * 128 * 2 >= (1ll << 31) || ws == 0,
          "train attention refused a small shape (L=%d nb=%d B=%d Hq=%d)", L, nb, B, Hq);
    return;
  }
  const bool need_anchor_null = !bwd && nulls && nb > 0;
  const bool valid = !(bwd ? nulls : need_anchor_null) && scale > 0.f;
  if (!valid) {
    CHECK(st == D3D_EINVAL, "invalid train attention pointers gave %d", st);
    return;
  }
  if (bwd && (!give_ws || ws_bytes < ws)) {
    CHECK(st == D3D_EWORKSPACE, "short train attention workspace gave %d", st);
    return;
  }
  CHECK(launched(st), "valid train attention call gave %d", st);
  ++g_accepted;
}

void check_status_strings() {
  for (int s = -64; s <= 64; ++s) {
    const char *m = d3d_status_string(s);
    CHECK(m != nullptr && std::strlen(m) > 0, "status %d", s);
  }
}

}  // namespace

int main(int argc, char **argv) {
  if (argc == 2 && std::strcmp(argv[1], "--plant-overflow") == 0) {
    std::vector<int32_t> v(static_cast<size_t>(argc) + 15);
    volatile int32_t x = v.data()[v.size()];
    return x == 12345 ? 3 : 0;
  }
  if (argc == 2 && std::strcmp(argv[1], "--plant-signed-overflow") == 0) {
    volatile int big = INT_MAX;
    volatile int y = big + argc - 1;
    return y == 0 ? 3 : 0;
  }
  if (argc != 3) {
    std::fprintf(stderr, "usage: host_fuzz <iterations> <seed>\n");
    return 2;
  }
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0) {
    // the fake device pointers below must never meet a real device
    std::fprintf(stderr, "host_fuzz runs only where no GPU is visible (found %d)\n", n_dev);
    return 2;
  }
  (void)hipGetLastError();
  const long iters = std::atol(argv[1]);
  g_state = std::strtoull(argv[2], nullptr, 0);
  check_status_strings();
  for (long it = 0; it < iters; ++it) {
    fuzz_build_descs();
    fuzz_build_descs_batch();
    fuzz_build_descs_device();
    fuzz_attention();
    fuzz_verify();
    fuzz_match();
    fuzz_select();
    fuzz_commit();
    fuzz_awl();
    fuzz_train_attn();
  }
  std::printf("host_fuzz: %ld iterations, %ld checks, %ld accepted calls\n", iters, g_checks, g_accepted);
  return 0;
}
