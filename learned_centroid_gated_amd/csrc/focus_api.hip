// C ABI of the Focus library: host-side validation, workspace carving and launch order.
// Every argument is checked before anything is enqueued, so invalid calls are testable on a
// host without a GPU; no HIP call is made on an error path.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/focus.h"
#include "focus_internal.hpp"

using namespace focus;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kIdxLimit = (int64_t)1 << 31;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Carves consecutive 256-byte aligned regions out of a workspace (or only counts them).
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + used) : nullptr;
    used += align_up(count * sizeof(T));
    return p;
  }
};

inline int hip_status(hipError_t e) { return e == hipSuccess ? FOCUS_OK : FOCUS_ERR_HIP; }

bool is_pow2_upto16(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// ------------------------------------------------------------------ assign plan
// The scores are either two products (H W_g, then Z C^T) or one product against the folded
// matrix W_g C^T, whichever needs fewer flops per token.
bool assign_folds(int d, int d_g, int K) {
  return (int64_t)d * K <= (int64_t)d * d_g + (int64_t)d_g * K;
}
inline int padded_k(int K) { return (K + 3) / 4 * 4; }

struct AssignWs {
  float* S;
  float* Z;
  float* Bt;
  _Float16* Bp;     // fp16 planes of the current product's B operand (2 x its size)
  float* bscale;    // per-row scales of those planes
  float* v;
  float2* partials;
  int32_t* flags;   // rows whose scores the fp16 products could not represent
  int32_t* nflags;
};

size_t assign_carve(void* ws, int64_t n, int d, int d_g, int K, AssignWs* out) {
  Carver c(ws);
  const bool fold = assign_folds(d, d_g, K);
  AssignWs w{};
  w.S = c.take<float>((size_t)n * padded_k(K));
  w.Z = fold ? nullptr : c.take<float>((size_t)n * d_g);
  w.Bt = c.take<float>((size_t)(fold ? K : d_g) * d);
  const size_t bmax = fold ? (size_t)K * d : std::max((size_t)d_g * d, (size_t)K * d_g);
  w.Bp = c.take<_Float16>(2 * bmax);
  w.bscale = c.take<float>((size_t)std::max(K, d_g));
  w.v = c.take<float>((size_t)padded_k(K));
  // column summaries: the Sinkhorn row pass's blocks, or the fused first step's row blocks of
  // the score product (at most one per 128 rows) and the exact rows' blocks
  const int64_t nparts = std::max<int64_t>(sinkhorn_blocks(n, K), (n + 127) / 128 + 256);
  w.partials = c.take<float2>((size_t)nparts * K);
  w.flags = c.take<int32_t>((size_t)std::max<int64_t>(n, 1));
  w.nflags = c.take<int32_t>(1);
  if (out) *out = w;
  return c.used;
}

// ------------------------------------------------------------------ attention plan
struct AttnWs {
  uint16_t *kg, *vg;
  _Float16* og;
  float* lseg;
  int32_t* kinfo;
  int32_t* tile_pre;
  int32_t* plan;
};

// Gathered K/V per membership, the per-membership key records, the group pass's fp16
// partial outputs and their log-sum-exp, and the tile prefix of the segments.
size_t attn_carve(void* ws, int64_t n, int Hq, int Hkv, int dh, int K, int top_k, AttnWs* out) {
  Carver c(ws);
  const int64_t nk = n * top_k;
  AttnWs w{};
  w.kg = c.take<uint16_t>((size_t)nk * Hkv * dh);
  w.vg = c.take<uint16_t>((size_t)nk * Hkv * dh);
  w.og = c.take<_Float16>((size_t)nk * Hq * dh);
  w.lseg = c.take<float>((size_t)nk * Hq);
  w.kinfo = c.take<int32_t>((size_t)nk * 4);
  w.tile_pre = c.take<int32_t>((size_t)K + 1);
  const int G = Hq / Hkv > 1 ? Hq / Hkv : 1;  // the size query takes unvalidated head counts
  const int T = attn_tile_tokens(G) > 1 ? attn_tile_tokens(G) : 1;
  w.plan = c.take<int32_t>((size_t)4 * attn_work_items(nk, T, K));
  if (out) *out = w;
  return c.used;
}

// Asymmetric top-k: K/V gathered along the key bucket (one entry per token) with its key
// records, the group pass's partials per query membership, the tile prefix and the plan.
size_t attn_asym_carve(void* ws, int64_t n, int Hq, int Hkv, int dh, int K, int top_k,
                       AttnWs* out) {
  Carver c(ws);
  const int64_t nq = n * top_k;
  AttnWs w{};
  w.kg = c.take<uint16_t>((size_t)n * Hkv * dh);
  w.vg = c.take<uint16_t>((size_t)n * Hkv * dh);
  w.og = c.take<_Float16>((size_t)nq * Hq * dh);
  w.lseg = c.take<float>((size_t)nq * Hq);
  w.kinfo = c.take<int32_t>((size_t)n * 4);
  w.tile_pre = c.take<int32_t>((size_t)K + 1);
  const int G = Hq / Hkv > 1 ? Hq / Hkv : 1;
  const int T = attn_tile_tokens(G) > 1 ? attn_tile_tokens(G) : 1;
  w.plan = c.take<int32_t>((size_t)4 * attn_work_items(nq, T, K));
  if (out) *out = w;
  return c.used;
}

int check_heads(int Hq, int Hkv, int d_head) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FOCUS_ERR_ARG;
  if (!is_pow2_upto16(Hq / Hkv)) return FOCUS_ERR_UNSUPPORTED;
  if (d_head != 64 && d_head != 128) return FOCUS_ERR_UNSUPPORTED;
  return FOCUS_OK;
}

int check_groups(int K, int top_k, int max_top_k) {
  if (K < 1 || K > 1024) return FOCUS_ERR_ARG;
  if (top_k < 1 || top_k > K) return FOCUS_ERR_ARG;
  if (top_k > max_top_k) return FOCUS_ERR_UNSUPPORTED;
  return FOCUS_OK;
}

int resolve_scale(float scale, int d_head, float* out) {
  if (isnan(scale) || isinf(scale)) return FOCUS_ERR_ARG;
  *out = scale > 0.f ? scale : (float)(1.0 / sqrt((double)d_head));
  return FOCUS_OK;
}

}  // namespace

namespace {
// Host-side checks of a focus_decode call apart from its workspace, in the order the entry
// point reports them; fills the launch shape. A call with B == 0 passes with s->B == 0.
int decode_check(const uint16_t* q, const int32_t* q_groups, const uint16_t* k_cache,
                 const uint16_t* v_cache, const int32_t* cache_len, const int32_t* cache_groups,
                 const int32_t* cache_offsets, const int32_t* cache_idx, int B, int64_t Lmax,
                 int Hq, int Hkv, int d_head, int K, int top_k, int64_t window, float scale,
                 uint16_t* out, float* lse, DecodeShape* s) {
  if (B < 0 || Lmax < 1 || window < 0) return FOCUS_ERR_ARG;
  if (int st = check_heads(Hq, Hkv, d_head)) return st;
  if (int st = check_groups(K, top_k, 4)) return st;
  float sc;
  if (int st = resolve_scale(scale, d_head, &sc)) return st;
  if (Lmax * (int64_t)top_k >= kIdxLimit) return FOCUS_ERR_SHAPE;
  *s = DecodeShape{};
  if (B == 0) return FOCUS_OK;
  if (!q || !q_groups || !k_cache || !v_cache || !cache_len || !cache_groups || !cache_offsets ||
      !cache_idx || !out || !lse)
    return FOCUS_ERR_ARG;
  if (!aligned16(q) || !aligned4(q_groups) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(cache_len) || !aligned4(cache_groups) || !aligned4(cache_offsets) ||
      !aligned4(cache_idx) || !aligned16(out) || !aligned4(lse))
    return FOCUS_ERR_ALIGN;
  s->B = B;
  s->Lmax = Lmax;
  s->Hq = Hq;
  s->Hkv = Hkv;
  s->G = Hq / Hkv;
  s->dh = d_head;
  s->K = K;
  s->top_k = top_k;
  s->window = window;
  s->scale = sc;
  s->splits = decode_splits(*s);
  return FOCUS_OK;
}

// ---------------------------------------------------------------- allocation-free decode
// Scratch of focus_decode_noalloc: a file-scope device array, one copy per GPU the library runs
// on, held until the process ends. In host code `scratch` names a host-side stand-in, not device
// memory: kernels get the device address from hipGetSymbolAddress, taken once per device with
// that device current and kept in scratch_ptr.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
void* scratch_ptr[kMaxDevices] = {};
std::mutex scratch_mutex;

// The calling thread's current device's scratch address, or nullptr on a HIP error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
}  // namespace

extern "C" {

const char* focus_status_string(int status) {
  switch (status) {
    case FOCUS_OK: return "FOCUS_OK";
    case FOCUS_ERR_ARG: return "FOCUS_ERR_ARG: null pointer or out-of-range argument";
    case FOCUS_ERR_SHAPE: return "FOCUS_ERR_SHAPE: sizes overflow the int32 index space";
    case FOCUS_ERR_UNSUPPORTED: return "FOCUS_ERR_UNSUPPORTED: shape has no kernel in this build";
    case FOCUS_ERR_ALIGN: return "FOCUS_ERR_ALIGN: device pointer not 16-byte aligned";
    case FOCUS_ERR_WORKSPACE: return "FOCUS_ERR_WORKSPACE: workspace missing or too small";
    case FOCUS_ERR_HIP: return "FOCUS_ERR_HIP: HIP runtime error while enqueueing";
    case FOCUS_ERR_SCRATCH:
      return "FOCUS_ERR_SCRATCH: the call needs more scratch than the allocation-free entry point holds";
    default: return "FOCUS_ERR_UNKNOWN";
  }
}

int focus_version(void) { return 500; }  // 0.5.0: adds the group-slotted membership entry points

// ============================================================================ assign
size_t focus_assign_workspace_size(int64_t n, int d, int d_g, int K) {
  if (n < 0 || d < 1 || d_g < 1 || K < 1) return 0;
  return assign_carve(nullptr, n, d, d_g, K, nullptr);
}

int focus_assign(const float* hidden, const float* w_g, const float* centroids, int64_t n, int d,
                 int d_g, int K, int top_k, int sinkhorn_iters, int32_t* groups,
                 float* col_potential, void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 0 || d < 1 || d_g < 1 || d_g > 1024 || sinkhorn_iters < 0) return FOCUS_ERR_ARG;
  if (d % 4 != 0 || d_g % 4 != 0) return FOCUS_ERR_UNSUPPORTED;
  if (int st = check_groups(K, top_k, 8)) return st;
  if (n * (int64_t)top_k >= kIdxLimit) return FOCUS_ERR_SHAPE;
  if (n == 0) return FOCUS_OK;
  if (!hidden || !w_g || !centroids || !groups) return FOCUS_ERR_ARG;
  if (!aligned16(hidden) || !aligned16(w_g) || !aligned16(centroids) || !aligned4(groups) ||
      !aligned4(col_potential) || !aligned16(workspace))
    return FOCUS_ERR_ALIGN;
  AssignWs w;
  const size_t need = assign_carve(workspace, n, d, d_g, K, &w);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  const int ldS = padded_k(K);
  hipError_t e;
  // The n-row products run as fp16 pair products (inner dimension a multiple of 32), else as
  // the bf16 split product. Rows the fp16 products cannot represent (hidden values beyond
  // fp16's range) are listed by the product that yields S (or by the first, when only it runs
  // on fp16), so no row is listed twice, and their scores recomputed exactly before Sinkhorn.
  // When S comes from an fp16 product spanning K <= 256 columns per block, that product's
  // epilogue also takes Sinkhorn's first row step (the exact rows add theirs).
  const bool fold = assign_folds(d, d_g, K);
  const bool s_f16 = (fold ? d : d_g) % 32 == 0;
  const bool fuse = sinkhorn_iters > 0 && s_f16 && K <= 256;
  bool listed = false;
  int64_t row_blocks = 0;
  auto product = [&](const float* a, const float* b, float* c, int64_t m, int nn, int kd,
                     int ldc, bool scores) -> hipError_t {
    if (kd % 32 != 0) return launch_gemm_nt_f32(a, b, c, m, nn, kd, ldc, st);
    const bool lists = scores || !s_f16;
    listed = listed || lists;
    return launch_gemm_nt_f16x3(a, b, w.Bp, w.bscale, c, m, nn, kd, ldc,
                                lists ? w.flags : nullptr, w.nflags,
                                scores && fuse ? w.partials : nullptr,
                                scores && fuse ? &row_blocks : nullptr, st);
  };
  e = launch_fill_i32(w.nflags, 0, 1, st);
  if (e == hipSuccess && fold) {
    // Bt = (W_g C^T)^T = C W_g^T  [K, d];  S = H Bt^T
    e = launch_gemm_nt_f32(centroids, w_g, w.Bt, K, d, d_g, d, st);
    if (e == hipSuccess) e = product(hidden, w.Bt, w.S, n, K, d, ldS, true);
  } else if (e == hipSuccess) {
    // Bt = W_g^T [d_g, d];  Z = H W_g;  S = Z C^T
    e = launch_transpose_f32(w_g, w.Bt, d, d_g, st);
    if (e == hipSuccess) e = product(hidden, w.Bt, w.Z, n, d_g, d, d_g, false);
    if (e == hipSuccess) e = product(w.Z, centroids, w.S, n, K, d_g, ldS, true);
  }
  if (e == hipSuccess && listed)
    e = launch_exact_rows(hidden, d, fold ? w.Bt : nullptr, w_g, centroids, d_g, K, w.flags,
                          w.nflags, n, w.S, ldS, fuse ? w.partials + row_blocks * K : nullptr,
                          st);
  if (e == hipSuccess) e = launch_fill_f32(w.v, 0.f, K, st);
  int t0 = 0;
  if (e == hipSuccess && fuse) {
    e = launch_sinkhorn_cols(w.partials, (int)(row_blocks + exact_rows_blocks(n)), n, K, w.v, st);
    t0 = 1;
  }
  const int nblk = sinkhorn_blocks(n, K);
  for (int t = t0; t < sinkhorn_iters && e == hipSuccess; ++t)
    e = launch_sinkhorn_iter(w.S, n, K, ldS, w.v, w.partials, nblk, st);
  if (e == hipSuccess) e = launch_topk(w.S, w.v, n, K, ldS, top_k, groups, st);
  if (e == hipSuccess && col_potential)
    e = hipMemcpyAsync(col_potential, w.v, sizeof(float) * K, hipMemcpyDeviceToDevice, st);
  return hip_status(e);
}

// ============================================================================ bucket
size_t focus_bucket_workspace_size(int batch, int64_t n, int K, int top_k) {
  (void)top_k;
  if (batch < 1 || n < 0 || K < 1) return 0;
  const int64_t nchunks = (n + kBucketChunk - 1) / kBucketChunk;
  Carver c(nullptr);
  c.take<int32_t>((size_t)batch * K * (nchunks > 0 ? nchunks : 1));
  c.take<int32_t>((size_t)batch * K);
  return c.used;
}

int focus_bucket(const int32_t* groups, int batch, int64_t n, int K, int top_k, int32_t* offsets,
                 int32_t* idx, int32_t* slot, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (batch < 1 || n < 0) return FOCUS_ERR_ARG;
  if (int st = check_groups(K, top_k, 8)) return st;
  if (n * (int64_t)top_k >= kIdxLimit) return FOCUS_ERR_SHAPE;
  if (!offsets) return FOCUS_ERR_ARG;
  if (n > 0 && (!groups || !idx || !slot)) return FOCUS_ERR_ARG;
  if (!aligned4(groups) || !aligned4(offsets) || !aligned4(idx) || !aligned4(slot) ||
      !aligned16(workspace))
    return FOCUS_ERR_ALIGN;
  const size_t need = focus_bucket_workspace_size(batch, n, K, top_k);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;
  Carver c(workspace);
  const int64_t nchunks = (n + kBucketChunk - 1) / kBucketChunk;
  int32_t* counts = c.take<int32_t>((size_t)batch * K * (nchunks > 0 ? nchunks : 1));
  int32_t* totals = c.take<int32_t>((size_t)batch * K);
  hipStream_t st = (hipStream_t)stream;
  if (n == 0) return hip_status(launch_fill_i32(offsets, 0, (int64_t)batch * (K + 1), st));
  return hip_status(launch_bucket(groups, batch, n, K, top_k, offsets, idx, slot, counts, totals,
                                  st));
}

int focus_bucket_append(const int32_t* new_groups, const int32_t* cache_len, int batch,
                        int64_t Lmax, int K, int top_k, const int32_t* offsets_in,
                        const int32_t* idx_in, int32_t* offsets_out, int32_t* idx_out,
                        void* stream) {
  if (batch < 1 || Lmax < 1) return FOCUS_ERR_ARG;
  if (int st = check_groups(K, top_k, 8)) return st;
  if (Lmax * (int64_t)top_k >= kIdxLimit || (int64_t)batch > 65535) return FOCUS_ERR_SHAPE;
  if (!new_groups || !cache_len || !offsets_in || !idx_in || !offsets_out || !idx_out)
    return FOCUS_ERR_ARG;
  if (offsets_in == offsets_out || idx_in == idx_out) return FOCUS_ERR_ARG;  // out of place
  if (!aligned4(new_groups) || !aligned4(cache_len) || !aligned4(offsets_in) || !aligned4(idx_in) ||
      !aligned4(offsets_out) || !aligned4(idx_out))
    return FOCUS_ERR_ALIGN;
  return hip_status(launch_bucket_append(new_groups, cache_len, batch, Lmax * top_k, K, top_k,
                                         offsets_in, idx_in, offsets_out, idx_out,
                                         (hipStream_t)stream));
}

// ============================================================================ attention
size_t focus_attention_workspace_size(int64_t n, int Hq, int Hkv, int d_head, int K, int top_k) {
  if (n < 0 || Hq < 1 || Hkv < 1 || d_head < 1 || K < 1 || top_k < 1) return 0;
  return attn_carve(nullptr, n, Hq, Hkv, d_head, K, top_k, nullptr);
}

int focus_attention_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n, int Hq,
                       int Hkv, int d_head, const int32_t* groups, const int32_t* offsets,
                       const int32_t* idx, const int32_t* slot, int K, int top_k, int64_t window,
                       float scale, uint16_t* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* stage_events,
                       int num_events) {
  if (n < 0 || window < 0) return FOCUS_ERR_ARG;
  if (num_events < 0 || num_events > 8 || (num_events > 0 && !stage_events)) return FOCUS_ERR_ARG;
  if (int st = check_heads(Hq, Hkv, d_head)) return st;
  if (int st = check_groups(K, top_k, 4)) return st;
  float sc;
  if (int st = resolve_scale(scale, d_head, &sc)) return st;
  if (n * (int64_t)top_k >= kIdxLimit) return FOCUS_ERR_SHAPE;
  if (n == 0) return FOCUS_OK;
  if (!q || !k || !v || !groups || !offsets || !idx || !slot || !out || !lse)
    return FOCUS_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(groups) ||
      !aligned4(offsets) || !aligned4(idx) || !aligned4(slot) || !aligned16(out) ||
      !aligned4(lse) || !aligned16(workspace))
    return FOCUS_ERR_ALIGN;
  AttnWs w;
  const size_t need = attn_carve(workspace, n, Hq, Hkv, d_head, K, top_k, &w);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;

  AttnShape s{};
  s.n = n;
  s.nk = n * top_k;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.G = Hq / Hkv;
  s.dh = d_head;
  s.K = K;
  s.top_k = top_k;
  s.window = window < n + 1 ? window : n + 1;  // a window beyond the sequence is the whole past
  s.scale = sc;
  hipStream_t st = (hipStream_t)stream;
  auto mark = [&](int i) -> hipError_t {
    if (i >= num_events || !stage_events[i]) return hipSuccess;
    return hipEventRecord((hipEvent_t)stage_events[i], st);
  };
  hipError_t e = mark(0);
  if (e == hipSuccess) e = launch_gather_kv(k, v, idx, groups, slot, s, w.kg, w.vg, w.kinfo, st);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) e = launch_tile_prefix(offsets, K, attn_tile_tokens(s.G), w.tile_pre, st);
  if (e == hipSuccess) e = launch_plan_tiles(offsets, w.tile_pre, w.kinfo, s, w.plan, st);
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess) e = mark(4);
  if (e == hipSuccess)
    e = launch_group_attention(q, w.kg, w.vg, offsets, w.tile_pre, w.kinfo, w.plan, s, w.og,
                               w.lseg, st);
  if (e == hipSuccess) e = mark(5);
  if (e == hipSuccess) e = mark(6);
  if (e == hipSuccess)
    e = launch_window_attention(q, k, v, w.og, w.lseg, slot, s, out, lse, st);
  if (e == hipSuccess) e = mark(7);
  return hip_status(e);
}

size_t focus_attention_asym_workspace_size(int64_t n, int Hq, int Hkv, int d_head, int K,
                                           int top_k) {
  if (n < 0 || Hq < 1 || Hkv < 1 || d_head < 1 || K < 1 || top_k < 1) return 0;
  return attn_asym_carve(nullptr, n, Hq, Hkv, d_head, K, top_k, nullptr);
}

int focus_attention_asym(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                         int Hq, int Hkv, int d_head, const int32_t* q_offsets,
                         const int32_t* q_idx, const int32_t* q_slot, int top_k,
                         const int32_t* k_offsets, const int32_t* k_idx, const int32_t* k_slot,
                         int K, int64_t window, float scale, uint16_t* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 0 || window < 0) return FOCUS_ERR_ARG;
  if (int st = check_heads(Hq, Hkv, d_head)) return st;
  if (int st = check_groups(K, top_k, 4)) return st;
  float sc;
  if (int st = resolve_scale(scale, d_head, &sc)) return st;
  if (n * (int64_t)top_k >= kIdxLimit) return FOCUS_ERR_SHAPE;
  if (n == 0) return FOCUS_OK;
  if (!q || !k || !v || !q_offsets || !q_idx || !q_slot || !k_offsets || !k_idx || !k_slot ||
      !out || !lse)
    return FOCUS_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(q_offsets) ||
      !aligned4(q_idx) || !aligned4(q_slot) || !aligned4(k_offsets) || !aligned4(k_idx) ||
      !aligned4(k_slot) || !aligned16(out) || !aligned4(lse) || !aligned16(workspace))
    return FOCUS_ERR_ALIGN;
  AttnWs w;
  const size_t need = attn_asym_carve(workspace, n, Hq, Hkv, d_head, K, top_k, &w);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;

  AttnShape s{};  // query side: n * top_k memberships
  s.n = n;
  s.nk = n * top_k;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.G = Hq / Hkv;
  s.dh = d_head;
  s.K = K;
  s.top_k = top_k;
  s.window = window < n + 1 ? window : n + 1;
  s.scale = sc;
  AttnShape sk = s;  // key side: one membership per token
  sk.nk = n;
  sk.top_k = 1;
  hipStream_t st = (hipStream_t)stream;
  // with one group per token the gather reads no group list (a key has no lower groups)
  hipError_t e = launch_gather_kv(k, v, k_idx, nullptr, k_slot, sk, w.kg, w.vg, w.kinfo, st);
  if (e == hipSuccess) e = launch_tile_prefix(q_offsets, K, attn_tile_tokens(s.G), w.tile_pre, st);
  if (e == hipSuccess)
    e = launch_plan_tiles_asym(q_offsets, w.tile_pre, q_idx, k_offsets, k_idx, s, w.plan, st);
  if (e == hipSuccess)
    e = launch_group_attention_asym(q, w.kg, w.vg, q_idx, w.kinfo, w.plan, s, w.og, w.lseg, st);
  if (e == hipSuccess) e = launch_window_attention(q, k, v, w.og, w.lseg, q_slot, s, out, lse, st);
  return hip_status(e);
}

int focus_soft_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                         int Hq, int Hkv, int d_head, const int32_t* groups, int K, int top_k,
                         int64_t window, float lambda, float scale, uint16_t* out, float* lse,
                         void* stream) {
  if (n < 0 || window < 0 || isnan(lambda) || isinf(lambda)) return FOCUS_ERR_ARG;
  if (int st = check_heads(Hq, Hkv, d_head)) return st;
  if (int st = check_groups(K, top_k, 4)) return st;
  float sc;
  if (int st = resolve_scale(scale, d_head, &sc)) return st;
  if (n * (int64_t)top_k >= kIdxLimit) return FOCUS_ERR_SHAPE;
  if (n == 0) return FOCUS_OK;
  if (!q || !k || !v || !groups || !out || !lse) return FOCUS_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(groups) || !aligned16(out) ||
      !aligned4(lse))
    return FOCUS_ERR_ALIGN;
  AttnShape s{};
  s.n = n;
  s.nk = n * top_k;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.G = Hq / Hkv;
  s.dh = d_head;
  s.K = K;
  s.top_k = top_k;
  s.window = window < n + 1 ? window : n + 1;
  s.scale = sc;
  // far-pair bias log sigmoid(lambda * a), a = +1/2 (shared group) or -1/2, as -log1p(exp(-x))
  auto log_sigmoid = [](double x) { return x >= 0 ? -log1p(exp(-x)) : x - log1p(exp(x)); };
  const float b_share = (float)log_sigmoid(0.5 * (double)lambda);
  const float b_none = (float)log_sigmoid(-0.5 * (double)lambda);
  return hip_status(launch_soft_attention(q, k, v, groups, s, b_none, b_share, out, lse,
                                          (hipStream_t)stream));
}

}  // extern "C"

namespace {

// ============================================================================ soft-gated training
// Workspace of the training path: the score products (W_g^T, the product operand's bf16 planes, Z,
// S), every Sinkhorn column potential v^0..v^T, the column partials, the soft assignment's two
// bf16 planes; and for the backward the rowwise dO . O, dG, dS, du, the backward column partials,
// two potential gradients and dZ.
struct TrainWs {
  float *Bt, *Z, *S, *vs;
  __bf16* Bp;
  float2* partials;
  __bf16 *gh, *gl;
  float *D, *dG, *dS, *du, *part, *dv, *dZ;
};

inline int train_groups_padded(int K) { return (K + 31) / 32 * 32; }

size_t train_carve(void* ws, int64_t n, int d, int d_g, int K, int Hq, int iters, TrainWs* out) {
  Carver c(ws);
  TrainWs w{};
  const int K4 = padded_k(K), KP = train_groups_padded(K);
  w.Bt = c.take<float>((size_t)d_g * d);
  w.Bp = c.take<__bf16>(3 * std::max((size_t)d_g * d, (size_t)K * d_g));
  w.Z = c.take<float>((size_t)n * d_g);
  w.S = c.take<float>((size_t)n * K4);
  w.vs = c.take<float>((size_t)(iters + 1) * K4);
  // column summaries: the Sinkhorn row pass's blocks, or the fused first step's row blocks of
  // the score product (at most one per 128 rows) and the exact rows' blocks
  const int64_t nparts = std::max<int64_t>(sinkhorn_blocks(n, K), (n + 127) / 128 + 256);
  w.partials = c.take<float2>((size_t)nparts * K);
  w.gh = c.take<__bf16>((size_t)n * KP);
  w.gl = c.take<__bf16>((size_t)n * KP);
  w.D = c.take<float>((size_t)n * Hq);
  w.dG = c.take<float>((size_t)n * K);
  w.dS = c.take<float>((size_t)n * K);
  w.du = c.take<float>((size_t)n);
  w.part = c.take<float>((size_t)train_sk_blocks(n) * K);
  w.dv = c.take<float>((size_t)2 * K4);
  w.dZ = c.take<float>((size_t)n * d_g);
  if (out) *out = w;
  return c.used;
}

// Checks shared by the training forward and backward, in the order they report.
int train_check(const float* hidden, const float* w_g, const float* centroids, int64_t n, int d,
                int d_g, int K, int sinkhorn_iters, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, int Hq, int Hkv, int d_head, int64_t window, float lambda,
                float scale, float* sc) {
  if (n < 0 || d < 1 || d_g < 1 || d_g > 1024 || sinkhorn_iters < 0 || sinkhorn_iters > 64 ||
      window < 0 || isnan(lambda) || isinf(lambda))
    return FOCUS_ERR_ARG;
  if (K < 1 || K > 1024) return FOCUS_ERR_ARG;
  if (K > 128 || d % 4 != 0 || d_g % 4 != 0) return FOCUS_ERR_UNSUPPORTED;
  if (int st = check_heads(Hq, Hkv, d_head)) return st;
  if (int st = resolve_scale(scale, d_head, sc)) return st;
  if (n * (int64_t)std::max(Hq, K) >= kIdxLimit || n * (int64_t)d >= ((int64_t)1 << 40))
    return FOCUS_ERR_SHAPE;
  if (n == 0) return FOCUS_OK;
  if (!hidden || !w_g || !centroids || !q || !k || !v) return FOCUS_ERR_ARG;
  if (!aligned16(hidden) || !aligned16(w_g) || !aligned16(centroids) || !aligned16(q) ||
      !aligned16(k) || !aligned16(v))
    return FOCUS_ERR_ALIGN;
  return FOCUS_OK;
}

// Scores, every Sinkhorn iterate and the soft assignment's planes, as the forward computes them.
hipError_t train_assign(const float* hidden, const float* w_g, const float* centroids, int64_t n,
                        int d, int d_g, int K, int iters, const TrainWs& w, hipStream_t st) {
  const int K4 = padded_k(K), KP = train_groups_padded(K);
  auto product = [&](const float* a, const float* b, float* c, int64_t m, int nn, int kd,
                     int ldc) -> hipError_t {
    if (kd % 32 != 0) return launch_gemm_nt_f32(a, b, c, m, nn, kd, ldc, st);
    hipError_t e2 = launch_split_planes(b, (int64_t)nn * kd, w.Bp, st);
    if (e2 != hipSuccess) return e2;
    return launch_gemm_nt_f32_planes(a, w.Bp, c, m, nn, kd, ldc, st);
  };
  // Z = H W_g (kept for the centroid gradient), S = Z C^T
  hipError_t e = launch_transpose_f32(w_g, w.Bt, d, d_g, st);
  if (e == hipSuccess) e = product(hidden, w.Bt, w.Z, n, d_g, d, d_g);
  if (e == hipSuccess) e = product(w.Z, centroids, w.S, n, K, d_g, K4);
  if (e == hipSuccess) e = launch_fill_f32(w.vs, 0.f, K4, st);
  const int nblk = sinkhorn_blocks(n, K);
  for (int t = 1; t <= iters && e == hipSuccess; ++t) {
    e = hipMemcpyAsync(w.vs + (size_t)t * K4, w.vs + (size_t)(t - 1) * K4, sizeof(float) * K4,
                       hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = launch_sinkhorn_iter(w.S, n, K, K4, w.vs + (size_t)t * K4, w.partials,
                                                  nblk, st);
  }
  const float* vprev = w.vs + (size_t)(iters > 0 ? iters - 1 : 0) * K4;
  const float* vlast = w.vs + (size_t)iters * K4;
  if (e == hipSuccess)
    e = launch_train_plan(w.S, n, K, K4, KP, vprev, vlast, iters, w.gh, w.gl, st);
  return e;
}

}  // namespace

extern "C" {

size_t focus_soft_train_workspace_size(int64_t n, int d, int d_g, int K, int Hq,
                                       int sinkhorn_iters) {
  if (n < 0 || d < 1 || d_g < 1 || K < 1 || Hq < 1 || sinkhorn_iters < 0) return 0;
  return train_carve(nullptr, n, d, d_g, K, Hq, sinkhorn_iters, nullptr);
}

int focus_soft_train_forward(const float* hidden, const float* w_g, const float* centroids,
                             int64_t n, int d, int d_g, int K, int sinkhorn_iters,
                             const uint16_t* q, const uint16_t* k, const uint16_t* v, int Hq,
                             int Hkv, int d_head, int64_t window, float lambda, float scale,
                             uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  float sc;
  if (int st = train_check(hidden, w_g, centroids, n, d, d_g, K, sinkhorn_iters, q, k, v, Hq, Hkv,
                           d_head, window, lambda, scale, &sc))
    return st;
  if (n == 0) return FOCUS_OK;
  if (!out || !lse) return FOCUS_ERR_ARG;
  if (!aligned16(out) || !aligned4(lse) || !aligned16(workspace)) return FOCUS_ERR_ALIGN;
  TrainWs w;
  const size_t need = train_carve(workspace, n, d, d_g, K, Hq, sinkhorn_iters, &w);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = train_assign(hidden, w_g, centroids, n, d, d_g, K, sinkhorn_iters, w, st);
  TrainShape s{n, Hq, Hkv, d_head, K, train_groups_padded(K), window, sc, lambda};
  if (e == hipSuccess) e = launch_train_attention(s, q, k, v, w.gh, w.gl, out, lse, st);
  return hip_status(e);
}

int focus_soft_train_backward(const float* hidden, const float* w_g, const float* centroids,
                              int64_t n, int d, int d_g, int K, int sinkhorn_iters,
                              const uint16_t* q, const uint16_t* k, const uint16_t* v, int Hq,
                              int Hkv, int d_head, int64_t window, float lambda, float scale,
                              const uint16_t* out, const float* lse, const uint16_t* dout,
                              float* d_centroids, float* d_w_g, float* d_hidden, void* workspace,
                              size_t workspace_bytes, void* stream) {
  float sc;
  if (int st = train_check(hidden, w_g, centroids, n, d, d_g, K, sinkhorn_iters, q, k, v, Hq, Hkv,
                           d_head, window, lambda, scale, &sc))
    return st;
  if (!d_centroids || !d_w_g) return FOCUS_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (n == 0) {  // empty sequence: zero gradients
    hipError_t e = launch_fill_f32(d_centroids, 0.f, (int64_t)K * d_g, st);
    if (e == hipSuccess) e = launch_fill_f32(d_w_g, 0.f, (int64_t)d * d_g, st);
    return hip_status(e);
  }
  if (!out || !lse || !dout) return FOCUS_ERR_ARG;
  if (!aligned16(out) || !aligned4(lse) || !aligned16(dout) || !aligned4(d_centroids) ||
      !aligned4(d_w_g) || !aligned4(d_hidden) || !aligned16(workspace))
    return FOCUS_ERR_ALIGN;
  TrainWs w;
  const size_t need = train_carve(workspace, n, d, d_g, K, Hq, sinkhorn_iters, &w);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;
  const int K4 = padded_k(K), T = sinkhorn_iters;
  hipError_t e = train_assign(hidden, w_g, centroids, n, d, d_g, K, T, w, st);
  TrainShape s{n, Hq, Hkv, d_head, K, train_groups_padded(K), window, sc, lambda};
  // attention: dG = dL/dg from every far pair, both sides
  if (e == hipSuccess) e = launch_train_delta(dout, out, n * Hq, d_head, w.D, st);
  if (e == hipSuccess) e = launch_fill_f32(w.dG, 0.f, n * K, st);
  if (e == hipSuccess)
    e = launch_train_attention_bwd(s, q, k, v, w.gh, w.gl, lse, dout, w.D, w.dG, st);
  // the plan exp(S + u^T + v^T), then every Sinkhorn iteration in reverse
  const float* vprev = w.vs + (size_t)(T > 0 ? T - 1 : 0) * K4;
  float* dv_cur = w.dv;
  float* dv_next = w.dv + K4;
  if (e == hipSuccess)
    e = launch_train_sk_plan_bwd(w.S, n, K, K4, vprev, w.vs + (size_t)T * K4, T, w.dG, w.dS, w.du,
                                 w.part, dv_cur, st);
  for (int t = T; t >= 1 && e == hipSuccess; --t) {
    e = launch_train_sk_iter_bwd(w.S, n, K, K4, w.vs + (size_t)(t - 1) * K4, w.vs + (size_t)t * K4,
                                 dv_cur, t == T ? w.du : nullptr, w.dS, w.part, dv_next, st);
    std::swap(dv_cur, dv_next);
  }
  // S = Z C^T, Z = H W_g
  if (e == hipSuccess) e = launch_train_dz(w.dS, centroids, n, K, d_g, w.dZ, st);
  if (e == hipSuccess) e = launch_fill_f32(d_centroids, 0.f, (int64_t)K * d_g, st);
  if (e == hipSuccess) e = launch_gemm_tn_atomic(w.dS, w.Z, n, K, d_g, d_centroids, st);
  if (e == hipSuccess) e = launch_fill_f32(d_w_g, 0.f, (int64_t)d * d_g, st);
  if (e == hipSuccess) e = launch_gemm_tn_atomic(hidden, w.dZ, n, d, d_g, d_w_g, st);
  if (e == hipSuccess && d_hidden) e = launch_gemm_nt_f32(w.dZ, w_g, d_hidden, n, d, d_g, d, st);
  return hip_status(e);
}

int focus_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n, int Hq,
                    int Hkv, int d_head, const int32_t* groups, const int32_t* offsets,
                    const int32_t* idx, const int32_t* slot, int K, int top_k, int64_t window,
                    float scale, uint16_t* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return focus_attention_ex(q, k, v, n, Hq, Hkv, d_head, groups, offsets, idx, slot, K, top_k,
                            window, scale, out, lse, workspace, workspace_bytes, stream, nullptr, 0);
}

// ============================================================================ decode
// The split partials: O and (max, sum) per query head and piece of each sequence's key list.
struct DecodeWs {
  float* part_o;
  float* part_ml;
};
size_t decode_carve(void* ws, int B, int Hq, int d_head, int splits, DecodeWs* out) {
  Carver c(ws);
  DecodeWs w{};
  w.part_o = c.take<float>((size_t)B * Hq * splits * d_head);
  w.part_ml = c.take<float>((size_t)B * Hq * splits * 2);
  if (out) *out = w;
  return c.used;
}

size_t focus_decode_workspace_size(int B, int64_t Lmax, int Hq, int Hkv, int d_head, int K,
                                   int top_k) {
  (void)K;
  if (B < 0 || Lmax < 1 || Hq < 1 || Hkv < 1 || d_head < 1 || top_k < 1) return 0;
  DecodeShape s{};
  s.B = B;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.G = Hq / Hkv;
  s.dh = d_head;
  return decode_carve(nullptr, B, Hq, d_head, decode_splits(s), nullptr);
}


int focus_decode(const uint16_t* q, const int32_t* q_groups, const uint16_t* k_cache,
                 const uint16_t* v_cache, const int32_t* cache_len, const int32_t* cache_groups,
                 const int32_t* cache_offsets, const int32_t* cache_idx, int B, int64_t Lmax,
                 int Hq, int Hkv, int d_head, int K, int top_k, int64_t window, float scale,
                 uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                 void* stream) {
  DecodeShape s;
  if (int st = decode_check(q, q_groups, k_cache, v_cache, cache_len, cache_groups, cache_offsets,
                            cache_idx, B, Lmax, Hq, Hkv, d_head, K, top_k, window, scale, out, lse,
                            &s))
    return st;
  if (s.B == 0) return FOCUS_OK;
  if (!aligned16(workspace)) return FOCUS_ERR_ALIGN;
  const size_t need = focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;
  DecodeWs w;
  decode_carve(workspace, B, Hq, d_head, s.splits, &w);
  return hip_status(launch_decode(q, q_groups, k_cache, v_cache, cache_len, cache_groups,
                                  cache_offsets, cache_idx, s, w.part_o, w.part_ml, out, lse,
                                  (hipStream_t)stream));
}

size_t focus_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

int focus_decode_noalloc(const uint16_t* q, const int32_t* q_groups, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* cache_len,
                         const int32_t* cache_groups, const int32_t* cache_offsets,
                         const int32_t* cache_idx, int B, int64_t Lmax, int Hq, int Hkv,
                         int d_head, int K, int top_k, int64_t window, float scale,
                         uint16_t* out, float* lse, void* stream) {
  DecodeShape s;
  if (int st = decode_check(q, q_groups, k_cache, v_cache, cache_len, cache_groups, cache_offsets,
                            cache_idx, B, Lmax, Hq, Hkv, d_head, K, top_k, window, scale, out, lse,
                            &s))
    return st;
  if (s.B == 0) return FOCUS_OK;
  // every scratch byte the kernels read is written earlier in the same call, so nothing is
  // cleared between calls
  if (focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k) > kScratchBytes)
    return FOCUS_ERR_SCRATCH;
  void* ws = device_scratch();
  if (!ws) return FOCUS_ERR_HIP;
  DecodeWs w;
  decode_carve(ws, B, Hq, d_head, s.splits, &w);
  return hip_status(launch_decode(q, q_groups, k_cache, v_cache, cache_len, cache_groups,
                                  cache_offsets, cache_idx, s, w.part_o, w.part_ml, out, lse,
                                  (hipStream_t)stream));
}

int focus_decode_paged(const uint16_t* q, const int32_t* q_groups, const uint16_t* k_pages,
                       const uint16_t* v_pages, int64_t num_pages, int page_size,
                       const int32_t* page_table, int64_t pages_per_seq, const int32_t* cache_len,
                       const int32_t* cache_groups, const int32_t* cache_offsets,
                       const int32_t* cache_idx, int B, int Hq, int Hkv, int d_head, int K,
                       int top_k, int64_t window, float scale, uint16_t* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || window < 0 || num_pages < 1 || page_size < 1 || pages_per_seq < 1)
    return FOCUS_ERR_ARG;
  if (int st = check_heads(Hq, Hkv, d_head)) return st;
  if (int st = check_groups(K, top_k, 4)) return st;
  float sc;
  if (int st = resolve_scale(scale, d_head, &sc)) return st;
  // pool rows and logical positions are kept as 32-bit ints
  if (num_pages > kIdxLimit / page_size || pages_per_seq > kIdxLimit / page_size)
    return FOCUS_ERR_SHAPE;
  const int64_t Lmax = pages_per_seq * page_size;
  if (Lmax * (int64_t)top_k >= kIdxLimit) return FOCUS_ERR_SHAPE;
  if (B == 0) return FOCUS_OK;
  if (!q || !q_groups || !k_pages || !v_pages || !page_table || !cache_len || !cache_groups ||
      !cache_offsets || !cache_idx || !out || !lse)
    return FOCUS_ERR_ARG;
  if (!aligned16(q) || !aligned4(q_groups) || !aligned16(k_pages) || !aligned16(v_pages) ||
      !aligned4(page_table) || !aligned4(cache_len) || !aligned4(cache_groups) ||
      !aligned4(cache_offsets) || !aligned4(cache_idx) || !aligned16(out) || !aligned4(lse) ||
      !aligned16(workspace))
    return FOCUS_ERR_ALIGN;
  const size_t need = focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;
  DecodeShape s{};
  s.B = B;
  s.Lmax = Lmax;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.G = Hq / Hkv;
  s.dh = d_head;
  s.K = K;
  s.top_k = top_k;
  s.window = window;
  s.scale = sc;
  s.splits = decode_splits(s);
  DecodeWs w;
  decode_carve(workspace, B, Hq, d_head, s.splits, &w);
  DecodePaging pg{page_table, page_size, pages_per_seq, num_pages};
  return hip_status(launch_decode(q, q_groups, k_pages, v_pages, cache_len, cache_groups,
                                  cache_offsets, cache_idx, s, w.part_o, w.part_ml, out, lse,
                                  (hipStream_t)stream, &pg));
}

int focus_slots_from_bucket(const int32_t* offsets, const int32_t* idx, int batch, int64_t Lmax,
                            int K, int top_k, int group_cap, int32_t* seg_len, int32_t* seg_pos,
                            int32_t* overflow, void* stream) {
  if (batch < 1 || Lmax < 1 || group_cap < 1) return FOCUS_ERR_ARG;
  if (int st = check_groups(K, top_k, 8)) return st;
  if (Lmax * (int64_t)top_k >= kIdxLimit || (int64_t)batch > 65535 ||
      (int64_t)K * group_cap >= kIdxLimit)
    return FOCUS_ERR_SHAPE;
  if (!offsets || !idx || !seg_len || !seg_pos || !overflow) return FOCUS_ERR_ARG;
  if (!aligned4(offsets) || !aligned4(idx) || !aligned4(seg_len) || !aligned4(seg_pos) ||
      !aligned4(overflow))
    return FOCUS_ERR_ALIGN;
  return hip_status(launch_slots_from_bucket(offsets, idx, batch, Lmax * top_k, K, group_cap,
                                             seg_len, seg_pos, overflow, (hipStream_t)stream));
}

int focus_slots_append(const int32_t* new_groups, const int32_t* cache_len, int batch, int K,
                       int top_k, int group_cap, int32_t* seg_len, int32_t* seg_pos,
                       int32_t* overflow, void* stream) {
  if (batch < 1 || group_cap < 1) return FOCUS_ERR_ARG;
  if (int st = check_groups(K, top_k, 8)) return st;
  if ((int64_t)K * group_cap >= kIdxLimit) return FOCUS_ERR_SHAPE;
  if (!new_groups || !cache_len || !seg_len || !seg_pos || !overflow) return FOCUS_ERR_ARG;
  if (!aligned4(new_groups) || !aligned4(cache_len) || !aligned4(seg_len) || !aligned4(seg_pos) ||
      !aligned4(overflow))
    return FOCUS_ERR_ALIGN;
  return hip_status(launch_slots_append(new_groups, cache_len, batch, K, top_k, group_cap, seg_len,
                                        seg_pos, overflow, (hipStream_t)stream));
}

int focus_decode_slots(const uint16_t* q, const int32_t* q_groups, const uint16_t* k_pages,
                       const uint16_t* v_pages, int64_t num_pages, int page_size,
                       const int32_t* page_table, int64_t pages_per_seq, const int32_t* cache_len,
                       const int32_t* cache_groups, const int32_t* seg_len,
                       const int32_t* seg_pos, int group_cap, int B, int Hq, int Hkv, int d_head,
                       int K, int top_k, int64_t window, float scale, uint16_t* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || window < 0 || num_pages < 1 || page_size < 1 || pages_per_seq < 1 ||
      group_cap < 1)
    return FOCUS_ERR_ARG;
  if (int st = check_heads(Hq, Hkv, d_head)) return st;
  if (int st = check_groups(K, top_k, 4)) return st;
  float sc;
  if (int st = resolve_scale(scale, d_head, &sc)) return st;
  if (num_pages > kIdxLimit / page_size || pages_per_seq > kIdxLimit / page_size)
    return FOCUS_ERR_SHAPE;
  const int64_t Lmax = pages_per_seq * page_size;
  if (Lmax * (int64_t)top_k >= kIdxLimit || (int64_t)K * group_cap >= kIdxLimit)
    return FOCUS_ERR_SHAPE;
  if (B == 0) return FOCUS_OK;
  if (!q || !q_groups || !k_pages || !v_pages || !page_table || !cache_len || !cache_groups ||
      !seg_len || !seg_pos || !out || !lse)
    return FOCUS_ERR_ARG;
  if (!aligned16(q) || !aligned4(q_groups) || !aligned16(k_pages) || !aligned16(v_pages) ||
      !aligned4(page_table) || !aligned4(cache_len) || !aligned4(cache_groups) ||
      !aligned4(seg_len) || !aligned4(seg_pos) || !aligned16(out) || !aligned4(lse) ||
      !aligned16(workspace))
    return FOCUS_ERR_ALIGN;
  const size_t need = focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k);
  if (!workspace || workspace_bytes < need) return FOCUS_ERR_WORKSPACE;
  DecodeShape s{};
  s.B = B;
  s.Lmax = Lmax;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.G = Hq / Hkv;
  s.dh = d_head;
  s.K = K;
  s.top_k = top_k;
  s.window = window;
  s.scale = sc;
  s.splits = decode_splits(s);
  DecodeWs w;
  decode_carve(workspace, B, Hq, d_head, s.splits, &w);
  DecodePaging pg{page_table, page_size, pages_per_seq, num_pages};
  DecodeSlots sl{seg_len, group_cap};
  return hip_status(launch_decode(q, q_groups, k_pages, v_pages, cache_len, cache_groups, nullptr,
                                  seg_pos, s, w.part_o, w.part_ml, out, lse,
                                  (hipStream_t)stream, &pg, &sl));
}

}  // extern "C"
