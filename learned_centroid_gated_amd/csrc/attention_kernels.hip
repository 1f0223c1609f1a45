// Gated sparse causal attention on gfx950.
//
// Pair rule ("Why Attend to Everything? Focus is the Key", Chinese technical summary,
// gist.science/zh, sections 2.1.2 and 2.1.3; Dutch technical summary, Kerncomponenten 3):
// query i attends key j <= i when i - j < window or the tokens share a group, with an exact
// softmax over the allowed pairs. The pairs are split between two passes so each is counted
// once: the window pass owns i - j < window; a far pair belongs to the lowest group the two
// tokens share. The group pass runs on contiguous group segments (K/V gathered per
// membership, Q rows read in place) and leaves one fp16 partial per membership; the window
// pass runs in original token order and merges those partials into its own by their
// log-sum-exp in its epilogue, writing the output back in token order.
//
// Flash kernel layout (both passes). A workgroup has 4 waves and 128 query rows: T = 128/G
// tokens times the G query heads of one kv head, so K/V tiles in LDS serve all G heads. A kv
// tile is 64 keys. Each wave owns 32 rows and computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from LDS, B = the wave's Q held in
// registers), so every lane holds one query column: the softmax row statistics live in one
// lane pair (l, l^32) and need a single cross-lane exchange. O^T = V^T P^T reuses the S^T
// accumulator layout directly as the B operand; V is stored transposed in LDS so the A
// operand (32 dims x 16 keys) is two 8-byte reads per lane.
#include <cstddef>
#include <type_traits>

#include "focus_internal.hpp"

namespace focus {

int attn_tile_tokens(int G) { return 128 / G; }

// ============================================================================ gather
// kg[s] = k[idx[s]], vg[s] = v[idx[s]] for every membership slot s, and kinfo[s] = (token
// position, the token's groups below this segment's group, -1 padded): the pair rule of the
// group pass needs only these, so its inner loop makes no dependent loads. Q is not gathered:
// each query row is read once, in place, by the group pass.
__global__ __launch_bounds__(256) void gather_kv_kernel(const i32x4_t* __restrict__ k,
                                                        const i32x4_t* __restrict__ v,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ groups,
                                                        const int32_t* __restrict__ slot,
                                                        int top_k, int64_t nk, int ckv,
                                                        i32x4_t* __restrict__ kg,
                                                        i32x4_t* __restrict__ vg,
                                                        i32x4_t* __restrict__ kinfo) {
  // A block copies 4 slots at a time (slot indices uniform: their tokens come from scalar
  // loads); thread t moves 16-byte chunk t (+256, ...) of each of the 4 rows, K chunks first.
  constexpr int SPB = 4;
  const int per = 2 * ckv;  // 16-byte chunks per slot
  const int t = threadIdx.x;
  for (int64_t s0 = (int64_t)blockIdx.x * SPB; s0 < nk; s0 += (int64_t)gridDim.x * SPB) {
    int32_t tok[SPB];
#pragma unroll
    for (int j = 0; j < SPB; ++j) tok[j] = s0 + j < nk ? idx[s0 + j] : -1;
    if (t < SPB && tok[t] >= 0) {
      // the membership's rank r among the token's ascending groups: lower groups come first
      const int64_t s = s0 + t;
      i32x4_t info = {tok[t], -1, -1, -1};
      for (int r = 0; r < top_k; ++r) {
        if (slot[(int64_t)tok[t] * top_k + r] == (int32_t)s) {
          for (int c2 = 0; c2 < r && c2 < 3; ++c2) info[1 + c2] = groups[(int64_t)tok[t] * top_k + c2];
          break;
        }
      }
      kinfo[s] = info;
    }
    for (int c = t; c < per; c += 256) {
      const bool isk = c < ckv;
      const int cc = isk ? c : c - ckv;
      const i32x4_t* src = isk ? k : v;
      i32x4_t* dst = isk ? kg : vg;
      i32x4_t val[SPB];
#pragma unroll
      for (int j = 0; j < SPB; ++j)
        if (tok[j] >= 0) val[j] = src[(int64_t)tok[j] * ckv + cc];
#pragma unroll
      for (int j = 0; j < SPB; ++j)
        if (tok[j] >= 0) dst[(s0 + j) * ckv + cc] = val[j];
    }
  }
}

hipError_t launch_gather_kv(const uint16_t* k, const uint16_t* v, const int32_t* idx,
                            const int32_t* groups, const int32_t* slot, const AttnShape& s,
                            uint16_t* kg, uint16_t* vg, int32_t* kinfo, hipStream_t stream) {
  const int ckv = s.Hkv * s.dh / 8;
  int64_t blocks = (s.nk + 3) / 4;  // 4 slots per block
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gather_kv_kernel, dim3(blocks), dim3(256), 0, stream, (const i32x4_t*)k,
                     (const i32x4_t*)v, idx, groups, slot, s.top_k, s.nk, ckv, (i32x4_t*)kg,
                     (i32x4_t*)vg, (i32x4_t*)kinfo);
  return hipGetLastError();
}

// ============================================================================ tile prefix
// tile_pre[g] = number of query tiles of T slots in segments 0..g-1; tile_pre[K] = total.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ off, int K,
                                                           int T, int32_t* __restrict__ tile_pre) {
  __shared__ int wsum[16];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  int x = t < K ? (off[t + 1] - off[t] + T - 1) / T : 0;
  int incl = x;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (l >= o) incl += y;
  }
  if (l == 63) wsum[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int q = 0; q < w; ++q) wbase += wsum[q];
  if (t < K) tile_pre[t] = wbase + incl - x;
  if (t == 0) {
    int total = 0;
    for (int q = 0; q < 16; ++q) total += wsum[q];
    tile_pre[K] = total;
  }
}

hipError_t launch_tile_prefix(const int32_t* offsets, int K, int T, int32_t* tile_pre,
                              hipStream_t stream) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, stream, offsets, K, T, tile_pre);
  return hipGetLastError();
}

// ============================================================================ work plan
// plan[item] = (q0, q1, kv_lo, ntiles) of group-pass work item `item`, for item < w_max (items
// past the last real one get q0 == q1). Items are (segment, query tile) in segment order, the
// heaviest tiles of a segment first; ntiles stops at the first key tile whose pairs all fall
// inside the window for the tile's last query (positions ascend within a segment).
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int32_t* __restrict__ seg_off,
                                                         const int32_t* __restrict__ tile_pre,
                                                         const i32x4_t* __restrict__ kinfo, int K,
                                                         int T, int window, int w_max,
                                                         i32x4_t* __restrict__ plan) {
  constexpr int KT_ = 64;
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= w_max) return;
  i32x4_t p = {0, 0, 0, 0};
  if (item < tile_pre[K]) {
    int lo = 0, hi = K - 1;  // largest g with tile_pre[g] <= item (a non-empty segment)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_pre[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int nt = tile_pre[lo + 1] - tile_pre[lo];
    const int t = nt - 1 - (item - tile_pre[lo]);
    const int s_lo = seg_off[lo], s_hi = seg_off[lo + 1];
    const int q0 = s_lo + t * T, q1 = min(q0 + T, s_hi);
    const int tpos_hi = kinfo[q1 - 1][0];
    int lo_t = 0, hi_t = (q1 - 1 - s_lo) / KT_ + 1;
    while (lo_t < hi_t) {
      const int mid = (lo_t + hi_t) >> 1;
      if (tpos_hi - kinfo[s_lo + mid * KT_][0] < window) hi_t = mid;
      else lo_t = mid + 1;
    }
    p = i32x4_t{q0, q1, s_lo, lo_t};
  }
  plan[item] = p;
}

int attn_work_items(int64_t nk, int T, int K) { return (int)((nk + T - 1) / T + K); }

hipError_t launch_plan_tiles(const int32_t* offsets, const int32_t* tile_pre, const int32_t* kinfo,
                             const AttnShape& s, int32_t* plan, hipStream_t stream) {
  const int T = attn_tile_tokens(s.G);
  const int w_max = attn_work_items(s.nk, T, s.K);
  const int window = (int)(s.window < s.n ? s.window : s.n);
  hipLaunchKernelGGL(plan_tiles_kernel, dim3((w_max + 255) / 256), dim3(256), 0, stream, offsets,
                     tile_pre, (const i32x4_t*)kinfo, s.K, T, window, w_max, (i32x4_t*)plan);
  return hipGetLastError();
}

// Asymmetric top-k: plan[item] = (q0, q1, kv_lo, kv_hi) with query slots [q0, q1) of the
// query bucket's segment g and key slots [kv_lo, kv_hi] of the key bucket's segment g: the keys
// of group g at positions up to the tile's last query position minus the window, the only ones
// with a far pair in the item (kv_hi = kv_lo - 1: none). Items in the same order as above.
__global__ __launch_bounds__(256) void plan_tiles_asym_kernel(
    const int32_t* __restrict__ q_off, const int32_t* __restrict__ tile_pre,
    const int32_t* __restrict__ q_idx, const int32_t* __restrict__ k_off,
    const int32_t* __restrict__ k_idx, int K, int T, int window, int w_max,
    i32x4_t* __restrict__ plan) {
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= w_max) return;
  i32x4_t p = {0, 0, 0, -1};
  if (item < tile_pre[K]) {
    int lo = 0, hi = K - 1;  // largest g with tile_pre[g] <= item (a non-empty segment)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_pre[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int nt = tile_pre[lo + 1] - tile_pre[lo];
    const int t = nt - 1 - (item - tile_pre[lo]);
    const int q0 = q_off[lo] + t * T, q1 = min(q0 + T, q_off[lo + 1]);
    const int limit = q_idx[q1 - 1] - window;  // far keys sit at positions <= limit
    int a = k_off[lo], b = k_off[lo + 1];       // first key slot past the limit, in [a, b]
    const int kv_lo = a;
    while (a < b) {
      const int mid = (a + b) >> 1;
      if (k_idx[mid] <= limit) a = mid + 1;
      else b = mid;
    }
    p = i32x4_t{q0, q1, kv_lo, a - 1};
  }
  plan[item] = p;
}

hipError_t launch_plan_tiles_asym(const int32_t* q_off, const int32_t* tile_pre,
                                  const int32_t* q_idx, const int32_t* k_off,
                                  const int32_t* k_idx, const AttnShape& s, int32_t* plan,
                                  hipStream_t stream) {
  const int T = attn_tile_tokens(s.G);
  const int w_max = attn_work_items(s.nk, T, s.K);
  const int window = (int)(s.window < s.n ? s.window : s.n);
  hipLaunchKernelGGL(plan_tiles_asym_kernel, dim3((w_max + 255) / 256), dim3(256), 0, stream,
                     q_off, tile_pre, q_idx, k_off, k_idx, s.K, T, window, w_max,
                     (i32x4_t*)plan);
  return hipGetLastError();
}

// ============================================================================ flash kernel
struct FlashArgs {
  const uint16_t* q;  // [n, Hq, DH] in token order (group pass: row of slot s is kinfo[s].x)
  const uint16_t* k;  // group: gathered [nk, Hkv, DH]; window: [n, Hkv, DH]
  const uint16_t* v;
  _Float16* og;       // group pass out / window pass in: [nk, Hq, DH] normalised partials
  float* lseg;        // group pass out / window pass in: [nk, Hq] natural log, -inf if empty
  uint16_t* out;      // window pass: [n, Hq, DH] bf16 merged output
  float* lse;         // window pass: [n, Hq] merged natural-log sum of exp
  const int32_t* slot;  // window pass: [n, top_k] membership slots of each token
  int top_k;
  int64_t n;          // tokens
  int Hq, Hkv, G, T;
  int window;         // clamped to n: a window of n tokens already spans every causal pair
  float sl2;          // scale * log2(e)
  const int32_t* seg_off;   // group: [K+1]
  const int32_t* tile_pre;  // group: [K+1]
  const i32x4_t* kinfo;     // group: per slot (position, lower groups, -1 padded)
  const i32x4_t* plan;      // group: per work item (q0, q1, kv_lo, ntiles), asymmetric
                            // (q0, q1, kv_lo, kv_hi); q0 == q1: none
  int w_max;                // group: work items per kv head (upper bound)
  int K;
  int tiles_per_head;       // window: ceil(n / T)
  const int32_t* qidx;      // asymmetric group pass: query slot -> token position
  const int32_t* groups;    // soft gate: [n, top_k] memberships
  float soft_b0, soft_b1;   // soft gate: far-pair logit bias without / with a shared group,
                            // in raw q.k units (log sigmoid(lambda * (share - 1/2)) / scale)
  float soft_shift;         // soft gate with bias rows: the row shift, max(b0, b1), natural log
  int soft_mark_none;       // soft gate with bias rows: the rows mark pairs sharing no group
                            // (b1 > b0, lambda > 0), else pairs sharing one
};

constexpr int KT = 64;  // keys per kv tile

// K and V tiles live in LDS row-major, 2*DH bytes per key row, with the 16-byte chunks of row r
// permuted by chunk ^ swz(r) (swz in focus_internal.hpp).

// Ownership bias rows (group pass, MKS > 0): mrow[j][key][t] is bf16 1.0 when the key shares a
// lower group with query token 16 j + t of the tile, else 0. One extra MFMA k-step per 16
// tokens multiplies them with a per-lane one-hot of the row's token scaled by -2^100, which
// pushes every excluded score to about -2^100 before the softmax sees it.
template <int DH, int MKS>
struct FlashSmem {
  __bf16 k[KT * DH];
  __bf16 v[KT * DH];
  __bf16 mrow[MKS > 0 ? MKS : 1][KT][16];
  int kpos[KT];
  int klow[3][KT];
};

// Tile classes seen by one wave.
enum { kSkip = 0, kEdge = 1, kFar = 2, kFull = 3 };


constexpr float kMaskBias = -0x1p100f;   // ownership bias of an excluded pair (before scaling)
constexpr float kMaskFloor = -0x1p99f;   // raw row maxima below this are fully masked rows

// NLOW = top_k - 1: lower groups per membership that matter for the ownership rule (group
// pass), and top_k - 1 for the window pass, whose merge reads top_k group parts per token.
// MKS = 16-token k-steps of the MFMA ownership bias (0: per-element compare instead).
// SOFT (window pass only): the training-time soft gate instead of the hard pair rule: every
// causal pair is attended, far pairs with a logit bias that depends on whether the two tokens
// share a group (the tile's key groups are staged in LDS like the group pass's key records),
// and there are no group parts to merge. SMASK (soft gate, T * top_k <= 32): each key of a tile
// gets a 32-bit mask of the query tokens' group slots (slot c*T + t: group c of token t) that
// it holds, so the per-element test is one AND with the row's own slots.
// ASYM (group pass, asymmetric top-k): query slots come from the bucket of the groups each
// token looks at and key slots from a second bucket in which every token sits in one group,
// so the two slot spaces differ: query positions come from qidx, the plan gives each item's
// key range, tile classes compare positions only, and no ownership rule is needed (a key has
// one group, so each far pair meets exactly one of the query's memberships).
template <int DH, bool GROUP, int NLOW, int MKS, bool SOFT = false, bool SMASK = false,
          bool ASYM = false>
__global__ __launch_bounds__(256, 2) void flash_kernel(const FlashArgs a) {
  using Smem = FlashSmem<DH, (SOFT && MKS > 0) ? 1 : MKS>;  // soft gate: one share row block
  constexpr int CH = DH / 8;             // 16-byte chunks per key row
  constexpr int ROWS_PER_INST = 64 / CH; // key rows one wave-wide 1 KB LDS load covers
  constexpr int INSTS = KT / ROWS_PER_INST / 4;  // per wave, for each of K and V
  constexpr int NS = DH / 16;            // MFMA k-steps over the head dimension
  constexpr int ND = DH / 32;            // 32-wide output tiles over the head dimension
  constexpr int RB = 2 * DH;             // bytes per key row
  static_assert(MKS == 0 || (GROUP && NLOW > 0) || (SOFT && SMASK && MKS == 3),
                "bias rows: the group pass's ownership rule, or the soft gate's share term");
  constexpr bool SBIAS = SOFT && MKS > 0;  // soft gate: far-pair share term on the MFMA
  static_assert(NLOW >= 0 && NLOW <= 3, "top_k is 1 to 4");
  static_assert(!(SOFT && GROUP), "the soft gate runs on the window pass");
  static_assert(!SMASK || SOFT, "slot masks belong to the soft gate");
  static_assert(!ASYM || (GROUP && NLOW == 0 && MKS == 0), "asymmetric: group pass, one key group");
  __shared__ __attribute__((aligned(1024))) Smem smem[2];  // double buffer: one barrier per tile
  __shared__ __attribute__((aligned(16))) int qlow_s[3][32];  // MKS > 0: query tokens' lower groups, -2 if none
  __shared__ __attribute__((aligned(16))) int qslot_s[SMASK ? 32 : 1];  // SMASK: slot groups, -2 if none

  const int tid = threadIdx.x, l = tid & 63, jq = l & 31, hg = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---------------------------------------------------------------- work item
  const int W = GROUP ? a.w_max : a.tiles_per_head;
  const int64_t comb = xcd_remap(blockIdx.x, (int64_t)a.Hkv * W);
  if (comb < 0) return;
  const int h = (int)(comb / W);
  const int item = (int)(comb - (int64_t)h * W);
  const int window = a.window;

  int q0, q1, kv_lo, kv_hi, ntiles;  // slots (group) or tokens (window); all below 2^31
  if constexpr (GROUP) {
    const i32x4_t pl = a.plan[item];  // one load replaces the searches of the work item
    q0 = pl[0];
    q1 = pl[1];
    kv_lo = pl[2];
    if constexpr (ASYM) {
      kv_hi = pl[3];
      ntiles = kv_hi >= kv_lo ? (kv_hi - kv_lo) / KT + 1 : 0;
    } else {
      kv_hi = q1 - 1;  // last key slot any query of the tile may see
      ntiles = pl[3];
    }
    if (q0 >= q1) return;
  } else {
    q0 = item * a.T;
    q1 = (int)min((int64_t)q0 + a.T, a.n);
    kv_lo = SOFT ? 0 : max(q0 - window + 1, 0);
    kv_hi = q1 - 1;  // last key index any query of the tile may see
  }

  // ---------------------------------------------------------------- this lane's query row
  const int r = wave * 32 + jq;
  const int head_local = r / a.T, tok_local = r % a.T;
  const int hq = h * a.G + head_local;
  const int qi = q0 + tok_local;
  const bool qvalid = qi < q1;
  const int wt0 = (wave * 32) % a.T;
  const int wtn = a.T < 32 ? a.T : 32;
  const int wq_lo = q0 + wt0;
  const int wq_hi = min(q0 + wt0 + wtn, q1) - 1;
  const bool wave_active = wq_hi >= wq_lo;

  int qpos = 0, wpos_lo = 0, wpos_hi = 0;
  int qlow[3] = {-2, -2, -2};
  if constexpr (ASYM) {
    if (qvalid) qpos = a.qidx[qi];
    if (wave_active) {
      wpos_lo = a.qidx[wq_lo];
      wpos_hi = a.qidx[wq_hi];
    }
  } else if constexpr (GROUP) {
    if (qvalid) {
      i32x4_t qinfo = a.kinfo[qi];
      qpos = qinfo[0];
#pragma unroll
      for (int c = 0; c < NLOW; ++c) qlow[c] = qinfo[1 + c] >= 0 ? qinfo[1 + c] : -2;
    }
    if (wave_active) {
      wpos_lo = a.kinfo[wq_lo][0];
      wpos_hi = a.kinfo[wq_hi][0];
    }
  } else {
    qpos = qi;
  }

  // window pass: the token's membership slots load with the query row, their group LSEs with
  // the first tile, so the merge epilogue starts with both in registers
  constexpr int TK = NLOW + 1;
  int srow[GROUP ? 1 : TK];
  float Lr[GROUP ? 1 : TK];
  if constexpr (!GROUP) {
#pragma unroll
    for (int r = 0; r < TK; ++r) srow[r] = (qvalid && !SOFT) ? a.slot[(int64_t)qi * TK + r] : -1;
  }
  // soft gate: this row's token's groups (-2 where none or out of range: never matches a key)
  int qg[SOFT ? TK : 1];
  uint32_t qmask = 0;  // SMASK: this row's token's group slots
  if constexpr (SOFT) {
#pragma unroll
    for (int c = 0; c < TK; ++c) {
      const int g = qvalid ? a.groups[(int64_t)qi * TK + c] : -2;
      qg[c] = (g >= 0 && g < a.K) ? g : -2;
      if (SMASK && qg[c] >= 0) qmask |= 1u << (c * a.T + tok_local);
    }
  }

  bf16x8_t qreg[NS];
  {
    const int qrow = qvalid ? (GROUP ? qpos : qi) : 0;
    const uint16_t* qp = a.q + ((int64_t)qrow * a.Hq + hq) * DH + 8 * hg;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qreg[s] = qvalid ? *(const bf16x8_t*)(qp + 16 * s) : bf16x8_t{};
  }

  // query side of the ownership bias: -2^100 at this row's token (T <= 32: token = jq % T)
  bf16x8_t qm[MKS > 0 ? MKS : 1];
  // soft gate with bias rows: every logit of a row is shifted by minus the larger far-pair bias
  // (lse adds it back), so the far pairs that carry the smaller bias need c = smaller - larger
  // (<= 0) and the others nothing: the large offsets land on suppressed pairs and the dominant
  // logits stay exact at any lambda. The rows mark the pairs that carry c; the MFMA adds c as
  // its three bf16 parts (8 + 8 + 8 significand bits hold all of fp32, so the sum is c
  // exactly), one k-step each over the same marked rows
  float soft_c = 0.f, soft_sh = 0.f;
  if constexpr (SBIAS) {
    soft_sh = a.soft_mark_none ? a.soft_b1 : a.soft_b0;
    const float c = a.soft_mark_none ? a.soft_b0 - a.soft_b1 : a.soft_b1 - a.soft_b0;
    const __bf16 c0 = to_bf16(c);
    const __bf16 c1 = to_bf16(c - (float)c0);
    const __bf16 c2 = to_bf16(c - (float)c0 - (float)c1);
    soft_c = c;
    const int tw = jq % a.T;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool hit = 8 * hg + e == tw;
      qm[0][e] = hit ? c0 : (__bf16)0.f;
      qm[1][e] = hit ? c1 : (__bf16)0.f;
      qm[2][e] = hit ? c2 : (__bf16)0.f;
    }
  } else if constexpr (MKS > 0) {
    const int tw = jq % a.T;
#pragma unroll
    for (int j = 0; j < MKS; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) qm[j][e] = (__bf16)(16 * j + 8 * hg + e == tw ? kMaskBias : 0.f);
  }
  // the tile's query tokens' records (for the lower-group table written after the first wait)
  i32x4_t tok_rec = {0, -2, -2, -2};
  if constexpr (GROUP && MKS > 0) {
    if (tid < 32 && tid < a.T && q0 + tid < q1) tok_rec = a.kinfo[q0 + tid];
  }

  // ---------------------------------------------------------------- kv tile range
  if constexpr (!GROUP) ntiles = (SOFT || window > 0) ? (kv_hi - kv_lo) / KT + 1 : 0;

  f32x16_t oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---------------------------------------------------------------- per-lane LDS addresses
  // Byte offsets from smem[0]; the buffer parity, the row block (32 keys for K, 16 for V) and
  // the mask k-step are added as instruction immediates.
  const char* lds = (const char*)smem;
  uint32_t krd[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    krd[s] = (uint32_t)(jq * RB + (((2 * s + hg) ^ (swz(jq) % CH)) * 16));
  // V through the transposing read: in each 16-lane group lane j receives element j%4 of the
  // 8-byte row slice read by lane 4e + j/4 (e = 0..3). Lane (16g + 4e + m) reads key row
  // 16 kq + 8 rr + 4 hg + e at dims 32 d + 16 (g%2) + 4m and so receives 4 keys of dim
  // 32 d + lane%32.
  const int e4 = (l & 15) >> 2, m4 = l & 3, g2 = (l >> 4) & 1;
  uint32_t vrd[ND][2];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 4 * hg + e4 + 8 * rr;
      const int c16 = 4 * d + 2 * g2 + (m4 >> 1);
      vrd[d][rr] = (uint32_t)(offsetof(Smem, v) + row * RB + ((c16 ^ (swz(row) % CH)) * 16) +
                              (m4 & 1) * 8);
    }
  const uint32_t mrd = (uint32_t)(offsetof(Smem, mrow) + jq * 32 + hg * 16);

  // ---------------------------------------------------------------- tile loads
  // Wave w moves key rows [w*KT/4, (w+1)*KT/4) of K and of V straight into LDS with
  // global_load_lds_dwordx4: one instruction fills 1 KB of LDS, lane L landing at byte 16*L,
  // i.e. row L / CH of the instruction's block, swizzled position L % CH, so lane L fetches the
  // global chunk (L % CH) ^ swz(row). Per-lane byte offsets are fixed; the tile moves a uniform
  // base.
  const uint32_t kstride_b = (uint32_t)a.Hkv * RB;  // bytes between consecutive key rows
  const char* khead = (const char*)a.k + (int64_t)h * RB;
  const char* vhead = (const char*)a.v + (int64_t)h * RB;
  uint32_t gofs[INSTS], gchunk[INSTS];
  int lrow[INSTS];
#pragma unroll
  for (int i = 0; i < INSTS; ++i) {
    lrow[i] = (wave * INSTS + i) * ROWS_PER_INST + l / CH;
    gchunk[i] = (uint32_t)(((l % CH) ^ (swz(lrow[i]) % CH)) * 16);
    gofs[i] = (uint32_t)lrow[i] * kstride_b + gchunk[i];
  }
  i32x4_t ireg = {0x7fffffff, -1, -1, -1};
  const int kkey = (MKS > 0 || SMASK) ? (tid >> 2) : tid;  // key whose record this thread loads

  auto issue_tile = [&](int ks, Smem& sb) __attribute__((always_inline)) {
    const char* kb = khead + (int64_t)ks * kstride_b;  // uniform tile base
    const char* vb = vhead + (int64_t)ks * kstride_b;
    const int nrow = kv_hi - ks;  // rows 0..nrow of the tile are valid
    if (nrow >= KT - 1) {
#pragma unroll
      for (int i = 0; i < INSTS; ++i) {
        dma16(kb, gofs[i], (char*)sb.k + (wave * INSTS + i) * 1024);
        dma16(vb, gofs[i], (char*)sb.v + (wave * INSTS + i) * 1024);
      }
    } else {
      // rows past the end re-read the last valid row; the mask drops them
#pragma unroll
      for (int i = 0; i < INSTS; ++i) {
        const uint32_t off = lrow[i] <= nrow ? gofs[i] : (uint32_t)nrow * kstride_b + gchunk[i];
        dma16(kb, off, (char*)sb.k + (wave * INSTS + i) * 1024);
        dma16(vb, off, (char*)sb.v + (wave * INSTS + i) * 1024);
      }
    }
    if constexpr (GROUP) {
      // load only the record fields in use: a partly dead load destination would make the
      // compiler wait for this load wherever it reuses those registers
      if (kkey < KT) {
        const int* rec = (const int*)&a.kinfo[ks + kkey];
        if constexpr (NLOW == 0) {
          ireg[0] = kkey <= nrow ? rec[0] : 0x7fffffff;
        } else if constexpr (NLOW == 1) {
          const i32x2_t t = kkey <= nrow ? *(const i32x2_t*)rec : i32x2_t{0x7fffffff, -1};
          ireg[0] = t[0];
          ireg[1] = t[1];
        } else if constexpr (NLOW == 2) {
          const bool in = kkey <= nrow;
          ireg[0] = in ? rec[0] : 0x7fffffff;
          ireg[1] = in ? rec[1] : -1;
          ireg[2] = in ? rec[2] : -1;
        } else {
          ireg = kkey <= nrow ? *(const i32x4_t*)rec : i32x4_t{0x7fffffff, -1, -1, -1};
        }
      }
    }
    if constexpr (SOFT) {
      // the key's groups (-1 where none, out of range or past the last key)
      if (kkey < KT) {
#pragma unroll
        for (int c = 0; c < TK; ++c) {
          const int g = kkey <= nrow ? a.groups[(int64_t)(ks + kkey) * TK + c] : -1;
          ireg[c] = (g >= 0 && g < a.K) ? g : -1;
        }
      }
    }
  };
  // Waits for this wave's loads go through the builtin (not inline asm), so the compiler's own
  // wait tracking sees them. They are placed on every path into the tile loop and at the end of
  // every step, so no load can look outstanding at the loop head: the compiler would otherwise
  // wait for the prefetch of the next tile before computing on the current one.
  auto finish_tile = [&](Smem& sb) __attribute__((always_inline)) {  // loads landed: publish
    if constexpr (GROUP && MKS > 0) {
      // thread (key, quarter tq) writes the bias row entries of tokens [tq*TPT, (tq+1)*TPT)
      constexpr int TPT = MKS * 4;
      const int tq = tid & 3;
      if (tq == 0) sb.kpos[kkey] = ireg[0];
      uint32_t word[TPT / 2];
#pragma unroll
      for (int u2 = 0; u2 < TPT / 2; ++u2) word[u2] = 0;
#pragma unroll
      for (int c1 = 0; c1 < NLOW; ++c1) {
#pragma unroll
        for (int u4 = 0; u4 < TPT / 4; ++u4) {
          const i32x4_t ql = *(const i32x4_t*)&qlow_s[c1][tq * TPT + 4 * u4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bool hit = false;
#pragma unroll
            for (int c2 = 0; c2 < NLOW; ++c2) hit = hit || ql[e] == ireg[1 + c2];
            const int u = 4 * u4 + e;
            word[u >> 1] |= hit ? (0x3F80u << (16 * (u & 1))) : 0u;
          }
        }
      }
      const int t0 = tq * TPT;
      char* dst = (char*)&sb.mrow[t0 >> 4][kkey][t0 & 15];
      if constexpr (TPT == 4) {
        *(i32x2_t*)dst = i32x2_t{(int)word[0], (int)word[1]};
      } else {
        *(i32x4_t*)dst = i32x4_t{(int)word[0], (int)word[1], (int)word[2], (int)word[3]};
      }
    } else if constexpr (SMASK) {
      // thread (key, quarter tq) matches the key's groups against slots [8 tq, 8 tq + 8); the
      // quad's four parts are OR-ed on the VALU and kpos holds the key's slot mask
      const int tq = tid & 3;
      uint32_t m = 0;
#pragma unroll
      for (int u4 = 0; u4 < 2; ++u4) {
        const i32x4_t qs = *(const i32x4_t*)&qslot_s[8 * tq + 4 * u4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bool hit = false;
#pragma unroll
          for (int c = 0; c < TK; ++c) hit = hit || (qs[e] >= 0 && qs[e] == ireg[c]);
          m |= hit ? 1u << (8 * tq + 4 * u4 + e) : 0u;
        }
      }
      m |= (uint32_t)dpp_move_i<0xB1>((int)m);
      m |= (uint32_t)dpp_move_i<0x4E>((int)m);
      if (tq == 0) sb.kpos[kkey] = (int)m;
      if constexpr (SBIAS) {
        // marked rows (T <= 16): thread tq writes tokens [4 tq, 4 tq + 4) of the key's row, 1.0
        // where the pair carries c (shares a group, or shares none when soft_mark_none);
        // entries of tokens past T are never selected by a row's one-hot
        const bool mark_none = a.soft_mark_none != 0;
        uint32_t w2[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * tq + e;
          uint32_t tm = 0;  // slots of token t
#pragma unroll
          for (int c = 0; c < TK; ++c) tm |= (t < a.T && c * a.T + t < 32) ? 1u << (c * a.T + t) : 0u;
          w2[e >> 1] |= (((m & tm) != 0u) != mark_none) ? (0x3F80u << (16 * (e & 1))) : 0u;
        }
        const i32x2_t wv = {(int)w2[0], (int)w2[1]};
        *(i32x2_t*)&sb.mrow[0][kkey][4 * tq] = wv;
      }
    } else if constexpr (GROUP || SOFT) {  // soft gate: kpos / klow hold the key's groups
      if (tid < KT) {
        sb.kpos[tid] = ireg[0];
#pragma unroll
        for (int c = 0; c < NLOW; ++c) sb.klow[c][tid] = ireg[1 + c];
      }
    }
  };

  // ---------------------------------------------------------------- one kv tile
  auto compute_tile = [&](int ks, const Smem& sm, const uint32_t par) __attribute__((always_inline)) {
    if (!wave_active) return;
    const int k_last = ks + KT - 1;
    int cls;
    if constexpr (GROUP) {
      const bool whole = k_last <= kv_hi;
      const int kp_first = __builtin_amdgcn_readfirstlane(sm.kpos[0]);
      const int kp_last = whole ? __builtin_amdgcn_readfirstlane(sm.kpos[KT - 1]) : 0x7fffffff;
      if constexpr (ASYM) {  // key and query slots are separate: positions decide
        if (wpos_hi - kp_first < window) cls = kSkip;
        else if (whole && wpos_lo - kp_last >= window) cls = kFull;
        else cls = kEdge;
      } else {
        if (ks > wq_hi || wpos_hi - kp_first < window) cls = kSkip;
        else if (whole && k_last <= wq_lo && wpos_lo - kp_last >= window)
          cls = (NLOW == 0 || MKS > 0) ? kFull : kFar;
        else cls = kEdge;
      }
    } else if constexpr (SBIAS) {
      if (ks > wq_hi) cls = kSkip;
      else if (wq_lo - k_last >= window) cls = kFull;  // all pairs far and causal: rows only
      else cls = kEdge;
    } else {
      if (ks > wq_hi || (!SOFT && wq_lo - k_last >= window)) cls = kSkip;
      else if (k_last <= wq_lo && wq_hi - ks < window) cls = kFull;
      else cls = kEdge;  // soft gate: also every tile with far pairs
    }
    if (cls == kSkip) return;

    // ------------------------------------------------------------ S^T = K Q^T (+ bias)
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
    if constexpr (SBIAS) {
      // one marked row block, one k-step per part of c; only in tiles whose pairs are all far
      // (edge tiles add the term per element, so near pairs never carry it)
      if (cls == kFull) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t mf = *(const bf16x8_t*)(lds + mrd + par + kb * 32 * 32);
#pragma unroll
          for (int j = 0; j < MKS; ++j)
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mf, qm[j], sacc[kb], 0, 0, 0);
        }
      }
    } else if constexpr (MKS > 0) {
#pragma unroll
      for (int j = 0; j < MKS; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t mf = *(const bf16x8_t*)(lds + mrd + par + (j * KT + kb * 32) * 32);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mf, qm[j], sacc[kb], 0, 0, 0);
        }
    }
    // K fragments are read KPF k-steps ahead of their MFMAs (a rolling window of registers), so
    // LDS latency overlaps the MFMAs of the steps before
    constexpr int KPF = 2;
    bf16x8_t kf[KPF + 1][2];
#pragma unroll
    for (int s = 0; s < KPF; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[s][kb] = *(const bf16x8_t*)(lds + krd[s] + par + kb * 32 * RB);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + KPF < NS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kf[(s + KPF) % (KPF + 1)][kb] = *(const bf16x8_t*)(lds + krd[s + KPF] + par + kb * 32 * RB);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % (KPF + 1)][kb], qreg[s], sacc[kb], 0, 0, 0);
    }
    {
      // keep 2 * KPF operand reads in flight: the scheduler would otherwise sink each read
      // next to its MFMA (masks: 0x100 LDS read, 0x008 MFMA); the bias step's operands, when
      // present, are read first like the K fragments
      constexpr int NM = 2 * (NS + (SBIAS ? 0 : MKS));  // MFMAs of the S product, one LDS read each
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KPF, 0);
#pragma unroll
      for (int i = 0; i < NM - 2 * KPF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KPF, 0);
    }

    // ------------------------------------------------------------ mask
    // accumulator element v of tile kb is key kb*32 + 8*(v/4) + 4*hg + v%4 of this tile: four
    // consecutive keys per group of four elements, read from LDS as one 16-byte vector
    if (cls != kFull) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int kk0 = kb * 32 + 8 * q4 + 4 * hg;
          bool ok[4] = {true, true, true, true};
          if constexpr (GROUP) {
            if (cls == kEdge) {
              const i32x4_t kp = *(const i32x4_t*)&sm.kpos[kk0];
#pragma unroll
              for (int e = 0; e < 4; ++e) ok[e] = qpos - kp[e] >= window;
            }
            if constexpr (MKS == 0) {
#pragma unroll
              for (int c2 = 0; c2 < NLOW; ++c2) {
                const i32x4_t kl = *(const i32x4_t*)&sm.klow[c2][kk0];
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                  for (int c1 = 0; c1 < NLOW; ++c1) ok[e] = ok[e] && kl[e] != qlow[c1];
              }
            }
          } else if constexpr (SOFT) {
            // causal; far pairs get the gate's bias, by whether the tokens share a group
            bool share[4] = {false, false, false, false};
            if constexpr (SMASK) {
              const i32x4_t km = *(const i32x4_t*)&sm.kpos[kk0];
#pragma unroll
              for (int e = 0; e < 4; ++e) share[e] = ((uint32_t)km[e] & qmask) != 0u;
            } else {
#pragma unroll
              for (int c2 = 0; c2 < TK; ++c2) {
                const i32x4_t kg = c2 == 0 ? *(const i32x4_t*)&sm.kpos[kk0]
                                           : *(const i32x4_t*)&sm.klow[c2 > 0 ? c2 - 1 : 0][kk0];
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                  for (int c1 = 0; c1 < TK; ++c1) share[e] = share[e] || kg[e] == qg[c1];
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int dd = qi - (ks + kk0 + e);
              ok[e] = dd >= 0;
              if constexpr (SBIAS) {  // near pairs take the row shift, far pairs the marked term
                const bool marked = share[e] != (a.soft_mark_none != 0);
                sacc[kb][4 * q4 + e] += dd < window ? -soft_sh : (marked ? soft_c : 0.f);
              } else {
                if (dd >= window) sacc[kb][4 * q4 + e] += share[e] ? a.soft_b1 : a.soft_b0;
              }
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)  // 0 <= d < window as one unsigned compare
              ok[e] = (uint32_t)(qi - (ks + kk0 + e)) < (uint32_t)window;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!ok[e]) sacc[kb][4 * q4 + e] = -INFINITY;
        }
    }

    // ------------------------------------------------------------ online softmax
    // row maximum: four independent chains of 8 (v_max3 steps), then over the lane pair
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) mx[2 * kb + (vi >> 3)] = fmaxf(mx[2 * kb + (vi >> 3)], sacc[kb][vi]);
    float tmax = pair32_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
    if constexpr (GROUP && MKS > 0) tmax = tmax < kMaskFloor ? -INFINITY : tmax;
    tmax *= a.sl2;
    // Lazy rescale: the reference max moves only when a row's max exceeds it by more than
    // kLazy (log2 units), so p = exp2(x - m_ref) stays below 2^kLazy and O is rescaled on
    // the first tile and almost never after. lse uses the same reference, so it is exact.
    constexpr float kLazy = 8.f;
    const bool bump = tmax > m_run + kLazy;
    if (__any(bump)) {
      const float m_next = bump ? tmax : m_run;
      const float alpha = m_next == -INFINITY ? 1.f : fast_exp2(m_run - m_next);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
      m_run = m_next;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8_t pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) {
        const float p = fast_exp2(__builtin_fmaf(sacc[kb][vi], a.sl2, -m_use));
        psum[vi & 3] += p;
        pb[kb * 2 + (vi >> 3)][vi & 7] = to_bf16(p);
      }
    l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);

    // ------------------------------------------------------------ O^T += V^T P^T
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const uint32_t kqo = ((kq >> 1) * 32 + (kq & 1) * 16) * RB;
#pragma unroll
      for (int d = 0; d < ND; ++d) {  // consecutive MFMAs feed independent accumulators
        bf16x4_t half[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          typedef short v4i16_t __attribute__((ext_vector_type(4)));
          const char* src = lds + vrd[d][rr] + par + kqo;
          v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(lds_void_t*)src);
          half[rr] = __builtin_bit_cast(bf16x4_t, t);
        }
        bf16x8_t vf = {half[0][0], half[0][1], half[0][2], half[0][3],
                       half[1][0], half[1][1], half[1][2], half[1][3]};
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kq], oacc[d], 0, 0, 0);
      }
    }
  };

  // group pass: the first tile's copies go out with the query-row loads and one wait covers
  // both (measured neutral to slightly worse for the window pass, which keeps two waits)
  if constexpr (!GROUP) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
    for (int r = 0; r < TK; ++r)
      Lr[r] = (!SOFT && srow[r] >= 0) ? a.lseg[(int64_t)srow[r] * a.Hq + hq] : -INFINITY;
  }
  if (ntiles > 0) issue_tile(kv_lo, smem[0]);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if constexpr (GROUP && MKS > 0) {
    if (tid < 32) {
#pragma unroll
      for (int c = 0; c < NLOW; ++c) qlow_s[c][tid] = tok_rec[1 + c] >= 0 ? tok_rec[1 + c] : -2;
    }
    __syncthreads();  // qlow_s is read by every tile's bias rows
  }
  if constexpr (SMASK) {
    if (tid < 32) {  // slot tid: group tid / T of token tid % T (-2 if none or past the tiles)
      const int c = tid / a.T, tt = tid % a.T;
      int g = -2;
      if (c < TK && q0 + tt < q1) {
        g = a.groups[(int64_t)(q0 + tt) * TK + c];
        g = (g >= 0 && g < a.K) ? g : -2;
      }
      qslot_s[tid] = g;
    }
    __syncthreads();  // qslot_s is read by every tile's key masks
  }
  if (ntiles > 0) {
    finish_tile(smem[0]);
    __syncthreads();
  }

  // unrolled by two so each copy addresses one LDS buffer through immediates
  auto step = [&](int it, auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    const int ks = kv_lo + it * KT;
    if (it + 1 < ntiles) issue_tile(ks + KT, smem[P ^ 1]);  // lands during compute
    compute_tile(ks, smem[P], (uint32_t)(P * sizeof(Smem)));
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (it + 1 < ntiles) {
      finish_tile(smem[P ^ 1]);
      __syncthreads();  // the next tile is in LDS and every wave is done with this one
    }
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
  }

  // ---------------------------------------------------------------- epilogue
  // Results leave through LDS. Each lane writes its row's values in the accumulator layout and
  // reads back 16 consecutive bytes of one row, so every global access of the wave covers whole
  // rows: in the accumulator layout one wave-wide access would touch 32 rows at 16 bytes each,
  // and the vector memory path spends a cycle per cache line touched. Lanes of rows without a
  // query stay active (shuffles and the window pass's barrier) but store nothing.
  const float l_tot = pair32_sum(l_run);
  const float L_own = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  constexpr int RPI = 64 / CH;  // rows per transposed access (CH lanes per row)
  const int cl = l % CH;        // this lane's 16-byte chunk of the row in transposed accesses
  // Oᵀ accumulator layout: lane holds dims d*32 + 8*g4 + 4*hg + 0..3 of its query row
  if constexpr (GROUP) {
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    // smem[ntiles & 1] is not the last tile's buffer: every wave finished reading it before the
    // loop's last barrier and no copy targets it since, so it needs no further barrier
    char* ep = (char*)&smem[ntiles & 1] + wave * (32 * RB);  // 32 fp16 rows of 2 DH bytes
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f16x4_t x = {(_Float16)(oacc[d][4 * g4] * inv), (_Float16)(oacc[d][4 * g4 + 1] * inv),
                           (_Float16)(oacc[d][4 * g4 + 2] * inv),
                           (_Float16)(oacc[d][4 * g4 + 3] * inv)};
        *(f16x4_t*)(ep + jq * RB + (((4 * d + g4) ^ (jq % CH)) * 16) + hg * 8) = x;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + l / CH;
      const int rr = wave * 32 + row;
      const int qr = q0 + rr % a.T;
      const i32x4_t x = *(const i32x4_t*)(ep + row * RB + ((cl ^ (row % CH)) * 16));
      if (qr < q1)
        *(i32x4_t*)(a.og + ((int64_t)qr * a.Hq + h * a.G + rr / a.T) * DH + 8 * cl) = x;
    }
    if (qvalid && hg == 0) a.lseg[(int64_t)qi * a.Hq + hq] = L_own;
  } else {
    // merge the window part with this token's group parts by log-sum-exp, in token order;
    // NLOW + 1 = top_k group parts per token
    float M = L_own;
#pragma unroll
    for (int r = 0; r < TK; ++r) M = fmaxf(M, Lr[r]);
    float w_own = 0.f, den = 0.f, cr[TK];
#pragma unroll
    for (int r = 0; r < TK; ++r) cr[r] = 0.f;
    if (M != -INFINITY) {
      w_own = L_own == -INFINITY ? 0.f : __expf(L_own - M);
      den = w_own;
#pragma unroll
      for (int r = 0; r < TK; ++r) {
        cr[r] = Lr[r] == -INFINITY ? 0.f : __expf(Lr[r] - M);
        den += cr[r];
      }
    }
    const float inv_den = den > 0.f ? 1.f / den : 0.f;
    const float c_own = l_tot > 0.f ? w_own * inv_den / l_tot : 0.f;
#pragma unroll
    for (int r = 0; r < TK; ++r) cr[r] *= inv_den;

    // group parts in the transposed layout, read in batches of NB rows per lane (all rows at
    // top_k <= 2) whose loads are all issued before any is used; a row without that part reads
    // slot 0 and its weight 0 leaves the sum untouched
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    constexpr int NI = 32 / RPI;
    constexpr int NB = TK * NI <= 16 ? NI : NI / 2;
    static_assert(NB * TK <= 16, "at most 16 loads in flight per lane");
    char* ep = (char*)smem + wave * (32 * 4 * DH);
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += NB) {
      f16x8_t gx[NB][TK];
      float gc[NB][TK];
#pragma unroll
      for (int ib = 0; ib < NB; ++ib) {
        const int row = (i0 + ib) * RPI + l / CH;
        const int hr = h * a.G + (wave * 32 + row) / a.T;
#pragma unroll
        for (int r = 0; r < TK; ++r) {
          gc[ib][r] = __shfl(cr[r], row, kWave);  // every lane takes part in the shuffles
          const int sl = max(__shfl(srow[r], row, kWave), 0);
          if constexpr (SOFT) gx[ib][r] = f16x8_t{};  // no group parts (their weight is 0)
          else gx[ib][r] = *(const f16x8_t*)(a.og + ((int64_t)sl * a.Hq + hr) * DH + 8 * cl);
        }
      }
      if (i0 == 0) {
        // the window part goes through LDS in fp32: 32 rows of 4 DH bytes per wave, spread over
        // both tile buffers once every wave is done with them
        static_assert(4 * 32 * 4 * DH <= 2 * sizeof(Smem), "merge staging exceeds the tile buffers");
        __syncthreads();
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4_t x = f32x4_t{oacc[d][4 * g4], oacc[d][4 * g4 + 1], oacc[d][4 * g4 + 2],
                                      oacc[d][4 * g4 + 3]} * c_own;
            *(f32x4_t*)(ep + jq * 4 * DH + (((8 * d + 2 * g4 + hg) ^ (jq & 15)) * 16)) = x;
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
#pragma unroll
      for (int ib = 0; ib < NB; ++ib) {
        const int row = (i0 + ib) * RPI + l / CH;
        const int rr = wave * 32 + row;
        const int qr = q0 + rr % a.T;
        const int hr = h * a.G + rr / a.T;
        f32x4_t lo = *(const f32x4_t*)(ep + row * 4 * DH + (((2 * cl) ^ (row & 15)) * 16));
        f32x4_t hi = *(const f32x4_t*)(ep + row * 4 * DH + (((2 * cl + 1) ^ (row & 15)) * 16));
#pragma unroll
        for (int r = 0; r < TK; ++r) {
          const float c = gc[ib][r];
          const f16x8_t x = gx[ib][r];
          const f32x4_t nlo = lo + c * f32x4_t{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
          const f32x4_t nhi = hi + c * f32x4_t{(float)x[4], (float)x[5], (float)x[6], (float)x[7]};
          lo = c != 0.f ? nlo : lo;
          hi = c != 0.f ? nhi : hi;
        }
        if (qr < q1) {
          const bf16x8_t o8 = {to_bf16(lo[0]), to_bf16(lo[1]), to_bf16(lo[2]), to_bf16(lo[3]),
                               to_bf16(hi[0]), to_bf16(hi[1]), to_bf16(hi[2]), to_bf16(hi[3])};
          *(bf16x8_t*)(a.out + ((int64_t)qr * a.Hq + hr) * DH + 8 * cl) = o8;
        }
      }
    }
    if (qvalid && hg == 0)
      a.lse[(int64_t)qi * a.Hq + hq] =
          den > 0.f ? M + __logf(den) + (SBIAS ? a.soft_shift : 0.f) : -INFINITY;
  }
}

template <bool GROUP, int NLOW, int MKS, bool SOFT = false, bool SMASK = false, bool ASYM = false>
static void flash_dispatch_dh(const FlashArgs& fa, int dh, int64_t blocks, hipStream_t stream) {
  if (dh == 128)
    hipLaunchKernelGGL((flash_kernel<128, GROUP, NLOW, MKS, SOFT, SMASK, ASYM>), dim3(blocks),
                       dim3(256), 0, stream, fa);
  else
    hipLaunchKernelGGL((flash_kernel<64, GROUP, NLOW, MKS, SOFT, SMASK, ASYM>), dim3(blocks),
                       dim3(256), 0, stream, fa);
}

template <int NLOW>
static void flash_dispatch_group(const FlashArgs& fa, int dh, int mks, int64_t blocks,
                                 hipStream_t stream) {
  if (mks == 1) flash_dispatch_dh<true, NLOW, 1>(fa, dh, blocks, stream);
  else if (mks == 2) flash_dispatch_dh<true, NLOW, 2>(fa, dh, blocks, stream);
  else flash_dispatch_dh<true, NLOW, 0>(fa, dh, blocks, stream);
}

hipError_t launch_group_attention(const uint16_t* q, const uint16_t* kg, const uint16_t* vg,
                                  const int32_t* offsets, const int32_t* tile_pre,
                                  const int32_t* kinfo, const int32_t* plan, const AttnShape& s,
                                  _Float16* og, float* lseg, hipStream_t stream) {
  FlashArgs fa{};
  fa.q = q;
  fa.k = kg;
  fa.v = vg;
  fa.og = og;
  fa.lseg = lseg;
  fa.n = s.n;
  fa.Hq = s.Hq;
  fa.Hkv = s.Hkv;
  fa.G = s.G;
  fa.T = attn_tile_tokens(s.G);
  fa.window = (int)(s.window < s.n ? s.window : s.n);
  fa.sl2 = s.scale * kLog2e;
  fa.seg_off = offsets;
  fa.tile_pre = tile_pre;
  fa.kinfo = (const i32x4_t*)kinfo;
  fa.plan = (const i32x4_t*)plan;
  fa.K = s.K;
  fa.top_k = s.top_k;
  // upper bound on the tiles of all segments: sum of ceil(size / T) <= ceil(nk / T) + K
  fa.w_max = attn_work_items(s.nk, fa.T, s.K);
  const int64_t blocks = xcd_grid((int64_t)s.Hkv * fa.w_max);
  if (blocks <= 0) return hipSuccess;
  // The ownership rule runs as an MFMA bias when a wave's rows span at most 32 tokens and the
  // scaled bias (-2^100 * scale * log2 e) still drives exp2 to zero; else per-element compares.
  const int mks = (fa.T <= 32 && fa.sl2 >= 0x1p-60f) ? (fa.T <= 16 ? 1 : 2) : 0;
  switch (s.top_k) {
    case 1: flash_dispatch_dh<true, 0, 0>(fa, s.dh, blocks, stream); break;
    case 2: flash_dispatch_group<1>(fa, s.dh, mks, blocks, stream); break;
    case 3: flash_dispatch_group<2>(fa, s.dh, mks, blocks, stream); break;
    default: flash_dispatch_group<3>(fa, s.dh, mks, blocks, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_group_attention_asym(const uint16_t* q, const uint16_t* kg, const uint16_t* vg,
                                       const int32_t* q_idx, const int32_t* kinfo,
                                       const int32_t* plan, const AttnShape& s, _Float16* og,
                                       float* lseg, hipStream_t stream) {
  FlashArgs fa{};
  fa.q = q;
  fa.k = kg;
  fa.v = vg;
  fa.og = og;
  fa.lseg = lseg;
  fa.n = s.n;
  fa.Hq = s.Hq;
  fa.Hkv = s.Hkv;
  fa.G = s.G;
  fa.T = attn_tile_tokens(s.G);
  fa.window = (int)(s.window < s.n ? s.window : s.n);
  fa.sl2 = s.scale * kLog2e;
  fa.kinfo = (const i32x4_t*)kinfo;
  fa.qidx = q_idx;
  fa.plan = (const i32x4_t*)plan;
  fa.K = s.K;
  fa.top_k = s.top_k;
  fa.w_max = attn_work_items(s.nk, fa.T, s.K);
  const int64_t blocks = xcd_grid((int64_t)s.Hkv * fa.w_max);
  if (blocks <= 0) return hipSuccess;
  flash_dispatch_dh<true, 0, 0, false, false, true>(fa, s.dh, blocks, stream);
  return hipGetLastError();
}

hipError_t launch_window_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const _Float16* og, const float* lseg, const int32_t* slot,
                                   const AttnShape& s, uint16_t* out, float* lse,
                                   hipStream_t stream) {
  FlashArgs fa{};
  fa.q = q;
  fa.k = k;
  fa.v = v;
  fa.og = (_Float16*)og;
  fa.lseg = (float*)lseg;
  fa.out = out;
  fa.lse = lse;
  fa.slot = slot;
  fa.top_k = s.top_k;
  fa.n = s.n;
  fa.Hq = s.Hq;
  fa.Hkv = s.Hkv;
  fa.G = s.G;
  fa.T = attn_tile_tokens(s.G);
  fa.window = (int)(s.window < s.n ? s.window : s.n);
  fa.sl2 = s.scale * kLog2e;
  fa.tiles_per_head = (int)((s.n + fa.T - 1) / fa.T);
  const int64_t blocks = xcd_grid((int64_t)s.Hkv * fa.tiles_per_head);
  if (blocks <= 0) return hipSuccess;
  switch (s.top_k) {
    case 1: flash_dispatch_dh<false, 0, 0>(fa, s.dh, blocks, stream); break;
    case 2: flash_dispatch_dh<false, 1, 0>(fa, s.dh, blocks, stream); break;
    case 3: flash_dispatch_dh<false, 2, 0>(fa, s.dh, blocks, stream); break;
    default: flash_dispatch_dh<false, 3, 0>(fa, s.dh, blocks, stream); break;
  }
  return hipGetLastError();
}

// The soft gate's forward: the window kernel over every causal pair (see flash_kernel's SOFT).
hipError_t launch_soft_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* groups, const AttnShape& s, float bias_none,
                                 float bias_share, uint16_t* out, float* lse, hipStream_t stream) {
  FlashArgs fa{};
  fa.q = q;
  fa.k = k;
  fa.v = v;
  fa.out = out;
  fa.lse = lse;
  fa.groups = groups;
  fa.top_k = s.top_k;
  fa.K = s.K;
  fa.n = s.n;
  fa.Hq = s.Hq;
  fa.Hkv = s.Hkv;
  fa.G = s.G;
  fa.T = attn_tile_tokens(s.G);
  fa.window = (int)(s.window < s.n ? s.window : s.n);
  fa.sl2 = s.scale * kLog2e;
  fa.soft_b0 = bias_none / s.scale;
  fa.soft_b1 = bias_share / s.scale;
  // bias-row path: rows shift by the larger bias, the rows mark the pairs with the smaller one
  fa.soft_mark_none = bias_share > bias_none ? 1 : 0;
  fa.soft_shift = bias_share > bias_none ? bias_share : bias_none;
  fa.tiles_per_head = (int)((s.n + fa.T - 1) / fa.T);
  const int64_t blocks = xcd_grid((int64_t)s.Hkv * fa.tiles_per_head);
  if (blocks <= 0) return hipSuccess;
  // the group test runs on 32-bit slot masks when the tile's query tokens have at most 32
  // group slots, else by comparing group ids
  const bool smask = fa.T * s.top_k <= 32;
  // with at most 16 query tokens per tile the far pairs' share term runs as three MFMA bias
  // k-steps and only tiles that reach the window or the diagonal keep per-element work
  if (smask && fa.T <= 16) {
    switch (s.top_k) {
      case 1: flash_dispatch_dh<false, 0, 3, true, true>(fa, s.dh, blocks, stream); break;
      case 2: flash_dispatch_dh<false, 1, 3, true, true>(fa, s.dh, blocks, stream); break;
      case 3: flash_dispatch_dh<false, 2, 3, true, true>(fa, s.dh, blocks, stream); break;
      default: flash_dispatch_dh<false, 3, 3, true, true>(fa, s.dh, blocks, stream); break;
    }
    return hipGetLastError();
  }
  switch (s.top_k) {
    case 1:
      if (smask) flash_dispatch_dh<false, 0, 0, true, true>(fa, s.dh, blocks, stream);
      else flash_dispatch_dh<false, 0, 0, true>(fa, s.dh, blocks, stream);
      break;
    case 2:
      if (smask) flash_dispatch_dh<false, 1, 0, true, true>(fa, s.dh, blocks, stream);
      else flash_dispatch_dh<false, 1, 0, true>(fa, s.dh, blocks, stream);
      break;
    case 3:
      if (smask) flash_dispatch_dh<false, 2, 0, true, true>(fa, s.dh, blocks, stream);
      else flash_dispatch_dh<false, 2, 0, true>(fa, s.dh, blocks, stream);
      break;
    default:
      if (smask) flash_dispatch_dh<false, 3, 0, true, true>(fa, s.dh, blocks, stream);
      else flash_dispatch_dh<false, 3, 0, true>(fa, s.dh, blocks, stream);
      break;
  }
  return hipGetLastError();
}

}  // namespace focus
