// Batched single-token decode against per-sequence caches with cached group memberships.
//
// Inference rule of "Why Attend to Everything? Focus is the Key" (Chinese technical summary,
// gist.science/zh, section 2.1.3): the new token attends its window and the members of the
// groups it joins. For sequence b the query sits at position p = L_b - 1. Its keys form a
// virtual list: the window [max(0, p - w' + 1), p] with w' = max(window, 1) (the token always
// sees itself), then for each query group g_r the segment members at positions <= p - w'
// whose lowest group shared with the query is g_r, so every allowed key appears once.
//
// Two kernels. Each block of the partial kernel first finds its sequence's plan: where the
// window starts and each query group's slice of the sequence's bucketed memberships (one wave per
// query group). It then resolves its own piece of the virtual list into key positions in LDS (-1
// for members that a lower shared query group owns), a chunk at a time, and reads every listed
// key's K and V rows, all kv heads of a token at once where the head count allows, keeping a
// running (max, sum, O) per query head. The pieces (`splits` per sequence, chosen from the batch
// shape) are merged by log-sum-exp in a second kernel. The path is HBM-bound: every allowed key
// costs one K row and one V row per kv head.
#include "focus_internal.hpp"

namespace focus {

constexpr int kDecHeads = 4;        // query heads per block
constexpr int kDecInfo = 12;        // per-sequence plan: lo, nl, -, then (segment start, count) x 4
constexpr int kDecBlocks = 512;     // partial-kernel blocks aimed for: two per compute unit
constexpr int kDecMaxSplits = 256;  // key-list pieces per (sequence, head group), at most
constexpr int kDecChunk = 1024;     // list entries a partial block resolves into LDS at a time

// Query heads per unit (hpb), units per block (upb) and blocks of units per sequence (nub) of
// the partial kernel. A unit is up to kDecHeads query heads of one kv head; a block's lane
// groups (16 at d_head 128, 32 at 64) split into upb units, upb the largest power of two that
// divides the sequence's unit count.
struct DecodeUnits {
  int hpb, upb, nub;
};
DecodeUnits decode_units(int Hq, int G, int dh) {
  DecodeUnits u{};
  u.hpb = G < kDecHeads ? G : kDecHeads;
  const int units = Hq / u.hpb, ng = dh == 128 ? 16 : 32;
  int g = ng;
  while (units % g != 0) g /= 2;  // ng is a power of two: the largest common power of two
  u.upb = g;
  u.nub = units / g;
  return u;
}

// Pieces per sequence: as many as keep the grid within kDecBlocks blocks. Every piece has the
// same length, so with at most two blocks per compute unit no unit runs a third piece after the
// others have finished; and two resident blocks of long pieces stream the scattered K/V rows
// faster than four of half the length (measured on the 64 x 65536 decode).
int decode_splits(const DecodeShape& s) {
  if (s.B < 1 || s.Hq < 1 || s.G < 1 || s.Hq % s.G != 0) return 1;
  const int64_t per = (int64_t)s.B * decode_units(s.Hq, s.G, s.dh).nub;
  if (per >= kDecBlocks) return 1;
  const int64_t sp = kDecBlocks / per;
  return (int)(sp < kDecMaxSplits ? sp : kDecMaxSplits);
}

// ============================================================================ plan
// inf = (lo, nl, 0, seg_lo_0, cnt_0, ..., seg_lo_3, cnt_3): the window is positions
// lo .. lo + nl - 1; query group r contributes the cnt_r members of its segment from index
// seg_lo_r on (indices into the sequence's member list), those at positions <= p - w'. One
// wave per query group finds the boundary with a 64-ary search: each step probes 64 evenly
// spaced members of [s0, s1) at once. Returns the count to every lane of the wave.
__device__ __forceinline__ int64_t seg_search(const int32_t* __restrict__ members, int64_t s0,
                                              int64_t s1, int64_t thr, int l) {
  // first member index in [s0, s1) at a position > thr (positions ascend in a segment).
  // Invariant: members below lo_i are at or before the boundary, members from hi_i on after.
  // Lane l probes lo_i + span*l/64; the probes at or before the boundary form a prefix of
  // n_le lanes, so the answer lies after the last of them and at or before the next.
  int64_t lo_i = s0, hi_i = s1;
  while (lo_i < hi_i) {
    const int64_t span = hi_i - lo_i;
    const bool le = (int64_t)members[lo_i + (span * l) / 64] <= thr;
    const int n_le = __popcll(__ballot(le));
    if (n_le == 0) break;  // even lo_i is past the boundary
    if (n_le < 64) hi_i = lo_i + (span * n_le) / 64;
    lo_i = lo_i + (span * (n_le - 1)) / 64 + 1;
  }
  return lo_i - s0;
}

// Memberships come bucketed (cache_off / cache_idx: offsets and one index list of capacity
// Lmax * top_k per sequence) or, with seg_len, group-slotted (cache_idx holds seg_pos: a row of
// gcap positions per (sequence, group), seg_len[b * K + g] of them in use). A listed position
// outside [0, p] is skipped, and a sequence's list never exceeds per_seq entries. With a page
// table an entry is the key's row in the shared page pool instead:
// table[b][pos / page] * page + pos % page, or -1 when the table entry is not a page of the pool.
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* q_groups;      // [B, top_k]
  const int32_t* cache_groups;  // [B, Lmax, top_k]
  const int32_t* cache_len;     // [B]
  const int32_t* cache_off;     // [B, K + 1] (bucketed)
  const int32_t* cache_idx;     // [B, Lmax * top_k] (bucketed) or seg_pos [B, K, gcap]
  const int32_t* seg_len;       // [B, K] (group-slotted), else null
  const int32_t* table;         // [B, pages_per_seq] (paged), else null
  int64_t Lmax, window, pages_per_seq, num_pages;
  int K, gcap, page;
  int64_t per_seq;  // list entries per sequence, at most
  int B;
  int64_t seq_rows;  // rows between consecutive sequences' caches (0: list rows are pool rows)
  int Hq, Hkv, G, top_k, splits;
  int hpb;  // query heads per unit (<= kDecHeads), all of one kv head
  int upb;  // units per block: divides the block's lane groups and the units of a sequence
  float sl2;
  float* part_o;   // [B, Hq, splits, DH] unnormalised
  float* part_ml;  // [B, Hq, splits, 2] (running max in log2 units, sum)
};

// x plus lane (l ^ 1), (l ^ 2), then the mirrored lane of the 8-lane half row and, for W = 16,
// of the 16-lane row: data-parallel-primitive moves on the VALU, with no LDS round trip.
// bound_ctrl makes every lane a valid source.
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                   CTRL, 0xF, 0xF, false));
}
template <int W>
__device__ __forceinline__ float group_sum(float x) {  // sum over the lane's aligned W-lane group
  static_assert(W == 8 || W == 16, "lane groups of 8 or 16");
  x = dpp_plus<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_plus<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_plus<0x141>(x);  // row_half_mirror
  if constexpr (W == 16) x = dpp_plus<0x140>(x);  // row_mirror
  return x;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The sequence's resolved key list is cut into `splits` contiguous pieces. A head unit is up to 4
// query heads of one kv head; a block serves `upb` units, so its lane groups split into `upb`
// units times NG / upb key slots. Groups of one slot take the same key, so when a block's
// units cover every kv head, each key's K and V rows (all kv heads, contiguous) are read whole
// by one block. Each lane holds 8 dims of its unit's query heads as bf16 pairs and reads one
// 16-byte chunk of the key's K and V rows; the dot products are reduced across the 16 lanes
// with row moves, and a running (max, sum, O) per head absorbs the key. A lane group keeps U
// keys' rows in flight (three rather than four measured faster on the scattered rows), their
// positions read from the block's resolved chunk of the list in LDS.
template <int DH>
__global__ __launch_bounds__(256) void decode_partial_kernel(const DecodeArgs a) {
  constexpr int CHK = DH / 8;          // 16-byte chunks per row: lanes per key
  constexpr int KPW = kWave / CHK;     // lane groups per wave
  constexpr int NG = 4 * KPW;          // lane groups per block
  constexpr int HD = kDecHeads;
  constexpr int U = 3;                 // keys in flight per lane group
  __shared__ float red_o[NG][HD][DH];
  __shared__ float red_ml[NG][HD][2];
  __shared__ int32_t inf[kDecInfo];
  __shared__ int32_t qg_s[4];
  __shared__ int32_t pos_s[kDecChunk];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int c = l % CHK, grp = wave * KPW + l / CHK;  // chunk of the row, lane group
  const int upb = a.upb, slots = NG / a.upb;           // units per block, keys taken at once
  const int ul = grp % upb, slot = grp / upb;
  const int nub = a.Hq / a.hpb / upb;                  // blocks of units per sequence
  // each XCD takes a contiguous range of sequences, so its address-translation working set is
  // its own sequences' caches rather than every cache
  const int64_t lin = xcd_remap(blockIdx.x, (int64_t)a.B * nub * a.splits);
  if (lin < 0) return;  // whole block: before any barrier
  const int sp = (int)(lin % a.splits);
  const int ub = (int)((lin / a.splits) % nub);
  const int b = (int)(lin / ((int64_t)a.splits * nub));
  const int hq0 = (ub * upb + ul) * a.hpb, h = hq0 / a.G;
  const int nh = a.hpb;

  // ---- the sequence's plan (every block of the sequence finds the same one)
  const int32_t* members = a.seg_len ? a.cache_idx + (int64_t)b * a.K * a.gcap
                                     : a.cache_idx + (int64_t)b * a.Lmax * a.top_k;
  int64_t L = a.cache_len[b];
  if (L < 1) L = 1;
  if (L > a.Lmax) L = a.Lmax;
  const int64_t p = L - 1;
  {
    const int64_t wl = a.window > 1 ? a.window : 1;  // the new token always sees itself
    const int64_t lo = p - wl + 1 > 0 ? p - wl + 1 : 0;
    if (wave < a.top_k) {
      const int g = a.q_groups[(int64_t)b * a.top_k + wave];
      bool repeat = false;  // a query group listed twice contributes its members once
      for (int r2 = 0; r2 < wave; ++r2) repeat = repeat || a.q_groups[(int64_t)b * a.top_k + r2] == g;
      int64_t s0 = 0, s1 = 0;
      if (g >= 0 && g < a.K && !repeat) {
        if (a.seg_len) {
          int64_t n = a.seg_len[(int64_t)b * a.K + g];
          n = n < 0 ? 0 : (n > a.gcap ? a.gcap : n);
          s0 = (int64_t)g * a.gcap;
          s1 = s0 + n;
        } else {
          const int32_t* off = a.cache_off + (int64_t)b * (a.K + 1);
          s0 = off[g];
          s1 = off[g + 1];
          if (s0 < 0 || s1 < s0 || s1 > a.per_seq) s0 = s1 = 0;  // not a bucket of this capacity
        }
      }
      const int64_t cnt = seg_search(members, s0, s1, p - wl, l);
      if (l == 0) {
        inf[3 + 2 * wave] = (int32_t)s0;
        inf[4 + 2 * wave] = (int32_t)cnt;
        qg_s[wave] = g;
      }
    } else if (tid == 64 * 3) {  // a lane of a wave without a search (top_k < 4)
      for (int rr = a.top_k; rr < 4; ++rr) {
        inf[3 + 2 * rr] = 0;
        inf[4 + 2 * rr] = 0;
      }
    }
    if (tid == 0) {
      inf[0] = (int32_t)lo;
      inf[1] = (int32_t)(p - lo + 1);
      inf[2] = 0;
    }
    __syncthreads();
    if (tid == 0) {  // the list holds at most per_seq entries
      int64_t run = inf[1];
      for (int r = 0; r < a.top_k; ++r) {
        const int64_t room = a.per_seq - run;
        if (inf[4 + 2 * r] > room) inf[4 + 2 * r] = (int32_t)room;
        run += inf[4 + 2 * r];
      }
    }
    __syncthreads();
  }
  const int64_t lo = inf[0], nl = inf[1];
  int64_t total = nl;
  for (int r = 0; r < a.top_k; ++r) total += inf[4 + 2 * r];
  const int64_t per = (total + a.splits - 1) / a.splits;
  const int64_t v0 = (int64_t)sp * per;
  const int64_t v1 = v0 + per < total ? v0 + per : total;

  // key position (or pool row) of virtual list entry vi, -1 for an entry that is dropped: a
  // member of a query group that a lower shared query group owns, or not a cached position
  auto entry = [&](int64_t vi) __attribute__((always_inline)) {
    int pos = -1;
    if (vi < nl) {
      pos = (int)(lo + vi);
    } else {
      int64_t rem = vi - nl;
      for (int r = 0; r < a.top_k; ++r) {
        const int64_t cnt = inf[4 + 2 * r];
        if (rem < cnt) {
          const int cand = members[inf[3 + 2 * r] + rem];
          if (cand < 0 || cand > p) break;  // not a cached position: skipped
          // owned by g_r unless the key also holds a lower query group
          bool owned = true;
          const int32_t* kg = a.cache_groups + ((int64_t)b * a.Lmax + cand) * a.top_k;
          for (int r2 = 0; r2 < a.top_k; ++r2) {
            const int g2 = qg_s[r2];
            if (g2 >= 0 && g2 < a.K && g2 < qg_s[r])
              for (int r3 = 0; r3 < a.top_k; ++r3) owned = owned && kg[r3] != g2;
          }
          pos = owned ? cand : -1;
          break;
        }
        rem -= cnt;
      }
    }
    if (a.table && pos >= 0) {
      const int64_t pg = a.table[(int64_t)b * a.pages_per_seq + pos / a.page];
      pos = (pg >= 0 && pg < a.num_pages) ? (int)(pg * a.page + pos % a.page) : -1;
    }
    return pos;
  };

  // this lane's slice of the query heads as bf16 pairs; scores are scaled after the reduction
  i32x4_t qr[HD];
#pragma unroll
  for (int hh = 0; hh < HD; ++hh) {
    const int hq = hq0 + (hh < nh ? hh : 0);
    qr[hh] = *(const i32x4_t*)(a.q + ((int64_t)b * a.Hq + hq) * DH + c * 8);
  }
  float m_run[HD], l_run[HD], o[HD][8];
#pragma unroll
  for (int hh = 0; hh < HD; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }

  const int64_t kv_stride = (int64_t)a.Hkv * DH;
  const uint16_t* kbase = a.kc + (int64_t)b * a.seq_rows * kv_stride + (int64_t)h * DH + c * 8;
  const uint16_t* vbase = a.vc + (int64_t)b * a.seq_rows * kv_stride + (int64_t)h * DH + c * 8;

  // the piece a chunk at a time: its positions resolved into LDS by the whole block, then
  // entries slot + k * slots of the chunk taken U at a time by each lane group
  for (int64_t c0 = v0; c0 < v1; c0 += kDecChunk) {
  const int cn = (int)(v1 - c0 < kDecChunk ? v1 - c0 : kDecChunk);
  __syncthreads();  // every lane group is done with the previous chunk's positions
  for (int i = tid; i < cn; i += 256) pos_s[i] = entry(c0 + i);
  __syncthreads();
  for (int i0 = slot; i0 < cn; i0 += U * slots) {
    int pk[U];
    i32x4_t kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * slots;
      pk[u] = i < cn ? pos_s[i] : -1;
      const int64_t row = pk[u] >= 0 ? pk[u] : 0;
      kr[u] = *(const i32x4_t*)(kbase + row * kv_stride);
      vr[u] = *(const i32x4_t*)(vbase + row * kv_stride);
    }
    // scores of the batch's U keys for every head (heads past nh are computed and ignored),
    // all before any reduction so the independent row-move chains interleave
    float sc[U][HD];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int hh = 0; hh < HD; ++hh) {
        // bf16 products are exact in fp32; two chains of two pairs each
        const float d0 = dot2_bf16((uint32_t)qr[hh][1], (uint32_t)kr[u][1],
                                   dot2_bf16((uint32_t)qr[hh][0], (uint32_t)kr[u][0], 0.f));
        const float d1 = dot2_bf16((uint32_t)qr[hh][3], (uint32_t)kr[u][3],
                                   dot2_bf16((uint32_t)qr[hh][2], (uint32_t)kr[u][2], 0.f));
        sc[u][hh] = d0 + d1;
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int hh = 0; hh < HD; ++hh) {
        const float x = group_sum<CHK>(sc[u][hh]) * a.sl2;
        sc[u][hh] = pk[u] >= 0 ? x : -INFINITY;  // pk is uniform within the lane group
      }
    // lazy running max, one test per batch: rescale only when a score passes the reference by
    // 2^8, so every weight below stays under 2^8
    float bmax[HD];
    bool bump = false;
#pragma unroll
    for (int hh = 0; hh < HD; ++hh) {
      bmax[hh] = sc[0][hh];
#pragma unroll
      for (int u = 1; u < U; ++u) bmax[hh] = fmaxf(bmax[hh], sc[u][hh]);
      bump = bump || bmax[hh] > m_run[hh] + 8.f;
    }
    if (bump) {
#pragma unroll
      for (int hh = 0; hh < HD; ++hh) {
        const bool bh = bmax[hh] > m_run[hh] + 8.f;
        const float alpha = !bh ? 1.f : m_run[hh] == -INFINITY ? 0.f : fast_exp2(m_run[hh] - bmax[hh]);
        l_run[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] *= alpha;
        m_run[hh] = bh ? bmax[hh] : m_run[hh];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = __uint_as_float((uint32_t)vr[u][e] << 16);
        vf[2 * e + 1] = __uint_as_float((uint32_t)vr[u][e] & 0xffff0000u);
      }
#pragma unroll
      for (int hh = 0; hh < HD; ++hh) {
        const float m_use = m_run[hh] == -INFINITY ? 0.f : m_run[hh];
        const float pw = fast_exp2(sc[u][hh] - m_use);  // 0 for a dropped entry
        l_run[hh] += pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = __builtin_fmaf(pw, vf[e], o[hh][e]);
      }
    }
  }
  }

  // ---- merge each unit's key slots and write this block's partial per head
  if (c == 0) {
#pragma unroll
    for (int hh = 0; hh < HD; ++hh) {
      red_ml[grp][hh][0] = m_run[hh];
      red_ml[grp][hh][1] = l_run[hh];
    }
  }
#pragma unroll
  for (int hh = 0; hh < HD; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[grp][hh][c * 8 + e] = o[hh][e];
  __syncthreads();
  for (int i = tid; i < upb * nh * DH; i += 256) {
    const int u = i / (nh * DH), hh = (i / DH) % nh, d = i % DH;
    float M = -INFINITY;
    for (int s2 = 0; s2 < slots; ++s2) M = fmaxf(M, red_ml[s2 * upb + u][hh][0]);
    float lsum = 0.f, acc = 0.f;
    if (M != -INFINITY)
      for (int s2 = 0; s2 < slots; ++s2) {
        const int g = s2 * upb + u;
        const float m = red_ml[g][hh][0];
        if (m == -INFINITY) continue;
        const float w = fast_exp2(m - M);
        lsum += w * red_ml[g][hh][1];
        acc += w * red_o[g][hh][d];
      }
    const int64_t pi = ((int64_t)b * a.Hq + (ub * upb + u) * a.hpb + hh) * a.splits + sp;
    a.part_o[pi * DH + d] = acc;
    if (d == 0) {
      a.part_ml[pi * 2] = M;
      a.part_ml[pi * 2 + 1] = lsum;
    }
  }
}

// The pieces' partials of each (sequence, query head) merged by log-sum-exp.
// Few pieces: one block per (sequence, head), a thread per output dimension that reads every
// piece's (max, sum) and O, in piece order.
constexpr int kCombineLoopMax = 16;  // pieces up to which the loop form runs
template <int DH>
__global__ __launch_bounds__(DH) void decode_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            int splits, uint16_t* __restrict__ out,
                                                            float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;  // b * Hq + hq
  const int d = threadIdx.x;
  const float2* ml = (const float2*)part_ml + bh * splits;
  const float* po = part_o + bh * splits * DH + d;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[s].x);
  float den = 0.f, acc = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
      const float2 m = ml[s];
      const float w = m.x == -INFINITY ? 0.f : fast_exp2(m.x - M);
      den += w * m.y;
      acc += w * po[(int64_t)s * DH];
    }
  }
  const float o = den > 0.f ? acc / den : 0.f;
  __bf16 ob = to_bf16(o);
  out[bh * DH + d] = *(uint16_t*)&ob;
  if (d == 0) lse[bh] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
}

// Many pieces (small batches): one block per (sequence, head, 32 output dimensions). The block's
// threads take the pieces' (max, sum) pairs one each for the common maximum and the denominator;
// then 16 groups of 32 lanes split the pieces (piece g, g + 16, ...) for the weighted sums,
// which are added in group order.
template <int DH>
__global__ __launch_bounds__(512) void decode_combine_wide_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = 512, DC = 32, NGRP = NT / DC, NW = NT / kWave;
  static_assert(kDecMaxSplits <= NT, "one piece per thread for the (max, sum) pairs");
  __shared__ float2 sml[kDecMaxSplits];
  __shared__ float red[NW];
  __shared__ float racc[NGRP][DC];
  const int64_t bh = blockIdx.x / (DH / DC);  // b * Hq + hq
  const int dc = blockIdx.x % (DH / DC);
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const float2 mine = tid < splits ? ((const float2*)part_ml)[bh * splits + tid]
                                   : make_float2(-INFINITY, 0.f);
  if (tid < splits) sml[tid] = mine;
  float x = mine.x;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  if (l == 0) red[w] = x;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[i]);
  __syncthreads();  // red is reused below
  float y = mine.x == -INFINITY ? 0.f : fast_exp2(mine.x - M) * mine.y;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) y += __shfl_xor(y, off);
  if (l == 0) red[w] = y;
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) den += red[i];
  const int dl = tid % DC, g = tid / DC, d = dc * DC + dl;
  float acc = 0.f;
  if (M != -INFINITY) {
    const float* po = part_o + bh * splits * DH + d;
#pragma unroll 4
    for (int s = g; s < splits; s += NGRP) {
      const float2 m = sml[s];
      const float wt = m.x == -INFINITY ? 0.f : fast_exp2(m.x - M);
      acc += wt * po[(int64_t)s * DH];
    }
  }
  racc[g][dl] = acc;
  __syncthreads();
  if (g == 0) {
    float a = racc[0][dl];
#pragma unroll
    for (int i = 1; i < NGRP; ++i) a += racc[i][dl];
    const float o = den > 0.f ? a / den : 0.f;
    __bf16 ob = to_bf16(o);
    out[bh * DH + d] = *(uint16_t*)&ob;
    if (d == 0) lse[bh] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
  }
}

template <int DH>
hipError_t launch_combine(const float* part_o, const float* part_ml, int B, int Hq, int splits,
                          uint16_t* out, float* lse, hipStream_t stream) {
  if (splits <= kCombineLoopMax)
    hipLaunchKernelGGL(decode_combine_kernel<DH>, dim3((int64_t)B * Hq), dim3(DH), 0, stream,
                       part_o, part_ml, splits, out, lse);
  else
    hipLaunchKernelGGL(decode_combine_wide_kernel<DH>, dim3((int64_t)B * Hq * (DH / 32)),
                       dim3(512), 0, stream, part_o, part_ml, splits, out, lse);
  return hipGetLastError();
}

hipError_t launch_decode(const uint16_t* q, const int32_t* q_groups, const uint16_t* kc,
                         const uint16_t* vc, const int32_t* cache_len, const int32_t* cache_groups,
                         const int32_t* cache_off, const int32_t* cache_idx, const DecodeShape& s,
                         float* part_o, float* part_ml, uint16_t* out, float* lse,
                         hipStream_t stream, const DecodePaging* pg, const DecodeSlots* sl) {
  if (s.splits < 1 || s.splits > kDecMaxSplits) return hipErrorInvalidValue;
  DecodeArgs a{};
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.q_groups = q_groups;
  a.cache_groups = cache_groups;
  a.cache_len = cache_len;
  a.cache_off = cache_off;
  a.cache_idx = cache_idx;
  a.seg_len = sl ? sl->seg_len : nullptr;
  a.gcap = sl ? sl->gcap : 0;
  a.table = pg ? pg->table : nullptr;
  a.page = pg ? pg->page_size : 1;
  a.pages_per_seq = pg ? pg->pages_per_seq : 0;
  a.num_pages = pg ? pg->num_pages : 0;
  a.Lmax = s.Lmax;
  a.window = s.window;
  a.K = s.K;
  a.per_seq = s.Lmax * s.top_k;  // the virtual list never exceeds top_k * L
  a.B = s.B;
  a.seq_rows = pg ? 0 : s.Lmax;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.top_k = s.top_k;
  a.splits = s.splits;
  a.sl2 = s.scale * kLog2e;
  a.part_o = part_o;
  a.part_ml = part_ml;
  const DecodeUnits du = decode_units(s.Hq, s.G, s.dh);
  a.hpb = du.hpb;
  a.upb = du.upb;
  const int64_t blocks = xcd_grid((int64_t)s.B * du.nub * s.splits);
  if (s.dh == 128) {
    hipLaunchKernelGGL(decode_partial_kernel<128>, dim3(blocks), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    return launch_combine<128>(part_o, part_ml, s.B, s.Hq, s.splits, out, lse, stream);
  }
  hipLaunchKernelGGL(decode_partial_kernel<64>, dim3(blocks), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return launch_combine<64>(part_o, part_ml, s.B, s.Hq, s.splits, out, lse, stream);
}

}  // namespace focus
