// Gated sparse causal attention on gfx950.
//
// Pair rule ("Why Attend to Everything? Focus is the Key", Chinese technical summary,
// gist.science/zh, sections 2.1.2 and 2.1.3; Dutch technical summary, Kerncomponenten 3):
// query i attends key j <= i when i - j < window or the tokens share a group, with an exact
// softmax over the allowed pairs. The pairs are split between two passes so each is counted
// once: the window pass owns i - j < window; a far pair belongs to the lowest group the two
// tokens share. The group pass runs on contiguous group segments (gathered Q/K/V); the merge
// combines the window part and the group parts by their log-sum-exp.
//
// Flash kernel layout (both passes). A workgroup has 4 waves and 128 query rows: T = 128/G
// tokens times the G query heads of one kv head, so K/V tiles in LDS serve all G heads. A kv
// tile is 64 keys. Each wave owns 32 rows and computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from LDS, B = the wave's Q held in
// registers), so every lane holds one query column: the softmax row statistics live in one
// lane pair (l, l^32) and need a single cross-lane exchange. O^T = V^T P^T reuses the S^T
// accumulator layout directly as the B operand; V is stored transposed in LDS so the A
// operand (32 dims x 16 keys) is two 8-byte reads per lane.
#include "focus_internal.hpp"

namespace focus {

int attn_tile_tokens(int G) { return 128 / G; }

// ============================================================================ gather
// qg[s] = q[idx[s]], kg[s] = k[idx[s]], vg[s] = v[idx[s]] for every membership slot s.
__global__ __launch_bounds__(256) void gather_qkv_kernel(const i32x4_t* __restrict__ q,
                                                         const i32x4_t* __restrict__ k,
                                                         const i32x4_t* __restrict__ v,
                                                         const int32_t* __restrict__ idx,
                                                         int64_t nk, int cq, int ckv,
                                                         i32x4_t* __restrict__ qg,
                                                         i32x4_t* __restrict__ kg,
                                                         i32x4_t* __restrict__ vg) {
  const int per = cq + 2 * ckv;  // 16-byte chunks per slot
  const int64_t total = nk * per;
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t base = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < total; base += stride) {
    i32x4_t val[4];
    int64_t dst[4];
    int which[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int64_t e = base + u * 256;
      which[u] = -1;
      if (e >= total) continue;
      int64_t s = e / per;
      int c = (int)(e - s * per);
      int32_t tok = idx[s];
      if (tok < 0) continue;
      if (c < cq) {
        val[u] = q[(int64_t)tok * cq + c];
        dst[u] = s * cq + c;
        which[u] = 0;
      } else if (c < cq + ckv) {
        c -= cq;
        val[u] = k[(int64_t)tok * ckv + c];
        dst[u] = s * ckv + c;
        which[u] = 1;
      } else {
        c -= cq + ckv;
        val[u] = v[(int64_t)tok * ckv + c];
        dst[u] = s * ckv + c;
        which[u] = 2;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (which[u] == 0) qg[dst[u]] = val[u];
      else if (which[u] == 1) kg[dst[u]] = val[u];
      else if (which[u] == 2) vg[dst[u]] = val[u];
    }
  }
}

hipError_t launch_gather_qkv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int32_t* idx, const AttnShape& s, uint16_t* qg, uint16_t* kg,
                             uint16_t* vg, hipStream_t stream) {
  const int cq = s.Hq * s.dh / 8, ckv = s.Hkv * s.dh / 8;
  int64_t total = s.nk * (cq + 2 * ckv);
  int64_t blocks = (total + 1023) / 1024;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gather_qkv_kernel, dim3(blocks), dim3(256), 0, stream, (const i32x4_t*)q,
                     (const i32x4_t*)k, (const i32x4_t*)v, idx, s.nk, cq, ckv, (i32x4_t*)qg,
                     (i32x4_t*)kg, (i32x4_t*)vg);
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

// ============================================================================ flash kernel
struct FlashArgs {
  const uint16_t* q;  // group: gathered [nk, Hq, DH]; window: [n, Hq, DH]
  const uint16_t* k;  // [rows, Hkv, DH]
  const uint16_t* v;
  float* o;           // [rows, Hq, DH] normalised partial output
  float* lse;         // [rows, Hq] natural-log sum of exp of the scaled logits (-inf if none)
  int64_t n;          // window: tokens
  int Hq, Hkv, G, T;
  int64_t window;
  float sl2;          // scale * log2(e)
  const int32_t* seg_off;   // group: [K+1]
  const int32_t* tile_pre;  // group: [K+1]
  const int32_t* pos;       // group: slot -> token position
  const int32_t* groups;    // group: [n, top_k], ascending
  int K, top_k;
  int tiles_per_head;       // window: ceil(n / T)
};

constexpr int KT = 64;  // keys per kv tile
constexpr int kMaxLow = 3;

template <int DH>
struct FlashSmem {
  static constexpr int KS = DH + 8;      // K tile row stride (bf16 elements)
  static constexpr int VS = KT + 8;      // transposed V row stride (bf16 elements)
  __bf16 k[KT * KS];
  __bf16 vt[DH * VS];
  int kpos[KT];
  int klow[KT * kMaxLow];
};

template <int DH, bool GROUP>
__global__ __launch_bounds__(256) void flash_kernel(const FlashArgs a) {
  using Smem = FlashSmem<DH>;
  constexpr int KS = Smem::KS, VS = Smem::VS;
  constexpr int CH = DH / 8;        // 16-byte chunks per row
  constexpr int RPP = 256 / CH;     // K rows per load pass
  constexpr int KPASS = KT / RPP;   // K load passes
  constexpr int VKPT = DH / 32;     // V keys per thread (transposed store)
  constexpr int NS = DH / 16;       // MFMA k-steps over the head dimension
  constexpr int ND = DH / 32;       // 32-wide output tiles over the head dimension
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, jq = l & 31, hg = l >> 5;

  // ---------------------------------------------------------------- work item
  const int W = GROUP ? a.tile_pre[a.K] : a.tiles_per_head;
  const int64_t comb = xcd_remap(blockIdx.x, (int64_t)a.Hkv * W);
  if (comb < 0) return;
  const int h = (int)(comb / W);
  const int item = (int)(comb - (int64_t)h * W);

  int64_t q0, q1;        // query index range [q0, q1): slots (group) or tokens (window)
  int64_t kv_lo;         // first key index
  int grp = 0;
  int64_t seg_hi = 0;
  if constexpr (GROUP) {
    int lo = 0, hi = a.K - 1;  // largest g with tile_pre[g] <= item
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (a.tile_pre[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    grp = lo;
    const int nt = a.tile_pre[grp + 1] - a.tile_pre[grp];
    const int t = nt - 1 - (item - a.tile_pre[grp]);  // heaviest tiles first
    const int64_t s_lo = a.seg_off[grp];
    seg_hi = a.seg_off[grp + 1];
    q0 = s_lo + (int64_t)t * a.T;
    q1 = q0 + a.T < seg_hi ? q0 + a.T : seg_hi;
    kv_lo = s_lo;
  } else {
    q0 = (int64_t)item * a.T;
    q1 = q0 + a.T < a.n ? q0 + a.T : a.n;
    kv_lo = q0 - a.window + 1 > 0 ? q0 - a.window + 1 : 0;
  }
  const int64_t kv_hi = q1 - 1;  // last key index any query of the tile may see

  // ---------------------------------------------------------------- this lane's query row
  const int r = wave * 32 + jq;
  const int head_local = r / a.T, tok_local = r % a.T;
  const int hq = h * a.G + head_local;
  const int64_t qi = q0 + tok_local;
  const bool qvalid = qi < q1;
  // token range of the wave's rows (rows of one wave are consecutive tokens of one head,
  // or all T tokens of the tile when T < 32)
  const int wt0 = (wave * 32) % a.T;
  const int wtn = a.T < 32 ? a.T : 32;
  const int64_t wq_lo = q0 + wt0;
  const int64_t wq_hi = (q0 + wt0 + wtn < q1 ? q0 + wt0 + wtn : q1) - 1;
  const bool wave_active = wq_hi >= wq_lo;

  int qpos = 0;
  int qlow[kMaxLow] = {-1, -1, -1};
  if constexpr (GROUP) {
    if (qvalid) {
      qpos = a.pos[qi];
      int c = 0;
      for (int rr = 0; rr < a.top_k; ++rr) {
        int gg = a.groups[(int64_t)qpos * a.top_k + rr];
        if (gg < grp && c < kMaxLow) qlow[c++] = gg;
      }
    }
  } else {
    qpos = (int)qi;
  }
  int wpos_lo = 0, wpos_hi = 0, tpos_hi = 0;
  if constexpr (GROUP) {
    if (wave_active) {
      wpos_lo = a.pos[wq_lo];
      wpos_hi = a.pos[wq_hi];
    }
    tpos_hi = a.pos[kv_hi];
  }

  bf16x8_t qreg[NS];
  {
    const uint16_t* qp = a.q + ((qvalid ? qi : 0) * a.Hq + hq) * (int64_t)DH + 8 * hg;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qreg[s] = qvalid ? *(const bf16x8_t*)(qp + 16 * s) : bf16x8_t{};
  }

  // ---------------------------------------------------------------- kv tile range
  int64_t ntiles = 0;
  if constexpr (GROUP) {
    // stop at the first tile whose pairs all fall inside the window (positions ascend)
    int64_t hi_t = (kv_hi - kv_lo) / KT + 1;
    int64_t lo_t = 0;
    while (lo_t < hi_t) {  // first tile t with tpos_hi - pos[kv_lo + t*KT] < window
      int64_t mid = (lo_t + hi_t) >> 1;
      if ((int64_t)tpos_hi - a.pos[kv_lo + mid * KT] < a.window) hi_t = mid;
      else lo_t = mid + 1;
    }
    ntiles = lo_t;
  } else {
    ntiles = a.window > 0 ? (kv_hi - kv_lo) / KT + 1 : 0;
  }

  f32x16_t oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // register staging of the next tile
  bf16x8_t kreg[KPASS];
  bf16x8_t vreg[VKPT];
  int kpos_reg = 0;
  int klow_reg[kMaxLow] = {-2, -2, -2};
  const int lc = tid % CH, lr = tid / CH;

  auto load_tile = [&](int64_t ks) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      int64_t row = ks + lr + p * RPP;
      kreg[p] = row <= kv_hi
                    ? *(const bf16x8_t*)(a.k + (row * a.Hkv + h) * (int64_t)DH + lc * 8)
                    : bf16x8_t{};
    }
#pragma unroll
    for (int e = 0; e < VKPT; ++e) {
      int64_t row = ks + lr * VKPT + e;
      vreg[e] = row <= kv_hi
                    ? *(const bf16x8_t*)(a.v + (row * a.Hkv + h) * (int64_t)DH + lc * 8)
                    : bf16x8_t{};
    }
    if constexpr (GROUP) {
      if (tid < KT) {
        int64_t row = ks + tid;
        kpos_reg = row <= kv_hi ? a.pos[row] : 0x7fffffff;
        if (a.top_k > 1) {
          int c = 0;
          klow_reg[0] = klow_reg[1] = klow_reg[2] = -2;
          if (row <= kv_hi)
            for (int rr = 0; rr < a.top_k; ++rr) {
              int gg = a.groups[(int64_t)kpos_reg * a.top_k + rr];
              if (gg < grp && c < kMaxLow) klow_reg[c++] = gg;
            }
        }
      }
    }
  };

  if (ntiles > 0) load_tile(kv_lo);
  for (int64_t it = 0; it < ntiles; ++it) {
    const int64_t ks = kv_lo + it * KT;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < KPASS; ++p) *(bf16x8_t*)&sm.k[(lr + p * RPP) * KS + lc * 8] = kreg[p];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (VKPT == 4) {
        bf16x4_t t4 = {vreg[0][e], vreg[1][e], vreg[2][e], vreg[3][e]};
        *(bf16x4_t*)&sm.vt[(lc * 8 + e) * VS + lr * 4] = t4;
      } else {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        bf16x2_t t2 = {vreg[0][e], vreg[1][e]};
        *(bf16x2_t*)&sm.vt[(lc * 8 + e) * VS + lr * 2] = t2;
      }
    }
    if constexpr (GROUP) {
      if (tid < KT) {
        sm.kpos[tid] = kpos_reg;
        for (int c = 0; c < kMaxLow; ++c) sm.klow[tid * kMaxLow + c] = klow_reg[c];
      }
    }
    __syncthreads();
    if (it + 1 < ntiles) load_tile(ks + KT);

    // ------------------------------------------------------------ per-wave skip / mask decision
    if (!wave_active) continue;
    const int64_t k_last = ks + KT - 1;
    bool skip, full;
    if constexpr (GROUP) {
      const int kpos_first = sm.kpos[0];
      const int kpos_last = k_last <= kv_hi ? sm.kpos[KT - 1] : 0x7fffffff;
      skip = ks > wq_hi || (int64_t)wpos_hi - kpos_first < a.window;
      full = k_last <= kv_hi && k_last <= wq_lo && (int64_t)wpos_lo - kpos_last >= a.window &&
             a.top_k == 1;
    } else {
      skip = ks > wq_hi || wq_lo - k_last >= a.window;
      full = k_last <= wq_lo && wq_hi - ks < a.window;
    }
    if (skip) continue;

    // ------------------------------------------------------------ S^T = K Q^T
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8_t kf = *(const bf16x8_t*)&sm.k[(kb * 32 + jq) * KS + s * 16 + 8 * hg];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[s], sacc[kb], 0, 0, 0);
      }
    }

    // ------------------------------------------------------------ mask + online softmax
    // element v of tile kb holds key kb*32 + 8*(v/4) + 4*hg + v%4 of this tile
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) {
        float x = sacc[kb][vi] * a.sl2;
        if (!full) {
          const int kk = kb * 32 + 8 * (vi >> 2) + 4 * hg + (vi & 3);
          const int64_t kidx = ks + kk;
          bool ok;
          if constexpr (GROUP) {
            const int kp = sm.kpos[kk];
            ok = qvalid && kidx <= qi && (int64_t)qpos - kp >= a.window;
            if (a.top_k > 1) {
#pragma unroll
              for (int c1 = 0; c1 < kMaxLow; ++c1)
#pragma unroll
                for (int c2 = 0; c2 < kMaxLow; ++c2)
                  ok = ok && !(qlow[c1] == sm.klow[kk * kMaxLow + c2]);
            }
          } else {
            ok = qvalid && kidx <= qi && qi - kidx < a.window;
          }
          x = ok ? x : -INFINITY;
        }
        sacc[kb][vi] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    bf16x8_t pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) {
        float p = fast_exp2(sacc[kb][vi] - m_use);
        psum += p;
        pb[kb * 2 + (vi >> 3)][vi & 7] = to_bf16(p);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] *= alpha;

    // ------------------------------------------------------------ O^T += V^T P^T
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int base = (kq >> 1) * 32 + (kq & 1) * 16 + 4 * hg;
        const __bf16* vp = &sm.vt[(d * 32 + jq) * VS + base];
        bf16x4_t lo = *(const bf16x4_t*)vp;
        bf16x4_t hi = *(const bf16x4_t*)(vp + 8);
        bf16x8_t vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kq], oacc[d], 0, 0, 0);
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  if (!qvalid) return;
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* op = a.o + (qi * a.Hq + hq) * (int64_t)DH;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4_t x = {oacc[d][4 * g4] * inv, oacc[d][4 * g4 + 1] * inv, oacc[d][4 * g4 + 2] * inv,
                   oacc[d][4 * g4 + 3] * inv};
      *(f32x4_t*)(op + d * 32 + g4 * 8 + 4 * hg) = x;
    }
  if (hg == 0)
    a.lse[qi * a.Hq + hq] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <bool GROUP>
static hipError_t flash_launch(const FlashArgs& fa, int dh, int64_t blocks, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  if (dh == 128)
    hipLaunchKernelGGL((flash_kernel<128, GROUP>), dim3(blocks), dim3(256), 0, stream, fa);
  else
    hipLaunchKernelGGL((flash_kernel<64, GROUP>), dim3(blocks), dim3(256), 0, stream, fa);
  return hipGetLastError();
}

hipError_t launch_group_attention(const uint16_t* qg, const uint16_t* kg, const uint16_t* vg,
                                  const int32_t* offsets, const int32_t* tile_pre,
                                  const int32_t* idx, const int32_t* groups, const AttnShape& s,
                                  float* og, float* lseg, hipStream_t stream) {
  FlashArgs fa{};
  fa.q = qg;
  fa.k = kg;
  fa.v = vg;
  fa.o = og;
  fa.lse = lseg;
  fa.n = s.n;
  fa.Hq = s.Hq;
  fa.Hkv = s.Hkv;
  fa.G = s.G;
  fa.T = attn_tile_tokens(s.G);
  fa.window = s.window;
  fa.sl2 = s.scale * kLog2e;
  fa.seg_off = offsets;
  fa.tile_pre = tile_pre;
  fa.pos = idx;
  fa.groups = groups;
  fa.K = s.K;
  fa.top_k = s.top_k;
  // upper bound on the tiles of all segments: sum of ceil(size / T) <= ceil(nk / T) + K
  int64_t w_max = (s.nk + fa.T - 1) / fa.T + s.K;
  return flash_launch<true>(fa, s.dh, xcd_grid((int64_t)s.Hkv * w_max), stream);
}

hipError_t launch_window_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const AttnShape& s, float* ol, float* lsel,
                                   hipStream_t stream) {
  FlashArgs fa{};
  fa.q = q;
  fa.k = k;
  fa.v = v;
  fa.o = ol;
  fa.lse = lsel;
  fa.n = s.n;
  fa.Hq = s.Hq;
  fa.Hkv = s.Hkv;
  fa.G = s.G;
  fa.T = attn_tile_tokens(s.G);
  fa.window = s.window;
  fa.sl2 = s.scale * kLog2e;
  fa.tiles_per_head = (int)((s.n + fa.T - 1) / fa.T);
  return flash_launch<false>(fa, s.dh, xcd_grid((int64_t)s.Hkv * fa.tiles_per_head), stream);
}

// ============================================================================ merge
// out[i,h] = sum_p exp(lse_p - L) * O_p over the window part and the token's group parts,
// L = log(sum_p exp(lse_p)); lse[i,h] = L.
template <int DH>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ol,
                                                    const float* __restrict__ lsel,
                                                    const float* __restrict__ og,
                                                    const float* __restrict__ lseg,
                                                    const int32_t* __restrict__ slot, int64_t n,
                                                    int Hq, int top_k, uint16_t* __restrict__ out,
                                                    float* __restrict__ lse) {
  constexpr int TPR = DH / 4;  // threads per (token, head)
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gt / TPR;
  const int c = (int)(gt % TPR);
  if (pair >= n * Hq) return;
  const int64_t i = pair / Hq;
  const int hh = (int)(pair - i * Hq);
  float ls[5];
  int64_t src[5];
  ls[0] = lsel[pair];
  src[0] = -1;
  float M = ls[0];
  for (int rr = 0; rr < top_k; ++rr) {
    int s = slot[i * top_k + rr];
    src[rr + 1] = s;
    ls[rr + 1] = s >= 0 ? lseg[(int64_t)s * Hq + hh] : -INFINITY;
    M = fmaxf(M, ls[rr + 1]);
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int p = 0; p <= top_k; ++p) {
      if (ls[p] == -INFINITY) continue;
      float w = __expf(ls[p] - M);
      den += w;
      const float* op = p == 0 ? ol + pair * DH : og + (src[p] * Hq + hh) * (int64_t)DH;
      f32x4_t x = *(const f32x4_t*)(op + 4 * c);
      acc += w * x;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  bf16x4_t o4 = {to_bf16(acc[0] * inv), to_bf16(acc[1] * inv), to_bf16(acc[2] * inv),
                 to_bf16(acc[3] * inv)};
  *(bf16x4_t*)(out + pair * DH + 4 * c) = o4;
  if (c == 0) lse[pair] = den > 0.f ? M + __logf(den) : -INFINITY;
}

hipError_t launch_merge(const float* ol, const float* lsel, const float* og, const float* lseg,
                        const int32_t* slot, const AttnShape& s, uint16_t* out, float* lse,
                        hipStream_t stream) {
  const int64_t threads = s.n * s.Hq * (s.dh / 4);
  const int64_t blocks = (threads + 255) / 256;
  if (s.dh == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(blocks), dim3(256), 0, stream, ol, lsel, og, lseg,
                       slot, s.n, s.Hq, s.top_k, out, lse);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(blocks), dim3(256), 0, stream, ol, lsel, og, lseg,
                       slot, s.n, s.Hq, s.top_k, out, lse);
  return hipGetLastError();
}

}  // namespace focus
