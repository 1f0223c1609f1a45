// Batched single-token decode against per-sequence caches with cached group memberships.
//
// Inference rule of "Why Attend to Everything? Focus is the Key" (Chinese technical summary,
// gist.science/zh, section 2.1.3): the new token attends its window and the members of the
// groups it joins. For sequence b the query sits at position p = L_b - 1. Its keys form a
// virtual list: the window [max(0, p - w' + 1), p] with w' = max(window, 1) (the token always
// sees itself), then for each query group g_r the segment members at positions <= p - w'
// whose lowest group shared with the query is g_r, so every allowed key appears once.
//
// The list is cut into `splits` contiguous pieces per (sequence, group of up to 4 query heads
// of one kv head). A 256-thread block first resolves 256 list entries into key positions in
// LDS (one per thread, dropping group members owned by a lower shared group), then every
// 16-lane group takes one key at a time: each lane holds 8 dims of the query heads in
// registers and reads one coalesced 16-byte chunk of the key's K and V rows, the dot products
// are reduced across the 16 lanes, and a running (max, sum, O) per head absorbs the key. The
// 16 lane groups' states are merged through LDS into one partial per block, and a second
// kernel merges the partials by their log-sum-exp. The path is HBM-bound: every allowed key
// costs one K row and one V row of the kv head.
#include "focus_internal.hpp"

namespace focus {

constexpr int kDecChunk = 256;   // list entries resolved per pass
constexpr int kDecHeads = 4;     // query heads per block

int decode_splits(const DecodeShape& s) {
  (void)s;
  return 16;
}

struct DecodeArgs {
  const uint16_t* q;
  const int32_t* q_groups;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* cache_len;
  const int32_t* cache_groups;
  const int32_t* cache_off;
  const int32_t* cache_idx;
  int B;
  int64_t Lmax;
  int Hq, Hkv, G, K, top_k, splits, hpb;  // hpb: query heads per block (<= kDecHeads)
  int64_t window;
  float sl2;
  float* part_o;   // [B, Hq, splits, DH] unnormalised
  float* part_ml;  // [B, Hq, splits, 2] (running max in log2 units, sum)
};

template <int W>
__device__ __forceinline__ float group_sum(float x) {  // sum over the lane's aligned W-lane group
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

template <int DH>
__global__ __launch_bounds__(256) void decode_partial_kernel(const DecodeArgs a) {
  constexpr int CHK = DH / 8;          // 16-byte chunks per row: lanes per key
  constexpr int KPW = kWave / CHK;     // keys per wave instruction
  constexpr int NG = 4 * KPW;          // lane groups per block
  constexpr int HD = kDecHeads;
  __shared__ int kpos[kDecChunk];
  __shared__ float red_o[NG][HD][DH];
  __shared__ float red_ml[NG][HD][2];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int c = l % CHK, grp = wave * KPW + l / CHK;  // chunk of the row, lane group
  const int64_t lin = blockIdx.x;
  const int sp = (int)(lin % a.splits);
  const int hgrp = (int)((lin / a.splits) % (a.Hq / a.hpb));  // head group
  const int b = (int)(lin / ((int64_t)a.splits * (a.Hq / a.hpb)));
  const int hq0 = hgrp * a.hpb, h = hq0 / a.G;
  const int nh = a.hpb;

  int64_t L = a.cache_len[b];
  if (L < 1) L = 1;
  if (L > a.Lmax) L = a.Lmax;
  const int64_t p = L - 1;
  const int64_t wl = a.window > 1 ? a.window : 1;
  const int64_t lo = p - wl + 1 > 0 ? p - wl + 1 : 0;
  const int64_t nl = p - lo + 1;

  // query groups, segment starts and the number of far members per group
  int qg[4];
  int64_t seg_lo[4], cnt[4];
  const int32_t* off = a.cache_off + (int64_t)b * (a.K + 1);
  const int32_t* cidx = a.cache_idx + (int64_t)b * a.Lmax * a.top_k;
  int64_t total = nl;
  for (int r = 0; r < a.top_k; ++r) {
    int g = a.q_groups[(int64_t)b * a.top_k + r];
    qg[r] = g;
    seg_lo[r] = 0;
    cnt[r] = 0;
    if (g < 0 || g >= a.K) continue;
    int64_t s0 = off[g], s1 = off[g + 1];
    int64_t lo_i = s0, hi_i = s1;  // first member at a position > p - wl
    while (lo_i < hi_i) {
      int64_t mid = (lo_i + hi_i) >> 1;
      if ((int64_t)cidx[mid] <= p - wl) lo_i = mid + 1;
      else hi_i = mid;
    }
    seg_lo[r] = s0;
    cnt[r] = lo_i - s0;
    total += cnt[r];
  }
  const int64_t per = (total + a.splits - 1) / a.splits;
  const int64_t v0 = (int64_t)sp * per;
  const int64_t v1 = v0 + per < total ? v0 + per : total;

  // this lane's slice of the query heads, pre-scaled to log2 units
  float qf[HD][8];
#pragma unroll
  for (int hh = 0; hh < HD; ++hh) {
    const int hq = hq0 + (hh < nh ? hh : 0);
    const i32x4_t raw = *(const i32x4_t*)(a.q + ((int64_t)b * a.Hq + hq) * DH + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[hh][2 * e] = __uint_as_float((uint32_t)raw[e] << 16) * a.sl2;
      qf[hh][2 * e + 1] = __uint_as_float((uint32_t)raw[e] & 0xffff0000u) * a.sl2;
    }
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
  const uint16_t* kbase = a.kc + (int64_t)b * a.Lmax * kv_stride + (int64_t)h * DH + c * 8;
  const uint16_t* vbase = a.vc + (int64_t)b * a.Lmax * kv_stride + (int64_t)h * DH + c * 8;

  for (int64_t c0 = v0; c0 < v1; c0 += kDecChunk) {
    // ---- resolve list entries c0 + tid into key positions (-1: not this query's key)
    {
      const int64_t vi = c0 + tid;
      int pos = -1;
      if (vi < v1) {
        if (vi < nl) {
          pos = (int)(lo + vi);
        } else {
          int64_t rem = vi - nl;
          for (int r = 0; r < a.top_k; ++r) {
            if (rem < cnt[r]) {
              const int cand = cidx[seg_lo[r] + rem];
              // owned by g_r unless the key also holds a lower query group
              bool owned = true;
              const int32_t* kg = a.cache_groups + ((int64_t)b * a.Lmax + cand) * a.top_k;
              for (int r2 = 0; r2 < a.top_k; ++r2) {
                const int g2 = qg[r2];
                if (g2 >= 0 && g2 < a.K && g2 < qg[r])
                  for (int r3 = 0; r3 < a.top_k; ++r3) owned = owned && kg[r3] != g2;
              }
              pos = owned ? cand : -1;
              break;
            }
            rem -= cnt[r];
          }
        }
      }
      kpos[tid] = pos;
    }
    __syncthreads();
    // ---- lane group grp absorbs entries grp, grp + NG, ... of this chunk, 4 at a time
    const int nent = (int)(v1 - c0 < kDecChunk ? v1 - c0 : kDecChunk);
    for (int j0 = grp; j0 < nent; j0 += 4 * NG) {
      int pk[4];
      i32x4_t kr[4], vr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * NG;
        pk[u] = j < nent ? kpos[j] : -1;
        const int64_t row = pk[u] >= 0 ? pk[u] : 0;
        kr[u] = *(const i32x4_t*)(kbase + row * kv_stride);
        vr[u] = *(const i32x4_t*)(vbase + row * kv_stride);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pk[u] < 0) continue;  // uniform within the lane group
        float kf[8], vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = __uint_as_float((uint32_t)kr[u][e] << 16);
          kf[2 * e + 1] = __uint_as_float((uint32_t)kr[u][e] & 0xffff0000u);
          vf[2 * e] = __uint_as_float((uint32_t)vr[u][e] << 16);
          vf[2 * e + 1] = __uint_as_float((uint32_t)vr[u][e] & 0xffff0000u);
        }
#pragma unroll
        for (int hh = 0; hh < HD; ++hh) {
          if (hh >= nh) break;
          float sdot = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sdot = __builtin_fmaf(qf[hh][e], kf[e], sdot);
          sdot = group_sum<CHK>(sdot);
          // lazy running max: rescale only when the score passes the reference by 2^8
          if (sdot > m_run[hh] + 8.f) {
            const float alpha = m_run[hh] == -INFINITY ? 0.f : fast_exp2(m_run[hh] - sdot);
            l_run[hh] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[hh][e] *= alpha;
            m_run[hh] = sdot;
          }
          const float pw = fast_exp2(sdot - m_run[hh]);
          l_run[hh] += pw;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hh][e] = __builtin_fmaf(pw, vf[e], o[hh][e]);
        }
      }
    }
    __syncthreads();
  }

  // ---- merge the lane groups' states and write this block's partial per head
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
  for (int i = tid; i < nh * DH; i += 256) {
    const int hh = i / DH, d = i % DH;
    float M = -INFINITY;
    for (int g = 0; g < NG; ++g) M = fmaxf(M, red_ml[g][hh][0]);
    float lsum = 0.f, acc = 0.f;
    if (M != -INFINITY)
      for (int g = 0; g < NG; ++g) {
        const float m = red_ml[g][hh][0];
        if (m == -INFINITY) continue;
        const float w = fast_exp2(m - M);
        lsum += w * red_ml[g][hh][1];
        acc += w * red_o[g][hh][d];
      }
    const int64_t pi = ((int64_t)b * a.Hq + hq0 + hh) * a.splits + sp;
    a.part_o[pi * DH + d] = acc;
    if (d == 0) {
      a.part_ml[pi * 2] = M;
      a.part_ml[pi * 2 + 1] = lsum;
    }
  }
}

template <int DH>
__global__ __launch_bounds__(DH) void decode_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            int Hq, int Hkv, int G, int splits,
                                                            uint16_t* __restrict__ out,
                                                            float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;  // b * Hq + hq
  (void)Hq;
  (void)Hkv;
  (void)G;
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[(bh * splits + s) * 2]);
  float den = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      int64_t pi = bh * splits + s;
      float m = part_ml[pi * 2];
      if (m == -INFINITY) continue;
      float w = fast_exp2(m - M);
      den += w * part_ml[pi * 2 + 1];
      acc += w * part_o[pi * DH + d];
    }
  }
  float o = den > 0.f ? acc / den : 0.f;
  __bf16 ob = to_bf16(o);
  out[bh * DH + d] = *(uint16_t*)&ob;
  if (d == 0) lse[bh] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
}

hipError_t launch_decode(const uint16_t* q, const int32_t* q_groups, const uint16_t* kc,
                         const uint16_t* vc, const int32_t* cache_len, const int32_t* cache_groups,
                         const int32_t* cache_off, const int32_t* cache_idx, const DecodeShape& s,
                         float* part_o, float* part_ml, uint16_t* out, float* lse,
                         hipStream_t stream) {
  DecodeArgs a{};
  a.q = q;
  a.q_groups = q_groups;
  a.kc = kc;
  a.vc = vc;
  a.cache_len = cache_len;
  a.cache_groups = cache_groups;
  a.cache_off = cache_off;
  a.cache_idx = cache_idx;
  a.B = s.B;
  a.Lmax = s.Lmax;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.K = s.K;
  a.top_k = s.top_k;
  a.splits = s.splits;
  a.window = s.window;
  a.sl2 = s.scale * kLog2e;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.hpb = s.G < kDecHeads ? s.G : kDecHeads;
  const int64_t blocks = (int64_t)s.B * (s.Hq / a.hpb) * s.splits;
  if (s.dh == 128) {
    hipLaunchKernelGGL(decode_partial_kernel<128>, dim3(blocks), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((int64_t)s.B * s.Hq), dim3(128), 0, stream,
                       part_o, part_ml, s.Hq, s.Hkv, s.G, s.splits, out, lse);
  } else {
    hipLaunchKernelGGL(decode_partial_kernel<64>, dim3(blocks), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((int64_t)s.B * s.Hq), dim3(64), 0, stream,
                       part_o, part_ml, s.Hq, s.Hkv, s.G, s.splits, out, lse);
  }
  return hipGetLastError();
}

}  // namespace focus
