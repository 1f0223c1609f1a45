// Batched single-token decode against per-sequence caches with cached group memberships.
//
// Inference rule of "Why Attend to Everything? Focus is the Key" (Chinese technical summary,
// gist.science/zh, section 2.1.3): the new token attends its window and the members of the
// groups it joins. For sequence b the query sits at position p = L_b - 1. Its keys form a
// virtual list: the window [max(0, p - w' + 1), p] with w' = max(window, 1) (the token always
// sees itself), then for each query group g_r the segment members at positions <= p - w'
// whose lowest group shared with the query is g_r, so every allowed key appears once.
//
// The list is cut into `splits` contiguous pieces per (sequence, kv head). A 256-thread block
// scores one key per thread (G query heads, q in LDS), then accumulates P V with one V row per
// wave instruction; running (max, sum, O) per head give one partial, and a second kernel merges
// the partials by their log-sum-exp. The path is HBM-bound: every allowed key costs one K row
// and one V row of the kv head.
#include "focus_internal.hpp"

namespace focus {

constexpr int kDecChunk = 256;
constexpr int kDecMaxG = 16;

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
  int Hq, Hkv, G, K, top_k, splits;
  int64_t window;
  float sl2;
  float* part_o;   // [B, Hkv, splits, G, DH] unnormalised
  float* part_ml;  // [B, Hkv, splits, G, 2] (running max in log2 units, sum)
};

template <int DH>
__global__ __launch_bounds__(256) void decode_partial_kernel(const DecodeArgs a) {
  constexpr int VPL = DH / 64;  // value dims per lane in the P V phase
  __shared__ float qs[kDecMaxG * DH];
  __shared__ float sc[kDecMaxG * kDecChunk];
  __shared__ float red[4 * kDecMaxG * DH];
  __shared__ float stat[kDecMaxG * 2];
  __shared__ float alpha_s[kDecMaxG];
  __shared__ int kpos[kDecChunk];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int64_t lin = blockIdx.x;
  const int sp = (int)(lin % a.splits);
  const int h = (int)((lin / a.splits) % a.Hkv);
  const int b = (int)(lin / ((int64_t)a.splits * a.Hkv));
  const int G = a.G;

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

  for (int i = tid; i < G * DH; i += 256) {
    int hl = i / DH, d = i % DH;
    uint16_t bits = a.q[((int64_t)b * a.Hq + h * G + hl) * DH + d];
    qs[i] = __uint_as_float((uint32_t)bits << 16);
  }
  if (tid < G) {
    stat[2 * tid] = -INFINITY;
    stat[2 * tid + 1] = 0.f;
  }
  float oacc[kDecMaxG][VPL];
  for (int hl = 0; hl < kDecMaxG; ++hl)
    for (int e = 0; e < VPL; ++e) oacc[hl][e] = 0.f;
  __syncthreads();

  const int64_t kv_stride = (int64_t)a.Hkv * DH;
  const uint16_t* kbase = a.kc + (int64_t)b * a.Lmax * kv_stride + (int64_t)h * DH;
  const uint16_t* vbase = a.vc + (int64_t)b * a.Lmax * kv_stride + (int64_t)h * DH;

  for (int64_t c0 = v0; c0 < v1; c0 += kDecChunk) {
    // ---- resolve this thread's key and score it against the G query heads
    const int64_t vi = c0 + tid;
    int pos = -1;
    if (vi < v1) {
      if (vi < nl) {
        pos = (int)(lo + vi);
      } else {
        int64_t rem = vi - nl;
        for (int r = 0; r < a.top_k; ++r) {
          if (rem < cnt[r]) {
            int cand = cidx[seg_lo[r] + rem];
            // owned by g_r unless the key also holds a lower query group
            bool owned = true;
            const int32_t* kg = a.cache_groups + ((int64_t)b * a.Lmax + cand) * a.top_k;
            for (int r2 = 0; r2 < a.top_k; ++r2) {
              int g2 = qg[r2];
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
    float s[kDecMaxG];
    for (int hl = 0; hl < G; ++hl) s[hl] = 0.f;
    if (pos >= 0) {
      const uint16_t* kp = kbase + (int64_t)pos * kv_stride;
      for (int d8 = 0; d8 < DH / 8; ++d8) {
        i32x4_t raw = *(const i32x4_t*)(kp + d8 * 8);
        float kf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t w = (uint32_t)raw[e];
          kf[2 * e] = __uint_as_float(w << 16);
          kf[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
        }
        for (int hl = 0; hl < G; ++hl) {
          const float* qq = qs + hl * DH + d8 * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) s[hl] += qq[e] * kf[e];
        }
      }
    }
    for (int hl = 0; hl < G; ++hl) sc[hl * kDecChunk + tid] = pos >= 0 ? s[hl] * a.sl2 : -INFINITY;
    __syncthreads();
    // ---- online softmax statistics per head: wave w handles heads w, w+4, ...
    for (int hl = wave; hl < G; hl += 4) {
      float mx = -INFINITY;
      for (int i = l; i < kDecChunk; i += 64) mx = fmaxf(mx, sc[hl * kDecChunk + i]);
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
      const float m_old = stat[2 * hl];
      const float m_new = fmaxf(m_old, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float sum = 0.f;
      for (int i = l; i < kDecChunk; i += 64) {
        float pp = fast_exp2(sc[hl * kDecChunk + i] - m_use);
        sc[hl * kDecChunk + i] = pp;
        sum += pp;
      }
      for (int o = 32; o >= 1; o >>= 1) sum += shfl_xor_f(sum, o);
      if (l == 0) {
        const float alpha = fast_exp2(m_old - m_use);
        stat[2 * hl] = m_new;
        stat[2 * hl + 1] = stat[2 * hl + 1] * alpha + sum;
        alpha_s[hl] = alpha;
      }
    }
    __syncthreads();
    // ---- rescale O and accumulate P V: wave w takes keys w, w+4, ...; lane l dims VPL*l..
    for (int hl = 0; hl < G; ++hl) {
      const float alpha = alpha_s[hl];
      for (int e = 0; e < VPL; ++e) oacc[hl][e] *= alpha;
    }
    for (int kk = wave; kk < kDecChunk; kk += 4) {
      const int kp = kpos[kk];
      if (kp < 0) continue;
      float vf[VPL];
      if constexpr (VPL == 2) {
        uint32_t w = *(const uint32_t*)(vbase + (int64_t)kp * kv_stride + 2 * l);
        vf[0] = __uint_as_float(w << 16);
        vf[1] = __uint_as_float(w & 0xffff0000u);
      } else {
        uint16_t w = vbase[(int64_t)kp * kv_stride + l];
        vf[0] = __uint_as_float((uint32_t)w << 16);
      }
      for (int hl = 0; hl < G; ++hl) {
        const float pp = sc[hl * kDecChunk + kk];
        for (int e = 0; e < VPL; ++e) oacc[hl][e] += pp * vf[e];
      }
    }
    __syncthreads();
  }
  // ---- reduce the 4 waves' O and write the partial
  for (int hl = 0; hl < G; ++hl)
    for (int e = 0; e < VPL; ++e) red[(wave * kDecMaxG + hl) * DH + VPL * l + e] = oacc[hl][e];
  __syncthreads();
  const int64_t pbase = (((int64_t)b * a.Hkv + h) * a.splits + sp) * G;
  for (int i = tid; i < G * DH; i += 256) {
    int hl = i / DH, d = i % DH;
    float x = 0.f;
    for (int w = 0; w < 4; ++w) x += red[(w * kDecMaxG + hl) * DH + d];
    a.part_o[(pbase + hl) * DH + d] = x;
  }
  if (tid < G) {
    a.part_ml[(pbase + tid) * 2] = stat[2 * tid];
    a.part_ml[(pbase + tid) * 2 + 1] = stat[2 * tid + 1];
  }
}

template <int DH>
__global__ __launch_bounds__(DH) void decode_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            int Hq, int Hkv, int G, int splits,
                                                            uint16_t* __restrict__ out,
                                                            float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;  // b * Hq + hq
  const int b = (int)(bh / Hq), hq = (int)(bh % Hq);
  const int h = hq / G, hl = hq % G;
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) {
    int64_t pi = (((int64_t)b * Hkv + h) * splits + s) * G + hl;
    M = fmaxf(M, part_ml[pi * 2]);
  }
  float den = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      int64_t pi = (((int64_t)b * Hkv + h) * splits + s) * G + hl;
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
  const int64_t blocks = (int64_t)s.B * s.Hkv * s.splits;
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
