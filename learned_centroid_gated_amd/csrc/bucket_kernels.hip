// Stable counting sort of top-k memberships into per-group segments.
//
// The membership sets are those of "Why Attend to Everything? Focus is the Key" (Chinese
// technical summary, gist.science/zh, section 2.1.3: a token belongs to its k best groups and
// only pairs that share a group are computed). Segments list each group's tokens in
// ascending position, which turns causality inside a group into slot order.
//
// Tokens are cut into chunks of kBucketChunk. Four kernels:
//   hist     per (sequence, chunk): count of memberships per group          -> counts[b][g][chunk]
//   chunkscan per (sequence, group): exclusive scan over chunks               -> counts (in place), totals[b][g]
//   groupscan per sequence: exclusive scan over groups                        -> offsets[b][*]
//   scatter  per (sequence, chunk): one wave walks the chunk 64 tokens at a time; the rank of a
//            membership among equal groups of earlier tokens in the same 64 comes from a
//            compare loop over LDS, so slot order equals token order inside every segment.
#include "focus_internal.hpp"

namespace focus {

__global__ __launch_bounds__(256) void bucket_hist_kernel(const int32_t* __restrict__ groups,
                                                          int64_t n, int K, int top_k, int nchunks,
                                                          int32_t* __restrict__ counts) {
  __shared__ int cnt[1024];
  const int chunk = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  for (int c = t; c < K; c += 256) cnt[c] = 0;
  __syncthreads();
  const int64_t tok = (int64_t)chunk * kBucketChunk + t;
  if (t < kBucketChunk && tok < n) {
    const int32_t* gp = groups + ((int64_t)b * n + tok) * top_k;
    for (int r = 0; r < top_k; ++r) {
      int g = gp[r];
      if (g >= 0 && g < K) atomicAdd(&cnt[g], 1);
    }
  }
  __syncthreads();
  int32_t* out = counts + (int64_t)b * K * nchunks;
  for (int c = t; c < K; c += 256) out[(int64_t)c * nchunks + chunk] = cnt[c];
}

// Exclusive scan of counts[b][g][0..nchunks) in place; totals[b][g] = the sum.
__global__ __launch_bounds__(256) void bucket_chunkscan_kernel(int32_t* __restrict__ counts,
                                                               int K, int nchunks,
                                                               int32_t* __restrict__ totals) {
  __shared__ int wsum[4];
  __shared__ int carry_s;
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x, l = t & 63, w = t >> 6;
  int32_t* row = counts + ((int64_t)b * K + g) * nchunks;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < nchunks; base += 256) {
    int i = base + t;
    int x = i < nchunks ? row[i] : 0;
    int incl = x;
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(incl, o, 64);
      if (l >= o) incl += y;
    }
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    int wbase = 0;
    for (int q = 0; q < w; ++q) wbase += wsum[q];
    int carry = carry_s;
    if (i < nchunks) row[i] = carry + wbase + incl - x;
    __syncthreads();
    if (t == 255) carry_s = carry + wbase + incl;
    __syncthreads();
  }
  if (t == 0) totals[(int64_t)b * K + g] = carry_s;
}

// offsets[b][g] = exclusive scan of totals over groups; unused idx slots set to -1.
__global__ __launch_bounds__(1024) void bucket_groupscan_kernel(const int32_t* __restrict__ totals,
                                                                int K, int64_t nk,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ idx) {
  __shared__ int wsum[16];
  const int b = blockIdx.x, t = threadIdx.x, l = t & 63, w = t >> 6;
  int x = t < K ? totals[(int64_t)b * K + t] : 0;
  int incl = x;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (l >= o) incl += y;
  }
  if (l == 63) wsum[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int q = 0; q < w; ++q) wbase += wsum[q];
  int32_t* off = offsets + (int64_t)b * (K + 1);
  if (t < K) off[t] = wbase + incl - x;
  int total = 0;
  for (int q = 0; q < 16; ++q) total += wsum[q];
  if (t == 0) off[K] = total;
  for (int64_t s = total + t; s < nk; s += 1024) idx[(int64_t)b * nk + s] = -1;
}

__global__ __launch_bounds__(64) void bucket_scatter_kernel(const int32_t* __restrict__ groups,
                                                            int64_t n, int K, int top_k, int nchunks,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ slot) {
  __shared__ int ctr[1024];
  __shared__ int bg[64 * 8];
  const int chunk = blockIdx.x, b = blockIdx.y, l = threadIdx.x;
  const int64_t nk = n * top_k;
  const int32_t* cb = counts + (int64_t)b * K * nchunks;
  const int32_t* off = offsets + (int64_t)b * (K + 1);
  for (int c = l; c < K; c += 64) ctr[c] = off[c] + cb[(int64_t)c * nchunks + chunk];
  const int64_t t0 = (int64_t)chunk * kBucketChunk;
  for (int s0 = 0; s0 < kBucketChunk; s0 += 64) {
    const int64_t tok = t0 + s0 + l;
    int my[8];
    for (int r = 0; r < top_k; ++r) {
      int g = -1;
      if (tok < n) {
        g = groups[((int64_t)b * n + tok) * top_k + r];
        if (g < 0 || g >= K) g = -1;
      }
      my[r] = g;
      bg[l * top_k + r] = g;
    }
    __syncthreads();
    int rank[8];
    for (int r = 0; r < top_k; ++r) rank[r] = 0;
    for (int jl = 0; jl < 64; ++jl) {
      const bool earlier = jl < l;
      for (int r2 = 0; r2 < top_k; ++r2) {
        int gj = bg[jl * top_k + r2];
        for (int r = 0; r < top_k; ++r) rank[r] += (earlier && gj == my[r] && gj >= 0) ? 1 : 0;
      }
    }
    int base[8];
    for (int r = 0; r < top_k; ++r) base[r] = my[r] >= 0 ? ctr[my[r]] : 0;
    __syncthreads();
    for (int r = 0; r < top_k; ++r) {
      if (tok >= n) break;
      int32_t s = -1;
      if (my[r] >= 0) {
        s = base[r] + rank[r];
        idx[(int64_t)b * nk + s] = (int32_t)tok;
        atomicAdd(&ctr[my[r]], 1);
      }
      slot[((int64_t)b * n + tok) * top_k + r] = s;
    }
    __syncthreads();
  }
}

__global__ void fill_i32_kernel(int32_t* p, int32_t value, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t count, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, stream, p, value, count);
  return hipGetLastError();
}

hipError_t launch_bucket(const int32_t* groups, int batch, int64_t n, int K, int top_k,
                         int32_t* offsets, int32_t* idx, int32_t* slot, int32_t* counts,
                         int32_t* totals, hipStream_t stream) {
  const int nchunks = (int)((n + kBucketChunk - 1) / kBucketChunk);
  hipLaunchKernelGGL(bucket_hist_kernel, dim3(nchunks, batch), dim3(256), 0, stream, groups, n, K,
                     top_k, nchunks, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bucket_chunkscan_kernel, dim3(K, batch), dim3(256), 0, stream, counts, K,
                     nchunks, totals);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bucket_groupscan_kernel, dim3(batch), dim3(1024), 0, stream, totals, K,
                     n * top_k, offsets, idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nchunks, batch), dim3(64), 0, stream, groups, n,
                     K, top_k, nchunks, counts, offsets, idx, slot);
  return hipGetLastError();
}

// ============================================================================ append
// One new token per sequence joins the bucketed memberships: its position is the largest so
// far, so each of its memberships goes at the end of its group's segment and every segment
// keeps ascending positions. Block (g, b) copies segment g of sequence b to its new place
// (shifted by the new memberships in lower groups) and appends the new token's entries of g.
__global__ __launch_bounds__(256) void bucket_append_kernel(const int32_t* __restrict__ new_groups,
                                                            const int32_t* __restrict__ cache_len,
                                                            int64_t cap, int K, int top_k,
                                                            const int32_t* __restrict__ off_in,
                                                            const int32_t* __restrict__ idx_in,
                                                            int32_t* __restrict__ off_out,
                                                            int32_t* __restrict__ idx_out) {
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int32_t pos = cache_len[b] - 1;  // the new token (no new token when the cache is empty)
  int lt = 0, eq = 0, valid = 0;
  if (pos >= 0) {
    for (int r = 0; r < top_k; ++r) {
      const int x = new_groups[(int64_t)b * top_k + r];
      if (x < 0 || x >= K) continue;  // dropped, as in the bucket sort
      ++valid;
      lt += x < g;
      eq += x == g;
    }
  }
  const int32_t* oi = off_in + (int64_t)b * (K + 1);
  int32_t* oo = off_out + (int64_t)b * (K + 1);
  // offsets that do not describe a bucket of at most cap - valid entries are treated as empty
  // segments, so no access leaves the index lists
  int32_t s0 = oi[g], s1 = oi[g + 1];
  if (s0 < 0 || s1 < s0 || (int64_t)s1 + valid > cap) s0 = s1 = 0;
  const int32_t d0 = s0 + lt;
  const int32_t* src = idx_in + (int64_t)b * cap;
  int32_t* dst = idx_out + (int64_t)b * cap;
  for (int32_t i = t; i < s1 - s0; i += 256) dst[d0 + i] = src[s0 + i];
  if (t < eq) dst[d0 + (s1 - s0) + t] = pos;
  if (t == 0) {
    oo[g] = d0;
    if (g == K - 1) oo[K] = oi[K] + valid;
  }
}

hipError_t launch_bucket_append(const int32_t* new_groups, const int32_t* cache_len, int batch,
                                int64_t cap, int K, int top_k, const int32_t* off_in,
                                const int32_t* idx_in, int32_t* off_out, int32_t* idx_out,
                                hipStream_t stream) {
  hipLaunchKernelGGL(bucket_append_kernel, dim3(K, batch), dim3(256), 0, stream, new_groups,
                     cache_len, cap, K, top_k, off_in, idx_in, off_out, idx_out);
  return hipGetLastError();
}

// ============================================================================ group slots
// Group-slotted memberships: the members of group g of sequence b are
// seg_pos[(b * K + g) * gcap + i] for i < seg_len[b * K + g], positions ascending. A new token is
// the newest of its sequence, so it joins each of its groups with one write at the end of that
// group's row: O(top_k) work per token. overflow[0] is set to 1 (and never cleared here) when a
// group would hold more than gcap members; those members are not stored.

// Block (g, b) copies segment g of sequence b from a bucket (offsets and index lists of
// capacity cap per sequence) into its row.
__global__ __launch_bounds__(256) void slots_from_bucket_kernel(const int32_t* __restrict__ off,
                                                                const int32_t* __restrict__ idx,
                                                                int64_t cap, int K, int gcap,
                                                                int32_t* __restrict__ seg_len,
                                                                int32_t* __restrict__ seg_pos,
                                                                int32_t* __restrict__ overflow) {
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int32_t* o = off + (int64_t)b * (K + 1);
  int32_t s0 = o[g], s1 = o[g + 1];
  if (s0 < 0 || s1 < s0 || (int64_t)s1 > cap) s0 = s1 = 0;  // not a bucket of this capacity
  int32_t n = s1 - s0;
  if (n > gcap) {
    if (t == 0) overflow[0] = 1;
    n = gcap;
  }
  const int32_t* src = idx + (int64_t)b * cap + s0;
  int32_t* dst = seg_pos + ((int64_t)b * K + g) * gcap;
  for (int32_t i = t; i < n; i += 256) dst[i] = src[i];
  if (t == 0) seg_len[(int64_t)b * K + g] = n;
}

// Thread (b, r) appends position cache_len[b] - 1 to the row of the token's r-th group. Invalid
// ids are dropped and a repeated id joins once, so no two threads touch one row.
__global__ __launch_bounds__(64) void slots_append_kernel(const int32_t* __restrict__ new_groups,
                                                          const int32_t* __restrict__ cache_len,
                                                          int batch, int K, int top_k, int gcap,
                                                          int32_t* __restrict__ seg_len,
                                                          int32_t* __restrict__ seg_pos,
                                                          int32_t* __restrict__ overflow) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i >= (int64_t)batch * top_k) return;
  const int b = (int)(i / top_k), r = (int)(i % top_k);
  const int32_t pos = cache_len[b] - 1;
  const int g = new_groups[i];
  if (pos < 0 || g < 0 || g >= K) return;
  for (int r2 = 0; r2 < r; ++r2)
    if (new_groups[(int64_t)b * top_k + r2] == g) return;
  int32_t* len = seg_len + (int64_t)b * K + g;
  const int32_t l = *len;
  if (l < 0 || l >= gcap) {
    overflow[0] = 1;
    return;
  }
  seg_pos[((int64_t)b * K + g) * gcap + l] = pos;
  *len = l + 1;
}

hipError_t launch_slots_from_bucket(const int32_t* off, const int32_t* idx, int batch, int64_t cap,
                                    int K, int gcap, int32_t* seg_len, int32_t* seg_pos,
                                    int32_t* overflow, hipStream_t stream) {
  hipLaunchKernelGGL(slots_from_bucket_kernel, dim3(K, batch), dim3(256), 0, stream, off, idx,
                     cap, K, gcap, seg_len, seg_pos, overflow);
  return hipGetLastError();
}

hipError_t launch_slots_append(const int32_t* new_groups, const int32_t* cache_len, int batch,
                               int K, int top_k, int gcap, int32_t* seg_len, int32_t* seg_pos,
                               int32_t* overflow, hipStream_t stream) {
  const int64_t n = (int64_t)batch * top_k;
  hipLaunchKernelGGL(slots_append_kernel, dim3((n + 63) / 64), dim3(64), 0, stream, new_groups,
                     cache_len, batch, K, top_k, gcap, seg_len, seg_pos, overflow);
  return hipGetLastError();
}

}  // namespace focus
