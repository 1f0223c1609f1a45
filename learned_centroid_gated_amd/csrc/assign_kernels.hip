// Centroid group assignment on gfx950: scores S = (H W_g) C^T on the matrix cores (fp32
// operands split exactly into two fp16 parts, or three bf16 parts), log-domain Sinkhorn
// balancing and top-k membership.
//
// Method: "Why Attend to Everything? Focus is the Key" (Chinese technical summary,
// gist.science/zh, section 2.1.1: projection into centroid space, similarity to K centroids,
// Sinkhorn in place of softmax so each group gets equal token mass; section 2.1.3: each token
// joins its k highest-scoring groups at inference).
#include <type_traits>

#include "focus_internal.hpp"

namespace focus {

// ============================================================================ NT GEMM
// C[m, n] = sum_k A[m, k] * B[n, k] for fp32 A, B, C on the bf16 matrix cores.
//
// Each fp32 operand x is split into three bf16 parts x = h + m + l + r: h = bf16(x),
// m = bf16(x - h), l = bf16(x - h - m), rounding to nearest even, with both subtractions exact
// in fp32. bf16 keeps 8 significant bits, so |m| <= 2^-8 |x|, |l| <= 2^-16 |x| and
// |r| <= 2^-24 |x|. A product a b keeps the six part products hh, hm, mh, hl, mm, lh; the
// dropped ones (ml, lm, ll) and the residues add up to less than about 2^-22 |a b|, i.e.
// fp32-level relative error. The six 32x32x16 bf16 MFMAs take 192 cycles where the fp32 MFMA
// needs 512 for the same block.
//
// Block tile 128 x (32*NT), k-chunks of 32: the chunk's fp32 tiles come from global memory into
// registers one chunk ahead, are split, and are stored as three bf16 planes per operand in
// LDS. A plane row holds the chunk's 32 values in four 16-byte quarters, quarter q of row r
// stored at position q ^ ((r / 4) % 4): 16 lanes reading one quarter of 16 consecutive rows
// (an MFMA operand) hit 16 distinct bank quads, and 8-byte writes of 8 whole rows cover every
// bank exactly twice. Each wave owns 32 rows and NT 32x32 accumulator tiles.
__device__ __forceinline__ int plane_at(int r, int c) {  // bf16 index of row r, column c < 32
  return r * 32 + (((c >> 3) ^ ((r >> 2) & 3)) << 3) + (c & 7);
}
struct Bf16x4Planes {
  bf16x4_t h, m, l;
};
__device__ __forceinline__ Bf16x4Planes split3(f32x4_t x) {
  Bf16x4Planes p;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h = (__bf16)x[e];
    const float r1 = x[e] - (float)h;
    const __bf16 m = (__bf16)r1;
    const float r2 = r1 - (float)m;
    p.h[e] = h;
    p.m[e] = m;
    p.l[e] = (__bf16)r2;
  }
  return p;
}

template <int NT>
__global__ __launch_bounds__(256, 3) void gemm_nt_split_kernel(const float* __restrict__ A,
                                                            const float* __restrict__ B,
                                                            float* __restrict__ C, int64_t M,
                                                            int N, int Kd, int ldc) {
  constexpr int BM = 128, BN = 32 * NT, BK = 32;
  __shared__ __attribute__((aligned(16))) __bf16 As[3][BM * BK];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[3][BN * BK];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, j = l & 31, g = l >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16_t{};

  f32x4_t ra[4], rb[NT];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + 256 * i, r = e >> 3, c = (e & 7) * 4;
      int64_t gr = m0 + r;
      ra[i] = (gr < M && k0 + c < Kd) ? *(const f32x4_t*)(A + gr * Kd + k0 + c) : f32x4_t{};
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      int e = tid + 256 * i, r = e >> 3, c = (e & 7) * 4;
      int gr = n0 + r;
      rb[i] = (gr < N && k0 + c < Kd) ? *(const f32x4_t*)(B + (int64_t)gr * Kd + k0 + c) : f32x4_t{};
    }
  };

  load(0);
  for (int k0 = 0; k0 < Kd; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + 256 * i, r = e >> 3, c = (e & 7) * 4;
      const Bf16x4Planes pl = split3(ra[i]);
      const int o = plane_at(r, c);
      *(bf16x4_t*)&As[0][o] = pl.h;
      *(bf16x4_t*)&As[1][o] = pl.m;
      *(bf16x4_t*)&As[2][o] = pl.l;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      int e = tid + 256 * i, r = e >> 3, c = (e & 7) * 4;
      const Bf16x4Planes pl = split3(rb[i]);
      const int o = plane_at(r, c);
      *(bf16x4_t*)&Bs[0][o] = pl.h;
      *(bf16x4_t*)&Bs[1][o] = pl.m;
      *(bf16x4_t*)&Bs[2][o] = pl.l;
    }
    __syncthreads();
    if (k0 + BK < Kd) load(k0 + BK);

#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
        a[p] = *(const bf16x8_t*)&As[p][plane_at(wave * 32 + j, ks * 16 + 8 * g)];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8_t b[3];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          b[p] = *(const bf16x8_t*)&Bs[p][plane_at(t * 32 + j, ks * 16 + 8 * g)];
        // small terms first
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[2], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[t], 0, 0, 0);
      }
    }
  }

  // 32x32 accumulator layout: lane l holds column l % 32, rows 8*(v/4) + 4*(l/32) + v%4.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int col = n0 + t * 32 + j;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int64_t row = m0 + wave * 32 + (v >> 2) * 8 + 4 * g + (v & 3);
      if (row < M && col < N) C[row * ldc + col] = acc[t][v];
    }
  }
}

hipError_t launch_gemm_nt_f32(const float* A, const float* B, float* C, int64_t M, int N, int Kd,
                              int ldc, hipStream_t stream) {
  dim3 block(256);
  int64_t mb = (M + 127) / 128;
  if (N <= 32) {
    hipLaunchKernelGGL(gemm_nt_split_kernel<1>, dim3(mb, (N + 31) / 32), block, 0, stream, A, B, C,
                       M, N, Kd, ldc);
  } else if (N <= 64) {
    hipLaunchKernelGGL(gemm_nt_split_kernel<2>, dim3(mb, (N + 63) / 64), block, 0, stream, A, B, C,
                       M, N, Kd, ldc);
  } else {
    hipLaunchKernelGGL(gemm_nt_split_kernel<4>, dim3(mb, (N + 127) / 128), block, 0, stream, A, B,
                       C, M, N, Kd, ldc);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- planes GEMM
// The same product when B has been split once into its planes (Bp[3][N][Kd], bf16): instead of
// every block loading and splitting the shared B tile for every k-chunk, the chunk's planes go
// from memory straight into LDS (global_load_lds, per-lane offsets that apply the quarter
// permutation) into a double buffer, one chunk ahead of the MFMAs that read them.
__global__ __launch_bounds__(256) void split_planes_kernel(const float* __restrict__ B,
                                                           int64_t count, __bf16* __restrict__ P) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < count;
       i += (int64_t)gridDim.x * 256 * 4) {
    if (i + 4 <= count) {
      const Bf16x4Planes pl = split3(*(const f32x4_t*)(B + i));
      *(bf16x4_t*)(P + i) = pl.h;
      *(bf16x4_t*)(P + count + i) = pl.m;
      *(bf16x4_t*)(P + 2 * count + i) = pl.l;
    } else {
      for (int64_t j = i; j < count; ++j) {
        const __bf16 h = (__bf16)B[j];
        const float r1 = B[j] - (float)h;
        const __bf16 m = (__bf16)r1;
        P[j] = h;
        P[count + j] = m;
        P[2 * count + j] = (__bf16)(r1 - (float)m);
      }
    }
  }
}

template <int NT>
__global__ __launch_bounds__(256, 2) void gemm_nt_planes_kernel(const float* __restrict__ A,
                                                                const __bf16* __restrict__ Bp,
                                                                float* __restrict__ C, int64_t M,
                                                                int N, int Kd, int ldc) {
  constexpr int BM = 128, BN = 32 * NT, BK = 32;
  constexpr int BTILE = 3 * BN * BK;             // bf16 per B tile (three planes)
  constexpr int BINSTS = BTILE * 2 / 1024;       // 1 KB copies per B tile
  constexpr int BPW = (BINSTS + 3) / 4;          // per wave
  __shared__ __attribute__((aligned(1024))) __bf16 As[3][BM * BK];
  __shared__ __attribute__((aligned(1024))) __bf16 Bs[2][BTILE];
  const int tid = threadIdx.x, l = tid & 63, j = l & 31, g = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;

  // copy ii of a B tile fills rows 16 (ii % (BN / 16)) .. + 15 of plane ii / (BN / 16); lane L
  // lands at row + L / 4, physical quarter L % 4, which holds logical quarter
  // (L % 4) ^ ((row / 4) % 4). Rows past N re-read row N - 1 (their columns are never stored).
  uint32_t boff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int ii = wave + 4 * i;
    const int pl = ii / (BN / 16), rb = ii % (BN / 16);
    const int r = rb * 16 + l / 4;
    const int q = (l % 4) ^ ((r >> 2) & 3);
    const int row = min(n0 + r, N - 1);
    boff[i] = (uint32_t)((((int64_t)pl * N + row) * Kd + 8 * q) * 2);
  }
  auto copy_b = [&](int k0, __bf16* dst) __attribute__((always_inline)) {
    const char* base = (const char*)(Bp + k0);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int ii = wave + 4 * i;
      if (ii < BINSTS) dma16(base, boff[i], (char*)dst + ii * 1024);
    }
  };
  auto lds_barrier = []() __attribute__((always_inline)) {  // LDS only: copies stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16_t{};

  f32x4_t ra[4];
  auto load_a = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + 256 * i, r = e >> 3, c = (e & 7) * 4;
      int64_t gr = m0 + r;
      ra[i] = gr < M ? *(const f32x4_t*)(A + gr * Kd + k0 + c) : f32x4_t{};
    }
  };

  // one k-chunk; the loop is unrolled by two so each B buffer is a fixed LDS address
  auto chunk = [&](int k0, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;  // B buffer of this chunk
    lds_barrier();  // every wave is done with As and with the other B buffer
    // The wait for ra below (vmcnt(0): these are the newest loads) also covers this chunk's B
    // copies, which went out before them.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + 256 * i, r = e >> 3, c = (e & 7) * 4;
      const Bf16x4Planes pl = split3(ra[i]);
      const int o = plane_at(r, c);
      *(bf16x4_t*)&As[0][o] = pl.h;
      *(bf16x4_t*)&As[1][o] = pl.m;
      *(bf16x4_t*)&As[2][o] = pl.l;
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (k0 + BK < Kd) {
      copy_b(k0 + BK, Bs[P ^ 1]);
      load_a(k0 + BK);
    }
    lds_barrier();  // As and this chunk's B planes are in LDS
    const __bf16* bsb = Bs[P];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
        a[p] = *(const bf16x8_t*)&As[p][plane_at(wave * 32 + j, ks * 16 + 8 * g)];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8_t b[3];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          b[p] = *(const bf16x8_t*)&bsb[p * BN * BK + plane_at(t * 32 + j, ks * 16 + 8 * g)];
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[2], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[t], 0, 0, 0);
      }
    }
  };
  copy_b(0, Bs[0]);
  load_a(0);
  for (int k0 = 0; k0 < Kd; k0 += 2 * BK) {
    chunk(k0, std::integral_constant<int, 0>{});
    if (k0 + BK < Kd) chunk(k0 + BK, std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int col = n0 + t * 32 + j;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int64_t row = m0 + wave * 32 + (v >> 2) * 8 + 4 * g + (v & 3);
      if (row < M && col < N) C[row * ldc + col] = acc[t][v];
    }
  }
}

hipError_t launch_split_planes(const float* B, int64_t count, __bf16* P, hipStream_t stream) {
  int64_t blocks = (count + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(split_planes_kernel, dim3(blocks), dim3(256), 0, stream, B, count, P);
  return hipGetLastError();
}

hipError_t launch_gemm_nt_f32_planes(const float* A, const __bf16* Bp, float* C, int64_t M, int N,
                                     int Kd, int ldc, hipStream_t stream) {
  if (Kd % 32 != 0) return hipErrorInvalidValue;
  dim3 block(256);
  int64_t mb = (M + 127) / 128;
  if (N <= 32) {
    hipLaunchKernelGGL(gemm_nt_planes_kernel<1>, dim3(mb, (N + 31) / 32), block, 0, stream, A, Bp,
                       C, M, N, Kd, ldc);
  } else if (N <= 64) {
    hipLaunchKernelGGL(gemm_nt_planes_kernel<2>, dim3(mb, (N + 63) / 64), block, 0, stream, A, Bp,
                       C, M, N, Kd, ldc);
  } else {
    hipLaunchKernelGGL(gemm_nt_planes_kernel<4>, dim3(mb, (N + 127) / 128), block, 0, stream, A,
                       Bp, C, M, N, Kd, ldc);
  }
  return hipGetLastError();
}

// ============================================================================ row layouts
// A row of K scores is spread over LPR lanes; lane q of the row holds columns
// 4q + 4*LPR*c + e (c < CPL, e < 4). Rows per wave: 64 / LPR.
// Row reductions over the row's LPR lanes (an aligned group): within a 16-lane row by VALU
// lane moves (pairs, quads, half-row mirror, row mirror: each step combines two disjoint
// halves of the group so far), across rows by lane shuffles.
template <int LPR>
__device__ __forceinline__ float row_max(float x) {
  if constexpr (LPR >= 2) x = fmaxf(x, dpp_move<0xB1>(x));
  if constexpr (LPR >= 4) x = fmaxf(x, dpp_move<0x4E>(x));
  if constexpr (LPR >= 8) x = fmaxf(x, dpp_move<0x141>(x));
  if constexpr (LPR >= 16) x = fmaxf(x, dpp_move<0x140>(x));
  if constexpr (LPR >= 32) x = fmaxf(x, shfl_xor_f(x, 16));
  if constexpr (LPR >= 64) x = fmaxf(x, shfl_xor_f(x, 32));
  return x;
}
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR >= 2) x += dpp_move<0xB1>(x);
  if constexpr (LPR >= 4) x += dpp_move<0x4E>(x);
  if constexpr (LPR >= 8) x += dpp_move<0x141>(x);
  if constexpr (LPR >= 16) x += dpp_move<0x140>(x);
  if constexpr (LPR >= 32) x += shfl_xor_f(x, 16);
  if constexpr (LPR >= 64) x += shfl_xor_f(x, 32);
  return x;
}

// Merge two (max, sum) summaries of exp: sum_i exp(x_i) = exp(m) * s.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * fast_exp2((m - M) * kLog2e) + s2 * fast_exp2((m2 - M) * kLog2e);
  m = M;
}

// ---------------------------------------------------------------------------- fp16 pair GEMM
// The same product from two-part fp16 splits on the fp16 matrix cores: x = h + m + r with
// h = fp16(x), m = fp16(x - h) (the subtraction is exact in fp32), rounding to nearest even.
// fp16 keeps 11 significant bits, so |m| <= 2^-11 |x| and |r| <= 2^-22 |x| while x - h is in
// fp16's normal range; below it (|x| < 2^-3) r is at most 2^-25 in absolute value. A product
// keeps hh, hm and mh; the dropped mm and the residues leave less than about 3 * 2^-22 of
// sum_k |a_k b_k| per output (plus 2^-25 sum_k |b_k| for A's small elements): fp32-level
// accuracy from three part products where the bf16 split needs six.
//
// fp16's range: each row n of B is scaled by an exact power of two 2^e_n that puts its largest
// magnitude in [2^14, 2^15) before splitting (split_pairs_kernel), and the output column is
// multiplied back by 2^-e_n. A is split as it is, so an element of magnitude above fp16's
// largest finite value (65504) or a non-finite one makes its row's outputs non-finite: such
// rows are appended to a list (flag_list, counted by flag_count) for an exact recomputation.
//
// Block tile (32 WAVES) x (32 NT), k-chunks of 32 as in the bf16 kernels: A streams from global
// memory into registers one chunk ahead and is split into two fp16 planes in LDS; B's planes
// were split once per call and go from memory straight into a double buffer in LDS.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

struct F16x4Pair {
  f16x4_t h, m;
};
__device__ __forceinline__ F16x4Pair split_pair(f32x4_t x) {
  F16x4Pair p;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const _Float16 h = (_Float16)x[e];
    p.h[e] = h;
    p.m[e] = (_Float16)(x[e] - (float)h);
  }
  return p;
}

// P[0][n][k] = h and P[1][n][k] = m of B[n][k] 2^e_n; scale_inv[n] = 2^-e_n. One block per row.
__global__ __launch_bounds__(256) void split_pairs_kernel(const float* __restrict__ B, int Kd,
                                                          int64_t count, _Float16* __restrict__ P,
                                                          float* __restrict__ scale_inv) {
  __shared__ float red[4];
  const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * Kd;
  float mx = 0.f;
  for (int k = tid; k < Kd; k += 256) mx = fmaxf(mx, fabsf(B[base + k]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (l == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (mx > 0.f && mx <= 3.402823466e38f) {
    int E;
    frexpf(mx, &E);  // mx in [2^(E-1), 2^E)
    e = 15 - E;
  }
  if (tid == 0) scale_inv[blockIdx.x] = ldexpf(1.f, -e);
  for (int k = tid; k < Kd; k += 256) {
    const float y = ldexpf(B[base + k], e);
    const _Float16 h = (_Float16)y;
    P[base + k] = h;
    P[count + base + k] = (_Float16)(y - (float)h);
  }
}

// With col_partials (the block then spans all N <= 32 NT columns): the epilogue also takes
// Sinkhorn's first row step on the block's rows, u_r = -logsumexp_c C[r, c] (the column
// potential starts at zero), and writes the block's summary of sum_r exp(C[r, c] + u_r) for
// every column as a (max, sum) pair: col_partials[blockIdx.x * N + c]. Rows that are listed
// (not finite) or past M stay out of the summary.
template <int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES, NT > 4 ? 2 : 4) void gemm_nt_f16x3_kernel(
    const float* __restrict__ A, const _Float16* __restrict__ Bp,
    const float* __restrict__ bscale, float* __restrict__ C, int64_t M, int N, int Kd, int ldc,
    int32_t* __restrict__ flag_list, int32_t* __restrict__ flag_count,
    float2* __restrict__ col_partials) {
  constexpr int NTH = 64 * WAVES;
  constexpr int BM = 32 * WAVES, BN = 32 * NT, BK = 32;
  constexpr int BTILE = 2 * BN * BK;           // fp16 per B tile (two planes)
  constexpr int BINSTS = BTILE * 2 / 1024;     // 1 KB copies per B tile
  constexpr int BPW = (BINSTS + WAVES - 1) / WAVES;
  constexpr int AV = BM * BK / 4 / NTH;        // float4 of A per thread per chunk
  static_assert(AV * 4 * NTH == BM * BK, "A tile splits evenly over the threads");
  __shared__ __attribute__((aligned(1024))) _Float16 As[2][BM * BK];
  __shared__ __attribute__((aligned(1024))) _Float16 Bs[2][BTILE];
  const int tid = threadIdx.x, l = tid & 63, j = l & 31, g = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;

  // copy ii of a B tile fills rows 16 (ii % (BN / 16)) .. + 15 of plane ii / (BN / 16), with the
  // quarter permutation of plane_at (rows past N re-read row N - 1; their columns are not stored)
  uint32_t boff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int ii = wave + WAVES * i;
    const int pl = ii / (BN / 16), rb = ii % (BN / 16);
    const int r = rb * 16 + l / 4;
    const int q = (l % 4) ^ ((r >> 2) & 3);
    const int row = min(n0 + r, N - 1);
    boff[i] = (uint32_t)((((int64_t)pl * N + row) * Kd + 8 * q) * 2);
  }
  auto copy_b = [&](int k0, _Float16* dst) __attribute__((always_inline)) {
    const char* base = (const char*)(Bp + k0);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int ii = wave + WAVES * i;
      if (ii < BINSTS) dma16(base, boff[i], (char*)dst + ii * 1024);
    }
  };
  auto lds_barrier = []() __attribute__((always_inline)) {  // LDS only: copies stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16_t{};

  f32x4_t ra[AV];
  auto load_a = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int e = tid + NTH * i, r = e >> 3, c = (e & 7) * 4;
      const int64_t gr = m0 + r;
      ra[i] = gr < M ? *(const f32x4_t*)(A + gr * Kd + k0 + c) : f32x4_t{};
    }
  };

  auto chunk = [&](int k0, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;  // B buffer of this chunk
    lds_barrier();  // every wave is done with As and with the other B buffer
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int e = tid + NTH * i, r = e >> 3, c = (e & 7) * 4;
      const F16x4Pair pr = split_pair(ra[i]);
      const int o = plane_at(r, c);
      *(f16x4_t*)&As[0][o] = pr.h;
      *(f16x4_t*)&As[1][o] = pr.m;
    }
    // the wait for ra (the newest loads) also covers this chunk's B copies, issued before them
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (k0 + BK < Kd) {
      copy_b(k0 + BK, Bs[P ^ 1]);
      load_a(k0 + BK);
    }
    lds_barrier();  // As and this chunk's B planes are in LDS
    const _Float16* bsb = Bs[P];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      f16x8_t a[2];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        a[p] = *(const f16x8_t*)&As[p][plane_at(wave * 32 + j, ks * 16 + 8 * g)];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f16x8_t b[2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
          b[p] = *(const f16x8_t*)&bsb[p * BN * BK + plane_at(t * 32 + j, ks * 16 + 8 * g)];
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[1], b[0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], b[1], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], b[0], acc[t], 0, 0, 0);
      }
    }
  };
  copy_b(0, Bs[0]);
  load_a(0);
  for (int k0 = 0; k0 < Kd; k0 += 2 * BK) {
    chunk(k0, std::integral_constant<int, 0>{});
    if (k0 + BK < Kd) chunk(k0 + BK, std::integral_constant<int, 1>{});
  }

  // accumulator element v of tile t is row wave*32 + (v/4)*8 + 4g + v%4, column t*32 + j
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = n0 + t * 32 + j;
    const float sc = col < N ? bscale[col] : 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc[t][v] *= sc;
      const int64_t row = m0 + wave * 32 + (v >> 2) * 8 + 4 * g + (v & 3);
      if (row < M && col < N) C[row * ldc + col] = acc[t][v];
    }
  }
  // a row with a non-finite output had an element of A outside fp16's range (or not finite):
  // every column of that row is then non-finite, so the first column block lists it
  if (flag_list && blockIdx.y == 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      bool bad = false;
#pragma unroll
      for (int t = 0; t < NT; ++t) bad = bad || !__builtin_isfinite(acc[t][v]);
      const uint64_t bal = __ballot(bad);
      if (l == 0 && bal != 0) {
        const int64_t r0 = m0 + wave * 32 + (v >> 2) * 8 + (v & 3);
        if ((uint32_t)bal != 0u && r0 < M) flag_list[atomicAdd(flag_count, 1)] = (int32_t)r0;
        if ((uint32_t)(bal >> 32) != 0u && r0 + 4 < M)
          flag_list[atomicAdd(flag_count, 1)] = (int32_t)(r0 + 4);
      }
    }
  }
  if (col_partials) {
    // row step: the 32 lanes of a half-wave hold one row's columns
    float u[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + wave * 32 + (v >> 2) * 8 + 4 * g + (v & 3);
      float mx = -INFINITY, bad = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t * 32 + j < N) {
          mx = fmaxf(mx, acc[t][v]);
          bad = __builtin_isfinite(acc[t][v]) ? bad : 1.f;
        }
      }
      mx = row_max<32>(mx);
      bad = row_max<32>(bad);
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t * 32 + j < N) sum += fast_exp2((acc[t][v] - mx) * kLog2e);
      sum = row_sum<32>(sum);
      u[v] = (row < M && bad == 0.f) ? -(mx + __logf(sum)) : -INFINITY;  // -inf: left out
    }
    // column summaries over the lane's 16 rows, then the other half-wave's, then the waves
    lds_barrier();  // every wave is done reading B from LDS
    float2* red = reinterpret_cast<float2*>(&Bs[0][0]);  // [WAVES][32 NT]
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float cm = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (u[v] != -INFINITY) cm = fmaxf(cm, acc[t][v] + u[v]);
      float cs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (u[v] != -INFINITY) cs += fast_exp2((acc[t][v] + u[v] - cm) * kLog2e);
      const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(cm), __float_as_uint(cm), false, false);
      const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(cs), __float_as_uint(cs), false, false);
      float m = __uint_as_float(pm[0]), sm = __uint_as_float(ps[0]);
      ms_merge(m, sm, __uint_as_float(pm[1]), __uint_as_float(ps[1]));
      if (g == 0) red[wave * (32 * NT) + t * 32 + j] = make_float2(m, sm);
    }
    lds_barrier();  // LDS only: the score stores above need not land before the merge
    for (int c = tid; c < 32 * NT && c < N; c += 64 * WAVES) {
      float m = red[c].x, sm = red[c].y;
#pragma unroll
      for (int w = 1; w < WAVES; ++w) ms_merge(m, sm, red[w * (32 * NT) + c].x, red[w * (32 * NT) + c].y);
      col_partials[(int64_t)blockIdx.x * N + c] = make_float2(m, sm);
    }
  }
}

template <int NT, int WAVES>
static int f16x3_blocks_per_cu() {  // resident blocks per CU, from the compiled resources
  static int v = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, gemm_nt_f16x3_kernel<NT, WAVES>,
                                                     64 * WAVES, 0) != hipSuccess)
      b = 1;
    return b > 0 ? b : 1;
  }();
  return v;
}

template <int NT>
static int64_t f16x3_launch(const float* A, const _Float16* Bp, const float* bscale, float* C,
                            int64_t M, int N, int Kd, int ldc, int32_t* flags, int32_t* nflags,
                            float2* partials, int cus, hipStream_t stream) {
  const int64_t t4 = (M + 127) / 128, t8 = (M + 255) / 256;
  const int ny = (N + 32 * NT - 1) / (32 * NT);
  if constexpr (NT == 8) {  // 256 columns: 128-row tiles only (two waves per SIMD)
    hipLaunchKernelGGL((gemm_nt_f16x3_kernel<8, 4>), dim3(t4, ny), dim3(256), 0, stream, A, Bp,
                       bscale, C, M, N, Kd, ldc, flags, nflags, partials);
    return t4;
  } else {
    // the HBM-bound time goes as rounds of resident blocks times the rows one round moves per
    // CU: 256-row tiles unless 128-row ones finish in fewer such rows
    const int b8 = f16x3_blocks_per_cu<NT, 8>(), b4 = f16x3_blocks_per_cu<NT, 4>();
    const int64_t r8 = (t8 + (int64_t)cus * b8 - 1) / ((int64_t)cus * b8);
    const int64_t r4 = (t4 + (int64_t)cus * b4 - 1) / ((int64_t)cus * b4);
    if (r8 * b8 * 256 <= r4 * b4 * 128) {
      hipLaunchKernelGGL((gemm_nt_f16x3_kernel<NT, 8>), dim3(t8, ny), dim3(512), 0, stream, A, Bp,
                         bscale, C, M, N, Kd, ldc, flags, nflags, partials);
      return t8;
    }
    hipLaunchKernelGGL((gemm_nt_f16x3_kernel<NT, 4>), dim3(t4, ny), dim3(256), 0, stream, A, Bp,
                       bscale, C, M, N, Kd, ldc, flags, nflags, partials);
    return t4;
  }
}

hipError_t launch_gemm_nt_f16x3(const float* A, const float* B, _Float16* Bp, float* bscale,
                                float* C, int64_t M, int N, int Kd, int ldc, int32_t* flags,
                                int32_t* nflags, float2* col_partials, int64_t* row_blocks,
                                hipStream_t stream) {
  if (Kd % 32 != 0 || N < 1 || (col_partials && N > 256)) return hipErrorInvalidValue;
  if (row_blocks) *row_blocks = 0;
  if (M < 1) return hipSuccess;
  hipLaunchKernelGGL(split_pairs_kernel, dim3(N), dim3(256), 0, stream, B, Kd, (int64_t)N * Kd,
                     Bp, bscale);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  int64_t rb;
  if (N <= 32) rb = f16x3_launch<1>(A, Bp, bscale, C, M, N, Kd, ldc, flags, nflags, col_partials, cus, stream);
  else if (N <= 64) rb = f16x3_launch<2>(A, Bp, bscale, C, M, N, Kd, ldc, flags, nflags, col_partials, cus, stream);
  else if (N <= 128 || !col_partials) rb = f16x3_launch<4>(A, Bp, bscale, C, M, N, Kd, ldc, flags, nflags, col_partials, cus, stream);
  else rb = f16x3_launch<8>(A, Bp, bscale, C, M, N, Kd, ldc, flags, nflags, col_partials, cus, stream);
  if (row_blocks) *row_blocks = rb;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- exact rows
// Scores of the listed rows again in fp32, written over S: S[row, c] = h_row . Ft[c] (Ft [K, d],
// row c the folded column W_g C_c^T), or (h_row W_g) . C[c] with W_g [d, d_g] and C [K, d_g].
// For rows the fp16 product could not represent; one block per listed row at a time.
//
// With partials (Sinkhorn's first row step fused into the product's epilogue): block b also
// takes that row step on its rows and writes its column summaries to partials[b * K + c] (every
// launched block writes its slot, also with no rows).
__global__ __launch_bounds__(256) void exact_rows_kernel(
    const float* __restrict__ H, int d, const float* __restrict__ Ft, const float* __restrict__ W,
    const float* __restrict__ Cm, int dg, int K, const int32_t* __restrict__ list,
    const int32_t* __restrict__ count, float* __restrict__ S, int ldS,
    float2* __restrict__ partials) {
  __shared__ float part[4][1024];  // d_g <= 1024
  __shared__ float zs[1024];
  __shared__ float sc[1024];       // K <= 1024: the row's scores
  __shared__ float red[2][4];
  const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
  const int cnt = *count;
  float pm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, ps[4] = {0.f, 0.f, 0.f, 0.f};
  auto wave_sum = [](float s) __attribute__((always_inline)) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    return s;
  };
  for (int li = blockIdx.x; li < cnt; li += gridDim.x) {
    const int64_t row = list[li];
    const float* h = H + row * d;
    float* srow = S + row * ldS;
    if (Ft) {
      // a wave takes 8 columns per pass over h, lanes over d (d % 4 == 0); each column's sum
      // runs in the same order as one column at a time
      for (int c0 = 8 * wave; c0 < K; c0 += 32) {
        f32x4_t a[8];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) a[cc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int k = 4 * l; k < d; k += 256) {
          const f32x4_t hv = *(const f32x4_t*)(h + k);
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            if (c0 + cc < K) {
              const f32x4_t fv = *(const f32x4_t*)(Ft + (int64_t)(c0 + cc) * d + k);
#pragma unroll
              for (int e = 0; e < 4; ++e) a[cc][e] = __builtin_fmaf(hv[e], fv[e], a[cc][e]);
            }
          }
        }
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const float s = wave_sum((a[cc][0] + a[cc][1]) + (a[cc][2] + a[cc][3]));
          if (l == 0 && c0 + cc < K) {
            srow[c0 + cc] = s;
            sc[c0 + cc] = s;
          }
        }
      }
    } else {
      float z[16];  // columns l + 64 q of z = h W_g, over this wave's rows k = wave + 4 i
#pragma unroll
      for (int q = 0; q < 16; ++q) z[q] = 0.f;
      for (int k = wave; k < d; k += 4) {
        const float hk = h[k];
        const float* wr = W + (int64_t)k * dg;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (l + 64 * q < dg) z[q] = __builtin_fmaf(hk, wr[l + 64 * q], z[q]);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (l + 64 * q < dg) part[wave][l + 64 * q] = z[q];
      __syncthreads();
      for (int c = tid; c < dg; c += 256) zs[c] = (part[0][c] + part[1][c]) + (part[2][c] + part[3][c]);
      __syncthreads();
      for (int c = wave; c < K; c += 4) {  // a wave per centroid, lanes over d_g
        const float* cr = Cm + (int64_t)c * dg;
        float s = 0.f;
        for (int k = l; k < dg; k += 64) s = __builtin_fmaf(zs[k], cr[k], s);
        s = wave_sum(s);
        if (l == 0) {
          srow[c] = s;
          sc[c] = s;
        }
      }
    }
    __syncthreads();
    if (partials) {  // u = -logsumexp_c S[row, c], then the columns' running summaries
      float mx = -INFINITY;
      for (int c = tid; c < K; c += 256) mx = fmaxf(mx, sc[c]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (l == 0) red[0][wave] = mx;
      __syncthreads();
      mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
      float sum = 0.f;
      for (int c = tid; c < K; c += 256) sum += fast_exp2((sc[c] - mx) * kLog2e);
      sum = wave_sum(sum);
      if (l == 0) red[1][wave] = sum;
      __syncthreads();
      const float u = -(mx + __logf((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (tid + 256 * q < K) ms_merge(pm[q], ps[q], sc[tid + 256 * q] + u, 1.f);
      __syncthreads();
    }
  }
  if (partials) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (tid + 256 * q < K) partials[(int64_t)blockIdx.x * K + tid + 256 * q] = make_float2(pm[q], ps[q]);
  }
}

int exact_rows_blocks(int64_t n) { return n < 256 ? (int)n : 256; }

hipError_t launch_exact_rows(const float* H, int d, const float* Ft, const float* W,
                             const float* Cm, int dg, int K, const int32_t* list,
                             const int32_t* count, int64_t n, float* S, int ldS,
                             float2* partials, hipStream_t stream) {
  const int blocks = exact_rows_blocks(n);
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(exact_rows_kernel, dim3(blocks), dim3(256), 0, stream, H, d, Ft, W, Cm, dg,
                     K, list, count, S, ldS, partials);
  return hipGetLastError();
}

// ============================================================================ transpose
__global__ __launch_bounds__(256) void transpose_f32_kernel(const float* __restrict__ B,
                                                            float* __restrict__ Bt, int R, int Cn) {
  __shared__ float tile[32][33];
  int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int y = ty; y < 32; y += 8)
    if (r0 + y < R && c0 + tx < Cn) tile[y][tx] = B[(int64_t)(r0 + y) * Cn + c0 + tx];
  __syncthreads();
  for (int y = ty; y < 32; y += 8)
    if (c0 + y < Cn && r0 + tx < R) Bt[(int64_t)(c0 + y) * R + r0 + tx] = tile[tx][y];
}

hipError_t launch_transpose_f32(const float* B, float* Bt, int Kd, int N, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_f32_kernel, dim3((N + 31) / 32, (Kd + 31) / 32), dim3(256), 0,
                     stream, B, Bt, Kd, N);
  return hipGetLastError();
}

__global__ void fill_f32_kernel(float* p, float value, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

hipError_t launch_fill_f32(float* p, float value, int64_t count, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks), dim3(256), 0, stream, p, value, count);
  return hipGetLastError();
}

// ============================================================================ Sinkhorn pass
// Row step u_i = -logsumexp_c(S_ic + v_c) for the block's rows, and the block's summary of
// sum_i exp(S_ic + u_i) for every column c as a (max, sum) pair.
template <int LPR, int CPL>
__global__ __launch_bounds__(256) void sinkhorn_rows_kernel(const float* __restrict__ S, int64_t n,
                                                            int K, int ldS,
                                                            const float* __restrict__ v,
                                                            float2* __restrict__ partials,
                                                            int64_t rows_per_block) {
  constexpr int RPW = kWave / LPR;
  constexpr int NC = 4 * CPL;
  __shared__ float2 red[4][NC * LPR];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, q = l % LPR, rg = l / LPR;
  const int64_t r_begin = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r_end = r_begin + rows_per_block < n ? r_begin + rows_per_block : n;

  float vv[NC];
  bool ok[NC];
  float cm[NC], cs[NC];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int col = 4 * q + 4 * LPR * c + e;
      ok[4 * c + e] = col < K;
      vv[4 * c + e] = col < K ? v[col] : 0.f;
      cm[4 * c + e] = -INFINITY;
      cs[4 * c + e] = 0.f;
    }

  // rows are loaded two row groups ahead of their reduction, into two buffers used in turn
  auto load_row = [&](int64_t row, f32x4_t (&x)[CPL]) __attribute__((always_inline)) {
    const float* sp = S + row * ldS;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = 4 * q + 4 * LPR * c;
      x[c] = (row < r_end && col < K) ? *(const f32x4_t*)(sp + col) : f32x4_t{};
    }
  };
  f32x4_t nxt[2][CPL];
  const int64_t row0 = r_begin + wave * RPW + rg;
  load_row(row0, nxt[0]);
  load_row(row0 + 4 * RPW, nxt[1]);
  auto one_row = [&](int64_t row, f32x4_t (&buf)[CPL]) __attribute__((always_inline)) {
    float s[NC];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * c + e] = buf[c][e];
    load_row(row + 8 * RPW, buf);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (ok[i]) mx = fmaxf(mx, s[i] + vv[i]);
    mx = row_max<LPR>(mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (ok[i]) sum += fast_exp2((s[i] + vv[i] - mx) * kLog2e);
    sum = row_sum<LPR>(sum);
    const float u = -(mx + __logf(sum));
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (!ok[i]) continue;
      float x = s[i] + u;
      float d = x - cm[i];
      float e = fast_exp2(-fabsf(d) * kLog2e);
      if (d > 0.f) {
        cs[i] = cs[i] * e + 1.f;
        cm[i] = x;
      } else {
        cs[i] += e;
      }
    }
  };
  for (int64_t row = row0; row < r_end; row += 8 * RPW) {
    one_row(row, nxt[0]);
    if (row + 4 * RPW < r_end) one_row(row + 4 * RPW, nxt[1]);
  }
  // combine the row groups of the wave (lanes with equal q, i.e. lane l with l ^ o for o >= LPR):
  // l ^ 8 by a row rotation, l ^ 16 and l ^ 32 by the row-swapping permutes (each lane then holds
  // its own and its partner's value, in some order), smaller distances by lane shuffles
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (o == 16 || o == 32) {
        const auto pm = o == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(cm[i]), __float_as_uint(cm[i]), false, false)
                                : __builtin_amdgcn_permlane32_swap(__float_as_uint(cm[i]), __float_as_uint(cm[i]), false, false);
        const auto ps = o == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(cs[i]), __float_as_uint(cs[i]), false, false)
                                : __builtin_amdgcn_permlane32_swap(__float_as_uint(cs[i]), __float_as_uint(cs[i]), false, false);
        float m = __uint_as_float(pm[0]), sm = __uint_as_float(ps[0]);
        ms_merge(m, sm, __uint_as_float(pm[1]), __uint_as_float(ps[1]));
        cm[i] = m;
        cs[i] = sm;
      } else {
        const float m2 = o == 8 ? dpp_move<0x128>(cm[i]) : shfl_xor_f(cm[i], o);  // row_ror:8
        const float s2 = o == 8 ? dpp_move<0x128>(cs[i]) : shfl_xor_f(cs[i], o);
        ms_merge(cm[i], cs[i], m2, s2);
      }
    }
  if (rg == 0) {
#pragma unroll
    for (int i = 0; i < NC; ++i) red[wave][i * LPR + q] = make_float2(cm[i], cs[i]);
  }
  __syncthreads();
  for (int t = tid; t < NC * LPR; t += 256) {
    int i = t / LPR, qq = t % LPR;
    int col = 4 * qq + 4 * LPR * (i / 4) + (i % 4);
    if (col >= K) continue;
    float m = red[0][t].x, s = red[0][t].y;
    for (int w = 1; w < 4; ++w) ms_merge(m, s, red[w][t].x, red[w][t].y);
    partials[(int64_t)blockIdx.x * K + col] = make_float2(m, s);
  }
}

// Column step: v_c = log(n / K) - logsumexp_i(S_ic + u_i), from the block summaries (fp64).
__global__ __launch_bounds__(256) void sinkhorn_cols_kernel(const float2* __restrict__ partials,
                                                            int nblocks, int K, double log_mass,
                                                            float* __restrict__ v) {
  __shared__ double sm[256], ss[256];
  const int c = blockIdx.x, t = threadIdx.x;
  double m = -INFINITY, s = 0.0;
  for (int b = t; b < nblocks; b += 256) {
    float2 p = partials[(int64_t)b * K + c];
    double pm = p.x, ps = p.y;
    double M = m > pm ? m : pm;
    if (M == -INFINITY) continue;
    s = s * exp(m - M) + ps * exp(pm - M);
    m = M;
  }
  sm[t] = m;
  ss[t] = s;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (t < o) {
      double m1 = sm[t], m2 = sm[t + o];
      double M = m1 > m2 ? m1 : m2;
      if (M != -INFINITY) {
        ss[t] = ss[t] * exp(m1 - M) + ss[t + o] * exp(m2 - M);
        sm[t] = M;
      }
    }
    __syncthreads();
  }
  if (t == 0) v[c] = (float)(log_mass - (sm[0] + log(ss[0])));
}

int sinkhorn_blocks(int64_t n, int K) {
  (void)K;
  int64_t b = (n + 255) / 256;
  if (b > 4096) b = 4096;
  if (b < 1) b = 1;
  return (int)b;
}

template <int LPR, int CPL>
static hipError_t sinkhorn_rows(const float* S, int64_t n, int K, int ldS, const float* v,
                                float2* partials, int nblocks, hipStream_t stream) {
  constexpr int gran = 4 * (kWave / LPR);
  int64_t rpb = (n + nblocks - 1) / nblocks;
  rpb = (rpb + gran - 1) / gran * gran;
  hipLaunchKernelGGL((sinkhorn_rows_kernel<LPR, CPL>), dim3(nblocks), dim3(256), 0, stream, S, n,
                     K, ldS, v, partials, rpb);
  return hipGetLastError();
}

// Lanes per row for K columns when every lane holds 16 of them (4 float4 chunks): the fewer
// lanes a row takes, the more rows a wave reduces at once and the shorter the shuffle trees.
int lanes_per_row(int K) {
  int lpr = 1;
  while (lpr < 64 && 16 * lpr < K) lpr *= 2;
  return lpr;
}

hipError_t launch_sinkhorn_cols(const float2* partials, int nblocks, int64_t n, int K, float* v,
                                hipStream_t stream) {
  hipLaunchKernelGGL(sinkhorn_cols_kernel, dim3(K), dim3(256), 0, stream, partials, nblocks, K,
                     log((double)n / (double)K), v);
  return hipGetLastError();
}

hipError_t launch_sinkhorn_iter(const float* S, int64_t n, int K, int ldS, float* v,
                                float2* partials, int nblocks, hipStream_t stream) {
  hipError_t e;
  switch (lanes_per_row(K)) {
    case 1: e = sinkhorn_rows<1, 4>(S, n, K, ldS, v, partials, nblocks, stream); break;
    case 2: e = sinkhorn_rows<2, 4>(S, n, K, ldS, v, partials, nblocks, stream); break;
    case 4: e = sinkhorn_rows<4, 4>(S, n, K, ldS, v, partials, nblocks, stream); break;
    case 8: e = sinkhorn_rows<8, 4>(S, n, K, ldS, v, partials, nblocks, stream); break;
    case 16: e = sinkhorn_rows<16, 4>(S, n, K, ldS, v, partials, nblocks, stream); break;
    case 32: e = sinkhorn_rows<32, 4>(S, n, K, ldS, v, partials, nblocks, stream); break;
    default: e = sinkhorn_rows<64, 4>(S, n, K, ldS, v, partials, nblocks, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sinkhorn_cols_kernel, dim3(K), dim3(256), 0, stream, partials, nblocks, K,
                     log((double)n / (double)K), v);
  return hipGetLastError();
}

// ============================================================================ top-k
// groups[i] = the top_k columns of S_i + v (equal values: lower column first), ascending.
constexpr int kNone = 0x7fffffff;

__device__ __forceinline__ bool better(float v2, int i2, float v1, int i1) {
  if (i2 == kNone) return false;
  if (i1 == kNone) return true;
  return v2 > v1 || (v2 == v1 && i2 < i1);
}

template <int LPR, int CPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ S,
                                                   const float* __restrict__ v, int64_t n, int K,
                                                   int ldS, int top_k,
                                                   int32_t* __restrict__ groups) {
  constexpr int RPW = kWave / LPR;
  constexpr int NC = 4 * CPL;
  const int l = threadIdx.x & 63, wave = threadIdx.x >> 6, q = l % LPR, rg = l / LPR;
  float vv[NC];
  int colx[NC];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int col = 4 * q + 4 * LPR * c + e;
      colx[4 * c + e] = col < K ? col : kNone;
      vv[4 * c + e] = col < K ? v[col] : 0.f;
    }
  // the block's waves walk row groups grid-stride, each loading its next row group while it
  // selects from the current one (a row group leaves the loop together: shuffles stay inside)
  const int64_t step = (int64_t)gridDim.x * 4 * RPW;
  f32x4_t nx[CPL];
  auto load_row = [&](int64_t row) {
    const float* sp = S + row * ldS;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = 4 * q + 4 * LPR * c;
      nx[c] = (row < n && col < K) ? *(const f32x4_t*)(sp + col) : f32x4_t{};
    }
  };
  int64_t row = (int64_t)blockIdx.x * 4 * RPW + wave * RPW + rg;
  load_row(row);
  for (; row < n; row += step) {
    float b[NC];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) b[4 * c + e] = nx[c][e] + vv[4 * c + e];
    load_row(row + step);
    unsigned taken = 0;
    int sel[8];
    for (int r = 0; r < top_k; ++r) {
      float bv = 0.f;
      int bi = kNone;
#pragma unroll
      for (int i = 0; i < NC; ++i)
        if (!((taken >> i) & 1u) && better(b[i], colx[i], bv, bi)) {
          bv = b[i];
          bi = colx[i];
        }
      // argmax over the row's lanes: `better` is a strict total order, so any pairing that
      // combines disjoint halves of the group gives every lane the same winner; within a 16-lane
      // row the pairs move on the VALU
      auto take = [&](float v2, int i2) __attribute__((always_inline)) {
        if (better(v2, i2, bv, bi)) {
          bv = v2;
          bi = i2;
        }
      };
      if constexpr (LPR >= 2) take(dpp_move<0xB1>(bv), dpp_move_i<0xB1>(bi));
      if constexpr (LPR >= 4) take(dpp_move<0x4E>(bv), dpp_move_i<0x4E>(bi));
      if constexpr (LPR >= 8) take(dpp_move<0x141>(bv), dpp_move_i<0x141>(bi));
      if constexpr (LPR >= 16) take(dpp_move<0x140>(bv), dpp_move_i<0x140>(bi));
      if constexpr (LPR >= 32) take(shfl_xor_f(bv, 16), shfl_xor_i(bi, 16));
      if constexpr (LPR >= 64) take(shfl_xor_f(bv, 32), shfl_xor_i(bi, 32));
      sel[r] = bi;
#pragma unroll
      for (int i = 0; i < NC; ++i)
        if (colx[i] == bi) taken |= 1u << i;
    }
    // ascending order of the selected set
    for (int a = 1; a < top_k; ++a) {
      int x = sel[a], p = a - 1;
      while (p >= 0 && sel[p] > x) {
        sel[p + 1] = sel[p];
        --p;
      }
      sel[p + 1] = x;
    }
    if (q == 0)
      for (int r = 0; r < top_k; ++r) groups[row * top_k + r] = sel[r];
  }
}

template <int LPR, int CPL>
static hipError_t topk_launch(const float* S, const float* v, int64_t n, int K, int ldS, int top_k,
                              int32_t* groups, hipStream_t stream) {
  const int64_t rpb = 4 * (kWave / LPR);
  int64_t blocks = (n + rpb - 1) / rpb;
  if (blocks > 8192) blocks = 8192;  // beyond that the blocks walk further row groups
  hipLaunchKernelGGL((topk_kernel<LPR, CPL>), dim3(blocks), dim3(256), 0, stream, S, v,
                     n, K, ldS, top_k, groups);
  return hipGetLastError();
}

hipError_t launch_topk(const float* S, const float* v, int64_t n, int K, int ldS, int top_k,
                       int32_t* groups, hipStream_t stream) {
  switch (lanes_per_row(K)) {
    case 1: return topk_launch<1, 4>(S, v, n, K, ldS, top_k, groups, stream);
    case 2: return topk_launch<2, 4>(S, v, n, K, ldS, top_k, groups, stream);
    case 4: return topk_launch<4, 4>(S, v, n, K, ldS, top_k, groups, stream);
    case 8: return topk_launch<8, 4>(S, v, n, K, ldS, top_k, groups, stream);
    case 16: return topk_launch<16, 4>(S, v, n, K, ldS, top_k, groups, stream);
    case 32: return topk_launch<32, 4>(S, v, n, K, ldS, top_k, groups, stream);
    default: return topk_launch<64, 4>(S, v, n, K, ldS, top_k, groups, stream);
  }
}

}  // namespace focus
