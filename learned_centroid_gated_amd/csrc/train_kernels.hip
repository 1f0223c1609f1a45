// Soft-gated training path on gfx950: the forward over every causal pair with the gate driven by
// the soft assignment, and the backward that trains only the centroids and the projection.
//
// Method: "Why Attend to Everything? Focus is the Key". Dutch technical summary, Kerncomponenten
// 1 (a token's soft assignment g_i from its affinity to the centroids), 2 (Sinkhorn balancing
// during training) and 4 (training computes every pair with soft gates); Chinese technical
// summary, section 2.1.2 (gate formula: far pairs gated by sigmoid(lambda a_ij), a_ij the group
// affinity) and section 2.2 (only the centroids and the projection are trained).
//
// Reading: g_i is row i of the balanced Sinkhorn plan exp(S + u + v); a_ij = g_i . g_j - 1/2;
// the gate multiplies the weight, i.e. far causal pairs (i - j >= window) add
// log sigmoid(lambda a_ij) to the logit scale q_i . k_j.
//
// Attention kernels (4 waves, 128 query rows = T tokens x the G query heads of one kv head, as in
// the inference flash kernel; 64-key tiles double-buffered in LDS by global_load_lds):
//   train_q_kernel<.., false>  forward: S^T = K Q^T and A^T = G_k g_q^T on the bf16 MFMA (g split
//                              into two bf16 parts, three part products), the gated logits, an
//                              online softmax, O^T += V^T P^T; writes out and lse.
//   train_q_kernel<.., true>   backward, query side: recomputes P from lse, dP^T = V dO^T,
//                              dS = P (dP - D), F = dS dlog sigmoid/da on far pairs, and adds
//                              dG_i += sum_j F_ij g_j (G_k^T F^T on the MFMA, F in bf16, g in two
//                              parts); G query heads summed in LDS, one atomic add per token and
//                              group.
//   train_k_kernel             backward, key side: each wave keeps 32 keys' K, V and g in registers
//                              and streams 64-row query tiles (Q, dO, lse, D and the tokens' g)
//                              through LDS, adding dG_j += sum_i F_ij g_i.
// Only far pairs carry the gate, so the backward visits only tiles with a far pair.
#include <cstddef>
#include <type_traits>

#include "focus_internal.hpp"

namespace focus {

namespace {

constexpr int KT = 64;  // keys per tile of the query-side kernel

// log2 sigmoid(y) and sigmoid(-y), without overflow for any finite y
__device__ __forceinline__ void gate_terms(float y, float& log2_sig, float& sig_neg) {
  const float t = fast_exp2(-fabsf(y) * kLog2e);  // exp(-|y|) in (0, 1]
  const float one_t = 1.f + t;
  log2_sig = fminf(y, 0.f) * kLog2e - __log2f(one_t);
  sig_neg = (y >= 0.f ? t : 1.f) / one_t;
}

// Two-part bf16 split of a soft-assignment value: x = hi + lo + r, |r| <= 2^-17 |x|.
__device__ __forceinline__ void split2(float x, __bf16& hi, __bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - (float)hi);
}

}  // namespace

// ============================================================================ plan and planes
// g_i = exp(S_i + u_i + v_c) with u_i = -logsumexp_c(S_ic + vprev_c) (the last row step), written
// as two bf16 planes [n, KP] (zero past K). iters == 0: g = exp(S). One wave per row.
__global__ __launch_bounds__(256) void train_plan_kernel(const float* __restrict__ S, int64_t n,
                                                         int K, int ldS, int KP,
                                                         const float* __restrict__ vprev,
                                                         const float* __restrict__ vlast,
                                                         int iters, __bf16* __restrict__ gh,
                                                         __bf16* __restrict__ gl) {
  const int l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const float* sp = S + row * ldS;
  float u = 0.f;
  if (iters > 0) {
    float mx = -INFINITY;
    for (int c = l; c < K; c += 64) mx = fmaxf(mx, sp[c] + vprev[c]);
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
    float sum = 0.f;
    for (int c = l; c < K; c += 64) sum += fast_exp2((sp[c] + vprev[c] - mx) * kLog2e);
    for (int o = 32; o >= 1; o >>= 1) sum += shfl_xor_f(sum, o);
    u = -(mx + __logf(sum));
  }
  for (int c = l; c < KP; c += 64) {
    __bf16 hi = (__bf16)0.f, lo = (__bf16)0.f;
    if (c < K) split2(__expf(sp[c] + u + (iters > 0 ? vlast[c] : 0.f)), hi, lo);
    gh[row * KP + c] = hi;
    gl[row * KP + c] = lo;
  }
}

hipError_t launch_train_plan(const float* S, int64_t n, int K, int ldS, int KP, const float* vprev,
                             const float* vlast, int iters, __bf16* gh, __bf16* gl,
                             hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(train_plan_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, S, n, K, ldS, KP,
                     vprev, vlast, iters, gh, gl);
  return hipGetLastError();
}

// D[i, h] = sum_d dO[i, h, d] * O[i, h, d] (bf16 rows): 16 lanes per row at head size 128.
template <int DH>
__global__ __launch_bounds__(256) void train_delta_kernel(const uint16_t* __restrict__ dout,
                                                          const uint16_t* __restrict__ out,
                                                          int64_t rows, float* __restrict__ D) {
  constexpr int LPR = DH / 8;  // lanes per row, 8 values each
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8_t a = *(const bf16x8_t*)(dout + row * DH + 8 * part);
    const bf16x8_t b = *(const bf16x8_t*)(out + row * DH + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
  for (int o = LPR / 2; o >= 1; o >>= 1) acc += shfl_xor_f(acc, o);
  if (row < rows && part == 0) D[row] = acc;
}

hipError_t launch_train_delta(const uint16_t* dout, const uint16_t* out, int64_t rows, int dh,
                              float* D, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int lpr = dh / 8;
  const int64_t blocks = (rows * lpr + 255) / 256;
  if (dh == 128)
    hipLaunchKernelGGL(train_delta_kernel<128>, dim3(blocks), dim3(256), 0, stream, dout, out, rows, D);
  else
    hipLaunchKernelGGL(train_delta_kernel<64>, dim3(blocks), dim3(256), 0, stream, dout, out, rows, D);
  return hipGetLastError();
}

// ============================================================================ query side
struct TrainArgs {
  const uint16_t* q;     // [n, Hq, DH]
  const uint16_t* k;     // [n, Hkv, DH]
  const uint16_t* v;
  const __bf16* gh;      // [n, KP] soft assignment, high part
  const __bf16* gl;      //         and low part
  uint16_t* out;         // forward: [n, Hq, DH]
  float* lse;            // forward out / backward in: [n, Hq] natural log
  const uint16_t* dout;  // backward: [n, Hq, DH]
  const float* D;        // backward: [n, Hq] rowwise dO . O
  float* dG;             // backward: [n, K] gradient of the soft assignment (atomic adds)
  int64_t n;
  int Hq, Hkv, G, T, K;
  int window;            // clamped to n + 1
  float sl2;             // scale * log2 e
  float lam;             // gate sharpness
  int items;             // work items per kv head
};

template <int DH, int KP>
struct TrainQSmem {
  __bf16 k[KT * DH];
  __bf16 v[KT * DH];
  __bf16 gh[KT * KP];
  __bf16 gl[KT * KP];
};

// Workgroups per CU the double-buffered tiles leave room for (160 KB of LDS per CU).
template <typename Smem>
constexpr int wgs_per_cu() {
  return 2 * 2 * sizeof(Smem) <= 160 * 1024 ? 2 : 1;
}

// SH (T <= 32, every wave holding the same tokens): the affinity and gate of each (token, key)
// pair are computed once per workgroup rather than once per head: wave w takes keys
// 16 w .. 16 w + 15 of the tile against all T tokens on the 16x16x32 bf16 MFMA, turns them into
// gate terms and leaves them in LDS for every wave's rows.
template <int DH, int KP, bool BWD, bool SH>
__global__ __launch_bounds__(256, (wgs_per_cu<TrainQSmem<DH, KP>>())) void train_q_kernel(const TrainArgs a) {
  using Smem = TrainQSmem<DH, KP>;
  constexpr int CH = DH / 8, RB = 2 * DH;     // 16-byte chunks and bytes per K/V row
  constexpr int CHG = KP / 8, RBG = 2 * KP;   // the same for a soft-assignment row
  constexpr int NS = DH / 16, ND = DH / 32;   // MFMA k-steps over dims, 32-wide output tiles
  constexpr int KS = KP / 16, NG = KP / 32;   // k-steps over groups, 32-wide group tiles
  constexpr int INSTS = KT * CH / 64 / 4;     // 1 KB copies per wave per K (and V) tile
  constexpr int INSTG = KT * CHG / 64 / 4;    // per wave per soft-assignment plane tile
  static_assert(INSTS >= 1 && INSTG >= 1, "tile copies");
  __shared__ __attribute__((aligned(1024))) Smem smem[2];
  static_assert(!SH || KP >= 32, "shared gates take 32-group k-steps");
  constexpr int GS = KT + 4;  // shared gate rows: one per token, padded against bank conflicts
  __shared__ __attribute__((aligned(16))) float gate_s[SH ? 32 : 1][SH ? GS : 1];
  __shared__ __attribute__((aligned(16))) float gsig_s[(SH && BWD) ? 32 : 1][(SH && BWD) ? GS : 1];

  const int tid = threadIdx.x, l = tid & 63, jq = l & 31, hg = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t comb = xcd_remap(blockIdx.x, (int64_t)a.Hkv * a.items);
  if (comb < 0) return;
  const int h = (int)(comb / a.items);
  const int item = (int)(comb - (int64_t)h * a.items);
  const int window = a.window;
  const int q0 = item * a.T;
  const int q1 = (int)min((int64_t)q0 + a.T, a.n);

  // this lane's query row
  const int r = wave * 32 + jq;
  const int head_local = r / a.T, tok = r % a.T;
  const int hq = h * a.G + head_local;
  const int qi = q0 + tok;
  const bool qvalid = qi < q1;
  const int wt0 = (wave * 32) % a.T;
  const int wq_lo = q0 + wt0;
  const int wq_hi = min(q0 + wt0 + (a.T < 32 ? a.T : 32), q1) - 1;
  const bool wave_active = wq_hi >= wq_lo;

  // key range: every causal key (forward) or the far ones (backward)
  const int kv_hi = BWD ? q1 - 1 - window : q1 - 1;
  const int ntiles = kv_hi >= 0 ? kv_hi / KT + 1 : 0;
  if (BWD && ntiles == 0) return;  // no far pair: nothing to add

  const int qrow = qvalid ? qi : q0;
  bf16x8_t qreg[NS], dreg[BWD ? NS : 1];
  {
    const uint16_t* qp = a.q + ((int64_t)qrow * a.Hq + hq) * DH + 8 * hg;
#pragma unroll
    for (int s = 0; s < NS; ++s) qreg[s] = *(const bf16x8_t*)(qp + 16 * s);
    if constexpr (BWD) {
      const uint16_t* dp = a.dout + ((int64_t)qrow * a.Hq + hq) * DH + 8 * hg;
#pragma unroll
      for (int s = 0; s < NS; ++s) dreg[s] = *(const bf16x8_t*)(dp + 16 * s);
    }
  }
  bf16x8_t gqh[SH ? 1 : KS], gql[SH ? 1 : KS];  // the token's soft assignment, groups 16 s + 8 hg .. + 7
  if constexpr (!SH) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      gqh[s] = *(const bf16x8_t*)(a.gh + (int64_t)qrow * KP + 16 * s + 8 * hg);
      gql[s] = *(const bf16x8_t*)(a.gl + (int64_t)qrow * KP + 16 * s + 8 * hg);
    }
  }
  // SH: the B operand of the shared affinity product, token 16 tt + l % 16 of the tile at groups
  // 32 s + 8 (l / 16) .. + 7 (zero past the tile's tokens)
  constexpr int KS2 = KP / 32;
  bf16x8_t gbh[SH ? 2 : 1][SH ? KS2 : 1], gbl[SH ? 2 : 1][SH ? KS2 : 1];
  if constexpr (SH) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tk = 16 * tt + (l & 15);
      const bool ok = tk < a.T && q0 + tk < q1;
#pragma unroll
      for (int s = 0; s < KS2; ++s) {
        const int64_t off = (int64_t)(ok ? q0 + tk : 0) * KP + 32 * s + 8 * (l >> 4);
        gbh[tt][s] = ok ? *(const bf16x8_t*)(a.gh + off) : bf16x8_t{};
        gbl[tt][s] = ok ? *(const bf16x8_t*)(a.gl + off) : bf16x8_t{};
      }
    }
  }
  float lse2 = 0.f, drow = 0.f;
  if constexpr (BWD) {
    lse2 = qvalid ? a.lse[(int64_t)qi * a.Hq + hq] * kLog2e : 0.f;
    drow = qvalid ? a.D[(int64_t)qi * a.Hq + hq] : 0.f;
  }

  f32x16_t oacc[BWD ? 1 : ND];
  f32x16_t gacc[BWD ? NG : 1];
  if constexpr (BWD) {
#pragma unroll
    for (int d = 0; d < NG; ++d) gacc[d] = f32x16_t{};
  } else {
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16_t{};
  }
  float m_run = -INFINITY, l_run = 0.f;

  // per-lane LDS addresses (bytes from smem[0]; the buffer parity and row block are immediates)
  const char* lds = (const char*)smem;
  uint32_t krd[NS], grd[KS];
#pragma unroll
  for (int s = 0; s < NS; ++s) krd[s] = (uint32_t)(jq * RB + (((2 * s + hg) ^ (swz(jq) % CH)) * 16));
#pragma unroll
  for (int s = 0; s < KS; ++s)
    grd[s] = (uint32_t)(jq * RBG + (((2 * s + hg) ^ (swz(jq) % CHG)) * 16));
  // transposing reads (lane 16 g + 4 e + m reads row 4 hg + e + 8 rr of a 16-row block, 8 bytes
  // at columns 32 d + 16 (g % 2) + 4 m, and receives 4 rows of column 32 d + lane % 32)
  const int e4 = (l & 15) >> 2, m4 = l & 3, g2 = (l >> 4) & 1;
  uint32_t vrd[BWD ? 1 : ND][2], gtr[BWD ? NG : 1][2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = 4 * hg + e4 + 8 * rr;
    if constexpr (!BWD) {
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const int c16 = 4 * d + 2 * g2 + (m4 >> 1);
        vrd[d][rr] = (uint32_t)(offsetof(Smem, v) + row * RB + ((c16 ^ (swz(row) % CH)) * 16) +
                                (m4 & 1) * 8);
      }
    } else {
#pragma unroll
      for (int d = 0; d < NG; ++d) {
        const int c16 = 4 * d + 2 * g2 + (m4 >> 1);
        gtr[d][rr] = (uint32_t)(row * RBG + ((c16 ^ (swz(row) % CHG)) * 16) + (m4 & 1) * 8);
      }
    }
  }

  // tile copies: wave w moves rows [w KT/4, (w+1) KT/4) of K, V and the two planes
  const uint32_t kstride = (uint32_t)a.Hkv * RB;
  const char* khead = (const char*)a.k + (int64_t)h * RB;
  const char* vhead = (const char*)a.v + (int64_t)h * RB;
  uint32_t gofs[INSTS], gch[INSTS], pofs[INSTG], pch[INSTG];
  int lrow[INSTS], prow[INSTG];
#pragma unroll
  for (int i = 0; i < INSTS; ++i) {
    lrow[i] = (wave * INSTS + i) * (64 / CH) + l / CH;
    gch[i] = (uint32_t)(((l % CH) ^ (swz(lrow[i]) % CH)) * 16);
    gofs[i] = (uint32_t)lrow[i] * kstride + gch[i];
  }
#pragma unroll
  for (int i = 0; i < INSTG; ++i) {
    prow[i] = (wave * INSTG + i) * (64 / CHG) + l / CHG;
    pch[i] = (uint32_t)(((l % CHG) ^ (swz(prow[i]) % CHG)) * 16);
    pofs[i] = (uint32_t)prow[i] * RBG + pch[i];
  }
  auto issue_tile = [&](int ks, Smem& sb) __attribute__((always_inline)) {
    const char* kb = khead + (int64_t)ks * kstride;
    const char* vb = vhead + (int64_t)ks * kstride;
    const char* hb = (const char*)a.gh + (int64_t)ks * RBG;
    const char* lb = (const char*)a.gl + (int64_t)ks * RBG;
    const int nrow = kv_hi - ks;  // rows past it re-read row nrow; the masks drop them
#pragma unroll
    for (int i = 0; i < INSTS; ++i) {
      const uint32_t off = lrow[i] <= nrow ? gofs[i] : (uint32_t)nrow * kstride + gch[i];
      dma16(kb, off, (char*)sb.k + (wave * INSTS + i) * 1024);
      dma16(vb, off, (char*)sb.v + (wave * INSTS + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < INSTG; ++i) {
      const uint32_t off = prow[i] <= nrow ? pofs[i] : (uint32_t)nrow * RBG + pch[i];
      dma16(hb, off, (char*)sb.gh + (wave * INSTG + i) * 1024);
      dma16(lb, off, (char*)sb.gl + (wave * INSTG + i) * 1024);
    }
  };

  auto compute_tile = [&](int ks, const uint32_t par) __attribute__((always_inline)) {
    if (!wave_active || ks > wq_hi) return;
    const bool far_any = wq_hi - ks >= window;
    if (BWD && !far_any) return;
    const int k_last = ks + KT - 1;
    const bool all_far = wq_lo - k_last >= window;              // every pair far and causal
    const bool all_near = k_last <= wq_lo && wq_hi - ks < window;  // every pair near and causal

    // S^T = K Q^T, and (backward) dP^T = V dO^T
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
    f32x16_t pacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf = *(const bf16x8_t*)(lds + krd[s] + par + kb * 32 * RB);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[s], sacc[kb], 0, 0, 0);
        if constexpr (BWD) {
          const bf16x8_t vf = *(const bf16x8_t*)(lds + offsetof(Smem, v) + krd[s] + par + kb * 32 * RB);
          pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dreg[s], pacc[kb], 0, 0, 0);
        }
      }
    // SH: this wave's share of the workgroup's gate tile, ahead of the score product so the
    // barrier below finds it done
    if constexpr (SH) {
      if (far_any) {
        const int krow = 16 * wave + (l & 15);  // key row of the tile
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          if (16 * tt >= a.T) break;
          f32x4_t a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS2; ++s) {
            const int cc = 4 * s + (l >> 4);  // 16-byte chunk of the key's plane rows
            const uint32_t ga = (uint32_t)(krow * RBG + ((cc ^ (swz(krow) % CHG)) * 16)) + par;
            const bf16x8_t hf = *(const bf16x8_t*)(lds + offsetof(Smem, gh) + ga);
            const bf16x8_t lf = *(const bf16x8_t*)(lds + offsetof(Smem, gl) + ga);
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hf, gbh[tt][s], a4, 0, 0, 0);
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hf, gbl[tt][s], a4, 0, 0, 0);
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lf, gbh[tt][s], a4, 0, 0, 0);
          }
          // element i: key 16 wave + 4 (l / 16) + i, token 16 tt + l % 16
          f32x4_t g4, s4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float l2s, sn;
            gate_terms(a.lam * (a4[i] - 0.5f), l2s, sn);
            g4[i] = l2s;
            s4[i] = sn;
          }
          const int tk = 16 * tt + (l & 15), kc = 16 * wave + 4 * (l >> 4);
          *(f32x4_t*)&gate_s[tk][kc] = g4;
          if constexpr (BWD) *(f32x4_t*)&gsig_s[tk][kc] = s4;
        }
      }
    }

    // A^T = G_k g_q^T from the two-part planes (hi hi + hi lo + lo hi)
    f32x16_t aacc[2] = {f32x16_t{}, f32x16_t{}};
    if (!SH && far_any) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t hf = *(const bf16x8_t*)(lds + offsetof(Smem, gh) + grd[s] + par + kb * 32 * RBG);
          const bf16x8_t lf = *(const bf16x8_t*)(lds + offsetof(Smem, gl) + grd[s] + par + kb * 32 * RBG);
          aacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, gqh[s], aacc[kb], 0, 0, 0);
          aacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, gql[s], aacc[kb], 0, 0, 0);
          aacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, gqh[s], aacc[kb], 0, 0, 0);
        }
    }

    // SH: every wave's gate terms are in LDS; this lane's row reads its token's
    f32x4_t gv[SH ? 2 : 1][SH ? 4 : 1], sv[(SH && BWD) ? 2 : 1][(SH && BWD) ? 4 : 1];
    if constexpr (SH) {
      if (far_any) {
        __syncthreads();
        if (!all_near) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              gv[kb][q4] = *(const f32x4_t*)&gate_s[tok][kb * 32 + 8 * q4 + 4 * hg];
              if constexpr (BWD) sv[kb][q4] = *(const f32x4_t*)&gsig_s[tok][kb * 32 + 8 * q4 + 4 * hg];
            }
        }
      }
    }

    // gated logits in log2 units; element v of tile kb is key kb*32 + 8*(v/4) + 4*hg + v%4
    float x[2][16], sgn[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) {
        const int key = ks + kb * 32 + 8 * (vi >> 2) + 4 * hg + (vi & 3);
        const int dd = qi - key;
        float xx = sacc[kb][vi] * a.sl2;
        float sn = 0.f;
        if (!all_near) {
          if (all_far || dd >= window) {
            float l2s;
            if constexpr (SH) {
              l2s = gv[kb][vi >> 2][vi & 3];
              if constexpr (BWD) sn = sv[kb][vi >> 2][vi & 3];
            } else {
              gate_terms(a.lam * (aacc[kb][vi] - 0.5f), l2s, sn);
            }
            xx += l2s;
          }
          if (!all_far && dd < 0) xx = -INFINITY;
        }
        if (!qvalid) xx = -INFINITY;
        x[kb][vi] = xx;
        sgn[kb][vi] = (all_far || dd >= window) ? sn : 0.f;
      }

    if constexpr (!BWD) {
      // online softmax with a lazily moved reference maximum (see the inference flash kernel)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int vi = 0; vi < 16; ++vi) mx = fmaxf(mx, x[kb][vi]);
      const float tmax = pair32_max(mx);
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
      float psum = 0.f;
      bf16x8_t pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int vi = 0; vi < 16; ++vi) {
          const float p = fast_exp2(x[kb][vi] - m_use);
          psum += p;
          pb[kb * 2 + (vi >> 3)][vi & 7] = to_bf16(p);
        }
      l_run += psum;
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t kqo = ((kq >> 1) * 32 + (kq & 1) * 16) * RB;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          bf16x4_t half[2];
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            typedef short v4i16_t __attribute__((ext_vector_type(4)));
            const char* src = lds + vrd[d][rr] + par + kqo;
            v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16_t*)(lds_void_t*)src);
            half[rr] = __builtin_bit_cast(bf16x4_t, t);
          }
          const bf16x8_t vf = {half[0][0], half[0][1], half[0][2], half[0][3],
                               half[1][0], half[1][1], half[1][2], half[1][3]};
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kq], oacc[d], 0, 0, 0);
        }
      }
    } else {
      // F = P (dP - D) lambda sigmoid(-lambda (a - 1/2)) on far pairs, then dG^T += G_k^T F^T
      bf16x8_t fb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int vi = 0; vi < 16; ++vi) {
          const float p = fast_exp2(x[kb][vi] - lse2);
          const float f = p * (pacc[kb][vi] - drow) * a.lam * sgn[kb][vi];
          fb[kb * 2 + (vi >> 3)][vi & 7] = to_bf16(f);
        }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t kqo = ((kq >> 1) * 32 + (kq & 1) * 16) * RBG;
#pragma unroll
        for (int d = 0; d < NG; ++d) {
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            const uint32_t base = part == 0 ? offsetof(Smem, gh) : offsetof(Smem, gl);
            bf16x4_t half[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
              typedef short v4i16_t __attribute__((ext_vector_type(4)));
              const char* src = lds + base + gtr[d][rr] + par + kqo;
              v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) v4i16_t*)(lds_void_t*)src);
              half[rr] = __builtin_bit_cast(bf16x4_t, t);
            }
            const bf16x8_t gf = {half[0][0], half[0][1], half[0][2], half[0][3],
                                 half[1][0], half[1][1], half[1][2], half[1][3]};
            gacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gf, fb[kq], gacc[d], 0, 0, 0);
          }
        }
      }
    }
  };

  if (ntiles > 0) issue_tile(0, smem[0]);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  auto step = [&](int it, auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    const int ks = it * KT;
    if (it + 1 < ntiles) issue_tile(ks + KT, smem[P ^ 1]);  // lands during compute
    compute_tile(ks, (uint32_t)(P * sizeof(Smem)));
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();  // the next tile is in LDS and every wave is done with this one
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
  }

  if constexpr (!BWD) {
    const float l_tot = pair32_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qvalid) {
      uint16_t* op = a.out + ((int64_t)qi * a.Hq + hq) * DH;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const bf16x4_t o4 = {to_bf16(oacc[d][4 * g4] * inv), to_bf16(oacc[d][4 * g4 + 1] * inv),
                               to_bf16(oacc[d][4 * g4 + 2] * inv),
                               to_bf16(oacc[d][4 * g4 + 3] * inv)};
          *(bf16x4_t*)(op + 32 * d + 8 * g4 + 4 * hg) = o4;
        }
      if (hg == 0) a.lse[(int64_t)qi * a.Hq + hq] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  } else {
    // sum the G query heads of each token in LDS (the tile buffers are free after the last
    // barrier of the loop), then one atomic add per (token, group)
    static_assert(128 * KP * 4 <= 2 * sizeof(Smem), "head sums exceed the tile buffers");
    float* red = (float*)smem;
#pragma unroll
    for (int d = 0; d < NG; ++d)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi)
        red[r * KP + 32 * d + 8 * (vi >> 2) + 4 * hg + (vi & 3)] = gacc[d][vi];
    __syncthreads();
    const int nt = q1 - q0;
    for (int idx = tid; idx < nt * a.K; idx += 256) {
      const int t = idx / a.K, c = idx - t * a.K;
      float s = 0.f;
      for (int hl = 0; hl < a.G; ++hl) s += red[(hl * a.T + t) * KP + c];
      if (s != 0.f) unsafeAtomicAdd(&a.dG[(int64_t)(q0 + t) * a.K + c], s);
    }
  }
}

// ============================================================================ key side
constexpr int QR = 64;  // query rows per streamed tile of the key-side kernel

template <int DH, int KP, int TQ>
struct TrainKSmem {
  __bf16 q[QR * DH];
  __bf16 d[QR * DH];
  __bf16 gh[TQ * KP];  // the tile's tokens' soft assignment (TQ rows, padded to 1 KB copies)
  __bf16 gl[TQ * KP];
  float lse2[QR];
  float D[QR];
};

// TQ: soft-assignment rows reserved per tile (the tile's T tokens, rounded up so the two planes
// are whole 1 KB copies)
template <int KP>
constexpr int train_k_tq(int T) {
  const int rows = T < 1024 / (2 * KP) ? 1024 / (2 * KP) : T;
  return rows;
}

// T = QR / G tokens per query tile (a compile-time constant, so row-to-token arithmetic folds).
template <int DH, int KP, int T, int TQ = train_k_tq<KP>(T)>
__global__ __launch_bounds__(256, (wgs_per_cu<TrainKSmem<DH, KP, TQ>>())) void train_k_kernel(const TrainArgs a) {
  using Smem = TrainKSmem<DH, KP, TQ>;
  constexpr int CH = DH / 8, RB = 2 * DH;
  constexpr int CHG = KP / 8, RBG = 2 * KP;
  constexpr int NS = DH / 16, KS = KP / 16, NG = KP / 32;
  constexpr int INSTS = QR * CH / 64 / 4;         // per wave per Q (and dO) tile
  constexpr int INSTG = (TQ * CHG + 63) / 64;     // per plane tile, spread over the waves
  static_assert(INSTS >= 1, "tile copies");
  static_assert(TQ * KP * 2 == INSTG * 1024, "the plane tiles are whole 1 KB copies");
  __shared__ __attribute__((aligned(1024))) Smem smem[2];

  const int tid = threadIdx.x, l = tid & 63, jq = l & 31, hg = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t comb = xcd_remap(blockIdx.x, (int64_t)a.Hkv * a.items);
  if (comb < 0) return;
  const int h = (int)(comb / a.items);
  const int blk = (int)(comb - (int64_t)h * a.items);
  const int window = a.window;
  const int k0 = blk * 128;
  const int kw_lo = k0 + wave * 32;
  const int key = kw_lo + jq;
  const bool kvalid = key < a.n;
  const int kw_hi = (int)min((int64_t)kw_lo + 31, a.n - 1);
  const bool wave_active = kw_lo < a.n;

  // query tiles with a far pair for some key of the block: tokens >= k0 + window
  const int64_t first_tok = (int64_t)k0 + window;
  if (first_tok >= a.n) return;
  const int t_begin = (int)(first_tok / T) * T;
  const int ntiles = (int)((a.n - t_begin + T - 1) / T);

  // this lane's key: K, V rows and soft assignment in registers (B operands)
  const int krow = kvalid ? key : (int)a.n - 1;
  bf16x8_t kreg[NS], vreg[NS], gkh[KS], gkl[KS];
  {
    const uint16_t* kp = a.k + ((int64_t)krow * a.Hkv + h) * DH + 8 * hg;
    const uint16_t* vp = a.v + ((int64_t)krow * a.Hkv + h) * DH + 8 * hg;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kreg[s] = *(const bf16x8_t*)(kp + 16 * s);
      vreg[s] = *(const bf16x8_t*)(vp + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      gkh[s] = *(const bf16x8_t*)(a.gh + (int64_t)krow * KP + 16 * s + 8 * hg);
      gkl[s] = *(const bf16x8_t*)(a.gl + (int64_t)krow * KP + 16 * s + 8 * hg);
    }
  }
  f32x16_t gacc[NG];
#pragma unroll
  for (int d = 0; d < NG; ++d) gacc[d] = f32x16_t{};

  // LDS reads: row m of a 32-row block as the A operand (Q, dO: rows of the tile; soft
  // assignment: the row's token)
  const char* lds = (const char*)smem;
  uint32_t qrd[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qrd[s] = (uint32_t)(jq * RB + (((2 * s + hg) ^ (swz(jq) % CH)) * 16));
  const int e4 = (l & 15) >> 2, m4 = l & 3, g2 = (l >> 4) & 1;

  // tile copies: Q and dO rows r = hl * T + t (head-major, as the query-side kernel) of tokens
  // t_0 + t, each 2 DH bytes; the planes' rows are the tile's tokens
  const uint32_t tok_b = (uint32_t)a.Hq * RB;  // bytes between one token's rows of a head
  uint32_t qofs[INSTS], qch[INSTS];
  int qrow_t[INSTS];
#pragma unroll
  for (int i = 0; i < INSTS; ++i) {
    const int lr = (wave * INSTS + i) * (64 / CH) + l / CH;  // tile row 0..QR-1
    qrow_t[i] = lr % T;
    qch[i] = (uint32_t)(((l % CH) ^ (swz(lr) % CH)) * 16);
    qofs[i] = (uint32_t)(lr % T) * tok_b + (uint32_t)(lr / T) * RB + qch[i];
  }
  uint32_t pofs[(INSTG + 3) / 4], pch[(INSTG + 3) / 4];
  int prow[(INSTG + 3) / 4];
#pragma unroll
  for (int j = 0; j < (INSTG + 3) / 4; ++j) {
    const int i = wave + 4 * j;  // copy i of the plane, by wave i % 4
    const int lin = i * 64 + l;  // 16-byte chunk of the plane tile
    prow[j] = lin / CHG;
    pch[j] = (uint32_t)(((lin % CHG) ^ (swz(prow[j]) % CHG)) * 16);
    pofs[j] = (uint32_t)prow[j] * RBG + pch[j];
  }
  float rec_lse = 0.f, rec_d = 0.f;
  const int rec_row = tid;  // thread < QR loads row tid's lse and D

  auto issue_tile = [&](int t0, Smem& sb) __attribute__((always_inline)) {
    const int nt = (int)min((int64_t)T, a.n - t0);  // tokens present
    const char* qb = (const char*)a.q + ((int64_t)t0 * a.Hq + (int64_t)h * a.G) * RB;
    const char* db = (const char*)a.dout + ((int64_t)t0 * a.Hq + (int64_t)h * a.G) * RB;
#pragma unroll
    for (int i = 0; i < INSTS; ++i) {
      // rows of missing tokens re-read token nt - 1 of the same head; their f is forced to 0
      const uint32_t off = qrow_t[i] < nt ? qofs[i]
                                          : qofs[i] - (uint32_t)(qrow_t[i] - (nt - 1)) * tok_b;
      dma16(qb, off, (char*)sb.q + (wave * INSTS + i) * 1024);
      dma16(db, off, (char*)sb.d + (wave * INSTS + i) * 1024);
    }
    const char* hb = (const char*)a.gh + (int64_t)t0 * RBG;
    const char* lb = (const char*)a.gl + (int64_t)t0 * RBG;
#pragma unroll
    for (int j = 0; j < (INSTG + 3) / 4; ++j) {
      if (wave + 4 * j < INSTG) {
        const int pr = prow[j] < nt ? prow[j] : nt - 1;
        const uint32_t off = (uint32_t)pr * RBG + pch[j];
        dma16(hb, off, (char*)sb.gh + (wave + 4 * j) * 1024);
        dma16(lb, off, (char*)sb.gl + (wave + 4 * j) * 1024);
      }
    }
    if (rec_row < QR) {
      const int t = rec_row % T, hl = rec_row / T;
      if (t < nt) {
        const int64_t idx = (int64_t)(t0 + t) * a.Hq + h * a.G + hl;
        rec_lse = a.lse[idx] * kLog2e;
        rec_d = a.D[idx];
      } else {
        rec_lse = 0.f;
        rec_d = 0.f;
      }
    }
  };
  auto finish_tile = [&](Smem& sb) __attribute__((always_inline)) {
    if (rec_row < QR) {
      sb.lse2[rec_row] = rec_lse;
      sb.D[rec_row] = rec_d;
    }
  };

  auto compute_tile = [&](int t0, const uint32_t par) __attribute__((always_inline)) {
    if (!wave_active) return;
    const int t_last = (int)min((int64_t)t0 + T, a.n) - 1;
    if (t_last - kw_lo < window) return;      // no far pair for this wave's keys
    const bool all_far = t0 - kw_hi >= window;  // every pair far (and causal)
    const Smem& sm = *(const Smem*)(lds + par);
    f32x16_t aacc = f32x16_t{};
    // T <= 32: a lane's rows 8 j + 4 hg + e of a block hold tokens (8 j + 4 hg + e) % T, so row
    // groups j >= JD repeat groups j % JD, and block 1 repeats block 0: the gate terms of block
    // 0's first JD groups serve every row
    constexpr int JD = T >= 32 ? 4 : (T >= 8 ? T / 8 : 1);
    float gl2[T <= 32 ? 4 * JD : 1], gsn[T <= 32 ? 4 * JD : 1];
#pragma unroll
    for (int b = 0; b < QR / 32; ++b) {
      // S = Q K^T and dP = dO V^T for rows 32 b .. 32 b + 31 (M) and the wave's keys (N)
      f32x16_t sacc = f32x16_t{}, pacc = f32x16_t{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8_t qf = *(const bf16x8_t*)(lds + par + offsetof(Smem, q) + qrd[s] + b * 32 * RB);
        const bf16x8_t df = *(const bf16x8_t*)(lds + par + offsetof(Smem, d) + qrd[s] + b * 32 * RB);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kreg[s], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(df, vreg[s], pacc, 0, 0, 0);
      }
      // A = G_q G_k^T: the rows' tokens repeat across blocks when T <= 32, so block 0's serves
      if (b == 0 || T > 32) {
        aacc = f32x16_t{};
        const int trow = (32 * b + jq) % T;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint32_t o = (uint32_t)(trow * RBG + (((2 * s + hg) ^ (swz(trow) % CHG)) * 16));
          const bf16x8_t hf = *(const bf16x8_t*)(lds + par + offsetof(Smem, gh) + o);
          const bf16x8_t lf = *(const bf16x8_t*)(lds + par + offsetof(Smem, gl) + o);
          aacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, gkh[s], aacc, 0, 0, 0);
          aacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, gkl[s], aacc, 0, 0, 0);
          aacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, gkh[s], aacc, 0, 0, 0);
        }
        if constexpr (T <= 32) {
#pragma unroll
          for (int i = 0; i < 4 * JD; ++i) gate_terms(a.lam * (aacc[i] - 0.5f), gl2[i], gsn[i]);
        }
      }
      // element v is row 32 b + 8 (v / 4) + 4 hg + v % 4 of the tile, key = this lane's key
      bf16x8_t fb[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row0 = 32 * b + 8 * j + 4 * hg;
        const f32x4_t l4 = *(const f32x4_t*)&sm.lse2[row0];
        const f32x4_t d4 = *(const f32x4_t*)&sm.D[row0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int vi = 4 * j + e;
          const int row = row0 + e;
          const int qi = t0 + row % T;
          const int dd = qi - key;
          float f = 0.f;
          if ((all_far || dd >= window) && qi < a.n && kvalid) {
            float l2s, sn;
            if constexpr (T <= 32) {
              l2s = gl2[4 * (j % JD) + e];
              sn = gsn[4 * (j % JD) + e];
            } else {
              gate_terms(a.lam * (aacc[vi] - 0.5f), l2s, sn);
            }
            const float p = fast_exp2(sacc[vi] * a.sl2 + l2s - l4[e]);
            f = p * (pacc[vi] - d4[e]) * a.lam * sn;
          }
          fb[j >> 1][(j & 1) * 4 + e] = to_bf16(f);
        }
      }
      // dG^T += G_q^T F over the block's rows: A = the rows' tokens' planes read transposed
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
        for (int d = 0; d < NG; ++d) {
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            bf16x4_t half[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
              const int trow = (32 * b + 16 * kq + 8 * rr + 4 * hg + e4) % T;
              const int c16 = 4 * d + 2 * g2 + (m4 >> 1);
              const uint32_t o = (uint32_t)(trow * RBG + ((c16 ^ (swz(trow) % CHG)) * 16) +
                                            (m4 & 1) * 8) +
                                 (part == 0 ? offsetof(Smem, gh) : offsetof(Smem, gl));
              typedef short v4i16_t __attribute__((ext_vector_type(4)));
              const char* src = lds + par + o;
              v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) v4i16_t*)(lds_void_t*)src);
              half[rr] = __builtin_bit_cast(bf16x4_t, t);
            }
            const bf16x8_t gf = {half[0][0], half[0][1], half[0][2], half[0][3],
                                 half[1][0], half[1][1], half[1][2], half[1][3]};
            gacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gf, fb[kq], gacc[d], 0, 0, 0);
          }
        }
      }
    }
  };

  issue_tile(t_begin, smem[0]);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  finish_tile(smem[0]);
  __syncthreads();
  auto step = [&](int it, auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    const int t0 = t_begin + it * T;
    if (it + 1 < ntiles) issue_tile(t0 + T, smem[P ^ 1]);
    compute_tile(t0, (uint32_t)(P * sizeof(Smem)));
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (it + 1 < ntiles) finish_tile(smem[P ^ 1]);
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
  }

  // lane holds groups 32 d + 8 (v / 4) + 4 hg + v % 4 of its key
  if (kvalid) {
#pragma unroll
    for (int d = 0; d < NG; ++d)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) {
        const int c = 32 * d + 8 * (vi >> 2) + 4 * hg + (vi & 3);
        if (c < a.K && gacc[d][vi] != 0.f) unsafeAtomicAdd(&a.dG[(int64_t)key * a.K + c], gacc[d][vi]);
      }
  }
}

// ============================================================================ launchers
template <int DH, int KP, bool BWD>
static void train_q_launch(const TrainArgs& a, hipStream_t stream) {
  const int64_t blocks = xcd_grid((int64_t)a.Hkv * a.items);
  // shared gates where every wave holds the same tokens and the tiles already take one
  // workgroup per CU (the gate tile then costs no occupancy)
  if constexpr (KP >= 64) {
    if (a.T <= 32) {
      hipLaunchKernelGGL((train_q_kernel<DH, KP, BWD, true>), dim3(blocks), dim3(256), 0, stream, a);
      return;
    }
  }
  hipLaunchKernelGGL((train_q_kernel<DH, KP, BWD, false>), dim3(blocks), dim3(256), 0, stream, a);
}

template <bool BWD>
static hipError_t train_q_dispatch(const TrainArgs& a, int dh, int KP, hipStream_t stream) {
  if (dh == 128) {
    if (KP == 32) train_q_launch<128, 32, BWD>(a, stream);
    else if (KP == 64) train_q_launch<128, 64, BWD>(a, stream);
    else train_q_launch<128, 128, BWD>(a, stream);
  } else {
    if (KP == 32) train_q_launch<64, 32, BWD>(a, stream);
    else if (KP == 64) train_q_launch<64, 64, BWD>(a, stream);
    else train_q_launch<64, 128, BWD>(a, stream);
  }
  return hipGetLastError();
}

template <int DH, int KP>
static void train_k_launch(const TrainArgs& a, hipStream_t stream) {
  const int64_t blocks = xcd_grid((int64_t)a.Hkv * a.items);
  switch (a.T) {  // QR / G tokens per query tile
    case 64: hipLaunchKernelGGL((train_k_kernel<DH, KP, 64>), dim3(blocks), dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((train_k_kernel<DH, KP, 32>), dim3(blocks), dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((train_k_kernel<DH, KP, 16>), dim3(blocks), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((train_k_kernel<DH, KP, 8>), dim3(blocks), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((train_k_kernel<DH, KP, 4>), dim3(blocks), dim3(256), 0, stream, a); break;
  }
}

hipError_t launch_train_attention(const TrainShape& s, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const __bf16* gh, const __bf16* gl,
                                  uint16_t* out, float* lse, hipStream_t stream) {
  TrainArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.gh = gh;
  a.gl = gl;
  a.out = out;
  a.lse = lse;
  a.n = s.n;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.Hq / s.Hkv;
  a.T = 128 / a.G;
  a.K = s.K;
  a.window = (int)(s.window < s.n + 1 ? s.window : s.n + 1);
  a.sl2 = s.scale * kLog2e;
  a.lam = s.lam;
  a.items = (int)((s.n + a.T - 1) / a.T);
  return train_q_dispatch<false>(a, s.dh, s.KP, stream);
}

hipError_t launch_train_attention_bwd(const TrainShape& s, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const __bf16* gh, const __bf16* gl,
                                      const float* lse, const uint16_t* dout, const float* D,
                                      float* dG, hipStream_t stream) {
  TrainArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.gh = gh;
  a.gl = gl;
  a.lse = (float*)lse;
  a.dout = dout;
  a.D = D;
  a.dG = dG;
  a.n = s.n;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.Hq / s.Hkv;
  a.K = s.K;
  a.window = (int)(s.window < s.n + 1 ? s.window : s.n + 1);
  a.sl2 = s.scale * kLog2e;
  a.lam = s.lam;
  // query side: 128-row tiles of T = 128 / G tokens
  a.T = 128 / a.G;
  a.items = (int)((s.n + a.T - 1) / a.T);
  hipError_t e = train_q_dispatch<true>(a, s.dh, s.KP, stream);
  if (e != hipSuccess) return e;
  // key side: 128 keys per workgroup, 64-row query tiles of QR / G tokens
  a.T = QR / a.G;
  a.items = (int)((s.n + 127) / 128);
  if (s.dh == 128) {
    if (s.KP == 32) train_k_launch<128, 32>(a, stream);
    else if (s.KP == 64) train_k_launch<128, 64>(a, stream);
    else train_k_launch<128, 128>(a, stream);
  } else {
    if (s.KP == 32) train_k_launch<64, 32>(a, stream);
    else if (s.KP == 64) train_k_launch<64, 64>(a, stream);
    else train_k_launch<64, 128>(a, stream);
  }
  return hipGetLastError();
}

// ============================================================================ Sinkhorn backward
// Row pass of the plan: with u_i = -logsumexp_c(S_ic + vprev_c) (0 without iterations) and
// P = exp(S + u + vlast), dE = dG o P; dS = dE, du_i = sum_c dE_ic, and the block's column sums
// of dE into part[block][c]. One wave per row, rows strided over the grid.
__global__ __launch_bounds__(256) void train_sk_plan_bwd_kernel(
    const float* __restrict__ S, int64_t n, int K, int ldS, const float* __restrict__ vprev,
    const float* __restrict__ vlast, int iters, const float* __restrict__ dG,
    float* __restrict__ dS, float* __restrict__ du, float* __restrict__ part) {
  __shared__ float colsum[4][1024];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int c = l; c < K; c += 64) colsum[w][c] = 0.f;
  for (int64_t row = (int64_t)blockIdx.x * 4 + w; row < n; row += (int64_t)gridDim.x * 4) {
    const float* sp = S + row * ldS;
    float u = 0.f;
    if (iters > 0) {
      float mx = -INFINITY;
      for (int c = l; c < K; c += 64) mx = fmaxf(mx, sp[c] + vprev[c]);
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
      float sum = 0.f;
      for (int c = l; c < K; c += 64) sum += fast_exp2((sp[c] + vprev[c] - mx) * kLog2e);
      for (int o = 32; o >= 1; o >>= 1) sum += shfl_xor_f(sum, o);
      u = -(mx + __logf(sum));
    }
    float rs = 0.f;
    for (int c = l; c < K; c += 64) {
      const float e = dG[row * K + c] * __expf(sp[c] + u + (iters > 0 ? vlast[c] : 0.f));
      dS[row * K + c] = e;
      rs += e;
      colsum[w][c] += e;
    }
    for (int o = 32; o >= 1; o >>= 1) rs += shfl_xor_f(rs, o);
    if (l == 0) du[row] = rs;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < K; c += 256)
    part[(int64_t)blockIdx.x * K + c] = colsum[0][c] + colsum[1][c] + colsum[2][c] + colsum[3][c];
}

// Iteration t in reverse: u = u^t from vprev = v^{t-1}; Wc = exp(S + u + vcur - log(n/K)) (the
// column step's weights), du_i <- du_i - sum_c dvcur_c Wc_ic, Wr = exp(S + vprev + u) (the row
// step's weights), dS -= dvcur o Wc + du Wr, and the block's column sums of du Wr into part.
// du_in == nullptr: the carried du is 0.
__global__ __launch_bounds__(256) void train_sk_iter_bwd_kernel(
    const float* __restrict__ S, int64_t n, int K, int ldS, const float* __restrict__ vprev,
    const float* __restrict__ vcur, const float* __restrict__ dvcur, float log_mass,
    const float* __restrict__ du_in, float* __restrict__ dS, float* __restrict__ part) {
  __shared__ float colsum[4][1024];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int c = l; c < K; c += 64) colsum[w][c] = 0.f;
  for (int64_t row = (int64_t)blockIdx.x * 4 + w; row < n; row += (int64_t)gridDim.x * 4) {
    const float* sp = S + row * ldS;
    float mx = -INFINITY;
    for (int c = l; c < K; c += 64) mx = fmaxf(mx, sp[c] + vprev[c]);
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
    float sum = 0.f;
    for (int c = l; c < K; c += 64) sum += fast_exp2((sp[c] + vprev[c] - mx) * kLog2e);
    for (int o = 32; o >= 1; o >>= 1) sum += shfl_xor_f(sum, o);
    const float u = -(mx + __logf(sum));
    float acc = 0.f;
    for (int c = l; c < K; c += 64) acc += dvcur[c] * __expf(sp[c] + u + vcur[c] - log_mass);
    for (int o = 32; o >= 1; o >>= 1) acc += shfl_xor_f(acc, o);
    const float du = (du_in ? du_in[row] : 0.f) - acc;
    for (int c = l; c < K; c += 64) {
      const float wc = __expf(sp[c] + u + vcur[c] - log_mass);
      const float wr = __expf(sp[c] + vprev[c] + u);
      dS[row * K + c] -= dvcur[c] * wc + du * wr;
      colsum[w][c] += du * wr;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < K; c += 256)
    part[(int64_t)blockIdx.x * K + c] = colsum[0][c] + colsum[1][c] + colsum[2][c] + colsum[3][c];
}

// out[c] = sign * sum over blocks of part[b][c], accumulated in fp64.
__global__ __launch_bounds__(256) void train_colsum_kernel(const float* __restrict__ part,
                                                           int nblocks, int K, float sign,
                                                           float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= K) return;
  double s = 0.0;
  for (int b = 0; b < nblocks; ++b) s += part[(int64_t)b * K + c];
  out[c] = (float)(sign * s);
}

int train_sk_blocks(int64_t n) {
  int64_t b = (n + 63) / 64;
  return (int)(b < 1 ? 1 : (b > 2048 ? 2048 : b));
}

hipError_t launch_train_sk_plan_bwd(const float* S, int64_t n, int K, int ldS, const float* vprev,
                                    const float* vlast, int iters, const float* dG, float* dS,
                                    float* du, float* part, float* dv, hipStream_t stream) {
  const int nb = train_sk_blocks(n);
  hipLaunchKernelGGL(train_sk_plan_bwd_kernel, dim3(nb), dim3(256), 0, stream, S, n, K, ldS, vprev,
                     vlast, iters, dG, dS, du, part);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(train_colsum_kernel, dim3((K + 255) / 256), dim3(256), 0, stream, part, nb, K,
                     1.f, dv);
  return hipGetLastError();
}

hipError_t launch_train_sk_iter_bwd(const float* S, int64_t n, int K, int ldS, const float* vprev,
                                    const float* vcur, const float* dvcur, const float* du_in,
                                    float* dS, float* part, float* dvprev, hipStream_t stream) {
  const int nb = train_sk_blocks(n);
  const float log_mass = (float)log((double)n / (double)K);
  hipLaunchKernelGGL(train_sk_iter_bwd_kernel, dim3(nb), dim3(256), 0, stream, S, n, K, ldS, vprev,
                     vcur, dvcur, log_mass, du_in, dS, part);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(train_colsum_kernel, dim3((K + 255) / 256), dim3(256), 0, stream, part, nb, K,
                     -1.f, dvprev);
  return hipGetLastError();
}

// ============================================================================ dense pieces
// dZ[i, c] = sum_k dS[i, k] C[k, c]: one block of 256 threads per 256 / d_g rows (d_g <= 256), or
// strided columns.
__global__ __launch_bounds__(256) void train_dz_kernel(const float* __restrict__ dS,
                                                       const float* __restrict__ C, int64_t n,
                                                       int K, int dg, float* __restrict__ dZ) {
  const int64_t idx0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t idx = idx0; idx < n * dg; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / dg;
    const int c = (int)(idx - i * dg);
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc += dS[i * K + k] * C[(int64_t)k * dg + c];
    dZ[idx] = acc;
  }
}

hipError_t launch_train_dz(const float* dS, const float* C, int64_t n, int K, int dg, float* dZ,
                           hipStream_t stream) {
  int64_t blocks = (n * dg + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(train_dz_kernel, dim3(blocks), dim3(256), 0, stream, dS, C, n, K, dg, dZ);
  return hipGetLastError();
}

// C[m, c] += sum over rows r of A[r, m] B[r, c] (A [R, M], B [R, N] row-major fp32; C zeroed by
// the caller): 64 x 64 output tiles, rows split into chunks of 512 per block, 32-row slabs staged
// in LDS, 4 x 4 outputs per thread, one atomic add per output and chunk.
__global__ __launch_bounds__(256) void gemm_tn_atomic_kernel(const float* __restrict__ A,
                                                             const float* __restrict__ B,
                                                             int64_t R, int M, int N,
                                                             float* __restrict__ C) {
  constexpr int TM = 64, TN = 64, SL = 32, CHUNK = 512;
  __shared__ float As[SL][TM + 4], Bs[SL][TN + 4];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TN;
  const int64_t r0 = (int64_t)blockIdx.z * CHUNK;
  const int64_t r1 = r0 + CHUNK < R ? r0 + CHUNK : R;
  float acc[4][4] = {};
  for (int64_t rs = r0; rs < r1; rs += SL) {
    for (int e = tid; e < SL * TM; e += 256) {
      const int rr = e / TM, mm = e % TM;
      const int64_t row = rs + rr;
      As[rr][mm] = (row < r1 && m0 + mm < M) ? A[row * M + m0 + mm] : 0.f;
      Bs[rr][mm] = (row < r1 && n0 + mm < N) ? B[row * N + n0 + mm] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int rr = 0; rr < SL; ++rr) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[rr][ty * 4 + i];
        bv[i] = Bs[rr][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, c = n0 + tx * 4 + j;
      if (m < M && c < N && acc[i][j] != 0.f) unsafeAtomicAdd(&C[(int64_t)m * N + c], acc[i][j]);
    }
}

hipError_t launch_gemm_tn_atomic(const float* A, const float* B, int64_t R, int M, int N, float* C,
                                 hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const dim3 grid((M + 63) / 64, (N + 63) / 64, (unsigned)((R + 511) / 512));
  hipLaunchKernelGGL(gemm_tn_atomic_kernel, grid, dim3(256), 0, stream, A, B, R, M, N, C);
  return hipGetLastError();
}

}  // namespace focus
