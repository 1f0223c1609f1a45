// Internal declarations of the Focus HIP library (gfx950 / CDNA4): device helpers and the
// host-side launchers each kernel source exports to the C-ABI layer in focus_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace focus {

// ------------------------------------------------------------------ vector types
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kXcds = 8;                 // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, kWave); }
__device__ __forceinline__ int shfl_xor_i(int x, int m) { return __shfl_xor(x, m, kWave); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum of x over the lane pair (l, l ^ 32) without a trip through LDS: gfx950's
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes 0..31 of its second,
// so with both operands equal to x each lane ends up holding the pair's two values.
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x of another lane of the same 16-lane row, moved on the VALU (data-parallel-primitive
// control CTRL: 0xB1 / 0x4E swap lanes l^1 / l^2 within quads, 0x141 mirrors the 8-lane half
// row, 0x140 the 16-lane row, 0x128 rotates the row by 8, i.e. l^8). Every lane is a valid
// source for these controls.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp_move_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

// Map a linear block id to a position in [0, total) so that each XCD receives one
// contiguous range: block b is dispatched to XCD b % 8, so consecutive ranges of work
// (and the data they share) stay in one XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t total) {
  int64_t per = (total + kXcds - 1) / kXcds;
  int64_t x = b % kXcds, j = b / kXcds;
  if (j >= per) return -1;
  int64_t c = x * per + j;
  return c < total ? c : -1;
}
inline int64_t xcd_grid(int64_t total) {
  int64_t per = (total + kXcds - 1) / kXcds;
  return per * kXcds;
}

// ------------------------------------------------------------------ LDS copies
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// One wave-wide global_load_lds_dwordx4: lane L copies 16 bytes from base + voff (base uniform,
// voff per lane) to LDS byte lds_dst + 16 L. Issued through inline asm so the compiler does not
// treat the copy as a pending write to every LDS location: with the builtin it waits for the
// whole copy before the first LDS read that follows, which serialises the prefetch of the next
// tile with the compute on the current one. The caller waits (vmcnt) before the data is read.
// The LDS destination goes in as a pointer operand (not an integer), so the compiler keeps
// treating the buffer as written by the asm statement. The instruction takes it in m0; the
// operand is constrained to m0, so the compiler itself loads m0 before the statement and never
// assumes m0 still holds an earlier value.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, void* lds_dst) {
  lds_char_t* m = (lds_char_t*)lds_dst;
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(m) : "memory");
}

// Tiles of bf16 rows in LDS keep each row's 16-byte chunks permuted by chunk ^ swz(row) (taken
// modulo the chunks per row). swz maps the 16 rows of a block to 16 distinct values whose even
// parts differ across any 4 consecutive rows, so both access patterns of a 256-byte-row tile are
// free of bank conflicts: 16 lanes reading one chunk of 16 consecutive rows (an MFMA operand read
// along the row) and 16 lanes reading 2 adjacent chunks of 4 consecutive rows (the transposing
// read). swz depends on the low 4 bits of the row only, so rows 16 apart share a permutation and
// every lane's LDS addresses differ between tiles and row blocks by compile-time constants.
__device__ __forceinline__ int swz(int row) {
  return ((row & 1) << 3) | (((row >> 1) & 1) << 2) | ((row >> 2) & 1) | (((row >> 3) & 1) << 1);
}

// s_waitcnt immediate for vmcnt(0) alone (gfx9 encoding: expcnt and lgkmcnt at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

// ------------------------------------------------------------------ launchers
// All launchers enqueue on `stream` and return hipSuccess or the launch error.

// C[M, ldc] (first N columns) = A[M, Kd] * B[N, Kd]^T, fp32 in and out, to fp32 accuracy on the
// bf16 MFMA (each operand split into three bf16 parts on the fly).
hipError_t launch_gemm_nt_f32(const float* A, const float* B, float* C, int64_t M, int N, int Kd,
                              int ldc, hipStream_t stream);
// The same product with B given as its three bf16 planes Bp[3][N][Kd] (split_planes below);
// requires Kd % 32 == 0. Bp must stay valid until the product has run.
hipError_t launch_gemm_nt_f32_planes(const float* A, const __bf16* Bp, float* C, int64_t M, int N,
                                     int Kd, int ldc, hipStream_t stream);
// P[p * count + i] = part p (0: bf16(x), 1: bf16 of the remainder, 2: bf16 of what is left) of
// x = B[i], for i < count.
hipError_t launch_split_planes(const float* B, int64_t count, __bf16* P, hipStream_t stream);
// Bt[N, Kd] = transpose of B[Kd, N], fp32.
hipError_t launch_transpose_f32(const float* B, float* Bt, int Kd, int N, hipStream_t stream);
// One Sinkhorn iteration on S [n, ldS] (first K columns): row step with the current v,
// column partials per block, then the column step that overwrites v.
hipError_t launch_sinkhorn_iter(const float* S, int64_t n, int K, int ldS, float* v, float2* partials,
                                int nblocks, hipStream_t stream);
int sinkhorn_blocks(int64_t n, int K);
hipError_t launch_topk(const float* S, const float* v, int64_t n, int K, int ldS, int top_k,
                       int32_t* groups, hipStream_t stream);
// C[M, N] (row stride ldc) = A[M, Kd] B[N, Kd]^T at fp32-level accuracy from two-part fp16
// splits (three fp16 MFMA part products). Needs Kd % 32 == 0. Bp (2 N Kd fp16) and bscale (N
// floats) are scratch for B's scaled planes. Rows of A whose outputs are not finite (an
// element beyond fp16's range, or not finite) are appended to flags (nflags counts them) when
// flags is given. With col_partials (N <= 256): the epilogue also takes Sinkhorn's first row
// step and writes one (max, sum) column summary row per row block, *row_blocks of them, to
// col_partials [*row_blocks, N]; listed rows stay out of them.
hipError_t launch_gemm_nt_f16x3(const float* A, const float* B, _Float16* Bp, float* bscale,
                                float* C, int64_t M, int N, int Kd, int ldc, int32_t* flags,
                                int32_t* nflags, float2* col_partials, int64_t* row_blocks,
                                hipStream_t stream);
// S[row, :K] in fp32 for the rows listed in list[0..*count): h_row . Ft[c] when Ft ([K, d]) is
// given, else (h_row W) . Cm[c] with W [d, d_g] and Cm [K, d_g]. n: the list's capacity. With
// partials: Sinkhorn's first row step on those rows too, one column summary row per launched
// block (exact_rows_blocks(n) of them) at partials [blocks, K].
int exact_rows_blocks(int64_t n);
hipError_t launch_exact_rows(const float* H, int d, const float* Ft, const float* W,
                             const float* Cm, int dg, int K, const int32_t* list,
                             const int32_t* count, int64_t n, float* S, int ldS,
                             float2* partials, hipStream_t stream);
// Sinkhorn's column step v_c = log(n / K) - logsumexp over the nblocks column summaries.
hipError_t launch_sinkhorn_cols(const float2* partials, int nblocks, int64_t n, int K, float* v,
                                hipStream_t stream);
hipError_t launch_fill_f32(float* p, float value, int64_t count, hipStream_t stream);
hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t count, hipStream_t stream);

// Stable counting sort of memberships (bucket).
constexpr int kBucketChunk = 64;  // tokens per chunk: one wave of the scatter pass, one step
hipError_t launch_bucket(const int32_t* groups, int batch, int64_t n, int K, int top_k,
                         int32_t* offsets, int32_t* idx, int32_t* slot, int32_t* counts,
                         int32_t* totals, hipStream_t stream);

// Appends one token per sequence to bucketed memberships (out of place; see focus.h).
hipError_t launch_bucket_append(const int32_t* new_groups, const int32_t* cache_len, int batch,
                                int64_t cap, int K, int top_k, const int32_t* off_in,
                                const int32_t* idx_in, int32_t* off_out, int32_t* idx_out,
                                hipStream_t stream);

// Group-slotted memberships (see bucket_kernels.hip): from a bucket, and the O(top_k) append.
hipError_t launch_slots_from_bucket(const int32_t* off, const int32_t* idx, int batch, int64_t cap,
                                    int K, int gcap, int32_t* seg_len, int32_t* seg_pos,
                                    int32_t* overflow, hipStream_t stream);
hipError_t launch_slots_append(const int32_t* new_groups, const int32_t* cache_len, int batch,
                               int K, int top_k, int gcap, int32_t* seg_len, int32_t* seg_pos,
                               int32_t* overflow, hipStream_t stream);

// Attention pieces.
struct AttnShape {
  int64_t n;     // tokens
  int64_t nk;    // memberships (n * top_k)
  int Hq, Hkv, G, dh, K, top_k;
  int64_t window;
  float scale;   // natural-units logit scale
};
hipError_t launch_gather_kv(const uint16_t* k, const uint16_t* v, const int32_t* idx,
                            const int32_t* groups, const int32_t* slot, const AttnShape& s,
                            uint16_t* kg, uint16_t* vg, int32_t* kinfo, hipStream_t stream);
hipError_t launch_tile_prefix(const int32_t* offsets, int K, int T, int32_t* tile_pre,
                              hipStream_t stream);
// group-pass work items per kv head (an upper bound: ceil(nk / T) + K)
int attn_work_items(int64_t nk, int T, int K);
hipError_t launch_plan_tiles(const int32_t* offsets, const int32_t* tile_pre, const int32_t* kinfo,
                             const AttnShape& s, int32_t* plan, hipStream_t stream);
hipError_t launch_group_attention(const uint16_t* q, const uint16_t* kg, const uint16_t* vg,
                                  const int32_t* offsets, const int32_t* tile_pre,
                                  const int32_t* kinfo, const int32_t* plan, const AttnShape& s,
                                  _Float16* og, float* lseg, hipStream_t stream);
// Asymmetric top-k (s.nk = query memberships, s.top_k = groups per query): the work plan from
// the query bucket (q_off, q_idx, tile prefix over q_off) and the key bucket (k_off, k_idx), and
// the group pass over keys gathered along the key bucket (kinfo from launch_gather_kv with
// top_k 1). The window pass is launch_window_attention with the query slots.
hipError_t launch_plan_tiles_asym(const int32_t* q_off, const int32_t* tile_pre,
                                  const int32_t* q_idx, const int32_t* k_off,
                                  const int32_t* k_idx, const AttnShape& s, int32_t* plan,
                                  hipStream_t stream);
hipError_t launch_group_attention_asym(const uint16_t* q, const uint16_t* kg, const uint16_t* vg,
                                       const int32_t* q_idx, const int32_t* kinfo,
                                       const int32_t* plan, const AttnShape& s, _Float16* og,
                                       float* lseg, hipStream_t stream);
hipError_t launch_window_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const _Float16* og, const float* lseg, const int32_t* slot,
                                   const AttnShape& s, uint16_t* out, float* lse,
                                   hipStream_t stream);
// Soft-gate forward over every causal pair: far-pair logits get bias_none / bias_share
// (natural-log units) by whether the tokens share a group.
hipError_t launch_soft_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* groups, const AttnShape& s, float bias_none,
                                 float bias_share, uint16_t* out, float* lse, hipStream_t stream);
int attn_tile_tokens(int G);  // query tokens per attention tile: 128 / G

// Soft-gated training path (train_kernels.hip).
struct TrainShape {
  int64_t n;
  int Hq, Hkv, dh, K;
  int KP;         // groups padded to a multiple of 32 (the soft-assignment planes' row length)
  int64_t window;
  float scale;    // natural-units logit scale
  float lam;      // gate sharpness lambda
};
// Soft assignment g = exp(S + u + vlast), u from vprev (the last row step; iters == 0: g =
// exp(S)), written as two bf16 planes gh, gl [n, KP] (zero past K).
hipError_t launch_train_plan(const float* S, int64_t n, int K, int ldS, int KP, const float* vprev,
                             const float* vlast, int iters, __bf16* gh, __bf16* gl,
                             hipStream_t stream);
// D[row] = dout[row] . out[row] over rows of dh bf16 values.
hipError_t launch_train_delta(const uint16_t* dout, const uint16_t* out, int64_t rows, int dh,
                              float* D, hipStream_t stream);
// Forward over every causal pair, far pairs gated by log sigmoid(lam (g_i . g_j - 1/2)).
hipError_t launch_train_attention(const TrainShape& s, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const __bf16* gh, const __bf16* gl,
                                  uint16_t* out, float* lse, hipStream_t stream);
// dG [n, K] += dL/dg from both sides of every far pair (dG zeroed by the caller).
hipError_t launch_train_attention_bwd(const TrainShape& s, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const __bf16* gh, const __bf16* gl,
                                      const float* lse, const uint16_t* dout, const float* D,
                                      float* dG, hipStream_t stream);
// Sinkhorn backward: the plan's row pass (dS = dG o P, du, dv = column sums), then one call per
// iteration in reverse (dS -= ..., dvprev = -column sums of du o Wr). part: train_sk_blocks(n) x K.
int train_sk_blocks(int64_t n);
hipError_t launch_train_sk_plan_bwd(const float* S, int64_t n, int K, int ldS, const float* vprev,
                                    const float* vlast, int iters, const float* dG, float* dS,
                                    float* du, float* part, float* dv, hipStream_t stream);
hipError_t launch_train_sk_iter_bwd(const float* S, int64_t n, int K, int ldS, const float* vprev,
                                    const float* vcur, const float* dvcur, const float* du_in,
                                    float* dS, float* part, float* dvprev, hipStream_t stream);
// dZ = dS C ([n, K] x [K, dg]); C[M, N] += A^T B over R rows (A [R, M], B [R, N]).
hipError_t launch_train_dz(const float* dS, const float* C, int64_t n, int K, int dg, float* dZ,
                           hipStream_t stream);
hipError_t launch_gemm_tn_atomic(const float* A, const float* B, int64_t R, int M, int N, float* C,
                                 hipStream_t stream);

// Decode.
struct DecodeShape {
  int B;
  int64_t Lmax;
  int Hq, Hkv, G, dh, K, top_k;
  int64_t window;
  float scale;
  int splits;  // key-range splits per (sequence, kv head)
};
int decode_splits(const DecodeShape& s);
// Paged caches: kc / vc are pools of num_pages pages of page_size token rows; position p of
// sequence b lives in row table[b * pages_per_seq + p / page_size] * page_size + p % page_size.
struct DecodePaging {
  const int32_t* table;
  int page_size;
  int64_t pages_per_seq, num_pages;
};
// Group-slotted cache memberships (cache_idx then holds seg_pos [B, K, gcap]; cache_off unused).
struct DecodeSlots {
  const int32_t* seg_len;  // [B, K]
  int gcap;
};
// pg == nullptr: kc / vc are [B, Lmax, Hkv, dh] per-sequence caches. sl == nullptr: bucketed
// cache memberships (cache_off [B, K + 1], cache_idx [B, Lmax * top_k]).
hipError_t launch_decode(const uint16_t* q, const int32_t* q_groups, const uint16_t* kc,
                         const uint16_t* vc, const int32_t* cache_len, const int32_t* cache_groups,
                         const int32_t* cache_off, const int32_t* cache_idx, const DecodeShape& s,
                         float* part_o, float* part_ml, uint16_t* out, float* lse,
                         hipStream_t stream, const DecodePaging* pg = nullptr,
                         const DecodeSlots* sl = nullptr);

}  // namespace focus
