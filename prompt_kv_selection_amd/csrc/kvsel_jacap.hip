// Jacap leverage scores for gfx950 (bf16 keys and outputs).
//
// Method (web page "Jacap: Preserving Nonlinear Information in KV-Cache
// Eviction", sections "Practical approximation" and "Algorithm 1: one
// eviction event"), per head over its N cached tokens:
//   z_i = k_i . mu_Q / (tau sqrt(d)), alpha = softmax(z) over all N tokens,
//   kappa_i = k_i^T Lambda_Q k_i (diagonal Lambda_Q),
//   w_i = [alpha_i (1 - alpha_i)]^2 kappa_i / d,
//   A = I + sum_j w_j u_j u_j^T (u_j: W_O v_j or v_j, given by the caller),
//   r_i = w_i u_i^T A^{-1} u_i = w_i |L^{-1} u_i|^2 with A = L L^T.
// The top scores (after protected tokens) are then selected and gathered by
// the refresh selection.
//
// Kernels:
//   jacap_logits   per (head, chunk): z and kappa of every token (a quad of
//                  lanes per token, 16-byte loads), the chunk's softmax
//                  partial (max, and Z - 1: the mass beyond the max).
//   jacap_weights  per (head, chunk): the head's partials merged in a fixed
//                  order (a lane per chunk, then a butterfly), then w of
//                  every token; also clears the selection's histograms.
//   jacap_gram     per (head, slice): the slice's part of sum w u u^T on MFMA
//                  (v_mfma_f32_32x32x16_bf16), lower tiles only: u^T (exact
//                  bf16) times (w u) split into bf16 hi + lo, about 16
//                  significant bits per product; fp32 accumulation.
//   jacap_reduce   per (head, part): the slices' parts summed in slice order.
//   jacap_factor   per head: A = I + the Gram matrix, Cholesky (fp32), then
//                  M = L^{-1}, both blocked by 8-column panels in LDS,
//                  stored as bf16 hi + lo.
//   jacap_leverage per (head, chunk): Y = M U^T on MFMA (hi and lo of M
//                  against the exact bf16 u, the k-steps of the lower
//                  triangle only), r = w * column sums of Y^2.
// The two N d^2 contractions are the MFMA part.  K is read once and U twice
// (the Gram matrix must be complete before any leverage score).

#include <math.h>

#include <algorithm>
#include <functional>
#include <type_traits>

#include "kvsel_internal.h"
#include "kvsel_jacap.h"

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kJThreads = 256;
constexpr int kJChunk = 1024;  // tokens per logits / weights / leverage workgroup
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Softmax partials as (m, s1): the maximum and Z - 1 with Z = sum exp(z - m),
// i.e. the mass of every term but the maximum's.  Keeping Z - 1 rather than Z
// lets 1 - alpha of the largest term be formed without cancellation.  Empty:
// (kNegBig, -1); one logit z: (z, 0).
__device__ __forceinline__ void lse1_merge(float& m, float& s1, float mo, float s1o) {
  if (mo > m) {
    s1 = fmaf(1.f + s1, __expf(m - mo), s1o);
    m = mo;
  } else {
    s1 = fmaf(1.f + s1o, __expf(mo - m), s1);
  }
}

// Sum over the four lanes of a quad (DPP quad permutations, no LDS).
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return v;
}

// z_i and kappa_i of the chunk's tokens; (max, sum exp(z - max)) of the chunk.
// A quad of lanes takes a token: lane p of the quad loads 16-byte pieces
// p, p + 4, ... of the row (64 contiguous bytes per row and load), so a
// pass covers 64 tokens and the reduction is two DPP steps.  kLogitPasses
// passes are loaded before any is reduced.
constexpr int kLogitPasses = 4;
template <int D>
__global__ __launch_bounds__(kJThreads) void jacap_logits_kernel(const JacapArgs j, const __bf16* __restrict__ K) {
  constexpr int CPL = D / 8 / 4;  // 16-byte pieces per lane
  constexpr int TPP = kJThreads / 4;
  const int head = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, part = tid & 3, slot = tid >> 2;
  __shared__ float sm[kJThreads / 64], sz[kJThreads / 64];
  float mu[CPL][8], lam[CPL][8];
#pragma unroll
  for (int q = 0; q < CPL; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mu[q][e] = j.mu[(long long)head * D + (part + 4 * q) * 8 + e];
      lam[q][e] = j.lambda[(long long)head * D + (part + 4 * q) * 8 + e];
    }
  if (head == 0 && c == 0 && tid == 0 && j.err != nullptr) *j.err = 0u;  // the later kernels raise flags
  const float scale = 1.f / (j.tau * sqrtf((float)D));
  float m = kNegBig, s = -1.f;
  const int t0 = c * kJChunk, t1 = min(t0 + kJChunk, j.N);
  const __bf16* kh = K + (long long)head * j.N * D;
  for (int base = t0; base < t1; base += kLogitPasses * TPP) {  // every lane takes part in the DPP steps
    uint4 raw[kLogitPasses][CPL];
#pragma unroll
    for (int h = 0; h < kLogitPasses; ++h) {
      const int t = min(base + h * TPP + slot, t1 - 1);  // rows past the chunk repeat its last (not stored)
#pragma unroll
      for (int q = 0; q < CPL; ++q) raw[h][q] = *reinterpret_cast<const uint4*>(kh + (long long)t * D + (part + 4 * q) * 8);
    }
#pragma unroll
    for (int h = 0; h < kLogitPasses; ++h) {
      float zz = 0.f, kk = 0.f;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const unsigned w[4] = {raw[h][q].x, raw[h][q].y, raw[h][q].z, raw[h][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(w[e] << 16), k1 = __uint_as_float(w[e] & 0xFFFF0000u);
          zz = fmaf(k0, mu[q][2 * e], zz);
          zz = fmaf(k1, mu[q][2 * e + 1], zz);
          kk = fmaf(lam[q][2 * e] * k0, k0, kk);
          kk = fmaf(lam[q][2 * e + 1] * k1, k1, kk);
        }
      }
      zz = quad_sum(zz);
      kk = quad_sum(kk);
      const int t = base + h * TPP + slot;
      if (t < t1 && part == 0) {
        const float z = zz * scale;
        j.z[(long long)head * j.N + t] = z;
        j.kappa[(long long)head * j.N + t] = kk;
        lse1_merge(m, s, z, 0.f);
      }
    }
  }
  // The chunk's partial: lanes of the wave, then the waves in order.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mo = __shfl_xor(m, o), so = __shfl_xor(s, o);
    lse1_merge(m, s, mo, so);
  }
  if ((tid & 63) == 0) {
    sm[tid >> 6] = m;
    sz[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = sm[0], ss = sz[0];
    for (int w = 1; w < kJThreads / 64; ++w) lse1_merge(mm, ss, sm[w], sz[w]);
    j.part[((long long)head * j.nch + c) * 2] = mm;
    j.part[((long long)head * j.nch + c) * 2 + 1] = ss;
  }
}

// w_i of the chunk's tokens from the head's softmax normaliser.
__global__ __launch_bounds__(kJThreads) void jacap_weights_kernel(const JacapArgs j, int D) {
  const int head = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  __shared__ float s_m, s_z;
  if (tid < 64) {  // the head's partials: lane l takes chunks l, l + 64, ..., then the wave merges
    float m = kNegBig, s = -1.f;
    for (int q = tid; q < j.nch; q += 64)
      lse1_merge(m, s, j.part[((long long)head * j.nch + q) * 2], j.part[((long long)head * j.nch + q) * 2 + 1]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float mo = __shfl_xor(m, o), so = __shfl_xor(s, o);
      lse1_merge(m, s, mo, so);
    }
    if (tid == 0) {  // lane 0's result, the same fixed order in every workgroup of the head
      s_m = m;
      s_z = s;
      if (!(isfinite(m) && isfinite(s) && s >= 0.f)) raise_error(j.err, kErrNonFinite);
    }
  }
  // The second moment is a variance-like diagonal: a negative (or NaN)
  // entry would make weights and scores negative and rank them wrongly.
  // Checked once per head; the later kernels run regardless.
  if (c == 0 && tid < 64) {
    bool bad = false;
    for (int d = tid; d < D; d += 64) bad = bad || !(j.lambda[(long long)head * D + d] >= 0.f);
    if (__ballot(bad) != 0 && tid == 0) raise_error(j.err, kErrDomain);
  }
  __syncthreads();
  const float M = s_m, s1 = s_z, iz = 1.f / (1.f + s1), invd = 1.f / (float)D;
  const int t0 = c * kJChunk, t1 = min(t0 + kJChunk, j.N);
  for (int t = t0 + tid; t < t1; t += kJThreads) {
    const long long i = (long long)head * j.N + t;
    const float d = j.z[i] - M;
    // alpha = e / Z and 1 - alpha = (Z - e) / Z = ((1 - e) + (Z - 1)) / Z: two
    // non-negative terms, so a saturated alpha keeps its complement.
    const float a = __expf(d) * iz;
    const float om = (s1 - expm1f(d)) * iz;
    const float rho = a * om;
    j.w[i] = rho * rho * j.kappa[i] * invd;
  }
  // The refresh selection's first-digit histograms start from zero: cleared
  // here (the grid, in 16-byte stores) instead of by a launch of their own.
  if (j.hist != nullptr) {
    const long long nwg = (long long)gridDim.x * gridDim.y, wg = (long long)blockIdx.y * gridDim.x + blockIdx.x;
    uint4* h4 = reinterpret_cast<uint4*>(j.hist);
    for (long long q = wg * kJThreads + tid; q < j.hist_words / 4; q += nwg * kJThreads) h4[q] = make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats as packed bf16 high parts (round to nearest even, one
// v_cvt_pk_bf16_f32) and the packed bf16 of what each high part leaves over.
__device__ __forceinline__ void split2(float x0, float x1, unsigned& hi, unsigned& lo) {
  hi = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
  const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){r0, r1}, bf16x2));
}

// Lower 32 x 32 tiles (p, r), p >= r, of the D x D Gram matrix computed by
// each of the four waves, coded p * (D / 32) + r (-1: none).  Tiles of a wave
// share their column r where possible, so that its B operands are read once.
template <int D>
__device__ constexpr int gram_tile(int wave, int q) {
  if constexpr (D == 128) {
    constexpr int t[4][3] = {{4, 8, 12}, {5, 9, 13}, {10, 14, 0}, {15, -1, -1}};
    return t[wave][q];
  } else {
    constexpr int t[4][3] = {{0, -1, -1}, {2, -1, -1}, {3, -1, -1}, {-1, -1, -1}};
    return t[wave][q];
  }
}

template <int D>
struct GramShape {
  static constexpr int TS = D == 128 ? 64 : 128;  // tokens per step: 512 units of 2 tokens x 8 features
  static_assert(TS / 2 * D / 8 == 512, "one unit per staging thread");
  static constexpr int RS = TS + 8;               // LDS row stride (elements)
  static constexpr int FG = D / 8;                // feature groups
  static constexpr int ARR = D * RS;              // one operand array
};

// One step's share of a staging thread: 2 tokens x 8 features of U and the
// 2 weights.
template <int D>
__device__ __forceinline__ void gram_load(const JacapArgs& j, const __bf16* __restrict__ U, int head, int t, int t1,
                                          int fg, uint4 (&d)[2], float (&w)[2]) {
  // Tokens past the slice load its last row (their weight is zeroed when
  // staged), so that no load sits in a branch.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tc = max(min(t + i, t1 - 1), 0);
    d[i] = *reinterpret_cast<const uint4*>(U + ((long long)head * j.N + tc) * D + fg * 8);
    w[i] = j.w[(long long)head * j.N + tc];
  }
}

// Writes the share into the operand arrays (feature-major: a row per feature,
// the step's tokens along it): u^T exactly, and (w u)^T as bf16 high + low.
template <int D>
__device__ __forceinline__ void gram_stage(__bf16* buf, int fg, int tg, const uint4 (&d)[2], const float (&wl)[2],
                                           int valid) {
  using S = GramShape<D>;
  float w[2];  // tokens past the slice weigh 0: every product has a (w u) factor, so they add nothing
#pragma unroll
  for (int i = 0; i < 2; ++i) w[i] = i < valid ? wl[i] : 0.f;
  __bf16* ut = buf;
  __bf16* bh = buf + S::ARR;
  __bf16* bl = buf + 2 * S::ARR;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned x[2] = {(&d[0].x)[q], (&d[1].x)[q]};
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // feature 8 fg + 2 q + h: the low (h = 0) or high bf16 of each word
      const int o = (fg * 8 + 2 * q + h) * S::RS + tg * 2;
      const unsigned u = h == 0 ? (x[0] & 0xFFFFu) | (x[1] << 16) : (x[0] >> 16) | (x[1] & 0xFFFF0000u);
      const float v0 = __uint_as_float(h == 0 ? x[0] << 16 : x[0] & 0xFFFF0000u) * w[0];
      const float v1 = __uint_as_float(h == 0 ? x[1] << 16 : x[1] & 0xFFFF0000u) * w[1];
      unsigned hi, lo;
      split2(v0, v1, hi, lo);
      *reinterpret_cast<unsigned*>(ut + o) = u;
      *reinterpret_cast<unsigned*>(bh + o) = hi;
      *reinterpret_cast<unsigned*>(bl + o) = lo;
    }
  }
}

template <int D, int WV>
__device__ __forceinline__ void gram_mfma(const __bf16* cur, int n, int g, f32x16 (&acc)[3]) {
  using S = GramShape<D>;
  constexpr int NT = D / 32;
#pragma unroll
  for (int k0 = 0; k0 < S::TS; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int tile = gram_tile<D>(WV, q);
      if (tile >= 0) {
        const int p = tile / NT, r = tile % NT;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + (p * 32 + n) * S::RS + k0 + 8 * g);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(cur + S::ARR + (r * 32 + n) * S::RS + k0 + 8 * g);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(cur + 2 * S::ARR + (r * 32 + n) * S::RS + k0 + 8 * g);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc[q], 0, 0, 0);
      }
    }
  }
}

// Part of sum_i w_i u_i u_i^T over tokens [slice * per, (slice + 1) * per) of
// the head, into gpart[head][slice][D][D] (lower 32 x 32 tiles only).  Each
// MFMA pair multiplies u^T (exact bf16) by the high and the low bf16 part of
// (w u): products correct to about 2^-17 relative, fp32 accumulation.
// Waves 0-3 multiply; waves 4-11 load and stage (16-byte loads of token rows,
// transposed in registers, into one of two LDS buffers) the next step while
// the others multiply the current one, so the staging arithmetic runs beside
// the MFMAs on the same SIMDs and a step needs one barrier.  The loads run
// kPre steps ahead of the staging (a ring of register sets).
constexpr int kPre = 5;
constexpr int kGramThreads = 768;  // waves 0-3 multiply, waves 4-11 stage
template <int D, int WV>  // WV < 4: the multiplying wave of that tile set; WV == 4: a staging wave
__device__ __forceinline__ void gram_body(const JacapArgs& j, const __bf16* __restrict__ U, __bf16* lds) {
  using S = GramShape<D>;
  constexpr bool kStage = WV == 4;
  const int head = blockIdx.y, slice = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, n = lane & 31, g = lane >> 5;
  // A staging wave stages whole feature rows: QW lanes take consecutive token
  // pairs of one feature group, so that its 4-byte LDS writes cover
  // consecutive banks (the two rows of a write fall on disjoint halves).
  constexpr int QW = S::TS / 2;
  const int ts = tid - 256;
  const int fg = (ts >> 6) * (64 / QW) + lane / QW, tg = lane % QW;
  const int per = (j.N + j.slices - 1) / j.slices;
  const int t0 = min(slice * per, j.N), t1 = min(t0 + per, j.N);
  const int steps = (t1 - t0 + S::TS - 1) / S::TS;
  constexpr int R = kPre + 1;
  static_assert(R % 2 == 0, "the ring period must be even");
  f32x16 acc[3];
  uint4 d[R][2];
  float w[R][2];
  if constexpr (kStage) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) gram_load<D>(j, U, head, t0 + u * S::TS + tg * 2, t1, fg, d[u], w[u]);
    if (steps > 0) gram_stage<D>(lds, fg, tg, d[0], w[0], t1 - (t0 + tg * 2));
  } else {
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[q] = f32x16{};
  }
  __syncthreads();
  // Step st multiplies buffer st & 1; the staging waves load step st + kPre
  // into register set (st + kPre) % R and stage step st + 1 from set
  // (st + 1) % R into the other buffer.  Loads and staging past the last step
  // are harmless (rows clamped to the slice, buffers never multiplied).
  // Whole blocks of R steps run without a branch, so that the compiler's wait
  // counts see the full depth of the load ring; the remaining steps follow
  // with a test each.
  auto step = [&](int st, auto uc) {
    constexpr int u = decltype(uc)::value;
    if constexpr (kStage) {
      gram_load<D>(j, U, head, t0 + (st + kPre) * S::TS + tg * 2, t1, fg, d[(u + kPre) % R], w[(u + kPre) % R]);
      gram_stage<D>(lds + ((u + 1) & 1) * 3 * S::ARR, fg, tg, d[(u + 1) % R], w[(u + 1) % R],
                    t1 - (t0 + (st + 1) * S::TS + tg * 2));
    } else {
      gram_mfma<D, WV>(lds + (u & 1) * 3 * S::ARR, n, g, acc);
    }
    __syncthreads();
  };
  const int full = steps / R * R;
  for (int s0 = 0; s0 < full; s0 += R) {
    step(s0 + 0, std::integral_constant<int, 0>{});
    step(s0 + 1, std::integral_constant<int, 1>{});
    step(s0 + 2, std::integral_constant<int, 2>{});
    step(s0 + 3, std::integral_constant<int, 3>{});
    step(s0 + 4, std::integral_constant<int, 4>{});
    step(s0 + 5, std::integral_constant<int, 5>{});
  }
  static_assert(R == 6, "the unrolled blocks above and the tail below assume a ring of six");
  if (full + 0 < steps) step(full + 0, std::integral_constant<int, 0>{});
  if (full + 1 < steps) step(full + 1, std::integral_constant<int, 1>{});
  if (full + 2 < steps) step(full + 2, std::integral_constant<int, 2>{});
  if (full + 3 < steps) step(full + 3, std::integral_constant<int, 3>{});
  if (full + 4 < steps) step(full + 4, std::integral_constant<int, 4>{});
  if constexpr (!kStage) {
    float* out = j.gpart + ((long long)head * j.slices + slice) * D * D;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      constexpr int NT = D / 32;
      const int tile = gram_tile<D>(WV, q);
      if (tile >= 0) {
        const int p = tile / NT, r = tile % NT;
#pragma unroll
        for (int e = 0; e < 16; ++e) out[(p * 32 + acc_row(e, g)) * D + r * 32 + n] = acc[q][e];
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kGramThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void jacap_gram_kernel(const JacapArgs j, const __bf16* __restrict__ U) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * 3 * GramShape<D>::ARR];
  switch (threadIdx.x >> 6) {  // every wave runs the same steps and barriers
    case 0: gram_body<D, 0>(j, U, lds); break;
    case 1: gram_body<D, 1>(j, U, lds); break;
    case 2: gram_body<D, 2>(j, U, lds); break;
    case 3: gram_body<D, 3>(j, U, lds); break;
    default: gram_body<D, 4>(j, U, lds); break;
  }
}

// The slices' parts of each head summed in slice order into slice 0 (lower
// 32 x 32 tiles only: the Gram kernel writes no others), so that the
// factorisation reads one D x D matrix.  Grid (kRedParts, heads); a float4
// per thread and pass.
constexpr int kRedParts = 16;
template <int D>
__global__ __launch_bounds__(kJThreads) void jacap_reduce_kernel(const JacapArgs j) {
  constexpr int G4 = D * D / 4 / kRedParts;  // float4 groups per workgroup
  float4* g = reinterpret_cast<float4*>(j.gpart + (long long)blockIdx.y * j.slices * D * D);
  for (int i = threadIdx.x; i < G4; i += kJThreads) {
    const int e4 = blockIdx.x * G4 + i, r = (4 * e4) / D, c = (4 * e4) % D;
    if (r / 32 < c / 32) continue;  // upper tile
    float4 v = g[e4];
    for (int q = 1; q < j.slices; ++q) {
      const float4 x = g[(long long)q * D * D / 4 + e4];
      v.x += x.x;
      v.y += x.y;
      v.z += x.z;
      v.w += x.w;
    }
    g[e4] = v;
  }
}

// A = I + the slices' parts, then A = L L^T (Cholesky, fp32) and M = L^{-1},
// blocked by 8-column panels with A, L and M in LDS (row stride D + 4 floats:
// 16-byte aligned rows, consecutive rows four banks apart).  Lanes 0-7 of
// wave 0 (a row each) factor and invert an 8 x 8 diagonal block.  Per panel
// p, two barriers:
//   1. the rows below are solved against the inverse of diagonal block p (a
//      row per thread), and block row p of M is that inverse times the
//      running block row;
//   2. waves 1-3 take the rank-8 update of the trailing lower triangle in
//      4 x 4 units, and the rows of M below (L M = I right-looking:
//      X_i -= L_ip M_p); wave 0 meanwhile updates diagonal block p + 1 (the
//      first three units) and factors it (look-ahead).
// Only lower triangles are computed; the upper parts hold zeros.  M is stored
// as bf16 hi and lo.
template <int D>
__global__ __launch_bounds__(kJThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void jacap_factor_kernel(const JacapArgs j) {
  constexpr int S = D + 4;
  constexpr int P = D / 8;
  __shared__ __attribute__((aligned(16))) float a[D * S];
  __shared__ __attribute__((aligned(16))) float m[D * S];
  __shared__ __attribute__((aligned(16))) float li[64];   // inverse of the current diagonal block
  __shared__ __attribute__((aligned(16))) float tt[8 * D];  // block row p of M
  const int head = blockIdx.x, tid = threadIdx.x;
  const float* gp = j.gpart + (long long)head * j.slices * D * D;
  // A = I + the summed Gram matrix (its lower 32 x 32 tiles are written; only
  // the lower triangle is read).
  {
    constexpr int E4 = D * D / 4 / kJThreads;  // float4 groups per thread: g = tid + kJThreads * t
    float4 v[E4];
#pragma unroll
    for (int t = 0; t < E4; ++t) {
      const int e = 4 * (tid + kJThreads * t), r = e / D, c = e % D;
      v[t] = make_float4(r == c ? 1.f : 0.f, r == c + 1 ? 1.f : 0.f, r == c + 2 ? 1.f : 0.f, r == c + 3 ? 1.f : 0.f);
    }
    const float4* g4 = reinterpret_cast<const float4*>(gp);  // slice 0 holds the sum of the slices
#pragma unroll
    for (int t = 0; t < E4; ++t) {
      const float4 x = g4[tid + kJThreads * t];
      v[t].x += x.x;
      v[t].y += x.y;
      v[t].z += x.z;
      v[t].w += x.w;
    }
#pragma unroll
    for (int t = 0; t < E4; ++t) {  // upper elements (never written by the Gram kernel) are dropped
      const int e = 4 * (tid + kJThreads * t), r = e / D, c = e % D;
      *reinterpret_cast<float4*>(a + r * S + c) =
          make_float4(c <= r ? v[t].x : 0.f, c + 1 <= r ? v[t].y : 0.f, c + 2 <= r ? v[t].z : 0.f,
                      c + 3 <= r ? v[t].w : 0.f);
      *reinterpret_cast<float4*>(m + r * S + c) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();
  bool bad = false;  // a pivot that is not finite and positive (lanes 0-7 of wave 0)
  // The diagonal block of panel k0 / 8: lane i of wave 0 holds row i;
  // Cholesky and inverse (written to a, m and li).
  auto diag = [&](int k0) {
      if (tid < 8) {  // the diagonal block: lane i of wave 0 holds row i; Cholesky and inverse
        float x[8], y[8];
        {
          const float4 u0 = *reinterpret_cast<const float4*>(a + (k0 + tid) * S + k0);
          const float4 u1 = *reinterpret_cast<const float4*>(a + (k0 + tid) * S + k0 + 4);
          x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
          x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
        }
        float rsi = 0.f;  // 1 / L[i][i] of this lane's row
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(x[c]), c));
          bad |= !(d > 0.f && isfinite(d));
          const float dd = fmaxf(d, 1e-30f);
          const float rs = __builtin_amdgcn_rsqf(dd);
          if (tid == c) {
            x[c] = dd * rs;
            rsi = rs;
          } else if (tid > c) {
            x[c] *= rs;
          }
          // Column c of L below the diagonal, broadcast: row q's entry from lane q.
#pragma unroll
          for (int q = c + 1; q < 8; ++q) {
            const float lq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(x[c]), q));
            if (tid >= q) x[q] = fmaf(-x[c], lq, x[q]);
          }
        }
        // Row i of inv(L): y[q] = -rs_i sum_{k=q}^{i-1} L[i][k] y_k[q], rows in order
        // (row k's entries broadcast from lane k once it is final).
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (tid == k) {
#pragma unroll
            for (int q = 0; q < 8; ++q) y[q] = q < k ? -y[q] * rsi : (q == k ? rsi : 0.f);
          }
#pragma unroll
          for (int q = 0; q <= k; ++q) {
            const float yk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(y[q]), k));
            if (tid > k) y[q] = fmaf(x[k], yk, y[q]);  // accumulates sum_k L[i][k] y_k[q]
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = q <= tid ? x[q] : 0.f;
        float* ar = a + (k0 + tid) * S + k0;
        float* mr = m + (k0 + tid) * S + k0;
        *reinterpret_cast<float4*>(ar) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(ar + 4) = make_float4(x[4], x[5], x[6], x[7]);
        *reinterpret_cast<float4*>(mr) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(mr + 4) = make_float4(y[4], y[5], y[6], y[7]);
        *reinterpret_cast<float4*>(li + tid * 8) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(li + tid * 8 + 4) = make_float4(y[4], y[5], y[6], y[7]);
      }
  };
  // One 4 x 4 unit (rb >= cb) of the trailing lower triangle of panel k0 / 8.
  auto trail = [&](int k0, int q) {
    int rb = (int)((sqrtf(8.f * q + 1.f) - 1.f) * 0.5f);
    while (rb * (rb + 1) / 2 > q) --rb;
    while ((rb + 1) * (rb + 2) / 2 <= q) ++rb;
    const int cb = q - rb * (rb + 1) / 2;
    const int r0 = k0 + 8 + 4 * rb, c0 = k0 + 8 + 4 * cb;
    float lr[4][8], lc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 u0 = *reinterpret_cast<const float4*>(a + (r0 + i) * S + k0);
      const float4 u1 = *reinterpret_cast<const float4*>(a + (r0 + i) * S + k0 + 4);
      const float4 w0 = *reinterpret_cast<const float4*>(a + (c0 + i) * S + k0);
      const float4 w1 = *reinterpret_cast<const float4*>(a + (c0 + i) * S + k0 + 4);
      lr[i][0] = u0.x; lr[i][1] = u0.y; lr[i][2] = u0.z; lr[i][3] = u0.w;
      lr[i][4] = u1.x; lr[i][5] = u1.y; lr[i][6] = u1.z; lr[i][7] = u1.w;
      lc[i][0] = w0.x; lc[i][1] = w0.y; lc[i][2] = w0.z; lc[i][3] = w0.w;
      lc[i][4] = w1.x; lc[i][5] = w1.y; lc[i][6] = w1.z; lc[i][7] = w1.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* dst = a + (r0 + i) * S + c0;
      float4 v = *reinterpret_cast<const float4*>(dst);
      float o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
#pragma unroll
        for (int k = 0; k < 8; ++k) o[q2] = fmaf(-lr[i][k], lc[q2][k], o[q2]);
      if (rb == cb) {  // keep the upper part of a diagonal unit at zero
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) o[q2] = q2 <= i ? o[q2] : 0.f;
      }
      *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
    }
  
  };
  diag(0);
  __syncthreads();
  for (int p = 0; p < P; ++p) {
    const int k0 = p * 8;
    // Rows below: L[r][k0 + q] = sum_c A[r][k0 + c] inv(L_pp)[q][c].
    const int r = k0 + 8 + tid;
    if (r < D) {
      float* row = a + r * S + k0;
      const float4 v0 = *reinterpret_cast<const float4*>(row), v1 = *reinterpret_cast<const float4*>(row + 4);
      const float y[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float t = 0.f;
#pragma unroll
        for (int c = 0; c <= q; ++c) t = fmaf(y[c], li[q * 8 + c], t);
        o[q] = t;
      }
      *reinterpret_cast<float4*>(row) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(row + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
    // Block row p of M: inv(L_pp) times the running block row (rows k0 ..
    // k0 + 7 of m, which hold minus the earlier panels' contributions left of
    // the diagonal), into tt; the diagonal block is inv(L_pp) itself.
    for (int u = tid; u < 2 * k0 + 16; u += kJThreads) {
      const int ii = u % 8, c0 = (u / 8) * 4;
      float o[4] = {0.f, 0.f, 0.f, 0.f};
      if (c0 < k0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float l = li[ii * 8 + q];  // zero for q > ii
          const float4 xv = *reinterpret_cast<const float4*>(m + (k0 + q) * S + c0);
          o[0] = fmaf(l, xv.x, o[0]);
          o[1] = fmaf(l, xv.y, o[1]);
          o[2] = fmaf(l, xv.z, o[2]);
          o[3] = fmaf(l, xv.w, o[3]);
        }
      } else {
        const float4 lv = *reinterpret_cast<const float4*>(li + ii * 8 + (c0 - k0));
        o[0] = lv.x; o[1] = lv.y; o[2] = lv.z; o[3] = lv.w;
      }
      *reinterpret_cast<float4*>(tt + ii * D + c0) = make_float4(o[0], o[1], o[2], o[3]);
    }
    __syncthreads();
    // Wave 0 updates the next diagonal block (the first three trailing
    // units) and factors it, while waves 1-3 take the other trailing units
    // and the rows of M below.
    const int T = (D - k0 - 8) / 4;
    const int ntri = T * (T + 1) / 2;
    if (tid < 64) {
      if (p + 1 < P) {
        if (tid < 3) trail(k0, tid);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        diag(k0 + 8);
      }
    } else {
      const int t3 = tid - 64;
      for (int q = 3 + t3; q < ntri; q += 192) trail(k0, q);
      // Rows below of the running M: X[i][c] -= sum_k L[i][k0 + k] M_p[k][c] for
      // c < k0 + 8 (4 x 4 units); block row p of M moves from tt into m.
      {
        const int RQ = (D - k0 - 8) / 4, CQ = (k0 + 8) / 4;
        // The trailing units and these share one index space: index i of
        // thread t3 is t3 + 192 k, trailing unit 3 + i below ntri - 3, unit
        // i - (ntri - 3) here above it.
        for (int u = ((t3 - (ntri - 3)) % 192 + 192) % 192; u < RQ * CQ; u += 192) {
          const int r0 = k0 + 8 + 4 * (u / CQ), c0 = 4 * (u % CQ);
          float4 tv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) tv[k] = *reinterpret_cast<const float4*>(tt + k * D + c0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 l0 = *reinterpret_cast<const float4*>(a + (r0 + i) * S + k0);
            const float4 l1 = *reinterpret_cast<const float4*>(a + (r0 + i) * S + k0 + 4);
            const float l[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            float* dst = m + (r0 + i) * S + c0;
            float4 x = *reinterpret_cast<const float4*>(dst);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              x.x = fmaf(-l[k], tv[k].x, x.x);
              x.y = fmaf(-l[k], tv[k].y, x.y);
              x.z = fmaf(-l[k], tv[k].z, x.z);
              x.w = fmaf(-l[k], tv[k].w, x.w);
            }
            *reinterpret_cast<float4*>(dst) = x;
          }
        }
        for (int u = t3; u < 2 * k0; u += 192) {
          const int ii = u % 8, c0 = (u / 8) * 4;
          *reinterpret_cast<float4*>(m + (k0 + ii) * S + c0) = *reinterpret_cast<const float4*>(tt + ii * D + c0);
        }
      }
    }
    __syncthreads();
  }
  if (bad) raise_error(j.err, kErrNonFinite);
  __bf16* mh = j.minv + (long long)head * 2 * D * D;
  __bf16* ml = mh + D * D;
  for (int e = tid; e < D * D; e += kJThreads) {
    __bf16 hi, lo;
    split_bf16(m[(e / D) * S + e % D], hi, lo);
    mh[e] = hi;
    ml[e] = lo;
  }
}

// r_t = w_t |M u_t|^2 for the chunk's tokens: Y = M U^T on MFMA, a wave
// taking 64 tokens at a time as two 32-token column groups that share every
// M operand read; row tile p of M (lower triangular) only needs the k-steps
// up to its diagonal.  M's high and low parts multiply the exact bf16 u; each
// lane sums the squares of its rows of Y and the two halves of the wave hold
// the other rows of the same tokens.  M (hi, lo) is staged in LDS.
template <int D>
__global__ __launch_bounds__(kJThreads) void jacap_leverage_kernel(const JacapArgs j, const __bf16* __restrict__ U) {
  constexpr int RS = D + 8;
  constexpr int KS = D / 16;  // k-steps of a full row
  __shared__ __attribute__((aligned(16))) __bf16 mh[D * RS], ml[D * RS];
  const int head = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  const __bf16* gm = j.minv + (long long)head * 2 * D * D;
  for (int e = tid; e < D * D / 8; e += kJThreads) {
    const int r = e / (D / 8), c8 = e % (D / 8);
    *reinterpret_cast<uint4*>(&mh[r * RS + c8 * 8]) = *reinterpret_cast<const uint4*>(&gm[r * D + c8 * 8]);
    *reinterpret_cast<uint4*>(&ml[r * RS + c8 * 8]) = *reinterpret_cast<const uint4*>(&gm[D * D + r * D + c8 * 8]);
  }
  __syncthreads();
  const int t0 = c * kJChunk, t1 = min(t0 + kJChunk, j.N);
  for (int b0 = t0 + wave * 64; b0 < t1; b0 += 4 * 64) {
    // M's operands are read from LDS in every pass (kept out of registers
    // across passes, which leaves room for a second workgroup per CU).
    asm volatile("" ::: "memory");
    bf16x8 ub[2][KS];  // the two groups' u, loaded once for all row tiles
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      const int t = min(b0 + cg * 32 + n, t1 - 1);  // columns past the chunk repeat its last token (not written)
      const __bf16* ur = U + ((long long)head * j.N + t) * D;
#pragma unroll
      for (int k = 0; k < KS; ++k) ub[cg][k] = *reinterpret_cast<const bf16x8*>(ur + 16 * k + 8 * g);
    }
    float sq[2] = {0.f, 0.f};
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int k = 0; k < 2 * (p + 1); ++k) {  // M[row][col] = 0 for col > row
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&mh[(p * 32 + n) * RS + 16 * k + 8 * g]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&ml[(p * 32 + n) * RS + 16 * k + 8 * g]);
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
          acc[cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, ub[cg][k], acc[cg], 0, 0, 0);
          acc[cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, ub[cg][k], acc[cg], 0, 0, 0);
        }
      }
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int e = 0; e < 16; ++e) sq[cg] = fmaf(acc[cg][e], acc[cg][e], sq[cg]);
    }
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      const float other = __shfl_xor(sq[cg], 32);
      const float tot = g == 0 ? sq[cg] + other : other + sq[cg];
      const int t = b0 + cg * 32 + n;
      if (g == 0 && t < t1) {
        const long long i = (long long)head * j.N + t;
        j.r[i] = j.w[i] * tot;
      }
    }
  }
}

template <int D>
hipError_t launch_all(const JacapArgs& j, const __bf16* K, const __bf16* U, hipStream_t st,
                      const std::function<hipError_t(const char*, const std::function<hipError_t()>&)>& timed) {
  const dim3 chunks(j.nch, j.heads);
  hipError_t e = timed("jacap_logits", [&] {
    hipLaunchKernelGGL((jacap_logits_kernel<D>), chunks, dim3(kJThreads), 0, st, j, K);
    return hipGetLastError();
  });
  if (e == hipSuccess)
    e = timed("jacap_weights", [&] {
      hipLaunchKernelGGL(jacap_weights_kernel, chunks, dim3(kJThreads), 0, st, j, D);
      return hipGetLastError();
    });
  if (e == hipSuccess)
    e = timed("jacap_gram", [&] {
      hipLaunchKernelGGL((jacap_gram_kernel<D>), dim3(j.slices, j.heads), dim3(kGramThreads), 0, st, j, U);
      return hipGetLastError();
    });
  if (e == hipSuccess && j.slices > 1)
    e = timed("jacap_reduce", [&] {
      hipLaunchKernelGGL((jacap_reduce_kernel<D>), dim3(kRedParts, j.heads), dim3(kJThreads), 0, st, j);
      return hipGetLastError();
    });
  if (e == hipSuccess)
    e = timed("jacap_factor", [&] {
      hipLaunchKernelGGL((jacap_factor_kernel<D>), dim3(j.heads), dim3(kJThreads), 0, st, j);
      return hipGetLastError();
    });
  if (e == hipSuccess)
    e = timed("jacap_leverage", [&] {
      hipLaunchKernelGGL((jacap_leverage_kernel<D>), chunks, dim3(kJThreads), 0, st, j, U);
      return hipGetLastError();
    });
  return e;
}

}  // namespace

int jacap_chunks(int N) { return (N + kJChunk - 1) / kJChunk; }
// Gram slices per head: about one workgroup per CU over all heads, each slice
// at least 512 tokens, at most 32 slices.
int jacap_slices(int N, int heads) {
  const int fill = (256 + heads - 1) / heads;
  return std::max(1, std::min({32, fill, (N + 511) / 512}));
}

hipError_t launch_jacap_scores(const JacapArgs& j, int D, const void* K, const void* U, hipStream_t st,
                               const std::function<hipError_t(const char*, const std::function<hipError_t()>&)>& timed) {
  if (D == 128) return launch_all<128>(j, (const __bf16*)K, (const __bf16*)U, st, timed);
  if (D == 64) return launch_all<64>(j, (const __bf16*)K, (const __bf16*)U, st, timed);
  return hipErrorNotSupported;
}

}  // namespace kvsel
