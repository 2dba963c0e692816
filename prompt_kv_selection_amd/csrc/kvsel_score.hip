// Window scoring kernels for gfx950: logits of the W window queries against
// the whole prompt on MFMA, causal row statistics, and prefix votes.
//
// Method (web page "SnapKV: selecting the KV cache for long prompts with an
// observation window", section "votes must come from the causal softmax over
// the full prompt"): for window row i (query position P + i) and prompt
// position j, l[i][j] = q_i . k_j / sqrt(D); row i sees j <= P + i, and its
// softmax denominator covers every visible prefix and window position.  The
// vote of prefix position j < P is the sum over window rows of the softmax
// probability.
//
// Tiling.  One MFMA tile is 32 window rows x 32 prompt positions.  Qwin is the
// A operand (rows) and stays in VGPRs for the whole workgroup; a tile of 32 K
// rows is the B operand, loaded straight from HBM, each lane taking 16 bytes
// per k-step from one K row.  In the 32x32 accumulator a lane owns one
// position (lane % 32) and 16 of the 32 window rows, so
//   * the per-row max / sum of exponentials run inside the lane across the
//     positions it visits, then across the 32 lanes of its half,
//   * the vote of a position is a sum over the lane's 16 rows plus the 16 rows
//     of lane ^ 32.
// Logits are kept in base 2: x = (q . k) * log2(e) / sqrt(D), so every
// exponential is one v_exp_f32.
//
// Two kernels: window_stats writes per-chunk (max, sum) partials of every
// window row; window_votes merges the partials of its head, recomputes the
// logits of its chunk and writes the votes.  Summation orders are fixed per
// position (rows in a fixed order), so equal key rows get bit-equal votes.

#include <math.h>

#include "kvsel_internal.h"

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;   // finite "no position seen yet" max
constexpr float kLn2 = 0.693147180559945309f;

// Window row held in accumulator register r by lane half g (32x32 MFMA
// output layout: lane l holds column l % 32, rows 8*(r/4) + 4*(l/32) + r%4).
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Operand registers of one 32-row tile (a Qwin row block or 32 K rows).
template <typename T, int D>
struct Operands;

template <int D>
struct Operands<__bf16, D> {
  static constexpr int NS = D / 16;  // k-steps of v_mfma_f32_32x32x16_bf16
  bf16x8 v[NS];
  // Lane half g takes elements [16 s + 8 g, 16 s + 8 g + 8) of the row.
  __device__ __forceinline__ void load(const __bf16* __restrict__ row, int g) {
    const uint4* p = reinterpret_cast<const uint4*>(row);
#pragma unroll
    for (int s = 0; s < NS; ++s) v[s] = __builtin_bit_cast(bf16x8, p[2 * s + g]);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < NS; ++s) v[s] = bf16x8{};
  }
};

template <int D>
struct Operands<float, D> {
  static constexpr int NQ = D / 8;  // 4 k-steps of v_mfma_f32_32x32x2_f32 per float4
  f32x4 v[NQ];
  // Lane half g takes elements [8 q + 4 g, 8 q + 4 g + 4) of the row; k-step
  // (q, e) pairs element 8q+e (half 0) with 8q+4+e (half 1).
  __device__ __forceinline__ void load(const float* __restrict__ row, int g) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row);
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[q] = p[2 * q + g];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[q] = f32x4{};
  }
};

template <int D>
__device__ __forceinline__ f32x16 tile_dot(const Operands<__bf16, D>& a, const Operands<__bf16, D>& b) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < Operands<__bf16, D>::NS; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v[s], b.v[s], acc, 0, 0, 0);
  return acc;
}

template <int D>
__device__ __forceinline__ f32x16 tile_dot(const Operands<float, D>& a, const Operands<float, D>& b) {
  f32x16 acc = {};
#pragma unroll
  for (int q = 0; q < Operands<float, D>::NQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[q][e], b.v[q][e], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge (m2, z) with (mo, zo): running maximum in base 2 and the sum of
// exponentials rescaled to it.
__device__ __forceinline__ void lse_merge(float& m, float& z, float mo, float zo) {
  const float mn = fmaxf(m, mo);
  z = z * exp2_fast(m - mn) + zo * exp2_fast(mo - mn);
  m = mn;
}

struct Where {
  int e, h, hl, c;
};

__device__ __forceinline__ Where locate_chunk(const Launch& a) {
  Where w;
  w.e = find_seg<kFieldItem>(a, blockIdx.x);
  const Seg& s = a.seg[w.e];
  const int local = blockIdx.x - s.item0;
  w.hl = local / s.nch;
  w.c = local - w.hl * s.nch;
  w.h = s.h0 + w.hl;
  return w;
}

template <typename T, int D, int RB>
__device__ __forceinline__ void load_queries(const Launch& a, const Seg& s, int h, const T* __restrict__ Q,
                                             int n, int g, Operands<T, D> (&qa)[RB]) {
  const T* q = Q + ((long long)s.b * a.heads + h) * (long long)a.W * D;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rb * 32 + n;
    if (row < a.W)
      qa[rb].load(q + (long long)row * D, g);
    else
      qa[rb].zero();
  }
}

// Per-chunk row statistics.  Workgroup = kWaves waves over kChunk positions
// of one (sequence, head); writes, for every window row i < W, the base-2
// maximum of the visible logits in the chunk and the sum of exp2(x - max).
template <typename T, int D, int RB>
__global__ __launch_bounds__(kWaves * 64) void window_stats_kernel(const Launch a, const T* __restrict__ Q,
                                                                  const T* __restrict__ K,
                                                                  float* __restrict__ part_m,
                                                                  float* __restrict__ part_z) {
  const Where w = locate_chunk(a);
  const Seg& s = a.seg[w.e];
  const int L = s.L, W = a.W, P = L - W;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, g = lane >> 5;

  Operands<T, D> qa[RB];
  load_queries<T, D, RB>(a, s, w.h, Q, n, g, qa);
  const T* kb = K + s.kv_off + (long long)w.h * L * D;

  float m[RB][16], z[RB][16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      m[rb][r] = kNegBig;
      z[rb][r] = 0.f;
    }

  const int p_begin = w.c * kChunk + wave * (kWaveTiles * 32);
  for (int t = 0; t < kWaveTiles; ++t) {
    const int p0 = p_begin + t * 32;
    if (p0 >= L) break;
    const int j = p0 + n;
    Operands<T, D> kt;
    kt.load(kb + (long long)min(j, L - 1) * D, g);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x16 acc = tile_dot<D>(qa[rb], kt);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = rb * 32 + acc_row(r, g);
        const bool visible = (j < L) && (i < W) && (j <= P + i);
        const float x = visible ? acc[r] * a.scale2 : -INFINITY;
        const float mn = fmaxf(m[rb][r], x);
        z[rb][r] = z[rb][r] * exp2_fast(m[rb][r] - mn) + exp2_fast(x - mn);
        m[rb][r] = mn;
      }
    }
  }

  // Across the 32 lanes of each half (same rows, different positions).
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) {
        const float mo = __shfl_xor(m[rb][r], off);
        const float zo = __shfl_xor(z[rb][r], off);
        lse_merge(m[rb][r], z[rb][r], mo, zo);
      }

  __shared__ float sm[kWaves][RB * 32], sz[kWaves][RB * 32];
  if (n == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = rb * 32 + acc_row(r, g);
        sm[wave][i] = m[rb][r];
        sz[wave][i] = z[rb][r];
      }
  }
  __syncthreads();
  if ((int)threadIdx.x < W) {
    const int i = threadIdx.x;
    float mm = sm[0][i], zz = sz[0][i];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) lse_merge(mm, zz, sm[v][i], sz[v][i]);
    const long long slot = (s.part_base + (long long)w.h * s.nch + w.c) * W + i;
    part_m[slot] = mm;
    part_z[slot] = zz;
  }
}

// Votes of the prefix positions of one chunk.  Merges the head's partial row
// statistics, recomputes the chunk's logits and sums the softmax
// probabilities over the window rows.
template <typename T, int D, int RB>
__global__ __launch_bounds__(kWaves * 64) void window_votes_kernel(
    const Launch a, const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ part_m,
    const float* __restrict__ part_z, float* __restrict__ votes, float* __restrict__ row_stats) {
  const Where w = locate_chunk(a);
  const Seg& s = a.seg[w.e];
  const int L = s.L, W = a.W, P = L - W;
  if (w.c * kChunk >= P) return;  // chunk holds window positions only
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, g = lane >> 5;

  __shared__ float s_m[RB * 32], s_iz[RB * 32];
  if ((int)threadIdx.x < RB * 32) {
    const int i = threadIdx.x;
    // Rows past W: zero queries give x = 0, so (m, 1/Z) = (0, 0) drops them.
    float mm = 0.f, iz = 0.f;
    if (i < W) {
      const long long base = (s.part_base + (long long)w.h * s.nch) * W + i;
      mm = kNegBig;
      for (int c = 0; c < s.nch; ++c) mm = fmaxf(mm, part_m[base + (long long)c * W]);
      float zz = 0.f;
      for (int c = 0; c < s.nch; ++c) {
        const long long k = base + (long long)c * W;
        zz += part_z[k] * exp2_fast(part_m[k] - mm);
      }
      iz = 1.f / zz;
      if (row_stats != nullptr && w.c == 0) {
        float* rs = row_stats + (((long long)s.b * a.heads + w.h) * W + i) * 2;
        rs[0] = mm * kLn2;
        rs[1] = zz;
      }
    }
    s_m[i] = mm;
    s_iz[i] = iz;
  }
  __syncthreads();

  Operands<T, D> qa[RB];
  load_queries<T, D, RB>(a, s, w.h, Q, n, g, qa);
  float mr[RB][16], izr[RB][16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = rb * 32 + acc_row(r, g);
      mr[rb][r] = s_m[i];
      izr[rb][r] = s_iz[i];
    }

  const T* kb = K + s.kv_off + (long long)w.h * L * D;
  float* vout = votes + s.vote_off + (long long)w.h * s.vote_ld;
  const int p_begin = w.c * kChunk + wave * (kWaveTiles * 32);
  for (int t = 0; t < kWaveTiles; ++t) {
    const int p0 = p_begin + t * 32;
    if (p0 >= P) break;
    const int j = p0 + n;
    Operands<T, D> kt;
    kt.load(kb + (long long)min(j, L - 1) * D, g);
    float tot = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x16 acc = tile_dot<D>(qa[rb], kt);
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part += exp2_fast(acc[r] * a.scale2 - mr[rb][r]) * izr[rb][r];
      tot += part;
    }
    const float other = __shfl_xor(tot, 32);
    // Same expression for every position: (half 0 rows) + (half 1 rows).
    const float v = g == 0 ? tot + other : other + tot;
    if (g == 0 && j < P) vout[j] = v;
  }
}

template <typename T, int D, int RB>
static hipError_t stats_t(const Launch& a, int items, const void* Q, const void* K, float* pm, float* pz,
                          hipStream_t st) {
  hipLaunchKernelGGL((window_stats_kernel<T, D, RB>), dim3(items), dim3(kWaves * 64), 0, st, a,
                     (const T*)Q, (const T*)K, pm, pz);
  return hipGetLastError();
}

template <typename T, int D, int RB>
static hipError_t votes_t(const Launch& a, int items, const void* Q, const void* K, const float* pm,
                          const float* pz, float* votes, float* rs, hipStream_t st) {
  hipLaunchKernelGGL((window_votes_kernel<T, D, RB>), dim3(items), dim3(kWaves * 64), 0, st, a,
                     (const T*)Q, (const T*)K, pm, pz, votes, rs);
  return hipGetLastError();
}

#define KVSEL_DISPATCH(FN, ...)                                                              \
  do {                                                                                       \
    const int rb = (a.W + 31) / 32;                                                          \
    if (dtype == 1) {                                                                        \
      if (a.D == 128) {                                                                      \
        if (rb == 1) return FN<__bf16, 128, 1>(__VA_ARGS__);                                 \
        if (rb == 2) return FN<__bf16, 128, 2>(__VA_ARGS__);                                 \
        if (rb == 3) return FN<__bf16, 128, 3>(__VA_ARGS__);                                 \
        return FN<__bf16, 128, 4>(__VA_ARGS__);                                              \
      }                                                                                      \
      if (rb == 1) return FN<__bf16, 64, 1>(__VA_ARGS__);                                    \
      if (rb == 2) return FN<__bf16, 64, 2>(__VA_ARGS__);                                    \
      if (rb == 3) return FN<__bf16, 64, 3>(__VA_ARGS__);                                    \
      return FN<__bf16, 64, 4>(__VA_ARGS__);                                                 \
    }                                                                                        \
    if (a.D == 128) {                                                                        \
      if (rb == 1) return FN<float, 128, 1>(__VA_ARGS__);                                    \
      if (rb == 2) return FN<float, 128, 2>(__VA_ARGS__);                                    \
      if (rb == 3) return FN<float, 128, 3>(__VA_ARGS__);                                    \
      return FN<float, 128, 4>(__VA_ARGS__);                                                 \
    }                                                                                        \
    if (rb == 1) return FN<float, 64, 1>(__VA_ARGS__);                                       \
    if (rb == 2) return FN<float, 64, 2>(__VA_ARGS__);                                       \
    if (rb == 3) return FN<float, 64, 3>(__VA_ARGS__);                                       \
    return FN<float, 64, 4>(__VA_ARGS__);                                                    \
  } while (0)

hipError_t launch_window_stats(const Launch& a, int items, int dtype, const void* Q, const void* K,
                               float* part_m, float* part_z, hipStream_t st) {
  KVSEL_DISPATCH(stats_t, a, items, Q, K, part_m, part_z, st);
}

hipError_t launch_window_votes(const Launch& a, int items, int dtype, const void* Q, const void* K,
                               const float* part_m, const float* part_z, float* votes,
                               float* row_stats, hipStream_t st) {
  KVSEL_DISPATCH(votes_t, a, items, Q, K, part_m, part_z, votes, row_stats, st);
}

}  // namespace kvsel
