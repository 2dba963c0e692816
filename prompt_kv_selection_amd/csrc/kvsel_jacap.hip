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
//   jacap_logits   per (head, chunk): z and kappa of every token (a group of
//                  D/8 lanes per token, 16-byte loads), the chunk's softmax
//                  partial (max, sum of exp).
//   jacap_weights  per (head, chunk): the head's partials merged in a fixed
//                  order, then w of every token.
//   jacap_gram     per (head, slice): the slice's part of sum w u u^T on MFMA
//                  (v_mfma_f32_32x32x16_bf16).  x = sqrt(w) u is split into
//                  bf16 hi + lo and x x^T ~ hi hi^T + hi lo^T + lo hi^T, about
//                  16 significant bits per product; fp32 accumulation.
//   jacap_factor   per head: A = I + the slices' parts, Cholesky in LDS
//                  (fp32), then M = L^{-1} (right-looking, in LDS), stored as
//                  bf16 hi + lo.
//   jacap_leverage per (head, chunk): Y = M U^T on MFMA (hi and lo of M
//                  against the exact bf16 u), r = w * column sums of Y^2.
// The two N d^2 contractions are the MFMA part; everything else streams K
// and U once.

#include <math.h>

#include <algorithm>
#include <functional>

#include "kvsel_internal.h"

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kJThreads = 256;
constexpr int kJChunk = 1024;  // tokens per logits / weights / leverage workgroup
constexpr int kGramSub = 64;   // tokens per Gram step (LDS tile)
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Eight consecutive bf16 values (16 bytes) as floats.
__device__ __forceinline__ void load8(const __bf16* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void lse_merge(float& m, float& z, float mo, float zo) {
  const float d = mo - m;
  const float e = __expf(-fabsf(d));
  z = d > 0.f ? fmaf(z, e, zo) : fmaf(zo, e, z);
  m = fmaxf(m, mo);
}

// z_i and kappa_i of the chunk's tokens; (max, sum exp(z - max)) of the chunk.
template <int D>
__global__ __launch_bounds__(kJThreads) void jacap_logits_kernel(const JacapArgs j, const __bf16* __restrict__ K) {
  constexpr int LPT = D / 8;               // lanes per token
  constexpr int TPP = kJThreads / LPT;     // tokens per pass
  const int head = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, part = tid % LPT, slot = tid / LPT;
  __shared__ float sm[kJThreads / 64], sz[kJThreads / 64];
  float mu[8], lam[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mu[e] = j.mu[(long long)head * D + part * 8 + e];
    lam[e] = j.lambda[(long long)head * D + part * 8 + e];
  }
  if (head == 0 && c == 0 && tid == 0 && j.err != nullptr) *j.err = 0u;  // the later kernels raise flags
  const float scale = 1.f / (j.tau * sqrtf((float)D));
  float m = kNegBig, s = 0.f;
  const int t0 = c * kJChunk, t1 = min(t0 + kJChunk, j.N);
  for (int base = t0; base < t1; base += TPP) {  // every lane takes part in the shuffles
    const int t = base + slot;
    float zz = 0.f, kk = 0.f;
    if (t < t1) {
      float k[8];
      load8(K + ((long long)head * j.N + t) * D + part * 8, k);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        zz = fmaf(k[e], mu[e], zz);
        kk = fmaf(lam[e] * k[e], k[e], kk);
      }
    }
#pragma unroll
    for (int o = LPT / 2; o >= 1; o >>= 1) {
      zz += __shfl_xor(zz, o, LPT);
      kk += __shfl_xor(kk, o, LPT);
    }
    if (t < t1) {
      const float z = zz * scale;
      if (part == 0) {
        j.z[(long long)head * j.N + t] = z;
        j.kappa[(long long)head * j.N + t] = kk;
      }
      if (part == 0) lse_merge(m, s, z, 1.f);
    }
  }
  // The chunk's partial: lanes of the wave, then the waves in order.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mo = __shfl_xor(m, o), so = __shfl_xor(s, o);
    lse_merge(m, s, mo, so);
  }
  if ((tid & 63) == 0) {
    sm[tid >> 6] = m;
    sz[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = sm[0], ss = sz[0];
    for (int w = 1; w < kJThreads / 64; ++w) lse_merge(mm, ss, sm[w], sz[w]);
    j.part[((long long)head * j.nch + c) * 2] = mm;
    j.part[((long long)head * j.nch + c) * 2 + 1] = ss;
  }
}

// w_i of the chunk's tokens from the head's softmax normaliser.
__global__ __launch_bounds__(kJThreads) void jacap_weights_kernel(const JacapArgs j, int D) {
  const int head = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  __shared__ float s_m, s_z;
  if (tid == 0) {  // the head's partials in chunk order: every workgroup gets the same (M, Z)
    float m = kNegBig, s = 0.f;
    for (int q = 0; q < j.nch; ++q)
      lse_merge(m, s, j.part[((long long)head * j.nch + q) * 2], j.part[((long long)head * j.nch + q) * 2 + 1]);
    s_m = m;
    s_z = s;
    if (!(isfinite(m) && isfinite(s) && s > 0.f)) raise_error(j.err, kErrNonFinite);
  }
  __syncthreads();
  const float M = s_m, iz = 1.f / s_z, invd = 1.f / (float)D;
  const int t0 = c * kJChunk, t1 = min(t0 + kJChunk, j.N);
  for (int t = t0 + tid; t < t1; t += kJThreads) {
    const long long i = (long long)head * j.N + t;
    const float a = __expf(j.z[i] - M) * iz;
    const float rho = a * (1.f - a);
    j.w[i] = rho * rho * j.kappa[i] * invd;
  }
}

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// Part of sum_i w_i u_i u_i^T over tokens [slice * per, (slice + 1) * per) of
// the head, into gpart[head][slice][D][D].  Tile (p, q) of the D x D result
// (32 x 32) belongs to wave (p * (D / 32) + q) % 4; x^T (features x tokens)
// is staged in LDS as hi and lo parts, a row of kGramSub + 8 elements.
template <int D>
__global__ __launch_bounds__(kJThreads) void jacap_gram_kernel(const JacapArgs j, const __bf16* __restrict__ U) {
  constexpr int NT = D / 32;               // tiles per side
  constexpr int TPW = NT * NT / 4;         // tiles per wave (4 or 1)
  constexpr int RS = kGramSub + 8;         // LDS row stride (elements)
  __shared__ __bf16 xh[D * RS], xl[D * RS];
  const int head = blockIdx.y, slice = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  const int per = (j.N + j.slices - 1) / j.slices;
  const int t0 = slice * per, t1 = min(t0 + per, j.N);
  f32x16 acc[TPW];
#pragma unroll
  for (int q = 0; q < TPW; ++q) acc[q] = f32x16{};
  for (int s0 = t0; s0 < t1; s0 += kGramSub) {
    __syncthreads();  // the previous step's operands have been read
    // Stage x = sqrt(w) u of kGramSub tokens, transposed: consecutive
    // threads take consecutive tokens of one 8-feature group.
    for (int e = tid; e < kGramSub * (D / 8); e += kJThreads) {
      const int tk = e % kGramSub, f8 = e / kGramSub, t = s0 + tk;
      float u[8];
      float sw = 0.f;
      if (t < t1) {
        load8(U + ((long long)head * j.N + t) * D + f8 * 8, u);
        sw = sqrtf(fmaxf(j.w[(long long)head * j.N + t], 0.f));
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = 0.f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __bf16 hi, lo;
        split_bf16(sw * u[q], hi, lo);
        xh[(f8 * 8 + q) * RS + tk] = hi;
        xl[(f8 * 8 + q) * RS + tk] = lo;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int tile = wave * TPW + q;
      const int p = tile / NT, r = tile % NT;
#pragma unroll
      for (int k0 = 0; k0 < kGramSub; k0 += 16) {
        const int ra = (p * 32 + n) * RS + k0 + 8 * g, rb = (r * 32 + n) * RS + k0 + 8 * g;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&xh[ra]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&xl[ra]);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&xh[rb]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&xl[rb]);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[q], 0, 0, 0);
      }
    }
  }
  float* out = j.gpart + ((long long)head * j.slices + slice) * D * D;
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int tile = wave * TPW + q;
    const int p = tile / NT, r = tile % NT;
#pragma unroll
    for (int e = 0; e < 16; ++e) out[(p * 32 + acc_row(e, g)) * D + r * 32 + n] = acc[q][e];
  }
}

// A = I + the slices' parts; Cholesky A = L L^T in LDS (fp32, column by
// column); M = L^{-1} by forward substitution (a column of M per thread);
// M stored as bf16 hi and lo, row-major, for the leverage contraction.
template <int D>
__global__ __launch_bounds__(kJThreads) void jacap_factor_kernel(const JacapArgs j) {
  __shared__ float a[D * (D + 1)];  // row stride D + 1
  constexpr int S = D + 1;
  const int head = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < D * D; e += kJThreads) {
    const int r = e / D, c = e % D;
    float v = r == c ? 1.f : 0.f;
    for (int s = 0; s < j.slices; ++s) v += j.gpart[(((long long)head * j.slices + s) * D + r) * D + c];
    a[r * S + c] = v;
  }
  __syncthreads();
  __shared__ int s_bad;
  if (tid == 0) s_bad = 0;
  for (int c = 0; c < D; ++c) {
    if (tid == 0) {
      const float d = a[c * S + c];
      if (!(d > 0.f) || !isfinite(d)) s_bad = 1;
      a[c * S + c] = sqrtf(fmaxf(d, 1e-30f));
    }
    __syncthreads();
    const float inv = 1.f / a[c * S + c];
    for (int r = c + 1 + tid; r < D; r += kJThreads) a[r * S + c] *= inv;
    __syncthreads();
    // Trailing update of the lower triangle: (r, k) with c < k <= r.
    const int rem = D - c - 1;
    for (int e = tid; e < rem * rem; e += kJThreads) {
      const int r = c + 1 + e / rem, k = c + 1 + e % rem;
      if (k <= r) a[r * S + k] -= a[r * S + c] * a[k * S + c];
    }
    __syncthreads();
  }
  if (tid == 0 && s_bad) raise_error(j.err, kErrNonFinite);
  // M = L^{-1}, right-looking: start from I; step k scales row k by 1/L[k][k]
  // and removes L[i][k] times row k from every row i > k (columns <= k are
  // the only non-zero ones of row k).
  __shared__ float m[D * (D + 1)];
  for (int e = tid; e < D * D; e += kJThreads) m[(e / D) * S + e % D] = (e / D == e % D) ? 1.f : 0.f;
  __syncthreads();
  for (int k = 0; k < D; ++k) {
    const float inv = 1.f / a[k * S + k];
    for (int c2 = tid; c2 <= k; c2 += kJThreads) m[k * S + c2] *= inv;
    __syncthreads();
    const int rows = D - k - 1, cols = k + 1;
    for (int e = tid; e < rows * cols; e += kJThreads) {
      const int i = k + 1 + e / cols, c2 = e % cols;
      m[i * S + c2] -= a[i * S + k] * m[k * S + c2];
    }
    __syncthreads();
  }
  __bf16* mh = j.minv + (long long)head * 2 * D * D;
  __bf16* ml = mh + D * D;
  for (int e = tid; e < D * D; e += kJThreads) {
    __bf16 hi, lo;
    split_bf16(m[(e / D) * S + e % D], hi, lo);
    mh[e] = hi;
    ml[e] = lo;
  }
}

// r_t = w_t |M u_t|^2 for the chunk's tokens: per 32-token block, Y = M U^T
// as (D / 32) tiles of 32 x 32, M's hi and lo against the exact bf16 u, and
// each lane sums the squares of its rows; the two halves of the wave hold
// the other rows of the same tokens.  M (hi, lo) is staged in LDS.
template <int D>
__global__ __launch_bounds__(kJThreads) void jacap_leverage_kernel(const JacapArgs j, const __bf16* __restrict__ U) {
  constexpr int RS = D + 8;
  __shared__ __bf16 mh[D * RS], ml[D * RS];
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
  for (int b0 = t0 + wave * 32; b0 < t1; b0 += 4 * 32) {
    const int t = min(b0 + n, t1 - 1);  // rows past the chunk repeat its last token (not written)
    const __bf16* ur = U + ((long long)head * j.N + t) * D;
    bf16x8 ub[D / 16];  // the token's u, loaded once for all row tiles
#pragma unroll
    for (int k = 0; k < D / 16; ++k) ub[k] = *reinterpret_cast<const bf16x8*>(ur + 16 * k + 8 * g);
    float sq = 0.f;
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      f32x16 acc = {};
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&mh[(p * 32 + n) * RS + 16 * k + 8 * g]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&ml[(p * 32 + n) * RS + 16 * k + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, ub[k], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, ub[k], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) sq = fmaf(acc[e], acc[e], sq);
    }
    const float other = __shfl_xor(sq, 32);
    const float tot = g == 0 ? sq + other : other + sq;
    if (g == 0 && b0 + n < t1) {
      const long long i = (long long)head * j.N + b0 + n;
      j.r[i] = j.w[i] * tot;
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
      hipLaunchKernelGGL((jacap_gram_kernel<D>), dim3(j.slices, j.heads), dim3(kJThreads), 0, st, j, U);
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
int jacap_slices(int N) { return std::max(1, std::min(32, (N + 2047) / 2048)); }

hipError_t launch_jacap_scores(const JacapArgs& j, int D, const void* K, const void* U, hipStream_t st,
                               const std::function<hipError_t(const char*, const std::function<hipError_t()>&)>& timed) {
  if (D == 128) return launch_all<128>(j, (const __bf16*)K, (const __bf16*)U, st, timed);
  if (D == 64) return launch_all<64>(j, (const __bf16*)K, (const __bf16*)U, st, timed);
  return hipErrorNotSupported;
}

}  // namespace kvsel
