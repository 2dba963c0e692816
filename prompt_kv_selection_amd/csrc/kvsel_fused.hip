// Single-read window scoring for gfx950: logits, causal row statistics and
// prefix votes with K read from HBM exactly once.
//
// Method (web page "SnapKV: selecting the KV cache for long prompts with an
// observation window", section "votes must come from the causal softmax over
// the full prompt"): l[i][j] = q_i . k_j / sqrt(D) for window row i (query
// P + i); row i sees j <= P + i and its softmax denominator covers every
// visible prefix and window position; the vote of prefix position j < P is the
// sum over the window rows of the softmax probability.
//
// Why one kernel.  A vote needs each row's final maximum and normaliser, which
// depend on all L positions of the head, so a plain implementation reads K
// twice.  Here the logits of a chunk stay in VGPRs while the chunk's
// (max, sum of exponentials) partials are exchanged with the other chunks of
// the same head; then the votes are formed from the registers.
//
// Schedule.  A cooperative launch of two 4-wave workgroups per CU (all
// co-resident).  Work proceeds in rounds: in a round every workgroup owns one
// chunk of S = 4 * TT * 32 positions of some head (heads_per_round heads of a
// segment, each split over ceil(L / S) workgroups).  Round r's exchange is
// hidden behind round r + 1's K stream: the workgroup streams round r + 1
// into a second register set before it waits for round r's partials.
//
// Exchange.  Partials are written with agent-scope stores and read with
// agent-scope loads (both bypass the per-XCD L2), and a per-head counter is
// bumped with an agent-scope atomic after the stores have completed
// (s_waitcnt); no L2 writeback or invalidate is needed.  Every wait is bounded:
// on timeout the kernel records a flag in `status` and carries on, so the grid
// always drains.
//
// K tiles (32 positions x D) are loaded with 16-byte coalesced loads (1 KB
// contiguous per wave instruction) and staged through LDS into the MFMA
// operand layout; direct per-lane row loads leave the HBM stream well below
// its peak on this chip.  Merges of partials run in a fixed order, so every
// workgroup of a head derives bit-identical (max, normaliser), and equal keys
// get bit-equal votes.

#include <math.h>

#include "kvsel_internal.h"

// Instrumentation hook at pipeline-step boundaries (step k, point 0..3);
// empty unless a profiling build defines it.
#ifndef KVSEL_FUSED_MARK
#define KVSEL_FUSED_MARK(k, point)
#endif

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr float kNegBig = -1.0e30f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kFusedWaves = 4;
constexpr int kFusedThreads = kFusedWaves * 64;
constexpr long kSpinLimit = 1L << 22;

__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void lse_merge(float& m, float& z, float mo, float zo) {
  const float mn = fmaxf(m, mo);
  z = z * exp2_fast(m - mn) + zo * exp2_fast(mo - mn);
  m = mn;
}

struct Work {
  int e, h, c, hs;
  bool on;
};

// The (segment, head, chunk) this workgroup owns in round r, if any.
__device__ __forceinline__ Work round_work(const Launch& a, int r) {
  Work w{0, 0, 0, 0, false};
  if (r < 0 || r >= a.rounds) return w;
  int e = 0;
  for (int k = 1; k < a.n; ++k)
    if (r >= a.seg[k].fr0) e = k;
  const Seg& s = a.seg[e];
  const int slot = blockIdx.x;
  const int hh = slot / s.fc;
  const int c = slot - hh * s.fc;
  if (hh >= s.fhpr) return w;
  const int hl = (r - s.fr0) * s.fhpr + hh;
  if (hl >= s.nh) return w;
  w.e = e;
  w.h = s.h0 + hl;
  w.c = c;
  w.hs = s.b * a.heads + w.h;
  w.on = true;
  return w;
}

// Qwin rows of the head into LDS in the MFMA operand layout's row order
// (rows past W are zero).
template <int D, int RB>
__device__ __forceinline__ void load_q(const Launch& a, const Work& w, const __bf16* __restrict__ Q,
                                       uint4* __restrict__ s_q) {
  constexpr int PR = D / 8, ST = PR + 1;
  const __bf16* q = Q + (long long)w.hs * a.W * D;
  for (int idx = threadIdx.x; idx < RB * 32 * PR; idx += kFusedThreads) {
    const int row = idx / PR, col = idx - row * PR;
    s_q[row * ST + col] =
        row < a.W ? *reinterpret_cast<const uint4*>(q + (long long)row * D + col * 8) : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
}

// Per-head exchange record in the workspace (kHeadRec bytes, zeroed before
// the launch): two arrival counters, the encoded row maxima, and the
// fixed-point row normalisers.
// Each row's words sit on their own 64-byte line so that the atomics of the
// head's chunks on different rows do not serialise on one line.
constexpr int kRowStride = 64;                       // bytes between rows
constexpr int kHeadRec = 128 + 2 * 64 * kRowStride;  // counters + max rows + sum rows
constexpr double kFix = 68719476736.0;   // 2^36: fixed-point scale of the normaliser sums
struct HeadRec {
  unsigned* cnt_max;
  unsigned* cnt_sum;
  char* rows;
  __device__ __forceinline__ unsigned* m_enc(int i) const {  // order-preserving code of the row max
    return reinterpret_cast<unsigned*>(rows + i * kRowStride);
  }
  __device__ __forceinline__ unsigned long long* z_fix(int i) const {  // sum of round(z_c * 2^36)
    return reinterpret_cast<unsigned long long*>(rows + (64 + i) * kRowStride);
  }
};
__device__ __forceinline__ HeadRec head_rec(unsigned* ex, int hs) {
  char* base = reinterpret_cast<char*>(ex) + (long long)hs * kHeadRec;
  HeadRec r;
  r.cnt_max = reinterpret_cast<unsigned*>(base);
  r.cnt_sum = reinterpret_cast<unsigned*>(base + 64);
  r.rows = base + 128;
  return r;
}
// Monotone map of floats to unsigned integers (larger float, larger code).
__device__ __forceinline__ unsigned f2ord(float f) {
  const unsigned b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord2f(unsigned u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ void agent_add(unsigned* p, unsigned v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bounded wait for `target` arrivals (thread 0 only); returns false on timeout.
__device__ __forceinline__ bool wait_count(unsigned* cnt, unsigned target, unsigned* status) {
  long spins = 0;
  while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  return true;
}

// Phase A: stream one chunk of K into logits x (base 2, -inf where masked),
// fold the chunk's row maxima into the head's maxima, count the arrival.
template <int D, int RB, int TT>
__device__ __forceinline__ void phase_stream(const Launch& a, const Work& w, const __bf16* __restrict__ Q,
                                             const __bf16* __restrict__ K, uint4* __restrict__ s_q,
                                             uint4* __restrict__ stage, float (&x)[TT][RB][16],
                                             float* __restrict__ s_red, unsigned* __restrict__ ex) {
  constexpr int PR = D / 8;       // 16-byte pieces per K row
  constexpr int NL = PR / 2;      // pieces per lane per 32-row tile
  constexpr int ST = PR + 1;      // LDS row stride in pieces (one pad)
  const Seg& s = a.seg[w.e];
  const int L = s.L, W = a.W, P = L - W;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  load_q<D, RB>(a, w, Q, s_q);
  const __bf16* kh = K + s.kv_off + (long long)w.h * L * D;
  const int pw = w.c * a.S + wave * TT * 32;

#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int p0 = pw + t * 32;
    if (p0 < L) {
      uint4 v[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int q = lane + 64 * i;
        const int row = min(p0 + q / PR, L - 1);
        v[i] = *reinterpret_cast<const uint4*>(kh + (long long)row * D + (q % PR) * 8);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int q = lane + 64 * i;
        stage[(q / PR) * ST + q % PR] = v[i];
      }
      __builtin_amdgcn_wave_barrier();
      bf16x8 kb[D / 16];
#pragma unroll
      for (int k = 0; k < D / 16; ++k) kb[k] = __builtin_bit_cast(bf16x8, stage[n * ST + 2 * k + g]);
      __builtin_amdgcn_wave_barrier();
      const int j = p0 + n;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x16 acc = {};
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
          const bf16x8 qk = __builtin_bit_cast(bf16x8, s_q[(rb * 32 + n) * ST + 2 * k + g]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qk, kb[k], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = rb * 32 + acc_row(r, g);
          const bool visible = (j < L) && (i < W) && (j <= P + i);
          x[t][rb][r] = visible ? acc[r] * a.scale2 : -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[t][rb][r] = -INFINITY;
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float mm = kNegBig;
#pragma unroll
      for (int t = 0; t < TT; ++t) mm = fmaxf(mm, x[t][rb][r]);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
      if (n == 0) s_red[wave * RB * 32 + rb * 32 + acc_row(r, g)] = mm;
    }
  __syncthreads();
  const HeadRec hr = head_rec(ex, w.hs);
  if ((int)threadIdx.x < W) {
    const int i = threadIdx.x;
    float mm = s_red[i];
#pragma unroll
    for (int v = 1; v < kFusedWaves; ++v) mm = fmaxf(mm, s_red[v * RB * 32 + i]);
    __hip_atomic_fetch_max(hr.m_enc(i), f2ord(mm), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The arrival is counted at the start of the next pipeline step
  // (announce()), once these atomics have completed.
}

// Phase B: once every chunk of the head has folded in its maxima, turn the
// logits into u = exp2(x - m) in place and add the chunk's row sums (fixed
// point, so the total does not depend on arrival order) to the head's sums.
template <int D, int RB, int TT>
__device__ __forceinline__ void phase_normalise(const Launch& a, const Work& w, float (&x)[TT][RB][16],
                                                float* __restrict__ s_red, float* __restrict__ s_m,
                                                int* __restrict__ s_flag, unsigned* __restrict__ ex,
                                                unsigned* __restrict__ status) {
  constexpr int ROWS = RB * 32;
  const Seg& s = a.seg[w.e];
  const int W = a.W;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  const HeadRec hr = head_rec(ex, w.hs);
  if (tid == 0 && !wait_count(hr.cnt_max, (unsigned)s.fc, status)) s_flag[0] = 1;  // sticky
  __syncthreads();
  if (tid < ROWS)
    s_m[tid] = tid < W ? ord2f(__hip_atomic_load(hr.m_enc(tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) : 0.f;
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float m = s_m[rb * 32 + acc_row(r, g)];
      float zz = 0.f;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        x[t][rb][r] = exp2_fast(x[t][rb][r] - m);
        zz += x[t][rb][r];
      }
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) zz += __shfl_xor(zz, off);
      if (n == 0) s_red[wave * ROWS + rb * 32 + acc_row(r, g)] = zz;
    }
  __syncthreads();
  if (tid < W) {
    float zz = s_red[tid];
#pragma unroll
    for (int v = 1; v < kFusedWaves; ++v) zz += s_red[v * ROWS + tid];
    const unsigned long long fix = (unsigned long long)__double2ll_rn((double)zz * kFix);
    __hip_atomic_fetch_add(hr.z_fix(tid), fix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Counted at the start of the next pipeline step (announce()).
}

// Count this workgroup's earlier contributions to the exchange records: the
// row maxima of round km and the row sums of round ks (either may be absent).
// The waitcnt makes sure those atomics have completed before the counters
// move; by now they have had a whole phase to do so.
__device__ __forceinline__ void announce(const Launch& a, int km, int ks, unsigned* ex) {
  const Work wm = round_work(a, km);
  const Work ws = round_work(a, ks);
  if (!wm.on && !ws.on) return;
  if ((int)threadIdx.x < a.W) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (wm.on && km >= 0) agent_add(head_rec(ex, wm.hs).cnt_max, 1u);
    if (ws.on && ks >= 0) agent_add(head_rec(ex, ws.hs).cnt_sum, 1u);
  }
}

// Phase C: once the head's row sums are complete, write the votes of this
// chunk's prefix positions: sum over the window rows of u / Z.
template <int D, int RB, int TT>
__device__ __forceinline__ void phase_votes(const Launch& a, const Work& w, const float (&u)[TT][RB][16],
                                            float* __restrict__ s_iz, int* __restrict__ s_flag,
                                            unsigned* __restrict__ ex, unsigned* __restrict__ status,
                                            float* __restrict__ votes, float* __restrict__ row_stats) {
  constexpr int ROWS = RB * 32;
  const Seg& s = a.seg[w.e];
  const int L = s.L, W = a.W, P = L - W;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  const HeadRec hr = head_rec(ex, w.hs);
  if (tid == 0 && !wait_count(hr.cnt_sum, (unsigned)s.fc, status)) s_flag[1] = 1;  // sticky
  __syncthreads();
  if (tid < ROWS) {
    float iz = 0.f;  // rows past W hold u = 0
    if (tid < W) {
      const unsigned long long fix = __hip_atomic_load(hr.z_fix(tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const double Z = (double)fix / kFix;
      iz = (s_flag[0] | s_flag[1]) ? __builtin_nanf("") : (float)(1.0 / Z);  // NaN marks a timed-out exchange
      if (row_stats != nullptr && w.c == 0) {
        const float m = ord2f(__hip_atomic_load(hr.m_enc(tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        float* rs = row_stats + ((long long)w.hs * W + tid) * 2;
        rs[0] = m * kLn2;
        rs[1] = (float)Z;
      }
    }
    s_iz[tid] = iz;
  }
  __syncthreads();
  float izr[RB][16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) izr[rb][r] = s_iz[rb * 32 + acc_row(r, g)];
  float* vout = votes + s.vote_off + (long long)w.h * s.vote_ld;
  const int pw = w.c * a.S + wave * TT * 32;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int p0 = pw + t * 32;
    if (p0 < P) {
      float tot = 0.f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += u[t][rb][r] * izr[rb][r];
        tot += sum;
      }
      const float other = __shfl_xor(tot, 32);
      const float v = g == 0 ? tot + other : other + tot;
      const int j = p0 + n;
      if (g == 0 && j < P) vout[j] = v;
    }
  }
  __syncthreads();
}

// One step k of the three-set pipeline: stream round k, normalise round
// k - 1, vote round k - 2 (X0 receives round k, X2 holds round k - 1, X1
// round k - 2).  Each exchange wait is covered by a full K stream.
template <int D, int RB, int TT>
__device__ __forceinline__ void step3(const Launch& a, int k, const __bf16* __restrict__ Q,
                                      const __bf16* __restrict__ K, float (&X0)[TT][RB][16], float (&X1)[TT][RB][16],
                                      float (&X2)[TT][RB][16], uint4* s_q, uint4* stage, float* s_red, float* s_m,
                                      float* s_iz, int* s_flag, unsigned* ex, unsigned* status, float* votes,
                                      float* row_stats) {
  KVSEL_FUSED_MARK(k, 0);
  announce(a, k - 1, k - 2, ex);
  const Work w0 = round_work(a, k);
  if (w0.on) phase_stream<D, RB, TT>(a, w0, Q, K, s_q, stage, X0, s_red, ex);
  KVSEL_FUSED_MARK(k, 1);
  if (k >= 1) {
    const Work w1 = round_work(a, k - 1);
    if (w1.on) phase_normalise<D, RB, TT>(a, w1, X2, s_red, s_m, s_flag, ex, status);
  }
  KVSEL_FUSED_MARK(k, 2);
  if (k >= 2) {
    const Work w2 = round_work(a, k - 2);
    if (w2.on) phase_votes<D, RB, TT>(a, w2, X1, s_iz, s_flag, ex, status, votes, row_stats);
  }
  KVSEL_FUSED_MARK(k, 3);
}

// One step k of the two-set pipeline: stream round k into X0, then
// normalise and vote round k - 1 from X1 (the second exchange wait is not
// covered).
template <int D, int RB, int TT>
__device__ __forceinline__ void step2(const Launch& a, int k, const __bf16* __restrict__ Q,
                                      const __bf16* __restrict__ K, float (&X0)[TT][RB][16], float (&X1)[TT][RB][16],
                                      uint4* s_q, uint4* stage, float* s_red, float* s_m, float* s_iz, int* s_flag,
                                      unsigned* ex, unsigned* status, float* votes, float* row_stats) {
  announce(a, k - 1, -1, ex);
  const Work w0 = round_work(a, k);
  if (w0.on) phase_stream<D, RB, TT>(a, w0, Q, K, s_q, stage, X0, s_red, ex);
  if (k >= 1) {
    const Work w1 = round_work(a, k - 1);
    if (w1.on) {
      phase_normalise<D, RB, TT>(a, w1, X1, s_red, s_m, s_flag, ex, status);
      announce(a, -1, k - 1, ex);
      phase_votes<D, RB, TT>(a, w1, X1, s_iz, s_flag, ex, status, votes, row_stats);
    }
  }
}

template <int D, int RB, int TT, int NSETS>
__global__ __launch_bounds__(kFusedThreads, 2) void window_fused_kernel(const Launch a, const __bf16* __restrict__ Q,
                                                                       const __bf16* __restrict__ K,
                                                                       unsigned* __restrict__ ex,
                                                                       unsigned* __restrict__ status,
                                                                       float* __restrict__ votes,
                                                                       float* __restrict__ row_stats) {
  __shared__ uint4 s_stage[kFusedWaves][32 * (D / 8 + 1)];
  __shared__ uint4 s_q[RB * 32 * (D / 8 + 1)];
  __shared__ float s_red[kFusedWaves * RB * 32];
  __shared__ float s_m[RB * 32], s_iz[RB * 32];
  __shared__ int s_flag[2];  // a timed-out exchange in this workgroup (then votes are NaN)
  if (threadIdx.x == 0) s_flag[0] = s_flag[1] = 0;
  __syncthreads();
  uint4* stage = s_stage[threadIdx.x >> 6];
  if constexpr (NSETS == 3) {
    float xa[TT][RB][16], xb[TT][RB][16], xc[TT][RB][16];
    const int steps = a.rounds + 2;
    for (int k = 0; k < steps; k += 3) {
      step3<D, RB, TT>(a, k, Q, K, xa, xb, xc, s_q, stage, s_red, s_m, s_iz, s_flag, ex, status, votes, row_stats);
      if (k + 1 >= steps) break;
      step3<D, RB, TT>(a, k + 1, Q, K, xb, xc, xa, s_q, stage, s_red, s_m, s_iz, s_flag, ex, status, votes, row_stats);
      if (k + 2 >= steps) break;
      step3<D, RB, TT>(a, k + 2, Q, K, xc, xa, xb, s_q, stage, s_red, s_m, s_iz, s_flag, ex, status, votes, row_stats);
    }
  } else {
    float xa[TT][RB][16], xb[TT][RB][16];
    const int steps = a.rounds + 1;
    for (int k = 0; k < steps; k += 2) {
      step2<D, RB, TT>(a, k, Q, K, xa, xb, s_q, stage, s_red, s_m, s_iz, s_flag, ex, status, votes, row_stats);
      if (k + 1 >= steps) break;
      step2<D, RB, TT>(a, k + 1, Q, K, xb, xa, s_q, stage, s_red, s_m, s_iz, s_flag, ex, status, votes, row_stats);
    }
  }
}

__global__ void fill_u32_kernel(unsigned* p, long long n, unsigned v) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Register sets of the pipeline and tiles per wave per round: each set
// holds W x S / 256 floats per lane, so wide windows get the shallower
// pipeline.
template <int D, int RB>
constexpr int tiles_per_wave() {
  return 2;
}
template <int D, int RB>
constexpr int pipeline_sets() {
  return RB == 1 ? 3 : 2;
}
template <int D, int RB>
void* fused_kernel_ptr() {
  return (void*)window_fused_kernel<D, RB, tiles_per_wave<D, RB>(), pipeline_sets<D, RB>()>;
}

struct GridCache {
  int device = -1;
  int grid[2][2] = {{-1, -1}, {-1, -1}};
};
GridCache g_grid;

template <int D, int RB>
int grid_for() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (g_grid.device != dev) {
    g_grid = GridCache{};
    g_grid.device = dev;
  }
  int& slot = g_grid.grid[D == 128][RB - 1];
  if (slot < 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fused_kernel_ptr<D, RB>(),
                                                     kFusedThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    slot = per_cu >= 2 ? 2 * cus : per_cu * cus;
  }
  return slot;
}

template <int D, int RB>
hipError_t launch_t(const Launch& a, const void* Q, const void* K, unsigned* ex, unsigned* status, float* votes,
                    float* row_stats, hipStream_t st) {
  const int grid = grid_for<D, RB>();
  if (grid <= 0) return hipErrorNotSupported;
  Launch la = a;
  const __bf16* q = (const __bf16*)Q;
  const __bf16* k = (const __bf16*)K;
  void* args[] = {&la, &q, &k, &ex, &status, &votes, &row_stats};
  return hipLaunchCooperativeKernel((const void*)fused_kernel_ptr<D, RB>(), dim3(grid),
                                    dim3(kFusedThreads), args, 0, st);
}

}  // namespace

int fused_positions(int W, int D) {
  (void)D;
  return W <= 32 ? kFusedWaves * tiles_per_wave<128, 1>() * 32 : kFusedWaves * tiles_per_wave<128, 2>() * 32;
}

int fused_grid(int W, int D) {
  if (W > 64 || (D != 64 && D != 128)) return 0;
  if (D == 128) return W <= 32 ? grid_for<128, 1>() : grid_for<128, 2>();
  return W <= 32 ? grid_for<64, 1>() : grid_for<64, 2>();
}

int fused_exchange_bytes() { return kHeadRec; }

hipError_t launch_fused_scoring(const Launch& a, const void* Q, const void* K, unsigned* ex, unsigned* status,
                                float* votes, float* row_stats, hipStream_t st) {
  if (a.W > 64 || a.S != fused_positions(a.W, a.D)) return hipErrorNotSupported;
  if (a.D == 128)
    return a.W <= 32 ? launch_t<128, 1>(a, Q, K, ex, status, votes, row_stats, st)
                     : launch_t<128, 2>(a, Q, K, ex, status, votes, row_stats, st);
  if (a.D == 64)
    return a.W <= 32 ? launch_t<64, 1>(a, Q, K, ex, status, votes, row_stats, st)
                     : launch_t<64, 2>(a, Q, K, ex, status, votes, row_stats, st);
  return hipErrorNotSupported;
}

hipError_t launch_fill_u32(unsigned* p, long long n, unsigned v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace kvsel
