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
// twice.  Here the logits of a chunk stay in VGPRs while the head's row maxima
// and row sums are agreed on across the workgroups that hold its chunks.
//
// Schedule.  A cooperative launch of one workgroup per CU (all co-resident).
// Work proceeds in rounds; in a round every workgroup owns one chunk of
// S = 512 positions of some head (heads_per_round heads, each split over
// ceil(L / S) workgroups).  Two register sets form a pipeline: in step k the
// workgroup streams round k while it normalises and votes round k - 1, and
// the K ring keeps a whole round of loads in flight through the exchanges.
//
// Roles inside a workgroup.  Four streaming waves and one controller wave.
//  * Streaming waves read global memory only through direct-to-LDS loads of
//    K tiles (global_load_lds_dwordx4, 1 KB contiguous per instruction) into a
//    private ring of four 32-row tiles, issued ahead and waited for with
//    explicit vmcnt counts, so the HBM stream never drains while they compute.
//    They form the logits on MFMA (v_mfma_f32_32x32x16_bf16, Qwin rows from
//    LDS), exponentials and votes, and talk to the controller through LDS.
//  * The controller wave does every other global access: it loads Qwin
//    (double-buffered in LDS), folds the waves' partial row maxima into the
//    head's maxima (atomic max on order-preserving codes), adds the partial
//    row sums to the head's sums (fixed point round(z * 2^30) plus an arrival
//    count in the top bits, one 64-bit atomic add per row: the total does not
//    depend on arrival order), polls for completion, broadcasts the final
//    values through LDS, and writes the votes.  Its global traffic therefore
//    never sits in the streaming waves' in-order vmcnt queue.
// All exchange accesses are agent scope (they bypass the per-XCD L2); every
// wait is bounded, and a timed-out wait records a flag and marks the head's
// votes NaN, so the grid always drains.
//
// LDS tiles use an XOR swizzle (piece c of row r stored at c ^ (r % pieces))
// so that the direct-to-LDS writes stay contiguous and the MFMA operand reads
// are free of bank conflicts.

#include <math.h>

#include "kvsel_internal.h"

// Instrumentation hook in the streaming waves (step k, point 0..3); empty
// unless a profiling build defines it.
#ifndef KVSEL_FUSED_MARK
#define KVSEL_FUSED_MARK(k, point)
#endif

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr float kNegBig = -1.0e30f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kSW = 4;                    // streaming waves
constexpr int kThreads = (kSW + 1) * 64;  // plus one controller wave
constexpr int kTT = 4;                    // 32-position tiles per streaming wave per round
constexpr int kNBuf = 4;                  // K tiles in flight per streaming wave
constexpr int kS = kSW * kTT * 32;        // positions per workgroup per round
constexpr long kSpin = 1L << 22;          // bound of every wait loop

__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

// ---- per-(sequence, head) exchange record in the workspace, zeroed per call
constexpr int kRowStride = 64;                          // bytes between rows (one line each)
constexpr int kHeadRec = 64 + 2 * 32 * kRowStride;      // counter line, 32 max rows, 32 sum rows
constexpr double kZScale = 1073741824.0;                // 2^30
constexpr unsigned long long kArrive = 1ull << 55;      // one arrival in the sum words
constexpr unsigned long long kSumMask = kArrive - 1;
struct HeadRec {
  unsigned* cnt_max;  // chunks whose maxima are folded in
  char* rows;
  __device__ __forceinline__ unsigned* m_enc(int i) const { return reinterpret_cast<unsigned*>(rows + i * kRowStride); }
  __device__ __forceinline__ unsigned long long* z_word(int i) const {
    return reinterpret_cast<unsigned long long*>(rows + (32 + i) * kRowStride);
  }
};
__device__ __forceinline__ HeadRec head_rec(unsigned* ex, int hs) {
  char* base = reinterpret_cast<char*>(ex) + (long long)hs * kHeadRec;
  return HeadRec{reinterpret_cast<unsigned*>(base), base + 64};
}
// Monotone map of floats to unsigned integers (larger float, larger code).
__device__ __forceinline__ unsigned f2ord(float f) {
  const unsigned b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord2f(unsigned u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// ---- LDS signalling between the waves of the workgroup.  A wave's LDS
// operations complete in order, so data written before a signal is visible to
// a wave that has seen the signal.
struct Sync {
  unsigned cnt_a, cnt_b, cnt_c;    // streaming-wave arrivals (max, sum, votes partials)
  unsigned q_ready;                // Qwin of rounds < q_ready is in LDS
  unsigned m_ready, z_ready;       // final row max / normaliser of rounds < value broadcast
  unsigned timeout;
};
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned lds_get(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_wait_ge(unsigned* p, unsigned target, unsigned* timeout) {
  long spins = 0;
  while (lds_get(p) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpin) {
      *timeout = 1;
      break;
    }
  }
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_add(unsigned* p) {
  lds_fence();
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_set(unsigned* p, unsigned v) {
  lds_fence();
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---- direct-to-LDS K tiles (streaming waves)
template <int D>
struct TileGeom {
  static constexpr int PR = D / 8;         // 16-byte pieces per row
  static constexpr int NL = PR / 2;        // load instructions per 32-row tile (64 pieces each)
  static constexpr int PIECES = 32 * PR;   // pieces per tile
};

// Issue the loads of the 32-row tile starting at p0 into an LDS tile.  Piece c
// of tile row r lands at r * PR + (c ^ (r % PR)).
template <int D>
__device__ __forceinline__ void issue_tile(const __bf16* __restrict__ kh, int L, int p0, const uint4* lds_tile,
                                           int lane) {
  using G = TileGeom<D>;
  const unsigned base = (unsigned)(uintptr_t)lds_tile;
#pragma unroll
  for (int i = 0; i < G::NL; ++i) {
    const int piece = i * 64 + lane;
    const int r = piece / G::PR;
    const int c = (piece % G::PR) ^ (r & (G::PR - 1));
    const int row = min(p0 + r, L - 1);
    const __bf16* g = kh + (long long)row * D + c * 8;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(base + i * 1024)), "v"(g)
                 : "memory", "m0");
  }
}

// Wait until at most `tiles_after` tiles' loads of this wave are outstanding.
template <int D>
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  constexpr int NL = TileGeom<D>::NL;
  switch (tiles_after) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * NL) : "memory"); break;
  }
}

// The tile stream of one streaming wave: tile q = round * kTT + t covers
// positions c * kS + wave * kTT * 32 + t * 32 of the round's head.
struct Stream {
  unsigned issued;  // bit (q % 32): tile q has loads outstanding
};

template <int D>
__device__ __forceinline__ void stream_issue(const Launch& a, const __bf16* __restrict__ K, int q, int wave,
                                             int lane, uint4 (*ring)[TileGeom<D>::PIECES], Stream& st) {
  const int k = q / kTT, t = q - (q / kTT) * kTT;
  const Work w = round_work(a, k);
  if (!w.on) return;
  const Seg& s = a.seg[w.e];
  const int p0 = w.c * kS + wave * kTT * 32 + t * 32;
  if (p0 >= s.L) return;
  issue_tile<D>(K + s.kv_off + (long long)w.h * s.L * D, s.L, p0, ring[q % kNBuf], lane);
  st.issued |= 1u << (q & 31);
}

__device__ __forceinline__ int tiles_after(const Stream& st, int q) {
  int n = 0;
#pragma unroll
  for (int j = 1; j < kNBuf; ++j) n += (st.issued >> ((q + j) & 31)) & 1u;
  return n;
}

// Phase A (streaming wave): logits of round k into x, row maxima to LDS.
template <int D>
__device__ __forceinline__ void phase_stream(const Launch& a, const Work& w, int k, const __bf16* __restrict__ K,
                                             uint4 (*ring)[TileGeom<D>::PIECES], const uint4* __restrict__ qbuf,
                                             float (&x)[kTT][16], Stream& st, float* s_maxp, Sync* sy) {
  using G = TileGeom<D>;
  const Seg& s = a.seg[w.e];
  const int L = s.L, W = a.W, P = L - W;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  lds_wait_ge(&sy->q_ready, (unsigned)k + 1, &sy->timeout);
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    const int q = k * kTT + t;
    const int p0 = w.c * kS + wave * kTT * 32 + t * 32;
    if (p0 < L) {
      wait_tiles<D>(tiles_after(st, q));
      const uint4* tile = ring[q % kNBuf];
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int c = 2 * kk + g;
        const int off = n * G::PR + (c ^ (n & (G::PR - 1)));
        const bf16x8 kb = __builtin_bit_cast(bf16x8, tile[off]);
        const bf16x8 qa = __builtin_bit_cast(bf16x8, qbuf[off]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, acc, 0, 0, 0);
      }
      const int j = p0 + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = acc_row(r, g);
        const bool visible = (j < L) && (i < W) && (j <= P + i);
        x[t][r] = visible ? acc[r] * a.scale2 : -INFINITY;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[t][r] = -INFINITY;
    }
    lds_fence();  // operands are in registers before the slot is reused
    st.issued &= ~(1u << (q & 31));
    stream_issue<D>(a, K, q + kNBuf, wave, lane, ring, st);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float mm = kNegBig;
#pragma unroll
    for (int t = 0; t < kTT; ++t) mm = fmaxf(mm, x[t][r]);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
    if (n == 0) s_maxp[wave * 32 + acc_row(r, g)] = mm;
  }
  lds_add(&sy->cnt_a);
}

// Streaming waves that own no chunk in round k still advance their tile
// stream (issue the tiles kNBuf ahead).
template <int D>
__device__ __forceinline__ void phase_skip(const Launch& a, int k, const __bf16* __restrict__ K,
                                           uint4 (*ring)[TileGeom<D>::PIECES], Stream& st) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < kTT; ++t) stream_issue<D>(a, K, k * kTT + t + kNBuf, wave, lane, ring, st);
}

// Phase B (streaming wave): u = exp2(x - m) in place, partial row sums to LDS.
__device__ __forceinline__ void phase_normalise(int k, float (&x)[kTT][16], const float* s_m, float* s_zp, Sync* sy) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  lds_wait_ge(&sy->m_ready, (unsigned)k + 1, &sy->timeout);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float m = s_m[acc_row(r, g)];
    float zz = 0.f;
#pragma unroll
    for (int t = 0; t < kTT; ++t) {
      x[t][r] = exp2_fast(x[t][r] - m);
      zz += x[t][r];
    }
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) zz += __shfl_xor(zz, off);
    if (n == 0) s_zp[wave * 32 + acc_row(r, g)] = zz;
  }
  lds_add(&sy->cnt_b);
}

// Phase C (streaming wave): votes of the wave's positions into LDS.
__device__ __forceinline__ void phase_votes(int k, const float (&u)[kTT][16], const float* s_iz, float* s_votes,
                                            Sync* sy) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  lds_wait_ge(&sy->z_ready, (unsigned)k + 1, &sy->timeout);
  float iz[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) iz[r] = s_iz[acc_row(r, g)];
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    float tot = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) tot += u[t][r] * iz[r];
    const float other = __shfl_xor(tot, 32);
    const float v = g == 0 ? tot + other : other + tot;
    if (g == 0) s_votes[wave * kTT * 32 + t * 32 + n] = v;
  }
  lds_add(&sy->cnt_c);
}

// Controller: load Qwin of round k into an LDS buffer (swizzled like K).
template <int D>
__device__ __forceinline__ void ctl_load_q(const Launch& a, int k, const __bf16* __restrict__ Q, uint4* qbuf) {
  using G = TileGeom<D>;
  const Work w = round_work(a, k);
  if (!w.on) return;
  const int lane = threadIdx.x & 63;
  const __bf16* q = Q + (long long)w.hs * a.W * D;
  uint4 v[G::NL];
#pragma unroll
  for (int i = 0; i < G::NL; ++i) {
    const int piece = i * 64 + lane;
    const int r = piece / G::PR, c = piece % G::PR;
    v[i] = r < a.W ? *reinterpret_cast<const uint4*>(q + (long long)r * D + c * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < G::NL; ++i) {
    const int piece = i * 64 + lane;
    const int r = piece / G::PR, c = piece % G::PR;
    qbuf[r * G::PR + (c ^ (r & (G::PR - 1)))] = v[i];
  }
}

// Controller: bounded poll of a global counter (lane 0), wave-uniform result.
__device__ __forceinline__ bool ctl_poll(unsigned* cnt, unsigned target, unsigned* status) {
  int ok = 1;
  if ((threadIdx.x & 63) == 0) {
    long spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpin) {
        __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
    }
  }
  return __shfl(ok, 0) != 0;
}

template <int D>
__device__ void controller(const Launch& a, const __bf16* __restrict__ Q, unsigned* __restrict__ ex,
                           unsigned* __restrict__ status, float* __restrict__ votes, float* __restrict__ row_stats,
                           uint4 (*qbufs)[TileGeom<D>::PIECES], float (*s_maxp)[kSW * 32],
                           float (*s_zp)[kSW * 32], float (*s_m)[32], float (*s_iz)[32],
                           float (*s_votes)[kS], Sync* sy) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  ctl_load_q<D>(a, 0, Q, qbufs[0]);
  ctl_load_q<D>(a, 1, Q, qbufs[1]);
  lds_set(&sy->q_ready, 2u);
  unsigned on_a = 0, on_b = 0, on_c = 0;  // owned rounds whose phase A / B / C partials were awaited
  for (int k = 0; k < a.rounds + 1; ++k) {
    const Work w0 = round_work(a, k), w1 = round_work(a, k - 1);
    // (1) Final maxima of round k - 1: all of its chunks have folded theirs in.
    if (w1.on) {
      const HeadRec hr = head_rec(ex, w1.hs);
      const bool ok = ctl_poll(hr.cnt_max, (unsigned)a.seg[w1.e].fc, status);
      if (lane < W) {
        const float m = ord2f(__hip_atomic_load(hr.m_enc(lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        s_m[(k - 1) & 1][lane] = ok ? m : __builtin_nanf("");
      }
    }
    if (k >= 1) lds_set(&sy->m_ready, (unsigned)k);
    // (2) Fold this workgroup's maxima of round k into the head's.
    if (w0.on) {
      ++on_a;
      lds_wait_ge(&sy->cnt_a, kSW * on_a, &sy->timeout);
      if (lane < W) {
        float mm = s_maxp[k & 1][lane];
#pragma unroll
        for (int v = 1; v < kSW; ++v) mm = fmaxf(mm, s_maxp[k & 1][v * 32 + lane]);
        __hip_atomic_fetch_max(head_rec(ex, w0.hs).m_enc(lane), f2ord(mm), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // Qwin of round k + 2 goes into the buffer of round k: its last user (the
    // latest owned round of the same parity) has finished phase A, which was
    // awaited above or at an earlier step.
    ctl_load_q<D>(a, k + 2, Q, qbufs[k & 1]);
    lds_set(&sy->q_ready, (unsigned)(k + 3));
    // (3) Add this workgroup's row sums of round k - 1 (value and arrival).
    if (w1.on) {
      ++on_b;
      lds_wait_ge(&sy->cnt_b, kSW * on_b, &sy->timeout);
      if (lane < W) {
        float zz = s_zp[(k - 1) & 1][lane];
#pragma unroll
        for (int v = 1; v < kSW; ++v) zz += s_zp[(k - 1) & 1][v * 32 + lane];
        const unsigned long long fix = (unsigned long long)__double2ll_rn((double)zz * kZScale) + kArrive;
        __hip_atomic_fetch_add(head_rec(ex, w1.hs).z_word(lane), fix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // The maxima must have landed before their arrival is counted.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (w0.on && lane == 0)
      __hip_atomic_fetch_add(head_rec(ex, w0.hs).cnt_max, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // (4) Final normalisers of round k - 1: every sum word carries fc arrivals.
    if (w1.on) {
      const HeadRec hr = head_rec(ex, w1.hs);
      const unsigned fc = (unsigned)a.seg[w1.e].fc;
      unsigned long long zw = 0;
      bool done = false;
      long spins = 0;
      while (!done) {
        zw = lane < W ? __hip_atomic_load(hr.z_word(lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : (unsigned long long)fc << 55;
        done = __ballot((unsigned)(zw >> 55) < fc) == 0;
        if (!done) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kSpin) {
            if (lane == 0) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
      if (lane < W) {
        const double Z = (double)(zw & kSumMask) / kZScale;
        s_iz[(k - 1) & 1][lane] = done ? (float)(1.0 / Z) : __builtin_nanf("");
        if (row_stats != nullptr && w1.c == 0) {
          float* rs = row_stats + ((long long)w1.hs * W + lane) * 2;
          rs[0] = s_m[(k - 1) & 1][lane] * kLn2;
          rs[1] = (float)Z;
        }
      }
    }
    if (k >= 1) lds_set(&sy->z_ready, (unsigned)k);
    // (5) Votes of round k - 1 to memory (prefix positions only).
    if (w1.on) {
      ++on_c;
      lds_wait_ge(&sy->cnt_c, kSW * on_c, &sy->timeout);
      const Seg& s = a.seg[w1.e];
      const int P = s.L - W;
      float* vout = votes + s.vote_off + (long long)w1.h * s.vote_ld;
      const int j0 = w1.c * kS;
      for (int i = lane; i < kS; i += 64)
        if (j0 + i < P) vout[j0 + i] = s_votes[(k - 1) & 1][i];
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void window_fused_kernel(const Launch a, const __bf16* __restrict__ Q,
                                                                  const __bf16* __restrict__ K,
                                                                  unsigned* __restrict__ ex,
                                                                  unsigned* __restrict__ status,
                                                                  float* __restrict__ votes,
                                                                  float* __restrict__ row_stats) {
  using G = TileGeom<D>;
  __shared__ uint4 s_ring[kSW][kNBuf][G::PIECES];
  __shared__ uint4 s_q[2][G::PIECES];
  __shared__ float s_maxp[2][kSW * 32], s_zp[2][kSW * 32];
  __shared__ float s_m[2][32], s_iz[2][32];
  __shared__ float s_votes[2][kS];
  __shared__ Sync sy;
  if (threadIdx.x == 0) sy = Sync{0, 0, 0, 0, 0, 0, 0};
  __syncthreads();  // the only workgroup barrier; afterwards waves meet through LDS flags
  const int wave = threadIdx.x >> 6;
  if (wave == kSW) {
    controller<D>(a, Q, ex, status, votes, row_stats, s_q, s_maxp, s_zp, s_m, s_iz, s_votes, &sy);
    if ((threadIdx.x & 63) == 0 && sy.timeout)
      __hip_atomic_fetch_or(status, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int lane = threadIdx.x & 63;
  uint4 (*ring)[G::PIECES] = s_ring[wave];
  Stream st{0u};
  for (int q = 0; q < kNBuf; ++q) stream_issue<D>(a, K, q, wave, lane, ring, st);
  float xa[kTT][16], xb[kTT][16];
  // Step k streams round k into one register set while round k - 1 is
  // normalised and voted from the other; the sets swap every step.  The
  // exchanges of round k - 1 overlap the loads of round k + 1, which the
  // ring has already issued.
  auto step = [&](int k, float (&X0)[kTT][16], float (&X1)[kTT][16]) {
    KVSEL_FUSED_MARK(k, 0);
    const Work w0 = round_work(a, k);
    if (w0.on)
      phase_stream<D>(a, w0, k, K, ring, s_q[k & 1], X0, st, s_maxp[k & 1], &sy);
    else
      phase_skip<D>(a, k, K, ring, st);
    KVSEL_FUSED_MARK(k, 1);
    if (round_work(a, k - 1).on) {
      phase_normalise(k - 1, X1, s_m[(k - 1) & 1], s_zp[(k - 1) & 1], &sy);
      KVSEL_FUSED_MARK(k, 2);
      phase_votes(k - 1, X1, s_iz[(k - 1) & 1], s_votes[(k - 1) & 1], &sy);
    }
    KVSEL_FUSED_MARK(k, 3);
  };
  const int steps = a.rounds + 1;
  for (int k = 0; k < steps; k += 2) {
    step(k, xa, xb);
    if (k + 1 >= steps) break;
    step(k + 1, xb, xa);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ void fill_u32_kernel(unsigned* p, long long n, unsigned v) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

struct GridCache {
  int device = -1;
  int grid[2] = {-1, -1};
};
GridCache g_grid;

template <int D>
int grid_for() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (g_grid.device != dev) {
    g_grid = GridCache{};
    g_grid.device = dev;
  }
  int& slot = g_grid.grid[D == 128];
  if (slot < 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)window_fused_kernel<D>, kThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    slot = per_cu >= 1 ? cus : 0;
  }
  return slot;
}

template <int D>
hipError_t launch_t(const Launch& a, const void* Q, const void* K, unsigned* ex, unsigned* status, float* votes,
                    float* row_stats, hipStream_t st) {
  const int grid = grid_for<D>();
  if (grid <= 0) return hipErrorNotSupported;
  Launch la = a;
  const __bf16* q = (const __bf16*)Q;
  const __bf16* k = (const __bf16*)K;
  void* args[] = {&la, &q, &k, &ex, &status, &votes, &row_stats};
  return hipLaunchCooperativeKernel((const void*)window_fused_kernel<D>, dim3(grid), dim3(kThreads), args, 0, st);
}

}  // namespace

int fused_positions(int W, int D) {
  (void)D;
  return W <= 32 ? kS : 0;
}

int fused_grid(int W, int D) {
  if (W > 32) return 0;
  if (D == 128) return grid_for<128>();
  if (D == 64) return grid_for<64>();
  return 0;
}

int fused_exchange_bytes() { return kHeadRec; }

hipError_t launch_fused_scoring(const Launch& a, const void* Q, const void* K, unsigned* ex, unsigned* status,
                                float* votes, float* row_stats, hipStream_t st) {
  if (a.W > 32 || a.S != kS) return hipErrorNotSupported;
  if (a.D == 128) return launch_t<128>(a, Q, K, ex, status, votes, row_stats, st);
  if (a.D == 64) return launch_t<64>(a, Q, K, ex, status, votes, row_stats, st);
  return hipErrorNotSupported;
}

hipError_t launch_fill_u32(unsigned* p, long long n, unsigned v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace kvsel
