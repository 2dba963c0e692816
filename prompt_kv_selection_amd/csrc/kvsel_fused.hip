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
// twice.  Here the exponentials of a chunk stay in VGPRs until the head's row
// statistics have been agreed on across the workgroups that hold its chunks.
//
// Schedule.  One workgroup per CU, all resident together (checked at start).
// Work proceeds in rounds; in a round every workgroup owns one chunk of
// S = 512 positions of some head (heads_per_round heads, each split over
// fc = ceil(L / S) workgroups).  A round's logits wait two rounds for the
// head-wide statistics: in step k the workgroup streams round k into one of
// two register sets (and reduces it to the chunk's own row statistics), votes
// round k - 2 from a third set kept in LDS, then moves round k - 1 from the
// other register set into LDS.  The exchange of round k - 2 overlapped the
// streaming of rounds k - 1 and k.
//
// Exchange.  A vote is sum_i exp2(x_ij - M_i) / Z_i.  With the chunk's own
// maxima m_i the streamed exponentials are u_ij = exp2(x_ij - m_i) and
// z_i = sum_j u_ij, and the vote is sum_i u_ij * exp2(m_i - M_i) / Z_i with
// M_i = max over chunks of m_i and Z_i = sum over chunks of
// z_i * exp2(m_i - M_i).  So one exchange per round suffices: every workgroup
// stores (m_i, z_i) of its chunk as one 64-bit word per row into its own slot
// (no atomics), and while the next rounds stream reads the fc slots of the
// head and merges them in a fixed order (the result does not depend on arrival order).  The
// lowest mantissa bit of every published m_i is set, and the same tagged m_i
// is used for the chunk's exponentials, so a set bit marks a written word in a
// slot array that starts zeroed.
//
// Roles inside a workgroup.  Eight streaming waves, an exchange wave, a
// memory wave and a publisher wave.
//  * Streaming waves read global memory only through direct-to-LDS loads of
//    K tiles (global_load_lds_dwordx4, 1 KB contiguous per instruction) into a
//    private 32-row tile buffer, one tile in flight per wave: the next tile is
//    issued as soon as the current one's operands are in registers.  Eight
//    tiles (64 KB) in flight per CU keep HBM busy; deeper queues would only
//    lengthen the wait of every other memory access of the CU, the exchange's
//    included.  They
//    form the logits on MFMA (v_mfma_f32_32x32x16_bf16, Qwin rows from LDS),
//    exponentials and votes, and talk to the other two waves through LDS.
//  * The exchange wave only reads the head's slots and merges them, so a
//    slow exchange never holds up the publication of the next round.
//  * The publisher wave stores the chunk's slot as soon as the streaming
//    waves have their row statistics.
//  * The memory wave loads Qwin (double buffered in LDS) and writes the
//    votes.
// All exchange accesses are agent scope (they bypass the per-XCD L2); every
// wait is bounded, and a timed-out wait records a flag and marks the head's
// votes NaN, so the grid always drains.
//
// LDS tiles use an XOR swizzle (piece c of row r stored at c ^ (r % pieces))
// so that the direct-to-LDS writes stay contiguous and the MFMA operand reads
// are free of bank conflicts.

#include <math.h>

#include <algorithm>

#include "kvsel_internal.h"

// Instrumentation hooks in the streaming waves (step k, point 0..3) and the
// controller (step k, point 4..7); empty unless a profiling build defines them.
#ifndef KVSEL_FUSED_MARK
#define KVSEL_FUSED_MARK(k, point)
#endif
#ifndef KVSEL_FUSED_CTL_MARK
#define KVSEL_FUSED_CTL_MARK(k, point)
#endif

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr float kNegBig = -1.0e30f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr int kSW = 8;                    // streaming waves (two per SIMD)
constexpr int kThreads = (kSW + 3) * 64;  // plus the exchange, memory and publisher waves
constexpr int kTT = 2;                    // 32-position tiles per streaming wave per round
constexpr int kNBuf = 1;                  // K tiles in flight per streaming wave
constexpr int kS = kSW * kTT * 32;        // positions per workgroup per round
constexpr int kLag = 2;                   // steps between streaming a round and voting it
// Round-indexed LDS buffers and arrival counters.  Streaming waves of a
// workgroup are at most kLag + 1 rounds apart (a wave in step k has the
// statistics of round k - kLag - 1, which needed every wave's round
// k - kLag - 1), so kNR > kLag + 1 rounds never share an entry while in use.
constexpr int kNR = 4;
static_assert(kNR > kLag + 1, "round-indexed entries outlive the skew of the waves");
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

// ---- reductions over the 32 lanes of each half-wave on the VALU (DPP):
// row_shr 1, 2, 4, 8 inside each 16-lane row, then row_bcast15 into rows 1
// and 3; the results are in lanes 31 (half 0) and 63 (half 1).  Lanes whose
// DPP source is out of range take the neutral value.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_f(float neutral, float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(neutral), __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_f<0x111>(v, v));
  v = fmaxf(v, dpp_f<0x112>(v, v));
  v = fmaxf(v, dpp_f<0x114>(v, v));
  v = fmaxf(v, dpp_f<0x118>(v, v));
  return fmaxf(v, dpp_f<0x142, 0xA>(v, v));
}
__device__ __forceinline__ float half_sum(float v) {
  v += dpp_f<0x111>(0.f, v);
  v += dpp_f<0x112>(0.f, v);
  v += dpp_f<0x114>(0.f, v);
  v += dpp_f<0x118>(0.f, v);
  return v + dpp_f<0x142, 0xA>(0.f, v);
}

// Merge (mo, zo) into (m, z): running maximum in base 2 and the sum of
// exponentials rescaled to it.
__device__ __forceinline__ void lse_merge(float& m, float& z, float mo, float zo) {
  const float d = mo - m;
  const float e = exp2_fast(-fabsf(d));
  z = d > 0.f ? fmaf(z, e, zo) : fmaf(zo, e, z);
  m = fmaxf(m, mo);
}

// ---- exchange slots in the workspace, zeroed per call: per (sequence,
// head, chunk) 32 words of 64 bits, word i = (tagged m_i bits, z_i bits).
constexpr int kSlotWords = 32;
__device__ __forceinline__ float tag_max(float m) { return __uint_as_float(__float_as_uint(m) | 1u); }
__device__ __forceinline__ unsigned long long pack_slot(float m, float z) {
  return ((unsigned long long)__float_as_uint(z) << 32) | __float_as_uint(m);
}

// ---- LDS signalling between the waves of the workgroup.  A wave's LDS
// operations complete in order, so data written before a signal is visible to
// a wave that has seen the signal.
struct Sync {
  // Streaming-wave arrivals (row statistics, votes), counted per round
  // modulo kNR: a streaming wave can run up to kLag + 1 rounds ahead of
  // another, so a single running count could reach a round's target early.
  unsigned cnt_b[kNR], cnt_c[kNR];
  unsigned q_ready;                // Qwin of rounds < q_ready is in LDS
  unsigned s_ready;                // vote scales of rounds < s_ready are in LDS
  unsigned v_done;                 // votes of rounds < v_done have left LDS
  unsigned timeout;
  unsigned abort;                  // the grid is not all resident: every wave leaves its loop
};
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned lds_get(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until *p >= target.  Returns false if the workgroup is aborting (the
// caller then leaves its loop); a wait past the spin bound records a timeout
// and returns true, so the grid always drains.
__device__ __forceinline__ bool lds_wait_ge(Sync* sy, unsigned* p, unsigned target) {
  long spins = 0;
  while (lds_get(p) < target) {
    if (lds_get(&sy->abort)) return false;
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpin) {
      sy->timeout = 1;
      break;
    }
  }
  asm volatile("" ::: "memory");
  return !lds_get(&sy->abort);
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

// Issue the loads of the 32-row tile starting at row p0 of a head's K (rows
// past L repeat row L - 1) into an LDS tile: one scalar base address and a
// 32-bit offset per lane.  Piece c of tile row r lands at r * PR + (c ^ (r % PR)).
template <int D>
__device__ __forceinline__ void issue_tile(const __bf16* __restrict__ kh, int L, int p0, const uint4* lds_tile,
                                           int lane) {
  using G = TileGeom<D>;
  const unsigned base = (unsigned)(uintptr_t)lds_tile;
  // The base is wave-uniform; make that explicit for the scalar operand
  // (readfirstlane returns int: each half is widened as unsigned).
  const unsigned long long fa = (unsigned long long)(uintptr_t)(kh + (long long)p0 * D);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(fa >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)fa);
  const __bf16* first = (const __bf16*)(((unsigned long long)hi << 32) | (unsigned long long)lo);
  const int rows = min(32, L - p0);
#pragma unroll
  for (int i = 0; i < G::NL; ++i) {
    const int piece = i * 64 + lane;
    const int r = piece / G::PR;
    const int c = (piece % G::PR) ^ (r & (G::PR - 1));
    const unsigned off = (unsigned)((min(r, rows - 1) * G::PR + c) * 16);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(base + i * 1024)), "v"(off), "s"(first)
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

// The K tiles one streaming wave owns in a round: kTT consecutive 32-row
// tiles of one head from row p0 (rows past L repeat row L - 1).  A wave's
// tiles form one sequence (its existing tiles of round k, then of round
// k + 1, ...) through its single buffer: at most one tile is outstanding, and
// at the start of step k it is the wave's first tile of round k, if any.
static_assert(kNBuf == 1, "one tile in flight per streaming wave");
struct WaveTiles {
  const __bf16* kh;  // the head's K
  int L, p0;
  bool on;           // the workgroup owns the round
};

template <int D>
__device__ __forceinline__ WaveTiles wave_tiles(const Launch& a, const __bf16* __restrict__ K, int k, int wave) {
  WaveTiles t{K, 0, 0, false};
  const Work w = round_work(a, k);
  if (!w.on) return t;
  const Seg& s = a.seg[w.e];
  t.kh = K + s.kv_off + (long long)w.h * s.L * D;
  t.L = s.L;
  t.p0 = w.c * kS + wave * kTT * 32;
  t.on = true;
  return t;
}

template <int D>
__device__ __forceinline__ void issue_wave_tile(const WaveTiles& wt, int t, uint4* buf, int& issued) {
  if (wt.on && wt.p0 + 32 * t < wt.L) {
    issue_tile<D>(wt.kh, wt.L, wt.p0 + 32 * t, buf, threadIdx.x & 63);
    ++issued;
  }
}

// Phase A (streaming wave): the logits of round k, twice from the same
// operands.  Q.K^T (a lane per position, its window rows in registers) is
// kept in x for the votes; K.Q^T (a lane per window row, positions in
// registers) gives the row statistics with lane-local reductions: the
// maximum and the sum of exp2 over the lane's positions, then one merge of
// the two half-waves, which hold the same rows over different positions.
// Logits stay unscaled; exponents are fma(l, scale2, -m) with m already
// scaled.  The wave's (max, sum) per row go to LDS.  The buffer is refilled
// with the wave's next tile as soon as the operands are read.
// With kLse the row statistics are given, and only Q.K^T is formed.
template <int D, bool kLse>
__device__ __forceinline__ void phase_stream(const Launch& a, int k, const WaveTiles& cur, const WaveTiles& nxt,
                                             uint4* buf, const uint4* __restrict__ qbuf,
                                             f32x16 (&x)[kTT], int& issued, int& consumed, float* s_maxp,
                                             float* s_zp, Sync* sy) {
  using G = TileGeom<D>;
  const int L = cur.L, W = a.W, P = L - W;
  const float sc = a.scale2;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), n = lane & 31, g = lane >> 5;
  if (!lds_wait_ge(sy, &sy->q_ready, (unsigned)k + 1)) return;
  float mrow = kNegBig, zrow = 0.f;  // row n over this lane's positions of the round
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    const int p0 = cur.p0 + 32 * t;
    if (p0 < L) {
      wait_tiles<D>(issued - consumed - 1);
      const uint4* tile = buf;
      // Operands in groups of four k-steps: their LDS reads are issued
      // together, and the registers of a group are free for the next.
      constexpr int kGroup = 4;
      f32x16 acc = {}, act = {};
#pragma unroll
      for (int k0 = 0; k0 < D / 16; k0 += kGroup) {
        bf16x8 qa[kGroup], kb[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          const int off = n * G::PR + ((2 * (k0 + u) + g) ^ (n & (G::PR - 1)));
          kb[u] = __builtin_bit_cast(bf16x8, tile[off]);
          qa[u] = __builtin_bit_cast(bf16x8, qbuf[off]);
        }
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[u], kb[u], acc, 0, 0, 0);
          if constexpr (!kLse) act = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[u], qa[u], act, 0, 0, 0);
        }
      }
      // Every operand has been read: refill the buffer before the VALU work,
      // with tile t + 1 of this round or else the first of the next.
      lds_fence();
      ++consumed;
      if (t + 1 < kTT && p0 + 32 < L)
        issue_wave_tile<D>(cur, t + 1, buf, issued);
      else
        issue_wave_tile<D>(nxt, 0, buf, issued);
      x[t] = acc;
      if constexpr (kLse) continue;
      // act[r]: row n at position p0 + acc_row(r, g).  Only a tile that
      // reaches the window or the end of the prompt needs the mask.
      float tm = kNegBig;
      if (p0 + 32 <= P) {
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, act[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = p0 + acc_row(r, g);
          if (!(j < L && j <= P + n)) act[r] = -INFINITY;
          tm = fmaxf(tm, act[r]);
        }
      }
      const float tms = tm * sc;
      float tz = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) tz += exp2_fast(fmaf(act[r], sc, -tms));
      lse_merge(mrow, zrow, tms, tz);
    } else if (t == 0) {  // no tile of this round: the next round's first
      issue_wave_tile<D>(nxt, 0, buf, issued);
    }
  }
  if constexpr (!kLse) {
    // Lane n and lane n + 32 merge (half 0, half 1) in that order.
    const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mrow), __float_as_uint(mrow), false, false);
    const auto pz = __builtin_amdgcn_permlane32_swap(__float_as_uint(zrow), __float_as_uint(zrow), false, false);
    float m = __uint_as_float(pm[0]), z = __uint_as_float(pz[0]);
    lse_merge(m, z, __uint_as_float(pm[1]), __uint_as_float(pz[1]));
    if (g == 0) {
      s_maxp[wave * 32 + n] = m;
      s_zp[wave * 32 + n] = z;
    }
  }
  lds_add(&sy->cnt_b[k % kNR]);
}

// The wave's logits of a round kept in LDS between its two steps:
// element 4q + e of tile t of lane l is component e of float4 (t * 4 + q) * 64
// + l (each instruction moves 1 KB contiguous, free of bank conflicts).
__device__ __forceinline__ void store_x(float4* sx, const f32x16 (&x)[kTT]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < kTT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      sx[(t * 4 + q) * 64 + lane] = make_float4(x[t][4 * q], x[t][4 * q + 1], x[t][4 * q + 2], x[t][4 * q + 3]);
}

// Phase B (streaming wave): votes of round k's positions into LDS from the
// logits kept in LDS and the head-wide row log-normalisers in base 2
// (M_i + log2 Z_i, so that exp2(x - M_i - log2 Z_i) is the probability).
// Prefix positions are visible to every window row, so no mask is needed;
// rows past W have zero logits and an infinite log-normaliser.  Equal key
// rows give bit-equal votes.
__device__ __forceinline__ void phase_votes(const Launch& a, int k, const float4* sx, const float* s_m,
                                            float* s_votes, Sync* sy) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), n = lane & 31, g = lane >> 5;
  const float sc = a.scale2;
  if (!lds_wait_ge(sy, &sy->s_ready, (unsigned)k + 1)) return;
  if (!lds_wait_ge(sy, &sy->v_done, (unsigned)(k >= 1 ? k - 1 : 0))) return;  // round k - 2 left this buffer
  float mr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) mr[r] = s_m[acc_row(r, g)];
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    float xt[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = sx[(t * 4 + q) * 64 + lane];
      xt[4 * q] = v.x;
      xt[4 * q + 1] = v.y;
      xt[4 * q + 2] = v.z;
      xt[4 * q + 3] = v.w;
    }
    float tot = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) tot += exp2_fast(fmaf(xt[r], sc, -mr[r]));
    const auto pt = __builtin_amdgcn_permlane32_swap(__float_as_uint(tot), __float_as_uint(tot), false, false);
    const float v = __uint_as_float(pt[0]) + __uint_as_float(pt[1]);
    if (g == 0) s_votes[wave * kTT * 32 + t * 32 + n] = v;
  }
  lds_add(&sy->cnt_c[k % kNR]);
}

// Controller: start loading Qwin of round k into an LDS buffer with
// direct-to-LDS loads, swizzled like K (rows W..31 repeat row W - 1 until
// ctl_finish_q clears them).  Returns whether the round is owned.
template <int D>
__device__ __forceinline__ bool ctl_issue_q(const Launch& a, int k, const __bf16* __restrict__ Q, uint4* qbuf) {
  const Work w = round_work(a, k);
  if (!w.on) return false;
  issue_tile<D>(Q + (long long)w.hs * a.W * D, a.W, 0, qbuf, threadIdx.x & 63);
  return true;
}

// Controller, once the Qwin loads have landed: rows W..31 become zero.
template <int D>
__device__ __forceinline__ void ctl_finish_q(int W, uint4* qbuf) {
  using G = TileGeom<D>;
  for (int p = W * G::PR + (int)(threadIdx.x & 63); p < G::PIECES; p += 64) qbuf[p] = make_uint4(0u, 0u, 0u, 0u);
}


// Exchange wave: the head-wide row statistics of round r from the fc slots of
// its head.  Lane l handles row l % 32 over the slots of parity l / 32 (the
// words of rows >= W are never written and never read), kBatch slots per
// lane per pass, all loads of a pass in flight together.  A pass is reread
// until every word carries its tag (bounded).  Within a pass the maximum
// comes first and the rescaled sum follows in slot order; passes, then the
// two halves, are merged in order, so every workgroup of the head computes
// bit-identical statistics.
__device__ __forceinline__ bool ctl_head_stats(const Launch& a, const Work& w, const unsigned long long* ex,
                                               float& M, float& Z) {
  const Seg& s = a.seg[w.e];
  const int fc = s.fc, W = a.W;
  const int lane = threadIdx.x & 63, i = lane & 31, half = lane >> 5;
  const unsigned long long* base = ex + (s.fslot_base + (long long)w.h * fused_slot_stride(fc)) * kSlotWords;
  float mm = kNegBig, zz = 0.f;
  bool ok = true;
  constexpr int kBatch = 32;  // words per lane in flight
  static_assert(2 * kBatch == 64, "a pass reads the slots of one padding unit (fused_slot_stride)");
  // Word (slot c0 + 2u + half, row i) sits at a wave-uniform base plus a
  // 32-bit lane offset.  Slots up to the padded stride exist, so every load
  // of a pass is in bounds; those past fc are ignored.
  const unsigned lane_off = (unsigned)(half * kSlotWords + i) * 8u;
  for (int c0 = 0; c0 < fc; c0 += 2 * kBatch) {
    unsigned long long v[kBatch];
    const char* pass_base = (const char*)(base + (long long)c0 * kSlotWords);
    long spins = 0;
    for (;;) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[u] = __hip_atomic_load((const unsigned long long*)(pass_base + lane_off + u * 2 * kSlotWords * 8),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool valid = true;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int c = c0 + 2 * u + half;
        if (c < fc && i < W) valid = valid && (v[u] & 1ull) != 0;
      }
      if (__ballot(!valid) == 0) break;
      if (++spins > kSpin) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    float bm = kNegBig;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (c0 + 2 * u + half < fc && i < W) bm = fmaxf(bm, __uint_as_float((unsigned)v[u]));
    float bz = 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (c0 + 2 * u + half < fc && i < W)
        bz = fmaf(__uint_as_float((unsigned)(v[u] >> 32)), exp2_fast(__uint_as_float((unsigned)v[u]) - bm), bz);
    lse_merge(mm, zz, bm, bz);
  }
  const float mo = __shfl_xor(mm, 32), zo = __shfl_xor(zz, 32);
  if (half == 0) lse_merge(mm, zz, mo, zo);
  M = mm;
  Z = zz;
  return __ballot(!ok) == 0;
}

// Exchange wave: the head statistics of each round in turn from the slots
// (overlapping the streaming of the next rounds) into the round's statistics
// buffer, once the votes of round j - kNR, which read the same buffer, are
// done.  s_ready = j + 1 announces round j.
template <int D>
__device__ void ctl_exchange(const Launch& a, unsigned long long* __restrict__ ex, unsigned* __restrict__ status,
                             float* __restrict__ row_stats, float (*s_m)[32], Sync* sy) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  unsigned votes_due[kNR] = {};  // owned rounds up to j - kNR, per residue: their votes must be done
  for (int j = 0; j < a.rounds; ++j) {
    const Work w = round_work(a, j);
    if (j >= kNR && round_work(a, j - kNR).on) ++votes_due[j % kNR];
    if (w.on) {
      float M, Z;
      const bool ok = ctl_head_stats(a, w, ex, M, Z);
      if (!ok && lane == 0) raise_error(a.err, kErrExchangeWait);
      if (__ballot(ok && lane < W && !stats_ok(M, Z)) != 0 && lane == 0) raise_error(a.err, kErrNonFinite);
      if (!lds_wait_ge(sy, &sy->cnt_c[j % kNR], kSW * votes_due[j % kNR])) return;
      if (lane < W) {
        s_m[j % kNR][lane] = ok ? M + __log2f(Z) : __builtin_nanf("");
        if (row_stats != nullptr && w.c == 0) {
          float* rs = row_stats + ((long long)w.hs * W + lane) * 2;
          rs[0] = M * kLn2;
          rs[1] = Z;
        }
      } else if (lane < 32) {  // rows past W: zero queries, dropped by the infinite normaliser
        s_m[j % kNR][lane] = INFINITY;
      }
    }
    lds_set(&sy->s_ready, (unsigned)(j + 1));
    KVSEL_FUSED_CTL_MARK(j, 4);
  }
}

// Exchange wave with the row statistics given as natural-log log-sum-exps
// (lse[sequence][head][W]): the base-2 log-normaliser is lse * log2(e).
// Each round's values are loaded one round ahead.
__device__ void ctl_lse(const Launch& a, const float* __restrict__ lse, float (*s_m)[32], Sync* sy) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  auto load = [&](int r) -> float {
    const Work w = round_work(a, r);
    return (w.on && lane < W) ? lse[(long long)w.hs * W + lane] : 0.f;
  };
  unsigned votes_due[kNR] = {};  // as in ctl_exchange
  float next = load(0);
  for (int j = 0; j < a.rounds; ++j) {
    const Work w = round_work(a, j);
    if (j >= kNR && round_work(a, j - kNR).on) ++votes_due[j % kNR];
    const float cur = next;
    next = load(j + 1);
    if (__ballot(w.on && lane < W && !isfinite(cur)) != 0 && lane == 0) raise_error(a.err, kErrNonFinite);
    if (w.on) {
      if (!lds_wait_ge(sy, &sy->cnt_c[j % kNR], kSW * votes_due[j % kNR])) return;
      if (lane < 32) s_m[j % kNR][lane] = lane < W ? cur * kLog2e : INFINITY;  // rows past W drop out
    }
    lds_set(&sy->s_ready, (unsigned)(j + 1));
  }
}

// Publisher wave.  Once round k's phase A is done, the chunk's (m, z) of
// round k, merged from the streaming waves' pairs, goes to its slot.  A wave
// of its own, so that publication never waits behind a Qwin load or a votes
// write (which waits for the previous exchange).
__device__ void ctl_publish(const Launch& a, unsigned long long* __restrict__ ex, float (*s_maxp)[kSW * 32],
                            float (*s_zp)[kSW * 32], Sync* sy) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  unsigned on_b[kNR] = {};  // owned rounds awaited so far, per residue
  for (int k = 0; k < a.rounds; ++k) {
    const Work w0 = round_work(a, k);
    if (!w0.on) continue;
    ++on_b[k % kNR];
    if (!lds_wait_ge(sy, &sy->cnt_b[k % kNR], kSW * on_b[k % kNR])) return;
    if (lane < W) {
      // Merge the waves' (max, sum) pairs in wave order against the tagged
      // chunk maximum.
      float m = s_maxp[k % kNR][lane];
#pragma unroll
      for (int v = 1; v < kSW; ++v) m = fmaxf(m, s_maxp[k % kNR][v * 32 + lane]);
      m = tag_max(m);
      // A wave with no visible position in the row has sum 0 and the
      // sentinel maximum, whose ulp is huge: it adds nothing.
      float zz = 0.f;
#pragma unroll
      for (int v = 0; v < kSW; ++v) {
        const float zv = s_zp[k % kNR][v * 32 + lane];
        if (zv != 0.f) zz += zv * exp2_fast(s_maxp[k % kNR][v * 32 + lane] - m);  // a NaN sum propagates
      }
      const Seg& s = a.seg[w0.e];
      unsigned long long* slot =
          ex + (s.fslot_base + (long long)w0.h * fused_slot_stride(s.fc) + w0.c) * kSlotWords;
      __hip_atomic_store(slot + lane, pack_slot(m, zz), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    KVSEL_FUSED_CTL_MARK(k, 5);
  }
}

// Memory wave.  Step k: (1) Qwin of round k + 2 into the buffer of round k
// once round k's phase A is done; (2) votes of round k - kLag to memory, then
// the votes buffer may be reused (v_done).
template <int D>
__device__ void ctl_memory(const Launch& a, const __bf16* __restrict__ Q, float* __restrict__ votes,
                           uint4 (*qbufs)[TileGeom<D>::PIECES], float (*s_votes)[kS], Sync* sy) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  // Qwin of rounds 0 and 1 was issued before the residency handshake.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  ctl_finish_q<D>(W, qbufs[0]);
  ctl_finish_q<D>(W, qbufs[1]);
  lds_set(&sy->q_ready, 2u);
  unsigned on_b[kNR] = {}, on_c[kNR] = {};  // owned rounds awaited so far, per residue
  for (int k = 0; k < a.rounds + kLag; ++k) {
    const int kv = k - kLag;  // round whose votes leave in this step
    const Work w0 = round_work(a, k), w1 = round_work(a, kv);
    if (w0.on) {
      ++on_b[k % kNR];
      if (!lds_wait_ge(sy, &sy->cnt_b[k % kNR], kSW * on_b[k % kNR])) return;
    }
    if (ctl_issue_q<D>(a, k + 2, Q, qbufs[k & 1])) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      ctl_finish_q<D>(W, qbufs[k & 1]);
    }
    lds_set(&sy->q_ready, (unsigned)(k + 3));
    KVSEL_FUSED_CTL_MARK(k, 6);
    if (w1.on) {
      ++on_c[kv % kNR];
      if (!lds_wait_ge(sy, &sy->cnt_c[kv % kNR], kSW * on_c[kv % kNR])) return;
      const Seg& s = a.seg[w1.e];
      const int P = s.L - W;
      float* vout = votes + s.vote_off + (long long)w1.h * s.vote_ld;
      const int j0 = w1.c * kS;
      for (int i = lane; i < kS; i += 64)
        if (j0 + i < P) vout[j0 + i] = s_votes[kv & 1][i];
    }
    if (kv >= 0) lds_set(&sy->v_done, (unsigned)(kv + 1));  // votes of rounds <= kv are out of LDS
    KVSEL_FUSED_CTL_MARK(k, 7);
  }
}

// Fallback when the grid is not all resident (ABORT): the workgroups take
// whole (segment, head) units from a counter and score each one alone, in
// two passes over its K (row statistics, then votes), so no workgroup ever
// waits for another.  The streaming waves do the passes; every wave of the
// workgroup takes part in each barrier.  Slower than the round schedule,
// same arithmetic.
template <int D>
__device__ __forceinline__ void solo_pass(const Launch& a, const Seg& s, const __bf16* __restrict__ kh, int limit,
                                          bool votes_pass, uint4 (*ring)[TileGeom<D>::PIECES], const uint4* qbuf,
                                          const float* s_m, const float* s_iz, float* vout, float (&m)[16],
                                          float (&z)[16]) {
  using G = TileGeom<D>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int L = s.L, P = L - a.W;
  const int tiles = (limit + 31) / 32;
  const int nw = tiles > wave ? (tiles - wave + kSW - 1) / kSW : 0;  // tiles wave, wave + kSW, ...
  float mr[16], iz[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mr[r] = votes_pass ? s_m[acc_row(r, g)] : 0.f;
    iz[r] = votes_pass ? s_iz[acc_row(r, g)] : 0.f;
  }
  int issued = 0;
  for (; issued < kNBuf && issued < nw; ++issued)
    issue_tile<D>(kh, L, (wave + kSW * issued) * 32, ring[issued % kNBuf], lane);
  for (int i = 0; i < nw; ++i) {
    wait_tiles<D>(issued - i - 1);
    const uint4* tile = ring[i % kNBuf];
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int c = 2 * kk + g;
      const int off = n * G::PR + (c ^ (n & (G::PR - 1)));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qbuf[off]),
                                                    __builtin_bit_cast(bf16x8, tile[off]), acc, 0, 0, 0);
    }
    lds_fence();
    if (issued < nw) {
      issue_tile<D>(kh, L, (wave + kSW * issued) * 32, ring[issued % kNBuf], lane);
      ++issued;
    }
    const int j = (wave + kSW * i) * 32 + n;
    if (votes_pass) {
      float tot = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) tot += exp2_fast(acc[r] * a.scale2 - mr[r]) * iz[r];
      const float other = __shfl_xor(tot, 32);
      const float v = g == 0 ? tot + other : other + tot;
      if (g == 0 && j < P) vout[j] = v;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, g);
        const float x = (j < L && j <= P + row) ? acc[r] * a.scale2 : -INFINITY;
        const float d = x - m[r];
        const float e = exp2_fast(-fabsf(d));
        z[r] = d > 0.f ? fmaf(z[r], e, 1.f) : z[r] + e;
        m[r] = fmaxf(m[r], x);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D>
__device__ void solo_heads(const Launch& a, const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                           unsigned* __restrict__ counter, float* __restrict__ votes, float* __restrict__ row_stats,
                           uint4 (*s_ring)[kNBuf][TileGeom<D>::PIECES], uint4* qbuf, float* s_maxp, float* s_zp,
                           float* s_m, float* s_iz) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, W = a.W;
  const bool streams = wave < kSW;
  const Seg& last = a.seg[a.n - 1];
  const unsigned units = (unsigned)(last.row0 + last.nh);
  __shared__ unsigned s_unit;
  for (;;) {
    if (threadIdx.x == 0) s_unit = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned u = s_unit;
    __syncthreads();
    if (u >= units) break;
    const int e = find_seg<kFieldRow>(a, (int)u);
    const Seg& s = a.seg[e];
    if (s.L < s.C) continue;  // bypass: nothing to score
    const int h = s.h0 + ((int)u - s.row0);
    const int hs = s.b * a.heads + h;
    if (wave == 0) {
      issue_tile<D>(Q + (long long)hs * W * D, W, 0, qbuf, lane);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      ctl_finish_q<D>(W, qbuf);
    }
    __syncthreads();
    const __bf16* kh = K + s.kv_off + (long long)h * s.L * D;
    float m[16], z[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      m[r] = kNegBig;
      z[r] = 0.f;
    }
    if (streams) solo_pass<D>(a, s, kh, s.L, false, s_ring[wave], qbuf, s_m, s_iz, nullptr, m, z);
    // This wave's (max, sum) per row, then the waves merged in order.
    if (streams) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float mh0 = half_max(m[r]);
      const float m0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(mh0), 31));
      const float m1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(mh0), 63));
      const float mh = g == 0 ? m0 : m1;
      const float zz = half_sum(z[r] != 0.f ? z[r] * exp2_fast(m[r] - mh) : 0.f);  // a NaN sum propagates
      if ((lane & 31) == 31) {
        s_maxp[wave * 32 + acc_row(r, g)] = mh;
        s_zp[wave * 32 + acc_row(r, g)] = zz;
      }
    }
    }
    __syncthreads();
    if ((int)threadIdx.x < W) {
      const int i = threadIdx.x;
      float M = s_maxp[i];
      for (int v = 1; v < kSW; ++v) M = fmaxf(M, s_maxp[v * 32 + i]);
      float Z = 0.f;
      for (int v = 0; v < kSW; ++v) {
        const float zv = s_zp[v * 32 + i];
        if (zv != 0.f) Z += zv * exp2_fast(s_maxp[v * 32 + i] - M);  // a NaN sum propagates
      }
      s_m[i] = M;
      s_iz[i] = 1.f / Z;
      if (!stats_ok(M, Z)) raise_error(a.err, kErrNonFinite);
      if (row_stats != nullptr) {
        float* rs = row_stats + ((long long)hs * W + i) * 2;
        rs[0] = M * kLn2;
        rs[1] = Z;
      }
    } else if ((int)threadIdx.x < 32) {
      s_m[threadIdx.x] = 0.f;  // rows past W: zero queries, dropped by 1/Z = 0
      s_iz[threadIdx.x] = 0.f;
    }
    __syncthreads();
    float* vout = votes + s.vote_off + (long long)h * s.vote_ld;
    if (streams) solo_pass<D>(a, s, kh, s.L - W, true, s_ring[wave], qbuf, s_m, s_iz, vout, m, z);
    __syncthreads();  // s_m, s_iz and qbuf are rewritten for the next unit
  }
}

template <int D, bool kLse>
__global__ __launch_bounds__(kThreads, 1) void window_fused_kernel(const Launch a, const __bf16* __restrict__ Q,
                                                                  const __bf16* __restrict__ K,
                                                                  const float* __restrict__ lse,
                                                                  unsigned long long* __restrict__ ex,
                                                                  unsigned* __restrict__ status,
                                                                  float* __restrict__ votes,
                                                                  float* __restrict__ row_stats) {
  using G = TileGeom<D>;
  __shared__ uint4 s_ring[kSW][kNBuf][G::PIECES];
  __shared__ uint4 s_q[2][G::PIECES];
  __shared__ float4 s_x[kSW][kTT * 4 * 64];  // each wave's logits of one round
  __shared__ float s_maxp[kNR][kSW * 32], s_zp[kNR][kSW * 32];
  __shared__ float s_m[kNR][32], s_iz[32];
  __shared__ float s_votes[2][kS];
  __shared__ Sync sy;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  unsigned arrived = 0u;
  if (!kLse && wave == kSW && lane == 0) arrived = arrive(status);
  if (threadIdx.x == 0) sy = Sync{};
  __syncthreads();  // afterwards waves meet through LDS flags (and once more at the end)
  // The first K tiles and Qwin of rounds 0 and 1.
  WaveTiles cur{K, 0, 0, false};
  int issued = 0, consumed = 0;
  if (wave < kSW) {
    cur = wave_tiles<D>(a, K, 0, wave);
    issue_wave_tile<D>(cur, 0, s_ring[wave][0], issued);
  } else if (wave == kSW + 1) {
    ctl_issue_q<D>(a, 0, Q, s_q[0]);
    ctl_issue_q<D>(a, 1, Q, s_q[1]);
  }
  if (wave == kSW) {
    if constexpr (kLse)
      ctl_lse(a, lse, s_m, &sy);  // no workgroup waits for another
    else if (decide(status, arrived, a.err, kFlagScoringFallback, a.residency_ticks) == kFusedGo)
      ctl_exchange<D>(a, ex, status, row_stats, s_m, &sy);
    else
      lds_set(&sy.abort, 1u);  // not all resident: every wave leaves its loop
  } else if (wave == kSW + 1) {
    ctl_memory<D>(a, Q, votes, s_q, s_votes, &sy);
  } else if (wave == kSW + 2) {
    if constexpr (!kLse) ctl_publish(a, ex, s_maxp, s_zp, &sy);
  } else {
    uint4* buf = s_ring[wave][0];
    float4* sx = s_x[wave];
    f32x16 xa[kTT], xb[kTT];
    bool on1 = false, on2 = false;  // rounds k - 1 and k - 2 owned
    // Step k streams round k into one register set (with this wave's row
    // statistics), votes round k - 2 from the logits in LDS, then moves round
    // k - 1 from the other register set into LDS; the register sets swap
    // every step.  The exchange of round k - 2 overlapped the streaming of
    // rounds k - 1 and k.
    auto step = [&](int k, f32x16 (&X0)[kTT], f32x16 (&X1)[kTT]) {
      KVSEL_FUSED_MARK(k, 0);
      const WaveTiles nxt = wave_tiles<D>(a, K, k + 1, wave);
      if (cur.on) {
        phase_stream<D, kLse>(a, k, cur, nxt, buf, s_q[k & 1], X0, issued, consumed, s_maxp[k % kNR],
                              s_zp[k % kNR], &sy);
      } else {
        issue_wave_tile<D>(nxt, 0, buf, issued);  // nothing was outstanding
      }
      KVSEL_FUSED_MARK(k, 1);
      if (on2) phase_votes(a, k - 2, sx, s_m[(k - 2) % kNR], s_votes[(k - 2) & 1], &sy);
      KVSEL_FUSED_MARK(k, 2);
      if (on1) store_x(sx, X1);  // after the votes above have read sx (LDS order within the wave)
      KVSEL_FUSED_MARK(k, 3);
      on2 = on1;
      on1 = cur.on;
      cur = nxt;
    };
    const int steps = a.rounds + kLag;
    for (int k = 0; k < steps; k += 2) {
      step(k, xa, xb);
      if (k + 1 >= steps || lds_get(&sy.abort)) break;
      step(k + 1, xb, xa);
      if (lds_get(&sy.abort)) break;
    }
  }
  // Every wave's loads have landed before LDS is reused or the wave ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (!kLse) {
    if (sy.abort) {  // not all resident: whole heads, one workgroup each
      solo_heads<D>(a, Q, K, status + 3, votes, row_stats, s_ring, s_q[0], s_maxp[0], s_zp[0], s_m[0], s_iz);
      return;
    }
  }
  if (threadIdx.x == 0 && sy.timeout) raise_error(a.err, kErrLdsWait);
}

__global__ void fill_u32_kernel(unsigned* p, long long n, unsigned v) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Zero up to kZeroRanges ranges of 16-byte units in one launch (n[] in units).
struct ZeroUnits {
  uint4* p[kZeroRanges];
  long long n[kZeroRanges];
};
__global__ void zero_kernel(const ZeroUnits z) {
  long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
#pragma unroll
  for (int r = 0; r < kZeroRanges; ++r) {
    if (i < z.n[r]) {
      z.p[r][i] = make_uint4(0u, 0u, 0u, 0u);
      return;
    }
    i -= z.n[r];
  }
}

// Validating mode: any non-finite element among n 16-byte units.
__global__ void check_finite_kernel(const uint4* __restrict__ p, long long n, int bf16, unsigned* err) {
  bool bad = false;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const uint4 u = p[i];
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (bf16)  // two bf16 values per word: exponent bits all ones
        bad = bad || (w[q] & 0x7F80u) == 0x7F80u || (w[q] & 0x7F800000u) == 0x7F800000u;
      else
        bad = bad || (w[q] & 0x7F800000u) == 0x7F800000u;
    }
  }
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) raise_error(err, kErrNonFinite);
}

// Validating mode for float32 arrays of any length and 4-byte alignment
// (the handed-over log-sum-exps): scalar loads, every element checked.
__global__ void check_finite_f32_kernel(const float* __restrict__ p, long long n, unsigned* err) {
  bool bad = false;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    bad = bad || (__float_as_uint(p[i]) & 0x7F800000u) == 0x7F800000u;
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) raise_error(err, kErrNonFinite);
}

struct GridCache {
  int device = -1;
  int grid[2][2] = {{-1, -1}, {-1, -1}};
};
GridCache g_grid;

template <int D, bool kLse>
int grid_for() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (g_grid.device != dev) {
    g_grid = GridCache{};
    g_grid.device = dev;
  }
  int& slot = g_grid.grid[kLse][D == 128];
  if (slot < 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)window_fused_kernel<D, kLse>, kThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    slot = per_cu >= 1 ? cus : 0;
  }
  return slot;
}

template <int D, bool kLse>
hipError_t launch_t(const Launch& a, const void* Q, const void* K, const float* lse, unsigned long long* ex,
                    unsigned* status, float* votes, float* row_stats, hipStream_t st) {
  const int grid = grid_for<D, kLse>();
  if (grid <= 0) return hipErrorNotSupported;
  Launch la = a;
  const __bf16* q = (const __bf16*)Q;
  const __bf16* k = (const __bf16*)K;
  hipLaunchKernelGGL((window_fused_kernel<D, kLse>), dim3(grid), dim3(kThreads), 0, st, la, q, k, lse, ex, status,
                     votes, row_stats);
  return hipGetLastError();
}

}  // namespace

int fused_positions(int W, int D) {
  (void)D;
  return W <= 32 ? kS : 0;
}

int fused_grid(int W, int D) {
  if (W > 32) return 0;
  // The variant with given row statistics has the same resources.
  if (D == 128) return grid_for<128, false>();
  if (D == 64) return grid_for<64, false>();
  return 0;
}

int fused_exchange_bytes() { return kSlotWords * 8; }

hipError_t launch_fused_scoring(const Launch& a, const void* Q, const void* K, const float* lse, unsigned* ex,
                                unsigned* status, float* votes, float* row_stats, hipStream_t st) {
  if (a.W > 32 || a.S != kS) return hipErrorNotSupported;
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(ex);
  if (lse != nullptr) {
    if (a.D == 128) return launch_t<128, true>(a, Q, K, lse, slots, status, votes, nullptr, st);
    if (a.D == 64) return launch_t<64, true>(a, Q, K, lse, slots, status, votes, nullptr, st);
    return hipErrorNotSupported;
  }
  if (a.D == 128) return launch_t<128, false>(a, Q, K, nullptr, slots, status, votes, row_stats, st);
  if (a.D == 64) return launch_t<64, false>(a, Q, K, nullptr, slots, status, votes, row_stats, st);
  return hipErrorNotSupported;
}

hipError_t launch_zero(const ZeroRanges& r, hipStream_t st) {
  ZeroUnits z{};
  long long total = 0;
  for (int i = 0; i < kZeroRanges; ++i) {
    if (r.bytes[i] <= 0) continue;
    if ((uintptr_t)r.p[i] % 16 || r.bytes[i] % 16) return hipErrorInvalidValue;
    z.p[i] = (uint4*)r.p[i];
    z.n[i] = r.bytes[i] / 16;
    total += z.n[i];
  }
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, z);
  return hipGetLastError();
}

hipError_t launch_check_finite(const void* p, long long n16, int dtype, unsigned* err, hipStream_t st) {
  if (n16 <= 0) return hipSuccess;
  const long long blocks = std::min<long long>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(check_finite_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint4*)p, n16,
                     dtype == 1 ? 1 : 0, err);
  return hipGetLastError();
}

hipError_t launch_check_finite_f32(const float* p, long long n, unsigned* err, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long long blocks = std::min<long long>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(check_finite_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, err);
  return hipGetLastError();
}

hipError_t launch_fill_u32(unsigned* p, long long n, unsigned v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace kvsel
