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
// slot array that the workgroups clear before the residency decision.
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
//  * The selection wave (when the selection is fused, see below) takes each
//    round's votes out of LDS, writes them, and selects.
// All exchange accesses are agent scope (they bypass the per-XCD L2); every
// wait is bounded, and a timed-out wait records a flag and marks the head's
// votes NaN, so the grid always drains.
//
// Fused selection (web page "SnapKV: selecting the KV cache for long prompts
// with an observation window", sections "pooling spreads a peak into a
// neighbourhood preference" and "one full selection computed from Q and K").
// The chunks of a head are segments of its selection: pooling of width k
// (odd, at most 7) over the prefix votes with zero padding (avg divides by k)
// or the in-range maximum; the C - W prefix positions with the highest pooled
// score, equal scores to the lowest index, ascending, then the W window
// positions; K and V rows gathered with the same indices.  During the
// streaming the selection wave takes each round's votes out of LDS, writes
// them, publishes the chunk's first and last three votes (tagged halo words)
// and stores the pooled scores of its interior positions as radix keys (float
// bits: scores are >= 0) in the chunk's key slot; nothing there waits on
// memory.  After the streaming all waves run the end phase in four steps, each
// waiting only for the same step of the row's other chunks: the edge
// positions and a 64-bin coarse histogram per chunk, the fine histogram inside
// the coarse bin of the threshold tau, the candidates of tau's first digit,
// and the pick (the rest of tau, then each chunk's picks in index order, the
// K/V copy and the window).  Every published word carries count + 1, so a
// written word is never zero and no atomics are needed.  This path is opt-in:
// its end phase costs more device-scope round trips than the separate
// selection kernels take in all.
// Nothing is cleared by a separate launch, with or without the fused
// selection: before it arrives, each workgroup clears its share of the words
// the call publishes (exchange slots, halo, histogram, count and flag words)
// and of the words the selection kernels after it in the call need at zero,
// and the arrival and the residency decision carry a per-call token instead
// of counting from zero.  GO therefore also means every shared word is
// clear.  On ABORT (not all resident) the workgroups take work from
// token-tagged counters instead: the chunks' statistics, then their votes
// (two passes over K), then with the fused selection whole rows'
// selections, each phase waiting only on work already claimed by running
// workgroups.
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
constexpr int kThreads = (kSW + 4) * 64;  // plus the exchange, memory, publisher and selection waves
constexpr int kThreadsPlain = (kSW + 3) * 64;  // without the selection wave
constexpr int kExWave = kSW, kMemWave = kSW + 1, kPubWave = kSW + 2, kSelWave = kSW + 3;
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

// A flag of the call: the tagged word when nothing was cleared before the
// call (the fused selection), else the header's flag word.
__device__ __forceinline__ void flag_error(const Launch& a, const FusedSel& f, unsigned bit) {
  if (f.token != 0ull)
    raise_tagged(f.errw, f.token, bit);
  else
    raise_error(a.err, bit);
}

// Debug builds: an index outside its range is recorded in the call's flags.
__device__ __forceinline__ void fused_debug_check(const Launch& a, const FusedSel& f, bool ok) {
  if constexpr (kDebug)
    if (!ok) flag_error(a, f, kErrIndexRange);
}

__device__ __forceinline__ unsigned long long load64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Token-tagged counters: (tag << 24) | count, where a word whose tag is not
// this call's counts as zero.  Adding returns the count before the add.  An
// add is one atomic add; the call's first add finds another tag there and
// swaps in (tag, n), and adds that reached the old word before that swap are
// made again.  (Counts stay far below 2^24; a carry out of a stale count
// into the tag bits cannot produce this call's tag but by a 2^-40 chance.)
__device__ __forceinline__ unsigned tok_add(unsigned long long* w, unsigned long long tag, unsigned n) {
  for (;;) {
    const unsigned long long old =
        __hip_atomic_fetch_add(w, (unsigned long long)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((old >> 24) == tag) return (unsigned)(old & 0xFFFFFFull);
    unsigned long long cur = old + n;
    while ((cur >> 24) != tag) {
      unsigned long long expect = cur;
      if (__hip_atomic_compare_exchange_strong(w, &expect, (tag << 24) | (unsigned long long)n, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        return 0u;
      cur = expect;
    }
  }
}
__device__ __forceinline__ unsigned tok_count(const unsigned long long* w, unsigned long long tag) {
  const unsigned long long cur = load64(w);
  return (cur >> 24) == tag ? (unsigned)(cur & 0xFFFFFFull) : 0u;
}

// ---- exchange slots in the workspace, cleared per call: per (sequence,
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
  unsigned issued;                 // the clears of the shared words are issued (fused selection)
  unsigned zeroed;                 // every workgroup's shared words are clear (after GO)
  unsigned go;                     // the residency decision (kFusedGo / kFusedAbort), once taken
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
                                           int lane, bool nt = false) {
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
    // Non-temporal (nt, wave-uniform) where the call's K is larger than the
    // last-level cache: each K row is read once, and cached lines would only
    // evict the exchange slots and the votes (measured: 58.5 against 62.4 µs
    // on a 32-head L=32768 layer).  A smaller K stays cached for the
    // selection's copy of the kept rows.
    if (nt)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(base + i * 1024)), "v"(off), "s"(first)
                   : "memory", "m0");
    else
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
  bool nt;           // non-temporal loads
};

template <int D>
__device__ __forceinline__ WaveTiles wave_tiles(const Launch& a, const __bf16* __restrict__ K, int k, int wave) {
  WaveTiles t{K, 0, 0, false, a.k_nt != 0};
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
    issue_tile<D>(wt.kh, wt.L, wt.p0 + 32 * t, buf, threadIdx.x & 63, wt.nt);
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
__device__ __forceinline__ void ctl_exchange(const Launch& a, const FusedSel& f, unsigned long long* __restrict__ ex,
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
      if (!ok && lane == 0) flag_error(a, f, kErrExchangeWait);
      if (__ballot(ok && lane < W && !stats_ok(M, Z)) != 0 && lane == 0) flag_error(a, f, kErrNonFinite);
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
__device__ __forceinline__ void ctl_lse(const Launch& a, const FusedSel& f, const float* __restrict__ lse, float (*s_m)[32],
                        Sync* sy) {
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
    if (__ballot(w.on && lane < W && !isfinite(cur)) != 0 && lane == 0) flag_error(a, f, kErrNonFinite);
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
__device__ __forceinline__ void ctl_publish(const Launch& a, unsigned long long* __restrict__ ex, float (*s_maxp)[kSW * 32],
                            float (*s_zp)[kSW * 32], Sync* sy) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  unsigned on_b[kNR] = {};  // owned rounds awaited so far, per residue
  // The slots this workgroup writes are clear: every workgroup cleared its
  // share before the decision (GO).
  if (!lds_wait_ge(sy, &sy->zeroed, 1u)) return;
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
__device__ __forceinline__ void ctl_memory(const Launch& a, bool write_votes, const __bf16* __restrict__ Q, float* __restrict__ votes,
                           uint4 (*qbufs)[TileGeom<D>::PIECES], float (*s_votes)[kS], Sync* sy) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  // Qwin of rounds 0 and 1 was issued before the residency handshake.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  ctl_finish_q<D>(W, qbufs[0]);
  ctl_finish_q<D>(W, qbufs[1]);
  lds_set(&sy->q_ready, 2u);
  unsigned on_b[kNR] = {}, on_c[kNR] = {};  // owned rounds awaited so far, per residue
  for (int k = 0; k < a.rounds + (write_votes ? kLag : 0); ++k) {
    const int kv = k - kLag;  // round whose votes leave in this step
    const Work w0 = round_work(a, k), w1 = write_votes ? round_work(a, kv) : Work{0, 0, 0, 0, false};
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
    if (write_votes && kv >= 0) lds_set(&sy->v_done, (unsigned)(kv + 1));  // votes of rounds <= kv are out of LDS
    KVSEL_FUSED_CTL_MARK(k, 7);
  }
}

// ===================================================================
// Fused selection
// ===================================================================

__device__ __forceinline__ uint32_t sel_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return b == 0x80000000u ? 0u : b;  // -0 ranks as +0
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
  return v;
}
// Inclusive prefix sum over the lanes of the wave.
__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Pooled score of the centre of a window of 7 (w[3]) for width k (odd,
// 1..7): avg sums the k neighbours (out-of-range ones are the zero padding,
// already in w) in ascending order and divides by k; max takes the maximum
// (out-of-range neighbours are -inf in w).  Unused slots (|offset| > k / 2)
// are -1 for avg (they sort below every score) and -inf for max, so the
// ascending sum of the top k equals the sum of the k neighbours in
// ascending order.
__device__ __forceinline__ float pool7(float (&w)[7], int k, bool mx) {
  if (k == 1) return w[3];
  if (mx) {
    float res = w[3];
#pragma unroll
    for (int t = 0; t < 7; ++t) res = fmaxf(res, w[t]);
    return res;
  }
#pragma unroll
  for (int i = 1; i < 7; ++i)
#pragma unroll
    for (int q = i; q > 0; --q) {
      const float lo = fminf(w[q - 1], w[q]), hi = fmaxf(w[q - 1], w[q]);
      w[q - 1] = lo;
      w[q] = hi;
    }
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < 7; ++t)
    if (t >= 7 - k) sum += w[t];
  return sum / (float)k;
}

// Window of 7 around position j (centre w[3]) of a row of P prefix votes,
// given the value at j + o for |o| <= 3 through `at`; offsets beyond the
// pooling radius are unused.
template <typename At>
__device__ __forceinline__ float pool_at(int j, int P, int k, bool mx, At at) {
  const int r = k >> 1;
  float w[7];
#pragma unroll
  for (int t = 0; t < 7; ++t) {
    const int o = t - 3, q = j + o;
    const bool used = o >= -r && o <= r;
    const bool in = q >= 0 && q < P;
    w[t] = !used ? (mx ? -INFINITY : -1.f) : (in ? at(t) : (mx ? -INFINITY : 0.f));
  }
  return pool7(w, k, mx);
}

// The chunk a workgroup owns in round r, as the selection sees it.
struct SelRound {
  bool own;        // the workgroup owns a chunk in round r
  bool on;         // ... and it holds prefix positions (the chunk takes part in the selection)
  int e, h, c, row, P, nchp, count, L;
  long long sl;    // exchange-slot index of the chunk (slots of a head's chunks are consecutive)
  long long vbase; // element offset of the row in the votes, pooled scores and candidates
};

__device__ __forceinline__ SelRound sel_round(const Launch& a, int r) {
  SelRound q{};
  const Work w = round_work(a, r);
  if (!w.on) return q;
  const Seg& s = a.seg[w.e];
  q.own = true;
  q.e = w.e;
  q.h = w.h;
  q.c = w.c;
  q.L = s.L;
  q.P = s.L - a.W;
  q.nchp = (q.P + kS - 1) / kS;
  q.count = s.C - a.W;
  q.row = s.row0 + (w.h - s.h0);
  q.sl = s.fslot_base + (long long)w.h * fused_slot_stride(s.fc) + w.c;
  q.vbase = s.vote_off + (long long)w.h * s.vote_ld;
  q.on = w.c < q.nchp;
  return q;
}

// Exchange wave: clear this workgroup's share of ranges r0 .. r1 - 1 of
// f.clr.  At kernel start, before any other load of the workgroup is issued,
// the words the call's workgroups publish to each other (exchange, count,
// halo and histogram slots: the first f.clr_early ranges); the arrival
// follows once those stores are done, so GO means every such word is clear,
// and nothing is published before GO.  Right after the arrival, the words
// only later kernels of the call read (clear once the launch ends), so that
// they do not delay the arrival.
__device__ __forceinline__ void sel_clear(const FusedSel& f, int r0, int r1) {
  const int lane = threadIdx.x & 63;
  const long long nwg = gridDim.x;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r < r0 || r >= r1) continue;
    const long long n = f.clr_words[r];
    const long long per = (n + nwg - 1) / nwg;
    const long long lo = per * blockIdx.x, hi = min(n, lo + per);
    for (long long i = lo + lane; i < hi; i += 64) store64(f.clr[r] + i, 0ull);
  }
}
// Arrival: the workgroup's own word takes the call's token (a store: no
// atomics to contend).
__device__ __forceinline__ void sel_arrive(const FusedSel& f) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clears are done
  if ((threadIdx.x & 63) == 0) store64(f.flags + blockIdx.x, f.token);
}

// Exchange wave: the residency decision of the call.  Workgroup 0, once it
// sees every arrival token of this call, decides GO (GO needs every
// workgroup resident, workgroup 0 among them; only one workgroup polls the
// grid's words, the others the decision word alone, so the polling stays
// off the memory system the K stream uses); any workgroup that has waited
// past the bound decides ABORT.  Both are a compare-and-swap of the one
// decision word to this call's token plus the decision, and the first one
// for this token wins, so every workgroup follows the same decision.  The
// wait always ends: ABORT is decided by the bound at the latest.
__device__ __forceinline__ unsigned sel_decide(const Launch& a, const FusedSel& f) {
  const int lane = threadIdx.x & 63;
  unsigned long long* dec = f.flags + kFlagWordsMax;
  const unsigned grid = gridDim.x;
  const long long t0 = wall_clock64();
  for (;;) {
    // The decision word and (workgroup 0) every arrival token, loaded together.
    unsigned long long cur = 0ull;
    if (lane == 0) cur = load64(dec);
    bool mine = blockIdx.x == 0 && !f.force_abort;
    if (blockIdx.x == 0) {
#pragma unroll
      for (int t = 0; t < kFlagWordsMax / 64; ++t) {
        const unsigned i = (unsigned)(lane + 64 * t);
        if (i < grid) mine = mine && load64(f.flags + i) == f.token;
      }
    }
    const bool all = __ballot(!mine) == 0ull;
    cur = ((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((int)(cur >> 32)) << 32) |
          (unsigned)__builtin_amdgcn_readfirstlane((int)cur);
    if ((cur & ~3ull) == f.token) return (unsigned)(cur & 3ull);
    unsigned want = 0u;
    if (all) want = kFusedGo;
    if (want == 0u && (f.force_abort || wall_clock64() - t0 > a.residency_ticks)) want = kFusedAbort;
    if (want != 0u) {
      // The swap's outcome is the decision: ours if it took, else the value
      // that was there (another workgroup's decision for this token).
      unsigned long long now = 0ull;
      if (lane == 0) {
        unsigned long long expect = cur;
        now = __hip_atomic_compare_exchange_strong(dec, &expect, f.token | want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                  ? (f.token | want)
                  : expect;
      }
      now = ((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((int)(now >> 32)) << 32) |
            (unsigned)__builtin_amdgcn_readfirstlane((int)now);
      if ((now & ~3ull) == f.token) return (unsigned)(now & 3ull);
      continue;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Bounded wait of the calling wave (or lane) until pred() holds (pred must
// give a wave-uniform answer when the whole wave waits).  False once fifty
// residency bounds (10 ms) have passed: far beyond any wait of a working
// call, short enough that a broken one drains quickly.
template <typename Pred>
__device__ __forceinline__ bool sel_wait(const Launch& a, Pred pred) {
  const long long t0 = wall_clock64();
  for (;;) {
    if (pred()) return true;
    if (wall_clock64() - t0 > 50 * a.residency_ticks) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Lanes of the wave where pred holds, and those of them below this lane.
__device__ __forceinline__ uint32_t wave_count(bool pred) { return (uint32_t)__popcll(__ballot(pred)); }
__device__ __forceinline__ uint32_t lanes_below(bool pred) {
  const unsigned long long m = __ballot(pred);
  return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Digit of tau in a histogram of nb bins held by the wave (lane l holds
// bins (63 - l) * per .. + per - 1, per = nb / 64, in h[]): the bin holding
// the need-th largest key, and how many keys of that bin are still needed.
// False if the bins add up to less than need.
__device__ __forceinline__ bool find_digit(const uint32_t (&h)[32], int per, uint32_t need, uint32_t& digit,
                                           uint32_t& left) {
  const int lane = threadIdx.x & 63;
  const int base = (63 - lane) * per;
  uint32_t sum = 0u;
#pragma unroll
  for (int t = 0; t < 32; ++t)
    if (t < per) sum += h[t];
  const uint32_t incl = wave_incl_u32(sum), excl = incl - sum;
  const bool here = excl < need && need <= incl;
  const unsigned long long hb = __ballot(here);
  if (hb == 0ull) return false;
  uint32_t d = 0u, n = 0u, cum = excl;
  bool found = false;
#pragma unroll
  for (int t = 31; t >= 0; --t) {
    if (t < per) {
      const bool hit = !found && cum + h[t] >= need;
      if (hit) {
        d = (uint32_t)(base + t);
        n = need - cum;
        found = true;
      }
      cum += h[t];
    }
  }
  const int bl = __builtin_ctzll(hb);
  digit = (uint32_t)__builtin_amdgcn_readlane((int)d, bl);
  left = (uint32_t)__builtin_amdgcn_readlane((int)n, bl);
  return true;
}

// The lane where a running count over the lanes (each lane's value c, in the
// order of the lanes) first reaches need, and how much of that lane's value
// is still needed; false if the values add up to less than need.
__device__ __forceinline__ bool wave_find(uint32_t c, uint32_t need, int& at, uint32_t& left) {
  const uint32_t incl = wave_incl_u32(c), excl = incl - c;
  const unsigned long long hb = __ballot(excl < need && need <= incl);
  if (hb == 0ull) return false;
  at = __builtin_ctzll(hb);
  left = need - (uint32_t)__builtin_amdgcn_readlane((int)excl, at);
  return true;
}

// Pooled scores of a lane's 8 positions (S0 + u) from its window values ext
// (positions S0 - 3 .. S0 + 10).
__device__ __forceinline__ void sel_pool8(const Launch& a, const SelRound& q, const float (&ext)[14], float (&pv)[8]) {
  const int S0 = q.c * kS + (threadIdx.x & 63) * 8;
#pragma unroll
  for (int u = 0; u < 8; ++u) pv[u] = pool_at(S0 + u, q.P, a.kernel, a.pooling == 1, [&](int t) { return ext[u + t]; });
}

// Stage A of a round (selection wave, during the streaming): the chunk's
// votes v (lane * 8 + u of the chunk) go to memory; a chunk holding prefix
// positions publishes its first and last three votes (tagged halo words) and
// stores the pooled scores of every position whose window it holds in its
// key slot.  Nothing here waits for memory, so the streaming never does
// either; the three positions at each edge whose windows reach into a
// neighbour are pooled in the end phase.
__device__ __forceinline__ void sel_stage_a(const Launch& a, const FusedSel& f, const SelRound& q, const float (&v)[8],
                                            float* __restrict__ votes) {
  const int lane = threadIdx.x & 63;
  const int S0 = q.c * kS + lane * 8;  // this lane's first position
  float* vo = votes + q.vbase;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (S0 + u < q.P) vo[S0 + u] = v[u];
  if (!q.on) return;
  if (lane == 0)
#pragma unroll
    for (int t = 0; t < 3; ++t) store64(f.halo + q.sl * kHaloWords + t, (1ull << 32) | __float_as_uint(v[t]));
  if (lane == 63)
#pragma unroll
    for (int t = 0; t < 3; ++t) store64(f.halo + q.sl * kHaloWords + 3 + t, (1ull << 32) | __float_as_uint(v[5 + t]));
  float ext[14];  // positions S0 - 3 .. S0 + 10; lane 0's first three and lane 63's last three are not known yet
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    ext[t] = __shfl_up(v[5 + t], 1);
    ext[11 + t] = __shfl_down(v[t], 1);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) ext[3 + u] = v[u];
  float pv[8];
  sel_pool8(a, q, ext, pv);
  float* ks = f.kslot + q.sl * kS + lane * 8;
  reinterpret_cast<float4*>(ks)[0] = make_float4(pv[0], pv[1], pv[2], pv[3]);
  reinterpret_cast<float4*>(ks)[1] = make_float4(pv[4], pv[5], pv[6], pv[7]);
}

// Selection wave during the streaming: stage A of each owned round once the
// streaming waves have its votes in LDS.  The votes leave LDS first, so the
// streaming waves may reuse the buffer at once.
__device__ __forceinline__ void ctl_select(const Launch& a, const FusedSel& f, float* __restrict__ votes,
                                           float (*s_votes)[kS], Sync* sy) {
  if (!lds_wait_ge(sy, &sy->go, 1u) || lds_get(&sy->go) != kFusedGo) return;
  const int lane = threadIdx.x & 63;
  unsigned on_c[kNR] = {};
  for (int ra = 0; ra < a.rounds; ++ra) {
    const SelRound q = sel_round(a, ra);
    KVSEL_FUSED_MARK(ra, 0);
    if (q.own) {
      ++on_c[ra % kNR];
      if (!lds_wait_ge(sy, &sy->cnt_c[ra % kNR], kSW * on_c[ra % kNR])) return;
      KVSEL_FUSED_MARK(ra, 1);
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = s_votes[ra & 1][lane * 8 + u];
      lds_set(&sy->v_done, (unsigned)(ra + 1));  // the votes of rounds <= ra have left LDS
      sel_stage_a(a, f, q, v, votes);
      KVSEL_FUSED_MARK(ra, 3);
    } else {
      lds_set(&sy->v_done, (unsigned)(ra + 1));
    }
  }
}

// ---- end phase (all waves of the workgroup, after the streaming)
//
// Each chunk the workgroup holds goes to one wave, which takes it through
// five steps; a step's waits are for the same step of the row's other
// chunks, so every wave runs a step for all its chunks before the next.
//  1  edges: the three positions at each end are pooled with the
//     neighbours' halos; then the chunk's keys give its coarse histogram
//     (64 bins: bits 31..26), published as 64 words of count + 1.
//  2  coarse: once every chunk's words are there, their sum gives the coarse
//     bin D0 of tau and how many of its keys are needed; the chunk publishes
//     its fine histogram inside D0 (32 bins: bits 25..21), count + 1.
//  3  fine: once those are there, the first digit d1 (bits 31..21) of tau and
//     the keys still needed in bin d1; the chunk stores its keys of bin d1 with
//     their positions in its own range of the candidate list and, once they
//     are written, its count word: keys above bin d1 and its candidates.
//  4  pick: once every count word is there, each lane takes one chunk's
//     candidates; the remaining 21 bits of tau come from them bit by bit (a
//     ballot per held candidate), and every chunk's candidates above and on
//     tau tell where the chunk's picks go; it writes them in index order
//     (tau-equal ones lowest index first) and copies their K and V rows; the
//     row's last prefix chunk adds the window.
// Words published for other workgroups are cleared by their owners before the
// arrival and carry count + 1 (or the +1 of the count word), so a written word
// is never zero.

// The chunk's keys (lane * 8 + u), read back from its key slot (written by
// this workgroup); positions past P are 0.
__device__ __forceinline__ void sel_load_keys(const FusedSel& f, const SelRound& q, uint32_t (&key)[8]) {
  const int lane = threadIdx.x & 63;
  const int S0 = q.c * kS + lane * 8;
  const float4* ks = reinterpret_cast<const float4*>(f.kslot + q.sl * kS + lane * 8);
  const float4 x = ks[0], y = ks[1];
  const float pv[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
  for (int u = 0; u < 8; ++u) key[u] = S0 + u < q.P ? sel_key(pv[u]) : 0u;
}

// Histogram of the chunk's keys over the bins of field (key >> shift) & mask
// (mask 63 or 31), counting only keys for which pass(key) holds: lane b ends
// with the count of bin b.  One round per distinct bin of the wave.
template <typename Pass>
__device__ __forceinline__ uint32_t sel_hist64(const uint32_t (&key)[8], int valid, int shift, uint32_t mask,
                                               Pass pass) {
  const int lane = threadIdx.x & 63;
  uint32_t pend = 0u;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (u < valid && pass(key[u])) pend |= 1u << u;
  uint32_t mine = 0u;
  for (int it = 0; it < 64; ++it) {
    const unsigned long long any = __ballot(pend != 0u);
    if (any == 0ull) break;
    const int leader = __builtin_ctzll(any);
    uint32_t fb = 0u;
#pragma unroll
    for (int u = 7; u >= 0; --u)
      if ((pend >> u) & 1u) fb = (key[u] >> shift) & mask;
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)fb, leader);
    uint32_t tot = 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool hit = ((pend >> u) & 1u) && ((key[u] >> shift) & mask) == b;
      tot += wave_count(hit);
      if (hit) pend &= ~(1u << u);
    }
    if ((uint32_t)lane == b) mine = tot;
  }
  return mine;
}

// Step 1: the edge positions, then the chunk's coarse histogram.
__device__ __forceinline__ bool sel_end_edges(const Launch& a, const FusedSel& f, const SelRound& q,
                                              const float* __restrict__ votes) {
  const int lane = threadIdx.x & 63;
  const int S0 = q.c * kS + lane * 8;
  const bool left = q.c > 0, right = (q.c + 1) * kS < q.P;
  const bool reads = (lane < 3 && left) || (lane >= 3 && lane < 6 && right);
  const unsigned long long* src =
      !reads ? nullptr : (lane < 3 ? f.halo + (q.sl - 1) * kHaloWords + 3 + lane : f.halo + (q.sl + 1) * kHaloWords + (lane - 3));
  unsigned long long hw = reads ? load64(src) : 0ull;
  const bool edge_lane = (lane == 0 && left) || (lane == 63 && right);
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = edge_lane && S0 + u < q.P ? votes[q.vbase + S0 + u] : 0.f;
  const bool ok = sel_wait(a, [&] {
    const bool missing = reads && (hw >> 32) == 0ull;
    if (__ballot(missing) == 0ull) return true;
    if (missing) hw = load64(src);
    return false;
  });
  if (!ok) {
    if (lane == 0) flag_error(a, f, kErrSelectWait);
    return false;
  }
  float ext[14];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    ext[t] = __uint_as_float((unsigned)__builtin_amdgcn_readlane((int)(unsigned)hw, t));
    ext[11 + t] = __uint_as_float((unsigned)__builtin_amdgcn_readlane((int)(unsigned)hw, 3 + t));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) ext[3 + u] = v[u];
  const int valid = max(0, min(8, q.P - S0));
  float pv[8];
  sel_pool8(a, q, ext, pv);
  float* ks = f.kslot + q.sl * kS + lane * 8;
  const uint32_t emask = (lane == 0 && left ? 7u : 0u) | (lane == 63 && right ? 0xE0u : 0u);
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (((emask >> u) & 1u) && u < valid) ks[u] = pv[u];
  uint32_t key[8];
  sel_load_keys(f, q, key);  // after the edge stores (the same wave's accesses to an address stay in order)
  if (f.pooled != nullptr) {
    const float* kf = f.kslot + q.sl * kS + lane * 8;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < valid) f.pooled[q.vbase + S0 + u] = kf[u];
  }
  const uint32_t cnt = sel_hist64(key, valid, 26, 63u, [](uint32_t) { return true; });
  store32(f.cslot + q.sl * 64 + lane, cnt + 1u);
  return true;
}

// The row's histogram over 64 bins from every chunk's published words
// (words of chunk i at base + i * stride, bin b at + b), polled until all are
// written: lane l gets the count of bin 63 - l (highest first).  Only lanes
// below `bins` take part (the rest get 0).  False on a timeout.
__device__ __forceinline__ bool sel_row_hist(const Launch& a, const unsigned* base, int stride, int nchp, int bins,
                                             uint32_t& count) {
  const int lane = threadIdx.x & 63;
  const int b = bins - 1 - lane;
  return sel_wait(a, [&] {
    uint32_t sum = 0u;
    bool all = true;
    constexpr int kBatch = 16;
    for (int i0 = 0; i0 < nchp; i0 += kBatch) {
      uint32_t w[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) w[t] = (lane < bins && i0 + t < nchp) ? load32(base + (i0 + t) * stride + b) : 1u;
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        all = all && w[t] != 0u;
        sum += w[t] - 1u;
      }
    }
    count = sum;
    return __ballot(!all) == 0ull;
  });
}

// Step 2: the coarse bin of tau, then the chunk's fine histogram inside it.
__device__ __forceinline__ bool sel_end_coarse(const Launch& a, const FusedSel& f, const SelRound& q, uint32_t* st) {
  const int lane = threadIdx.x & 63;
  uint32_t cnt = 0u, need0 = 0u;
  int at = 0;
  const bool ok = sel_row_hist(a, f.cslot + (q.sl - q.c) * 64, 64, q.nchp, 64, cnt) &&
                  wave_find(cnt, (uint32_t)q.count, at, need0);
  if (!ok) {
    if (lane == 0) flag_error(a, f, kErrSelectWait);
    return false;
  }
  const uint32_t d0 = 63u - (uint32_t)at;
  uint32_t key[8];
  sel_load_keys(f, q, key);
  const int valid = max(0, min(8, q.P - (q.c * kS + lane * 8)));
  const uint32_t fc = sel_hist64(key, valid, 21, 31u, [&](uint32_t k) { return (k >> 26) == d0; });
  if (lane < 32) store32(f.fslot + q.sl * 32 + lane, fc + 1u);
  if (lane == 0) {
    st[0] = d0;
    st[1] = need0;
  }
  return true;
}

// Step 3: the first digit of tau, then the chunk's candidates and count word.
__device__ __forceinline__ bool sel_end_fine(const Launch& a, const FusedSel& f, const SelRound& q, uint32_t* st) {
  const int lane = threadIdx.x & 63;
  const uint32_t d0 = st[0], need0 = st[1];
  uint32_t cnt = 0u, need = 0u;
  int at = 0;
  const bool ok = sel_row_hist(a, f.fslot + (q.sl - q.c) * 32, 32, q.nchp, 32, cnt) && wave_find(cnt, need0, at, need);
  if (!ok) {
    if (lane == 0) flag_error(a, f, kErrSelectWait);
    return false;
  }
  const uint32_t d1 = d0 * 32u + 31u - (uint32_t)at;
  uint32_t key[8];
  sel_load_keys(f, q, key);
  const int S0 = q.c * kS + lane * 8;
  const int valid = max(0, min(8, q.P - S0));
  uint32_t tot_above = 0u, tot_mine = 0u;
  bool mine_u[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    tot_above += wave_count(u < valid && (key[u] >> 21) > d1);
    mine_u[u] = u < valid && (key[u] >> 21) == d1;
  }
  unsigned long long* cb = f.cand + q.vbase + q.c * kS;  // the chunk's own range
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t at_u = tot_mine + lanes_below(mine_u[u]);
    if (mine_u[u]) store64(cb + at_u, ((unsigned long long)(S0 + u) << 32) | key[u]);
    tot_mine += wave_count(mine_u[u]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the candidates are there before the count word says so
  if (lane == 0) {
    store64(f.cw + q.sl, (unsigned long long)(tot_above + 1u) | ((unsigned long long)tot_mine << 20));
    st[2] = d1;
    st[3] = need;
  }
  return true;
}

// Copy n rows of D bf16 (RU 16-byte pieces each) by the wave: output row
// out_row0 + i from input row in_row0 + (list ? list[i] : first + i).
template <int RU>
__device__ __forceinline__ void wave_copy_rows(const uint4* __restrict__ Ki, const uint4* __restrict__ Vi,
                                               uint4* __restrict__ Ko, uint4* __restrict__ Vo, long long in_row0,
                                               long long out_row0, const int32_t* list, int first, int n) {
  const int lane = threadIdx.x & 63;
  constexpr int kFly = 4;
  const int total = n * RU;
  for (int e0 = 0; e0 < total; e0 += kFly * 64) {
    uint4 kv[kFly], vv[kFly];
#pragma unroll
    for (int t = 0; t < kFly; ++t) {
      const int e = min(e0 + t * 64 + lane, total - 1);
      const int i = e / RU;
      const long long from = (in_row0 + (list ? list[i] : first + i)) * RU + e % RU;
      kv[t] = Ki[from];
      vv[t] = Vi[from];
    }
#pragma unroll
    for (int t = 0; t < kFly; ++t) {
      const int e = e0 + t * 64 + lane;
      if (e < total) {
        const long long to = (out_row0 + e / RU) * RU + e % RU;
        store_stream(Ko + to, kv[t]);
        store_stream(Vo + to, vv[t]);
      }
    }
  }
}

// Step 4: tau, the chunk's picks in index order and their rows (see above).
// Chunk i of the row is lane i % 64 of group i / 64 (at most kPickGroups);
// each lane holds up to kHeld of its chunk's candidates per group and re-reads
// the rest where a chunk has more.
constexpr int kPickGroups = 2;
constexpr int kHeld = 16;
template <int D>
__device__ __forceinline__ void sel_end_pick(const Launch& a, const FusedSel& f, const SelRound& q, const uint32_t* st,
                                             const __bf16* __restrict__ K, int32_t* list) {
  constexpr int RU = D * 2 / 16;
  const int lane = threadIdx.x & 63;
  const Seg& s = a.seg[q.e];
  const unsigned long long* cw0 = f.cw + (q.sl - q.c);  // the row's first chunk
  const int nchp = q.nchp;
  unsigned long long w[kPickGroups];
  const bool ok = sel_wait(a, [&] {
    bool all = true;
#pragma unroll
    for (int g = 0; g < kPickGroups; ++g) {
      const int i = g * 64 + lane;
      w[g] = i < nchp ? load64(cw0 + i) : 1ull;
      all = all && w[g] != 0ull;
    }
    return __ballot(!all) == 0ull;
  });
  if (!ok) {
    if (lane == 0) flag_error(a, f, kErrSelectWait);
    return;
  }
  uint32_t above[kPickGroups], len[kPickGroups], ck[kPickGroups][kHeld];
  bool extra = false;
#pragma unroll
  for (int g = 0; g < kPickGroups; ++g) {
    const int i = g * 64 + lane;
    above[g] = i < nchp ? (uint32_t)(w[g] & 0xFFFFFu) - 1u : 0u;
    len[g] = i < nchp ? (uint32_t)(w[g] >> 20) & 0xFFFFFu : 0u;
    extra = extra || len[g] > (uint32_t)kHeld;
    const unsigned long long* cb = f.cand + q.vbase + (long long)i * kS;
#pragma unroll
    for (int t = 0; t < kHeld; ++t) ck[g][t] = (uint32_t)t < len[g] ? (uint32_t)load64(cb + t) : 0u;
  }
  const bool any_extra = __ballot(extra) != 0ull;
  uint32_t key[8];
  sel_load_keys(f, q, key);
  // The rest of tau, bit by bit.
  uint32_t prefix = st[2], need = st[3];
  for (int bit = 20; bit >= 0; --bit) {
    const uint32_t target = (prefix << 1) | 1u;
    uint32_t tot = 0u;
#pragma unroll
    for (int g = 0; g < kPickGroups; ++g)
#pragma unroll
      for (int t = 0; t < kHeld; ++t) tot += wave_count((uint32_t)t < len[g] && (ck[g][t] >> bit) == target);
    if (any_extra) {
      uint32_t more = 0u;
#pragma unroll
      for (int g = 0; g < kPickGroups; ++g) {
        const unsigned long long* cb = f.cand + q.vbase + (long long)(g * 64 + lane) * kS;
        for (uint32_t t = kHeld; t < len[g]; ++t) more += ((uint32_t)load64(cb + t) >> bit) == target;
      }
      tot += wave_sum_u32(more);
    }
    if (tot >= need) {
      prefix = target;
    } else {
      prefix <<= 1;
      need -= tot;
    }
  }
  const uint32_t tau = prefix, need_eq = need;
  // Every chunk's picks in index order: above its bin, above tau among its
  // candidates, and the tau-equal ones still needed (lowest index first).
  uint32_t before = 0u, take_c = 0u, carry_p = 0u, carry_e = 0u;
#pragma unroll
  for (int g = 0; g < kPickGroups; ++g) {
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int t = 0; t < kHeld; ++t)
      if ((uint32_t)t < len[g]) {
        gt += ck[g][t] > tau;
        eq += ck[g][t] == tau;
      }
    if (len[g] > (uint32_t)kHeld) {
      const unsigned long long* cb = f.cand + q.vbase + (long long)(g * 64 + lane) * kS;
      for (uint32_t t = kHeld; t < len[g]; ++t) {
        const uint32_t kk = (uint32_t)load64(cb + t);
        gt += kk > tau;
        eq += kk == tau;
      }
    }
    const uint32_t eq_incl = wave_incl_u32(eq);
    const uint32_t eqb = carry_e + eq_incl - eq;
    const uint32_t take = need_eq > eqb ? min(eq, need_eq - eqb) : 0u;
    const uint32_t picks = above[g] + gt + take;
    const uint32_t p_incl = wave_incl_u32(picks);
    if (q.c >= g * 64 && q.c < g * 64 + 64) {
      before = (uint32_t)__builtin_amdgcn_readlane((int)(carry_p + p_incl - picks), q.c - g * 64);
      take_c = (uint32_t)__builtin_amdgcn_readlane((int)take, q.c - g * 64);
    }
    carry_e += (uint32_t)__builtin_amdgcn_readlane((int)eq_incl, 63);
    carry_p += (uint32_t)__builtin_amdgcn_readlane((int)p_incl, 63);
  }
  // This chunk's picks.
  const int S0 = q.c * kS + lane * 8;
  const int valid = max(0, min(8, q.P - S0));
  uint32_t seen = 0u;  // tau-equal keys of the chunk before this lane's current one
  {
    uint32_t eqb = 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) eqb += u < valid && key[u] == tau;
    seen = wave_incl_u32(eqb) - eqb;
  }
  uint32_t pm = 0u;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (u >= valid) continue;
    if (key[u] > tau) {
      pm |= 1u << u;
    } else if (key[u] == tau) {
      if (seen < take_c) pm |= 1u << u;
      ++seen;
    }
  }
  const uint32_t np = (uint32_t)__popc(pm);
  const uint32_t p_incl = wave_incl_u32(np);
  const uint32_t n_c = (uint32_t)__builtin_amdgcn_readlane((int)p_incl, 63);
  uint32_t slot = p_incl - np;
  int32_t* out = f.indices + s.idx_off + (long long)q.h * s.idx_ld;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if ((pm >> u) & 1u) {
      fused_debug_check(a, f, before + slot < (uint32_t)q.count);
      if (before + slot < (uint32_t)q.count) {  // always, unless a timed-out wait left the counts short
        out[before + slot] = S0 + u;
        list[slot] = S0 + u;
      }
      ++slot;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint4* Ki = reinterpret_cast<const uint4*>(K);
  const uint4* Vi = reinterpret_cast<const uint4*>(f.V);
  uint4* Ko = reinterpret_cast<uint4*>(f.K_out);
  uint4* Vo = reinterpret_cast<uint4*>(f.V_out);
  const long long in_row0 = s.kv_off / D + (long long)q.h * s.L;
  const long long out_row0 = s.out_off + (long long)q.h * s.out_ld;
  const int n_copy = (int)min(n_c, (uint32_t)q.count > before ? (uint32_t)q.count - before : 0u);
  wave_copy_rows<RU>(Ki, Vi, Ko, Vo, in_row0, out_row0 + before, list, 0, n_copy);
  if (q.c == nchp - 1) {  // the window follows the picks
    for (int i = lane; i < a.W; i += 64) out[q.count + i] = q.P + i;
    wave_copy_rows<RU>(Ki, Vi, Ko, Vo, in_row0, out_row0 + q.count, nullptr, q.P, a.W);
  }
}

// End phase of the fused selection (all waves): the workgroup's chunks are
// dealt to its waves, which run each step for all of theirs before the next.
// lds: per round four words (the digits and what is still needed), then per
// wave kS words for its picks.
template <int D>
__device__ __forceinline__ void sel_finish(const Launch& a, const FusedSel& f, const __bf16* __restrict__ K,
                                           const float* __restrict__ votes, uint32_t* lds) {
  constexpr int kWv = kThreads / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* st = lds;
  int32_t* list = reinterpret_cast<int32_t*>(lds + 4 * kFusedMaxRounds) + wave * kS;
  KVSEL_FUSED_MARK(20, 0);
  constexpr uint32_t kFail = 0xFFFFFFFFu;  // in a round's first word: a step timed out
  for (int step = 0; step < 4; ++step) {
    for (int r = 0, n = 0; r < a.rounds; ++r) {
      const SelRound q = sel_round(a, r);
      if (!q.on) continue;
      if (n++ % kWv != wave) continue;
      uint32_t* sr = st + 4 * r;
      bool ok = true;
      if (step == 0)
        ok = sel_end_edges(a, f, q, votes);
      else if (sr[0] == kFail)
        continue;
      else if (step == 1)
        ok = sel_end_coarse(a, f, q, sr);
      else if (step == 2)
        ok = sel_end_fine(a, f, q, sr);
      else
        sel_end_pick<D>(a, f, q, sr, K, list);
      if (lane == 0 && (step == 0 || !ok)) sr[0] = ok ? 0u : kFail;
    }
    KVSEL_FUSED_MARK(20, 1 + step);
  }
}

// ---- fallback (ABORT: not all resident), of both kernel variants

// Claims and completion counts of the fallback.  Nothing was cleared before
// the call, so they are token-tagged: a claim is a compare-and-swap loop.
__device__ __forceinline__ unsigned fb_claim(unsigned long long* w, unsigned long long tag, unsigned n = 1u) {
  return tok_add(w, tag, n);
}
__device__ __forceinline__ unsigned fb_count(const unsigned long long* w, unsigned long long tag) {
  return tok_count(w, tag);
}

// Inclusive scan over the workgroup (kThreads); total gets the sum.
__device__ __forceinline__ uint32_t wg_incl(uint32_t v, uint32_t* sh, uint32_t& total) {
  constexpr int kWv = kThreads / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_incl_u32(v);
  if (lane == 63) sh[wv] = v;
  __syncthreads();
  uint32_t base = 0u, tot = 0u;
#pragma unroll
  for (int i = 0; i < kWv; ++i) {
    const uint32_t t = sh[i];
    if (i < wv) base += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return v + base;
}

// Work item t of the fallback's scoring phases: (row, group of up to
// kFbChunks chunks) over the launch's rows, group-minor.  Groups amortise
// an item's fixed costs (Qwin load, claim, completion count) over several
// chunks; a row still has several items, so every workgroup gets work.
constexpr int kFbChunks = 4;
struct FbItem {
  bool on;
  int e, h, c, nc, row;  // chunks c .. c + nc - 1 of row `row`
};
__device__ __forceinline__ int fb_groups(const Seg& s) { return (s.fc + kFbChunks - 1) / kFbChunks; }
__device__ __forceinline__ FbItem fb_item(const Launch& a, unsigned t) {
  FbItem it{false, 0, 0, 0, 0, 0};
  unsigned base = 0;
  for (int e = 0; e < a.n; ++e) {
    const Seg& s = a.seg[e];
    const unsigned ng = (unsigned)fb_groups(s);
    const unsigned n = (unsigned)s.nh * ng;
    if (t < base + n) {
      const unsigned loc = t - base;
      it.on = true;
      it.e = e;
      it.h = s.h0 + (int)(loc / ng);
      it.c = (int)(loc % ng) * kFbChunks;
      it.nc = min(kFbChunks, s.fc - it.c);
      it.row = s.row0 + (it.h - s.h0);
      return it;
    }
    base += n;
  }
  return it;
}
__device__ __forceinline__ int fb_rows(const Launch& a) { return a.seg[a.n - 1].row0 + a.seg[a.n - 1].nh; }

// One pass of the streaming waves over positions [lo, hi) of a head's K
// (tiles lo + 32 t, wave-strided): with votes, the votes of the prefix
// positions from the base-2 log-normalisers s_m (agent-scope stores, read by
// other workgroups later); without, the lane's running (max, sum) per row.
template <int D>
__device__ __forceinline__ void fb_pass(const Launch& a, int L, int P, const __bf16* __restrict__ kh, int lo, int hi, bool with_votes,
                        uint4 (*ring)[TileGeom<D>::PIECES], const uint4* qbuf, const float* s_m, float* vout,
                        float (&m)[16], float (&z)[16]) {
  using G = TileGeom<D>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const float sc = a.scale2;
  const int tiles = (hi - lo + 31) / 32;
  const int nw = tiles > wave ? (tiles - wave + kSW - 1) / kSW : 0;
  float mr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) mr[r] = with_votes ? s_m[acc_row(r, g)] : 0.f;
  int issued = 0;
  if (nw > 0) {
    issue_tile<D>(kh, L, lo + wave * 32, ring[0], lane, a.k_nt != 0);
    issued = 1;
  }
  for (int i = 0; i < nw; ++i) {
    wait_tiles<D>(0);
    const uint4* tile = ring[0];
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
      issue_tile<D>(kh, L, lo + (wave + kSW * issued) * 32, ring[0], lane, a.k_nt != 0);
      ++issued;
    }
    const int j = lo + (wave + kSW * i) * 32 + n;
    if (with_votes) {
      float tot = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) tot += exp2_fast(fmaf(acc[r], sc, -mr[r]));
      const float other = __shfl_xor(tot, 32);
      const float v = g == 0 ? tot + other : other + tot;
      if (g == 0 && j < hi && j < P) __hip_atomic_store(vout + j, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, g);
        const float x = (j < hi && j <= P + row) ? acc[r] * sc : -INFINITY;
        const float d = x - m[r];
        const float e = exp2_fast(-fabsf(d));
        z[r] = d > 0.f ? fmaf(z[r], e, 1.f) : z[r] + e;
        m[r] = fmaxf(m[r], x);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Qwin of (sequence, head) hs into qbuf (wave kExWave), rows W..31 cleared.
template <int D>
__device__ __forceinline__ void fb_load_q(const Launch& a, const __bf16* __restrict__ Q, int hs, uint4* qbuf) {
  if ((int)(threadIdx.x >> 6) == kExWave) {
    issue_tile<D>(Q + (long long)hs * a.W * D, a.W, 0, qbuf, threadIdx.x & 63);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    ctl_finish_q<D>(a.W, qbuf);
  }
}

// Pooled score of position j of a row whose votes other workgroups wrote.
__device__ __forceinline__ float fb_pooled(const Launch& a, const float* v, int j, int P) {
  return pool_at(j, P, a.kernel, a.pooling == 1, [&](int t) {
    return __hip_atomic_load(v + j + t - 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
}

// Whole-row selection by the workgroup: three radix digits of tau over the
// row's pooled keys (recomputed from the votes in each pass), then the picks
// in index order and their K and V rows, then the window.
template <int D>
__device__ __forceinline__ void fb_select_row(const Launch& a, const FusedSel& f, int e, int h, const float* __restrict__ votes,
                              const __bf16* __restrict__ K, uint32_t* lds) {
  constexpr int RU = D * 2 / 16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const Seg& s = a.seg[e];
  const int P = s.L - a.W, count = s.C - a.W;
  const long long vbase = s.vote_off + (long long)h * s.vote_ld;
  const float* v = votes + vbase;
  uint32_t* hist = lds;             // 2048 bins
  uint32_t* sh = lds + 2048;        // 32 words of scan scratch, then the digit and what is still needed
  int32_t* list = reinterpret_cast<int32_t*>(lds + 2048 + 64);  // kThreads picks
  uint32_t prefix = 0u, need = (uint32_t)count;
  for (int digit = 0; digit < 3; ++digit) {
    const int shift = digit == 0 ? 21 : (digit == 1 ? 10 : 0);
    const int bits = digit == 2 ? 10 : 11;
    const int nb = 1 << bits;
    for (int d = tid; d < nb; d += kThreads) hist[d] = 0u;
    __syncthreads();
    for (int j = tid; j < P; j += kThreads) {
      const float pv = fb_pooled(a, v, j, P);
      const uint32_t k = sel_key(pv);
      if (digit == 0 && f.pooled != nullptr) f.pooled[vbase + j] = pv;
      if (digit == 0 || (k >> (shift + bits)) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    if (wv == 0) {
      const int per = nb / 64;
      uint32_t hh[32];
#pragma unroll
      for (int t = 0; t < 32; ++t) hh[t] = t < per ? hist[(63 - lane) * per + t] : 0u;
      uint32_t dg = 0u, left = 0u;
      if (!find_digit(hh, per, need, dg, left)) {
        dg = 0u;
        left = 0u;
        if (lane == 0) flag_error(a, f, kErrSelectWait);
      }
      if (lane == 0) {
        sh[32] = dg;
        sh[33] = left;
      }
    }
    __syncthreads();
    prefix = (prefix << bits) | sh[32];
    need = sh[33];
    __syncthreads();
  }
  const uint32_t tau = prefix, need_eq = need;
  int32_t* out = f.indices + s.idx_off + (long long)h * s.idx_ld;
  const uint4* Ki = reinterpret_cast<const uint4*>(K);
  const uint4* Vi = reinterpret_cast<const uint4*>(f.V);
  uint4* Ko = reinterpret_cast<uint4*>(f.K_out);
  uint4* Vo = reinterpret_cast<uint4*>(f.V_out);
  const long long in_row0 = s.kv_off / D + (long long)h * s.L;
  const long long out_row0 = s.out_off + (long long)h * s.out_ld;
  uint32_t before = 0u, eq_seen = 0u;
  for (int base = 0; base < P; base += kThreads) {
    const int j = base + tid;
    const uint32_t k = j < P ? sel_key(fb_pooled(a, v, j, P)) : 0u;
    const bool gt = j < P && k > tau, eq = j < P && k == tau;
    uint32_t eq_tot, take_tot;
    const uint32_t eq_rank = wg_incl(eq ? 1u : 0u, sh, eq_tot) - (eq ? 1u : 0u);
    const bool take = gt || (eq && eq_seen + eq_rank < need_eq);
    const uint32_t pos = wg_incl(take ? 1u : 0u, sh, take_tot) - (take ? 1u : 0u);
    fused_debug_check(a, f, !take || before + pos < (uint32_t)count);
    if (take && before + pos < (uint32_t)count) {
      out[before + pos] = j;
      list[pos] = j;
    }
    __syncthreads();
    const int n = (int)min(take_tot, (uint32_t)count > before ? (uint32_t)count - before : 0u);
    for (int q = tid; q < n * RU; q += kThreads) {
      const long long from = (in_row0 + list[q / RU]) * RU + q % RU, to = (out_row0 + before + q / RU) * RU + q % RU;
      store_stream(Ko + to, Ki[from]);
      store_stream(Vo + to, Vi[from]);
    }
    before += take_tot;
    eq_seen += eq_tot;
    __syncthreads();
  }
  for (int i = tid; i < a.W; i += kThreads) out[count + i] = P + i;
  for (int q = tid; q < a.W * RU; q += kThreads) {
    const long long from = (in_row0 + P + q / RU) * RU + q % RU, to = (out_row0 + count + q / RU) * RU + q % RU;
    store_stream(Ko + to, Ki[from]);
    store_stream(Vo + to, Vi[from]);
  }
  (void)lane;
}

// The fallback (ABORT: not all resident): scoring in two phases over (row,
// chunk) items, statistics then votes (with handed-over statistics only the
// votes), then with the fused selection whole rows' selections.  Items are
// claimed in order from token-tagged counters, and a phase waits only for
// items of the phase before, which running workgroups have claimed, so the
// fallback finishes with any number of workgroups, and every workgroup that
// runs takes part.
template <int D, bool kLse, bool kSel>
__device__ __forceinline__ void sel_fallback(const Launch& a, const FusedSel& f, const __bf16* __restrict__ Q,
                             const __bf16* __restrict__ K, const float* __restrict__ lse,
                             unsigned long long* __restrict__ ex, float* __restrict__ votes,
                             float* __restrict__ row_stats, uint4 (*ring)[TileGeom<D>::PIECES], uint4* qbuf,
                             float* s_maxp, float* s_zp, float* s_m, uint32_t* lds_u32) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const bool streams = wave < kSW;
  const unsigned long long tag = token_tag(f.token);
  unsigned long long* ctr = f.flags + kFlagWordsMax + 1;
  const int W = a.W;
  __shared__ unsigned s_claim;
  unsigned items = 0;
  for (int e = 0; e < a.n; ++e) items += (unsigned)(a.seg[e].nh * fb_groups(a.seg[e]));
  for (int phase = kLse ? 1 : 0; phase < 2; ++phase) {
    for (;;) {
      if (tid == 0) s_claim = fb_claim(ctr + phase, tag);
      __syncthreads();
      const unsigned t = s_claim;
      __syncthreads();
      if (t >= items) break;
      const FbItem it = fb_item(a, t);
      const Seg& s = a.seg[it.e];
      const int L = s.L, P = L - W;
      const int hs = s.b * a.heads + it.h;
      const long long sl = s.fslot_base + (long long)it.h * fused_slot_stride(s.fc) + it.c;
      // The chunk statistics go to the chunk's key slot, which nothing clears
      // (a workgroup that starts late still clears its share of the exchange
      // slots).
      unsigned long long* fbs = reinterpret_cast<unsigned long long*>(f.kslot);
      const __bf16* kh = K + s.kv_off + (long long)it.h * L * D;
      const int lo = it.c * kS, hi = min(L, lo + it.nc * kS);
      fb_load_q<D>(a, Q, hs, qbuf);
      if (phase == 1 && tid == 0) {  // the statistics of every chunk of the row are there
        const bool ok = kLse || sel_wait(a, [&] { return fb_count(f.rowfb + 2ll * it.row, tag) >= (unsigned)s.fc; });
        if (!ok) flag_error(a, f, kErrExchangeWait);
      }
      __syncthreads();
      float m[16], z[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        m[r] = kNegBig;
        z[r] = 0.f;
      }
      if (phase == 0) {
        if (streams) fb_pass<D>(a, L, P, kh, lo, hi, false, ring + wave, qbuf, s_m, nullptr, m, z);
        if (streams) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float mh0 = half_max(m[r]);
            const float m0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(mh0), 31));
            const float m1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(mh0), 63));
            const float mh = g == 0 ? m0 : m1;
            const float zz = half_sum(z[r] != 0.f ? z[r] * exp2_fast(m[r] - mh) : 0.f);
            if ((lane & 31) == 31) {
              s_maxp[wave * 32 + acc_row(r, g)] = mh;
              s_zp[wave * 32 + acc_row(r, g)] = zz;
            }
          }
        }
        __syncthreads();
        if (tid < W) {  // the chunk's (max, sum) per row into its slot
          float M = s_maxp[tid];
          for (int w2 = 1; w2 < kSW; ++w2) M = fmaxf(M, s_maxp[w2 * 32 + tid]);
          float Z = 0.f;
          for (int w2 = 0; w2 < kSW; ++w2) {
            const float zv = s_zp[w2 * 32 + tid];
            if (zv != 0.f) Z += zv * exp2_fast(s_maxp[w2 * 32 + tid] - M);
          }
          store64(fbs + sl * (kS / 2) + tid, pack_slot(M, Z));
          // The item's other chunks hold nothing: zero sums, skipped by the merge.
          for (int q = 1; q < it.nc; ++q) store64(fbs + (sl + q) * (kS / 2) + tid, pack_slot(kNegBig, 0.f));
        }
      } else {
        if (tid < 32) {  // the row's log-normalisers: merged slots in chunk order, or the given ones
          float lm = INFINITY;
          if (tid < W) {
            if (kLse) {
              lm = lse[(long long)hs * W + tid] * kLog2e;
              if (!isfinite(lm)) flag_error(a, f, kErrNonFinite);
            } else {
              const unsigned long long* s0 = fbs + (sl - it.c) * (kS / 2) + tid;
              float M = kNegBig, Z = 0.f;
              for (int c2 = 0; c2 < s.fc; ++c2) {
                const unsigned long long wd = load64(s0 + (long long)c2 * (kS / 2));
                const float mo = __uint_as_float((unsigned)wd), zo = __uint_as_float((unsigned)(wd >> 32));
                if (zo != 0.f) lse_merge(M, Z, mo, zo);
              }
              if (!stats_ok(M, Z)) flag_error(a, f, kErrNonFinite);
              lm = M + __log2f(Z);
              if (row_stats != nullptr && it.c == 0) {
                row_stats[((long long)hs * W + tid) * 2] = M * kLn2;
                row_stats[((long long)hs * W + tid) * 2 + 1] = Z;
              }
            }
          }
          s_m[tid] = lm;  // rows past W: zero queries, dropped by the infinite normaliser
        }
        __syncthreads();
        float* vout = votes + s.vote_off + (long long)it.h * s.vote_ld;
        if (streams) fb_pass<D>(a, L, P, kh, lo, min(hi, P), true, ring + wave, qbuf, s_m, vout, m, z);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) (void)fb_claim(f.rowfb + 2ll * it.row + phase, tag, (unsigned)it.nc);  // chunks done
      __syncthreads();
    }
  }
  if constexpr (!kSel) return;
  const int rows = fb_rows(a);
  for (;;) {
    if (tid == 0) s_claim = fb_claim(ctr + 2, tag);
    __syncthreads();
    const unsigned t = s_claim;
    __syncthreads();
    if (t >= (unsigned)rows) break;
    const int e = find_seg<kFieldRow>(a, (int)t);
    const Seg& s = a.seg[e];
    const int h = s.h0 + ((int)t - s.row0);
    if (tid == 0) {  // every chunk's votes of the row are there
      const bool ok = sel_wait(a, [&] { return fb_count(f.rowfb + 2ll * t + 1, tag) >= (unsigned)s.fc; });
      if (!ok) flag_error(a, f, kErrSelectWait);
    }
    __syncthreads();
    fb_select_row<D>(a, f, e, h, votes, K, lds_u32);
    __syncthreads();
  }
  (void)lane;
}

template <int D, bool kLse, bool kSel>
__global__ __launch_bounds__(kSel ? kThreads : kThreadsPlain, 1) void window_fused_kernel(const Launch a, const FusedSel f,
                                                                  const __bf16* __restrict__ Q,
                                                                  const __bf16* __restrict__ K,
                                                                  const float* __restrict__ lse,
                                                                  unsigned long long* __restrict__ ex,
                                                                  float* __restrict__ votes,
                                                                  float* __restrict__ row_stats) {
  using G = TileGeom<D>;
  __shared__ uint4 s_ring[kSW][kNBuf][G::PIECES];
  __shared__ uint4 s_q[2][G::PIECES];
  __shared__ float4 s_x[kSW][kTT * 4 * 64];  // each wave's logits of one round
  __shared__ float s_maxp[kNR][kSW * 32], s_zp[kNR][kSW * 32];
  __shared__ float s_m[kNR][32];
  __shared__ float s_votes[2][kS];
  __shared__ Sync sy;
  static_assert(sizeof(s_x) >= 4 * (4 * kFusedMaxRounds + (kThreads / 64) * kS), "the end phase's words fit s_x");
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // Variants whose workgroups wait for each other: those that exchange row
  // statistics or select.
  constexpr bool kHandshake = kSel || !kLse;
  KVSEL_FUSED_MARK(23, 0);
  if (threadIdx.x == 0) {
    sy = Sync{};
    sy.zeroed = kHandshake ? 0u : 1u;
  }
  __syncthreads();  // afterwards waves meet through LDS flags (and once more at the end)
  // The clears go first, so that they do not queue behind the K tiles (the
  // decision that follows them gates the publication of every round); then
  // the first K tiles and Qwin of rounds 0 and 1.
  if (wave == kExWave) {
    KVSEL_FUSED_MARK(22, 0);
    sel_clear(f, 0, f.clr_early);
    KVSEL_FUSED_MARK(22, 1);
    lds_set(&sy.issued, 1u);
  } else if (wave < kSW || wave == kMemWave) {
    (void)lds_wait_ge(&sy, &sy.issued, 1u);
  }
  WaveTiles cur{K, 0, 0, false};
  int issued = 0, consumed = 0;
  if (wave < kSW) {
    cur = wave_tiles<D>(a, K, 0, wave);
    issue_wave_tile<D>(cur, 0, s_ring[wave][0], issued);
  } else if (wave == kMemWave) {
    ctl_issue_q<D>(a, 0, Q, s_q[0]);
    ctl_issue_q<D>(a, 1, Q, s_q[1]);
  }
  if (wave == kExWave) {
    if constexpr (kHandshake) {
      // Arrive once the clears are done, clear the words later kernels
      // use, decide; then the statistics.
      sel_arrive(f);
      sel_clear(f, f.clr_early, 4);
      KVSEL_FUSED_MARK(22, 2);
      KVSEL_FUSED_MARK(23, 4);
      const unsigned d = sel_decide(a, f);
      KVSEL_FUSED_MARK(23, 5);
      lds_set(&sy.zeroed, 1u);  // every workgroup's clears are done (GO), or nothing is published (ABORT)
      if (d != kFusedGo && lane == 0) flag_error(a, f, kFlagScoringFallback);
      lds_set(&sy.go, d);
      if (d != kFusedGo)
        lds_set(&sy.abort, 1u);  // not all resident: every wave leaves its loop
      else if constexpr (kLse)
        ctl_lse(a, f, lse, s_m, &sy);
      else
        ctl_exchange<D>(a, f, ex, row_stats, s_m, &sy);
    } else {
      sel_clear(f, f.clr_early, 4);
      ctl_lse(a, f, lse, s_m, &sy);  // no workgroup waits for another
    }
  } else if (wave == kMemWave) {
    ctl_memory<D>(a, !kSel, Q, votes, s_q, s_votes, &sy);
  } else if (wave == kPubWave) {
    if constexpr (!kLse) ctl_publish(a, ex, s_maxp, s_zp, &sy);
  } else if (wave == kSelWave) {
    if constexpr (kSel) ctl_select(a, f, votes, s_votes, &sy);
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
  KVSEL_FUSED_MARK(23, 1);
  __syncthreads();
  KVSEL_FUSED_MARK(23, 2);
  if (sy.abort) {  // not all resident: work from counters (statistics, votes, with the fused selection rows)
    sel_fallback<D, kLse, kSel>(a, f, Q, K, lse, ex, votes, row_stats, s_ring[0], s_q[0], s_maxp[0], s_zp[0],
                                s_m[0], reinterpret_cast<uint32_t*>(&s_x[0][0]));
    return;
  }
  if constexpr (kSel) sel_finish<D>(a, f, K, votes, reinterpret_cast<uint32_t*>(&s_x[0][0]));  // the selection's end phase
  KVSEL_FUSED_MARK(23, 3);
  if (threadIdx.x == 0 && sy.timeout) flag_error(a, f, kErrLdsWait);
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
  int grid[2][2][2] = {};  // [kSel][kLse][D == 128], 0: not looked up yet (-1: does not fit)
};
GridCache g_grid;

// One workgroup per CU when the kernel fits a CU at all (the same grid for
// every variant of a head size: the workgroups of a call must all fit).
template <int D, bool kLse, bool kSel>
int grid_for() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (g_grid.device != dev) {
    g_grid = GridCache{};
    g_grid.device = dev;
  }
  int& slot = g_grid.grid[kSel][kLse][D == 128];
  if (slot == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)window_fused_kernel<D, kLse, kSel>,
                                                     kSel ? kThreads : kThreadsPlain, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    slot = per_cu >= 1 ? cus : -1;
  }
  return slot > 0 ? slot : 0;
}

template <int D, bool kLse, bool kSel>
hipError_t launch_t(const Launch& a, const FusedSel& f, const void* Q, const void* K, const float* lse,
                    unsigned long long* ex, float* votes, float* row_stats, hipStream_t st) {
  const int grid = grid_for<D, kLse, kSel>();
  if (grid <= 0 || grid > kFlagWordsMax) return hipErrorNotSupported;
  Launch la = a;
  const __bf16* q = (const __bf16*)Q;
  const __bf16* k = (const __bf16*)K;
  hipLaunchKernelGGL((window_fused_kernel<D, kLse, kSel>), dim3(grid), dim3(kSel ? kThreads : kThreadsPlain), 0, st,
                     la, f, q, k, lse, ex, votes, row_stats);
  return hipGetLastError();
}

template <int D, bool kLse>
hipError_t launch_d(const Launch& a, const FusedSel& f, const void* Q, const void* K, const float* lse,
                    unsigned long long* ex, float* votes, float* row_stats, hipStream_t st) {
  if (f.on) return launch_t<D, kLse, true>(a, f, Q, K, lse, ex, votes, row_stats, st);
  return launch_t<D, kLse, false>(a, f, Q, K, lse, ex, votes, row_stats, st);
}

}  // namespace

int fused_positions(int W, int D) {
  (void)D;
  return W <= 32 ? kS : 0;
}

int fused_grid(int W, int D) {
  if (W > 32) return 0;
  // The variants with given row statistics or the fused selection fit a CU
  // the same way (checked at launch).
  if (D == 128) return grid_for<128, false, false>();
  if (D == 64) return grid_for<64, false, false>();
  return 0;
}

int fused_exchange_bytes() { return kSlotWords * 8; }

hipError_t launch_fused_scoring(const Launch& a, const void* Q, const void* K, const float* lse, unsigned* ex,
                                float* votes, float* row_stats, const FusedSel& sel, hipStream_t st) {
  if (a.W > 32 || a.S != kS) return hipErrorNotSupported;
  if (sel.on && (!fused_select_kernel_ok(a.kernel) || a.group > 1)) return hipErrorNotSupported;
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(ex);
  if (lse != nullptr) {
    if (a.D == 128) return launch_d<128, true>(a, sel, Q, K, lse, slots, votes, nullptr, st);
    if (a.D == 64) return launch_d<64, true>(a, sel, Q, K, lse, slots, votes, nullptr, st);
    return hipErrorNotSupported;
  }
  if (a.D == 128) return launch_d<128, false>(a, sel, Q, K, nullptr, slots, votes, row_stats, st);
  if (a.D == 64) return launch_d<64, false>(a, sel, Q, K, nullptr, slots, votes, row_stats, st);
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
