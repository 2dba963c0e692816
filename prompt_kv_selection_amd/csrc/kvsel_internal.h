// Internal declarations shared by the HIP sources of libkvsel.
//
// Work is described by a small table of segments passed to every kernel by
// value.  A segment is one sequence b (prompt length L, budget C) restricted
// to a contiguous range of heads [h0, h0 + nh).  Heads, layers and sequences
// are independent units of the selection, so any partition into segments
// gives the same results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


namespace kvsel {

constexpr int kMaxSegs = 16;       // segments per launch
constexpr int kWaves = 4;          // waves per scoring workgroup
constexpr int kWaveTiles = 8;      // 32-position tiles per wave
constexpr int kChunk = kWaves * kWaveTiles * 32;  // positions per scoring workgroup
constexpr int kTopkThreads = 1024;
constexpr int kPoolBlock = 256;

struct Seg {
  int b;          // sequence index (Q and row-stat offsets)
  // Heads below are query heads; scoring items and K/V run over the K/V
  // heads (Launch::group query heads each).
  int L;          // prompt length
  int C;          // budget (includes the window); L < C means bypass
  int nout;       // rows to emit per head: min(L, C), or the gather count
  int h0, nh;     // head range
  int nch;        // scoring chunks per K/V head, ceil(L / kChunk)
  int item0;      // first scoring workgroup of this segment in the launch
  int row0;       // first (segment, head) row of this segment in the launch
  int gitem0;     // first gather workgroup of this segment in the launch
  int gblk;       // gather workgroups per head
  int idx_ld;     // indices between heads
  int out_ld;     // K_out / V_out rows between heads
  int vote_ld;    // votes / pooled floats between heads
  long long kv_off;    // element offset of (b, K/V head 0, row 0) in K and V
  long long idx_off;   // element offset of (b, head 0) in indices
  long long out_off;   // row offset of (b, head 0) in K_out / V_out
  long long vote_off;  // element offset of (b, head 0) in votes / pooled
  long long part_base; // two-pass partial-stat slot of (b, K/V head 0, chunk 0); a slot has group_rows rows
  long long fslot_base;  // single-read exchange slot of (b, head 0, chunk 0)
  // single-read scoring schedule (see kvsel_fused.hip)
  int fc;         // chunks per head, ceil(L / S)
  int fhpr;       // heads per round
  int fr0;        // first round of this segment
  int fnr;        // rounds of this segment
};

struct Launch {
  int n;          // segments in use
  int heads;      // heads per sequence (stride of Qwin and row stats)
  int W, D;
  int kernel, pooling;
  int window;     // 1: append the window positions after the picks
  float scale2;   // log2(e) / sqrt(D)
  int S;          // single-read scoring: positions per workgroup per round
  int rounds;     // single-read scoring: rounds over all segments
  int seg_size;   // selection: positions per emit workgroup (multiple of 2048)
  unsigned* err;  // error flags of the call (the workspace header word), or nullptr
  // With token != 0 the two-pass scoring kernels record their flags in the
  // tagged header word errw instead (raise_flag), so that a launch of the
  // call may clear word 0 for the kernels after it.
  unsigned long long token;
  unsigned long long* errw;
  // 1: the two-pass kernels load K tiles non-temporally (a call whose K is
  // larger than the last-level cache keeps none of it for the second pass
  // anyway, and cached lines would only evict what is still useful).
  int k_nt;
  int group;      // query heads per K/V head (grouped-query attention); 0 or 1: one each
  long long residency_ticks;  // wall-clock ticks of the residency bound (kResidencyMicros)
  Seg seg[kMaxSegs];
};

// The K/V head that query head h (of a segment) reads: consecutive query
// heads share one K/V head, group at a time (as repeat_kv expands them).
__host__ __device__ inline int kv_head(const Launch& a, int h) { return a.group > 1 ? h / a.group : h; }
// Window rows scored together against one K/V head: the group's query heads.
__host__ __device__ inline int group_rows(const Launch& a) { return (a.group > 1 ? a.group : 1) * a.W; }

// Error flags of a call, ORed into Launch::err.
enum : unsigned {
  kErrExchangeWait = 1u,  // single-read scoring: a wait for another workgroup's statistics timed out
  kErrLdsWait = 2u,       // single-read scoring: a wait between the waves of a workgroup timed out
  kErrSelectWait = 4u,    // selection: a wait for another workgroup's histogram or counts timed out
  kErrNonFinite = 8u,     // a non-finite input (validating mode) or a non-finite or zero row normaliser
  kErrDomain = 16u,       // an input outside its documented domain (a negative second-moment entry)
  kErrIndexRange = 32u,   // built with KVSEL_DEBUG: an index outside its range reached a row copy
  // Not errors: which way a residency handshake went.
  kFlagScoringFallback = 256u,  // single-read scoring: not all resident, (row, chunk) items from counters
  kFlagSelectFallback = 512u,   // cooperative selection: not all resident, whole rows by one workgroup
};
// The workspace header: word 0 holds the flags of the last call (cleared by
// every call), word kStickyWord the OR of every call's flags since the
// caller last reset it (kvsel_status_flags).
constexpr int kStickyWord = 4;
// Calls that clear nothing before they start (the fused selection) record
// their flags in the 64-bit header word at byte 8 instead of word 0:
// (tag << 24) | flags, where tag identifies the call (token_tag); a flag
// word whose tag is not the last call's carries none of its flags.
constexpr int kTaggedWord = 2;  // in 32-bit words: bytes 8..15
__host__ __device__ inline unsigned long long token_tag(unsigned long long token) {
  return (token >> 2) & ((1ull << 40) - 1);
}
__device__ inline void raise_tagged(unsigned long long* w, unsigned long long token, unsigned bit) {
  const unsigned long long tag = token_tag(token);
  unsigned long long cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const unsigned long long nv = (cur >> 24) == tag ? (cur | bit) : ((tag << 24) | bit);
    if (nv == cur) break;
    unsigned long long expect = cur;
    if (__hip_atomic_compare_exchange_strong(w, &expect, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
    cur = expect;
  }
  unsigned* sticky = reinterpret_cast<unsigned*>(w) - kTaggedWord + kStickyWord;
  __hip_atomic_fetch_or(sticky, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void raise_error(unsigned* err, unsigned bit) {
  if (err != nullptr) {
    __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(err + kStickyWord, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
// A flag of a scoring kernel: the tagged word with a token, else word 0.
__device__ inline void raise_flag(const Launch& a, unsigned bit) {
  if (a.token != 0ull)
    raise_tagged(a.errw, a.token, bit);
  else
    raise_error(a.err, bit);
}
// A 16-byte store of an output nothing in the call reads back (the kept K
// and V rows): non-temporal, so it does not fill the L2 with dirty lines
// that the kernel's end, or the next call's K stream, would have to write
// back.
typedef unsigned kvsel_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(uint4* p, const uint4& v) {
  const kvsel_u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<kvsel_u32x4*>(p));
}
// Ranges of 32-bit words a kernel clears for the kernels after it in the
// call (empty ranges have n = 0).
constexpr int kClearRanges = 4;
struct WordRanges {
  unsigned* p[kClearRanges];
  long long n[kClearRanges];
};
// Debug builds (KVSEL_DEBUG defined) check every index that turns into a row
// address (the K/V copies, the gather of caller indices) and record a
// violation as kErrIndexRange in the call's flags, or, for entry points
// without a workspace header, in a library-wide word (kvsel_debug_flags).
// The access itself is still clamped or skipped: the check never traps.
// Release builds compile the checks away.
#ifdef KVSEL_DEBUG
constexpr bool kDebug = true;
// The word of entry points without a workspace header (one per translation
// unit; the gather and step kernels that can have none live in
// kvsel_select.hip, whose word kvsel_debug_flags reads).
static __device__ unsigned g_debug_word;
#else
constexpr bool kDebug = false;
#endif
__device__ inline void debug_raise(unsigned* err, unsigned bit) {
#ifdef KVSEL_DEBUG
  if (err != nullptr)
    raise_error(err, bit);
  else
    __hip_atomic_fetch_or(&g_debug_word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  (void)err;
  (void)bit;
#endif
}
#define KVSEL_DEBUG_CHECK(ok, err)                        \
  do {                                                    \
    if constexpr (kDebug) {                               \
      if (!(ok)) debug_raise((err), kErrIndexRange);      \
    }                                                     \
  } while (0)
// The library-wide debug word (host side, kvsel_select.hip): its value, then
// cleared if reset; -1 in release builds.
int debug_flags_read(int reset);

// A window row's statistics are usable: finite maximum, finite positive normaliser.
__device__ inline bool stats_ok(float m, float z) { return isfinite(m) && isfinite(z) && z > 0.f; }

// Segment holding `item` given the per-segment start field (sorted ascending).
template <int Field>
__device__ __forceinline__ int find_seg(const Launch& a, int item) {
  int e = 0;
  for (int k = 1; k < a.n; ++k) {
    const int start = Field == 0 ? a.seg[k].item0 : Field == 1 ? a.seg[k].row0 : a.seg[k].gitem0;
    if (item >= start) e = k;
  }
  return e;
}

enum { kFieldItem = 0, kFieldRow = 1, kFieldGather = 2 };

// Host-side launchers (return hipSuccess or the launch error).
// window_stats also zeroes the words of clear (the selection's histograms
// or the cooperative selection's words, and header word 0), which only the
// kernels after it use.
hipError_t launch_window_stats(const Launch& a, int items, int dtype, const void* Q, const void* K,
                               float* part_m, float* part_z, const WordRanges& clear, hipStream_t st);
// With lse != nullptr ([sequence][head][W] natural-log row log-sum-exps,
// one per window row) the partials are not read and no row statistics are
// written.
hipError_t launch_window_votes(const Launch& a, int items, int dtype, const void* Q, const void* K,
                               const float* part_m, const float* part_z, const float* lse, float* votes,
                               float* row_stats, hipStream_t st);
// Pooling (pooled may be nullptr: histogram of the input only) with the
// first-digit histogram of each row added into hist[row][2048] (nullptr: none).
hipError_t launch_pool(const Launch& a, int rows, int max_n, const float* votes, float* pooled,
                       uint32_t* hist, hipStream_t st);
// Top-(C-W) per row given the first-digit histograms, in three launches.
// launch_candidates counts, per segment of a row (seg_size positions), the
// scores above the boundary digit and copies the boundary digit's scores to
// cand (one word per score, same layout as scores).  launch_threshold finds
// each row's threshold score from them and how many picks above it and
// positions on it precede each segment, into cut (2 words per row) and
// segcnt (2 * kMaxSegRow words per row).  launch_emit writes every row's
// picks ascending, then the window positions (a.window), and copies their K
// and V rows when K != nullptr (dtype, D give the row size); bypass rows
// (L < C) keep every position.
constexpr int kSegUnit = 2048;    // positions per emit pass
constexpr int kMaxSegRow = 512;   // emit segments per row
int selection_seg_size(long long max_positions);
hipError_t launch_candidates(const Launch& a, int rows, int max_n, const float* scores, const uint32_t* hist,
                             uint32_t* cand, uint32_t* segcnt, hipStream_t st);
hipError_t launch_threshold(const Launch& a, int rows, const uint32_t* hist, const uint32_t* cand, uint32_t* cut,
                            uint32_t* segcnt, hipStream_t st);
hipError_t launch_emit(const Launch& a, int rows, int max_positions, int dtype, const float* scores,
                       const uint32_t* cut, const uint32_t* segcnt, int32_t* indices, const void* K, const void* V,
                       void* K_out, void* V_out, hipStream_t st);
// Threshold and picks of whole rows of at most select_rows_max() prefix
// positions, one workgroup per row, from the pooled scores and their
// first-digit histograms (launch_pool): the picks ascending, then the window
// positions (a.window), into the indices.  Bypass rows are left alone.
int select_rows_max();
hipError_t launch_select_hist(const Launch& a, int rows, const float* scores, const uint32_t* hist,
                              int32_t* indices, hipStream_t st);
// Cooperative selection: coop_segment() positions of a row per workgroup,
// at most coop_max_segments() per row, grid (segs, rows) of at most
// coop_grid_capacity() workgroups; pooling, top-(C-W), window and the K/V
// copy in one launch (pooling widths 1, 3, 5, 7).  coop [rows][coop_row_words()]
// and status (kFusedStatusWords) start at zero.  pooled may be nullptr.
int coop_max_segments();
int coop_segment();
int coop_row_words();
int coop_grid_capacity(int D, int dtype);
hipError_t launch_select_coop(const Launch& a, int rows, int segs, int dtype, const float* votes, float* pooled,
                              unsigned* coop, unsigned* status, int32_t* indices, const void* K, const void* V,
                              void* K_out, void* V_out, hipStream_t st);
// Split selection: rows * splits workgroups, each finding its row's
// threshold and writing and copying slots [split * count / splits, (split
// + 1) * count / splits) of the picks and a share of the window (pooling
// widths 1, 3, 5, 7).  split_kpt() gives the kernel variant (1 ..)
// covering max_p prefix positions (0: none, above split_max_positions()); a
// workgroup's share of the picks must fit split_list_capacity(variant)
// entries.  pooled may be nullptr.  Needs no zeroed words.
int split_kpt(int max_p);
int split_max_positions();
int split_max_splits();
int split_list_capacity(int kpt);
int split_grid_capacity(int kpt, int D, int dtype);
hipError_t launch_select_split(const Launch& a, int rows, int splits, int kpt, int dtype, const float* votes,
                               float* pooled, int32_t* indices, const void* K, const void* V, void* K_out, void* V_out,
                               hipStream_t st);
// Single-read scoring (persistent kernel, one workgroup per CU).
// fused_positions() gives S for the kernel variant, fused_grid() the grid (0
// if the variant cannot run); launch_fused_scoring() returns
// hipErrorNotSupported when the shape is not covered.
// The cooperative selection's status block: kFusedStatusWords zeroed words:
// error flags, arrived groups, the residency decision (kFusedGo or
// kFusedAbort; a host-written kFusedAbort forces the fallback), the
// fallback's work counter, then kArriveGroups arrival counters kArriveStride
// words apart (same-address atomics serialise, so the workgroups' arrivals
// are spread over separate lines).
constexpr unsigned kFusedGo = 1, kFusedAbort = 2;
constexpr int kArriveGroups = 16;
constexpr int kArriveStride = 64;
constexpr int kFusedStatusWords = kArriveStride * (kArriveGroups + 1);
// Residency handshake of kernels whose workgroups wait for each other (the
// single-read scoring and the cooperative selection).  They need every
// workgroup of the grid running at once, which a plain launch of a grid that
// fits the device gives on an otherwise idle device but does not promise.
// It runs in two parts so that it can overlap work that depends on no other
// workgroup:
//  * arrival, issued at kernel start before any K load (so the atomic is
//    not queued behind the first tiles): one of kArriveGroups counters on
//    separate lines (arrivals on one word would be serialised);
//  * the decision, in the exchange wave before its first read of another
//    workgroup's slot: the last arrival of a group counts the group, the
//    last group decides GO; a workgroup that has waited longer than the
//    bound decides ABORT.  Both are a compare-and-swap on one zeroed word,
//    so every workgroup follows the same decision, and GO implies that all
//    of them are resident.
// The residency bound: a workgroup that has waited this long for the others
// to arrive decides ABORT.  200 us, in ticks of the device's constant-rate
// wall clock (s_memrealtime), whose rate the host reads from the device
// (hipDeviceAttributeWallClockRate) and passes in Launch::residency_ticks.
constexpr long long kResidencyMicros = 200;
// Workgroup number and count over the whole grid (1-, 2- or 3-dimensional).
__device__ inline unsigned flat_block() {
  return blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
}
__device__ inline unsigned flat_grid() { return gridDim.x * gridDim.y * gridDim.z; }
__device__ inline unsigned arrival_group(unsigned grid) {
  const unsigned ng = grid < (unsigned)kArriveGroups ? grid : (unsigned)kArriveGroups;
  return flat_block() % ng;
}
__device__ inline unsigned arrive(unsigned* status) {
  unsigned* ctr = status + kArriveStride * (1 + arrival_group(flat_grid()));
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}
// The first half of the decision, once the arrival's count has returned:
// the last arrival of a group counts the group, and the last group decides
// GO.  Lane 0 of the calling wave acts.
__device__ inline void decide_begin(unsigned* status, unsigned arrived) {
  if ((threadIdx.x & 63) == 0) {
    unsigned* groups = status + 1;
    unsigned* state = status + 2;
    const unsigned grid = flat_grid();
    const unsigned ng = grid < (unsigned)kArriveGroups ? grid : (unsigned)kArriveGroups;
    const unsigned g = arrival_group(grid);
    const unsigned members = (grid - g + ng - 1) / ng;
    if (arrived == members) {
      const unsigned done = __hip_atomic_fetch_add(groups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
      if (done == ng) {
        unsigned expect = 0u;
        __hip_atomic_compare_exchange_strong(state, &expect, kFusedGo, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}
// The second half: wait for the decision, deciding ABORT after the bound.
// Lane 0 of the calling wave waits; the decision is returned to every lane.
// An ABORT is also recorded as fallback_bit in the call's flags (err).
__device__ inline unsigned decide_end(unsigned* status, unsigned* err, unsigned fallback_bit, long long ticks) {
  unsigned s = 0u;
  if ((threadIdx.x & 63) == 0) {
    unsigned* state = status + 2;
    const long long t0 = wall_clock64();
    while ((s = __hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0u) {
      if (wall_clock64() - t0 > ticks) {
        unsigned expect = 0u;
        __hip_atomic_compare_exchange_strong(state, &expect, kFusedAbort, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (s == kFusedAbort) raise_error(err, fallback_bit);
  }
  return (unsigned)__builtin_amdgcn_readfirstlane((int)s);
}
__device__ inline unsigned decide(unsigned* status, unsigned arrived, unsigned* err, unsigned fallback_bit,
                                  long long ticks) {
  decide_begin(status, arrived);
  return decide_end(status, err, fallback_bit, ticks);
}

// The single-read scoring kernel's per-call words, and the selection that
// can be fused into it (pooling, top-k, window, K/V copy).  Shared words are
// cleared by the kernel's workgroups, a share each, before they arrive (and
// so are words that the kernels after it in the call need at zero); the
// arrival, the residency decision and the fallback's counters carry a
// per-call token instead of starting from zero, and the kernel's flags go to
// the tagged header word, so the call needs no fill launch.
constexpr int kHaloWords = 8;           // per chunk: its first 3 and last 3 votes, tagged

struct FusedSel {
  int on;                       // 1: select in the scoring kernel (the selection's arrays are used)
  int force_abort;              // testing: decide ABORT at once
  unsigned long long token;     // this call's token (low two bits zero)
  unsigned long long* errw;     // the header's tagged flag word (kTaggedWord)
  unsigned long long* flags;    // [grid] arrival tokens, then the decision word, then 3 claim counters
  unsigned long long* cw;       // [exchange slot] the chunk's count word
  unsigned long long* halo;     // [exchange slot][kHaloWords]
  unsigned long long* clr[4];   // ranges of 8-byte words the launch clears (a share per workgroup), or nullptr
  long long clr_words[4];
  int clr_early;                // the first clr_early ranges are published words: cleared before the arrival
  unsigned* cslot;              // [exchange slot][64] the chunk's coarse histogram, count + 1
  unsigned* fslot;              // [exchange slot][32] its fine histogram inside the coarse bin of tau, count + 1
  unsigned long long* rowfb;    // [row][2] fallback completion counters (token-tagged)
  unsigned long long* cand;     // candidates, indexed like the votes
  float* pooled;                // optional pooled scores out (indexed like the votes), or nullptr
  float* kslot;                 // [exchange slot][512] the chunk's pooled scores, kept for the end phase
  int32_t* indices;
  const void* V;
  void* K_out;
  void* V_out;
};
constexpr int kFlagWordsMax = 1024;     // arrival tokens of a grid of up to this many workgroups
constexpr int kFusedMaxRounds = 2048;   // rounds of one fused-selection launch
constexpr int kFusedFlagWords = kFlagWordsMax + 8;
// Pooling widths the fused selection covers (radius up to 3).
__host__ __device__ inline bool fused_select_kernel_ok(int kernel) { return kernel >= 1 && kernel <= 7 && kernel % 2 == 1; }

int fused_positions(int W, int D);
int fused_grid(int W, int D);
int fused_exchange_bytes();  // per (sequence, head, chunk) exchange slot
// Exchange slots per head for fc chunks: fc rounded up to whole read passes
// of the exchange wave (the padding is never written and never merged).
__host__ __device__ inline int fused_slot_stride(int fc) { return (fc + 63) / 64 * 64; }
// With lse != nullptr (as for launch_window_votes) the workgroups exchange
// nothing and need not be co-resident: exchange is not used.
// With sel.on the kernel also selects: indices and K/V rows are written.
// Nothing needs clearing before the launch: the workgroups clear sel.clr's
// ranges (the exchange slots among them) before their arrival, and the
// arrival, the decision, the fallback's counters and the flags carry
// sel.token.  sel.force_abort decides ABORT at once (testing).
hipError_t launch_fused_scoring(const Launch& a, const void* Q, const void* K, const float* lse, unsigned* exchange,
                                float* votes, float* row_stats, const FusedSel& sel, hipStream_t st);
hipError_t launch_fill_u32(unsigned* p, long long n, unsigned v, hipStream_t st);
// Zero up to kZeroRanges byte ranges in one launch (16-byte aligned pointers
// and sizes, else hipErrorInvalidValue; empty ranges are skipped).
constexpr int kZeroRanges = 4;
struct ZeroRanges {
  void* p[kZeroRanges];
  long long bytes[kZeroRanges];
};
hipError_t launch_zero(const ZeroRanges& r, hipStream_t st);
// Validating mode: sets kErrNonFinite in *err if any of the n 16-byte units
// at p holds a non-finite value of the element type (dtype 1: bf16, 0: fp32).
hipError_t launch_check_finite(const void* p, long long n16, int dtype, unsigned* err, hipStream_t st);
// The same for n float32 values (any count, 4-byte alignment).
hipError_t launch_check_finite_f32(const float* p, long long n, unsigned* err, hipStream_t st);
// Refresh selection: turn the selection's relative entries into final
// indices (protected head first) and gather token ids with them.
hipError_t launch_refresh_finish(int rows, int n, int keep, int head, int tail, bool picked, int32_t* indices,
                                 const int32_t* tokens, int32_t* tokens_out, hipStream_t st);
int gather_rows_per_block(int D, int dtype);

// Streaming-read probes (kvsel_probe.hip): mode 0, 1, 2 direct-to-LDS tiles
// (8 waves x 1 tile, 8 waves x 2 tiles, 4 waves x 4 tiles in flight; bytes a
// multiple of 128 KB), mode 3 vector loads; one workgroup per CU (cus).
int probe_sink_words(int cus);
hipError_t launch_probe(int mode, const void* src, long long bytes, unsigned* sink, int cus, hipStream_t st);

hipError_t launch_gather(const Launch& a, int items, int dtype, const void* K, const void* V,
                         const int32_t* indices, void* K_out, void* V_out, hipStream_t st);

}  // namespace kvsel
