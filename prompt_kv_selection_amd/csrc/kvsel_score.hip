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
// rows is the B operand, streamed from HBM into a per-wave LDS ring with
// coalesced 1 KiB direct-to-LDS loads, then read by each lane as 16 bytes per
// k-step of one K row.  In the 32x32 accumulator a lane owns one
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

// Instrumentation hook (kernel k: 0 statistics, 1 votes; point 0..15 of the
// calling wave); empty unless a profiling build defines it.
#ifndef KVSEL_SCORE_MARK
#define KVSEL_SCORE_MARK(k, point)
#endif

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;   // finite "no position seen yet" max
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Window row held in accumulator register r by lane half g (32x32 MFMA
// output layout: lane l holds column l % 32, rows 8*(r/4) + 4*(l/32) + r%4).
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// ---- K tiles: 32 prompt rows streamed from HBM straight into LDS.
//
// Each wave owns a ring of RING tile buffers.  A tile load is NL
// global_load_lds_dwordx4 instructions: instruction i moves 64 consecutive
// 16-byte pieces of the tile (1 KiB, coalesced), lane l's piece landing at
// LDS byte M0 + 16 l.  Piece c of tile row r is stored at slot
// r * PR + (c ^ (r % PR)), so the operand reads below (32 rows, one piece
// each) hit distinct LDS banks.
template <typename T, int D>
struct TileGeom {
  static constexpr int PR = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
  static constexpr int NL = PR / 2;                   // load instructions per tile
  static constexpr int PIECES = 32 * PR;              // pieces per tile
  static constexpr int RING = PR >= 32 ? 1 : 2;       // tiles in flight per wave (LDS budget)
};

// Byte offsets (from the tile's first row) of lane's piece in each load
// instruction; fixed for the life of the kernel.
template <typename T, int D>
struct TileOffsets {
  using G = TileGeom<T, D>;
  unsigned v[G::NL];
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int i = 0; i < G::NL; ++i) v[i] = piece_offset(i, lane, 32);
  }
  // Offset with rows at or past `rows` replaced by row rows - 1.
  static __device__ __forceinline__ unsigned piece_offset(int i, int lane, int rows) {
    const int piece = i * 64 + lane;
    const int r = piece / G::PR;
    const int c = (piece % G::PR) ^ (r & (G::PR - 1));
    return (unsigned)((min(r, rows - 1) * G::PR + c) * 16);
  }
};

// Load the `rows` (1..32) rows starting at `first` as one tile; rows past
// `rows` repeat the last row (read, never used).
// With kNT the loads are non-temporal.
template <typename T, int D, bool kNT>
__device__ __forceinline__ void issue_tile(const T* first, int rows, const TileOffsets<T, D>& off,
                                           const uint4* lds_tile, int lane) {
  using G = TileGeom<T, D>;
  const unsigned base = (unsigned)(uintptr_t)lds_tile;
#pragma unroll
  for (int i = 0; i < G::NL; ++i) {
    const unsigned o = rows >= 32 ? off.v[i] : TileOffsets<T, D>::piece_offset(i, lane, rows);
    if constexpr (kNT)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(base + i * 1024)), "v"(o), "s"(first)
                   : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(base + i * 1024)), "v"(o), "s"(first)
                   : "memory", "m0");
  }
}

// Wait until at most `after` of this wave's tile loads are still in flight
// (the loads of one wave complete in issue order).  These loads are not seen
// by the compiler's own wait insertion, so every wait on them is explicit.
template <int NL>
__device__ __forceinline__ void wait_tiles(int after) {
  switch (after) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory"); break;
  }
}

// Operand registers of one 32-row tile (a Qwin row block or 32 K rows).
// Lane half g takes pieces 2 s + g (s < PR / 2) of row lane % 32: for bf16
// these are the 8-element k-steps of v_mfma_f32_32x32x16_bf16; for fp32 each
// piece feeds four v_mfma_f32_32x32x2f32 steps, pairing element 8q+e (half 0)
// with 8q+4+e (half 1).
template <typename T, int D>
struct Operands;

template <int D>
struct Operands<__bf16, D> {
  static constexpr int NS = D / 16;
  bf16x8 v[NS];
  __device__ __forceinline__ void from_tile(const uint4* tile, int n, int g) {
    constexpr int PR = TileGeom<__bf16, D>::PR;
#pragma unroll
    for (int s = 0; s < NS; ++s) v[s] = __builtin_bit_cast(bf16x8, tile[n * PR + ((2 * s + g) ^ (n & (PR - 1)))]);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < NS; ++s) v[s] = bf16x8{};
  }
};

template <int D>
struct Operands<float, D> {
  static constexpr int NQ = D / 8;
  f32x4 v[NQ];
  __device__ __forceinline__ void from_tile(const uint4* tile, int n, int g) {
    constexpr int PR = TileGeom<float, D>::PR;
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[q] = __builtin_bit_cast(f32x4, tile[n * PR + ((2 * q + g) ^ (n & (PR - 1)))]);
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

// Add one logit x to (running maximum m, sum z of exp2(. - m)) with a single
// exponential: exp2(-|x - m|) rescales whichever side is smaller.
__device__ __forceinline__ void online_add(float& m, float& z, float x) {
#pragma clang fp contract(off)
  const float d = x - m;
  const float e = exp2_fast(-fabsf(d));
  z = d > 0.f ? fmaf(z, e, 1.f) : z + e;
  m = fmaxf(m, x);
}

// Merge (mo, zo) into (m, z): running maximum in base 2 and the sum of
// exponentials rescaled to it (one exponential: the larger side keeps scale 1).
__device__ __forceinline__ void lse_merge(float& m, float& z, float mo, float zo) {
#pragma clang fp contract(off)
  const float d = mo - m;
  const float e = exp2_fast(-fabsf(d));
  z = d > 0.f ? fmaf(z, e, zo) : fmaf(zo, e, z);
  m = fmaxf(m, mo);
}

// Qwin row block rb (32 rows) is staged through LDS like a K tile, by wave
// rb, so that no load the compiler tracks is pending in the tile loops.
template <typename T, int D, int RB>
__device__ __forceinline__ void issue_queries(const Launch& a, const Seg& s, int h, const T* __restrict__ Q,
                                              uint4 (*qt)[TileGeom<T, D>::PIECES], const TileOffsets<T, D>& off,
                                              int wave, int lane) {
  if (wave < RB) {  // the group's query heads are consecutive: one block of group_rows rows
    const long long qh = (long long)s.b * a.heads + (long long)h * (a.group > 1 ? a.group : 1);
    const T* q = Q + qh * (long long)a.W * D + (long long)wave * 32 * D;
    issue_tile<T, D, false>(q, min(32, group_rows(a) - wave * 32), off, qt[wave], lane);
  }
}

// Operands of the staged Qwin; rows past group_rows are zero.
template <typename T, int D, int RB>
__device__ __forceinline__ void queries_from_lds(const Launch& a, const uint4 (*qt)[TileGeom<T, D>::PIECES], int n,
                                                 int g, Operands<T, D> (&qa)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    qa[rb].from_tile(qt[rb], n, g);
    if (rb * 32 + n >= group_rows(a)) qa[rb].zero();
  }
}

// Waves of a scoring workgroup.  Up to two 32-row blocks of window rows, four
// waves, each holding the Qwin operands in registers and two K tiles in
// flight.  Three or four blocks of bf16 rows (grouped heads), eight waves,
// two per SIMD, each with one tile in flight and the Qwin operands read from
// LDS per tile: a tile's MFMA and exponential chains for 128 rows take a
// wave about 2 us, so with one wave per SIMD nothing would cover them (fp32
// tiles are twice the size and do not fit eight waves' buffers).  The item
// is kChunk positions either way.
template <typename T, int D, int RB>
struct ScoreGeom {
  static constexpr bool kQLds = RB >= 3 && sizeof(T) == 2;  // Qwin operands (and, for votes, row scales) from LDS
  static constexpr int NW = kQLds ? 8 : kWaves;            // waves per workgroup
  static constexpr int WT = kChunk / (NW * 32);            // tiles per wave per item
  static constexpr int RING = kQLds ? 1 : TileGeom<T, D>::RING;  // tiles in flight per wave
  static_assert(NW * WT * 32 == kChunk, "an item is kChunk positions");
  // Row statistics are kept per sub-range of kSubTiles tiles of every item
  // (a wave's tiles of each item form SUB of them), and a chunk's partial
  // merges the kSubs sub-ranges in order: the same summation for either
  // wave count, so grouped heads match their expanded heads bit for bit.
  static constexpr int kSubTiles = 4;
  static constexpr int SUB = WT / kSubTiles;
  static constexpr int kSubs = NW * SUB;
  static_assert(SUB * kSubTiles == WT && kSubs == kChunk / (32 * kSubTiles), "sub-ranges tile the item");
};

// One scoring item: chunk c (kChunk positions) of head h of segment e.  A
// wave covers WT tiles of the chunk starting at pb, of which nt hold
// positions below the kernel's limit (L for statistics, P for votes).
template <typename T, int D>
struct Item {
  int e, h, c, pb, nt;
  const T* kh;
  int L;
};

template <typename T, int D, bool kVotes, int WT>
__device__ __forceinline__ Item<T, D> locate_item(const Launch& a, const T* __restrict__ K, int item, int wave) {
  Item<T, D> it;
  it.e = find_seg<kFieldItem>(a, item);
  const Seg& s = a.seg[it.e];
  const int local = item - s.item0;
  const int hl = local / s.nch;
  it.c = local - hl * s.nch;
  it.h = s.h0 + hl;
  it.L = s.L;
  it.kh = K + s.kv_off + (long long)it.h * s.L * D;
  it.pb = it.c * kChunk + wave * (WT * 32);
  const int limit = kVotes ? s.L - a.W : s.L;
  it.nt = max(0, min(WT, (limit - it.pb + 31) / 32));
  return it;
}

// Contiguous, balanced range of items of this workgroup.
__device__ __forceinline__ void item_range(int items, int& lo, int& hi) {
  lo = (int)((long long)blockIdx.x * items / gridDim.x);
  hi = (int)((long long)(blockIdx.x + 1) * items / gridDim.x);
}

// The K tile stream of one wave over all items of its workgroup's range:
// tile loads run up to RING tiles ahead of the consumer, across item
// boundaries; buffer = tile count % RING.
template <typename T, int D, bool kVotes, int WT, int RING, bool kNT>
struct WaveStream {
  using G = TileGeom<T, D>;
  uint4 (*ring)[G::PIECES];
  TileOffsets<T, D> off;
  int issued, done;  // tiles issued / consumed by this wave
  int item, hi, t;   // issue cursor: item, next tile in it
  Item<T, D> cur;    // the cursor's item
  __device__ __forceinline__ void start(const Launch& a, const T* __restrict__ K, int lo, int hi_, int wave,
                                        int lane) {
    off.init(lane);
    issued = done = 0;
    hi = hi_;
    item = lo;
    t = 0;
    if (item < hi) cur = locate_item<T, D, kVotes, WT>(a, K, item, wave);
    for (int r = 0; r < RING; ++r) issue_next(a, K, wave, lane);
  }
  __device__ __forceinline__ void issue_next(const Launch& a, const T* __restrict__ K, int wave, int lane) {
    while (item < hi && t >= cur.nt) {
      ++item;
      t = 0;
      if (item < hi) cur = locate_item<T, D, kVotes, WT>(a, K, item, wave);
    }
    if (item >= hi) return;
    const int p0 = cur.pb + t * 32;
    issue_tile<T, D, kNT>(cur.kh + (long long)p0 * D, min(32, cur.L - p0), off, ring[issued % RING], lane);
    ++t;
    ++issued;
  }
  // The next tile in stream order has landed; returns its buffer.
  __device__ __forceinline__ const uint4* wait() {
    wait_tiles<G::NL>(issued - done - 1);
    return ring[done % RING];
  }
  // After the operand reads of the tile (waited for here): reuse its buffer
  // for the next load.
  __device__ __forceinline__ void release(const Launch& a, const T* __restrict__ K, int wave, int lane) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    ++done;
    issue_next(a, K, wave, lane);
  }
};

// Stage Qwin of (segment e, head h) and read it into operand registers
// (unless they are read from LDS per tile).  On entry no wave still reads qt;
// on exit every wave has its copy, or qt holds it.  Waits for all of this
// wave's loads in flight (a K tile stream drains once here).
template <typename T, int D, int RB>
__device__ __forceinline__ void stage_queries(const Launch& a, int e, int h, const T* __restrict__ Q,
                                              uint4 (*qt)[TileGeom<T, D>::PIECES], const TileOffsets<T, D>& off,
                                              int wave, int lane, Operands<T, D> (&qa)[RB]) {
  issue_queries<T, D, RB>(a, a.seg[e], h, Q, qt, off, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (!ScoreGeom<T, D, RB>::kQLds) queries_from_lds<T, D, RB>(a, qt, lane & 31, lane >> 5, qa);
}

// Row block rb's Qwin operands: the registers staged above, or read from
// LDS for this tile (rows past group_rows are zero).
template <typename T, int D, int RB>
__device__ __forceinline__ Operands<T, D> query_block(const Launch& a, const uint4 (*qt)[TileGeom<T, D>::PIECES],
                                                      const Operands<T, D> (&qa)[RB], int rb, int n, int g) {
  if constexpr (ScoreGeom<T, D, RB>::kQLds) {
    Operands<T, D> q;
    q.from_tile(qt[rb], n, g);
    if (rb * 32 + n >= group_rows(a)) q.zero();
    return q;
  } else {
    return qa[rb];
  }
}

// Partial row statistics.  Persistent workgroups of kWaves waves walk a
// contiguous range of (sequence, head, chunk) items.  Consecutive items of
// one head form a run; for each window row i < W the run's base-2 maximum of
// the visible logits and sum of exp2(x - max) are written to the slot of its
// last chunk, and the other chunks of the run get (kNegBig, 0), which leaves
// any merge unchanged.
template <typename T, int D, int RB, bool kNT>
__global__ __launch_bounds__((ScoreGeom<T, D, RB>::NW * 64)) void window_stats_kernel(const Launch a, int items,
                                                                  const T* __restrict__ Q,
                                                                  const T* __restrict__ K,
                                                                  float* __restrict__ part_m,
                                                                  float* __restrict__ part_z,
                                                                  const WordRanges clear) {
  // Every multiply-add below is written out (fmaf) and nothing else is
  // fused, so the statistics do not depend on how the compiler schedules a
  // kernel variant: grouped heads match their expanded heads bit for bit.
#pragma clang fp contract(off)
  using G = TileGeom<T, D>;
  using SG = ScoreGeom<T, D, RB>;
  __shared__ uint4 ring[SG::NW][SG::RING][G::PIECES];
  __shared__ uint4 qt[RB][G::PIECES];
  __shared__ float sm[2][SG::kSubs][RB * 32], sz[2][SG::kSubs][RB * 32];
  const int W = a.W, R = group_rows(a);  // rows: window row i of the group's query head i / W
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  int lo, hi;
  item_range(items, lo, hi);

  KVSEL_SCORE_MARK(0, 0);
  WaveStream<T, D, false, SG::WT, SG::RING, kNT> ws;
  ws.ring = ring[wave];
  ws.start(a, K, lo, hi, wave, lane);

  // Side duty: clear the words the kernels after this one use, 16 bytes a
  // store where the range allows.
  {
    const long long t0 = (long long)blockIdx.x * blockDim.x + threadIdx.x, nt = (long long)gridDim.x * blockDim.x;
#pragma unroll
    for (int r = 0; r < kClearRanges; ++r) {
      const bool wide = (reinterpret_cast<uintptr_t>(clear.p[r]) & 15) == 0;
      const long long n4 = wide ? clear.n[r] / 4 : 0;
      for (long long q = t0; q < n4; q += nt) reinterpret_cast<uint4*>(clear.p[r])[q] = make_uint4(0u, 0u, 0u, 0u);
      for (long long q = 4 * n4 + t0; q < clear.n[r]; q += nt) clear.p[r][q] = 0u;
    }
  }

  Operands<T, D> qa[RB];
  // This lane's running statistics of the current run: row n of each row
  // block over the lane's half of every tile's positions.
  float m[SG::SUB][RB], z[SG::SUB][RB];
  int runs = 0;
  for (int item = lo; item < hi; ++item) {
    const Item<T, D> it = locate_item<T, D, false, SG::WT>(a, K, item, wave);
    const Seg& s = a.seg[it.e];
    const int L = s.L, P = L - W;
    const bool first = item == lo || find_seg<kFieldItem>(a, item - 1) != it.e ||
                       (item - 1 - s.item0) / s.nch != it.h - s.h0;
    const bool last = item + 1 == hi || find_seg<kFieldItem>(a, item + 1) != it.e ||
                      (item + 1 - s.item0) / s.nch != it.h - s.h0;
    if (first) {
      // qt is free: every wave read it before the barrier that ended the
      // previous staging, and has since passed that run's final barrier.
      stage_queries<T, D, RB>(a, it.e, it.h, Q, qt, ws.off, wave, lane, qa);
      KVSEL_SCORE_MARK(0, 1);
#pragma unroll
      for (int u = 0; u < SG::SUB; ++u)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          m[u][rb] = kNegBig;
          z[u][rb] = 0.f;
        }
    }

    for (int t = 0; t < it.nt; ++t) {
      const int p0 = it.pb + t * 32;
      const int j = p0 + n;
      Operands<T, D> kt;
      kt.from_tile(ws.wait(), n, g);
      KVSEL_SCORE_MARK(0, 2 + (t & 7));
      ws.release(a, K, wave, lane);  // the tile is in registers: refill its buffer now
      // K.Q^T puts a lane on a window row (row n of the block) and its
      // registers on positions p0 + acc_row(r, g), so the tile's maximum
      // and sum of exponentials are lane-local, then merged into the run's
      // statistics once per tile.  Rows past R hold zero queries and are
      // never written, so only the causal bound (position <= P + window row)
      // masks, and only in tiles reaching past P.  A row block lies within
      // one query head (W is a multiple of 32 when heads are grouped).
      const bool full = p0 + 31 <= P;
      (void)j;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x16 act = tile_dot<D>(kt, query_block<T, D, RB>(a, qt, qa, rb, n, g));
        const int i = (rb * 32) % W + n;  // this lane's window row
        float tm = kNegBig;
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) tm = fmaxf(tm, act[r]);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jj = p0 + acc_row(r, g);
            if (!(jj < L && jj <= P + i)) act[r] = -INFINITY;
            tm = fmaxf(tm, act[r]);
          }
        }
        const float tms = tm * a.scale2;
        float tz = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) tz += exp2_fast(fmaf(act[r], a.scale2, -tms));
        // The tile's sub-range (t / kSubTiles) keeps its own running statistics.
#pragma unroll
        for (int u = 0; u < SG::SUB; ++u)
          if (t / SG::kSubTiles == u) lse_merge(m[u][rb], z[u][rb], tms, tz);
      }
    }

    const long long slot = (s.part_base + (long long)it.h * s.nch + it.c) * R;
    if (!last) {
      // The run's statistics go to its last chunk; the others hold the
      // neutral element of the merge.
      if ((int)threadIdx.x < R) {
        part_m[slot + threadIdx.x] = kNegBig;
        part_z[slot + threadIdx.x] = 0.f;
      }
      continue;
    }

    // Lane n and lane n + 32 hold the same row over the two halves of the
    // positions: merged in that order.
#pragma unroll
    for (int u = 0; u < SG::SUB; ++u)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mo = __shfl_xor(m[u][rb], 32), zo = __shfl_xor(z[u][rb], 32);
        if (g == 0) lse_merge(m[u][rb], z[u][rb], mo, zo);
      }

    // Run k uses buffer k & 1: the merge of run k happens before any wave
    // passes the barrier of run k + 1.  Sub-range wave * SUB + u of the item.
    const int pbuf = runs++ & 1;
    if (g == 0) {
#pragma unroll
      for (int u = 0; u < SG::SUB; ++u)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          sm[pbuf][wave * SG::SUB + u][rb * 32 + n] = m[u][rb];
          sz[pbuf][wave * SG::SUB + u][rb * 32 + n] = z[u][rb];
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < R) {
      const int i = threadIdx.x;
      float mm = sm[pbuf][0][i], zz = sz[pbuf][0][i];
#pragma unroll
      for (int v = 1; v < SG::kSubs; ++v) lse_merge(mm, zz, sm[pbuf][v][i], sz[pbuf][v][i]);
      part_m[slot + i] = mm;
      part_z[slot + i] = zz;
    }
  }
  KVSEL_SCORE_MARK(0, 10);
}

// Final (max, 1/sum) of every row of K/V head h (R = group_rows rows) from
// its nch partials, into s_m / s_iz (rows R .. RB*32-1 get (0, 0): with zero
// queries their logits are 0, so they add nothing).  Thread t < G*R (G =
// kMergeGroups) merges row t % R over chunks t / R, t / R + G, ...; the G
// results per row are then merged through LDS.  The merge order depends on
// the chunks only, not on R, so a row's statistics are the same whether its
// query head is scored alone or with its group.
constexpr int kMergeGroups = 2;
static_assert(kMergeGroups * 128 <= kWaves * 64, "every row of a 128-row group has its threads");
template <int RBW>
__device__ __forceinline__ void merge_partials(const Launch& a, const Seg& s, int h,
                                               const float* __restrict__ part_m, const float* __restrict__ part_z,
                                               float* __restrict__ row_stats, bool write_stats, float* s_gm,
                                               float* s_gz, float* s_m, float* s_iz) {
  const int W = group_rows(a), t = threadIdx.x;  // W: rows of the slot here
  const int G = kMergeGroups;
  const long long base = (s.part_base + (long long)h * s.nch) * W;
  if (t < G * W) {
    const int i = t % W, grp = t / W;
    float mm = kNegBig, zz = 0.f;
    int c = grp;
    // Batches of kMergeBatch independent loads (one batch covers 32 chunks),
    // merged in chunk order.
    constexpr int kMergeBatch = 16;
    for (; c < s.nch; c += kMergeBatch * G) {
      float pm[kMergeBatch], pz[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const bool in = c + u * G < s.nch;
        pm[u] = in ? part_m[base + (long long)(c + u * G) * W + i] : kNegBig;
        pz[u] = in ? part_z[base + (long long)(c + u * G) * W + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u)
        if (c + u * G < s.nch) lse_merge(mm, zz, pm[u], pz[u]);
    }
    s_gm[t] = mm;
    s_gz[t] = zz;
  }
  __syncthreads();
  if (t < RBW) {
    float mm = 0.f, iz = 0.f;
    if (t < W) {
      float zz = 0.f;
      mm = kNegBig;
      for (int grp = 0; grp < G; ++grp) lse_merge(mm, zz, s_gm[grp * W + t], s_gz[grp * W + t]);
      iz = 1.f / zz;
      if (write_stats && !stats_ok(mm, zz)) raise_flag(a, kErrNonFinite);
      if (row_stats != nullptr && write_stats) {
        // row t of the slot: window row t % a.W of query head h * group + t / a.W
        float* rs = row_stats + (((long long)s.b * a.heads) * a.W + (long long)h * W + t) * 2;
        rs[0] = mm * kLn2;
        rs[1] = zz;
      }
    }
    s_m[t] = mm;
    s_iz[t] = iz;
  }
  __syncthreads();
}

// Votes of prefix positions.  Persistent workgroups walk a contiguous range of
// items; at each new head they merge its partial row statistics, then
// recompute each chunk's logits and sum the softmax probabilities over the
// window rows.
template <typename T, int D, int RB, bool kNT>
__global__ __launch_bounds__((ScoreGeom<T, D, RB>::NW * 64)) void window_votes_kernel(
    const Launch a, int items, const T* __restrict__ Q, const T* __restrict__ K,
    const float* __restrict__ part_m, const float* __restrict__ part_z, const float* __restrict__ lse,
    float* __restrict__ votes, float* __restrict__ row_stats) {
#pragma clang fp contract(off)  // as in window_stats_kernel
  using G = TileGeom<T, D>;
  using SG = ScoreGeom<T, D, RB>;
  __shared__ uint4 ring[SG::NW][SG::RING][G::PIECES];
  __shared__ uint4 qt[RB][G::PIECES];
  __shared__ __align__(16) float s_m[RB * 32], s_iz[RB * 32];
  __shared__ float s_gm[SG::NW * 64], s_gz[SG::NW * 64];
  const int W = a.W, R = group_rows(a), Gq = a.group > 1 ? a.group : 1;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  int lo, hi;
  item_range(items, lo, hi);

  KVSEL_SCORE_MARK(1, 0);
  WaveStream<T, D, true, SG::WT, SG::RING, kNT> ws;
  ws.ring = ring[wave];
  ws.start(a, K, lo, hi, wave, lane);

  Operands<T, D> qa[RB];
  // Row scales of the lane's accumulator rows (registers, or read from LDS
  // per tile with eight waves).
  float mr[SG::kQLds ? 1 : RB][16], izr[SG::kQLds ? 1 : RB][16];
  int qe = -1, qh = -1;
  for (int item = lo; item < hi; ++item) {
    const Item<T, D> it = locate_item<T, D, true, SG::WT>(a, K, item, wave);
    const Seg& s = a.seg[it.e];
    const int L = s.L, P = L - W;
    if (it.c * kChunk >= P) continue;  // chunk holds window positions only
    if (it.e != qe || it.h != qh) {
      // With operands read from LDS every wave is done with the previous
      // head's Qwin and scales before they are rewritten.
      if (SG::kQLds && qe >= 0) __syncthreads();
      stage_queries<T, D, RB>(a, it.e, it.h, Q, qt, ws.off, wave, lane, qa);
      qe = it.e;
      qh = it.h;
      if (lse != nullptr) {
        // Row log-sum-exps handed over by the caller: exp(l - lse) is the
        // probability itself, so M = lse * log2(e) and 1/Z = 1.
        if ((int)threadIdx.x < RB * 32) {
          const int i = threadIdx.x;  // window row i % W of query head it.h * Gq + i / W
          const bool row = i < R;
          const float l = row ? lse[((long long)s.b * a.heads) * W + (long long)it.h * R + i] : 0.f;
          if (row && it.c == 0 && !isfinite(l)) raise_flag(a, kErrNonFinite);
          s_m[i] = l * kLog2e;
          s_iz[i] = row ? 1.f : 0.f;
        }
        __syncthreads();
      } else {
        // The run holding chunk 0 of the head starts there: its workgroup
        // alone writes the row statistics.
        merge_partials<RB * 32>(a, s, it.h, part_m, part_z, row_stats, it.c == 0, s_gm, s_gz, s_m, s_iz);
      }
      if constexpr (!SG::kQLds) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = rb * 32 + acc_row(r, g);
            mr[rb][r] = s_m[i];
            izr[rb][r] = s_iz[i];
          }
        // Nobody reads qt or s_m again before the next staging rewrites them.
        __syncthreads();
      }
      KVSEL_SCORE_MARK(1, 1);
    }

    // Votes of each query head of the group: its row blocks' sums.
    float* vout = votes + s.vote_off + (long long)it.h * Gq * s.vote_ld;
    for (int t = 0; t < it.nt; ++t) {
      const int j = it.pb + t * 32 + n;
      Operands<T, D> kt;
      kt.from_tile(ws.wait(), n, g);
      KVSEL_SCORE_MARK(1, 2 + (t & 7));
      ws.release(a, K, wave, lane);  // the tile is in registers: refill its buffer now
      float tot = 0.f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f32x16 acc = tile_dot<D>(query_block<T, D, RB>(a, qt, qa, rb, n, g), kt);
        const int sr = SG::kQLds ? 0 : rb;  // the scales' register set
        if constexpr (SG::kQLds) {
          // acc_row(r, g) for r = 4q .. 4q + 3 is four consecutive rows.
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 m4 = *reinterpret_cast<const float4*>(&s_m[rb * 32 + 8 * q + 4 * g]);
            const float4 z4 = *reinterpret_cast<const float4*>(&s_iz[rb * 32 + 8 * q + 4 * g]);
            mr[0][4 * q] = m4.x;
            mr[0][4 * q + 1] = m4.y;
            mr[0][4 * q + 2] = m4.z;
            mr[0][4 * q + 3] = m4.w;
            izr[0][4 * q] = z4.x;
            izr[0][4 * q + 1] = z4.y;
            izr[0][4 * q + 2] = z4.z;
            izr[0][4 * q + 3] = z4.w;
          }
        }
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) part = fmaf(exp2_fast(fmaf(acc[r], a.scale2, -mr[sr][r])), izr[sr][r], part);
        tot += part;
        if (rb + 1 == RB || (Gq > 1 && ((rb + 1) * 32) % W == 0)) {  // the last row block of a query head
          const float other = __shfl_xor(tot, 32);
          // Same expression for every position: (half 0 rows) + (half 1 rows).
          const float v = g == 0 ? tot + other : other + tot;
          if (g == 0 && j < P) vout[(long long)((rb * 32) / W) * s.vote_ld + j] = v;
          tot = 0.f;
        }
      }
    }
  }
  KVSEL_SCORE_MARK(1, 10);
}

// Persistent grid: as many workgroups as can be resident at once (cached per
// kernel variant and device), never more than there are items.
template <typename Kern>
static int resident_grid(Kern kern, int threads, int items) {
  static int per_cu[64] = {};
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return items;
  if (per_cu[dev] == 0) {
    int n = 0, c = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess || n < 1) n = 1;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 1;
    cus[dev] = c;
    per_cu[dev] = n;
  }
  const long long slots = (long long)per_cu[dev] * cus[dev];
  return (int)(items < slots ? items : slots);
}

template <typename T, int D, int RB, bool kNT>
static hipError_t stats_nt(const Launch& a, int items, const void* Q, const void* K, float* pm, float* pz,
                           const WordRanges& clear, hipStream_t st) {
  constexpr int threads = ScoreGeom<T, D, RB>::NW * 64;
  const int grid = resident_grid(window_stats_kernel<T, D, RB, kNT>, threads, items);
  hipLaunchKernelGGL((window_stats_kernel<T, D, RB, kNT>), dim3(grid), dim3(threads), 0, st, a, items,
                     (const T*)Q, (const T*)K, pm, pz, clear);
  return hipGetLastError();
}
template <typename T, int D, int RB>
static hipError_t stats_t(const Launch& a, int items, const void* Q, const void* K, float* pm, float* pz,
                          const WordRanges& clear, hipStream_t st) {
  return a.k_nt ? stats_nt<T, D, RB, true>(a, items, Q, K, pm, pz, clear, st)
                : stats_nt<T, D, RB, false>(a, items, Q, K, pm, pz, clear, st);
}

template <typename T, int D, int RB>
static hipError_t votes_t(const Launch& a, int items, const void* Q, const void* K, const float* pm,
                          const float* pz, const float* lse, float* votes, float* rs, hipStream_t st) {
  constexpr int threads = ScoreGeom<T, D, RB>::NW * 64;
  if (a.k_nt) {
    const int grid = resident_grid(window_votes_kernel<T, D, RB, true>, threads, items);
    hipLaunchKernelGGL((window_votes_kernel<T, D, RB, true>), dim3(grid), dim3(threads), 0, st, a, items,
                       (const T*)Q, (const T*)K, pm, pz, lse, votes, rs);
  } else {
    const int grid = resident_grid(window_votes_kernel<T, D, RB, false>, threads, items);
    hipLaunchKernelGGL((window_votes_kernel<T, D, RB, false>), dim3(grid), dim3(threads), 0, st, a, items,
                       (const T*)Q, (const T*)K, pm, pz, lse, votes, rs);
  }
  return hipGetLastError();
}

#define KVSEL_DISPATCH(FN, ...)                                                              \
  do {                                                                                       \
    const int rb = (group_rows(a) + 31) / 32;                                                \
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
                               float* part_m, float* part_z, const WordRanges& clear, hipStream_t st) {
  KVSEL_DISPATCH(stats_t, a, items, Q, K, part_m, part_z, clear, st);
}

hipError_t launch_window_votes(const Launch& a, int items, int dtype, const void* Q, const void* K,
                               const float* part_m, const float* part_z, const float* lse, float* votes,
                               float* row_stats, hipStream_t st) {
  KVSEL_DISPATCH(votes_t, a, items, Q, K, part_m, part_z, lse, votes, row_stats, st);
}

}  // namespace kvsel
