// Selection kernels for gfx950: 1-D pooling of the votes, per-head top-k with
// lowest-index ties, and the K/V gather.
//
// Method (web page "SnapKV: selecting the KV cache for long prompts with an
// observation window"):
//  * section "pooling spreads a peak into a neighbourhood preference":
//    stride-1 pooling of width k (odd) over the prefix votes with zero
//    padding; avg divides by k at the edges too; max takes the in-range
//    maximum;
//  * section "one full selection computed from Q and K": keep the C - W
//    prefix positions with the highest pooled score (equal scores go to the
//    lowest index), append the W window positions, and gather K and V rows
//    with the same indices; a prompt shorter than the budget keeps every
//    position.
//
// Top-k.  Pooled scores are finite and >= 0, so their float32 bit patterns
// order like the values (-0 is read as +0).  A most-significant-first radix select (digits of
// 11, 11 and 10 bits) finds the threshold pattern tau of the (C-W)-th largest
// score and how many tau-equal positions are still needed.  The first digit's
// histogram is built by the pooling kernel across many workgroups.  A
// candidates workgroup per (segment, row) then counts its positions above the
// boundary digit and copies the boundary digit's scores into the segment's
// range of a candidate buffer; one 1024-thread workgroup per row gathers the
// (few) candidates into LDS, finishes the select there and turns the
// per-segment counts above tau and on tau into prefixes.  An emit workgroup
// per segment then knows how many picks precede it: it scans its positions
// in index order, writes its picks (the lowest tau-equal indices first) at
// their final slots, and copies their K and V rows.

#include <mutex>

#include "kvsel_internal.h"

// Instrumentation hook at the phases of the select kernel (point 0..4);
// empty unless a profiling build defines it.
#ifndef KVSEL_SELECT_MARK
#define KVSEL_SELECT_MARK(point)
#endif

// Instrumentation hook of the cooperative selection (point 0..7 of the
// calling workgroup); empty unless a profiling build defines it.
#ifndef KVSEL_SELROWS_MARK
#define KVSEL_SELROWS_MARK(point)
#endif

namespace kvsel {

// Radix key of a score word.  Scores are >= 0, so the bit patterns order like
// the values, except that -0 (sign bit alone) would rank above every positive
// score: it is taken as +0, which it equals.
__device__ __forceinline__ uint32_t score_key(uint32_t bits) { return bits == 0x80000000u ? 0u : bits; }

// Inclusive scan over the NT threads of the block; `total` gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  constexpr int kWavesPerBlock = NT / 64;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) sh[wv] = v;
  __syncthreads();
  if (wv == 0) {
    uint32_t t = lane < kWavesPerBlock ? sh[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kWavesPerBlock; off <<= 1) {
      const uint32_t o = __shfl_up(t, off);
      if (lane >= off) t += o;
    }
    if (lane < kWavesPerBlock) sh[lane] = t;
  }
  __syncthreads();
  const uint32_t base = wv ? sh[wv - 1] : 0u;
  total = sh[kWavesPerBlock - 1];
  __syncthreads();
  return v + base;
}

// Given hist[] (LDS) of the digits of the candidates, find the digit holding
// the need-th largest: returns (digit, rank of the target inside the digit).
template <int NT>
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int nb, uint32_t need, uint32_t* sh,
                                           uint32_t* s_digit, uint32_t* s_need) {
  const int tid = threadIdx.x;
  const int per = nb / NT;
  uint32_t local = 0;
  for (int u = 0; u < per; ++u) local += hist[nb - 1 - (tid * per + u)];
  uint32_t total;
  const uint32_t incl = block_scan<NT>(local, sh, total);
  const uint32_t excl = incl - local;
  if (excl < need && need <= incl) {
    uint32_t cum = excl;
    for (int u = 0; u < per; ++u) {
      const uint32_t d = (uint32_t)(nb - 1 - (tid * per + u));
      if (cum + hist[d] >= need) {
        *s_digit = d;
        *s_need = need - cum;
        break;
      }
      cum += hist[d];
    }
  }
  __syncthreads();
}

constexpr int kCand = 16384;
constexpr int kPoolSpan = 8;
constexpr int kMaxPoolRadius = 31;  // pooling width up to 63
static_assert(2 * kMaxPoolRadius < kPoolBlock, "the right halo is loaded by one thread per position");

// Candidates kernel: workgroup (segment, row).  Every workgroup of a row
// derives the same first digit d1 (bits 31..21 of the threshold) from the
// row's histogram, counts its segment's positions whose digit is above d1
// and copies the scores whose digit is d1 (the candidates) to the start of
// the segment's own range of the row's candidate buffer.  The segment's two
// counts go to segcnt: [q] above d1, [kMaxSegRow + q] candidates.
constexpr int kCandThreads = 256;
constexpr int kCandPer = kSegUnit / kCandThreads;

__global__ __launch_bounds__(kCandThreads) void candidates_kernel(const Launch a, const float* __restrict__ scores,
                                                                  const uint32_t* __restrict__ ghist,
                                                                  uint32_t* __restrict__ cand,
                                                                  uint32_t* __restrict__ segcnt) {
  const int row = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  if (s.L < s.C) return;  // bypass: every position is kept
  const int h = s.h0 + (row - s.row0);
  const int W = a.window ? a.W : 0;
  const int P = s.L - W;
  const int segsz = a.seg_size;
  const int j0 = seg * segsz;
  if (j0 >= P) return;
  const int end = min(P, j0 + segsz);
  const long long off = s.vote_off + (long long)h * s.vote_ld;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores) + off;
  uint32_t* crow = cand + off + j0;

  // The first unit's scores are requested before the histogram so that the
  // two latencies overlap.
  uint32_t kk[kCandPer];
#pragma unroll
  for (int u = 0; u < kCandPer; ++u) {
    const int j = j0 + u * kCandThreads + tid;
    kk[u] = j < end ? score_key(key[j]) : 0u;
  }
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh[8];
  __shared__ uint32_t wave_n[kCandThreads / 64];
  __shared__ uint32_t s_digit, s_need;
  const uint32_t* gh = ghist + (long long)row * 2048;
  for (int d = tid; d < 2048; d += kCandThreads) hist[d] = gh[d];
  __syncthreads();
  pick_digit<kCandThreads>(hist, 2048, (uint32_t)(s.C - W), sh, &s_digit, &s_need);
  const uint32_t d1 = s_digit;

  uint32_t above = 0, base = 0;  // base: candidates of the earlier units (block-uniform)
  for (int jb = j0; jb < end; jb += kSegUnit) {
    if (jb != j0) {
#pragma unroll
      for (int u = 0; u < kCandPer; ++u) {
        const int j = jb + u * kCandThreads + tid;
        kk[u] = j < end ? score_key(key[j]) : 0u;
      }
    }
    // Count, scan the per-wave counts, then write at the scanned offsets.
    uint32_t mine = 0;
#pragma unroll
    for (int u = 0; u < kCandPer; ++u) {
      const int j = jb + u * kCandThreads + tid;
      const uint32_t d = kk[u] >> 21;
      above += j < end && d > d1;
      mine += (uint32_t)__popcll(__ballot(j < end && d == d1));
    }
    if (lane == 0) wave_n[wv] = mine;
    __syncthreads();
    uint32_t wbase = base, unit_n = 0;
    for (int v = 0; v < kCandThreads / 64; ++v) {
      wbase += v < wv ? wave_n[v] : 0u;
      unit_n += wave_n[v];
    }
#pragma unroll
    for (int u = 0; u < kCandPer; ++u) {
      const int j = jb + u * kCandThreads + tid;
      const bool hit = j < end && (kk[u] >> 21) == d1;
      const unsigned long long m = __ballot(hit);
      const uint32_t slot =
          wbase + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (hit) crow[slot] = kk[u];
      wbase += (uint32_t)__popcll(m);
    }
    base += unit_n;
    __syncthreads();  // wave_n is rewritten by the next unit
  }
  uint32_t total;
  (void)block_scan<kCandThreads>(above, sh, total);
  if (tid == 0) {
    uint32_t* sc = segcnt + (long long)row * 2 * kMaxSegRow;
    sc[seg] = total;
    sc[kMaxSegRow + seg] = base;
  }
}

// Threshold kernel: one 1024-thread workgroup per (sequence, head) row.  It
// takes the row's candidates (the scores of first digit d1, segment by
// segment from the candidates kernel) into LDS, resolves the remaining 21
// bits there (two radix digits of 11 and 10 bits; with more than kCand
// candidates the digits read the candidate buffer instead), and rewrites the
// segment counts as exclusive prefixes over the segments: picks above tau and
// tau-equal positions before segment q, which is where the emit workgroup of
// segment q starts.
__global__ __launch_bounds__(kTopkThreads) void threshold_kernel(const Launch a, const uint32_t* __restrict__ ghist,
                                                                 const uint32_t* __restrict__ cand,
                                                                 uint32_t* __restrict__ cut,
                                                                 uint32_t* __restrict__ segcnt) {
  const int row = blockIdx.x;
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  if (s.L < s.C) return;
  const int h = s.h0 + (row - s.row0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int kWavesPerBlock = kTopkThreads / 64;
  const int W = a.window ? a.W : 0;
  const int P = s.L - W;
  const int segsz = a.seg_size;
  const int nseg = (P + segsz - 1) / segsz;
  const uint32_t* crow = cand + s.vote_off + (long long)h * s.vote_ld;
  uint32_t* sc = segcnt + (long long)row * 2 * kMaxSegRow;

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t cand_key[kCand];
  __shared__ uint32_t sgt[kMaxSegRow], seq[kMaxSegRow], cbase[kMaxSegRow];
  __shared__ uint32_t sh[32];
  __shared__ uint32_t s_digit, s_need;
  static_assert(kMaxSegRow <= kTopkThreads, "one thread per segment in the scans");

  KVSEL_SELECT_MARK(0);
  const uint32_t* gh = ghist + (long long)row * 2048;
  for (int d = tid; d < 2048; d += kTopkThreads) hist[d] = gh[d];
  const uint32_t nq = tid < nseg ? sc[kMaxSegRow + tid] : 0u;
  if (tid < nseg) sgt[tid] = sc[tid];
  __syncthreads();
  pick_digit<kTopkThreads>(hist, 2048, (uint32_t)(s.C - W), sh, &s_digit, &s_need);
  const uint32_t d1 = s_digit;
  uint32_t need = s_need;
  uint32_t ncand;
  const uint32_t cincl = block_scan<kTopkThreads>(nq, sh, ncand);
  if (tid < nseg) cbase[tid] = cincl - nq;
  __syncthreads();
  const bool in_lds = ncand <= (uint32_t)kCand;

  // Segment q's candidates are crow[q * segsz + i], i < n_q; in LDS they sit
  // at cand_key[cbase[q] + i].  One wave per segment.
  KVSEL_SELECT_MARK(1);
  if (in_lds) {
    for (int q = wv; q < nseg; q += kWavesPerBlock) {
      const uint32_t n = (q + 1 < nseg ? cbase[q + 1] : ncand) - cbase[q];
      for (uint32_t i = lane; i < n; i += 64) cand_key[cbase[q] + i] = crow[(long long)q * segsz + i];
    }
    __syncthreads();
  }
  KVSEL_SELECT_MARK(2);
  uint32_t prefix = d1;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const int bits = pass == 0 ? 11 : 10;
    const int hi = shift + bits;
    const uint32_t nb = 1u << bits;
    for (int d = tid; d < 2048; d += kTopkThreads) hist[d] = 0u;
    __syncthreads();
    if (in_lds) {
      for (uint32_t i = tid; i < ncand; i += kTopkThreads) {
        const uint32_t k = cand_key[i];
        if ((k >> hi) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1u)], 1u);
      }
    } else {
      for (int q = wv; q < nseg; q += kWavesPerBlock) {
        const uint32_t n = (q + 1 < nseg ? cbase[q + 1] : ncand) - cbase[q];
        for (uint32_t i = lane; i < n; i += 64) {
          const uint32_t k = crow[(long long)q * segsz + i];
          if ((k >> hi) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1u)], 1u);
        }
      }
    }
    __syncthreads();
    pick_digit<kTopkThreads>(hist, (int)nb, need, sh, &s_digit, &s_need);
    prefix = (prefix << bits) | s_digit;
    need = s_need;
    __syncthreads();
  }
  const uint32_t tau = prefix;
  KVSEL_SELECT_MARK(3);

  // Candidates above tau and on tau, per segment (one wave per segment).
  for (int q = wv; q < nseg; q += kWavesPerBlock) {
    const uint32_t n = (q + 1 < nseg ? cbase[q + 1] : ncand) - cbase[q];
    uint32_t gt = 0, eq = 0;
    for (uint32_t i0 = 0; i0 < n; i0 += 64) {
      const uint32_t i = i0 + lane;
      const uint32_t k = i < n ? (in_lds ? cand_key[cbase[q] + i] : crow[(long long)q * segsz + i]) : 0u;
      gt += (uint32_t)__popcll(__ballot(i < n && k > tau));
      eq += (uint32_t)__popcll(__ballot(i < n && k == tau));
    }
    if (lane == 0) {
      sgt[q] += gt;
      seq[q] = eq;
    }
  }
  __syncthreads();
  // Exclusive prefixes over the segments, one scan per count.
  const uint32_t g = tid < nseg ? sgt[tid] : 0u, e = tid < nseg ? seq[tid] : 0u;
  uint32_t tg, te;
  const uint32_t gi = block_scan<kTopkThreads>(g, sh, tg);
  const uint32_t ei = block_scan<kTopkThreads>(e, sh, te);
  if (tid < nseg) {
    sc[tid] = gi - g;
    sc[kMaxSegRow + tid] = ei - e;
  }
  if (tid == 0) {
    cut[2 * row] = tau;
    cut[2 * row + 1] = need;
  }
  KVSEL_SELECT_MARK(4);
}

// Emit kernel: workgroup (segment, row).  Output slots [dst0, dst0 + n) get
// the positions src[0..n) and, with RU > 0, their K and V rows (RU 16-byte
// pieces per row, consecutive threads on consecutive pieces).
constexpr int kEmitThreads = 256;
constexpr int kEmitPer = kSegUnit / kEmitThreads;

template <int RU>
__device__ __forceinline__ void emit_rows(int n, int dst0, const int32_t* src, int32_t* out, long long in_row0,
                                          long long out_row0, const uint4* __restrict__ K,
                                          const uint4* __restrict__ V, uint4* __restrict__ Ko,
                                          uint4* __restrict__ Vo) {
  for (int i = threadIdx.x; i < n; i += kEmitThreads) out[dst0 + i] = src[i];
  if (RU > 0) {
    constexpr int kFly = 4;  // pieces of K and of V in flight per thread
    const int total = n * RU;
    for (int e0 = 0; e0 < total; e0 += kFly * kEmitThreads) {
      // Every slot is loaded (past the end: the last piece again), so the
      // pieces stay in registers; only the stores are guarded.
      uint4 kv[kFly], vv[kFly];
#pragma unroll
      for (int f = 0; f < kFly; ++f) {
        const int e = min(e0 + f * kEmitThreads + (int)threadIdx.x, total - 1);
        const long long from = (in_row0 + src[e / RU]) * RU + e % RU;
        kv[f] = K[from];
        vv[f] = V[from];
      }
#pragma unroll
      for (int f = 0; f < kFly; ++f) {
        const int e = e0 + f * kEmitThreads + (int)threadIdx.x;
        if (e < total) {
          const long long to = (out_row0 + dst0 + e / RU) * RU + e % RU;
          store_stream(Ko + to, kv[f]);
          store_stream(Vo + to, vv[f]);
        }
      }
    }
  }
}

template <int RU>
__global__ __launch_bounds__(kEmitThreads) void emit_kernel(const Launch a, const float* __restrict__ scores,
                                                            const uint32_t* __restrict__ cut,
                                                            const uint32_t* __restrict__ segcnt,
                                                            int32_t* __restrict__ indices,
                                                            const uint4* __restrict__ K, const uint4* __restrict__ V,
                                                            uint4* __restrict__ Ko, uint4* __restrict__ Vo) {
  const int row = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  const int h = s.h0 + (row - s.row0);
  int32_t* out = indices + s.idx_off + (long long)h * s.idx_ld;
  const long long in_row0 = RU > 0 ? s.kv_off / a.D + (long long)kv_head(a, h) * s.L : 0;
  const long long out_row0 = RU > 0 ? s.out_off + (long long)h * s.out_ld : 0;
  const int segsz = a.seg_size;
  __shared__ int32_t src[kSegUnit];
  __shared__ uint32_t stage[kSegUnit + kSegUnit / kEmitPer];
  __shared__ uint32_t sh[8];

  if (s.L < s.C) {  // bypass: position j goes to slot j
    const int end = min(s.L, (seg + 1) * segsz);
    for (int j0 = seg * segsz; j0 < end; j0 += kSegUnit) {
      const int n = min(kSegUnit, end - j0);
      for (int i = tid; i < n; i += kEmitThreads) src[i] = j0 + i;
      __syncthreads();
      emit_rows<RU>(n, j0, src, out, in_row0, out_row0, K, V, Ko, Vo);
      __syncthreads();
    }
    return;
  }
  const int W = a.window ? a.W : 0, P = s.L - W;
  const int count = s.C - W;
  const int nseg = (P + segsz - 1) / segsz;
  if (seg > nseg) return;
  if (seg == nseg) {  // the window positions follow the picks
    if (W == 0) return;
    for (int w = tid; w < W; w += kEmitThreads) src[w] = P + w;
    __syncthreads();
    emit_rows<RU>(W, count, src, out, in_row0, out_row0, K, V, Ko, Vo);
    return;
  }

  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + s.vote_off + (long long)h * s.vote_ld);
  const int end = min(P, (seg + 1) * segsz);
  // The first pass's scores are loaded before the segment counts so that the
  // two latencies overlap.
  uint32_t first[kEmitPer];
#pragma unroll
  for (int u = 0; u < kEmitPer; ++u) {
    const int j = seg * segsz + u * kEmitThreads + tid;
    first[u] = j < end ? score_key(key[j]) : 0u;
  }
  // Picks above tau and tau-equal positions in the segments before this one
  // (exclusive prefixes written by the threshold kernel).
  const uint32_t* sc = segcnt + (long long)row * 2 * kMaxSegRow;
  const uint32_t tau = cut[2 * row], need_eq = cut[2 * row + 1];
  uint32_t gt_run = sc[seg], eq_run = sc[kMaxSegRow + seg];

  for (int j0 = seg * segsz; j0 < end; j0 += kSegUnit) {
    // Coalesced loads staged through LDS; thread t then scans positions
    // j0 + t * kEmitPer + u in order (rows of kEmitPer + 1 words: no conflicts).
#pragma unroll
    for (int u = 0; u < kEmitPer; ++u) {
      const int i = u * kEmitThreads + tid;
      const int j = j0 + i;
      const uint32_t v = j0 == seg * segsz ? first[u] : (j < end ? score_key(key[j]) : 0u);
      stage[(i / kEmitPer) * (kEmitPer + 1) + i % kEmitPer] = v;
    }
    __syncthreads();
    uint32_t kk[kEmitPer];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < kEmitPer; ++u) {
      kk[u] = stage[tid * (kEmitPer + 1) + u];
      const bool in = j0 + tid * kEmitPer + u < end;
      ngt += in && kk[u] > tau;
      neq += in && kk[u] == tau;
    }
    const uint32_t packed = (ngt << 16) | neq;
    uint32_t total;
    const uint32_t ex = block_scan<kEmitThreads>(packed, sh, total) - packed;
    // Slot of a pick = picks above tau before it + min(tau-equal before it,
    // need_eq); those of this pass are consecutive from dst0.
    const uint32_t dst0 = gt_run + min(eq_run, need_eq);
    uint32_t gb = gt_run + (ex >> 16), eb = eq_run + (ex & 0xFFFFu);
#pragma unroll
    for (int u = 0; u < kEmitPer; ++u) {
      const int j = j0 + tid * kEmitPer + u;
      if (j < end) {
        const bool gt = kk[u] > tau, eq = kk[u] == tau;
        if (gt || (eq && eb < need_eq)) {
          const uint32_t dst = gb + min(eb, need_eq);
          if (dst < (uint32_t)count) src[dst - dst0] = j;
        }
        gb += gt;
        eb += eq;
      }
    }
    gt_run += total >> 16;
    eq_run += total & 0xFFFFu;
    const uint32_t dst1 = min(gt_run + min(eq_run, need_eq), (uint32_t)count);
    __syncthreads();
    emit_rows<RU>((int)(dst1 - min(dst0, dst1)), (int)dst0, src, out, in_row0, out_row0, K, V, Ko, Vo);
    __syncthreads();
  }
}

// Avg pooling sums the k neighbours (zero padding included) in ascending
// order, so equal neighbour multisets give bit-equal pooled scores.  `c`
// points at the centre of a zero-padded run of at least r values per side.
template <int KW>
__device__ __forceinline__ float avg_sorted(const float* c) {
  constexpr int r = KW / 2;
  float x[KW];
#pragma unroll
  for (int o = 0; o < KW; ++o) x[o] = c[o - r];
#pragma unroll
  for (int i = 1; i < KW; ++i)
#pragma unroll
    for (int k = i; k > 0; --k) {
      const float lo = fminf(x[k - 1], x[k]), hi = fmaxf(x[k - 1], x[k]);
      x[k - 1] = lo;
      x[k] = hi;
    }
  float sum = 0.f;
#pragma unroll
  for (int o = 0; o < KW; ++o) sum += x[o];
  return sum / (float)KW;
}

__device__ float avg_sorted_any(const float* c, int kw) {
  // Same ascending order without a local array: each step adds every copy of
  // the next larger value among the kw neighbours.  At most kw steps; a NaN
  // among the neighbours is never counted and makes the result NaN.
  const int r = kw / 2;
  float sum = 0.f, cur = -INFINITY;
  int added = 0;
  for (int step = 0; step < kw && added < kw; ++step) {
    float v = INFINITY;
    for (int o = -r; o <= r; ++o)
      if (c[o] > cur) v = fminf(v, c[o]);
    int copies = 0;
    for (int o = -r; o <= r; ++o) copies += c[o] == v;
    if (copies == 0) break;
    for (int m = 0; m < copies; ++m) sum += v;
    added += copies;
    cur = v;
  }
  return added == kw ? sum / (float)kw : __builtin_nanf("");
}

// Pooling of the prefix votes fused with the first radix digit of the
// selection: each workgroup pools kPoolBlock * kPoolSpan positions of one row and
// adds its LDS histogram of bits 31..21 of the pooled scores to the row's
// histogram.  With pooled == nullptr the input is taken as already pooled
// (histogram only); with ghist == nullptr no histogram is built.
__global__ __launch_bounds__(kPoolBlock) void pool_hist_kernel(const Launch a, const float* __restrict__ votes,
                                                               float* __restrict__ pooled,
                                                               uint32_t* __restrict__ ghist) {
  const int row = blockIdx.x;
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  if (s.L < s.C) return;
  const int h = s.h0 + (row - s.row0);
  const int P = s.L - (a.window ? a.W : 0);
  const int base = blockIdx.y * kPoolBlock * kPoolSpan;
  if (base >= P) return;
  __shared__ uint32_t hist[2048];
  if (ghist != nullptr) {
    for (int d = threadIdx.x; d < 2048; d += kPoolBlock) hist[d] = 0u;
    __syncthreads();
  }
  const float* v = votes + s.vote_off + (long long)h * s.vote_ld;
  float* o = pooled ? pooled + s.vote_off + (long long)h * s.vote_ld : nullptr;
  const int kw = a.kernel, r = kw / 2;
  // The block's positions plus a halo of r on each side, staged through LDS
  // with coalesced loads; out-of-range neighbours are the zero padding (avg)
  // or excluded (max: -inf never wins, the centre is always in range).
  constexpr int kSpan = kPoolBlock * kPoolSpan;
  __shared__ float tile[kSpan + 2 * kMaxPoolRadius];
  __shared__ float res_out[kSpan];  // pooled scores, written out coalesced
  const float pad = a.pooling == 1 ? -INFINITY : 0.f;
  {
    // Every load is issued before the first LDS write (one latency).
    float tv[kPoolSpan];
#pragma unroll
    for (int u = 0; u < kPoolSpan; ++u) {
      const int p = base - r + u * kPoolBlock + (int)threadIdx.x;
      tv[u] = (p >= 0 && p < P) ? v[p] : pad;
    }
    const int ph = base - r + kSpan + (int)threadIdx.x;  // right halo, 2r <= 62 < kPoolBlock
    const float th = ((int)threadIdx.x < 2 * r && ph >= 0 && ph < P) ? v[ph] : pad;
#pragma unroll
    for (int u = 0; u < kPoolSpan; ++u) tile[u * kPoolBlock + threadIdx.x] = tv[u];
    if ((int)threadIdx.x < 2 * r) tile[kSpan + threadIdx.x] = th;
  }
  __syncthreads();
  // Each thread pools kPoolSpan consecutive positions; equal first digits of
  // neighbouring positions are counted once per run, which keeps the LDS
  // atomics off the few hot bins of smooth score profiles.
  const int i0 = threadIdx.x * kPoolSpan;
  uint32_t run_bin = 0xFFFFFFFFu, run_len = 0;
  for (int u = 0; u < kPoolSpan; ++u) {
    const int j = base + i0 + u;
    if (j >= P) break;
    const float* c = tile + i0 + u + r;  // centre
    float res;
    if (o == nullptr || kw == 1) {
      res = c[0];
    } else if (a.pooling == 1) {
      res = c[0];
      for (int q = -r; q <= r; ++q) res = fmaxf(res, c[q]);
    } else {
      switch (kw) {
        case 3: res = avg_sorted<3>(c); break;
        case 5: res = avg_sorted<5>(c); break;
        case 7: res = avg_sorted<7>(c); break;
        case 9: res = avg_sorted<9>(c); break;
        case 11: res = avg_sorted<11>(c); break;
        default: res = avg_sorted_any(c, kw); break;
      }
    }
    res_out[i0 + u] = res;
    const uint32_t bin = score_key(__float_as_uint(res)) >> 21;
    if (bin != run_bin) {
      if (run_len && ghist != nullptr) atomicAdd(&hist[run_bin], run_len);
      run_bin = bin;
      run_len = 0;
    }
    ++run_len;
  }
  if (run_len && ghist != nullptr) atomicAdd(&hist[run_bin], run_len);
  __syncthreads();
  if (o)
    for (int i = threadIdx.x; i < kSpan && base + i < P; i += kPoolBlock) o[base + i] = res_out[i];
  if (ghist != nullptr) {
    uint32_t* gh = ghist + (long long)row * 2048;
    for (int d = threadIdx.x; d < 2048; d += kPoolBlock)
      if (hist[d]) atomicAdd(gh + d, hist[d]);
  }
}

// K/V gather: one 16-byte piece of one row per thread.  RU = pieces per row.
template <int RU>
__global__ __launch_bounds__(256) void gather_kernel(const Launch a, const uint4* __restrict__ K,
                                                     const uint4* __restrict__ V,
                                                     const int32_t* __restrict__ idx, uint4* __restrict__ Ko,
                                                     uint4* __restrict__ Vo) {
  constexpr int RPB = 256 / RU;
  const Seg& s = a.seg[find_seg<kFieldGather>(a, blockIdx.x)];
  const int local = blockIdx.x - s.gitem0;
  const int hl = local / s.gblk, blk = local - hl * s.gblk;
  const int h = s.h0 + hl;
  const int m = blk * RPB + (int)threadIdx.x / RU, part = (int)threadIdx.x % RU;
  if (m >= s.nout) return;
  int src = idx[s.idx_off + (long long)h * s.idx_ld + m];
  KVSEL_DEBUG_CHECK(src >= 0 && src < s.L, a.err);
  src = min(max(src, 0), s.L - 1);  // never read outside the head's rows
  const long long in_row = s.kv_off / a.D + (long long)kv_head(a, h) * s.L + src;
  const long long out_row = s.out_off + (long long)h * s.out_ld + m;
  const uint4 kv = K[in_row * RU + part];
  const uint4 vv = V[in_row * RU + part];
  store_stream(Ko + out_row * RU + part, kv);
  store_stream(Vo + out_row * RU + part, vv);
}

hipError_t launch_pool(const Launch& a, int rows, int max_n, const float* votes, float* pooled, uint32_t* hist,
                       hipStream_t st) {
  const int yb = (max_n + kPoolBlock * kPoolSpan - 1) / (kPoolBlock * kPoolSpan);
  if (rows <= 0 || yb <= 0) return hipSuccess;
  hipLaunchKernelGGL(pool_hist_kernel, dim3(rows, yb), dim3(kPoolBlock), 0, st, a, votes, pooled, hist);
  return hipGetLastError();
}

// ---- threshold and picks of whole rows (rows of at most kSelMaxP positions)
//
// Given a row's pooled scores and the histogram of their first radix digit
// (bits 31..21, built by pool_hist_kernel across many workgroups), one
// 1024-thread workgroup per row finds the boundary digit, compacts that
// digit's scores (the candidates) into LDS, resolves the remaining 21 bits
// over them, and writes the picks in index order (tau-equal positions lowest
// index first) followed by the window positions.  Position u * 1024 + t
// belongs to thread t (column u), so the loads are coalesced; the output
// order comes from per-(column, wave) counts and one scan over them.
constexpr int kSelThreads = 1024;
constexpr int kSelCols = 36;
constexpr int kSelMaxP = kSelThreads * kSelCols;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelCand = 32768;  // candidates held in LDS (more: the digits scan the registers)

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(const Launch a, const float* __restrict__ scores,
                                                                  const uint32_t* __restrict__ ghist,
                                                                  int32_t* __restrict__ indices) {
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  const int h = s.h0 + (row - s.row0);
  int32_t* out = indices + s.idx_off + (long long)h * s.idx_ld;
  if (s.L < s.C) {  // bypass: every position is kept
    for (int m = tid; m < s.L; m += kSelThreads) out[m] = m;
    return;
  }
  const int W = a.window ? a.W : 0;
  const int P = s.L - W, count = s.C - W;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t cw[kSelCols * kSelWaves];  // per (column, wave) counts, then their exclusive prefixes
  __shared__ uint32_t cl[kSelCand];
  __shared__ uint32_t sh[32];
  __shared__ uint32_t s_digit, s_need;

  // Every load is issued before the first use.
  const uint32_t* kr = reinterpret_cast<const uint32_t*>(scores + s.vote_off + (long long)h * s.vote_ld);
  uint32_t key[kSelCols];
#pragma unroll
  for (int u = 0; u < kSelCols; ++u) {
    const int j = u * kSelThreads + tid;
    key[u] = j < P ? score_key(kr[j]) : 0u;
  }
  const uint32_t* gh = ghist + (long long)row * 2048;
  for (int d = tid; d < 2048; d += kSelThreads) hist[d] = gh[d];
  __syncthreads();
  pick_digit<kSelThreads>(hist, 2048, (uint32_t)count, sh, &s_digit, &s_need);
  const uint32_t d1 = s_digit;
  uint32_t need = s_need;

  // Candidates of the boundary digit, compacted into LDS in any order.
  uint64_t cm = 0;
#pragma unroll
  for (int u = 0; u < kSelCols; ++u)
    if (u * kSelThreads + tid < P && (key[u] >> 21) == d1) cm |= 1ull << u;
  const uint32_t nmine = (uint32_t)__popcll(cm);
  uint32_t ncand;
  uint32_t coff = block_scan<kSelThreads>(nmine, sh, ncand) - nmine;
  const bool in_lds = ncand <= (uint32_t)kSelCand;
  if (in_lds) {
#pragma unroll
    for (int u = 0; u < kSelCols; ++u)
      if ((cm >> u) & 1ull) cl[coff++] = key[u];
  }
  __syncthreads();
  // The other two digits (11 and 10 bits) over the candidates.
  uint32_t prefix = d1;
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const int bits = pass == 1 ? 11 : 10;
    const int nb = 1 << bits;
    for (int d = tid; d < nb; d += kSelThreads) hist[d] = 0u;
    __syncthreads();
    if (in_lds) {
      for (uint32_t i = tid; i < ncand; i += kSelThreads) {
        const uint32_t k = cl[i];
        if ((k >> (shift + bits)) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kSelCols; ++u) {
        const uint32_t k = key[u];
        if (((cm >> u) & 1ull) && (k >> (shift + bits)) == prefix)
          atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    pick_digit<kSelThreads>(hist, nb, need, sh, &s_digit, &s_need);
    prefix = (prefix << bits) | s_digit;
    need = s_need;
  }
  const uint32_t tau = prefix, need_eq = need;

  // Rank of each tau-equal position among them in index order: counts per
  // (column, wave), one scan, then the lanes below in the wave.
#pragma unroll
  for (int u = 0; u < kSelCols; ++u) {
    const uint64_t m = __ballot(u * kSelThreads + tid < P && key[u] == tau);
    if (lane == 0) cw[u * kSelWaves + wv] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  uint32_t tot;
  {
    const uint32_t c = tid < kSelCols * kSelWaves ? cw[tid] : 0u;
    const uint32_t ex = block_scan<kSelThreads>(c, sh, tot) - c;
    if (tid < kSelCols * kSelWaves) cw[tid] = ex;
  }
  __syncthreads();
  uint64_t pm = 0;  // this thread's picks, bit u for column u
#pragma unroll
  for (int u = 0; u < kSelCols; ++u) {
    const bool valid = u * kSelThreads + tid < P;
    const bool eq = valid && key[u] == tau;
    const uint64_t m = __ballot(eq);
    const uint32_t rank = cw[u * kSelWaves + wv] + lanes_below(m);
    if ((valid && key[u] > tau) || (eq && rank < need_eq)) pm |= 1ull << u;
  }
  __syncthreads();  // the eq prefixes are read
  // Output slot of each pick: counts per (column, wave), one scan.
#pragma unroll
  for (int u = 0; u < kSelCols; ++u) {
    const uint64_t m = __ballot((pm >> u) & 1ull);
    if (lane == 0) cw[u * kSelWaves + wv] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  {
    const uint32_t c = tid < kSelCols * kSelWaves ? cw[tid] : 0u;
    const uint32_t ex = block_scan<kSelThreads>(c, sh, tot) - c;
    if (tid < kSelCols * kSelWaves) cw[tid] = ex;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kSelCols; ++u) {
    const bool pick = (pm >> u) & 1ull;
    const uint64_t m = __ballot(pick);
    if (pick) {
      const uint32_t slot = cw[u * kSelWaves + wv] + lanes_below(m);
      KVSEL_DEBUG_CHECK(slot < (uint32_t)count, a.err);
      if (slot < (uint32_t)count) out[slot] = u * kSelThreads + tid;
    }
  }
  for (int i = tid; i < W; i += kSelThreads) out[count + i] = P + i;
}

int select_rows_max() { return kSelMaxP; }

hipError_t launch_select_hist(const Launch& a, int rows, const float* scores, const uint32_t* hist,
                              int32_t* indices, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(select_hist_kernel, dim3(rows), dim3(kSelThreads), 0, st, a, scores, hist, indices);
  return hipGetLastError();
}

// Pooling of width KW over the window w (registers, centre w[KW / 2]), as in
// pool_hist_kernel.
template <int KW, bool MAX>
__device__ __forceinline__ float pool_window(const float (&w)[KW]) {
  constexpr int r = KW / 2;
  if (KW == 1) return w[0];
  if (MAX) {
    float res = w[r];
#pragma unroll
    for (int q = 0; q < KW; ++q) res = fmaxf(res, w[q]);
    return res;
  }
  return avg_sorted<KW>(w + r);
}

// ---- cooperative selection: segments of a row in parallel
//
// A row's P prefix positions are cut into segments of kCoopSeg positions,
// one 512-thread workgroup each (thread t owns kCoopPer consecutive
// positions of its segment), which pools its votes into keys kept in
// registers.  The threshold tau of the (C-W)-th largest key is found digit
// by digit (11, 11 and 10 bits): every segment adds its histogram of the
// digit (over its keys that match the digits found so far) into the row's
// histogram with device-scope atomics, and every segment reads the row's
// histogram until its bins add up to the number of keys taking part (P,
// then the count of the chosen bin): bins only grow, so a matching sum
// means every bin is final.  Each segment then publishes its counts above
// and on tau (one 64-bit word, zero until written), and from the earlier
// segments' counts knows where its picks go: it writes them in index order
// (tau-equal ones lowest index first) and copies their K and V rows, and a
// share of the window's rows.  The grid must be resident at once; the
// residency handshake decides this, and otherwise the first workgroup of
// each row runs every segment of its row in turn, with the same arithmetic
// and results.
//
// Candidate round.  When the first digit's boundary bin holds at most
// kCandCap keys (the usual case), the last two digits and the count
// exchange are replaced by one exchange: each segment publishes its keys of
// that bin with their positions (at offsets the first digit's atomic adds
// returned, so the row's candidates fill a dense range) and its count of
// keys above the bin; every segment then resolves tau and every segment's
// counts from the same list in LDS.
constexpr int kCoopThreads = 512;
constexpr int kCoopPer = 8;
constexpr int kCoopSeg = kCoopThreads * kCoopPer;
constexpr int kCoopMaxSeg = 64;
constexpr int kCoopStride = kCoopPer + 1;         // LDS words per thread (odd: conflict-free reads)
constexpr int kCoopHalo = kCoopThreads * kCoopStride;  // LDS index of the halo slots
constexpr int kCoopHist = 2048 + 2048 + 1024;     // the row's histograms of the three digits
constexpr int kCandCap = kCoopSeg;                // candidates of the candidate round (64-bit entries)
// The row's words: histograms, the segments' 64-bit counts, the candidates.
constexpr int kCoopRowWords = kCoopHist + 2 * kCoopMaxSeg + 2 * kCandCap;
static_assert(kMaxPoolRadius >= 3, "pooling widths up to 7");

// Wait until word i of p is non-zero for every i < n (one wave polls,
// then the workgroup meets).  Bounded: a timed-out wait sets an error flag.
__device__ void coop_wait(const unsigned long long* p, int n, unsigned* err) {
  if (threadIdx.x < 64) {
    long spins = 0;
    for (;;) {
      bool ok = true;
      for (int i = threadIdx.x; i < n; i += 64)
        ok = ok && __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0ull;
      if (__ballot(!ok) == 0) break;
      if (++spins > (1L << 22)) {
        if (threadIdx.x == 0) raise_error(err, kErrSelectWait);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Read the row histogram gh[nb] into hist until its bins add up to total.
template <int NT>
__device__ void coop_read_hist(const uint32_t* gh, int nb, uint32_t total, uint32_t* hist, uint32_t* sh,
                               unsigned* err) {
  long spins = 0;
  for (;;) {
    uint32_t part = 0;
    for (int d = threadIdx.x; d < nb; d += NT) {
      const uint32_t c = __hip_atomic_load(gh + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hist[d] = c;
      part += c;
    }
    uint32_t sum;
    (void)block_scan<NT>(part, sh, sum);
    if (sum == total) break;
    if (++spins > (1L << 20)) {
      if (threadIdx.x == 0) raise_error(err, kErrSelectWait);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __syncthreads();
}

// Keys of segment g: pooled scores of positions g * kCoopSeg + t * kCoopPer + u
// (0 past P), through LDS with r neighbours on each side.
template <int KW, bool MAX>
__device__ __forceinline__ void coop_keys(const float* __restrict__ v, int P, int g, float* sv,
                                          uint32_t (&key)[kCoopPer]) {
  constexpr int r = KW / 2;
  const int tid = threadIdx.x, j0 = g * kCoopSeg;
  const float pad = MAX ? -INFINITY : 0.f;
  auto at = [](int i) {  // LDS index of segment position i (-r <= i < kCoopSeg + r)
    return i < 0 ? kCoopHalo + (i + r) : (i >= kCoopSeg ? kCoopHalo + r + (i - kCoopSeg)
                                                         : (i / kCoopPer) * kCoopStride + i % kCoopPer);
  };
  __syncthreads();  // the previous segment's reads are done
  float tv[kCoopPer];
#pragma unroll
  for (int k = 0; k < kCoopPer; ++k) {
    const int p = j0 + k * kCoopThreads + tid;
    tv[k] = p < P ? v[p] : pad;
  }
  float hl = pad, hh = pad;
  if (tid < r) {
    const int pl = j0 - r + tid, ph = j0 + kCoopSeg + tid;
    hl = pl >= 0 && pl < P ? v[pl] : pad;
    hh = ph < P ? v[ph] : pad;
  }
#pragma unroll
  for (int k = 0; k < kCoopPer; ++k) sv[at(k * kCoopThreads + tid)] = tv[k];
  if (tid < r) {
    sv[at(tid - r)] = hl;
    sv[at(kCoopSeg + tid)] = hh;
  }
  __syncthreads();
  float w[KW];
  const int i0 = tid * kCoopPer;
#pragma unroll
  for (int q = 0; q < KW - 1; ++q) w[q + 1] = sv[at(i0 - r + q)];
#pragma unroll
  for (int u = 0; u < kCoopPer; ++u) {
#pragma unroll
    for (int q = 0; q < KW - 1; ++q) w[q] = w[q + 1];
    w[KW - 1] = sv[at(i0 + u + r)];
    key[u] = j0 + i0 + u < P ? score_key(__float_as_uint(pool_window<KW, MAX>(w))) : 0u;
  }
}

// This segment's histogram of a digit (bits shift .. shift + bits - 1) over
// its keys whose higher bits equal prefix (all keys for the first digit),
// into hist (LDS).
__device__ __forceinline__ void coop_local_hist(const uint32_t (&key)[kCoopPer], int valid, int shift, int bits,
                                                uint32_t prefix, bool first, uint32_t* hist) {
  const int tid = threadIdx.x, nb = 1 << bits;
  for (int d = tid; d < nb; d += kCoopThreads) hist[d] = 0u;
  __syncthreads();
  uint32_t run_bin = 0xFFFFFFFFu, run_len = 0;  // equal digits of consecutive positions: one atomic per run
#pragma unroll
  for (int u = 0; u < kCoopPer; ++u) {
    const uint32_t k = key[u];
    if (u < valid && (first || (k >> (shift + bits)) == prefix)) {
      const uint32_t b = (k >> shift) & (uint32_t)(nb - 1);
      if (b != run_bin) {
        if (run_len) atomicAdd(&hist[run_bin], run_len);
        run_bin = b;
        run_len = 0;
      }
      ++run_len;
    }
  }
  if (run_len) atomicAdd(&hist[run_bin], run_len);
  __syncthreads();
}

// Add the LDS histogram hist[1 << bits] into gh with device-scope atomics.
// With ret != nullptr the bins' values before this segment's adds are kept
// in ret (LDS).
__device__ __forceinline__ void coop_push_hist(int bits, const uint32_t* hist, uint32_t* gh, uint32_t* ret) {
  const int tid = threadIdx.x, nb = 1 << bits;
  if (ret != nullptr) {
    for (int d = tid; d < nb; d += kCoopThreads)
      if (hist[d]) ret[d] = __hip_atomic_fetch_add(gh + d, hist[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  for (int d = tid; d < nb; d += kCoopThreads)
    if (hist[d]) __hip_atomic_fetch_add(gh + d, hist[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Candidate round, reading side: wait until the nseg count words and the
// n candidate entries are all written (non-zero), then take the count words
// (cw) and the candidates' keys (ck) into LDS.  Bounded: a timed-out wait
// sets an error flag.
__device__ void coop_read_candidates(const unsigned long long* cnt, int nseg, const unsigned long long* cbuf, int n,
                                     unsigned long long* cw, uint32_t* ck, uint32_t* sh, unsigned* err) {
  const int tid = threadIdx.x;
  long spins = 0;
  for (;;) {
    uint32_t missing = 0;
    if (tid < nseg) {
      const unsigned long long c = __hip_atomic_load(cnt + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      missing += c == 0ull;
      cw[tid] = c;
    }
    for (int i = tid; i < n; i += kCoopThreads) {
      const unsigned long long e = __hip_atomic_load(cbuf + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      missing += e == 0ull;
      ck[i] = (uint32_t)e;
    }
    uint32_t total;
    (void)block_scan<kCoopThreads>(missing, sh, total);
    if (total == 0) break;
    if (++spins > (1L << 20)) {
      if (tid == 0) raise_error(err, kErrSelectWait);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __syncthreads();
}

// Copy output rows m0 .. m0 + n of K and V from source rows first + i
// (sel == nullptr) or sel[i] (LDS), then output rows m1 .. m1 + n1 from
// source rows first1 + i, in one pass (one round of loads where both fit):
// RU 16-byte pieces per row, consecutive threads on consecutive pieces, kFly
// pieces of each in flight per thread.  Source rows are clamped into the
// head's L rows: never a read outside them.
template <int RU, int NT = kCoopThreads, int kFly = 4>
__device__ __forceinline__ void coop_copy_rows(int m0, int n, int first, const int32_t* sel, int m1, int n1,
                                               int first1, int L, long long in_row0, long long out_row0,
                                               const uint4* __restrict__ K, const uint4* __restrict__ V,
                                               uint4* __restrict__ Ko, uint4* __restrict__ Vo) {
  const int total = (n + n1) * RU, tid = threadIdx.x;
  for (int e0 = 0; e0 < total; e0 += kFly * NT) {
    uint4 kv[kFly], vv[kFly];
#pragma unroll
    for (int f = 0; f < kFly; ++f) {
      const int e = min(e0 + f * NT + tid, total - 1);
      const int i = e / RU;
      const int src = min(max(i < n ? (sel ? sel[i] : first + i) : first1 + (i - n), 0), L - 1);
      const long long from = (in_row0 + src) * RU + e % RU;
      kv[f] = K[from];
      vv[f] = V[from];
    }
#pragma unroll
    for (int f = 0; f < kFly; ++f) {
      const int e = e0 + f * NT + tid;
      if (e < total) {
        const int i = e / RU;
        const long long to = (out_row0 + (i < n ? m0 + i : m1 + (i - n))) * RU + e % RU;
        store_stream(Ko + to, kv[f]);
        store_stream(Vo + to, vv[f]);
      }
    }
  }
}

template <int RU, int KW, bool MAX>
__global__ __launch_bounds__(kCoopThreads) void select_coop_kernel(
    const Launch a, const float* __restrict__ votes, float* __restrict__ pooled, unsigned* __restrict__ coop,
    unsigned* __restrict__ status, int32_t* __restrict__ indices, const uint4* __restrict__ K,
    const uint4* __restrict__ V, uint4* __restrict__ Ko, uint4* __restrict__ Vo) {
  const int seg = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  __shared__ float sv[kCoopHalo + 8];
  __shared__ uint32_t hist[2048];
  __shared__ int32_t picks[kCoopSeg];
  __shared__ uint32_t sh[32];
  __shared__ uint32_t s_digit, s_need;
  __shared__ unsigned s_go;
  __shared__ uint32_t s_cnt[kCoopMaxSeg], s_pre[kCoopMaxSeg];  // per-segment counts and prefixes
  __shared__ uint32_t s_ret[2048];                               // first-digit bins before this segment's adds
  __shared__ uint32_t s_cg[kCoopMaxSeg], s_ce[kCoopMaxSeg];      // candidates above / on tau per segment
  __shared__ unsigned long long s_cw[kCoopMaxSeg];                // the segments' count words
  __shared__ uint32_t s_h7[3 * 128];                               // the candidate round's three 7-bit digits
  static_assert(kCandCap <= kCoopHalo, "candidate keys alias sv");
  static_assert(kCandCap < 65536, "a candidate range packs into 16-bit fields");
  static_assert(kCoopPer == 8, "the window ranks below use 8 positions per thread");

  // Arrival first; the decision is taken once the own segment's keys are
  // in place (they depend on no other workgroup), before anything is
  // published.
  KVSEL_SELROWS_MARK(0);
  unsigned arrived = 0u;
  if (tid == 0) {
    arrived = arrive(status);
    s_digit = 0u;  // in range even if a timed-out wait leaves no bin chosen
    s_need = 0u;
  }
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  const int h = s.h0 + (row - s.row0);
  int32_t* out = indices + s.idx_off + (long long)h * s.idx_ld;
  const long long in_row0 = s.kv_off / a.D + (long long)kv_head(a, h) * s.L;
  const long long out_row0 = s.out_off + (long long)h * s.out_ld;
  // Output rows m0 .. m0 + n from source rows first + i (sel == nullptr)
  // or sel[i].
  auto copy = [&](int m0, int n, int first, const int32_t* sel, int m1 = 0, int n1 = 0, int first1 = 0) {
    coop_copy_rows<RU>(m0, n, first, sel, m1, n1, first1, s.L, in_row0, out_row0, K, V, Ko, Vo);
  };
  if (s.L < s.C) {  // bypass: every position, segment by segment
    if (tid == 0) s_go = decide(status, arrived, a.err, kFlagSelectFallback, a.residency_ticks);
    __syncthreads();
    const bool go = s_go == kFusedGo;
    if (!go && seg != 0) return;
    for (int g = go ? seg : 0; g < (go ? seg + 1 : (s.L + kCoopSeg - 1) / kCoopSeg); ++g) {
      const int m0 = g * kCoopSeg, n = max(0, min(kCoopSeg, s.L - m0));
      for (int i = tid; i < n; i += kCoopThreads) out[m0 + i] = m0 + i;
      copy(m0, n, m0, nullptr);
    }
    return;
  }
  const int W = a.window ? a.W : 0;
  const int P = s.L - W, count = s.C - W;
  const int nseg = (P + kCoopSeg - 1) / kCoopSeg;
  const float* v = votes + s.vote_off + (long long)h * s.vote_ld;
  uint32_t* words = coop + (long long)row * kCoopRowWords;
  uint32_t* gh1 = words;
  uint32_t* gh2 = words + 2048;
  uint32_t* gh3 = words + 4096;
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(words + kCoopHist);
  unsigned long long* cbuf = cnt + kCoopMaxSeg;  // the candidate round's entries (position + 1, key)
  uint32_t key[kCoopPer];
  auto valid_of = [&](int g) { return max(0, min(kCoopPer, P - g * kCoopSeg - tid * kCoopPer)); };
  // The own segment's keys, their first-digit histogram and its adds into
  // the row's histogram depend on no other workgroup: they overlap the
  // decision, whose group step is taken as soon as the keys are in.  After
  // an ABORT nothing reads the row's histogram: the fallback builds its
  // histograms in LDS.
  if (seg < nseg) coop_keys<KW, MAX>(v, P, seg, sv, key);
  KVSEL_SELROWS_MARK(14);
  if (tid == 0) decide_begin(status, arrived);
  if (seg < nseg) {
    coop_local_hist(key, valid_of(seg), 21, 11, 0u, true, hist);
    coop_push_hist(11, hist, gh1, s_ret);
  }
  KVSEL_SELROWS_MARK(15);
  if (tid == 0) s_go = decide_end(status, a.err, kFlagSelectFallback, a.residency_ticks);
  __syncthreads();
  const bool go = s_go == kFusedGo;
  KVSEL_SELROWS_MARK(1);
  if (go ? seg >= nseg : seg != 0) return;  // not all resident: the row's first workgroup does every segment
  const int g0 = go ? seg : 0, g1 = go ? seg + 1 : nseg;  // the segments this workgroup runs

  // The digits of tau: the first across the segments; then either the
  // candidate round or the other two digits and the count exchange.
  uint32_t prefix = 0u, need = (uint32_t)count, total = (uint32_t)P;
  bool cand_round = false;
  uint32_t* ck = reinterpret_cast<uint32_t*>(sv);  // candidate keys (the candidate round)
  for (int digit = 0; digit < 3; ++digit) {
    const int shift = digit == 0 ? 21 : (digit == 1 ? 10 : 0);
    const int bits = digit == 2 ? 10 : 11;
    uint32_t* gh = digit == 0 ? gh1 : (digit == 1 ? gh2 : gh3);
    uint32_t* rh = hist;  // the row's histogram of the digit (LDS)
    if (go) {
      if (digit == 0 && pooled != nullptr) {
        float* o = pooled + s.vote_off + (long long)h * s.vote_ld + seg * kCoopSeg + tid * kCoopPer;
        const int n = valid_of(seg);
#pragma unroll
        for (int u = 0; u < kCoopPer; ++u)
          if (u < n) o[u] = __uint_as_float(key[u]);
      }
      if (digit > 0) {  // the first digit's adds are in
        coop_local_hist(key, valid_of(seg), shift, bits, prefix, false, hist);
        coop_push_hist(bits, hist, gh, nullptr);
      }
      coop_read_hist<kCoopThreads>(gh, 1 << bits, total, hist, sh, a.err);
    } else {
      // One workgroup runs every segment of the row: the row's histogram is
      // summed in LDS (s_ret), segment by segment.
      rh = s_ret;
      for (int d = tid; d < (1 << bits); d += kCoopThreads) rh[d] = 0u;
      for (int g = 0; g < nseg; ++g) {
        coop_keys<KW, MAX>(v, P, g, sv, key);  // begins with a barrier: rh is cleared or summed
        if (digit == 0 && pooled != nullptr) {
          float* o = pooled + s.vote_off + (long long)h * s.vote_ld + g * kCoopSeg + tid * kCoopPer;
          const int n = valid_of(g);
#pragma unroll
          for (int u = 0; u < kCoopPer; ++u)
            if (u < n) o[u] = __uint_as_float(key[u]);
        }
        coop_local_hist(key, valid_of(g), shift, bits, prefix, digit == 0, hist);
        for (int d = tid; d < (1 << bits); d += kCoopThreads) rh[d] += hist[d];
      }
      __syncthreads();
    }
    pick_digit<kCoopThreads>(rh, 1 << bits, need, sh, &s_digit, &s_need);
    total = rh[s_digit];
    prefix = (prefix << bits) | s_digit;
    need = s_need;
    __syncthreads();  // hist is rewritten by the next digit
    KVSEL_SELROWS_MARK(2 + digit);
    if (digit == 0 && go && total <= (uint32_t)kCandCap) {  // the same for every segment of the row
      cand_round = true;
      break;
    }
  }
  if (cand_round) {
    // Publish this segment's keys of the boundary bin (at the offset its
    // first-digit add returned, so its candidates form one range) and a
    // count word: keys above the bin + 1, the range's start and length.
    const uint32_t d1 = prefix;
    const int n = valid_of(seg);
    uint32_t above = 0, mine = 0;
#pragma unroll
    for (int u = 0; u < kCoopPer; ++u) {
      above += u < n && (key[u] >> 21) > d1;
      mine += u < n && (key[u] >> 21) == d1;
    }
    uint32_t tot;  // both counts of a segment are at most kCoopSeg < 2^16: one scan of the pair
    const uint32_t incl = block_scan<kCoopThreads>(above | (mine << 16), sh, tot);
    const uint32_t tot_above = tot & 0xFFFFu, tot_mine = tot >> 16;
    const uint32_t base = s_ret[d1];  // meaningful when this segment has candidates
    uint32_t off = base + (incl >> 16) - mine;
#pragma unroll
    for (int u = 0; u < kCoopPer; ++u)
      if (u < n && (key[u] >> 21) == d1) {
        const unsigned long long j1 = (unsigned long long)(seg * kCoopSeg + tid * kCoopPer + u + 1);
        if (off < (uint32_t)kCandCap)  // always, unless a timed-out wait left the bin count short
          __hip_atomic_store(cbuf + off, (j1 << 32) | key[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ++off;
      }
    if (tid == 0) {
      const unsigned long long range = tot_mine ? ((unsigned long long)(tot_mine << 16) | base) : 0ull;
      __hip_atomic_store(cnt + seg, (unsigned long long)(tot_above + 1u) | (range << 32), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // sv becomes the candidate keys
    KVSEL_SELROWS_MARK(3);
    for (int i = tid; i < 3 * 128; i += kCoopThreads) s_h7[i] = 0u;  // the digits' bins (below)
    coop_read_candidates(cnt, nseg, cbuf, (int)total, s_cw, ck, sh, a.err);
    KVSEL_SELROWS_MARK(4);
    {
      // The other 21 bits of tau in three digits of 7 bits over the
      // candidates: each digit's 128-bin histogram (LDS atomics), then one
      // wave finds the bin holding the need-th largest.  Two barriers a digit.
      uint32_t t = prefix << 21;
      for (int dg = 0; dg < 3; ++dg) {
        const int shift = 14 - 7 * dg;
        const uint32_t hi = ~((1u << (shift + 7)) - 1u);  // tau's bits found so far
        uint32_t* h7 = s_h7 + 128 * dg;
        for (int i = tid; i < (int)total; i += kCoopThreads)
          if ((ck[i] & hi) == t) atomicAdd(&h7[(ck[i] >> shift) & 127u], 1u);
        __syncthreads();
        if (tid < 64) {  // lane l: bins 127 - 2l and 126 - 2l, highest first
          const uint32_t a0 = h7[127 - 2 * lane], a1 = h7[126 - 2 * lane];
          uint32_t incl = a0 + a1;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const uint32_t x = __shfl_up(incl, o);
            if (lane >= o) incl += x;
          }
          const uint32_t excl = incl - a0 - a1;
          if (excl < need && need <= incl) {
            const bool first = excl + a0 >= need;
            s_digit = first ? 127u - 2u * lane : 126u - 2u * lane;
            s_need = first ? need - excl : need - excl - a0;
          }
        }
        __syncthreads();
        t |= s_digit << shift;
        need = s_need;
      }
      prefix = t;
      KVSEL_SELROWS_MARK(11);
    }
    // Every segment's candidates above and on tau: a wave per segment over
    // the segment's range of candidates.
    for (int q = tid >> 6; q < nseg; q += kCoopThreads / 64) {
      const uint32_t range = (uint32_t)(s_cw[q] >> 32);
      const int lo = (int)(range & 0xFFFFu), hi = min(lo + (int)(range >> 16), (int)total);
      uint32_t gt = 0, eq = 0;
      for (int i = lo + lane; i < hi; i += 64) {
        gt += ck[i] > prefix;
        eq += ck[i] == prefix;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        gt += __shfl_xor(gt, o);
        eq += __shfl_xor(eq, o);
      }
      if (lane == 0) {
        s_cg[q] = gt;
        s_ce[q] = eq;
      }
    }
    __syncthreads();
    KVSEL_SELROWS_MARK(12);
  }
  const uint32_t tau = prefix, need_eq = need;
  if (!cand_round) {
    for (int g = g0; g < g1; ++g) {
      if (!go) coop_keys<KW, MAX>(v, P, g, sv, key);
      const int n = valid_of(g);
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int u = 0; u < kCoopPer; ++u) {
        gt += u < n && key[u] > tau;
        eq += u < n && key[u] == tau;
      }
      uint32_t tg, te;
      (void)block_scan<kCoopThreads>(gt, sh, tg);
      (void)block_scan<kCoopThreads>(eq, sh, te);
      if (tid == 0)
        __hip_atomic_store(cnt + g, (unsigned long long)(tg + 1u) | ((unsigned long long)te << 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    KVSEL_SELROWS_MARK(5);
    coop_wait(cnt, nseg, a.err);
    KVSEL_SELROWS_MARK(6);
  }

  // Phase 4: picks in index order at their final slots, and their rows.
  // Per segment: the picks and tau-equal positions of the earlier segments
  // (all counts at once, a lane each, and scanned).  In the candidate round
  // a segment's count word (already read into s_cw) holds its keys above the
  // boundary bin, and the candidates add those above and on tau.
  if (tid < 64) {
    uint32_t gq = 0u, eqq = 0u;
    if (tid < nseg) {
      const unsigned long long c =
          cand_round ? s_cw[tid] : __hip_atomic_load(cnt + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      gq = (uint32_t)c - 1u;
      eqq = (uint32_t)(c >> 32);
      if (cand_round) {  // the word holds the keys above the boundary bin and the candidate range
        gq += s_cg[tid];
        eqq = s_ce[tid];
      }
    }
    uint32_t eq_incl = eqq;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(eq_incl, o);
      if (tid >= o) eq_incl += t;
    }
    const uint32_t eqb = eq_incl - eqq;
    const uint32_t mine_picks = gq + (need_eq > eqb ? min(eqq, need_eq - eqb) : 0u);
    uint32_t p_incl = mine_picks;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(p_incl, o);
      if (tid >= o) p_incl += t;
    }
    s_cnt[tid] = eqb;              // tau-equal positions before segment tid
    s_pre[tid] = p_incl - mine_picks;  // picks before segment tid
  }
  __syncthreads();
  KVSEL_SELROWS_MARK(5);
  for (int g = g0; g < g1; ++g) {
    if (!go) coop_keys<KW, MAX>(v, P, g, sv, key);
    const uint32_t before = s_pre[g], eq_before = s_cnt[g];
    // One scan of both counts (each at most kCoopSeg < 2^16): keys above tau
    // and tau-equal keys before this thread's first position.  Tau-equal
    // positions are picked in index order while the row still needs them,
    // the first `left` of this segment's.
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int u = 0; u < kCoopPer; ++u) {
      const bool valid = g * kCoopSeg + tid * kCoopPer + u < P;
      gt += valid && key[u] > tau;
      eq += valid && key[u] == tau;
    }
    uint32_t tot;
    const uint32_t excl = block_scan<kCoopThreads>(gt | (eq << 16), sh, tot) - (gt | (eq << 16));
    KVSEL_SELROWS_MARK(7);
    const uint32_t gtb = excl & 0xFFFFu, eqb = excl >> 16;
    const uint32_t left = need_eq > eq_before ? need_eq - eq_before : 0u;
    uint32_t pm = 0, seen = eqb;
#pragma unroll
    for (int u = 0; u < kCoopPer; ++u) {
      const bool valid = g * kCoopSeg + tid * kCoopPer + u < P;
      if (valid && key[u] > tau) pm |= 1u << u;
      if (valid && key[u] == tau) {
        if (seen < left) pm |= 1u << u;
        ++seen;
      }
    }
    const uint32_t ntot = (tot & 0xFFFFu) + min(tot >> 16, left);
    uint32_t off = gtb + min(eqb, left);
#pragma unroll
    for (int u = 0; u < kCoopPer; ++u)
      if ((pm >> u) & 1u) {
        const int j = g * kCoopSeg + tid * kCoopPer + u;
        // Always inside the row's picks, unless a timed-out wait (a flagged
        // error) left the counts short.
        KVSEL_DEBUG_CHECK(before + off < (uint32_t)count && j < P, a.err);
        if (before + off < (uint32_t)count) out[before + off] = j;
        picks[off++] = j;
      }
    KVSEL_SELROWS_MARK(8);
    __syncthreads();
    KVSEL_SELROWS_MARK(6);
    // The window follows the picks: each segment writes and copies a share
    // of its rows, in the same pass as its picks' rows.
    const int w0 = (int)((long long)g * W / nseg), w1 = (int)((long long)(g + 1) * W / nseg);
    for (int i = w0 + tid; i < w1; i += kCoopThreads) out[count + i] = P + i;
    if (RU > 0)
      copy((int)before, (int)min(ntot, before < (uint32_t)count ? (uint32_t)count - before : 0u), 0, picks, count + w0,
           w1 - w0, P + w0);
    __syncthreads();  // picks[] is rewritten by the next segment
  }
  KVSEL_SELROWS_MARK(13);
  (void)lane;
}

int debug_flags_read(int reset) {
#ifdef KVSEL_DEBUG
  unsigned v = 0u;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_word), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess) return -1;
  if (reset) {
    const unsigned zero = 0u;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) != hipSuccess)
      return -1;
  }
  return (int)v;
#else
  (void)reset;
  return -1;
#endif
}

int coop_max_segments() { return kCoopMaxSeg; }
int coop_segment() { return kCoopSeg; }
int coop_row_words() { return kCoopRowWords; }

template <int RU>
hipError_t launch_select_coop_ru(const Launch& a, dim3 grid, const float* votes, float* pooled, unsigned* coop,
                                 unsigned* status, int32_t* indices, const uint4* k, const uint4* v, uint4* ko,
                                 uint4* vo, hipStream_t st) {
  const bool mx = a.pooling == 1;
#define KVSEL_COOP(KW, MX)                                                                                      \
  hipLaunchKernelGGL((select_coop_kernel<RU, KW, MX>), grid, dim3(kCoopThreads), 0, st, a, votes, pooled, coop, \
                     status, indices, k, v, ko, vo)
  switch (a.kernel) {
    case 1: KVSEL_COOP(1, false); break;
    case 3: if (mx) KVSEL_COOP(3, true); else KVSEL_COOP(3, false); break;
    case 5: if (mx) KVSEL_COOP(5, true); else KVSEL_COOP(5, false); break;
    case 7: if (mx) KVSEL_COOP(7, true); else KVSEL_COOP(7, false); break;
    default: return hipErrorNotSupported;
  }
#undef KVSEL_COOP
  return hipGetLastError();
}

int coop_grid_capacity(int D, int dtype) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const void* f = D * (dtype == 1 ? 2 : 4) / 16 == 8    ? (const void*)select_coop_kernel<8, 5, true>
                  : D * (dtype == 1 ? 2 : 4) / 16 == 16 ? (const void*)select_coop_kernel<16, 5, true>
                                                        : (const void*)select_coop_kernel<32, 5, true>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kCoopThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return per_cu * cus;
}

hipError_t launch_select_coop(const Launch& a, int rows, int segs, int dtype, const float* votes, float* pooled,
                              unsigned* coop, unsigned* status, int32_t* indices, const void* K, const void* V,
                              void* K_out, void* V_out, hipStream_t st) {
  if (rows <= 0 || segs <= 0) return hipSuccess;
  const dim3 grid(segs, rows);
  const uint4* k = (const uint4*)K;
  const uint4* v = (const uint4*)V;
  uint4* ko = (uint4*)K_out;
  uint4* vo = (uint4*)V_out;
  switch (a.D * (dtype == 1 ? 2 : 4) / 16) {
    case 8: return launch_select_coop_ru<8>(a, grid, votes, pooled, coop, status, indices, k, v, ko, vo, st);
    case 16:
      return launch_select_coop_ru<16>(a, grid, votes, pooled, coop, status, indices, k, v, ko, vo, st);
    case 32:
      return launch_select_coop_ru<32>(a, grid, votes, pooled, coop, status, indices, k, v, ko, vo, st);
    default: return hipErrorNotSupported;
  }
}

// ---- split selection: every workgroup of a row finds the threshold itself
//
// A row is split over S workgroups of NT threads.  Each of them
// stages the row's votes through LDS with coalesced loads, pools them into
// keys held in registers (thread t owns the KPT consecutive positions
// t * KPT ...), and finds the threshold tau of the (C-W)-th largest key and
// how many tau-equal positions are still needed.  Every workgroup of the row
// sees every key, so all of them find the same tau.  A workgroup then writes
// only its share of the output: the picks whose slots (index order, tau-equal
// positions lowest index first) fall in [split * count / S, (split + 1) *
// count / S), and a share of the window's slots, and copies those K and V
// rows.  No workgroup waits for another: there is no residency requirement
// and no exchange through memory, at the price of S reads of the row's votes
// (from the last-level cache after the first).
//
// First digit of tau (bits 31..21 of the key): one key per thread forms a
// sample, whose histogram gives an estimate b of the boundary bin.  Each
// thread then counts its keys above b + 3 and in each of the bins b - 3 ..
// b + 3 (packed counters in registers, no atomics per key); the boundary bin
// follows exactly from these counts whenever it lies in that window, and
// otherwise from a full histogram of the first digit (LDS atomics).  The
// other 21 bits come from three 7-bit digits over the boundary bin's keys,
// compacted into LDS when they fit there.
constexpr int kSplitWin = 7;   // first-digit bins counted exactly, centred on the estimate
constexpr int kSplitMaxS = 64;  // workgroups per row
constexpr int kSplitStage = 16384;  // positions staged in LDS at a time (at most)

// NT threads with KPT keys each; the row is staged in rounds of kStage
// positions, each held by kOwners threads.
template <int NT, int KPT>
struct SplitGeom {
  static constexpr int kStage = NT * KPT < kSplitStage ? NT * KPT : kSplitStage;
  static constexpr int kRounds = NT * KPT / kStage;
  static constexpr int kOwners = kStage / KPT;
  static constexpr int kLoads = kStage / NT;          // coalesced loads per thread per round
  static constexpr int kStride = KPT + 1;             // LDS words per owner (odd: conflict-free)
  static constexpr int kHalo = kOwners * kStride;     // LDS index of the halo slots
  static constexpr int kWords = kHalo + 2 * 3;        // staging words (pooling radius up to 3)
  static_assert(kRounds * kStage == NT * KPT && kOwners * kRounds == NT, "rounds hold whole owners");
};

// Keys of the calling thread's KPT positions: pooled votes of row v
// (P positions; 0 past P), staged through LDS round by round.
template <int NT, int KPT, int KW, bool MAX>
__device__ __forceinline__ void split_keys(const float* __restrict__ v, int P, float* sv, uint32_t (&key)[KPT]) {
  using G = SplitGeom<NT, KPT>;
  constexpr int r = KW / 2;
  constexpr int kLoads = G::kLoads;
  const float pad = MAX ? -INFINITY : 0.f;
  auto at = [](int i) {  // LDS index of round position i (-r <= i < kOwners * KPT + r)
    return i < 0 ? G::kHalo + (i + r)
                 : (i >= G::kOwners * KPT ? G::kHalo + r + (i - G::kOwners * KPT) : (i / KPT) * G::kStride + i % KPT);
  };
#pragma unroll
  for (int rd = 0; rd < G::kRounds; ++rd) {
    const int j0 = rd * G::kOwners * KPT;
    if (rd > 0) __syncthreads();  // the previous round's reads are done
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // each round derives its own addresses (none kept across rounds)
    float tv[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int p = j0 + q * NT + tid;
      tv[q] = p < P ? v[p] : pad;
    }
    float hl = pad, hh = pad;
    if (tid < r) {
      const int pl = j0 - r + tid, ph = j0 + G::kOwners * KPT + tid;
      hl = pl >= 0 && pl < P ? v[pl] : pad;
      hh = ph < P ? v[ph] : pad;
    }
#pragma unroll
    for (int q = 0; q < kLoads; ++q) sv[at(q * NT + tid)] = tv[q];
    if (tid < r) {
      sv[at(tid - r)] = hl;
      sv[at(G::kOwners * KPT + tid)] = hh;
    }
    __syncthreads();
    const int own = tid - rd * G::kOwners;  // this thread's place among the round's owners
    if (own >= 0 && own < G::kOwners) {
      float w[KW];
      const int i0 = own * KPT;
#pragma unroll
      for (int q = 0; q < KW - 1; ++q) w[q + 1] = sv[at(i0 - r + q)];
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
#pragma unroll
        for (int q = 0; q < KW - 1; ++q) w[q] = w[q + 1];
        w[KW - 1] = sv[at(i0 + u + r)];
        key[u] = j0 + i0 + u < P ? score_key(__float_as_uint(pool_window<KW, MAX>(w))) : 0u;
        if ((u & 15) == 15) asm volatile("" ::: "memory");  // LDS reads in groups of 16 keys (register pressure)
      }
    }
  }
  __syncthreads();  // sv is free for the candidates and the pick list
}

// An empty asm per key: values derived from the keys (their bins, the
// comparisons) are not kept across phases, which would double the registers.
template <int KPT>
__device__ __forceinline__ void split_launder(uint32_t (&key)[KPT]) {
#pragma unroll
  for (int u = 0; u < KPT; ++u) asm volatile("" : "+v"(key[u]));
}

template <int NT, int KPT, int RU>
__global__ __launch_bounds__(NT) void select_split_kernel(const Launch a, int rows, int splits,
                                                                     const float* __restrict__ votes,
                                                                     float* __restrict__ pooled,
                                                                     int32_t* __restrict__ indices,
                                                                     const uint4* __restrict__ K,
                                                                     const uint4* __restrict__ V,
                                                                     uint4* __restrict__ Ko, uint4* __restrict__ Vo) {
  using G = SplitGeom<NT, KPT>;
  const int tid = threadIdx.x, lane = tid & 63;
  // Workgroup b serves row b % rows, split b / rows: the splits of a row are
  // rows apart, which keeps them on one XCD when rows is a multiple of 8.
  const int row = (int)blockIdx.x % rows, sp = (int)blockIdx.x / rows;
  __shared__ float sv[G::kWords];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_h7[3 * 128];
  __shared__ uint32_t sh[32];
  __shared__ uint32_t s_win[kSplitWin + 1];
  __shared__ uint32_t s_digit, s_need;
  KVSEL_SELROWS_MARK(0);
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  const int h = s.h0 + (row - s.row0);
  int32_t* out = indices + s.idx_off + (long long)h * s.idx_ld;
  // RU == 0: indices only (no K/V rows; a.D may be 0).
  const long long in_row0 = RU > 0 ? s.kv_off / a.D + (long long)kv_head(a, h) * s.L : 0;
  const long long out_row0 = RU > 0 ? s.out_off + (long long)h * s.out_ld : 0;
  auto copy = [&](int m0, int n, int first, const int32_t* sel, int m1 = 0, int n1 = 0, int first1 = 0) {
    if constexpr (RU > 0)
      coop_copy_rows<RU, NT, 8>(m0, n, first, sel, m1, n1, first1, s.L, in_row0, out_row0, K, V, Ko, Vo);
  };
  if (s.L < s.C) {  // bypass: every position; this split's share of them
    const int m0 = (int)((long long)sp * s.L / splits), m1 = (int)((long long)(sp + 1) * s.L / splits);
    for (int m = m0 + tid; m < m1; m += NT) out[m] = m;
    if (m1 > m0) copy(m0, m1 - m0, m0, nullptr);
    return;
  }
  const int W = a.window ? a.W : 0;
  const int P = s.L - W, count = s.C - W;
  const float* v = votes + s.vote_off + (long long)h * s.vote_ld;
  if (tid < 3 * 128) s_h7[tid] = 0u;
  for (int d = tid; d < 2048; d += NT) hist[d] = 0u;
  if (tid <= kSplitWin) s_win[tid] = 0u;
  if (tid == 0) {
    s_digit = 0u;
    s_need = 0u;
  }

  uint32_t key[KPT];
  {
    const bool mx = a.pooling == 1;
    switch (a.kernel) {
      case 1: split_keys<NT, KPT, 1, false>(v, P, sv, key); break;
      case 3: if (mx) split_keys<NT, KPT, 3, true>(v, P, sv, key); else split_keys<NT, KPT, 3, false>(v, P, sv, key); break;
      case 5: if (mx) split_keys<NT, KPT, 5, true>(v, P, sv, key); else split_keys<NT, KPT, 5, false>(v, P, sv, key); break;
      default: if (mx) split_keys<NT, KPT, 7, true>(v, P, sv, key); else split_keys<NT, KPT, 7, false>(v, P, sv, key); break;
    }
  }
  const int n = max(0, min(KPT, P - tid * KPT));  // this thread's valid positions
  split_launder(key);
  KVSEL_SELROWS_MARK(1);
  if (pooled != nullptr && sp == 0) {
    float* o = pooled + s.vote_off + (long long)h * s.vote_ld + tid * KPT;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (u < n) o[u] = __uint_as_float(key[u]);
  }

  // Sample estimate of the boundary bin: one key per thread (two offsets,
  // alternating, against periodic patterns).
  const uint32_t k = (uint32_t)count;
  const int us = (tid & 1) ? KPT / 4 : (3 * KPT) / 4;
  uint32_t skey = 0u;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (u == us) skey = key[u];
  const bool has_sample = us < n;
  if (has_sample) atomicAdd(&hist[skey >> 21], 1u);
  uint32_t m;
  (void)block_scan<NT>(has_sample ? 1u : 0u, sh, m);  // also orders the adds before the reads
  int lo = 0;
  bool found = false;
  uint32_t b = 0u, need = k, ncand = 0u;
  if (m > 0) {
    const uint32_t rho = (uint32_t)min((unsigned long long)m, ((unsigned long long)k * m + (P - 1)) / (unsigned long long)P);
    pick_digit<NT>(hist, 2048, rho < 1u ? 1u : rho, sh, &s_digit, &s_need);
    lo = (int)s_digit - kSplitWin / 2;
    KVSEL_SELROWS_MARK(2);
    // Exact counts of the window's bins and of the keys above it.
    uint32_t above = 0u;
    unsigned long long c03 = 0ull, c46 = 0ull;  // 16-bit counters of bins lo .. lo + 3 and lo + 4 .. lo + 6
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int d = (int)(key[u] >> 21) - lo;
      const bool valid = u < n;
      above += valid && d >= kSplitWin;
      if (valid && d >= 0 && d < 4) c03 += 1ull << (16 * d);
      if (valid && d >= 4 && d < kSplitWin) c46 += 1ull << (16 * (d - 4));
    }
    // Per wave each field is at most 64 * KPT < 2^16.
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      above += __shfl_xor(above, o);
      c03 += __shfl_xor(c03, o);
      c46 += __shfl_xor(c46, o);
    }
    if (lane == 0) {
      atomicAdd(&s_win[kSplitWin], above);
#pragma unroll
      for (int d = 0; d < 4; ++d) atomicAdd(&s_win[d], (uint32_t)(c03 >> (16 * d)) & 0xFFFFu);
#pragma unroll
      for (int d = 4; d < kSplitWin; ++d) atomicAdd(&s_win[d], (uint32_t)(c46 >> (16 * (d - 4))) & 0xFFFFu);
    }
    __syncthreads();
    split_launder(key);
    KVSEL_SELROWS_MARK(3);
    uint32_t cum = s_win[kSplitWin];
    for (int d = kSplitWin - 1; d >= 0 && !found && cum < k; --d) {
      const uint32_t c = s_win[d];
      if (lo + d >= 0 && cum + c >= k) {
        found = true;
        b = (uint32_t)(lo + d);
        need = k - cum;
        ncand = c;
      }
      cum += c;
    }
  }
  if (!found) {  // the window missed (or no sample): the full first-digit histogram
    KVSEL_SELROWS_MARK(9);
    __syncthreads();
    for (int d = tid; d < 2048; d += NT) hist[d] = 0u;
    __syncthreads();
    uint32_t run_bin = 0xFFFFFFFFu, run_len = 0u;  // equal bins of consecutive positions: one add per run
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (u < n) {
        const uint32_t bin = key[u] >> 21;
        if (bin != run_bin) {
          if (run_len) atomicAdd(&hist[run_bin], run_len);
          run_bin = bin;
          run_len = 0u;
        }
        ++run_len;
      }
    }
    if (run_len) atomicAdd(&hist[run_bin], run_len);
    __syncthreads();
    pick_digit<NT>(hist, 2048, k, sh, &s_digit, &s_need);
    b = s_digit;
    need = s_need;
    ncand = hist[b];
  }
  split_launder(key);

  // The boundary bin's keys into LDS (any order), when they fit.
  uint32_t* cl = reinterpret_cast<uint32_t*>(sv);
  const bool in_lds = ncand <= (uint32_t)G::kWords;
  if (in_lds) {
    uint32_t mine = 0u;
#pragma unroll
    for (int u = 0; u < KPT; ++u) mine += u < n && (key[u] >> 21) == b;
    uint32_t tot;
    uint32_t off = block_scan<NT>(mine, sh, tot) - mine;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (u < n && (key[u] >> 21) == b) cl[off++] = key[u];
    __syncthreads();
  }
  split_launder(key);
  KVSEL_SELROWS_MARK(4);
  // The other 21 bits in three 7-bit digits: each digit's 128-bin histogram
  // (LDS atomics), then one wave finds the bin holding the need-th largest.
  uint32_t t = b << 21;
  for (int dg = 0; dg < 3; ++dg) {
    const int shift = 14 - 7 * dg;
    const uint32_t hi = ~((1u << (shift + 7)) - 1u);  // tau's bits found so far
    uint32_t* h7 = s_h7 + 128 * dg;
    if (in_lds) {
      for (int i = tid; i < (int)ncand; i += NT)
        if ((cl[i] & hi) == t) atomicAdd(&h7[(cl[i] >> shift) & 127u], 1u);
    } else {
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (u < n && (key[u] & hi) == t) atomicAdd(&h7[(key[u] >> shift) & 127u], 1u);
    }
    __syncthreads();
    if (tid < 64) {  // lane l: bins 127 - 2l and 126 - 2l, highest first
      const uint32_t a0 = h7[127 - 2 * lane], a1 = h7[126 - 2 * lane];
      uint32_t incl = a0 + a1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_up(incl, o);
        if (lane >= o) incl += x;
      }
      const uint32_t excl = incl - a0 - a1;
      if (excl < need && need <= incl) {
        const bool first = excl + a0 >= need;
        s_digit = first ? 127u - 2u * lane : 126u - 2u * lane;
        s_need = first ? need - excl : need - excl - a0;
      }
    }
    __syncthreads();
    t |= s_digit << shift;
    need = s_need;
  }
  const uint32_t tau = t, need_eq = need;
  split_launder(key);
  KVSEL_SELROWS_MARK(5);

  // Slots: picks in index order, tau-equal positions lowest index first.
  // Both counts of a row are below 2^16 (P < 65536): one scan of the pair.
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    gt += u < n && key[u] > tau;
    eq += u < n && key[u] == tau;
  }
  uint32_t tot;
  const uint32_t incl = block_scan<NT>(gt | (eq << 16), sh, tot);
  const uint32_t gt_before = (incl & 0xFFFFu) - gt, eq_before = (incl >> 16) - eq;
  KVSEL_SELROWS_MARK(6);
  const int s0 = (int)((long long)sp * count / splits), s1 = (int)((long long)(sp + 1) * count / splits);
  int32_t* list = reinterpret_cast<int32_t*>(sv);  // this split's source positions, by slot
  {
    uint32_t slot = gt_before + min(eq_before, need_eq), eqs = eq_before;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool valid = u < n;
      const bool e = valid && key[u] == tau;
      const bool pick = (valid && key[u] > tau) || (e && eqs < need_eq);
      eqs += e;
      if (pick) {
        KVSEL_DEBUG_CHECK(slot < (uint32_t)count, a.err);
        if ((int)slot >= s0 && (int)slot < s1) {
          out[slot] = tid * KPT + u;
          list[slot - s0] = tid * KPT + u;
        }
        ++slot;
      }
    }
  }
  // This split's share of the window (it follows the picks).
  const int w0 = (int)((long long)sp * W / splits), w1 = (int)((long long)(sp + 1) * W / splits);
  for (int i = w0 + tid; i < w1; i += NT) out[count + i] = P + i;
  __syncthreads();  // the list is complete
  KVSEL_SELROWS_MARK(7);
  copy(s0, max(0, s1 - s0), 0, list, count + w0, w1 - w0, P + w0);  // the picks and the window in one pass
  KVSEL_SELROWS_MARK(8);
}

// Variants of the split selection: (threads, keys per thread), the first
// covering max_p positions is used.  Rows are below 65536 positions (the
// slot scan packs two 16-bit counts).
constexpr int kSplitVariants = 4;
constexpr int kSplitNT[kSplitVariants] = {512, 512, 512, 1024};
constexpr int kSplitKPT[kSplitVariants] = {16, 32, 64, 64};
constexpr int kSplitWords[kSplitVariants] = {SplitGeom<512, 16>::kWords, SplitGeom<512, 32>::kWords,
                                             SplitGeom<512, 64>::kWords, SplitGeom<1024, 64>::kWords};
int split_kpt(int max_p) {
  for (int v = 0; v < kSplitVariants; ++v)
    if (max_p <= kSplitNT[v] * kSplitKPT[v] && max_p < 65536) return v + 1;
  return 0;
}
int split_max_positions() { return 65535; }
int split_max_splits() { return kSplitMaxS; }
int split_list_capacity(int kpt) { return kpt >= 1 && kpt <= kSplitVariants ? kSplitWords[kpt - 1] : 0; }

template <int NT, int KPT>
const void* split_kernel_ptr(int ru) {
  return ru == 0   ? (const void*)select_split_kernel<NT, KPT, 0>
         : ru == 8 ? (const void*)select_split_kernel<NT, KPT, 8>
         : ru == 16 ? (const void*)select_split_kernel<NT, KPT, 16>
                    : (const void*)select_split_kernel<NT, KPT, 32>;
}

// Workgroups of the split selection that fit the device at once (looked up
// once per device and variant).  D == 0: the indices-only variant.
int split_grid_capacity(int kpt, int D, int dtype) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int ru = D * (dtype == 1 ? 2 : 4) / 16;
  if (kpt < 1 || kpt > kSplitVariants) return 0;
  const int ki = kpt - 1, ri = ru == 0 ? 0 : ru == 8 ? 1 : ru == 16 ? 2 : 3;
  static std::mutex mu;
  static int cache_dev[kSplitVariants][4] = {}, cache_cap[kSplitVariants][4] = {};  // device + 1, capacity
  {
    std::lock_guard<std::mutex> lk(mu);
    if (cache_dev[ki][ri] == dev + 1) return cache_cap[ki][ri];
  }
  const void* f = kpt == 1   ? split_kernel_ptr<512, 16>(ru)
                  : kpt == 2 ? split_kernel_ptr<512, 32>(ru)
                  : kpt == 3 ? split_kernel_ptr<512, 64>(ru)
                             : split_kernel_ptr<1024, 64>(ru);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kSplitNT[ki], 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  std::lock_guard<std::mutex> lk(mu);
  cache_dev[ki][ri] = dev + 1;
  cache_cap[ki][ri] = per_cu * cus;
  return per_cu * cus;
}

template <int NT, int KPT>
hipError_t launch_split_kpt(const Launch& a, int rows, int splits, int ru, const float* votes, float* pooled,
                            int32_t* indices, const uint4* k, const uint4* v, uint4* ko, uint4* vo, hipStream_t st) {
  const dim3 grid((unsigned)(rows * splits));
  switch (ru) {
    case 0:
      hipLaunchKernelGGL((select_split_kernel<NT, KPT, 0>), grid, dim3(NT), 0, st, a, rows, splits, votes, pooled,
                         indices, k, v, ko, vo);
      break;
    case 8:
      hipLaunchKernelGGL((select_split_kernel<NT, KPT, 8>), grid, dim3(NT), 0, st, a, rows, splits, votes, pooled,
                         indices, k, v, ko, vo);
      break;
    case 16:
      hipLaunchKernelGGL((select_split_kernel<NT, KPT, 16>), grid, dim3(NT), 0, st, a, rows, splits, votes, pooled,
                         indices, k, v, ko, vo);
      break;
    case 32:
      hipLaunchKernelGGL((select_split_kernel<NT, KPT, 32>), grid, dim3(NT), 0, st, a, rows, splits, votes, pooled,
                         indices, k, v, ko, vo);
      break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_select_split(const Launch& a, int rows, int splits, int kpt, int dtype, const float* votes,
                               float* pooled, int32_t* indices, const void* K, const void* V, void* K_out, void* V_out,
                               hipStream_t st) {
  if (rows <= 0 || splits <= 0) return hipSuccess;
  if (splits > kSplitMaxS || (long long)rows * splits > 0x7FFFFFFFll) return hipErrorInvalidValue;
  if (a.kernel != 1 && a.kernel != 3 && a.kernel != 5 && a.kernel != 7) return hipErrorNotSupported;
  const int ru = K == nullptr ? 0 : a.D * (dtype == 1 ? 2 : 4) / 16;  // K == nullptr: indices only
  const uint4* k = (const uint4*)K;
  const uint4* v = (const uint4*)V;
  uint4* ko = (uint4*)K_out;
  uint4* vo = (uint4*)V_out;
  switch (kpt) {
    case 1: return launch_split_kpt<512, 16>(a, rows, splits, ru, votes, pooled, indices, k, v, ko, vo, st);
    case 2: return launch_split_kpt<512, 32>(a, rows, splits, ru, votes, pooled, indices, k, v, ko, vo, st);
    case 3: return launch_split_kpt<512, 64>(a, rows, splits, ru, votes, pooled, indices, k, v, ko, vo, st);
    case 4: return launch_split_kpt<1024, 64>(a, rows, splits, ru, votes, pooled, indices, k, v, ko, vo, st);
    default: return hipErrorNotSupported;
  }
}

int selection_seg_size(long long max_positions) {
  const long long units = (max_positions + kSegUnit - 1) / kSegUnit;
  const long long per = (units + kMaxSegRow - 1) / kMaxSegRow;
  return (int)(kSegUnit * (per < 1 ? 1 : per));
}

hipError_t launch_candidates(const Launch& a, int rows, int max_n, const float* scores, const uint32_t* hist,
                             uint32_t* cand, uint32_t* segcnt, hipStream_t st) {
  if (rows <= 0 || max_n <= 0) return hipSuccess;
  const dim3 grid((max_n + a.seg_size - 1) / a.seg_size, rows);
  hipLaunchKernelGGL(candidates_kernel, grid, dim3(kCandThreads), 0, st, a, scores, hist, cand, segcnt);
  return hipGetLastError();
}

hipError_t launch_threshold(const Launch& a, int rows, const uint32_t* hist, const uint32_t* cand, uint32_t* cut,
                            uint32_t* segcnt, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(threshold_kernel, dim3(rows), dim3(kTopkThreads), 0, st, a, hist, cand, cut, segcnt);
  return hipGetLastError();
}

hipError_t launch_emit(const Launch& a, int rows, int max_positions, int dtype, const float* scores,
                       const uint32_t* cut, const uint32_t* segcnt, int32_t* indices, const void* K, const void* V,
                       void* K_out, void* V_out, hipStream_t st) {
  if (rows <= 0 || max_positions <= 0) return hipSuccess;
  const dim3 grid((max_positions + a.seg_size - 1) / a.seg_size + 1, rows);
  const uint4* k = (const uint4*)K;
  const uint4* v = (const uint4*)V;
  uint4* ko = (uint4*)K_out;
  uint4* vo = (uint4*)V_out;
  const int ru = K == nullptr ? 0 : a.D * (dtype == 1 ? 2 : 4) / 16;
  if (ru == 0)
    hipLaunchKernelGGL(emit_kernel<0>, grid, dim3(kEmitThreads), 0, st, a, scores, cut, segcnt, indices, k, v, ko, vo);
  else if (ru == 8)
    hipLaunchKernelGGL(emit_kernel<8>, grid, dim3(kEmitThreads), 0, st, a, scores, cut, segcnt, indices, k, v, ko, vo);
  else if (ru == 16)
    hipLaunchKernelGGL(emit_kernel<16>, grid, dim3(kEmitThreads), 0, st, a, scores, cut, segcnt, indices, k, v, ko, vo);
  else
    hipLaunchKernelGGL(emit_kernel<32>, grid, dim3(kEmitThreads), 0, st, a, scores, cut, segcnt, indices, k, v, ko, vo);
  return hipGetLastError();
}

// Refresh selection: final indices of `rows` rows of `keep` entries.  The
// first `head` entries are the protected leading positions 0 .. head-1;
// entries head .. keep-1 were written by the selection relative to position
// `head` (picks ascending, then the protected tail) and are shifted, or, with
// no flexible budget (picked == 0), are the tail positions n - tail .. n-1.
// Token ids (tokens != nullptr) are gathered with the final indices.
__global__ void refresh_finish_kernel(int rows, int n, int keep, int head, int tail, int picked,
                                      int32_t* __restrict__ indices, const int32_t* __restrict__ tokens,
                                      int32_t* __restrict__ tokens_out) {
  const long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (e >= (long long)rows * keep) return;
  const int row = (int)(e / keep), m = (int)(e % keep);
  int idx;
  if (m < head)
    idx = m;
  else if (picked) {
    KVSEL_DEBUG_CHECK(indices[e] >= 0 && indices[e] < n - head, nullptr);
    idx = min(max(indices[e], 0), n - head - 1) + head;
  }
  else
    idx = n - tail + (m - head);
  indices[e] = idx;
  if (tokens != nullptr) tokens_out[e] = tokens[(long long)row * n + idx];
}

hipError_t launch_refresh_finish(int rows, int n, int keep, int head, int tail, bool picked, int32_t* indices,
                                 const int32_t* tokens, int32_t* tokens_out, hipStream_t st) {
  const long long total = (long long)rows * keep;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(refresh_finish_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, rows, n, keep,
                     head, tail, picked ? 1 : 0, indices, tokens, tokens_out);
  return hipGetLastError();
}

hipError_t launch_gather(const Launch& a, int items, int dtype, const void* K, const void* V,
                         const int32_t* indices, void* K_out, void* V_out, hipStream_t st) {
  if (items <= 0) return hipSuccess;
  const int ru = a.D * (dtype == 1 ? 2 : 4) / 16;
  const uint4* k = (const uint4*)K;
  const uint4* v = (const uint4*)V;
  uint4* ko = (uint4*)K_out;
  uint4* vo = (uint4*)V_out;
  if (ru == 8)
    hipLaunchKernelGGL(gather_kernel<8>, dim3(items), dim3(256), 0, st, a, k, v, indices, ko, vo);
  else if (ru == 16)
    hipLaunchKernelGGL(gather_kernel<16>, dim3(items), dim3(256), 0, st, a, k, v, indices, ko, vo);
  else
    hipLaunchKernelGGL(gather_kernel<32>, dim3(items), dim3(256), 0, st, a, k, v, indices, ko, vo);
  return hipGetLastError();
}

int gather_rows_per_block(int D, int dtype) { return 256 / (D * (dtype == 1 ? 2 : 4) / 16); }

}  // namespace kvsel
