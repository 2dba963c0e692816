// C ABI of libkvsel: argument validation, workspace layout and the launch
// sequence of the observation-window selection.  Declarations and the
// contract of every entry point are in include/kvsel.h.
//
// Argument rules follow the worked selection on the web page "SnapKV:
// selecting the KV cache for long prompts with an observation window"
// (section "one full selection computed from Q and K"): positive sizes,
// window not longer than the prompt, budget larger than the window, odd
// pooling width, avg or max pooling.  A prompt shorter than its budget is
// kept whole (same section, and section "prefill still reads the full K/V;
// the compressed cache serves decode").

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>
#include <string>
#include <unordered_map>
#include <vector>

#include "kvsel.h"
#include "kvsel_internal.h"
#include "kvsel_jacap.h"

using namespace kvsel;

// Workspace of the allocation-free entry point (kvsel_select_noalloc): a
// device array of the library, of which every GPU the library runs on holds
// its own copy, allocated with the code object and kept until the process
// ends.  In host code its name is only a stand-in, never an address: the
// device address is taken once per device with hipGetSymbolAddress and that
// address is what every launch receives.
constexpr size_t kScratchBytes = KVSEL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return KVSEL_OK;
}

constexpr int kMaxW = 128;
constexpr int kMaxKernel = 63;
constexpr long long kMaxL = 1LL << 24;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_shape(int heads, int W, int D, int dtype) {
  if (heads < 1) return fail(KVSEL_EINVAL, "heads must be >= 1 (got %d)", heads);
  if (W < 1) return fail(KVSEL_EINVAL, "window W must be >= 1 (got %d)", W);
  if (D < 1) return fail(KVSEL_EINVAL, "head dimension D must be >= 1 (got %d)", D);
  if (dtype != KVSEL_F32 && dtype != KVSEL_BF16) return fail(KVSEL_EINVAL, "unknown dtype %d", dtype);
  return KVSEL_OK;
}

// Limits of these kernels (valid for the method, not covered here).
int check_support(int W, int D) {
  if (D != 64 && D != 128) return fail(KVSEL_EUNSUPPORTED, "head dimension %d not supported (64 or 128)", D);
  if (W > kMaxW) return fail(KVSEL_EUNSUPPORTED, "window %d exceeds the supported maximum %d", W, kMaxW);
  return KVSEL_OK;
}

int check_pool(int kernel, int pooling) {
  if (kernel < 1 || kernel % 2 != 1) return fail(KVSEL_EINVAL, "pooling width must be odd and >= 1 (got %d)", kernel);
  if (pooling != KVSEL_POOL_AVG && pooling != KVSEL_POOL_MAX)
    return fail(KVSEL_EINVAL, "pooling must be KVSEL_POOL_AVG or KVSEL_POOL_MAX (got %d)", pooling);
  if (kernel > kMaxKernel) return fail(KVSEL_EUNSUPPORTED, "pooling width %d exceeds %d", kernel, kMaxKernel);
  return KVSEL_OK;
}

// Per-sequence layout of a (possibly ragged) batch.
struct Plan {
  int B = 0, heads = 0, W = 0, D = 0, dtype = 0;
  int group = 1;              // query heads per K/V head
  std::vector<int> L, C, nch, fc;
  std::vector<long long> cuL, cuC, cuP, part, fpart;  // exclusive prefix sums
  int fS = 0;                 // single-read scoring: positions per workgroup per round
  long long part_slots = 0;   // (sequence, head, chunk) partial-stat slots, either path
  long long vote_elems = 0;   // heads * sum of P_b
  size_t off_pm = 0, off_pz = 0, off_votes = 0, off_pooled = 0, off_cut = 0, off_segcnt = 0, off_ctr = 0,
         off_hist = 0, off_coop = 0, bytes = 0;
  // The selection fused into the single-read scoring kernel.
  size_t off_cw = 0, off_halo = 0, off_flags = 0, off_cslot = 0, off_fslot = 0, off_rowfb = 0, off_cand = 0,
         off_kslot = 0;
};

// The workspace starts with a 256-byte header; word 0 holds the error flags
// of the last selection call (kvsel_status).
constexpr size_t kHeaderBytes = 256;

// K bytes of a launch group above which its tiles are loaded
// non-temporally: beyond about this much the last-level cache (256 MiB)
// keeps little of K for a later read (the two-pass votes pass, the
// selection's copy of the kept rows, the same call repeated), and cached
// lines only evict what is still useful.  Measured: a 268 MB layer is
// faster with non-temporal loads on either scoring path, a 67 MB grouped
// layer and a 134 MB layer are slower.
constexpr double kTwoPassCachedBytes = 192.0 * 1024 * 1024;

// Cooperative-selection launches per launch group at most: rows whose grid
// does not fit the device at once are selected a subset at a time, each
// launch with its own status block.
constexpr int kCoopLaunches = 8;

// Selection workspace per (sequence, head) row: threshold and segment counts.
constexpr size_t kCutBytes = 2 * sizeof(uint32_t);
constexpr size_t kSegCntBytes = 2 * kMaxSegRow * sizeof(uint32_t);

// Host-side path of the last selection call on this thread (kvsel_last_path).
thread_local unsigned g_last_path = 0u;

// Process-wide options.
int g_scoring = KVSEL_SCORING_AUTO;
int g_force_fallback = 0;
int g_validate = 0;
int g_fused_select = 0;
int g_select = KVSEL_SELECT_AUTO;

// Per-call tokens of the fused selection: the arrival and decision words and
// the tagged flag word carry them, so nothing has to be cleared before a
// call.  Bits 2..31 count calls (never 0), bits 32..63 are random per process.
unsigned long long next_token() {
  static std::atomic<unsigned long long> calls{0};
  static const unsigned long long salt = [] {
    std::random_device rd;
    return ((unsigned long long)rd() ^ (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count()) &
           0xFFFFFFFFull;
  }();
  unsigned long long n = (++calls) & 0x3FFFFFFFull;
  if (n == 0) n = 1;
  return (salt << 32) | (n << 2);
}

// What the last selection call on a workspace left in its header: whether
// the call cleared word 0 (then word 0 holds its flags) and its token (the
// tagged word holds its flags when the tags match).
struct LastCall {
  bool cleared = false;  // the header was zeroed before the call
  unsigned long long token = 0;
};
std::mutex g_calls_mu;
std::unordered_map<const void*, LastCall> g_calls;

void record_call(const void* ws, bool cleared, unsigned long long token) {
  std::lock_guard<std::mutex> lk(g_calls_mu);
  g_calls[ws] = LastCall{cleared, token};
}

// The last call's flags from the header words (word 0, the tagged word).
unsigned last_call_flags(const void* ws, unsigned w0, unsigned long long tagged) {
  LastCall c;
  {
    std::lock_guard<std::mutex> lk(g_calls_mu);
    auto it = g_calls.find(ws);
    if (it == g_calls.end()) return w0;  // not a selection call of this process: word 0 as written
    c = it->second;
  }
  unsigned f = c.cleared ? w0 : 0u;
  if (c.token != 0 && (tagged >> 24) == token_tag(c.token)) f |= (unsigned)(tagged & 0xFFFFFFull);
  return f;
}

int make_plan(const int32_t* cu_L, const int32_t* C_host, int B, int heads, int W, int D, int dtype, Plan& p,
              int kv_heads = 0) {
  if (cu_L == nullptr || C_host == nullptr) return fail(KVSEL_EINVAL, "cu_L_host and C_host must not be NULL");
  if (B < 1) return fail(KVSEL_EINVAL, "batch B must be >= 1 (got %d)", B);
  int rc = check_shape(heads, W, D, dtype);
  if (rc) return rc;
  if (kv_heads == 0) kv_heads = heads;
  if (kv_heads < 1 || heads % kv_heads != 0)
    return fail(KVSEL_EINVAL, "query heads %d must be a positive multiple of the K/V heads %d", heads, kv_heads);
  p.group = heads / kv_heads;
  if (p.group > 1 && (W % 32 != 0 || p.group * W > 128))
    return fail(KVSEL_EUNSUPPORTED, "grouped heads need W a multiple of 32 and group * W <= 128 (group %d, W %d)",
                p.group, W);
  if (cu_L[0] != 0) return fail(KVSEL_EINVAL, "cu_L[0] must be 0 (got %d)", cu_L[0]);
  p.B = B;
  p.heads = heads;
  p.W = W;
  p.D = D;
  p.dtype = dtype;
  p.L.resize(B);
  p.C.resize(B);
  p.nch.resize(B);
  p.cuL.assign(B + 1, 0);
  p.cuC.assign(B + 1, 0);
  p.cuP.assign(B + 1, 0);
  p.part.assign(B + 1, 0);
  p.fpart.assign(B + 1, 0);
  p.fc.resize(B);
  p.fS = p.group == 1 ? fused_positions(W, D) : 0;  // grouped heads: two-pass scoring
  for (int b = 0; b < B; ++b) {
    const long long L = (long long)cu_L[b + 1] - cu_L[b];
    const int C = C_host[b];
    if (L < 1) return fail(KVSEL_EINVAL, "sequence %d: prompt length must be >= 1 (got %lld)", b, L);
    if (L > kMaxL) return fail(KVSEL_EUNSUPPORTED, "sequence %d: prompt length %lld exceeds %lld", b, L, kMaxL);
    if (W > L) return fail(KVSEL_EINVAL, "sequence %d: window %d exceeds prompt length %lld", b, W, L);
    if (C <= W) return fail(KVSEL_EINVAL, "sequence %d: budget %d must exceed the window %d", b, C, W);
    p.L[b] = (int)L;
    p.C[b] = C;
    p.nch[b] = L < C ? 0 : (int)((L + kChunk - 1) / kChunk);
    p.cuL[b + 1] = p.cuL[b] + L;
    p.cuC[b + 1] = p.cuC[b] + C;
    p.cuP[b + 1] = p.cuP[b] + (L - W);
    p.part[b + 1] = p.part[b] + (long long)(heads / p.group) * p.nch[b];
    p.fc[b] = (L < C || p.fS == 0) ? 0 : (int)((L + p.fS - 1) / p.fS);
    p.fpart[b + 1] = p.fpart[b] + (long long)heads * fused_slot_stride(p.fc[b]);
  }
  if ((rc = check_support(W, D))) return rc;
  p.part_slots = p.part[B];
  p.vote_elems = (long long)heads * p.cuP[B];
  size_t off = kHeaderBytes;
  p.off_pm = off;  // partial slots per (sequence, K/V head, chunk), group * W rows each
  off = align256(off + (size_t)p.part_slots * p.group * W * sizeof(float));
  p.off_pz = off;
  off = align256(off + (size_t)p.part_slots * p.group * W * sizeof(float));
  p.off_votes = off;
  off = align256(off + (size_t)p.vote_elems * sizeof(float));
  p.off_pooled = off;
  off = align256(off + (size_t)p.vote_elems * sizeof(float));
  p.off_cut = off;  // selection threshold per (sequence, head)
  off = align256(off + (size_t)B * heads * kCutBytes);
  p.off_segcnt = off;  // per-segment counts above / on the threshold
  off = align256(off + (size_t)B * heads * kSegCntBytes);
  p.off_ctr = off;  // single-read scoring: one exchange slot per (sequence, head, chunk)
  off = align256(off + (size_t)p.fpart[B] * fused_exchange_bytes());
  p.off_hist = off;  // first-digit histogram of the pooled scores, per (sequence, head)
  off = align256(off + (size_t)B * heads * 2048 * 4);
  p.off_coop = off;  // cooperative selection: status per launch (kCoopLaunches per launch group), then per-row words
  off = align256(off + (size_t)((B + kMaxSegs - 1) / kMaxSegs) * kCoopLaunches * kFusedStatusWords * sizeof(unsigned) +
                 (size_t)B * heads * coop_row_words() * sizeof(unsigned));
  // Fused selection (single-read shapes only): per exchange slot a count
  // word and the halo words; per launch group the arrival tokens, decision
  // and claim counters; per exchange slot the chunk's histograms; per row two
  // completion counters; the candidates, laid out like the votes; per
  // exchange slot the chunk's pooled scores.
  const bool fused_words = p.fS > 0;
  p.off_cw = off;
  off = align256(off + (fused_words ? (size_t)p.fpart[B] * 8 : 0));
  p.off_halo = off;
  off = align256(off + (fused_words ? (size_t)p.fpart[B] * kHaloWords * 8 : 0));
  p.off_cslot = off;  // per exchange slot the chunk's coarse and fine histograms
  off = align256(off + (fused_words ? (size_t)p.fpart[B] * 64 * 4 : 0));
  p.off_fslot = off;
  off = align256(off + (fused_words ? (size_t)p.fpart[B] * 32 * 4 : 0));
  p.off_flags = off;  // (the count, halo and histogram words above form one range the kernel clears)
  off = align256(off + (fused_words ? (size_t)((B + kMaxSegs - 1) / kMaxSegs) * kFusedFlagWords * 8 : 0));
  p.off_rowfb = off;
  off = align256(off + (fused_words ? (size_t)B * heads * 2 * 8 : 0));
  p.off_cand = off;
  off = align256(off + (fused_words ? (size_t)p.vote_elems * 8 : 0));
  p.off_kslot = off;  // per exchange slot the chunk's pooled scores
  off = align256(off + (fused_words ? (size_t)p.fpart[B] * p.fS * 4 : 0));
  p.bytes = off;
  return KVSEL_OK;
}

// Wall-clock ticks of the residency bound on the current device: the rate
// of the device's constant-rate clock (kHz) is read once per device.
long long residency_ticks() {
  static std::mutex mu;
  static int rate_khz[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int khz;
  {
    std::lock_guard<std::mutex> lk(mu);
    if (rate_khz[dev] == 0) {
      int r = 0;
      if (hipDeviceGetAttribute(&r, hipDeviceAttributeWallClockRate, dev) != hipSuccess || r <= 0)
        r = 100000;  // the CDNA constant clock runs at 100 MHz where the attribute is missing
      rate_khz[dev] = r;
    }
    khz = rate_khz[dev];
  }
  return kResidencyMicros * (long long)khz / 1000;
}

Launch base_launch(const Plan& p, int kernel, int pooling) {
  Launch a{};
  a.residency_ticks = residency_ticks();
  a.heads = p.heads;
  a.W = p.W;
  a.D = p.D;
  a.kernel = kernel;
  a.pooling = pooling;
  a.window = 1;
  a.scale2 = (float)(1.4426950408889634074 / sqrt((double)p.D));
  a.err = nullptr;
  a.group = p.group;
  return a;
}

int device_error(hipError_t e, const char* what) {
  return fail(KVSEL_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Optional event timing of every launch (kvsel_profile_enable).
struct TimedLaunch {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<TimedLaunch> g_prof;

// Set for the duration of an allocation-free call: no events are created.
thread_local bool g_no_events = false;

template <typename F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  if (g_no_events) return launch();
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on;
  }
  if (!on) return launch();
  TimedLaunch t{name, nullptr, nullptr};
  hipError_t e;
  if ((e = hipEventCreate(&t.start)) != hipSuccess) return e;
  if ((e = hipEventCreate(&t.stop)) != hipSuccess) return e;
  if ((e = hipEventRecord(t.start, st)) != hipSuccess) return e;
  if ((e = launch()) != hipSuccess) return e;
  if ((e = hipEventRecord(t.stop, st)) != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back(t);
  return hipSuccess;
}

void drop_profile_events() {
  for (auto& t : g_prof) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_prof.clear();
}

// lse: the window rows' natural-log log-sum-exps [sequence][head][W] handed
// over by the caller, or nullptr (then the scoring kernels find them).
int run_select(const void* Q, const void* K, const void* V, const float* lse, const Plan& p, int kernel,
               int pooling, int32_t* indices, void* K_out, void* V_out, float* row_stats, float* votes_opt,
               float* pooled_opt, void* workspace, hipStream_t st) {
  char* ws = (char*)workspace;
  float* pm = (float*)(ws + p.off_pm);
  float* pz = (float*)(ws + p.off_pz);
  float* votes = votes_opt ? votes_opt : (float*)(ws + p.off_votes);
  float* pooled = pooled_opt ? pooled_opt : (float*)(ws + p.off_pooled);
  unsigned* counters = (unsigned*)(ws + p.off_ctr);
  uint32_t* cut = (uint32_t*)(ws + p.off_cut);
  uint32_t* segcnt = (uint32_t*)(ws + p.off_segcnt);
  // The selection's candidate scores reuse the workspace votes buffer, which
  // nothing reads after pooling (or which is unused when votes_opt is given).
  uint32_t* cand = (uint32_t*)(ws + p.off_votes);

  // Single-read scoring needs every head of a round co-resident: each prompt
  // must fit one round of the grid (ceil(L / S) <= grid).
  bool fused_ok = p.dtype == KVSEL_BF16 && p.fS > 0 && (p.D == 64 || p.D == 128);
  const int grid = fused_ok ? fused_grid(p.W, p.D) : 0;
  fused_ok = fused_ok && grid > 0;
  bool need_scoring = false;
  for (int b = 0; b < p.B; ++b) need_scoring = need_scoring || p.L[b] >= p.C[b];
  for (int b = 0; b < p.B && fused_ok; ++b) fused_ok = p.fc[b] <= grid;
  if (g_scoring == KVSEL_SCORING_SINGLE_READ && need_scoring && !fused_ok)
    return fail(KVSEL_EUNSUPPORTED, "single-read scoring does not cover this shape (bf16, D 64/128, W <= 32, "
                                    "ceil(L / %d) <= %d)", p.fS, grid);
  // AUTO takes the faster path for the shape: the single-read kernel wherever
  // it applies (it reads K once), else two-pass.
  const bool use_fused = fused_ok && g_scoring != KVSEL_SCORING_TWO_PASS;
  uint32_t* hist = (uint32_t*)(ws + p.off_hist);
  // Rows of at most select_rows_max() prefix positions are resolved by one
  // workgroup each (threshold and picks) and copied by the gather kernel;
  // longer rows go through the segment-parallel candidates, threshold and
  // emit kernels.
  bool whole_rows = true;
  for (int b = 0; b < p.B && whole_rows; ++b) whole_rows = p.L[b] < p.C[b] || p.L[b] - p.W <= select_rows_max();
  // The cooperative selection (pooling, threshold, picks and K/V copy in
  // one launch, a workgroup per segment of a row) where its grid fits the
  // device at once.
  const int coop_cap = (kernel == 1 || kernel == 3 || kernel == 5 || kernel == 7) ? coop_grid_capacity(p.D, p.dtype) : 0;
  const int ngroups = (p.B + kMaxSegs - 1) / kMaxSegs;
  // The selection fused into the single-read scoring kernel, per launch
  // group: pooling widths up to 7, one query head per K/V head, and no
  // sequence shorter than its budget in the group.
  std::vector<char> fsel(ngroups, 0);
  bool any_fsel = false;
  for (int b0 = 0, gi = 0; b0 < p.B; b0 += kMaxSegs, ++gi) {
    bool ok = use_fused && g_fused_select && fused_select_kernel_ok(kernel) && p.group == 1;
    for (int b = b0; b < std::min(p.B, b0 + kMaxSegs) && ok; ++b) ok = p.L[b] >= p.C[b];
    {
      // Rounds of the launch group (as the launch below counts them).
      long long rounds = 0;
      const int grid = use_fused ? fused_grid(p.W, p.D) : 0;
      for (int b = b0; b < std::min(p.B, b0 + kMaxSegs) && ok; ++b) {
        const int fhpr = (p.fc[b] > 0 && grid > 0) ? std::min(p.heads, grid / p.fc[b]) : 0;
        rounds += fhpr > 0 ? (p.heads + fhpr - 1) / fhpr : 0;
      }
      ok = ok && rounds <= kFusedMaxRounds;
      // The end phase takes a row's chunks two groups of 64 at a time.
      for (int b = b0; b < std::min(p.B, b0 + kMaxSegs) && ok; ++b)
        ok = (p.L[b] - p.W + p.fS - 1) / p.fS <= 128;
    }
    fsel[gi] = ok;
    any_fsel = any_fsel || ok;
  }
  // Groups the cooperative selection takes (AUTO prefers it where its grid
  // fits the device: its workgroups share a row's keys, where the split
  // selection's each redo the whole row).  coop_launches() gives the
  // launches a group needs when its rows are taken a subset at a time (0:
  // more than kCoopLaunches, or rows longer than the segments cover).
  auto group_segments = [&](int b0) {
    const int nb = std::min(kMaxSegs, p.B - b0);
    int segs = 1;
    for (int b = b0; b < b0 + nb; ++b) {
      const int n = p.L[b] < p.C[b] ? p.L[b] : p.L[b] - p.W;
      segs = std::max(segs, (n + coop_segment() - 1) / coop_segment());
    }
    return segs;
  };
  auto coop_segments = [&](int b0) {
    const int nb = std::min(kMaxSegs, p.B - b0), segs = group_segments(b0);
    return segs <= coop_max_segments() && (long long)segs * nb * p.heads <= coop_cap ? segs : 0;
  };
  auto coop_launches = [&](int b0) {
    const int rows = std::min(kMaxSegs, p.B - b0) * p.heads, segs = group_segments(b0);
    if (segs > coop_max_segments() || coop_cap < segs) return 0;
    const int per = coop_cap / segs;  // rows per launch
    const int n = (rows + per - 1) / per;
    return n <= kCoopLaunches ? n : 0;
  };
  // The split selection per launch group: S workgroups per row, S as large
  // as the device holds at once (more rows than that: one each), and large
  // enough that a workgroup's share of the picks fits its list.
  std::vector<int> split_s(ngroups, 0), split_k(ngroups, 0);
  bool any_split = false;
  if (g_select != KVSEL_SELECT_EXCHANGE && (kernel == 1 || kernel == 3 || kernel == 5 || kernel == 7)) {
    for (int b0 = 0, gi = 0; b0 < p.B; b0 += kMaxSegs, ++gi) {
      if (fsel[gi] || (g_select == KVSEL_SELECT_AUTO && coop_segments(b0) > 0)) continue;
      const int nb = std::min(kMaxSegs, p.B - b0);
      int maxP = 0, maxCount = 0;
      for (int b = b0; b < b0 + nb; ++b)
        if (p.L[b] >= p.C[b]) {
          maxP = std::max(maxP, p.L[b] - p.W);
          maxCount = std::max(maxCount, p.C[b] - p.W);
        }
      const int kpt = split_kpt(maxP);
      if (kpt == 0) continue;
      const int rows = nb * p.heads;
      const int cap = split_grid_capacity(kpt, p.D, p.dtype);
      int S = std::max(1, std::min(split_max_splits(), cap / rows));
      S = std::max(S, (maxCount + split_list_capacity(kpt) - 1) / split_list_capacity(kpt));
      if (S > split_max_splits()) continue;
      split_s[gi] = S;
      split_k[gi] = kpt;
      any_split = true;
    }
  }
  if (g_select == KVSEL_SELECT_SPLIT)
    for (int gi = 0; gi < ngroups; ++gi)
      if (!fsel[gi] && split_s[gi] == 0)
        return fail(KVSEL_EUNSUPPORTED, "the split selection does not cover this call (pooling widths 1, 3, 5, 7; at "
                                        "most %d prefix positions)", split_max_positions());
  std::vector<int> coop_segs(ngroups, 0), coop_nl(ngroups, 0);
  bool any_coop = false;
  for (int b0 = 0, gi = 0; b0 < p.B; b0 += kMaxSegs, ++gi) {
    if (fsel[gi] || split_s[gi] > 0) continue;
    coop_nl[gi] = coop_launches(b0);
    coop_segs[gi] = coop_nl[gi] > 0 ? group_segments(b0) : 0;
    any_coop = any_coop || coop_segs[gi] > 0;
  }
  // Groups left to the per-row or segment-parallel chain (which use the
  // pooled scores' histograms).
  bool no_chain = true;
  for (int gi = 0; gi < ngroups; ++gi) no_chain = no_chain && (fsel[gi] || coop_segs[gi] > 0 || split_s[gi] > 0);
  unsigned* err = (unsigned*)ws;  // the header's error word
  {
    unsigned path = 0u;
    if (need_scoring)
      path |= use_fused ? KVSEL_PATH_SINGLE_READ : (lse != nullptr ? KVSEL_PATH_VOTES_ONLY : KVSEL_PATH_TWO_PASS);
    if (need_scoring && lse != nullptr) path |= KVSEL_PATH_HANDED_OVER;
    for (int b = 0; b < p.B; ++b)
      if (p.L[b] < p.C[b]) path |= KVSEL_PATH_BYPASS;
    if (any_coop) path |= KVSEL_PATH_SELECT_COOP;
    if (any_split) path |= KVSEL_PATH_SELECT_SPLIT;
    if (!no_chain) path |= whole_rows ? KVSEL_PATH_SELECT_ROWS : KVSEL_PATH_SELECT_SEGMENTS;
    if (any_fsel) path |= KVSEL_PATH_SELECT_FUSED;
    g_last_path = path;
  }
  // Calls whose first kernel clears what the call needs at zero launch no
  // fill: single-read calls whose every group selects in the scoring kernel
  // or with the cooperative or split selection, and two-pass calls that
  // compute the row statistics, every sequence at least its budget.  The
  // scoring kernel's workgroups clear the exchange slots (single-read), the
  // histograms (whole-row and segment selections), the cooperative
  // selection's words and, in the call's first launch, header word 0 (where
  // the selection kernels' flags go), a share each.  Such calls and every
  // single-read call carry a token: the scoring kernels' flags go to the
  // tagged header word, and the single-read arrival, decision and fallback
  // counters are token-tagged.
  bool self_clear = !g_validate && (use_fused || lse == nullptr);
  for (int b0 = 0, gi = 0; b0 < p.B && self_clear; b0 += kMaxSegs, ++gi) {
    bool ok = !use_fused || fsel[gi] || coop_segs[gi] > 0 || split_s[gi] > 0;
    for (int b = b0; b < std::min(p.B, b0 + kMaxSegs) && ok; ++b) ok = p.L[b] >= p.C[b];
    self_clear = ok;
  }
  const bool fill = !self_clear;
  const unsigned long long token = (use_fused && need_scoring) || self_clear ? next_token() : 0ull;
  record_call(ws, true, token);  // word 0 is cleared by the fill or by the call's first kernel
  if (fill) {
    // The header, and the histograms and the cooperative selection's words
    // that are in use, start at zero (on the two-pass path without the
    // cooperative selection the statistics kernel clears the histograms; a
    // single-read scoring kernel clears its own words).  The histograms and
    // the cooperative selection's words are contiguous.
    const bool hists = !no_chain && (use_fused || lse != nullptr);
    ZeroRanges z{};
    z.p[0] = ws;
    z.bytes[0] = 16;  // the call's flag words; the sticky word (kStickyWord) is left alone
    z.p[1] = ws + p.off_hist;
    z.bytes[1] = hists ? (long long)(p.off_coop - p.off_hist) : 0;
    z.p[2] = ws + p.off_coop;
    z.bytes[2] = any_coop ? (long long)(p.off_cw - p.off_coop) : 0;  // the fused selection's words follow
    hipError_t e = timed("fill", st, [&] { return launch_zero(z, st); });
    if (e != hipSuccess) return device_error(e, "fill launch");
  }
  if (g_validate) {
    // Validating mode: every input element of every sequence is finite.
    const size_t esz = p.dtype == KVSEL_BF16 ? 2 : 4;
    const long long q16 = (long long)p.B * p.heads * p.W * p.D * (long long)esz / 16;
    const long long kv16 = (long long)(p.heads / p.group) * p.cuL[p.B] * p.D * (long long)esz / 16;
    hipError_t e = timed("check", st, [&] {
      hipError_t r = launch_check_finite(Q, q16, p.dtype, err, st);
      if (r == hipSuccess) r = launch_check_finite(K, kv16, p.dtype, err, st);
      if (r == hipSuccess) r = launch_check_finite(V, kv16, p.dtype, err, st);
      if (r == hipSuccess && lse != nullptr) r = launch_check_finite_f32(lse, (long long)p.B * p.heads * p.W, err, st);
      return r;
    });
    if (e != hipSuccess) return device_error(e, "check launch");
  }

  for (int b0 = 0; b0 < p.B; b0 += kMaxSegs) {
    const int nb = std::min(kMaxSegs, p.B - b0);
    Launch a = base_launch(p, kernel, pooling);
    a.err = err;
    a.token = token;
    a.errw = (unsigned long long*)(ws + 4 * kTaggedWord);
    {
      // K tiles bypass the caches when the group's K is larger than the
      // last-level cache could keep for a later read.
      long long kv_rows = 0;
      for (int b = b0; b < b0 + nb; ++b) kv_rows += (long long)(p.heads / p.group) * p.L[b];
      const double k_bytes = (double)kv_rows * p.D * (p.dtype == KVSEL_BF16 ? 2 : 4);
      a.k_nt = k_bytes > kTwoPassCachedBytes ? 1 : 0;
    }
    a.n = nb;
    a.S = p.fS;
    a.rounds = 0;
    int items = 0, rows = 0, maxP = 0, maxN = 0;
    for (int k = 0; k < nb; ++k) {
      const int b = b0 + k;
      Seg& s = a.seg[k];
      s.b = b;
      s.L = p.L[b];
      s.C = p.C[b];
      s.nout = std::min(s.L, s.C);
      s.h0 = 0;
      s.nh = p.heads;
      s.nch = p.nch[b];
      s.item0 = items;
      s.row0 = rows;
      s.gitem0 = 0;
      s.gblk = 0;
      s.idx_ld = s.C;
      s.out_ld = s.C;
      s.vote_ld = s.L - p.W;
      s.kv_off = (long long)(p.heads / p.group) * p.cuL[b] * p.D;
      s.idx_off = (long long)p.heads * p.cuC[b];
      s.out_off = s.idx_off;
      s.vote_off = (long long)p.heads * p.cuP[b];
      s.part_base = p.part[b];
      s.fslot_base = p.fpart[b];
      s.fc = p.fc[b];
      s.fhpr = s.fc > 0 && grid > 0 ? std::min(s.nh, grid / s.fc) : 0;
      s.fnr = s.fhpr > 0 ? (s.nh + s.fhpr - 1) / s.fhpr : 0;
      s.fr0 = a.rounds;
      a.rounds += s.fnr;
      items += (s.nh / p.group) * s.nch;  // scoring items run over the K/V heads
      rows += s.nh;
      if (s.L >= s.C) maxP = std::max(maxP, s.L - p.W);
      maxN = std::max(maxN, s.L >= s.C ? s.L - p.W : s.L);
    }
    a.seg_size = selection_seg_size(maxN);
    uint32_t* ghist = hist + (long long)b0 * p.heads * 2048;
    uint32_t* gcut = (uint32_t*)((char*)cut + (size_t)b0 * p.heads * kCutBytes);
    uint32_t* gseg = (uint32_t*)((char*)segcnt + (size_t)b0 * p.heads * kSegCntBytes);
    hipError_t e;
    FusedSel sel{};
    if (use_fused) {
      // Every single-read launch: the token, the arrival tokens, decision and
      // fallback counters, the completion counts and chunk statistics of the
      // fallback; the exchange slots (not read with handed-over statistics)
      // are cleared by the kernel's workgroups, a share each.
      const int gi = b0 / kMaxSegs;
      sel.force_abort = g_force_fallback;
      sel.token = token;
      sel.errw = (unsigned long long*)(ws + 4 * kTaggedWord);
      sel.flags = (unsigned long long*)(ws + p.off_flags) + (long long)kFusedFlagWords * gi;
      sel.rowfb = (unsigned long long*)(ws + p.off_rowfb) + (long long)b0 * p.heads * 2;
      sel.kslot = (float*)(ws + p.off_kslot);
      sel.clr[0] = lse == nullptr ? (unsigned long long*)(ws + p.off_ctr) : nullptr;
      sel.clr_words[0] = lse == nullptr ? (long long)(p.off_hist - p.off_ctr) / 8 : 0;
      sel.clr_early = 1;  // the exchange slots; the rest only later kernels read
      if (!fill && coop_segs[gi] > 0) {
        // The cooperative selection's status blocks and row words of this
        // group, which its launches after this one need at zero.
        sel.clr[1] = (unsigned long long*)(ws + p.off_coop) + (long long)kFusedStatusWords * kCoopLaunches * gi / 2;
        sel.clr_words[1] = (long long)kFusedStatusWords * coop_nl[gi] / 2;  // the launches made
        sel.clr[2] = (unsigned long long*)(ws + p.off_coop) +
                     ((long long)kFusedStatusWords * kCoopLaunches * ngroups + (long long)b0 * p.heads * coop_row_words()) / 2;
        sel.clr_words[2] = (long long)rows * coop_row_words() / 2;
      }
      if (!fill && b0 == 0) {  // header words 0 and 1: the selection kernels' flags of this call
        sel.clr[3] = (unsigned long long*)ws;
        sel.clr_words[3] = 1;
      }
    }
    if (fsel[b0 / kMaxSegs]) {
      sel.on = 1;
      sel.cw = (unsigned long long*)(ws + p.off_cw);
      sel.halo = (unsigned long long*)(ws + p.off_halo);
      sel.cslot = (unsigned*)(ws + p.off_cslot);
      sel.fslot = (unsigned*)(ws + p.off_fslot);
      // Also cleared by the kernel's workgroups before they arrive: the
      // count, halo and histogram words (contiguous).
      sel.clr[1] = (unsigned long long*)(ws + p.off_cw);
      sel.clr_words[1] = (long long)(p.off_flags - p.off_cw) / 8;
      sel.clr_early = 2;
      sel.cand = (unsigned long long*)(ws + p.off_cand);
      sel.pooled = pooled_opt;
      sel.indices = indices;
      sel.V = V;
      sel.K_out = K_out;
      sel.V_out = V_out;
    }
    if (items > 0 && use_fused) {
      e = timed("window_fused", st,
                [&] { return launch_fused_scoring(a, Q, K, lse, counters, votes, row_stats, sel, st); });
      if (e != hipSuccess) return device_error(e, "window_fused launch");
      if (sel.on) continue;  // the selection ran in the same kernel
    } else if (items > 0 && lse != nullptr) {
      e = timed("window_votes", st,
                [&] { return launch_window_votes(a, items, p.dtype, Q, K, pm, pz, lse, votes, nullptr, st); });
      if (e != hipSuccess) return device_error(e, "window_votes launch");
    } else if (items > 0) {
      // Cleared by the statistics kernel for the kernels after it: the
      // histograms of a whole-row or segment selection; without a fill, the
      // cooperative selection's words of this group and (first group) header
      // words 0 and 1.
      const int gi = b0 / kMaxSegs;
      const bool chain = coop_segs[gi] == 0 && split_s[gi] == 0;
      WordRanges clear{};
      clear.p[0] = ghist;
      clear.n[0] = chain ? (long long)rows * 2048 : 0;
      if (!fill && coop_segs[gi] > 0) {
        clear.p[1] = (unsigned*)(ws + p.off_coop) + (long long)kFusedStatusWords * kCoopLaunches * gi;
        clear.n[1] = (long long)kFusedStatusWords * coop_nl[gi];  // the status lines of the launches made
        clear.p[2] = (unsigned*)(ws + p.off_coop) + (long long)kFusedStatusWords * kCoopLaunches * ngroups +
                     (long long)b0 * p.heads * coop_row_words();
        clear.n[2] = (long long)rows * coop_row_words();
      }
      if (!fill && b0 == 0) {
        clear.p[3] = (unsigned*)ws;
        clear.n[3] = 2;
      }
      e = timed("window_stats", st, [&] { return launch_window_stats(a, items, p.dtype, Q, K, pm, pz, clear, st); });
      if (e != hipSuccess) return device_error(e, "window_stats launch");
      e = timed("window_votes", st,
                [&] { return launch_window_votes(a, items, p.dtype, Q, K, pm, pz, nullptr, votes, row_stats, st); });
      if (e != hipSuccess) return device_error(e, "window_votes launch");
    }
    if (split_s[b0 / kMaxSegs] > 0) {
      e = timed("select", st, [&] {
        return launch_select_split(a, rows, split_s[b0 / kMaxSegs], split_k[b0 / kMaxSegs], p.dtype, votes, pooled_opt,
                                   indices, K, V, K_out, V_out, st);
      });
      if (e != hipSuccess) return device_error(e, "select launch");
      continue;
    }
    if (coop_segs[b0 / kMaxSegs] > 0) {
      const int gi = b0 / kMaxSegs, nl = coop_nl[gi];
      unsigned* cstatus0 = (unsigned*)(ws + p.off_coop) + (long long)kFusedStatusWords * kCoopLaunches * gi;
      unsigned* crows = (unsigned*)(ws + p.off_coop) +
                        (long long)kFusedStatusWords * kCoopLaunches * ngroups +
                        (long long)b0 * p.heads * coop_row_words();
      // Launch k takes rows [k * per, (k + 1) * per) of the group: its
      // segment table holds those rows' head ranges, renumbered from 0.
      const int per = (rows + nl - 1) / nl;
      for (int k = 0; k < nl; ++k) {
        const int r_lo = k * per, r_hi = std::min(rows, r_lo + per);
        if (r_lo >= r_hi) break;
        Launch ak = a;
        ak.n = 0;
        for (int q = 0; q < a.n; ++q) {
          const Seg& sq = a.seg[q];
          const int lo = std::max(sq.row0, r_lo), hi = std::min(sq.row0 + sq.nh, r_hi);
          if (lo >= hi) continue;
          Seg t = sq;
          t.h0 = sq.h0 + (lo - sq.row0);
          t.nh = hi - lo;
          t.row0 = lo - r_lo;
          ak.seg[ak.n++] = t;
        }
        unsigned* cstatus = cstatus0 + (long long)kFusedStatusWords * k;
        if (g_force_fallback) {
          e = launch_fill_u32(cstatus + 2, 1, kFusedAbort, st);  // decided before any workgroup arrives
          if (e != hipSuccess) return device_error(e, "fill launch");
        }
        e = timed("select", st, [&] {
          return launch_select_coop(ak, r_hi - r_lo, coop_segs[gi], p.dtype, votes, pooled_opt,
                                    crows + (long long)r_lo * coop_row_words(), cstatus, indices, K, V, K_out,
                                    V_out, st);
        });
        if (e != hipSuccess) return device_error(e, "select launch");
      }
      continue;
    }
    if (whole_rows) {
      if (items > 0) {
        e = timed("pool", st, [&] { return launch_pool(a, rows, maxP, votes, pooled, ghist, st); });
        if (e != hipSuccess) return device_error(e, "pool launch");
      }
      e = timed("select", st, [&] { return launch_select_hist(a, rows, pooled, ghist, indices, st); });
      if (e != hipSuccess) return device_error(e, "select launch");
      const int rpb = gather_rows_per_block(p.D, p.dtype);
      int gitems = 0;
      for (int k = 0; k < nb; ++k) {
        Seg& s = a.seg[k];
        s.gitem0 = gitems;
        s.gblk = (s.nout + rpb - 1) / rpb;
        gitems += s.nh * s.gblk;
      }
      e = timed("gather", st, [&] { return launch_gather(a, gitems, p.dtype, K, V, indices, K_out, V_out, st); });
      if (e != hipSuccess) return device_error(e, "gather launch");
      continue;
    }
    if (items > 0) {
      e = timed("pool", st, [&] { return launch_pool(a, rows, maxP, votes, pooled, ghist, st); });
      if (e != hipSuccess) return device_error(e, "pool launch");
      e = timed("candidates", st,
                [&] { return launch_candidates(a, rows, maxP, pooled, ghist, cand, gseg, st); });
      if (e != hipSuccess) return device_error(e, "candidates launch");
      e = timed("threshold", st, [&] { return launch_threshold(a, rows, ghist, cand, gcut, gseg, st); });
      if (e != hipSuccess) return device_error(e, "threshold launch");
    }
    e = timed("emit", st, [&] {
      return launch_emit(a, rows, maxN, p.dtype, pooled, gcut, gseg, indices, K, V, K_out, V_out, st);
    });
    if (e != hipSuccess) return device_error(e, "emit launch");
  }
  return ok();
}

// ---- allocation-free selection (kvsel_select_noalloc): the per-device
// scratch address (the array is declared at file scope above).
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The current device's scratch address, looked up on the first call made on
// that device.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(KVSEL_EUNSUPPORTED, "device ordinal %d exceeds the %d devices the scratch table holds", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_error(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || (uintptr_t)p % 256 != 0)
      return fail(KVSEL_EDEVICE, "scratch array at an unusable address %p", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVSEL_OK;
}

struct NoEvents {
  NoEvents() { g_no_events = true; }
  ~NoEvents() { g_no_events = false; }
};

}  // namespace

extern "C" {

int kvsel_version(void) { return (0 << 16) | 3; }

int kvsel_debug_flags(int reset) {
  const int v = debug_flags_read(reset);
  if (v < 0) return fail(KVSEL_EUNSUPPORTED, "not a KVSEL_DEBUG build (or the device word could not be read)");
  ok();
  return v;
}

int kvsel_set_option(int option, int value) {
  if (option == KVSEL_OPT_SCORING) {
    if (value < KVSEL_SCORING_AUTO || value > KVSEL_SCORING_SINGLE_READ)
      return fail(KVSEL_EINVAL, "invalid scoring value %d", value);
    g_scoring = value;
    return ok();
  }
  if (option == KVSEL_OPT_FORCE_FALLBACK) {
    if (value != 0 && value != 1) return fail(KVSEL_EINVAL, "invalid fallback value %d", value);
    g_force_fallback = value;
    return ok();
  }
  if (option == KVSEL_OPT_VALIDATE) {
    if (value != 0 && value != 1) return fail(KVSEL_EINVAL, "invalid validate value %d", value);
    g_validate = value;
    return ok();
  }
  if (option == KVSEL_OPT_FUSED_SELECT) {
    if (value != 0 && value != 1) return fail(KVSEL_EINVAL, "invalid fused-select value %d", value);
    g_fused_select = value;
    return ok();
  }
  if (option == KVSEL_OPT_SELECT) {
    if (value < KVSEL_SELECT_AUTO || value > KVSEL_SELECT_EXCHANGE) return fail(KVSEL_EINVAL, "invalid select value %d", value);
    g_select = value;
    return ok();
  }
  return fail(KVSEL_EINVAL, "unknown option %d", option);
}

int kvsel_get_option(int option) {
  if (option == KVSEL_OPT_SCORING) return g_scoring;
  if (option == KVSEL_OPT_FORCE_FALLBACK) return g_force_fallback;
  if (option == KVSEL_OPT_VALIDATE) return g_validate;
  if (option == KVSEL_OPT_FUSED_SELECT) return g_fused_select;
  if (option == KVSEL_OPT_SELECT) return g_select;
  return fail(KVSEL_EINVAL, "unknown option %d", option);
}

const char* kvsel_last_error(void) { return g_error.c_str(); }

int kvsel_status(const void* workspace, void* stream) {
  if (!workspace) return fail(KVSEL_EINVAL, "workspace must not be NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(KVSEL_EINVAL, "workspace must be 256-byte aligned");
  unsigned words[4] = {};
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(words, workspace, sizeof words, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return device_error(e, "status read");
  const unsigned flags =
      last_call_flags(workspace, words[0], ((unsigned long long)words[kTaggedWord + 1] << 32) | words[kTaggedWord]);
  if (flags & (kErrExchangeWait | kErrLdsWait | kErrSelectWait))
    return fail(KVSEL_EDEVICE, "a bounded device-side wait timed out (flags 0x%x): the outputs of that call are "
                               "unreliable", flags);
  if (flags & kErrIndexRange)
    return fail(KVSEL_EDEVICE, "an index outside its range reached a row copy (flags 0x%x, a KVSEL_DEBUG build "
                               "check): the outputs of that call are unreliable", flags);
  if (flags & kErrDomain)
    return fail(KVSEL_EINVAL, "an input outside its domain: a negative or NaN lambda_q entry (flags 0x%x)", flags);
  if (flags & kErrNonFinite)
    return fail(KVSEL_ENONFINITE, "a non-finite input value or a non-finite or zero row normaliser (flags 0x%x)",
                flags);
  return ok();
}

int kvsel_status_flags(const void* workspace, void* stream, int reset, unsigned* last_flags, unsigned* sticky_flags) {
  if (!workspace) return fail(KVSEL_EINVAL, "workspace must not be NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(KVSEL_EINVAL, "workspace must be 256-byte aligned");
  unsigned words[kStickyWord + 1] = {};
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(words, workspace, sizeof words, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && reset) {
    static const unsigned zero = 0u;
    e = hipMemcpyAsync((unsigned*)workspace + kStickyWord, &zero, sizeof zero, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  if (e != hipSuccess) return device_error(e, "status read");
  if (last_flags)
    *last_flags = last_call_flags(workspace, words[0],
                                  ((unsigned long long)words[kTaggedWord + 1] << 32) | words[kTaggedWord]);
  if (sticky_flags) *sticky_flags = words[kStickyWord];
  return ok();
}

unsigned kvsel_last_path(void) { return g_last_path; }

size_t kvsel_probe_sink_bytes(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return (size_t)probe_sink_words(cus) * sizeof(unsigned);
}

int kvsel_probe_stream(const void* src, size_t bytes, int mode, void* sink, size_t sink_bytes, void* stream) {
  if (!src || !sink) return fail(KVSEL_EINVAL, "src and sink must not be NULL");
  if (mode < 0 || mode > 4) return fail(KVSEL_EINVAL, "probe mode must be 0..4 (got %d)", mode);
  if ((uintptr_t)src % 16 || (uintptr_t)sink % 4) return fail(KVSEL_EINVAL, "src must be 16-byte aligned");
  if (mode != 3 && bytes % (128 * 1024) != 0)
    return fail(KVSEL_EINVAL, "tile probes read whole 128 KiB blocks (%zu bytes)", bytes);
  if (bytes % 16 != 0 || bytes == 0) return fail(KVSEL_EINVAL, "bytes must be a positive multiple of 16");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_error(e, "device query");
  if (sink_bytes < (size_t)probe_sink_words(cus) * sizeof(unsigned))
    return fail(KVSEL_EWORKSPACE, "sink of %zu bytes is smaller than the %zu required", sink_bytes,
                (size_t)probe_sink_words(cus) * sizeof(unsigned));
  e = timed(mode == 3 ? "probe_vector" : "probe_tiles", (hipStream_t)stream,
            [&] { return launch_probe(mode, src, (long long)bytes, (unsigned*)sink, cus, (hipStream_t)stream); });
  if (e != hipSuccess) return device_error(e, "probe launch");
  return ok();
}

size_t kvsel_varlen_workspace_bytes(const int32_t* cu_L_host, const int32_t* C_host, int B, int heads, int W,
                                    int D, int dtype) {
  Plan p;
  if (make_plan(cu_L_host, C_host, B, heads, W, D, dtype, p) != KVSEL_OK) return 0;
  ok();
  return p.bytes;
}

size_t kvsel_gqa_workspace_bytes(int q_heads, int kv_heads, int L, int W, int C, int D, int dtype) {
  if (kv_heads < 1) {
    fail(KVSEL_EINVAL, "kv_heads must be >= 1 (got %d)", kv_heads);
    return 0;
  }
  const int32_t cu[2] = {0, L};
  const int32_t c[1] = {C};
  Plan p;
  if (make_plan(cu, c, 1, q_heads, W, D, dtype, p, kv_heads) != KVSEL_OK) return 0;
  ok();
  return p.bytes;
}

size_t kvsel_workspace_bytes(int heads, int L, int W, int C, int D, int dtype) {
  const int32_t cu[2] = {0, L};
  const int32_t c[1] = {C};
  return kvsel_varlen_workspace_bytes(cu, c, 1, heads, W, D, dtype);
}

static int select_entry(const void* Qwin, const void* K, const void* V, const float* lse,
                        const int32_t* cu_L_host, const int32_t* C_host, int B, int W, int D, int heads, int kernel,
                        int pooling, int dtype, int32_t* indices, void* K_out, void* V_out, float* row_stats_opt,
                        float* votes_opt, float* pooled_opt, void* workspace, size_t workspace_bytes,
                        void* stream, int kv_heads = 0) {
  Plan p;
  int rc = make_plan(cu_L_host, C_host, B, heads, W, D, dtype, p, kv_heads);
  if (rc) return rc;
  if ((rc = check_pool(kernel, pooling))) return rc;
  if (!Qwin || !K || !V || !indices || !K_out || !V_out)
    return fail(KVSEL_EINVAL, "Qwin, K, V, indices, K_out and V_out must not be NULL");
  if (!workspace) return fail(KVSEL_EINVAL, "workspace must not be NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(KVSEL_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.bytes)
    return fail(KVSEL_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, p.bytes);
  const size_t esz = dtype == KVSEL_BF16 ? 2 : 4;
  if ((uintptr_t)Qwin % 16 || (uintptr_t)K % 16 || (uintptr_t)V % 16 || (uintptr_t)K_out % 16 ||
      (uintptr_t)V_out % 16)
    return fail(KVSEL_EINVAL, "Qwin, K, V, K_out and V_out must be 16-byte aligned");
  (void)esz;
  return run_select(Qwin, K, V, lse, p, kernel, pooling, indices, K_out, V_out, row_stats_opt, votes_opt,
                    pooled_opt, workspace, (hipStream_t)stream);
}

int kvsel_select_varlen(const void* Qwin, const void* K, const void* V, const int32_t* cu_L_host,
                        const int32_t* C_host, int B, int W, int D, int heads, int kernel, int pooling, int dtype,
                        int32_t* indices, void* K_out, void* V_out, float* row_stats_opt, float* votes_opt,
                        float* pooled_opt, void* workspace, size_t workspace_bytes, void* stream) {
  return select_entry(Qwin, K, V, nullptr, cu_L_host, C_host, B, W, D, heads, kernel, pooling, dtype, indices, K_out,
                      V_out, row_stats_opt, votes_opt, pooled_opt, workspace, workspace_bytes, stream);
}

int kvsel_select_varlen_lse(const void* Qwin, const void* K, const void* V, const float* row_lse,
                            const int32_t* cu_L_host, const int32_t* C_host, int B, int W, int D, int heads,
                            int kernel, int pooling, int dtype, int32_t* indices, void* K_out, void* V_out,
                            float* votes_opt, float* pooled_opt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!row_lse) return fail(KVSEL_EINVAL, "row_lse must not be NULL");
  if ((uintptr_t)row_lse % 4) return fail(KVSEL_EINVAL, "row_lse must be 4-byte aligned");
  return select_entry(Qwin, K, V, row_lse, cu_L_host, C_host, B, W, D, heads, kernel, pooling, dtype, indices,
                      K_out, V_out, nullptr, votes_opt, pooled_opt, workspace, workspace_bytes, stream);
}

int kvsel_select_gqa(const void* Qwin, const void* K, const void* V, const float* row_lse_opt, int L, int W, int C,
                     int D, int q_heads, int kv_heads, int kernel, int pooling, int dtype, int32_t* indices,
                     void* K_out, void* V_out, float* row_stats_opt, float* votes_opt, float* pooled_opt,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_heads < 1) return fail(KVSEL_EINVAL, "kv_heads must be >= 1 (got %d)", kv_heads);
  if (row_lse_opt && (uintptr_t)row_lse_opt % 4) return fail(KVSEL_EINVAL, "row_lse must be 4-byte aligned");
  if (row_lse_opt && row_stats_opt)
    return fail(KVSEL_EINVAL, "row statistics are not computed when they are handed over (row_lse)");
  const int32_t cu[2] = {0, L};
  const int32_t c[1] = {C};
  return select_entry(Qwin, K, V, row_lse_opt, cu, c, 1, W, D, q_heads, kernel, pooling, dtype, indices, K_out,
                      V_out, row_stats_opt, votes_opt, pooled_opt, workspace, workspace_bytes, stream, kv_heads);
}

int kvsel_select_lse(const void* Qwin, const void* K, const void* V, const float* row_lse, int L, int W, int C,
                     int D, int heads, int kernel, int pooling, int dtype, int32_t* indices, void* K_out,
                     void* V_out, float* votes_opt, float* pooled_opt, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const int32_t cu[2] = {0, L};
  const int32_t c[1] = {C};
  return kvsel_select_varlen_lse(Qwin, K, V, row_lse, cu, c, 1, W, D, heads, kernel, pooling, dtype, indices, K_out,
                                 V_out, votes_opt, pooled_opt, workspace, workspace_bytes, stream);
}

int kvsel_select(const void* Qwin, const void* K, const void* V, int L, int W, int C, int D, int heads, int kernel,
                 int pooling, int dtype, int32_t* indices, void* K_out, void* V_out, float* row_stats_opt,
                 float* votes_opt, float* pooled_opt, void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t cu[2] = {0, L};
  const int32_t c[1] = {C};
  return kvsel_select_varlen(Qwin, K, V, cu, c, 1, W, D, heads, kernel, pooling, dtype, indices, K_out, V_out,
                             row_stats_opt, votes_opt, pooled_opt, workspace, workspace_bytes, stream);
}

static size_t topk_workspace(int rows, int n) {
  return align256((size_t)rows * 2048 * 4) + align256((size_t)rows * kCutBytes) +
         align256((size_t)rows * kSegCntBytes) + align256((size_t)rows * n * 4);
}

size_t kvsel_topk_workspace_bytes(int rows, int n) {
  if (rows < 1 || n < 1) {
    fail(KVSEL_EINVAL, "rows and n must be >= 1 (got %d, %d)", rows, n);
    return 0;
  }
  ok();
  return topk_workspace(rows, n);
}

// Top-k over rows of scores described by a (one segment: positions 0 .. L-1 of
// each row at scores + vote_off + row * vote_ld, C - (window ? W : 0) picks,
// then the window positions when a.window), into out + idx_off + row * idx_ld.
static int run_topk(Launch& a, int rows, const float* scores, int32_t* out, void* workspace, hipStream_t st,
                    bool hist_zeroed = false) {
  const Seg& s = a.seg[0];
  const int n = s.L;
  a.seg_size = selection_seg_size(n);
  uint32_t* hist = (uint32_t*)workspace;
  uint32_t* cut = (uint32_t*)((char*)workspace + align256((size_t)rows * 2048 * 4));
  uint32_t* segcnt = (uint32_t*)((char*)cut + align256((size_t)rows * kCutBytes));
  uint32_t* cand = (uint32_t*)((char*)segcnt + align256((size_t)rows * kSegCntBytes));
  hipError_t e = hipSuccess;
  // The split selection (indices only, no pooling) where it covers the rows.
  const int W = a.window ? a.W : 0;
  const int kpt = g_select != KVSEL_SELECT_EXCHANGE ? split_kpt(n - W) : 0;
  if (kpt > 0) {
    const int count = s.C - W;
    int S = std::max(1, std::min(split_max_splits(), split_grid_capacity(kpt, 0, 0) / rows));
    S = std::max(S, (count + split_list_capacity(kpt) - 1) / split_list_capacity(kpt));
    if (S <= split_max_splits()) {
      Launch b = a;
      b.kernel = 1;
      b.pooling = KVSEL_POOL_AVG;
      e = timed("select", st, [&] {
        return launch_select_split(b, rows, S, kpt, KVSEL_F32, scores, nullptr, out, nullptr, nullptr, nullptr, nullptr,
                                   st);
      });
      if (e != hipSuccess) return device_error(e, "select launch");
      g_last_path = KVSEL_PATH_SELECT_SPLIT;
      return ok();
    }
  }
  if (g_select == KVSEL_SELECT_SPLIT)
    return fail(KVSEL_EUNSUPPORTED, "the split selection does not cover rows of %d scores (at most %d)", n - W,
                split_max_positions());
  g_last_path = n <= select_rows_max() ? KVSEL_PATH_SELECT_ROWS : KVSEL_PATH_SELECT_SEGMENTS;
  if (!hist_zeroed) {  // otherwise an earlier kernel of the call cleared the histograms
    e = timed("fill", st, [&] { return launch_fill_u32(hist, (long long)rows * 2048, 0u, st); });
    if (e != hipSuccess) return device_error(e, "fill launch");
  }
  e = timed("pool", st, [&] { return launch_pool(a, rows, n, scores, nullptr, hist, st); });
  if (e != hipSuccess) return device_error(e, "histogram launch");
  if (n <= select_rows_max()) {  // one workgroup per row
    e = timed("select", st, [&] { return launch_select_hist(a, rows, scores, hist, out, st); });
    if (e != hipSuccess) return device_error(e, "select launch");
    return ok();
  }
  e = timed("candidates", st, [&] { return launch_candidates(a, rows, n, scores, hist, cand, segcnt, st); });
  if (e != hipSuccess) return device_error(e, "candidates launch");
  e = timed("threshold", st, [&] { return launch_threshold(a, rows, hist, cand, cut, segcnt, st); });
  if (e != hipSuccess) return device_error(e, "threshold launch");
  e = timed("emit", st, [&] {
    return launch_emit(a, rows, n, 0, scores, cut, segcnt, out, nullptr, nullptr, nullptr, nullptr, st);
  });
  if (e != hipSuccess) return device_error(e, "emit launch");
  return ok();
}

int kvsel_topk(const float* scores, int rows, int n, int count, int32_t* out, int ld_out, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!scores || !out) return fail(KVSEL_EINVAL, "scores and out must not be NULL");
  if (rows < 1 || n < 1) return fail(KVSEL_EINVAL, "rows and n must be >= 1 (got %d, %d)", rows, n);
  if (count < 1 || count > n) return fail(KVSEL_EINVAL, "count must be in [1, n] (got %d, n = %d)", count, n);
  if (ld_out < count) return fail(KVSEL_EINVAL, "ld_out %d is smaller than count %d", ld_out, count);
  if (!workspace) return fail(KVSEL_EINVAL, "workspace must not be NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(KVSEL_EINVAL, "workspace must be 256-byte aligned");
  const size_t need = topk_workspace(rows, n);
  if (workspace_bytes < need)
    return fail(KVSEL_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
  Launch a{};
  a.n = 1;
  a.heads = rows;
  a.window = 0;
  Seg& s = a.seg[0];
  s.L = n;
  s.C = count;
  s.nout = count;
  s.nh = rows;
  s.idx_ld = ld_out;
  s.vote_ld = n;
  return run_topk(a, rows, scores, out, workspace, (hipStream_t)stream);
}

size_t kvsel_refresh_workspace_bytes(int rows, int n) { return kvsel_topk_workspace_bytes(rows, n); }

static int refresh_core(const float* scores, int rows, int n, int keep, int protect_head, int protect_tail,
                        const void* K, const void* V, int D, int dtype, const int32_t* tokens_opt, int32_t* indices,
                        void* K_out, void* V_out, int32_t* tokens_out_opt, void* workspace, hipStream_t st,
                        bool hist_zeroed = false);

int kvsel_refresh(const float* scores, int rows, int n, int keep, int protect_head, int protect_tail,
                  const void* K, const void* V, int D, int dtype, const int32_t* tokens_opt, int32_t* indices,
                  void* K_out, void* V_out, int32_t* tokens_out_opt, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!scores || !indices || !K || !V || !K_out || !V_out)
    return fail(KVSEL_EINVAL, "scores, indices, K, V, K_out and V_out must not be NULL");
  if (rows < 1 || n < 1) return fail(KVSEL_EINVAL, "rows and n must be >= 1 (got %d, %d)", rows, n);
  if (keep < 1 || keep > n) return fail(KVSEL_EINVAL, "keep must be in [1, n] (got %d, n = %d)", keep, n);
  if (protect_head < 0 || protect_tail < 0 || (long long)protect_head + protect_tail > keep)
    return fail(KVSEL_EINVAL, "protected head %d and tail %d must be >= 0 and fit the %d kept", protect_head,
                protect_tail, keep);
  if (!tokens_opt != !tokens_out_opt) return fail(KVSEL_EINVAL, "tokens and tokens_out go together");
  if (dtype != KVSEL_F32 && dtype != KVSEL_BF16) return fail(KVSEL_EINVAL, "unknown dtype %d", dtype);
  if (D != 64 && D != 128) return fail(KVSEL_EUNSUPPORTED, "head dimension %d not supported (64 or 128)", D);
  if ((uintptr_t)K % 16 || (uintptr_t)V % 16 || (uintptr_t)K_out % 16 || (uintptr_t)V_out % 16)
    return fail(KVSEL_EINVAL, "K, V, K_out and V_out must be 16-byte aligned");
  if (!workspace) return fail(KVSEL_EINVAL, "workspace must not be NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(KVSEL_EINVAL, "workspace must be 256-byte aligned");
  const size_t need = topk_workspace(rows, n);
  if (workspace_bytes < need)
    return fail(KVSEL_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
  return refresh_core(scores, rows, n, keep, protect_head, protect_tail, K, V, D, dtype, tokens_opt, indices, K_out,
                      V_out, tokens_out_opt, workspace, (hipStream_t)stream);
}

static int refresh_core(const float* scores, int rows, int n, int keep, int protect_head, int protect_tail,
                        const void* K, const void* V, int D, int dtype, const int32_t* tokens_opt, int32_t* indices,
                        void* K_out, void* V_out, int32_t* tokens_out_opt, void* workspace, hipStream_t st,
                        bool hist_zeroed) {
  const int flexible = keep - protect_head - protect_tail;
  if (flexible > 0) {
    // Positions protect_head .. n-1 of each row, the last protect_tail of
    // them appended as a window after the picks.
    Launch a{};
    a.n = 1;
    a.heads = rows;
    a.window = 1;
    a.W = protect_tail;
    Seg& s = a.seg[0];
    s.L = n - protect_head;
    s.C = keep - protect_head;
    s.nout = s.C;
    s.nh = rows;
    s.vote_off = protect_head;
    s.vote_ld = n;
    s.idx_off = protect_head;
    s.idx_ld = keep;
    const int rc = run_topk(a, rows, scores, indices, workspace, st, hist_zeroed);
    if (rc) return rc;
  }
  hipError_t e = timed("finish", st, [&] {
    return launch_refresh_finish(rows, n, keep, protect_head, protect_tail, flexible > 0, indices, tokens_opt,
                                 tokens_out_opt, st);
  });
  if (e != hipSuccess) return device_error(e, "finish launch");
  const int rpb = gather_rows_per_block(D, dtype);
  Launch g{};
  g.n = 1;
  g.heads = rows;
  g.D = D;
  Seg& gs = g.seg[0];
  gs.L = n;
  gs.C = keep;
  gs.nout = keep;
  gs.nh = rows;
  gs.gblk = (keep + rpb - 1) / rpb;
  gs.idx_ld = keep;
  gs.out_ld = keep;
  const long long items = (long long)rows * gs.gblk;
  if (items > 0x7FFFFFFFLL) return fail(KVSEL_EUNSUPPORTED, "gather grid too large");
  e = timed("gather", st, [&] { return launch_gather(g, (int)items, dtype, K, V, indices, K_out, V_out, st); });
  if (e != hipSuccess) return device_error(e, "gather launch");
  return ok();
}

// Jacap workspace: z, kappa, w, r ([heads][N] each), softmax partials, the
// Gram parts, L^{-1} (hi, lo), then the refresh selection's workspace.
struct JacapPlan {
  size_t off_z, off_kappa, off_w, off_r, off_part, off_gram, off_minv, off_sel, bytes;
};
static JacapPlan jacap_plan(int heads, int N, int D) {
  JacapPlan q{};
  const size_t hn = (size_t)heads * N * sizeof(float);
  size_t off = kHeaderBytes;  // the header's error word, as for the selection calls
  q.off_z = off;
  off = align256(off + hn);
  q.off_kappa = off;
  off = align256(off + hn);
  q.off_w = off;
  off = align256(off + hn);
  q.off_r = off;
  off = align256(off + hn);
  q.off_part = off;
  off = align256(off + (size_t)heads * jacap_chunks(N) * 2 * sizeof(float));
  q.off_gram = off;
  off = align256(off + (size_t)heads * jacap_slices(N, heads) * D * D * sizeof(float));
  q.off_minv = off;
  off = align256(off + (size_t)heads * 2 * D * D * 2);
  q.off_sel = off;
  off = align256(off + topk_workspace(heads, N));
  q.bytes = off;
  return q;
}

size_t kvsel_jacap_workspace_bytes(int heads, int N, int D) {
  if (heads < 1 || N < 1 || (D != 64 && D != 128)) {
    fail(KVSEL_EINVAL, "heads and N must be >= 1 and D 64 or 128 (got %d, %d, %d)", heads, N, D);
    return 0;
  }
  ok();
  return jacap_plan(heads, N, D).bytes;
}

int kvsel_jacap_select(const void* K, const void* V, const void* U, const float* mu_q, const float* lambda_q,
                       float tau, int heads, int N, int D, int dtype, int keep, int protect_head, int protect_tail,
                       const int32_t* tokens_opt, int32_t* indices, void* K_out, void* V_out,
                       int32_t* tokens_out_opt, float* scores_opt, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!K || !V || !U || !mu_q || !lambda_q || !indices || !K_out || !V_out)
    return fail(KVSEL_EINVAL, "K, V, U, mu_q, lambda_q, indices, K_out and V_out must not be NULL");
  if (heads < 1 || N < 1) return fail(KVSEL_EINVAL, "heads and N must be >= 1 (got %d, %d)", heads, N);
  if (!(tau > 0.f) || !isfinite(tau)) return fail(KVSEL_EINVAL, "temperature must be finite and > 0");
  if (keep < 1 || keep > N) return fail(KVSEL_EINVAL, "keep must be in [1, N] (got %d, N = %d)", keep, N);
  if (protect_head < 0 || protect_tail < 0 || (long long)protect_head + protect_tail > keep)
    return fail(KVSEL_EINVAL, "protected head %d and tail %d must be >= 0 and fit the %d kept", protect_head,
                protect_tail, keep);
  if (!tokens_opt != !tokens_out_opt) return fail(KVSEL_EINVAL, "tokens and tokens_out go together");
  if (dtype != KVSEL_F32 && dtype != KVSEL_BF16) return fail(KVSEL_EINVAL, "unknown dtype %d", dtype);
  if (dtype != KVSEL_BF16) return fail(KVSEL_EUNSUPPORTED, "Jacap scores need bf16 keys and outputs");
  if (D != 64 && D != 128) return fail(KVSEL_EUNSUPPORTED, "head dimension %d not supported (64 or 128)", D);
  if ((uintptr_t)K % 16 || (uintptr_t)V % 16 || (uintptr_t)U % 16 || (uintptr_t)K_out % 16 || (uintptr_t)V_out % 16)
    return fail(KVSEL_EINVAL, "K, V, U, K_out and V_out must be 16-byte aligned");
  if (!workspace) return fail(KVSEL_EINVAL, "workspace must not be NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(KVSEL_EINVAL, "workspace must be 256-byte aligned");
  const JacapPlan q = jacap_plan(heads, N, D);
  if (workspace_bytes < q.bytes)
    return fail(KVSEL_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, q.bytes);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  JacapArgs j{};
  j.heads = heads;
  j.N = N;
  j.nch = jacap_chunks(N);
  j.slices = jacap_slices(N, heads);
  j.tau = tau;
  j.mu = mu_q;
  j.lambda = lambda_q;
  j.z = (float*)(ws + q.off_z);
  j.kappa = (float*)(ws + q.off_kappa);
  j.w = (float*)(ws + q.off_w);
  j.r = scores_opt ? scores_opt : (float*)(ws + q.off_r);
  j.part = (float*)(ws + q.off_part);
  j.gpart = (float*)(ws + q.off_gram);
  j.minv = (__bf16*)(ws + q.off_minv);
  j.err = (unsigned*)ws;  // cleared by the first kernel
  record_call(workspace, true, 0ull);
  j.hist = (uint32_t*)(ws + q.off_sel);  // the selection's histograms, cleared by the weights kernel
  j.hist_words = (long long)heads * 2048;
  hipError_t e = launch_jacap_scores(j, D, K, U, st, [&](const char* name, const std::function<hipError_t()>& f) {
    return timed(name, st, f);
  });
  if (e != hipSuccess) return device_error(e, "jacap launch");
  return refresh_core(j.r, heads, N, keep, protect_head, protect_tail, K, V, D, dtype, tokens_opt, indices, K_out,
                      V_out, tokens_out_opt, ws + q.off_sel, st, true);
}

int kvsel_pool1d(const float* votes, int rows, int n, int kernel, int pooling, float* pooled, void* stream) {
  if (!votes || !pooled) return fail(KVSEL_EINVAL, "votes and pooled must not be NULL");
  if (votes == pooled) return fail(KVSEL_EINVAL, "pooled must not alias votes");
  if (rows < 1 || n < 1) return fail(KVSEL_EINVAL, "rows and n must be >= 1 (got %d, %d)", rows, n);
  int rc = check_pool(kernel, pooling);
  if (rc) return rc;
  Launch a{};
  a.n = 1;
  a.heads = rows;
  a.kernel = kernel;
  a.pooling = pooling;
  a.window = 0;
  Seg& s = a.seg[0];
  s.L = n;
  s.C = n;
  s.nh = rows;
  s.vote_ld = n;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed("pool", st, [&] { return launch_pool(a, rows, n, votes, pooled, nullptr, st); });
  if (e != hipSuccess) return device_error(e, "pool launch");
  return ok();
}

int kvsel_gather(const void* K, const void* V, const int32_t* indices, int ld_idx, int heads, int L, int count,
                 int D, int dtype, void* K_out, void* V_out, void* stream) {
  if (!K || !V || !indices || !K_out || !V_out) return fail(KVSEL_EINVAL, "pointers must not be NULL");
  if (heads < 1 || L < 1 || count < 1)
    return fail(KVSEL_EINVAL, "heads, L and count must be >= 1 (got %d, %d, %d)", heads, L, count);
  if (ld_idx < count) return fail(KVSEL_EINVAL, "ld_idx %d is smaller than count %d", ld_idx, count);
  if (dtype != KVSEL_F32 && dtype != KVSEL_BF16) return fail(KVSEL_EINVAL, "unknown dtype %d", dtype);
  if (D != 64 && D != 128) return fail(KVSEL_EUNSUPPORTED, "head dimension %d not supported (64 or 128)", D);
  if ((uintptr_t)K % 16 || (uintptr_t)V % 16 || (uintptr_t)K_out % 16 || (uintptr_t)V_out % 16)
    return fail(KVSEL_EINVAL, "K, V, K_out and V_out must be 16-byte aligned");
  const int rpb = gather_rows_per_block(D, dtype);
  Launch a{};
  a.n = 1;
  a.heads = heads;
  a.D = D;
  a.window = 0;
  Seg& s = a.seg[0];
  s.L = L;
  s.C = count;
  s.nout = count;
  s.nh = heads;
  s.gblk = (count + rpb - 1) / rpb;
  s.idx_ld = ld_idx;
  s.out_ld = count;
  const long long items = (long long)heads * s.gblk;
  if (items > 0x7FFFFFFFLL) return fail(KVSEL_EUNSUPPORTED, "gather grid too large");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed("gather", st, [&] { return launch_gather(a, (int)items, dtype, K, V, indices, K_out, V_out, st); });
  if (e != hipSuccess) return device_error(e, "gather launch");
  return ok();
}

int kvsel_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) drop_profile_events();
  g_prof_on = on != 0;
  return ok();
}

int kvsel_profile_read(kvsel_kernel_time* out, int max_entries) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<kvsel_kernel_time> acc;
  for (auto& t : g_prof) {
    hipError_t e = hipEventSynchronize(t.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) return device_error(e, "profile event");
    auto it = std::find_if(acc.begin(), acc.end(), [&](const kvsel_kernel_time& k) { return strcmp(k.name, t.name) == 0; });
    if (it == acc.end()) {
      kvsel_kernel_time k{};
      snprintf(k.name, sizeof k.name, "%s", t.name);
      acc.push_back(k);
      it = acc.end() - 1;
    }
    it->launches += 1;
    it->total_ms += ms;
  }
  for (int i = 0; i < (int)acc.size() && i < max_entries && out; ++i) out[i] = acc[i];
  ok();
  return (int)acc.size();
}

int kvsel_select_noalloc(const void* Qwin, const void* K, const void* V, int L, int W, int C, int D, int heads,
                         int kernel, int pooling, int dtype, int32_t* indices, void* K_out, void* V_out,
                         float* row_stats_opt, float* votes_opt, float* pooled_opt, void* stream) {
  const int32_t cu[2] = {0, L};
  const int32_t c[1] = {C};
  {
    Plan p;
    const int rc = make_plan(cu, c, 1, heads, W, D, dtype, p);
    if (rc) return rc;
    if (p.bytes > kScratchBytes)
      return fail(KVSEL_EWORKSPACE,
                  "kvsel_select_noalloc: this shape needs %zu bytes of scratch, more than the %zu bytes the "
                  "library holds per device; call kvsel_select with a workspace instead",
                  p.bytes, kScratchBytes);
  }
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  NoEvents guard;
  return kvsel_select(Qwin, K, V, L, W, C, D, heads, kernel, pooling, dtype, indices, K_out, V_out, row_stats_opt,
                      votes_opt, pooled_opt, ws, kScratchBytes, stream);
}

}  // extern "C"
