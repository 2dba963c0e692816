/*
 * kvsel.h -- observation-window (SnapKV) KV-cache selection on AMD MI355X.
 *
 * C ABI of libkvsel.so.  Every compute step runs in HIP kernels written for
 * gfx950; the host side only validates arguments, partitions the caller's
 * workspace and enqueues kernels on the caller's stream.
 *
 * What is computed (web page "SnapKV: selecting the KV cache for long prompts
 * with an observation window", charlestar.github.io, 2026-10-20):
 *   For one (sequence, head) with prompt length L, window W, budget C (the
 *   budget includes the window), P = L - W prefix positions
 *   [section "the prompt cache shrinks, the positions keep their origin"]:
 *     l[i][j] = Qwin[i] . K[j] / sqrt(D)        window row i = query at P + i
 *     alpha[i][j] = softmax over the visible positions j <= P + i, with the
 *                   denominator over every visible prefix AND window position
 *     s[j] = sum_i alpha[i][j]                  prefix votes, j < P
 *                   [section "votes must come from the causal softmax over the
 *                    full prompt"]
 *     pooled = 1-D pooling of s, stride 1, width k odd, zero padding; avg
 *              always divides by k; max takes the in-range maximum
 *                   [section "pooling spreads a peak into a neighbourhood
 *                    preference"]
 *     indices = the C - W prefix positions with the highest pooled score,
 *               equal scores going to the lowest index, in ascending order,
 *               followed by the window positions P .. L-1
 *     K_out, V_out = the rows of K and V at those indices, bit copies
 *                   [section "one full selection computed from Q and K"]
 *   When L < C the selection is bypassed: indices 0 .. L-1, K_out = K,
 *   V_out = V [sections "one full selection computed from Q and K" and
 *   "prefill still reads the full K/V; the compressed cache serves decode"].
 *   Heads (and layers, and sequences) are independent: each chooses its own
 *   indices [section "the prompt cache shrinks, the positions keep their
 *   origin"].
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers unless the name ends in _host.
 *     Every buffer is owned and allocated by the caller; the library keeps no
 *     device state between calls and allocates nothing.
 *   - Element types: dtype KVSEL_BF16 means Qwin, K, V, K_out, V_out hold
 *     bfloat16; KVSEL_F32 means float32.  Scores are float32, indices int32.
 *   - Layouts are row-major with the head dimension D contiguous.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; the library never synchronises.  Argument
 *     errors are detected on the host before anything is enqueued, and then
 *     no output is touched.  Device faults surface at the caller's next
 *     synchronisation.
 *   - Return value: KVSEL_OK or a negative kvsel_status_code; kvsel_last_error()
 *     returns a thread-local message describing the last failure.
 *   - Supported: D in {64, 128}, 1 <= W <= 128, L < 2^31 / D.  Inputs must be
 *     finite (the page's example rejects non-finite values and dot
 *     products [section "one full selection computed from Q and K"]).  This
 *     is a precondition, checked on the device without a host round trip:
 *     every call flags a non-finite or zero row normaliser (which a
 *     non-finite key or dot product produces), and the validating mode
 *     (KVSEL_OPT_VALIDATE) also scans every Qwin, K and V element; the flags
 *     are read with kvsel_status().
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVSEL_OK = 0,
  KVSEL_EINVAL = -1,       /* argument outside the method's rules or NULL pointer */
  KVSEL_EUNSUPPORTED = -2, /* valid for the method, not covered by these kernels */
  KVSEL_EWORKSPACE = -3,   /* workspace smaller than the *_workspace_bytes value */
  KVSEL_EDEVICE = -4,      /* a HIP call or kernel launch failed (kvsel_status: a device-side wait timed out) */
  KVSEL_ENONFINITE = -5    /* kvsel_status: a non-finite input or row normaliser was seen */
} kvsel_status_code;

enum { KVSEL_POOL_AVG = 0, KVSEL_POOL_MAX = 1 };
enum { KVSEL_F32 = 0, KVSEL_BF16 = 1 };

/* Process-wide options (kvsel_set_option / kvsel_get_option).
 * KVSEL_OPT_SCORING selects how the window scores are computed:
 *   KVSEL_SCORING_AUTO (default): the faster of the two for the shape:
 *     single-read wherever it applies, else two-pass;
 *   KVSEL_SCORING_TWO_PASS: one kernel for the row statistics, a second for
 *     the votes (K is read twice);
 *   KVSEL_SCORING_SINGLE_READ: one cooperative kernel that reads K once;
 *     it covers bf16, D in {64, 128}, W <= 32 and prompts short enough for
 *     one round of the co-resident grid; calls whose shape it does not cover
 *     return KVSEL_EUNSUPPORTED.
 * Both give the same indices and K/V rows up to the documented rounding of
 * the scores.  With the row statistics handed over (kvsel_select_lse and
 * kvsel_select_varlen_lse) there is one pass over K either way:
 * SINGLE_READ takes the persistent one-workgroup-per-CU kernel (same
 * coverage, no co-residency needed), TWO_PASS the votes kernel of the
 * two-pass path (every supported shape), AUTO the former where it applies.  The single-read kernel needs all its workgroups (one per CU)
 * resident at once; it checks that at start, and if the device is shared
 * with other work and they are not, it scores each head inside a single
 * workgroup instead (two passes over that head's K; same results, slower).
 * KVSEL_OPT_FORCE_FALLBACK (testing): 1 makes every single-read launch take
 *   that fallback, and every cooperative selection launch (whose workgroups
 *   also wait for each other) its own: the first workgroup of each row then
 *   runs all of the row's segments; 0 (default) off.
 * KVSEL_OPT_VALIDATE: 1 makes every selection call first scan its Qwin, K
 *   and V (and row_lse) for non-finite values (two extra reads of K and V);
 *   0 (default) off.
 * KVSEL_OPT_FUSED_SELECT: 1 runs the selection (pooling, top-k, window,
 *   K/V copy) inside the single-read scoring kernel, behind the streaming of
 *   later rounds, for calls where the single-read kernel runs, every head has
 *   its own K/V head, the pooling width is at most 7, no prompt is shorter
 *   than its budget and a workgroup owns at most 2048 chunks; such calls
 *   launch one kernel.  0 (default) runs the selection as separate launches,
 *   which is faster on MI355X today: the selection's end phase waits on
 *   device-scope round trips that the separate kernels avoid.  The indices
 *   and K/V rows are identical either way.  The fused kernel needs the same
 *   residency; when its workgroups are not all resident it takes work from
 *   counters instead (statistics and votes per chunk, two passes over K, then
 *   each row's selection in one workgroup).  KVSEL_OPT_FORCE_FALLBACK forces
 *   that too.
 * KVSEL_OPT_SELECT picks the selection kernels (when the selection is not
 *   fused into the scoring kernel):
 *   KVSEL_SELECT_AUTO (default): the cooperative selection where its grid
 *     fits the device at once, else the split selection where it applies
 *     (pooling widths 1, 3, 5, 7 and at most 65535 prefix positions per
 *     prompt), else the per-row or segment-parallel chain;
 *   KVSEL_SELECT_SPLIT: the split selection only; calls it does not cover
 *     return KVSEL_EUNSUPPORTED;
 *   KVSEL_SELECT_EXCHANGE: never the split selection: the cooperative
 *     selection where its grid fits the device, else the per-row or
 *     segment-parallel chain.
 *   The split selection gives each row S workgroups that each find the
 *   row's threshold on their own and write and copy a share of its output;
 *   no workgroup waits for another, so it suits calls with more rows than
 *   the device holds at once.  The indices and K/V rows are identical on
 *   every path.  The option applies to kvsel_topk and kvsel_refresh too
 *   (rows of at most 65535 scores; AUTO takes the split selection there).
 * Not thread-safe with respect to concurrent calls. */
enum {
  KVSEL_OPT_SCORING = 0,
  KVSEL_OPT_FORCE_FALLBACK = 1,
  KVSEL_OPT_VALIDATE = 2,
  KVSEL_OPT_FUSED_SELECT = 3,
  KVSEL_OPT_SELECT = 4
};
enum { KVSEL_SCORING_AUTO = 0, KVSEL_SCORING_TWO_PASS = 1, KVSEL_SCORING_SINGLE_READ = 2 };
enum { KVSEL_SELECT_AUTO = 0, KVSEL_SELECT_SPLIT = 1, KVSEL_SELECT_EXCHANGE = 2 };
int kvsel_set_option(int option, int value);
int kvsel_get_option(int option);

/* Library version, (major << 16) | minor. */
int kvsel_version(void);

/* Thread-local description of the last non-OK return ("" if none). */
const char* kvsel_last_error(void);

/* Debug builds (libkvsel_debug.so, compiled with KVSEL_DEBUG) check every
 * index that becomes a row address: the selection's picks, the gather of
 * caller indices, the refresh's positions.  A violation is clamped or skipped
 * as in release builds (nothing traps) and recorded as KVSEL_FLAG_INDEX_RANGE:
 * in the call's workspace header (kvsel_status returns KVSEL_EDEVICE), or,
 * for entry points without a workspace (kvsel_gather, kvsel_refresh's final
 * positions), in a library-wide word that this call returns (and clears when
 * `reset` is non-zero) after the device is idle.  Release builds return
 * KVSEL_EUNSUPPORTED.  Not for production use: the word is shared by every
 * caller of the library. */
int kvsel_debug_flags(int reset);

/* Device-side outcome of the last selection call (kvsel_select*,
 * kvsel_select*_lse, kvsel_select_gqa, kvsel_jacap_select) that used this
 * workspace: waits for `stream`, then reads
 * the flags the call's kernels left in the workspace header.  Returns
 * KVSEL_OK; KVSEL_ENONFINITE if a non-finite input (validating mode) or a
 * non-finite or zero row normaliser was seen (the outputs follow the
 * arithmetic but carry no meaning); KVSEL_EDEVICE if a bounded wait between
 * workgroups timed out (the outputs of that call are unreliable); or
 * KVSEL_EINVAL for a NULL or misaligned workspace, or for an input outside
 * its domain found on the device (kvsel_jacap_select: a negative or NaN
 * lambda_q entry).  Debug builds also report KVSEL_EDEVICE for an index
 * outside its range (see kvsel_debug_flags).  Each selection call
 * clears the flags at its start.  This is the only entry point that
 * synchronises. */
int kvsel_status(const void* workspace, void* stream);

/* Device-side flags of a workspace, for callers that check a run of calls
 * (a benchmark's timed region) or want to know which way a residency
 * handshake went.  Waits for `stream`, then stores the flags of the last call
 * in *last_flags and the OR of the flags of every call since the last reset
 * in *sticky_flags (either pointer may be NULL); with reset != 0 the sticky
 * word is then cleared.  A freshly allocated workspace holds arbitrary bits
 * there: reset once before the run.  KVSEL_OK, KVSEL_EINVAL (NULL or
 * misaligned workspace) or KVSEL_EDEVICE.  Synchronises; host memory only.
 * Flag bits (KVSEL_FLAG_*): the three waits, the non-finite and domain
 * conditions and the debug builds' index check that kvsel_status reports,
 * and two that are not errors: SCORING_FALLBACK (the single-read scoring
 * found its grid not all resident, as on a device shared with other work,
 * and its workgroups scored (head, chunk-range) items from counters in two
 * passes over K; the statistics are then merged in another grouping, so the
 * votes agree with the resident path up to rounding) and SELECT_FALLBACK
 * (the same for the cooperative selection, which then resolves each row in
 * one workgroup, with identical results). */
#define KVSEL_FLAG_EXCHANGE_WAIT 0x1u
#define KVSEL_FLAG_LDS_WAIT 0x2u
#define KVSEL_FLAG_SELECT_WAIT 0x4u
#define KVSEL_FLAG_NONFINITE 0x8u
#define KVSEL_FLAG_DOMAIN 0x10u
#define KVSEL_FLAG_INDEX_RANGE 0x20u
#define KVSEL_FLAG_SCORING_FALLBACK 0x100u
#define KVSEL_FLAG_SELECT_FALLBACK 0x200u
int kvsel_status_flags(const void* workspace, void* stream, int reset, unsigned* last_flags,
                       unsigned* sticky_flags);

/* Kernel path the library chose for the last selection call made on this
 * thread (host decisions, taken from the shape and the options):
 * KVSEL_PATH_* bits.  Scoring: SINGLE_READ (K streamed once, statistics
 * exchanged between workgroups), TWO_PASS (statistics pass, then votes pass),
 * VOTES_ONLY (handed-over statistics on the two-pass kernels), HANDED_OVER
 * (row_lse given); BYPASS (a prompt shorter than its budget); selection:
 * SELECT_COOP (one cooperative launch: pooling, top-k, picks and the K/V
 * copy), SELECT_ROWS (a workgroup per row, then the gather), SELECT_SEGMENTS
 * (the segment-parallel chain), SELECT_FUSED (the selection inside the
 * single-read scoring kernel), SELECT_SPLIT (one launch, S workgroups per row
 * that each find the threshold and copy a share of the rows).  kvsel_topk and
 * kvsel_refresh record their selection kernels too.  0 before the first
 * call. */
#define KVSEL_PATH_SINGLE_READ 0x1u
#define KVSEL_PATH_TWO_PASS 0x2u
#define KVSEL_PATH_VOTES_ONLY 0x4u
#define KVSEL_PATH_HANDED_OVER 0x8u
#define KVSEL_PATH_BYPASS 0x10u
#define KVSEL_PATH_SELECT_COOP 0x20u
#define KVSEL_PATH_SELECT_ROWS 0x40u
#define KVSEL_PATH_SELECT_SEGMENTS 0x80u
#define KVSEL_PATH_SELECT_FUSED 0x100u
#define KVSEL_PATH_SELECT_SPLIT 0x200u
unsigned kvsel_last_path(void);

/* Workspace bytes kvsel_select needs for these sizes; 0 if the arguments are
 * invalid (kvsel_last_error() says why).  Host-only, enqueues nothing. */
size_t kvsel_workspace_bytes(int heads, int L, int W, int C, int D, int dtype);

/* Full selection for `heads` independent heads of one sequence (a layer's
 * heads, or several layers folded into `heads`: results are identical).
 *   Qwin     [heads][W][D]  queries of prompt positions L-W .. L-1
 *   K, V     [heads][L][D]
 *   L, W, C  prompt length, window, budget (C includes W); rules: W >= 1,
 *            W <= L, C > W
 *   kernel   pooling width, odd, >= 1;  pooling  KVSEL_POOL_AVG | _MAX
 *   indices  out [heads][C] int32; the first min(L, C) entries of each head
 *            are written (ascending prefix picks, then L-W .. L-1)
 *   K_out, V_out  out [heads][C][D]; the first min(L, C) rows are written
 *   row_stats_opt out [heads][W][2] float32 (m_i, Z_i): the maximum logit of
 *            window row i over its visible positions, and
 *            Z_i = sum_j exp(l[i][j] - m_i); or NULL.  Not written for L < C.
 *   votes_opt, pooled_opt  out [heads][L-W] float32 votes / pooled scores, or
 *            NULL.  Not written for L < C.
 *   workspace, workspace_bytes  device scratch of at least
 *            kvsel_workspace_bytes(...) bytes, 256-byte aligned.  Its
 *            contents on entry do not matter: the call clears what it needs
 *            at zero, in its first kernel or, for some calls (a sequence
 *            shorter than its budget, handed-over statistics on the two-pass
 *            path, single-read scoring with a pooling width above 7, the
 *            validating mode), in a fill launch before it.  Calls that share
 *            a workspace must be ordered (one stream).
 */
int kvsel_select(const void* Qwin, const void* K, const void* V,
                 int L, int W, int C, int D, int heads,
                 int kernel, int pooling, int dtype,
                 int32_t* indices, void* K_out, void* V_out,
                 float* row_stats_opt, float* votes_opt, float* pooled_opt,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Selection with the window rows' softmax statistics handed over by the
 * caller.  Prefill attention already forms the full causal softmax of every
 * prompt query over the whole K [section "prefill still reads the full K/V;
 * the compressed cache serves decode"]; the normalisers of its last W query
 * rows are exactly those the votes need [section "votes must come from the
 * causal softmax over the full prompt"], so the row-statistics pass is
 * skipped and K is read once.
 *   row_lse  [heads][W] float32: lse_i = ln sum_{j <= P+i} exp(l[i][j]) of
 *            window row i over its visible prefix and window positions, l as
 *            above (the 1/sqrt(D) scale included).  From kvsel_select's
 *            row_stats_opt: lse_i = m_i + ln Z_i.  Finite, 4-byte aligned.
 * The votes are s[j] = sum_i exp(l[i][j] - lse_i): they follow the given
 * statistics (an error d_i in lse_i scales row i's probabilities by
 * exp(-d_i)).  Every other argument is as for kvsel_select; there is no
 * row-statistics output.  Workspace: kvsel_workspace_bytes(...). */
int kvsel_select_lse(const void* Qwin, const void* K, const void* V, const float* row_lse,
                     int L, int W, int C, int D, int heads,
                     int kernel, int pooling, int dtype,
                     int32_t* indices, void* K_out, void* V_out,
                     float* votes_opt, float* pooled_opt,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Grouped-query attention: q_heads query heads served by kv_heads K/V heads
 * (group G = q_heads / kv_heads).  The model's integration expands K/V to the
 * query heads before compressing each query head on its own [section "under
 * GQA the saving is not just C divided by L"]; this computes exactly that
 * result (query head h reads K/V head h / G, consecutive query heads sharing
 * one, as repeat_kv expands them), but streams each K/V head once for the
 * whole group instead of once per query head.
 *   Qwin    [q_heads][W][D]; K, V [kv_heads][L][D]
 *   indices [q_heads][C]; K_out, V_out [q_heads][C][D] (the expanded cache)
 *   row_lse_opt [q_heads][W] handed-over statistics (as for kvsel_select_lse),
 *           or NULL (then they are computed: two passes over each K/V head);
 *           row_stats_opt must be NULL when row_lse_opt is given
 *   row_stats_opt [q_heads][W][2], votes_opt / pooled_opt [q_heads][L-W] or NULL
 * Rules: q_heads a positive multiple of kv_heads >= 1; with G > 1, W a
 * multiple of 32 and G * W <= 128 (else KVSEL_EUNSUPPORTED).  Every other
 * argument as for kvsel_select.  Workspace: kvsel_gqa_workspace_bytes(...). */
size_t kvsel_gqa_workspace_bytes(int q_heads, int kv_heads, int L, int W, int C, int D, int dtype);
int kvsel_select_gqa(const void* Qwin, const void* K, const void* V, const float* row_lse_opt,
                     int L, int W, int C, int D, int q_heads, int kv_heads,
                     int kernel, int pooling, int dtype,
                     int32_t* indices, void* K_out, void* V_out,
                     float* row_stats_opt, float* votes_opt, float* pooled_opt,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for kvsel_select_varlen; 0 on invalid arguments. */
size_t kvsel_varlen_workspace_bytes(const int32_t* cu_L_host, const int32_t* C_host, int B,
                                    int heads, int W, int D, int dtype);

/* Ragged batch of B sequences, packed without padding.  SnapKV page,
 * section "one full selection computed from Q and K": its example selects
 * for one unpadded sample; a ragged batch is B such samples side by side,
 * each (sequence, head) selected on its own as in kvsel_select (section
 * "the prompt cache shrinks, the positions keep their origin": indices are
 * positions within the sequence).
 *   cu_L_host [B+1]  host array, cu_L[0] = 0, L_b = cu_L[b+1] - cu_L[b]
 *   C_host    [B]    host array, budget of each sequence; cu_C is its
 *                    exclusive prefix sum, cu_P that of P_b = L_b - W
 *   Qwin      [B][heads][W][D]
 *   K, V      sequence b is [heads][L_b][D] at element heads * cu_L[b] * D
 *   indices   sequence b is [heads][C_b] at element heads * cu_C[b]
 *   K_out, V_out  sequence b is [heads][C_b][D] at element heads * cu_C[b] * D
 *   row_stats_opt [B][heads][W][2] or NULL
 *   votes_opt, pooled_opt  sequence b is [heads][P_b] at heads * cu_P[b], or NULL
 * Every sequence must satisfy the rules of kvsel_select.  Outputs of a
 * bypassed sequence (L_b < C_b) follow kvsel_select.
 */
int kvsel_select_varlen(const void* Qwin, const void* K, const void* V,
                        const int32_t* cu_L_host, const int32_t* C_host, int B,
                        int W, int D, int heads, int kernel, int pooling, int dtype,
                        int32_t* indices, void* K_out, void* V_out,
                        float* row_stats_opt, float* votes_opt, float* pooled_opt,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Ragged batch with handed-over statistics (see kvsel_select_lse):
 * row_lse [B][heads][W] float32; every other argument as for
 * kvsel_select_varlen.  Workspace: kvsel_varlen_workspace_bytes(...). */
int kvsel_select_varlen_lse(const void* Qwin, const void* K, const void* V, const float* row_lse,
                            const int32_t* cu_L_host, const int32_t* C_host, int B,
                            int W, int D, int heads, int kernel, int pooling, int dtype,
                            int32_t* indices, void* K_out, void* V_out,
                            float* votes_opt, float* pooled_opt,
                            void* workspace, size_t workspace_bytes, void* stream);

/* kvsel_select_noalloc: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, results and kernels are those of kvsel_select,
 * without the workspace: the call uses a device array of the library,
 * KVSEL_NOALLOC_SCRATCH_BYTES bytes on every GPU it runs on, allocated with
 * the library's code object and held until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree, event or library allocation).
 * The caller still owns every input and output.
 *   Errors: those of kvsel_select, and KVSEL_EWORKSPACE when the shape needs
 *   more scratch than the array holds (kvsel_workspace_bytes() of the shape
 *   must not exceed KVSEL_NOALLOC_SCRATCH_BYTES; 32 heads of L = 32768 at
 *   W = 32, C = 1024, D = 128 fit).
 *   Every call on a GPU shares that GPU's array, which keeps the last call's
 *   contents (each call clears what must start at zero): calls that overlap
 *   on one GPU (other streams, other threads) race and must be serialised by
 *   the caller.  The device-side flags that kvsel_status reads for a
 *   workspace are kept in the array and are not readable through the ABI. */
#define KVSEL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int kvsel_select_noalloc(const void* Qwin, const void* K, const void* V, int L, int W, int C, int D, int heads,
                         int kernel, int pooling, int dtype, int32_t* indices, void* K_out, void* V_out,
                         float* row_stats_opt, float* votes_opt, float* pooled_opt, void* stream);

/* Steps of the selection as separate entry points (same definitions as
 * above), for callers that bring their own scores or indices.
 *
 * kvsel_topk: for each of `rows` score rows of length n (row r at
 *   scores + r * n, float32, every value finite and >= 0; -0 ranks as +0), write the `count`
 *   positions with the highest score, equal scores going to the lowest index,
 *   in ascending order, to out + r * ld_out.  1 <= count <= n.
 *   Workspace: kvsel_topk_workspace_bytes(rows, n) bytes, 256-byte aligned
 *   (0 is returned for invalid sizes).
 *   [section "one full selection computed from Q and K": ranking and tie rule]
 */
size_t kvsel_topk_workspace_bytes(int rows, int n);
int kvsel_topk(const float* scores, int rows, int n, int count, int32_t* out, int ld_out,
               void* workspace, size_t workspace_bytes, void* stream);

/* kvsel_refresh: the selection step of a periodic cache refresh.  For each
 * of `rows` rows (a head's n cached tokens: J kept earlier plus h recent),
 * keep exactly `keep` entries: the first protect_head positions (mandatory
 * prefix, attention sinks), the last protect_tail positions (recent window),
 * and the keep - protect_head - protect_tail highest-scoring positions in
 * between, equal scores going to the lowest index; indices ascending.
 * [web page "Signals from the future: KV cache eviction by counter-causal
 * surprise", section "architecture overview: the inference/refresh loop" and
 * its memory-refresh step: a refresh scores the J + h cached tokens and keeps
 * the top J; web page "Jacap: Preserving Nonlinear Information in KV-Cache
 * Eviction", section "Algorithm 2: a serving-safe integration sketch":
 * protected prefix, sinks and recent window first, the flexible budget filled
 * by score, and its sanity checks: the kept count equals the budget.]  The
 * score is the caller's (the pages' scores need the model).
 *   scores [rows][n] float32, every value finite and >= 0 (-0 ranks as +0)
 *   K, V [rows][n][D] (dtype), tokens_opt [rows][n] int32 or NULL
 *   indices out [rows][keep]; K_out, V_out out [rows][keep][D];
 *   tokens_out_opt out [rows][keep] (given with tokens_opt)
 * Rules: 1 <= keep <= n, protect_head, protect_tail >= 0,
 * protect_head + protect_tail <= keep.  Workspace:
 * kvsel_refresh_workspace_bytes(rows, n) bytes, 256-byte aligned. */
size_t kvsel_refresh_workspace_bytes(int rows, int n);
int kvsel_refresh(const float* scores, int rows, int n, int keep, int protect_head, int protect_tail,
                  const void* K, const void* V, int D, int dtype, const int32_t* tokens_opt,
                  int32_t* indices, void* K_out, void* V_out, int32_t* tokens_out_opt,
                  void* workspace, size_t workspace_bytes, void* stream);

/* kvsel_jacap_select: one Jacap eviction event per head over its N cached
 * tokens [web page "Jacap: Preserving Nonlinear Information in KV-Cache
 * Eviction", sections "Practical approximation", "Algorithm 1: one eviction
 * event" and "Algorithm 2: a serving-safe integration sketch"]:
 *   z_i = k_i . mu_Q / (tau sqrt(D)), alpha = softmax(z) over the N tokens,
 *   w_i = [alpha_i (1 - alpha_i)]^2 (k_i^T Lambda_Q k_i) / D,
 *   A = I + sum_j w_j u_j u_j^T, r_i = w_i u_i^T A^{-1} u_i (Cholesky of A),
 * then the selection of kvsel_refresh on the scores r: protected head and
 * tail, the flexible budget by score, ties to the lowest index, ascending,
 * K, V (and token ids) gathered.  Scores cover all N tokens, protected ones
 * included (the softmax is over the full pool).
 *   K, V, U [heads][N][D] bf16 device arrays: keys, values, and the output
 *           directions u_i (W_O v_i, or V itself as the page's cheaper proxy)
 *   mu_q, lambda_q [heads][D] float32 device arrays: the query mean and the
 *           diagonal second moment (lambda_q >= 0); tau > 0 the temperature
 *   indices out [heads][keep]; K_out, V_out out [heads][keep][D];
 *   tokens_opt / tokens_out_opt [heads][N] / [heads][keep] int32 or both NULL
 *   scores_opt out [heads][N] float32 leverage scores, or NULL
 *   keep, protect_head, protect_tail as for kvsel_refresh (n = N)
 * All pointers are device pointers owned by the caller; nothing is
 * allocated.  KVSEL_EINVAL: a NULL input or output, heads or N < 1, tau not
 * finite and positive, keep outside [1, N], protection that does not fit,
 * tokens without tokens_out, misaligned K, V, U, outputs (16 bytes) or
 * workspace (256 bytes).  KVSEL_EUNSUPPORTED: dtype other than bf16, D not
 * 64 or 128.  KVSEL_EWORKSPACE: workspace smaller than
 * kvsel_jacap_workspace_bytes(heads, N, D).  The two N D^2 contractions run
 * on bf16 MFMA with one operand exact (u) and the other (w u, or L^{-1})
 * split into bf16 high and low parts; logits, weights and the factorisation
 * are fp32.  kvsel_status(workspace) reports a non-finite or non-positive
 * normaliser or pivot (e.g. a non-finite key) as KVSEL_ENONFINITE, and a
 * negative or NaN lambda_q entry as KVSEL_EINVAL. */
size_t kvsel_jacap_workspace_bytes(int heads, int N, int D);
int kvsel_jacap_select(const void* K, const void* V, const void* U, const float* mu_q, const float* lambda_q,
                       float tau, int heads, int N, int D, int dtype, int keep, int protect_head,
                       int protect_tail, const int32_t* tokens_opt, int32_t* indices, void* K_out,
                       void* V_out, int32_t* tokens_out_opt, float* scores_opt, void* workspace,
                       size_t workspace_bytes, void* stream);

/* kvsel_pool1d: pooled[r][j] for `rows` rows of n votes (row-major), width
 * `kernel` odd >= 1, KVSEL_POOL_AVG (zero padding, divide by kernel) or
 * KVSEL_POOL_MAX (in-range maximum).  out may not alias votes.
 * [section "pooling spreads a peak into a neighbourhood preference"] */
int kvsel_pool1d(const float* votes, int rows, int n, int kernel, int pooling,
                 float* pooled, void* stream);

/* kvsel_gather: for each of `heads` heads, K_out[h][m] = K[h][indices[h*ld_idx+m]]
 * and V_out[h][m] likewise, for m < count; K, V are [heads][L][D], K_out,
 * V_out [heads][count][D].  Indices must lie in [0, L); the kernel clamps
 * out-of-range values into that range instead of faulting.
 * [section "one full selection computed from Q and K": K and V gathered with
 * the same indices] */
int kvsel_gather(const void* K, const void* V, const int32_t* indices, int ld_idx,
                 int heads, int L, int count, int D, int dtype,
                 void* K_out, void* V_out, void* stream);

/* Streaming-read probe for benchmarks (not part of the selection): reads
 * `bytes` of device memory at src once and writes a checksum word per wave
 * to sink (device memory of kvsel_probe_sink_bytes() bytes), so that the
 * time of the launch is what HBM (or the last-level cache) delivers to one
 * of the scoring kernels' access patterns.  mode 0: one workgroup per CU of
 * 8 waves, each with one 8 KiB tile of direct-to-LDS loads in flight (the
 * single-read scoring kernel's pattern); mode 1: the same with two tiles per
 * wave; mode 2: 4 waves with four tiles each; mode 3: 16-byte vector loads
 * into registers, grid-stride, four per lane in flight; mode 4: mode 0 with
 * non-temporal loads (the scoring kernels' loads of a K larger than the
 * last-level cache).  Modes 0-2 and 4 read whole 128 KiB blocks (bytes a
 * multiple of 131072).  Asynchronous on `stream`. */
size_t kvsel_probe_sink_bytes(void);
int kvsel_probe_stream(const void* src, size_t bytes, int mode, void* sink, size_t sink_bytes, void* stream);

/* Per-kernel timing for benchmarks (not part of the selection itself).
 * kvsel_profile_enable(1) clears the record and, until kvsel_profile_enable(0),
 * brackets every kernel this library launches with two HIP events recorded on
 * the launch stream.  kvsel_profile_read() waits for the recorded events,
 * fills up to max_entries records (one per kernel name: launches and summed
 * elapsed milliseconds) and returns how many kernel names were seen, or a
 * negative kvsel_status_code.  Host memory only; not for use under graph capture. */
typedef struct {
  char name[32];
  int launches;
  double total_ms;
} kvsel_kernel_time;

int kvsel_profile_enable(int on);
int kvsel_profile_read(kvsel_kernel_time* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
