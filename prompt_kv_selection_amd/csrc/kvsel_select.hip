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
// order like the values.  One 1024-thread workgroup per (sequence, head) row
// runs a 3-digit (11/11/10 bit) most-significant-first radix select with LDS
// histograms to find the threshold pattern tau and how many tau-equal
// positions are still needed; a single scan of packed (greater, equal)
// counts over the row in index order then writes the picks in ascending
// order, the lowest tau-equal indices first.

#include "kvsel_internal.h"

namespace kvsel {

// Inclusive scan over the 1024 threads of the block; `total` gets the sum.
__device__ __forceinline__ uint32_t block_scan_1024(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  constexpr int kWavesPerBlock = kTopkThreads / 64;
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

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const Launch a, const float* __restrict__ scores,
                                                            int32_t* __restrict__ indices) {
  const int row = blockIdx.x;
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  const int h = s.h0 + (row - s.row0);
  const int tid = threadIdx.x;
  int32_t* out = indices + s.idx_off + (long long)h * s.idx_ld;
  const int L = s.L;
  if (L < s.C) {  // bypass: keep the whole prompt
    for (int j = tid; j < L; j += kTopkThreads) out[j] = j;
    return;
  }
  const int W = a.window ? a.W : 0;
  const int P = L - W;
  const uint32_t count = (uint32_t)(s.C - W);
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + s.vote_off + (long long)h * s.vote_ld);

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh[32];
  __shared__ uint32_t s_prefix, s_need;
  uint32_t prefix = 0, need = count;

  // Radix select: after the three digits, `prefix` is the full pattern of
  // the count-th largest score and `need` the number of positions equal to
  // it that belong to the selection.
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const int bits = pass == 2 ? 10 : 11;
    const int hi = shift + bits;
    const uint32_t nb = 1u << bits;
    for (int d = tid; d < 2048; d += kTopkThreads) hist[d] = 0u;
    __syncthreads();
    for (int j = tid; j < P; j += kTopkThreads) {
      const uint32_t k = key[j];
      if (pass == 0 || (k >> hi) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1u)], 1u);
    }
    __syncthreads();
    // Thread t owns bins in descending order, so the inclusive scan counts
    // positions at or above each bin.
    const int per = (int)nb / kTopkThreads;
    uint32_t local = 0;
    for (int u = 0; u < per; ++u) local += hist[nb - 1u - (uint32_t)(tid * per + u)];
    uint32_t total;
    const uint32_t incl = block_scan_1024(local, sh, total);
    const uint32_t excl = incl - local;
    if (excl < need && need <= incl) {
      uint32_t cum = excl;
      for (int u = 0; u < per; ++u) {
        const uint32_t d = nb - 1u - (uint32_t)(tid * per + u);
        const uint32_t cnt = hist[d];
        if (cum + cnt >= need) {
          s_prefix = (prefix << bits) | d;
          s_need = need - cum;
          break;
        }
        cum += cnt;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    __syncthreads();
  }

  const uint32_t tau = prefix, need_eq = need;
  uint32_t gt_run = 0, eq_run = 0;
  constexpr int kPer = 8;
  for (int base = 0; base < P; base += kPer * kTopkThreads) {
    const int j0 = base + tid * kPer;
    uint32_t kk[kPer];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = j0 + u;
      kk[u] = j < P ? key[j] : 0u;
      if (j < P) {
        ngt += kk[u] > tau;
        neq += kk[u] == tau;
      }
    }
    const uint32_t packed = (ngt << 16) | neq;
    uint32_t total;
    const uint32_t ex = block_scan_1024(packed, sh, total) - packed;
    uint32_t eq_seen = eq_run + (ex & 0xFFFFu);
    uint32_t pos = gt_run + (ex >> 16) + min(eq_seen, need_eq);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = j0 + u;
      if (j < P) {
        bool take = kk[u] > tau;
        if (kk[u] == tau) {
          take = eq_seen < need_eq;
          ++eq_seen;
        }
        if (take) {
          if (pos < count) out[pos] = j;
          ++pos;
        }
      }
    }
    gt_run += total >> 16;
    eq_run += total & 0xFFFFu;
  }
  if (a.window)
    for (int w = tid; w < a.W; w += kTopkThreads) out[count + w] = P + w;
}

// Avg pooling sums the k neighbours (zero padding included) in ascending
// order, so equal neighbour multisets give bit-equal pooled scores.
template <int KW>
__device__ __forceinline__ float avg_sorted(const float* __restrict__ v, int j, int P) {
  constexpr int r = KW / 2;
  float x[KW];
#pragma unroll
  for (int o = 0; o < KW; ++o) {
    const int p = j - r + o;
    x[o] = (p >= 0 && p < P) ? v[p] : 0.f;
  }
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

__device__ float avg_sorted_any(const float* __restrict__ v, int j, int P, int kw) {
  float x[63];
  const int r = kw / 2;
  for (int o = 0; o < kw; ++o) {
    const int p = j - r + o;
    float val = (p >= 0 && p < P) ? v[p] : 0.f;
    int k = o;
    while (k > 0 && x[k - 1] > val) {
      x[k] = x[k - 1];
      --k;
    }
    x[k] = val;
  }
  float sum = 0.f;
  for (int o = 0; o < kw; ++o) sum += x[o];
  return sum / (float)kw;
}

__global__ __launch_bounds__(kPoolBlock) void pool_kernel(const Launch a, const float* __restrict__ votes,
                                                          float* __restrict__ pooled) {
  const int row = blockIdx.x;
  const Seg& s = a.seg[find_seg<kFieldRow>(a, row)];
  if (s.L < s.C) return;
  const int h = s.h0 + (row - s.row0);
  const int P = s.L - (a.window ? a.W : 0);
  const int j = blockIdx.y * kPoolBlock + threadIdx.x;
  if (j >= P) return;
  const float* v = votes + s.vote_off + (long long)h * s.vote_ld;
  float* o = pooled + s.vote_off + (long long)h * s.vote_ld;
  const int kw = a.kernel, r = kw / 2;
  if (a.pooling == 1) {
    float mx = v[j];
    const int lo = max(0, j - r), hi = min(P - 1, j + r);
    for (int p = lo; p <= hi; ++p) mx = fmaxf(mx, v[p]);
    o[j] = mx;
    return;
  }
  float res;
  switch (kw) {
    case 1: res = v[j]; break;
    case 3: res = avg_sorted<3>(v, j, P); break;
    case 5: res = avg_sorted<5>(v, j, P); break;
    case 7: res = avg_sorted<7>(v, j, P); break;
    case 9: res = avg_sorted<9>(v, j, P); break;
    case 11: res = avg_sorted<11>(v, j, P); break;
    default: res = avg_sorted_any(v, j, P, kw); break;
  }
  o[j] = res;
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
  src = min(max(src, 0), s.L - 1);  // never read outside the head's rows
  const long long in_row = s.kv_off / a.D + (long long)h * s.L + src;
  const long long out_row = s.out_off + (long long)h * s.out_ld + m;
  const uint4 kv = K[in_row * RU + part];
  const uint4 vv = V[in_row * RU + part];
  Ko[out_row * RU + part] = kv;
  Vo[out_row * RU + part] = vv;
}

hipError_t launch_pool(const Launch& a, int rows, int max_n, const float* votes, float* pooled, hipStream_t st) {
  const int yb = (max_n + kPoolBlock - 1) / kPoolBlock;
  if (rows <= 0 || yb <= 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3(rows, yb), dim3(kPoolBlock), 0, st, a, votes, pooled);
  return hipGetLastError();
}

hipError_t launch_topk(const Launch& a, int rows, const float* scores, int32_t* indices, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kTopkThreads), 0, st, a, scores, indices);
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
