// Internal declarations of the Jacap score kernels (kvsel_jacap.hip), used by
// the C entry point in kvsel_api.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <functional>

namespace kvsel {

// Jacap leverage scores (kvsel_jacap.hip): buffers per head of N tokens.
struct JacapArgs {
  int heads, N, nch, slices;
  float tau;
  const float* mu;      // [heads][D]
  const float* lambda;  // [heads][D]
  float* z;             // [heads][N] centre logits
  float* kappa;         // [heads][N]
  float* part;          // [heads][nch][2] softmax partials
  float* w;             // [heads][N]
  float* gpart;         // [heads][slices][D][D] parts of sum w u u^T
  __bf16* minv;         // [heads][2][D][D] L^{-1} as bf16 hi, lo
  float* r;             // [heads][N] leverage scores
  unsigned* err;
  uint32_t* hist;       // [hist_words] selection histograms, cleared by the weights kernel
  long long hist_words;
};
int jacap_chunks(int N);
int jacap_slices(int N, int heads);
hipError_t launch_jacap_scores(const JacapArgs& j, int D, const void* K, const void* U, hipStream_t st,
                               const std::function<hipError_t(const char*, const std::function<hipError_t()>&)>& timed);

}  // namespace kvsel
