// Host-side check of the library's argument validation and workspace
// planning, built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code only (tests/test_abi_host.py builds and runs it on the CPU).
//
// Every call here either fails validation or is given a workspace one byte
// smaller than the planned size, so it returns before any device work: the
// device pointers are placeholders that are never dereferenced, and no kernel
// is launched (also on a machine with a GPU).  Host arrays (cu_L, C) are heap
// blocks of exactly the documented length, so a read past their end is
// reported.  The exit status is the number of unexpected return codes.

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvsel.h"

namespace {

int g_bad = 0;

void expect(bool ok, const char* what, long long a, long long b) {
  if (!ok) {
    std::printf("UNEXPECTED %s (%lld, %lld): %s\n", what, a, b, kvsel_last_error());
    ++g_bad;
  }
}

// Placeholder device addresses, 256-byte aligned, never dereferenced.
void* fake(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x100000 + 0x1000 * i)); }

// Planned size, then a call one byte short: EWORKSPACE, or the validation
// error of the arguments the planner does not see (the pooling).
void plan_and_call(int heads, int L, int W, int C, int D, int dtype, int kernel, int pooling) {
  const size_t need = kvsel_workspace_bytes(heads, L, W, C, D, dtype);
  const int rc = kvsel_select(fake(1), fake(2), fake(3), L, W, C, D, heads, kernel, pooling, dtype,
                              static_cast<int32_t*>(fake(4)), fake(5), fake(6), nullptr, nullptr, nullptr, fake(7),
                              need > 0 ? need - 1 : 0, nullptr);
  const bool pooling_ok = kernel >= 1 && kernel % 2 == 1 && (pooling == KVSEL_POOL_AVG || pooling == KVSEL_POOL_MAX);
  if (need > 0 && pooling_ok)
    expect(rc == KVSEL_EWORKSPACE || rc == KVSEL_EUNSUPPORTED, "select with a short workspace", L, rc);
  else
    expect(rc == KVSEL_EINVAL || rc == KVSEL_EUNSUPPORTED, "select with invalid arguments", L, rc);
}

void varlen_case(const std::vector<int32_t>& lengths, const std::vector<int32_t>& budgets, int heads, int W, int D,
                 bool valid) {
  const int B = static_cast<int>(lengths.size());
  // Exactly B + 1 and B entries on the heap.
  int32_t* cu = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (B + 1)));
  int32_t* cb = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (B > 0 ? B : 1)));
  cu[0] = 0;
  for (int b = 0; b < B; ++b) {
    cu[b + 1] = cu[b] + lengths[b];
    cb[b] = budgets[b];
  }
  const size_t need = kvsel_varlen_workspace_bytes(cu, cb, B, heads, W, D, KVSEL_BF16);
  expect((need > 0) == valid, "varlen planning", B, static_cast<long long>(need));
  const int rc = kvsel_select_varlen(fake(1), fake(2), fake(3), cu, cb, B, W, D, heads, 5, KVSEL_POOL_AVG,
                                     KVSEL_BF16, static_cast<int32_t*>(fake(4)), fake(5), fake(6), nullptr, nullptr,
                                     nullptr, fake(7), need > 0 ? need - 1 : 0, nullptr);
  if (valid)
    expect(rc == KVSEL_EWORKSPACE, "varlen select with a short workspace", B, rc);
  else
    expect(rc == KVSEL_EINVAL || rc == KVSEL_EUNSUPPORTED, "varlen select with invalid batch", B, rc);
  std::free(cu);
  std::free(cb);
}

}  // namespace

int main() {
  expect(kvsel_version() > 0, "version", kvsel_version(), 0);
  (void)kvsel_last_error();

  // Options: valid and invalid values, restored afterwards.
  for (int opt = -1; opt <= 5; ++opt)
    for (int v = -1; v <= 3; ++v) {
      const int before = kvsel_get_option(opt);
      const int rc = kvsel_set_option(opt, v);
      if (rc == 0 && before >= 0) (void)kvsel_set_option(opt, before);
    }

  // Single-sequence planning over a grid of shapes, including the edges of
  // each rule and values near the int range.
  const int heads_v[] = {-1, 0, 1, 3, 32, 64, 1024};
  const int L_v[] = {-5, 0, 1, 31, 32, 33, 1024, 16384, 32768, 131072, 1 << 20, INT_MAX};
  const int W_v[] = {0, 1, 16, 32, 33, 64, 128};
  const int D_v[] = {0, 64, 96, 128, 256};
  for (int heads : heads_v)
    for (int L : L_v)
      for (int W : W_v)
        for (int D : D_v)
          for (int dtype : {(int)KVSEL_F32, (int)KVSEL_BF16, 7}) {
            const int C_v[] = {W, W + 1, L, L > INT_MAX - 5 ? L : L + 5};
            for (int C : C_v) {
              const size_t need = kvsel_workspace_bytes(heads, L, W, C, D, dtype);
              const bool valid_args = heads >= 1 && L >= 1 && W >= 1 && D >= 1 && W <= L && C > W &&
                                      (dtype == KVSEL_F32 || dtype == KVSEL_BF16);
              if (!valid_args) expect(need == 0, "planning accepted invalid arguments", L, W);
              if (static_cast<long long>(heads) * (L > 0 ? L : 0) <= (1ll << 24))
                plan_and_call(heads, L, W, C, D, dtype, 5, KVSEL_POOL_MAX);
            }
          }
  // Pooling arguments.
  for (int kernel : {-1, 0, 1, 2, 3, 63, 65})
    for (int pooling : {-1, (int)KVSEL_POOL_AVG, (int)KVSEL_POOL_MAX, 9})
      plan_and_call(32, 4096, 32, 512, 128, KVSEL_BF16, kernel, pooling);

  // Grouped heads.
  for (int q : {1, 8, 32, 33})
    for (int kv : {-1, 0, 1, 4, 8, 32, 64})
      for (int W : {16, 32, 64, 128}) (void)kvsel_gqa_workspace_bytes(q, kv, 8192, W, 1024, 128, KVSEL_BF16);

  // Ragged batches: up to 80 sequences (several launch groups), bypassed
  // sequences, and invalid ones.
  std::srand(12345);
  for (int t = 0; t < 40; ++t) {
    const int B = 1 + std::rand() % 80;
    std::vector<int32_t> Ls(B), Cs(B);
    for (int b = 0; b < B; ++b) {
      Ls[b] = 33 + std::rand() % 70000;
      Cs[b] = (std::rand() % 4 == 0) ? Ls[b] + 7 : 33 + std::rand() % Ls[b];
    }
    varlen_case(Ls, Cs, 32, 32, 128, true);
  }
  varlen_case({100, 50}, {64, 40}, 8, 32, 128, true);
  varlen_case({100, 20}, {64, 40}, 8, 32, 128, false);    // W > L
  varlen_case({100, 200}, {64, 32}, 8, 32, 128, false);   // C <= W
  varlen_case({}, {}, 8, 32, 128, false);                 // B = 0
  expect(kvsel_varlen_workspace_bytes(nullptr, nullptr, 1, 8, 32, 128, KVSEL_BF16) == 0, "NULL cu_L", 0, 0);
  {
    int32_t* cu = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * 3));
    int32_t* cb = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * 2));
    cu[0] = 0, cu[1] = 100, cu[2] = 50;  // decreasing offsets
    cb[0] = 40, cb[1] = 40;
    expect(kvsel_varlen_workspace_bytes(cu, cb, 2, 8, 32, 128, KVSEL_BF16) == 0, "decreasing cu_L", 0, 0);
    cu[0] = 1;  // cu_L[0] != 0
    expect(kvsel_varlen_workspace_bytes(cu, cb, 2, 8, 32, 128, KVSEL_BF16) == 0, "cu_L[0] != 0", 0, 0);
    std::free(cu);
    std::free(cb);
  }

  // The step entry points' planners.
  for (int rows : {-1, 0, 1, 7, 1024})
    for (int n : {-1, 0, 1, 1000, 131072}) {
      (void)kvsel_topk_workspace_bytes(rows, n);
      (void)kvsel_refresh_workspace_bytes(rows, n);
    }
  for (int heads : {0, 1, 32})
    for (int N : {0, 1, 8192, 131072})
      for (int D : {0, 64, 128, 256}) (void)kvsel_jacap_workspace_bytes(heads, N, D);

  // NULL workspace and arguments.
  expect(kvsel_status(nullptr, nullptr) == KVSEL_EINVAL, "status of NULL", 0, 0);
  unsigned last = 0, sticky = 0;
  expect(kvsel_status_flags(nullptr, nullptr, 0, &last, &sticky) == KVSEL_EINVAL, "flags of NULL", 0, 0);
  expect(kvsel_select(nullptr, fake(2), fake(3), 4096, 32, 512, 128, 32, 5, KVSEL_POOL_MAX, KVSEL_BF16,
                      static_cast<int32_t*>(fake(4)), fake(5), fake(6), nullptr, nullptr, nullptr, fake(7), 1 << 30,
                      nullptr) == KVSEL_EINVAL,
         "NULL Qwin", 0, 0);
  kvsel_kernel_time times[4];
  (void)kvsel_profile_read(times, 4);

  std::printf("plan_check: %d unexpected result(s)\n", g_bad);
  return g_bad;
}
