// Random argument sweep of every C-ABI entry point (kernels stubbed out), built
// with AddressSanitizer and UndefinedBehaviorSanitizer; device pointers are
// made-up addresses that nothing dereferences. argv[1]: number of calls.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <random>
#include "arrms.h"
#include "arrms_tuning.h"

int main(int argc, char **argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 100000;
  std::mt19937_64 g(12345);
  auto pick = [&](std::initializer_list<long long> v) { return *(v.begin() + g() % v.size()); };
  long calls = 0, ok = 0;
  for (int it = 0; it < n; ++it) {
    const bool sane = it % 2;
    int R = sane ? 1 + (int)(g() % 8) : (int)pick({0, 1, 2, 4, 8, 9, -1});
    int M = sane ? (int)pick({0, 1, 16, 1024, 2800, 65536}) : (int)pick({0, 1, 16, 1024, 2800, -1, 2147483647, 100000000});
    int H = sane ? (int)pick({8, 64, 128, 512, 2880, 6144, 7168, 8192, 16384}) : (int)pick({0, 1, 8, 64, 6144, 7168, 8192, 16384, 16392, -5, 2147483647});
    int flags = sane ? (int)(g() % 2) | (int)(g() % 2) * 4 | (int)(g() % 3) * 16 : (int)(g() % 256);
    float eps = (float)pick({0, 1, -1}) * 1e-6f;
    uintptr_t base = 0x100000000ull + (g() % 64) * 0x10000000ull;
    const void *rin[9];
    for (int r = 0; r < 9; ++r) rin[r] = (const void *)(base + r * 0x1000000000ull + (!sane && g() % 4 == 0 ? 8 : 0));
    void *res = (void *)(base + 20 * 0x1000000000ull);
    void *w = (void *)(base + 21 * 0x1000000000ull);
    void *out = g() % 8 ? (void *)(base + 22 * 0x1000000000ull) : nullptr;
    void *rout = g() % 8 ? (void *)(base + 23 * 0x1000000000ull) : res;
    void *q = g() % 4 ? (void *)(base + 24 * 0x1000000000ull) : nullptr;
    float *sc = g() % 4 ? (float *)(base + 25 * 0x1000000000ull + (sane ? 0 : (g() % 3) * 2)) : nullptr;
    hipStream_t st = nullptr;
    int rc;
    switch (it % 6) {
    case 0: rc = arrms_fused(rin, R, res, w, out, rout, q, sc, M, H, eps, flags, st); break;
    case 1: {
      long long ld[5];
      for (int i = 0; i < 5; ++i)
        ld[i] = pick({(long long)H, (long long)H + 8, (long long)H - 1, 0, -8, 1LL << 40, 1LL << 62,
                      9223372036854775807LL, -9223372036854775807LL - 1});
      rc = arrms_fused_strided(rin, R, res, w, out, rout, q, sc, M, H, ld[0], ld[1], ld[2], ld[3], ld[4], eps,
                               flags, st);
      break;
    }
    case 2: rc = arrms_fused_quant(rin, R, res, w, out, rout, q, sc, M, H, eps, flags, (int)(g() % 6) - 1, st); break;
    case 3: rc = arrms_allreduce_sum(rin, R, out, pick({0, 8, 16, 1LL << 31, 1LL << 62, -1, 9223372036854775807LL}),
                                     flags & 7, st); break;
    case 4: rc = arrms_query_path(M, H, R, flags); break;
    default:
      rc = arrms_fused_config(rin, R, res, w, out, rout, q, sc, M, H, eps, flags, (int)(g() % 7) - 1,
                              (int)pick({0, 64, 100, 192, 512, 1024, 2048, -64}), (int)(g() % 5) - 1,
                              (int)pick({0, 1, 256, 100000, -1}), (int)(g() % 5) - 1, st);
    }
    ++calls;
    if (rc >= 0) ++ok;
    (void)arrms_status_string(rc);
  }
  printf("calls %ld, accepted %ld\n", calls, ok);
  return 0;
}
