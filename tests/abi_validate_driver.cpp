// Host-only driver for the argument checks and workspace sizing of the C ABI
// (qlora_validate.cpp), built with AddressSanitizer and UndefinedBehavior-
// Sanitizer by tests/test_abi_cpu.py.  It feeds the checks null, misaligned,
// negative, zero and extreme arguments and prints one line per call; any
// sanitizer report makes the build's binary exit non-zero.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "qlora.h"
#include "qlora_validate.h"

static const uintptr_t kFake = 0x10000;  // aligned, never dereferenced

static qlora_nf4 nf4(int64_t N, int64_t K, int dq) {
  qlora_nf4 w;
  memset(&w, 0, sizeof(w));
  w.codes = (const uint8_t*)kFake;
  w.codebook = (const float*)kFake;
  w.N = N;
  w.K = K;
  w.blocksize = 64;
  w.dq_group = dq;
  if (dq) {
    w.absmax_q = (const uint8_t*)kFake;
    w.absmax_scale = (const float*)kFake;
  } else {
    w.absmax = (const float*)kFake;
  }
  return w;
}

static qlora_linear lin(int64_t N, int64_t K, int r, int dq = 0) {
  qlora_linear L;
  memset(&L, 0, sizeof(L));
  L.W0 = nf4(N, K, dq);
  L.A = (const void*)kFake;
  L.B = (const void*)kFake;
  L.r = r;
  L.alpha = 16.0f;
  return L;
}

int main() {
  const void* P = (const void*)kFake;
  const float* F = (const float*)kFake;
  const int64_t dims[] = {0, 64, 128, 4096, 14336, 28672, 4194240, 4194304, INT64_MAX / 2};
  const int64_t toks[] = {-1, 0, 1, 63, 64, 65, 511, 512, 8192, 2147483647LL, 2147483648LL, INT64_MAX};
  const int ranks[] = {-1, 0, 1, 16, 64, 128, 129};
  long calls = 0;
  for (int64_t N : dims)
    for (int64_t K : dims)
      for (int r : ranks)
        for (int dq : {0, 256, 3}) {
          qlora_linear L = lin(N, K, r, dq);
          for (int64_t M : toks) {
            printf("%d %d %zu %d %d\n", qv_linear_fwd(&L, P, M, P, F, P, SIZE_MAX),
                   qv_linear_bwd(&L, P, P, F, M, P, P, P, P, SIZE_MAX), qlora_linear_workspace_bytes(&L, M),
                   qv_linear_fwd_static(&L, P, M, P, F, (size_t)64 << 20), qv_merge(&L, 0, P));
            qlora_mlp mp;
            mp.gate = lin(N, K, r, dq);
            mp.up = lin(N, K, r, dq);
            mp.down = lin(K, N, r, dq);
            qlora_mlp_saved S = {(void*)kFake, (void*)kFake, (float*)kFake, (float*)kFake, (float*)kFake};
            qlora_mlp_grads G = {(void*)kFake, (void*)kFake, (void*)kFake, (void*)kFake, (void*)kFake,
                                 (void*)kFake};
            printf("%d %d %zu\n", qv_mlp_fwd(&mp, P, M, P, &S, P, SIZE_MAX),
                   qv_mlp_bwd(&mp, P, P, &S, M, P, &G, P, SIZE_MAX), qlora_mlp_workspace_bytes(&mp, M));
            printf("%zu %d\n", qv_linear_ce_ws(M, K, N, 1024, 1),
                   qv_linear_ce(P, M, K, P, N, (const int32_t*)kFake, 1024, F, F, P, P, SIZE_MAX));
            printf("%zu %d\n", qv_rmsnorm_ws(M, K), qv_rmsnorm_bwd(P, P, P, F, M, K, P, F, P, SIZE_MAX));
            calls += 9;
          }
        }
  // null and misaligned pointers
  qlora_linear L = lin(256, 256, 8);
  printf("%d %d %d\n", qv_linear_fwd(nullptr, P, 16, P, F, P, SIZE_MAX),
         qv_linear_fwd(&L, (const void*)(kFake + 2), 16, P, F, P, SIZE_MAX),
         qv_dequantize(nullptr, 0, P));
  printf("%d\n", qv_quantize(nullptr, 64, 64, F, 64, 0, (const uint8_t*)kFake, F, nullptr, nullptr));
  printf("calls %ld\n", calls);
  return 0;
}
