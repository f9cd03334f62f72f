// Host-only check of the split plan of the LoRA down-projection against the
// workspace bound the sizing uses: for every total rank rt <= rmax, the
// split partials a launch writes (splits * M * rt floats, when it splits)
// never exceed qplan::down_part_floats(M, Kred, rmax).  Prints "ok" or the
// first violation.
#include <stdio.h>

#include "qlora_plan.h"

int main() {
  const int64_t Ms[] = {1, 7, 16, 31, 32, 33, 48, 63, 64, 65, 100, 127, 128, 129, 300, 511, 512, 1000,
                        1024, 2048, 2049, 4096, 8191, 8192, 16384};
  const int64_t Ks[] = {64, 128, 960, 1024, 2048, 4096, 8192, 14336, 28672};
  long checked = 0;
  for (int64_t M : Ms)
    for (int64_t K : Ks)
      for (int rmax = 1; rmax <= 256; ++rmax) {
        const size_t bound = qplan::down_part_floats(M, K, rmax);
        for (int rt = 1; rt <= rmax; ++rt) {
          const int s = qplan::plan_down_splits(M, K, rt);
          const int used = qplan::down_splits_used(K, s);
          const size_t need = used > 1 ? (size_t)used * M * rt : 0;
          ++checked;
          if (need > bound || used > s || s < 1) {
            printf("violation M=%lld K=%lld rmax=%d rt=%d splits=%d used=%d need=%zu bound=%zu\n", (long long)M,
                   (long long)K, rmax, rt, s, used, need, bound);
            return 1;
          }
        }
      }
  printf("ok %ld\n", checked);
  return 0;
}
