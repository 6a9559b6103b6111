/* A plain C99 caller of the library's host-only entry points (no GPU use):
 * the boundary must compile and link from C without any C++ or torch type.
 * Prints one line per result for tests/test_abi_c.py to compare with the
 * Python binding. */
#include <stdint.h>
#include <stdio.h>

#include "mla.h"

int main(void) {
  int s;
  for (s = 0; s <= 5; ++s) printf("status %d %s\n", s, mla_status_string(s));

  {
    const int32_t lens[4] = {100, 0, 1000, 64};
    int32_t fu[4], lu[4];
    int64_t ft[4];
    int b;
    int st = mla_split_plan(4, lens, 7, fu, lu, ft);
    printf("split_plan_status %d\n", st);
    for (b = 0; b < 4; ++b) printf("plan %d %d %d %lld\n", b, fu[b], lu[b], (long long)ft[b]);
    printf("split_plan_zero_splits %d\n", mla_split_plan(4, lens, 0, fu, lu, ft));
  }

  {
    mla_dims_t d;
    int64_t ob = -1, lb = -1;
    d.batch = 64;
    d.q_len = 1;
    d.heads = 128;
    d.d_nope = 128;
    d.d_rope = 64;
    d.d_latent = 512;
    d.d_v = 128;
    d.q_dtype = MLA_BF16;
    d.kv_dtype = MLA_BF16;
    d.flags = 0;
    printf("workspace_status %d\n", mla_workspace_bytes(&d, 256, &ob, &lb));
    printf("workspace %lld %lld\n", (long long)ob, (long long)lb);
    d.heads = 0;
    printf("workspace_bad_dims %d\n", mla_workspace_bytes(&d, 256, &ob, &lb));
  }
  return 0;
}
