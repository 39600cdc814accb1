// Prints the launch plan of attn_fwd (attn_internal.h, host-only code) for the cases
// given on stdin, one "B H Sq d causal dtype cus" per line, as
// "block_m schedule head_group" lines.  Built and run by tests/test_plan_host.py.
#include <cstdio>

#include "../exact_attention_82_amd/csrc/attn_internal.h"

int main() {
  int B, H, Sq, d, causal, dtype, cus;
  while (std::scanf("%d %d %d %d %d %d %d", &B, &H, &Sq, &d, &causal, &dtype, &cus) == 7) {
    const attn::FwdPlan pl = attn::plan_fwd(B, H, Sq, d, causal, dtype, cus);
    std::printf("%d %d %d\n", pl.block_m, pl.pair_order, pl.head_group);
  }
  return 0;
}
