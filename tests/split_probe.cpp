// Prints the split count attn_splitkv_num_splits picks (attn_internal.h, host-only code)
// for the cases given on stdin, one "B H Sq Sk cus" per line.  Built and run by
// tests/test_plan_host.py.
#include <cstdio>

#include "../exact_attention_82_amd/csrc/attn_internal.h"

int main() {
  int B, H, Sq, Sk, cus;
  while (std::scanf("%d %d %d %d %d", &B, &H, &Sq, &Sk, &cus) == 5)
    std::printf("%d\n", attn::splitkv_count(B, H, Sq, Sk, cus));
  return 0;
}
