// Host-only tuning logic of attn_internal.h, run on the CPU by tests/test_plan_host.py.
// stdin commands, one per line:
//   cand B H Sq d causal dtype cus      -> the candidate plan ids, default first
//   legal plan bh d causal dtype        -> 1 / 0
//   choose n t0 t1 ... t(n-1)           -> index attn_tune would pick from these medians
#include <cstdio>
#include <cstring>

#include "../exact_attention_82_amd/csrc/attn_internal.h"

int main() {
  char cmd[16];
  while (std::scanf("%15s", cmd) == 1) {
    if (!std::strcmp(cmd, "cand")) {
      int B, H, Sq, d, causal, dtype, cus;
      if (std::scanf("%d %d %d %d %d %d %d", &B, &H, &Sq, &d, &causal, &dtype, &cus) != 7) return 1;
      int out[attn::kMaxPlan];
      const int n = attn::tune_candidates(B, H, Sq, d, causal, dtype, cus, out, attn::kMaxPlan);
      for (int i = 0; i < n; ++i) std::printf("%d%c", out[i], i + 1 < n ? ' ' : '\n');
    } else if (!std::strcmp(cmd, "legal")) {
      long long bh;
      int plan, d, causal, dtype;
      if (std::scanf("%d %lld %d %d %d", &plan, &bh, &d, &causal, &dtype) != 5) return 1;
      std::printf("%d\n", attn::plan_legal(plan, bh, d, causal, dtype) ? 1 : 0);
    } else if (!std::strcmp(cmd, "choose")) {
      int n;
      if (std::scanf("%d", &n) != 1 || n < 1 || n > 64) return 1;
      double t[64];
      for (int i = 0; i < n; ++i)
        if (std::scanf("%lf", &t[i]) != 1) return 1;
      std::printf("%d\n", attn::choose_plan(t, n, attn::kTuneMargin));
    } else {
      return 1;
    }
  }
  return 0;
}
