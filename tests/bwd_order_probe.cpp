// Prints the dispatch order of the causal backward launches (attn_internal.h, host-only
// code): for each input line "Sq Sk", one line per launch ("kv" dK/dV, "q" dQ) of
// "tile:part:length" items in position order (part -1: a whole sweep).
#include <cstdio>
#include "../exact_attention_82_amd/csrc/attn_internal.h"

int main() {
  int Sq, Sk;
  while (std::scanf("%d %d", &Sq, &Sk) == 2) {
    const int L = attn::bwd_long_tiles(Sq, Sk, 1);
    const int nkt = (Sk + 127) / 128;
    std::printf("kv");
    for (int m = 0; m < nkt + L; ++m) {
      int hi = 0, pj = 0;
      attn::bwd_item(m, L, nkt - L,
                     [&](int i) { return (attn::bwd_query_tiles(Sq, Sk, i, 1) + 1) / 2; },
                     [&](int j) { return attn::bwd_query_tiles(Sq, Sk, L + j, 1); }, &hi, &pj);
      const int kt = hi >= 0 ? hi : L + pj, part = hi >= 0 ? pj : -1;
      const int n = attn::bwd_query_tiles(Sq, Sk, kt, 1);
      std::printf(" %d:%d:%d", kt, part, part < 0 ? n : (n + 1) / 2);
    }
    std::printf("\nq");
    const int LQ = attn::bwd_long_qtiles(Sq, Sk, 1);
    const int nqt = (Sq + 127) / 128;
    for (int m = 0; m < nqt + LQ; ++m) {
      int hi = 0, pj = 0;
      attn::bwd_item(m, LQ, nqt - LQ,
                     [&](int i) { return (attn::bwd_key_tiles(Sq, Sk, nqt - 1 - i, 1) + 1) / 2; },
                     [&](int j) { return attn::bwd_key_tiles(Sq, Sk, nqt - 1 - LQ - j, 1); }, &hi, &pj);
      const int qt = hi >= 0 ? nqt - 1 - hi : nqt - 1 - LQ - pj, part = hi >= 0 ? pj : -1;
      const int n = attn::bwd_key_tiles(Sq, Sk, qt, 1);
      std::printf(" %d:%d:%d", qt, part, part < 0 ? n : (n + 1) / 2);
    }
    std::printf("\n");
  }
  return 0;
}
