// Internal interface between the C ABI layer (api.cpp: argument checks, dispatch) and
// the HIP kernels (attn_kernels.hip: device code and launches).  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace attn {

// Tile geometry shared by the dispatcher and the kernels.
constexpr int kThreads = 256;     // 4 wavefronts of 64 lanes
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;  // query rows owned by one wavefront
constexpr int kBlockM = 128;      // query rows per workgroup
constexpr int kMaxPrefetchKeys = 512;  // keys past the end a sweep may request (ring depth)

// Keys per tile of the key sweep, by element type and head dim.
// Keys per tile of the four-wavefront kernels (one group per workgroup) ...
constexpr int block_n(int dtype, int d) {
  (void)d;
  return dtype == 0 ? 32 : dtype == 1 ? 32 : 64;  // fp32 | bf16 | fp8
}
// (bf16 d = 64 sweeps 32-key tiles with three workgroups per CU when a workgroup sweeps at
// most kShortSweep keys, and 64-key tiles with two beyond: the third workgroup pays for
// the extra barriers of the smaller tiles on short sweeps, not on long ones)
constexpr int kShortSweep = 4096;
constexpr int block_n_for(int dtype, int d, int sweep_keys) {
  return (dtype == 1 && d == 64 && sweep_keys > kShortSweep) ? 64 : block_n(dtype, d);
}
// ... and of the two-group kernels (tile pairs, two groups per tile), whose hand-off
// between the groups needs a 64-key stage at d = 64.
constexpr int block_n_two_groups(int dtype, int d) {
  return dtype == 1 ? (d == 64 ? 64 : 32) : 64;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;       // plain mode
  float* lse;     // plain mode
  float* ws_m;    // split mode: [n][B*H*Sq]
  float* ws_l;    // split mode: [n][B*H*Sq]
  float* ws_u;    // split mode: [n][B*H*Sq][d]
  int B, H, Sq, Sk, d;
  int dtype;      // attn_dtype
  int causal;     // 0 / 1
  int num_splits; // 1 in plain mode
  int chunk;      // keys per split (split mode)
  int split_mode; // 0: O and lse; 1: workspace states
  float scale_log2;  // scale * q_descale * k_descale * log2(e)
  float v_scale;     // v_descale
  int pair_order;    // schedule: 0 causal longest first / plain, 1 complementary causal
                     // tiles per CU, 2 causal tile pairs shared by the two groups of one
                     // workgroup, 3 two groups splitting each tile's keys (small grids)
  int head_group;    // heads whose query tiles are scheduled together (divides B*H)
  // Ragged batch (attn_fwd_varlen): sequence offsets per head block, or null.  Then Sq
  // and Sk hold the largest lengths and q/k/v/o/lse point at [H][total][...] blocks.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  // O written as bf16 (round to nearest even) instead of fp32: `o` then points at
  // uint16 elements (plain modes only; the split workspace stays fp32).
  int o_bf16;
};

// Launch plan of a forward call: query rows per workgroup and the causal schedule.
struct FwdPlan {
  int block_m;
  int pair_order;
  int head_group;
};

// The causal pair kernel (two four-wavefront groups per workgroup sharing a pair of
// query tiles) exists for bf16 with d <= 128: two rings of 64 KiB fit in the LDS.
constexpr bool pairs_supported(int dtype, int d) { return dtype == 1 && d <= 128; }

// The two-group kernel that splits each tile's keys: bf16 with d <= 128 and fp8 with
// d = 128 (the LDS hand-off at the end needs 16 KiB ring stages).
constexpr bool dual_supported(int dtype, int d) {
  return (dtype == 1 && d <= 128) || (dtype == 2 && d == 128);
}
inline int dual_schedule(long long nwg, int dtype, int d, int cus) {
  return (dual_supported(dtype, d) && cus > 0 && nwg <= cus) ? 3 : 0;
}

// head_group: the largest power of two dividing B*H whose query tiles (head_group *
// ceil(Sq / 128) workgroups) fit in one XCD's resident set of 64 workgroups, so that
// those workgroups share the heads' key/value tiles in the XCD's L2 -- and at most an
// eighth of the heads: each XCD takes an eighth of the renumbered grid, so a larger
// group would spread one head's query tiles over several XCDs, each fetching the
// head's keys and values from memory (measured: 3x the algorithmic reads at B=1,
// H=16, Sq=512 with a group of 16).
inline int head_group(long long bh, int nqt) {
  int g = 1;
  while (bh % (2 * g) == 0 && (long long)(2 * g) * nqt <= 64 && 16LL * g <= bh) g *= 2;
  return g;
}

// Causal sweeps differ in length by up to nqt times.  In order of preference:
//   3: (causal or not) two groups per workgroup splitting each tile's keys, when the
//      grid has at most one workgroup per CU (a second wavefront per SIMD; causal: the
//      longest tile's sweep, halved, is shorter than a pair's half, and no group waits
//      at a phase change -- measured 5-25 % ahead of 2 on such grids);
//   2: one workgroup per pair of tiles (t, nqt-1-t) whose two groups split the pair's
//      keys evenly, when one such workgroup per CU covers the grid;
//   1: workgroups i and i + grid/2, which share a CU when the whole grid is resident
//      (at most `per_cu` per CU), get complementary tiles t and nqt-1-t;
//   0: longest sweeps first (causal), or the plain order.
inline FwdPlan plan_fwd(int B, int H, int Sq, int d, int causal, int dtype, int cus) {
  const long long bh = (long long)B * H;
  const long long nqt = (Sq + kBlockM - 1) / kBlockM;
  FwdPlan pl{kBlockM, 0, head_group(bh, (int)nqt)};
  pl.pair_order = dual_schedule(bh * nqt, dtype, d, cus);
  if (pl.pair_order == 0 && causal && cus > 0 && pairs_supported(dtype, d) &&
      bh * ((nqt + 1) / 2) <= cus) {
    pl.pair_order = 2;
    pl.block_m = 2 * kBlockM;
    return pl;
  }
  if (pl.pair_order == 0 && causal && cus > 0) {
    const int per_cu = (d >= 256 || dtype == 0) ? 1 : 2;
    if (bh * nqt <= (long long)cus * per_cu) pl.pair_order = 1;
  }
  return pl;
}

// Split count for attn_fwd_splitkv chosen from the shape.  The split-K section of "AI
// 大模型之 FlashAttention_02" (interface and implementation constraints) notes that a
// split adds a state write-back and a second launch, so short sequences may not gain,
// and that the choice should follow the actual shape rather than the SM count alone.
// Rule: 1 when the unsplit grid already gives every CU a workgroup or the keys are too
// few; else the largest power of two n <= kMaxAutoSplits with B*H*ceil(Sq/128)*n <= CUs
// (one workgroup per CU: the two-group kernel) and chunks of >= kMinSplitKeys keys.
// Measured at B=1, H=8, Sq=128, Sk=32768, d=128 fp8 (8 query tiles): n = 16 / 32 / 64
// take 44.5 / 39.0 / 45.6 us with the merge; the rule picks 32.
constexpr int kMinSplitKeys = 1024;
constexpr int kMaxAutoSplits = 64;
inline int splitkv_count(int B, int H, int Sq, int Sk, int cus) {
  const long long base = (long long)B * H * ((Sq + kBlockM - 1) / kBlockM);
  if (cus <= 0 || base >= cus) return 1;
  int n = 1;
  while (2 * n <= kMaxAutoSplits && base * 2 * n <= cus && (long long)Sk >= 2LL * n * kMinSplitKeys) n *= 2;
  return n;
}

// ---- shape-keyed tuning ("Inside FlashAttention-3", 7.1 Kernel Tuning: time the candidate
// configurations on first use and keep the best; "AI 大模型之 FlashAttention_02", 3.3: the
// best block configuration differs by shape, and the choice must stay reproducible).
//
// A launch plan of attn_fwd is the schedule (pair_order 0-3 above) and, for the schedules
// that use it (0 and 3), the head group; it is exchanged as one integer,
//     plan = schedule + 4 * log2(head_group),  head_group a power of two <= 64.
constexpr int kMaxPlan = 4 * 7;
inline int encode_plan(int sched, int head_group) {
  int lg = 0;
  while ((1 << lg) < head_group) ++lg;
  return sched + 4 * lg;
}
inline int plan_sched(int plan) { return plan & 3; }
inline int plan_head_group(int plan) { return 1 << (plan >> 2); }

// Whether `plan` is a launch plan the kernels implement for this call: the schedule exists
// for (dtype, d, causal) and the head group divides B*H (schedules 1 and 2 ignore it and
// take 1).
inline bool plan_legal(int plan, long long bh, int d, int causal, int dtype) {
  if (plan < 0 || plan >= kMaxPlan) return false;
  const int s = plan_sched(plan), g = plan_head_group(plan);
  if (bh % g != 0) return false;
  switch (s) {
    case 0: return true;
    case 1: return causal == 1 && g == 1;
    case 2: return causal == 1 && g == 1 && pairs_supported(dtype, d);
    case 3: return dual_supported(dtype, d);
  }
  return false;
}

// The plan of the fixed rule (plan_fwd), as a plan id.
inline int default_plan(int B, int H, int Sq, int d, int causal, int dtype, int cus) {
  const FwdPlan pl = plan_fwd(B, H, Sq, d, causal, dtype, cus);
  const bool uses_group = pl.pair_order == 0 || pl.pair_order == 3;
  return encode_plan(pl.pair_order, uses_group ? pl.head_group : 1);
}

// Candidates timed by attn_tune, default first: every legal schedule, with head groups
// 1, 2, 4, ... (dividing B*H, up to 64) for the schedules that use one.  Returns the count.
inline int tune_candidates(int B, int H, int Sq, int d, int causal, int dtype, int cus,
                           int* out, int cap) {
  const long long bh = (long long)B * H;
  int n = 0;
  const int def = default_plan(B, H, Sq, d, causal, dtype, cus);
  if (n < cap) out[n++] = def;
  for (int s = 0; s < 4; ++s)
    for (int lg = 0; lg < 7; ++lg) {
      const int p = s + 4 * lg;
      if (p != def && plan_legal(p, bh, d, causal, dtype) && n < cap) out[n++] = p;
    }
  return n;
}

// The pick from measured median times (same order as the candidates, candidate 0 = the
// default): the fastest, unless it beats the default by less than `margin` (relative), in
// which case the default stays; equal times go to the earlier candidate.  Deterministic for
// given times; the margin keeps run-to-run noise from flipping the choice.
inline int choose_plan(const double* med, int n, double margin) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (med[i] < med[best]) best = i;
  return (best != 0 && med[best] < (1.0 - margin) * med[0]) ? best : 0;
}
constexpr double kTuneMargin = 0.02;

struct MergeArgs {
  const float* ws_m;
  const float* ws_l;
  const float* ws_u;
  float* o;
  float* lse;
  int64_t rows;  // B*H*Sq
  int d;
  int num_splits;
};

struct WorkspaceLayout {
  size_t m_off, l_off, u_off, total;
};

inline WorkspaceLayout workspace_layout(int64_t rows, int d, int n) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WorkspaceLayout w;
  size_t ml = size_t(n) * size_t(rows) * sizeof(float);
  w.m_off = 0;
  w.l_off = up(ml);
  w.u_off = w.l_off + up(ml);
  w.total = w.u_off + size_t(n) * size_t(rows) * size_t(d) * sizeof(float);
  return w;
}

// Backward.  The caller's workspace holds dO rounded to bf16, the per-row term
// D_i = sum_d dO_id O_id and lse in log2 units (+inf for rows with no visible key).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* o;
  const float* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  uint16_t* do16;  // workspace [B*H*Sq][d]
  float* dsum;     // workspace [B*H*Sq]
  float* lse2;     // workspace [B*H*Sq]
  int B, H, Sq, Sk, d;
  int causal;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int long_tiles;    // key tiles 0..long_tiles-1 are swept in two halves (causal, small grids)
  float* pdk;        // workspace [B*H][long_tiles*128][d]: second halves' dK
  float* pdv;        // same for dV
  int long_qtiles;   // the last long_qtiles query tiles' dQ sweeps go in two halves (same)
  float* pdq;        // workspace [B*H][long_qtiles*128][d]: second halves' dQ
};

// Query tiles (of 32 rows) the dK/dV sweep of 128-key tile kt visits: rows from
// kt*128 - (Sk - Sq) on (causal), rounded down to a tile.
constexpr int bwd_query_tiles(int Sq, int Sk, int kt, int causal) {
  int beg = causal ? kt * 128 - (Sk - Sq) : 0;
  beg = beg > 0 ? (beg / 32) * 32 : 0;
  return beg < Sq ? (Sq - beg + 31) / 32 : 0;
}

// Causal key tiles whose sweep covers more than a third of the query tiles (a prefix: the
// sweeps shrink with kt).  When a grid is resident all at once, these are swept in two
// halves by two workgroups so that no workgroup runs much longer than the others.
inline int bwd_long_tiles(int Sq, int Sk, int causal) {
  if (!causal) return 0;
  const int nq = (Sq + 31) / 32, nkt = (Sk + 127) / 128;
  int n = 0;
  while (n < nkt && 3 * bwd_query_tiles(Sq, Sk, n, 1) > nq) ++n;
  return n;
}

// Key tiles (of 32) the dQ sweep of 128-row query tile qt visits: up to the tile's last
// row's diagonal (causal).
constexpr int bwd_key_tiles(int Sq, int Sk, int qt, int causal) {
  int kend = Sk;
  if (causal) {
    const int last = ((qt + 1) * 128 < Sq ? (qt + 1) * 128 : Sq) - 1;
    kend = last + (Sk - Sq) + 1;
    kend = kend < 0 ? 0 : kend > Sk ? Sk : kend;
  }
  return (kend + 31) / 32;
}

// Causal query tiles whose dQ sweep covers more than a third of the longest one (a
// suffix: the sweeps grow with qt), swept in two halves under the same condition as the
// long key tiles.
inline int bwd_long_qtiles(int Sq, int Sk, int causal) {
  if (!causal) return 0;
  const int nqt = (Sq + 127) / 128;
  const int longest = bwd_key_tiles(Sq, Sk, nqt - 1, 1);
  int n = 0;
  while (n < nqt && 3 * bwd_key_tiles(Sq, Sk, nqt - 1 - n, 1) > longest) ++n;
  return n;
}

// Dispatch order of a causal backward launch with split tiles: the 2*nl halves of the nl
// long tiles and the nw other tiles, merged so that longer sweeps start first (the
// hardware hands workgroups to CUs in index order as they free up, so this is the
// longest-first rule of list scheduling).  half_len(i) is the sweep length of either half
// of long tile i, whole_len(j) that of other tile j; both are non-increasing.  Position m
// gets *half = i, *part = 0/1 for a half of long tile i, or *half = -1, *part = j for other
// tile j.  Ties go to the halves.  (A merge-path search: O(log) per call.)
template <class HL, class WL>
constexpr void bwd_item(int m, int nl, int nw, HL half_len, WL whole_len, int* half, int* part) {
  const int na = 2 * nl;
  int lo = m - nw > 0 ? m - nw : 0;
  int hi = m < na ? m : na;
  while (lo < hi) {  // largest a (halves before position m) consistent with the merge
    const int a = (lo + hi + 1) / 2;
    if (m - a >= nw || half_len((a - 1) / 2) >= whole_len(m - a)) lo = a;
    else hi = a - 1;
  }
  const int a = lo, b = m - lo;
  if (a < na && (b >= nw || half_len(a / 2) >= whole_len(b))) {
    *half = a / 2;
    *part = a % 2;
  } else {
    *half = -1;
    *part = b;
  }
}

struct BwdWorkspaceLayout {
  size_t do_off, dsum_off, lse2_off, pdk_off, pdv_off, pdq_off, total;
};

inline BwdWorkspaceLayout bwd_workspace_layout(int64_t bh, int Sq, int Sk, int d, int causal) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows = size_t(bh) * size_t(Sq);
  const int lt = bwd_long_tiles(Sq, Sk, causal);
  const size_t prow = size_t(bh) * size_t(lt) * 128;
  const size_t qrow = size_t(bh) * size_t(bwd_long_qtiles(Sq, Sk, causal)) * 128;
  BwdWorkspaceLayout w;
  w.do_off = 0;
  w.dsum_off = up(rows * size_t(d) * 2);
  w.lse2_off = w.dsum_off + up(rows * sizeof(float));
  w.pdk_off = w.lse2_off + up(rows * sizeof(float));
  w.pdv_off = w.pdk_off + up(prow * size_t(d) * sizeof(float));
  w.pdq_off = w.pdv_off + up(prow * size_t(d) * sizeof(float));
  w.total = w.pdq_off + up(qrow * size_t(d) * sizeof(float));
  return w;
}

// The backward kernels exist for bf16 with d = 64, 128 or 256.
constexpr bool bwd_supported(int dtype, int d) { return dtype == 1 && (d == 64 || d == 128 || d == 256); }

// Launchers (attn_kernels.hip).  Return a hipError_t value as int.
int launch_fwd(const FwdArgs& a, void* stream);
int launch_merge(const MergeArgs& a, void* stream);
int launch_bwd(const BwdArgs& a, void* stream);
const char* bwd_kernel_name(int d, int which);  // which: 0 prologue, 1 dK/dV, 2 dQ, 3 combine
// Compute units of the current device (cached per device), or 0 if unknown.
int device_cu_count();
// Size of the static device array attn_fwd_splitkv_noalloc uses as its workspace, and
// that array's address on the current device (looked up once per device; nullptr with
// *hip_err set if the lookup fails).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;  // ATTN_NOALLOC_SCRATCH_BYTES
void* noalloc_scratch(int* hip_err);
const char* fwd_kernel_name(int dtype, int d, int split_mode, int sched, int sweep_keys);

}  // namespace attn
