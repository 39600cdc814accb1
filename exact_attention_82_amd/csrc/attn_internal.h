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
constexpr int block_n(int dtype, int d) {
  return dtype == 0 ? 32 : dtype == 1 ? (d == 64 ? 64 : 32) : 64;  // fp32 | bf16 | fp8
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
  int pair_order;    // causal query-tile order: 0 longest first, 1 complementary pairs
  int head_group;    // heads whose query tiles are scheduled together (divides B*H)
};

// Launch plan of a forward call: query rows per workgroup and the causal tile order.
struct FwdPlan {
  int block_m;
  int pair_order;
  int head_group;
};

// Causal workgroups have key sweeps of very different lengths.  When the whole grid is
// resident at once (at most `per_cu` workgroups per CU), workgroups i and i + grid/2
// land on the same CU, so pairing query tile t with tile nqt-1-t gives every CU the
// same work; otherwise the longest sweeps go first.
//
// head_group: the largest power of two dividing B*H whose query tiles (head_group *
// ceil(Sq / 128) workgroups) fit in one XCD's resident set of 64 workgroups, so that
// those workgroups share the heads' key/value tiles in the XCD's L2.
inline int head_group(long long bh, int nqt) {
  int g = 1;
  while (bh % (2 * g) == 0 && (long long)(2 * g) * nqt <= 64) g *= 2;
  return g;
}

inline FwdPlan plan_fwd(int B, int H, int Sq, int d, int causal, int dtype, int cus) {
  FwdPlan pl{kBlockM, 0, head_group((long long)B * H, (Sq + kBlockM - 1) / kBlockM)};
  if (causal) {
    const long long nwg = (long long)B * H * ((Sq + kBlockM - 1) / kBlockM);
    const int per_cu = (d >= 256 || dtype == 0) ? 1 : 2;
    pl.pair_order = (cus > 0 && nwg <= (long long)cus * per_cu) ? 1 : 0;
  }
  return pl;
}

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

// Launchers (attn_kernels.hip).  Return a hipError_t value as int.
int launch_fwd(const FwdArgs& a, void* stream);
int launch_merge(const MergeArgs& a, void* stream);
// Compute units of the current device (cached per device), or 0 if unknown.
int device_cu_count();
const char* fwd_kernel_name(int dtype, int d, int split_mode);

}  // namespace attn
