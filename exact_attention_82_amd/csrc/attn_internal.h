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
};

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
const char* fwd_kernel_name(int dtype, int d, int split_mode);

}  // namespace attn
