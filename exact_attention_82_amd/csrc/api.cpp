// C ABI of the attention library: argument checks, workspace layout and dispatch.
//
// Every check runs before anything is launched, so a refused call has no effect on the
// outputs and makes no HIP call.  The launches live in attn_kernels.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr double kLog2e = 1.4426950408889634073599246810019;
constexpr int64_t kMaxIndex = int64_t(1) << 46;  // element counts addressed with 64-bit offsets

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }
bool supported_dtype(int t) { return t == ATTN_F32 || t == ATTN_BF16 || t == ATTN_FP8_E4M3; }
bool positive_finite(float x) { return std::isfinite(x) && x > 0.0f; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks common to the entry points; num_splits is the split count of a split-KV
// call (1 otherwise), which multiplies the grid.
attn_status check_shape(int B, int H, int Sq, int Sk, int d, int dtype, int num_splits = 1) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SHAPE;
  if (!supported_d(d) || !supported_dtype(dtype)) return ATTN_ERR_UNSUPPORTED;
  const int64_t bh = int64_t(B) * H;
  if (bh * Sq * d >= kMaxIndex || bh * Sk * d >= kMaxIndex) return ATTN_ERR_SHAPE;
  // Workgroup indices are 32-bit: the forward grid (one workgroup per 128 query rows per
  // (batch, head), times the split count) and the backward's (per 128 keys, at most twice
  // that with split key tiles) must stay below 2^31.
  const int64_t tiles = ceil_div(Sq > Sk ? Sq : Sk, attn::kBlockM);
  if (bh * tiles * 2 * num_splits >= (int64_t(1) << 31)) return ATTN_ERR_SHAPE;
  // One (batch, head) slice is addressed with 32-bit byte offsets, including the tile
  // loads the key sweep issues past the end of the sequence (at most a few tiles).
  const int64_t eb = dtype == ATTN_F32 ? 4 : dtype == ATTN_BF16 ? 2 : 1;
  const int64_t longest = (Sq > Sk ? Sq : Sk) + attn::kMaxPrefetchKeys;
  if (longest * d * eb >= (int64_t(1) << 31)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// ---- plans chosen by attn_tune / attn_tune_splitkv, keyed by the full shape and the device
struct PlanKey {
  int dev, cus, dtype, d, causal, B, H, Sq, Sk;
  bool operator<(const PlanKey& o) const {
    return std::tie(dev, cus, dtype, d, causal, B, H, Sq, Sk) <
           std::tie(o.dev, o.cus, o.dtype, o.d, o.causal, o.B, o.H, o.Sq, o.Sk);
  }
};
std::mutex g_plan_mu;
std::map<PlanKey, int> g_plans;         // attn_fwd plan ids
std::map<PlanKey, int> g_split_counts;  // attn_fwd_splitkv chunk counts (causal = -1)
std::atomic<int> g_tuned{0};            // entries in either map (0: no lookup at all)

PlanKey plan_key(int B, int H, int Sq, int Sk, int d, int causal, int dtype) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  return PlanKey{dev, attn::device_cu_count(), dtype, d, causal, B, H, Sq, Sk};
}

attn::FwdPlan plan_of_id(int plan, int B, int H, int Sq) {
  const int s = attn::plan_sched(plan);
  (void)B; (void)H; (void)Sq;
  return attn::FwdPlan{s == 2 ? 2 * attn::kBlockM : attn::kBlockM, s, attn::plan_head_group(plan)};
}

// Plan id attn_fwd uses for this call: the tuned one if attn_tune (or attn_plan_set) stored
// one for this shape on this device, else the fixed rule's.
int plan_id_for(int B, int H, int Sq, int Sk, int d, int causal, int dtype) {
  if (g_tuned.load(std::memory_order_acquire) > 0) {
    const PlanKey key = plan_key(B, H, Sq, Sk, d, causal, dtype);
    std::lock_guard<std::mutex> lock(g_plan_mu);
    auto it = g_plans.find(key);
    if (it != g_plans.end()) return it->second;
  }
  return attn::default_plan(B, H, Sq, d, causal, dtype, attn::device_cu_count());
}

// Kernel plan of attn_fwd; it depends on the device's CU count (a cached HIP query) and on
// a tuned choice for the shape, if any.
attn::FwdPlan plan_for(int B, int H, int Sq, int Sk, int d, int causal, int dtype) {
  const int id = plan_id_for(B, H, Sq, Sk, d, causal, dtype);
  attn::FwdPlan pl = plan_of_id(id, B, H, Sq);
  if (pl.pair_order == 1 || pl.pair_order == 2) pl.head_group = 1;
  return pl;
}

// Schedule of attn_fwd_splitkv: the two-group kernel when the grid has at most one
// workgroup per CU.
int splitkv_schedule(int B, int H, int Sq, int d, int dtype, int num_splits) {
  const long long nwg = (long long)B * H * ((Sq + attn::kBlockM - 1) / attn::kBlockM) * num_splits;
  return attn::dual_schedule(nwg, dtype, d, attn::device_cu_count());
}

// Checks shared by the split-KV entry points (all but the workspace); sl2 receives the
// score factor scale * q_descale * k_descale * log2(e).
attn_status check_splitkv(const void* q, const void* k, const void* v, int num_splits, int B,
                          int H, int Sq, int Sk, int d, float scale, int causal, int dtype,
                          float q_descale, float k_descale, float v_descale, float* sl2) {
  attn_status st = check_shape(B, H, Sq, Sk, d, dtype);
  if (st != ATTN_OK) return st;
  if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_ARG;
  st = check_shape(B, H, Sq, Sk, d, dtype, num_splits);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ATTN_ERR_ALIGN;
  if ((causal != 0 && causal != 1) || !positive_finite(scale) || !positive_finite(q_descale) ||
      !positive_finite(k_descale) || !positive_finite(v_descale))
    return ATTN_ERR_ARG;
  *sl2 = static_cast<float>(double(scale) * double(q_descale) * double(k_descale) * kLog2e);
  if (!positive_finite(*sl2)) return ATTN_ERR_ARG;
  return ATTN_OK;
}

// The dense forward with a given plan.
int launch_dense(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Sq, int Sk, int d, float sl2, int causal, int dtype, bool o_bf16,
                 const attn::FwdPlan& pl, void* stream) {
  attn::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = static_cast<float*>(o); a.lse = lse;
  a.o_bf16 = o_bf16;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.dtype = dtype; a.causal = causal;
  a.num_splits = 1; a.chunk = Sk; a.split_mode = 0;
  a.scale_log2 = sl2;
  a.v_scale = 1.0f;
  a.pair_order = pl.pair_order;
  a.head_group = pl.head_group;
  return attn::launch_fwd(a, stream);
}

// Checks of a dense forward call (attn_fwd, attn_tune); sl2 receives scale * log2(e).
attn_status check_dense(const void* q, const void* k, const void* v, const void* o,
                        const void* lse, int B, int H, int Sq, int Sk, int d, float scale,
                        int causal, int dtype, float* sl2) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  attn_status st = check_shape(B, H, Sq, Sk, d, dtype);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  if ((causal != 0 && causal != 1) || !positive_finite(scale)) return ATTN_ERR_ARG;
  *sl2 = static_cast<float>(double(scale) * kLog2e);
  if (!positive_finite(*sl2)) return ATTN_ERR_ARG;
  return ATTN_OK;
}

// Median duration (ms) of `reps` launches of fn on `stream`, after two untimed ones, from HIP
// events around each launch (synchronises).  Negative on a HIP error (code in *err).
template <typename F>
double time_launches(F&& fn, int reps, void* stream, int* err) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<hipEvent_t> ev(2 * size_t(reps), nullptr);
  double med = -1.0;
  int e = 0;
  for (auto& x : ev)
    if (e == 0) e = int(hipEventCreate(&x));
  for (int i = 0; i < 2 && e == 0; ++i) e = fn();
  for (int r = 0; r < reps && e == 0; ++r) {
    e = int(hipEventRecord(ev[2 * r], s));
    if (e == 0) e = fn();
    if (e == 0) e = int(hipEventRecord(ev[2 * r + 1], s));
  }
  if (e == 0) e = int(hipEventSynchronize(ev[2 * reps - 1]));
  if (e == 0) {
    std::vector<double> t(reps);
    for (int r = 0; r < reps && e == 0; ++r) {
      float ms = 0.0f;
      e = int(hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]));
      t[r] = ms;
    }
    if (e == 0) {
      std::sort(t.begin(), t.end());
      med = t[reps / 2];
    }
  }
  for (auto& x : ev)
    if (x) (void)hipEventDestroy(x);
  *err = e;
  return e == 0 ? med : -1.0;
}

// The split kernel writing chunk states into the workspace at ws (layout w).
int launch_splitkv(const void* q, const void* k, const void* v, void* ws,
                   const attn::WorkspaceLayout& w, int num_splits, int B, int H, int Sq, int Sk,
                   int d, float sl2, int causal, int dtype, float v_descale, void* stream) {
  char* base = static_cast<char*>(ws);
  attn::FwdArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.ws_m = reinterpret_cast<float*>(base + w.m_off);
  a.ws_l = reinterpret_cast<float*>(base + w.l_off);
  a.ws_u = reinterpret_cast<float*>(base + w.u_off);
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.dtype = dtype; a.causal = causal;
  a.num_splits = num_splits;
  a.chunk = static_cast<int>(ceil_div(Sk, num_splits));
  a.split_mode = 1;
  a.scale_log2 = sl2;
  a.v_scale = v_descale;
  a.pair_order = splitkv_schedule(B, H, Sq, d, dtype, num_splits);
  a.head_group = attn::head_group(int64_t(B) * H, int((Sq + attn::kBlockM - 1) / attn::kBlockM));
  return attn::launch_fwd(a, stream);
}

// The merge kernel reading the chunk states at ws (layout w).
int launch_merge_ws(const void* ws, const attn::WorkspaceLayout& w, int num_splits, float* o,
                    float* lse, int64_t rows, int d, void* stream) {
  const char* base = static_cast<const char*>(ws);
  attn::MergeArgs a{};
  a.ws_m = reinterpret_cast<const float*>(base + w.m_off);
  a.ws_l = reinterpret_cast<const float*>(base + w.l_off);
  a.ws_u = reinterpret_cast<const float*>(base + w.u_off);
  a.o = o; a.lse = lse;
  a.rows = rows; a.d = d; a.num_splits = num_splits;
  return attn::launch_merge(a, stream);
}

attn_status launched(int hip_err) {
  if (hip_err != 0) {
    g_last_hip_error = hip_err;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                     int B, int H, int Sq, int Sk, int d, float scale, int causal,
                     attn_dtype dtype, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, dtype, ATTN_F32, stream);
}

attn_status attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Sq, int Sk, int d, float scale, int causal,
                        attn_dtype dtype, attn_dtype out_dtype, void* stream) {
  float sl2 = 0.0f;
  attn_status st = check_dense(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, dtype, &sl2);
  if (st != ATTN_OK) return st;
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;

  const attn::FwdPlan pl = plan_for(B, H, Sq, Sk, d, causal, dtype);
  return launched(launch_dense(q, k, v, o, lse, B, H, Sq, Sk, d, sl2, causal, dtype,
                               out_dtype == ATTN_BF16, pl, stream));
}

attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int B, int H, int max_seqlen_q, int max_seqlen_k,
                            int total_q, int total_k, int d, float scale, int causal,
                            attn_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL;
  if (total_q < 1 || total_k < 1) return ATTN_ERR_SHAPE;
  // the per-sequence limits are those of a dense call with the largest lengths
  attn_status st = check_shape(B, H, max_seqlen_q, max_seqlen_k, d, dtype);
  if (st != ATTN_OK) return st;
  if (int64_t(H) * total_q * d >= kMaxIndex || int64_t(H) * total_k * d >= kMaxIndex)
    return ATTN_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return ATTN_ERR_ALIGN;
  if ((causal != 0 && causal != 1) || !positive_finite(scale)) return ATTN_ERR_ARG;
  const float sl2 = static_cast<float>(double(scale) * kLog2e);
  if (!positive_finite(sl2)) return ATTN_ERR_ARG;

  attn::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Sq = max_seqlen_q; a.Sk = max_seqlen_k; a.d = d;
  a.dtype = dtype; a.causal = causal;
  a.num_splits = 1; a.chunk = max_seqlen_k; a.split_mode = 0;
  a.scale_log2 = sl2;
  a.v_scale = 1.0f;
  a.pair_order = 0;  // plain kernel: one workgroup per (sequence, head, 128-row tile)
  a.head_group = 1;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.total_q = total_q; a.total_k = total_k;
  return launched(attn::launch_fwd(a, stream));
}

int attn_splitkv_num_splits(int B, int H, int Sq, int Sk, int d, attn_dtype dtype) {
  if (check_shape(B, H, Sq, Sk, d, dtype) != ATTN_OK) return 0;
  if (g_tuned.load(std::memory_order_acquire) > 0) {
    const PlanKey key = plan_key(B, H, Sq, Sk, d, -1, dtype);
    std::lock_guard<std::mutex> lock(g_plan_mu);
    auto it = g_split_counts.find(key);
    if (it != g_split_counts.end()) return it->second;
  }
  return attn::splitkv_count(B, H, Sq, Sk, attn::device_cu_count());
}

size_t attn_splitkv_workspace_bytes(int B, int H, int Sq, int d, int num_splits) {
  if (B < 1 || H < 1 || Sq < 1 || !supported_d(d)) return 0;
  if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return 0;
  const int64_t rows = int64_t(B) * H * Sq;
  if (rows * d >= kMaxIndex) return 0;
  return attn::workspace_layout(rows, d, num_splits).total;
}

attn_status attn_fwd_splitkv(const void* q, const void* k, const void* v,
                             void* ws, size_t ws_bytes, int num_splits,
                             int B, int H, int Sq, int Sk, int d, float scale, int causal,
                             attn_dtype dtype, float q_descale, float k_descale,
                             float v_descale, void* stream) {
  if (!q || !k || !v || !ws) return ATTN_ERR_NULL;
  float sl2 = 0.0f;
  attn_status st = check_splitkv(q, k, v, num_splits, B, H, Sq, Sk, d, scale, causal, dtype,
                                 q_descale, k_descale, v_descale, &sl2);
  if (st != ATTN_OK) return st;
  if (!aligned16(ws)) return ATTN_ERR_ALIGN;
  const attn::WorkspaceLayout w = attn::workspace_layout(int64_t(B) * H * Sq, d, num_splits);
  if (ws_bytes < w.total) return ATTN_ERR_WORKSPACE;
  return launched(launch_splitkv(q, k, v, ws, w, num_splits, B, H, Sq, Sk, d, sl2, causal, dtype,
                                 v_descale, stream));
}

attn_status attn_merge(const void* ws, size_t ws_bytes, int num_splits, float* o, float* lse,
                       int B, int H, int Sq, int d, void* stream) {
  if (!ws || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Sq < 1) return ATTN_ERR_SHAPE;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(ws) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_ARG;
  const int64_t rows = int64_t(B) * H * Sq;
  if (rows * d >= kMaxIndex) return ATTN_ERR_SHAPE;
  const attn::WorkspaceLayout w = attn::workspace_layout(rows, d, num_splits);
  if (ws_bytes < w.total) return ATTN_ERR_WORKSPACE;
  return launched(launch_merge_ws(ws, w, num_splits, o, lse, rows, d, stream));
}

attn_status attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, float* o,
                                     float* lse, int num_splits, int B, int H, int Sq, int Sk,
                                     int d, float scale, int causal, attn_dtype dtype,
                                     float q_descale, float k_descale, float v_descale,
                                     void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  float sl2 = 0.0f;
  attn_status st = check_splitkv(q, k, v, num_splits, B, H, Sq, Sk, d, scale, causal, dtype,
                                 q_descale, k_descale, v_descale, &sl2);
  if (st != ATTN_OK) return st;
  if (!aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  const int64_t rows = int64_t(B) * H * Sq;
  const attn::WorkspaceLayout w = attn::workspace_layout(rows, d, num_splits);
  if (w.total > attn::kNoallocScratchBytes) return ATTN_ERR_WORKSPACE;
  // The states of this call go to the GPU's static array: every entry is written by the
  // split kernel before the merge reads it, so nothing needs clearing.
  int err = 0;
  void* ws = attn::noalloc_scratch(&err);
  if (ws == nullptr) return launched(err != 0 ? err : 1);
  st = launched(launch_splitkv(q, k, v, ws, w, num_splits, B, H, Sq, Sk, d, sl2, causal, dtype,
                               v_descale, stream));
  if (st != ATTN_OK) return st;
  return launched(launch_merge_ws(ws, w, num_splits, o, lse, rows, d, stream));
}

size_t attn_bwd_workspace_bytes(int B, int H, int Sq, int Sk, int d, int causal) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || !supported_d(d) || (causal != 0 && causal != 1)) return 0;
  const int64_t bh = int64_t(B) * H;
  if (bh * Sq * d >= kMaxIndex || bh * Sk * d >= kMaxIndex) return 0;
  return attn::bwd_workspace_layout(bh, Sq, Sk, d, causal).total;
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const float* o,
                     const float* dout, const float* lse, float* dq, float* dk, float* dv,
                     void* ws, size_t ws_bytes, int B, int H, int Sq, int Sk, int d,
                     float scale, int causal, attn_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !ws) return ATTN_ERR_NULL;
  attn_status st = check_shape(B, H, Sq, Sk, d, dtype);
  if (st != ATTN_OK) return st;
  if (!attn::bwd_supported(dtype, d)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(ws))
    return ATTN_ERR_ALIGN;
  if ((causal != 0 && causal != 1) || !positive_finite(scale)) return ATTN_ERR_ARG;
  const float sl2 = static_cast<float>(double(scale) * kLog2e);
  if (!positive_finite(sl2)) return ATTN_ERR_ARG;
  const int64_t bh = int64_t(B) * H;
  const attn::BwdWorkspaceLayout w = attn::bwd_workspace_layout(bh, Sq, Sk, d, causal);
  if (ws_bytes < w.total) return ATTN_ERR_WORKSPACE;

  char* base = static_cast<char*>(ws);
  attn::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.do16 = reinterpret_cast<uint16_t*>(base + w.do_off);
  a.dsum = reinterpret_cast<float*>(base + w.dsum_off);
  a.lse2 = reinterpret_cast<float*>(base + w.lse2_off);
  a.pdk = reinterpret_cast<float*>(base + w.pdk_off);
  a.pdv = reinterpret_cast<float*>(base + w.pdv_off);
  a.pdq = reinterpret_cast<float*>(base + w.pdq_off);
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = sl2;
  // Split the long causal key tiles only when the whole dK/dV grid is resident at once
  // (two workgroups per CU); larger grids already balance as workgroups finish.
  const int64_t nkt = (Sk + attn::kBlockM - 1) / attn::kBlockM;
  const int cus = attn::device_cu_count();
  a.long_tiles = (cus > 0 && bh * nkt <= 2 * int64_t(cus)) ? attn::bwd_long_tiles(Sq, Sk, causal) : 0;
  // the same for the dQ grid and its long query tiles
  const int64_t nqt = (Sq + attn::kBlockM - 1) / attn::kBlockM;
  a.long_qtiles = (cus > 0 && bh * nqt <= 2 * int64_t(cus)) ? attn::bwd_long_qtiles(Sq, Sk, causal) : 0;
  return launched(attn::launch_bwd(a, stream));
}

const char* attn_bwd_kernel_name(int d, attn_dtype dtype, int which) {
  if (!attn::bwd_supported(dtype, d) || which < 0 || which > 3) return "unsupported";
  return attn::bwd_kernel_name(d, which);
}

int attn_block_m(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                 int num_splits) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || !supported_d(d) || !supported_dtype(dtype)) return 0;
  if (causal != 0 && causal != 1) return 0;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return 0;
  if (num_splits >= 1) return attn::kBlockM;
  return plan_for(B, H, Sq, Sk, d, causal, dtype).block_m;
}

int attn_block_n(int d, attn_dtype dtype) {
  if (!supported_d(d) || !supported_dtype(dtype)) return 0;
  return attn::block_n(dtype, d);
}

int64_t attn_num_workgroups(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                            int num_splits) {
  const int bm = attn_block_m(B, H, Sq, Sk, d, causal, dtype, num_splits);
  if (bm == 0) return -1;
  return int64_t(B) * H * ceil_div(Sq, bm) * (num_splits >= 1 ? num_splits : 1);
}

const char* attn_kernel_name(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                             int num_splits) {
  if (attn_block_m(B, H, Sq, Sk, d, causal, dtype, num_splits) == 0) return "unsupported";
  if (num_splits >= 1)
    return attn::fwd_kernel_name(dtype, d, 1, splitkv_schedule(B, H, Sq, d, dtype, num_splits),
                                 static_cast<int>(ceil_div(Sk, num_splits)));
  return attn::fwd_kernel_name(dtype, d, 0, plan_for(B, H, Sq, Sk, d, causal, dtype).pair_order, Sk);
}

// ---------------------------------------------------------------- shape-keyed tuning
attn_status attn_tune(const void* q, const void* k, const void* v, float* o, float* lse,
                      int B, int H, int Sq, int Sk, int d, float scale, int causal,
                      attn_dtype dtype, int reps, int* plan, void* stream) {
  float sl2 = 0.0f;
  attn_status st = check_dense(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, dtype, &sl2);
  if (st != ATTN_OK) return st;
  if (reps < 1 || reps > 1000) return ATTN_ERR_ARG;
  const int cus = attn::device_cu_count();
  int cand[attn::kMaxPlan];
  const int n = attn::tune_candidates(B, H, Sq, d, causal, dtype, cus, cand, attn::kMaxPlan);
  std::vector<double> med(n);
  for (int i = 0; i < n; ++i) {
    const attn::FwdPlan pl = plan_of_id(cand[i], B, H, Sq);
    int err = 0;
    med[i] = time_launches([&] { return launch_dense(q, k, v, o, lse, B, H, Sq, Sk, d, sl2, causal,
                                                     dtype, false, pl, stream); },
                           reps, stream, &err);
    if (err != 0) return launched(err);
  }
  const int best = cand[attn::choose_plan(med.data(), n, attn::kTuneMargin)];
  {
    std::lock_guard<std::mutex> lock(g_plan_mu);
    g_plans[plan_key(B, H, Sq, Sk, d, causal, dtype)] = best;
    g_tuned.store(int(g_plans.size() + g_split_counts.size()), std::memory_order_release);
  }
  if (plan) *plan = best;
  // leave the chosen plan's result in o and lse
  st = launched(launch_dense(q, k, v, o, lse, B, H, Sq, Sk, d, sl2, causal, dtype, false,
                             plan_of_id(best, B, H, Sq), stream));
  if (st != ATTN_OK) return st;
  return launched(int(hipStreamSynchronize(static_cast<hipStream_t>(stream))));
}

attn_status attn_tune_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                              int B, int H, int Sq, int Sk, int d, float scale, int causal,
                              attn_dtype dtype, float q_descale, float k_descale,
                              float v_descale, int reps, int* num_splits, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  float sl2 = 0.0f;
  attn_status st = check_splitkv(q, k, v, 1, B, H, Sq, Sk, d, scale, causal, dtype, q_descale,
                                 k_descale, v_descale, &sl2);
  if (st != ATTN_OK) return st;
  if (!aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  if (reps < 1 || reps > 1000) return ATTN_ERR_ARG;
  const int64_t rows = int64_t(B) * H * Sq;
  // candidates: the rule's count first, then 1, 2, 4, ... 64 (chunks of at least one key,
  // states within the static array, grid indices in range)
  const int def = attn::splitkv_count(B, H, Sq, Sk, attn::device_cu_count());
  std::vector<int> cand{def};
  for (int c = 1; c <= attn::kMaxAutoSplits; c *= 2)
    if (c != def && c <= Sk && check_shape(B, H, Sq, Sk, d, dtype, c) == ATTN_OK &&
        attn::workspace_layout(rows, d, c).total <= attn::kNoallocScratchBytes)
      cand.push_back(c);
  if (attn::workspace_layout(rows, d, def).total > attn::kNoallocScratchBytes) return ATTN_ERR_WORKSPACE;
  int err = 0;
  void* ws = attn::noalloc_scratch(&err);
  if (ws == nullptr) return launched(err != 0 ? err : 1);
  std::vector<double> med(cand.size());
  for (size_t i = 0; i < cand.size(); ++i) {
    const int c = cand[i];
    const attn::WorkspaceLayout w = attn::workspace_layout(rows, d, c);
    med[i] = time_launches([&] {
      const int e = launch_splitkv(q, k, v, ws, w, c, B, H, Sq, Sk, d, sl2, causal, dtype,
                                   v_descale, stream);
      return e != 0 ? e : launch_merge_ws(ws, w, c, o, lse, rows, d, stream);
    }, reps, stream, &err);
    if (err != 0) return launched(err);
  }
  const int best = cand[attn::choose_plan(med.data(), int(cand.size()), attn::kTuneMargin)];
  {
    std::lock_guard<std::mutex> lock(g_plan_mu);
    g_split_counts[plan_key(B, H, Sq, Sk, d, -1, dtype)] = best;
    g_tuned.store(int(g_plans.size() + g_split_counts.size()), std::memory_order_release);
  }
  if (num_splits) *num_splits = best;
  const attn::WorkspaceLayout w = attn::workspace_layout(rows, d, best);
  st = launched(launch_splitkv(q, k, v, ws, w, best, B, H, Sq, Sk, d, sl2, causal, dtype, v_descale,
                               stream));
  if (st == ATTN_OK) st = launched(launch_merge_ws(ws, w, best, o, lse, rows, d, stream));
  if (st != ATTN_OK) return st;
  return launched(int(hipStreamSynchronize(static_cast<hipStream_t>(stream))));
}

int attn_plan_get(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype) {
  if (check_shape(B, H, Sq, Sk, d, dtype) != ATTN_OK || (causal != 0 && causal != 1)) return -1;
  return plan_id_for(B, H, Sq, Sk, d, causal, dtype);
}

attn_status attn_plan_set(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                          int plan) {
  attn_status st = check_shape(B, H, Sq, Sk, d, dtype);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!attn::plan_legal(plan, int64_t(B) * H, d, causal, dtype)) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_plan_mu);
  g_plans[plan_key(B, H, Sq, Sk, d, causal, dtype)] = plan;
  g_tuned.store(int(g_plans.size() + g_split_counts.size()), std::memory_order_release);
  return ATTN_OK;
}

void attn_plan_clear(void) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  g_plans.clear();
  g_split_counts.clear();
  g_tuned.store(0, std::memory_order_release);
}

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H, Sq and Sk must be >= 1 and the tensors indexable";
    case ATTN_ERR_ALIGN: return "pointers must be 16-byte aligned";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim (64, 128, 256) or dtype";
    case ATTN_ERR_WORKSPACE: return "split-KV workspace too small";
    case ATTN_ERR_HIP: return "HIP kernel launch failed";
    case ATTN_ERR_ARG: return "causal must be 0/1; scale and descales finite and > 0; "
                              "1 <= num_splits <= ATTN_MAX_SPLITS";
  }
  return "unknown status";
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
