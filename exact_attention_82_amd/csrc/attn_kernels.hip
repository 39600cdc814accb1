// Exact attention forward kernels for CDNA4 (gfx950).
//
// One workgroup of four 64-lane wavefronts owns a tile of 128 query rows of one
// (batch, head) and sweeps every visible key tile of that head, the sequence-level
// work partition of "AI 大模型之 FlashAttention_02" (section "From head-level to
// sequence-level parallelism"); each wavefront owns 32 of the rows and shares the key
// and value tiles with the other three, so no reduction between wavefronts is ever
// needed (the same page, section "How to reduce communication between warps").
//
// Per key tile a wavefront computes the transposed score block S^T = K Q^T with
// 32x32 MFMAs.  In the 32x32 accumulator layout lane (c, g) -- c = lane % 32,
// g = lane / 32 -- holds column c (one query row) and 16 rows (keys)
// 8*(j/4) + 4*g + j%4, j = 0..15.  So each lane owns half of its query's scores in
// registers: the row maximum and row sum are in-lane, plus one exchange with the
// partner lane c + 32.  The probabilities then feed O^T += V^T P^T directly as the B
// operand of the next MFMA (no trip through LDS), and V^T comes from LDS, where the
// value tile is stored transposed with its keys ordered to match the accumulator
// layout above.
//
// The online softmax is the two-level recurrence of "Inside FlashAttention-3",
// section 2: running maximum m, running sum l, correction exp(m_old - m_new) of what
// was accumulated, with the division by l deferred to the write-back
// ("AI 大模型之 FlashAttention_02", same section as above).  Scores are kept in
// log2 units (scale * log2(e) folded into one multiply) so every exponential is a
// single v_exp_f32.  The correction is applied lazily: the reference maximum moves
// only when a new score exceeds it by more than kTau (log2 units), which bounds the
// unnormalised probabilities by 2^kTau and leaves the exact result unchanged (the
// final division uses the same reference), while skipping most rescales of the
// output accumulator.
//
// Split mode computes, for one chunk of the keys, the unnormalised state (m, l, u) of
// the split-K section of "AI 大模型之 FlashAttention_02" and stores it in a
// workspace; the merge kernel at the end of this file combines the chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// Both lanes c and c+32 receive op(x[c], x[c+32]) via one permlane swap.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return a > b ? a : b;
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------ element traits
// kKPL: contraction elements one lane supplies per MFMA; kKS: contraction depth of one
// MFMA (two lane halves); kTau: lazy-rescale threshold in log2 units.
template <int DT> struct Traits;

template <> struct Traits<DT_BF16> {
  using Op = bf16x8_t;
  static constexpr int kBytes = 2, kKPL = 8, kKS = 16;
  static constexpr bool kVT = true;  // value tile stored transposed in LDS
  static constexpr int kKPad = 16, kVPad = 16;
  static constexpr float kTau = 8.0f;
  static constexpr float kPScale = 1.0f;
  __device__ static f32x16_t mfma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static Op load(const void* p) { return *reinterpret_cast<const Op*>(p); }
  __device__ static Op zero() { return Op{}; }
};

template <> struct Traits<DT_FP8> {
  using Op = long;
  static constexpr int kBytes = 1, kKPL = 8, kKS = 16;
  static constexpr bool kVT = true;
  static constexpr int kKPad = 8, kVPad = 8;
  // FP8 probabilities are scaled by 2^8 before rounding to E4M3 (max 448) so that
  // they sit in the format's normal range; the exact rescale keeps them <= 1 first.
  static constexpr float kTau = 0.0f;
  static constexpr float kPScale = 256.0f;
  __device__ static f32x16_t mfma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
  }
  __device__ static Op load(const void* p) { return *reinterpret_cast<const long*>(p); }
  __device__ static Op zero() { return 0; }
};

template <> struct Traits<DT_F32> {
  using Op = float;
  static constexpr int kBytes = 4, kKPL = 1, kKS = 2;
  static constexpr bool kVT = false;  // value tile kept as [key][d]
  static constexpr int kKPad = 4, kVPad = 16;
  static constexpr float kTau = 8.0f;
  static constexpr float kPScale = 1.0f;
  __device__ static f32x16_t mfma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static Op load(const void* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static Op zero() { return 0.0f; }
};

// ------------------------------------------------------------------ tile geometry
template <int DT, int D, int BN> struct Geo {
  using TR = Traits<DT>;
  static constexpr int EB = TR::kBytes;
  static constexpr int K_STRIDE = D * EB + TR::kKPad;               // bytes per key row
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int V_STRIDE = TR::kVT ? BN * EB + TR::kVPad : D * EB + TR::kVPad;
  static constexpr int V_ROWS = TR::kVT ? D : BN;
  static constexpr int V_BYTES = V_ROWS * V_STRIDE;
  static constexpr int K_OFF_V = (K_BYTES + 15) / 16 * 16;
  static constexpr int BUF = (K_OFF_V + V_BYTES + 15) / 16 * 16;    // one stage
  // K tile: 16-byte chunks, row-major, loaded as they are.
  static constexpr int K_CPR = D * EB / 16;
  static constexpr int K_CHUNKS = BN * K_CPR;
  static constexpr int K_PER_THREAD = (K_CHUNKS + kThreads - 1) / kThreads;
  // V tile, transposed: items of 8 keys x 8 bytes of one key row each.
  static constexpr int VT_W = 8 / EB;                                // d elements per item row
  static constexpr int VT_ITEMS = (BN / 8) * (D / (TR::kVT ? VT_W : 1));
  static constexpr int VT_PER_THREAD = (VT_ITEMS + kThreads - 1) / kThreads;
  // V tile, natural (fp32): like K.
  static constexpr int V_CHUNKS = BN * K_CPR;
  static constexpr int V_PER_THREAD = (V_CHUNKS + kThreads - 1) / kThreads;
};

// Transposed value rows store the keys of each 16-key group in the order
// 0-3, 8-11, 4-7, 12-15.  The MFMA B operand of lane half g holds keys
// {4g..4g+3, 8+4g..8+4g+3} of each 16-key step (the accumulator layout of S^T), so
// this order lets every lane read its 8 keys with one contiguous load.  A staging
// item kq covers positions 8kq..8kq+7, i.e. keys kbase+{0..3, 8..11} with
// kbase = 16*(kq/2) + 4*(kq%2).

template <int DT, int D, int BN>
struct Staging {
  using G = Geo<DT, D, BN>;
  u32x4_t kreg[G::K_PER_THREAD];
  u32x2_t vreg[Traits<DT>::kVT ? G::VT_PER_THREAD * 8 : 1];
  u32x4_t vnat[Traits<DT>::kVT ? 1 : G::V_PER_THREAD];
};

// Issue the global loads of the key/value tile starting at key k0 into registers.
// Keys at or past Sk are zero-filled.
template <int DT, int D, int BN>
__device__ __forceinline__ void load_tile(Staging<DT, D, BN>& st, const uint8_t* Kg,
                                          const uint8_t* Vg, int k0, int Sk, int tid) {
  using G = Geo<DT, D, BN>;
  constexpr int EB = G::EB;
#pragma unroll
  for (int r = 0; r < G::K_PER_THREAD; ++r) {
    const int idx = tid + r * kThreads;
    u32x4_t val = {0u, 0u, 0u, 0u};
    if (idx < G::K_CHUNKS) {
      const int row = idx / G::K_CPR, col = idx % G::K_CPR;
      const int key = k0 + row;
      if (key < Sk) val = *reinterpret_cast<const u32x4_t*>(Kg + (size_t(key) * D * EB) + col * 16);
    }
    st.kreg[r] = val;
  }
  if constexpr (Traits<DT>::kVT) {
#pragma unroll
    for (int r = 0; r < G::VT_PER_THREAD; ++r) {
      const int idx = tid + r * kThreads;
      const int kq = idx % (BN / 8), dcol = idx / (BN / 8);
      const int kbase = (kq >> 1) * 16 + (kq & 1) * 4;  // keys kbase+{0..3, 8..11}
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u32x2_t val = {0u, 0u};
        if (idx < G::VT_ITEMS) {
          const int key = k0 + kbase + (i < 4 ? i : i + 4);
          if (key < Sk) val = *reinterpret_cast<const u32x2_t*>(Vg + size_t(key) * D * EB + dcol * 8);
        }
        st.vreg[r * 8 + i] = val;
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < G::V_PER_THREAD; ++r) {
      const int idx = tid + r * kThreads;
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (idx < G::V_CHUNKS) {
        const int row = idx / G::K_CPR, col = idx % G::K_CPR;
        const int key = k0 + row;
        if (key < Sk) val = *reinterpret_cast<const u32x4_t*>(Vg + size_t(key) * D * EB + col * 16);
      }
      st.vnat[r] = val;
    }
  }
}

// Write 16 bytes to LDS at a byte offset that is a multiple of ALIGN.
template <int ALIGN>
__device__ __forceinline__ void lds_store16(uint8_t* p, u32x4_t v) {
  if constexpr (ALIGN % 16 == 0) {
    *reinterpret_cast<u32x4_t*>(p) = v;
  } else if constexpr (ALIGN % 8 == 0) {
    reinterpret_cast<u32x2_t*>(p)[0] = u32x2_t{v[0], v[1]};
    reinterpret_cast<u32x2_t*>(p)[1] = u32x2_t{v[2], v[3]};
  } else {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    q[0] = v[0]; q[1] = v[1]; q[2] = v[2]; q[3] = v[3];
  }
}

// Move the staged tile from registers into one LDS stage.
template <int DT, int D, int BN>
__device__ __forceinline__ void store_tile(const Staging<DT, D, BN>& st, uint8_t* buf, int tid) {
  using G = Geo<DT, D, BN>;
  uint8_t* kb = buf;
  uint8_t* vb = buf + G::K_OFF_V;
#pragma unroll
  for (int r = 0; r < G::K_PER_THREAD; ++r) {
    const int idx = tid + r * kThreads;
    if (idx < G::K_CHUNKS) {
      const int row = idx / G::K_CPR, col = idx % G::K_CPR;
      lds_store16<(G::K_STRIDE % 16 == 0) ? 16 : (G::K_STRIDE % 8 == 0 ? 8 : 4)>(
          kb + row * G::K_STRIDE + col * 16, st.kreg[r]);
    }
  }
  if constexpr (Traits<DT>::kVT) {
#pragma unroll
    for (int r = 0; r < G::VT_PER_THREAD; ++r) {
      const int idx = tid + r * kThreads;
      if (idx >= G::VT_ITEMS) continue;
      const int kq = idx % (BN / 8), dcol = idx / (BN / 8);
      const u32x2_t* in = &st.vreg[r * 8];
      if constexpr (DT == DT_BF16) {
        // in[i] holds d = 4*dcol + {0,1} (word 0) and {2,3} (word 1) of key i.
        // Output row e (d = 4*dcol + e) is 8 keys x 2 bytes = 4 words.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t o;
          o[0] = __builtin_amdgcn_perm(in[1][w], in[0][w], sel);
          o[1] = __builtin_amdgcn_perm(in[3][w], in[2][w], sel);
          o[2] = __builtin_amdgcn_perm(in[5][w], in[4][w], sel);
          o[3] = __builtin_amdgcn_perm(in[7][w], in[6][w], sel);
          *reinterpret_cast<u32x4_t*>(vb + (dcol * 4 + e) * G::V_STRIDE + kq * 16) = o;
        }
      } else {
        // fp8: in[i] holds d = 8*dcol + 0..3 (word 0) and 4..7 (word 1) of key i.
        // Output row e is 8 keys x 1 byte = 2 words.
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 2, b = e & 3;
          const uint32_t s2 = uint32_t(b) | (uint32_t(b + 4) << 8);  // byte b of lo, byte b of hi
          const uint32_t t01 = __builtin_amdgcn_perm(in[1][w], in[0][w], s2);
          const uint32_t t23 = __builtin_amdgcn_perm(in[3][w], in[2][w], s2);
          const uint32_t t45 = __builtin_amdgcn_perm(in[5][w], in[4][w], s2);
          const uint32_t t67 = __builtin_amdgcn_perm(in[7][w], in[6][w], s2);
          u32x2_t o;
          o[0] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
          o[1] = __builtin_amdgcn_perm(t67, t45, 0x05040100u);
          *reinterpret_cast<u32x2_t*>(vb + (dcol * 8 + e) * G::V_STRIDE + kq * 8) = o;
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < G::V_PER_THREAD; ++r) {
      const int idx = tid + r * kThreads;
      if (idx < G::V_CHUNKS) {
        const int row = idx / G::K_CPR, col = idx % G::K_CPR;
        lds_store16<(G::V_STRIDE % 16 == 0) ? 16 : 4>(vb + row * G::V_STRIDE + col * 16, st.vnat[r]);
      }
    }
  }
}

// Probabilities of one 16-key MFMA step (elements 8h..8h+7 of a score block) as the
// B operand of the value product.
template <int DT>
__device__ __forceinline__ typename Traits<DT>::Op pack_p(const f32x16_t& s, int h);

template <>
__device__ __forceinline__ bf16x8_t pack_p<DT_BF16>(const f32x16_t& s, int h) {
  f32x8_t x = {s[8 * h + 0], s[8 * h + 1], s[8 * h + 2], s[8 * h + 3],
               s[8 * h + 4], s[8 * h + 5], s[8 * h + 6], s[8 * h + 7]};
  return __builtin_convertvector(x, bf16x8_t);
}

template <>
__device__ __forceinline__ long pack_p<DT_FP8>(const f32x16_t& s, int h) {
  const float k = Traits<DT_FP8>::kPScale;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[8 * h + 0] * k, s[8 * h + 1] * k, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[8 * h + 2] * k, s[8 * h + 3] * k, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(s[8 * h + 4] * k, s[8 * h + 5] * k, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(s[8 * h + 6] * k, s[8 * h + 7] * k, hi, true);
  return (long)(((unsigned long)(uint32_t)hi << 32) | (uint32_t)lo);
}

constexpr int waves_per_eu(int dt, int d) { return (d >= 256 || dt == DT_F32) ? 1 : 2; }

// ------------------------------------------------------------------ forward kernel
template <int DT, int D, int BN, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(waves_per_eu(DT, D), waves_per_eu(DT, D))))
void attn_fwd_kernel(FwdArgs p) {
  using TR = Traits<DT>;
  using G = Geo<DT, D, BN>;
  using Op = typename TR::Op;
  constexpr int EB = TR::kBytes;
  constexpr int KSTEPS = D / TR::kKS;  // MFMAs over d per 32-key block of S^T
  constexpr int NKB = BN / 32;         // 32-key blocks per tile
  constexpr int NDB = D / 32;          // 32-row blocks of O^T

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * G::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, g = lane >> 5;

  // ---- which (batch*head, query tile, split) this workgroup owns.  The linear index
  // runs over batch*head fastest, so consecutive workgroups (which the dispatcher
  // spreads over the XCDs round-robin) keep one head's key/value stream per XCD.
  const int BH = p.B * p.H;
  const int nqt = ceil_div_i(p.Sq, kBlockM);
  int x = blockIdx.x;
  const int bh = x % BH;
  x /= BH;
  int qt = x % nqt;
  const int split = x / nqt;
  if (p.causal && !SPLIT) qt = nqt - 1 - qt;  // longest key sweeps first
  const int q0 = qt * kBlockM;
  const int r0 = q0 + wave * kRowsPerWave;    // first query row of this wavefront
  const int row = r0 + c;                     // query row of this lane
  const int off = p.Sk - p.Sq;                // causal: key j visible to row i iff j <= i + off

  int kbeg = 0, kend = p.Sk;
  if (SPLIT) {
    const long long b = (long long)split * p.chunk;
    kbeg = (int)(b < p.Sk ? b : p.Sk);
    const long long e = b + p.chunk;
    kend = (int)(e < p.Sk ? e : p.Sk);
  }
  int kend_wg = kend;
  if (p.causal) {
    const int last_row = min(q0 + kBlockM, p.Sq) - 1;
    kend_wg = min(kend, last_row + off + 1);
  }
  const int ntiles = kend_wg > kbeg ? ceil_div_i(kend_wg - kbeg, BN) : 0;

  const size_t q_base = size_t(bh) * p.Sq * D;
  const size_t kv_base = size_t(bh) * p.Sk * D;
  const uint8_t* Qg = reinterpret_cast<const uint8_t*>(p.q) + q_base * EB;
  const uint8_t* Kg = reinterpret_cast<const uint8_t*>(p.k) + kv_base * EB;
  const uint8_t* Vg = reinterpret_cast<const uint8_t*>(p.v) + kv_base * EB;

  // ---- Q operands for the whole sweep, in registers (B operand of S^T = K Q^T).
  Op qop[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qop[ks] = (row < p.Sq)
                  ? TR::load(Qg + (size_t(row) * D + ks * TR::kKS + g * TR::kKPL) * EB)
                  : TR::zero();
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_inff();  // reference maximum, log2 units (same in lanes c, c+32)
  float l_run = 0.0f;               // this lane's share of the row sum
  const float sl2 = p.scale_log2;

  Staging<DT, D, BN> st;
  if (ntiles > 0) {
    load_tile<DT, D, BN>(st, Kg, Vg, kbeg, p.Sk, tid);
    store_tile<DT, D, BN>(st, smem, tid);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = kbeg + t * BN;
    if (t + 1 < ntiles) load_tile<DT, D, BN>(st, Kg, Vg, k0 + BN, p.Sk, tid);
    const uint8_t* kb = smem + (t & 1) * G::BUF;
    const uint8_t* vb = kb + G::K_OFF_V;

    bool active = r0 < p.Sq;
    if (p.causal) active = active && (k0 <= min(r0 + kRowsPerWave - 1, p.Sq - 1) + off);
    if (active) {
      // ---- S^T = K Q^T for the tile's 32-key blocks
      f32x16_t s[NKB];
#pragma unroll
      for (int b = 0; b < NKB; ++b) {
        s[b] = f32x16_t{};
        const uint8_t* krow = kb + (b * 32 + c) * G::K_STRIDE + g * TR::kKPL * EB;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          s[b] = TR::mfma(TR::load(krow + ks * TR::kKS * EB), qop[ks], s[b]);
      }
      // ---- masks: keys past the chunk / sequence end, and the causal diagonal
      const bool need_mask = (k0 + BN > kend) || (p.causal && (k0 + BN - 1 > r0 + off));
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < NKB; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + b * 32 + (j >> 2) * 8 + g * 4 + (j & 3);
            const bool vis = key < kend && (!p.causal || key <= row + off);
            if (!vis) s[b][j] = -__builtin_inff();
          }
      }
      // ---- online softmax (log2 units)
      float mx = -__builtin_inff();
#pragma unroll
      for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = mx > s[b][j] ? mx : s[b][j];
      mx = pair_max(mx);
      const float mt = mx * sl2;
      if (__builtin_amdgcn_ballot_w64(mt > m_run + TR::kTau)) {
        const float m_new = m_run > mt ? m_run : mt;
        const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
        m_run = m_new;
      }
      const float ms = (m_run == -__builtin_inff()) ? 0.0f : m_run;
      float ls = 0.0f;
#pragma unroll
      for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][j], sl2, -ms));
          s[b][j] = e;
          ls += e;
        }
      l_run += ls;
      // ---- O^T += V^T P^T
#pragma unroll
      for (int b = 0; b < NKB; ++b) {
        if constexpr (TR::kVT) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const Op pb = pack_p<DT>(s[b], h);
            const uint8_t* vrow = vb + c * G::V_STRIDE + (b * 32 + h * 16 + g * 8) * EB;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              oacc[db] = TR::mfma(TR::load(vrow + db * 32 * G::V_STRIDE), pb, oacc[db]);
          }
        } else {
#pragma unroll
          for (int tt = 0; tt < 16; ++tt) {
            const int key = b * 32 + (tt >> 2) * 8 + g * 4 + (tt & 3);
            const uint8_t* vrow = vb + key * G::V_STRIDE + c * EB;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              oacc[db] = TR::mfma(TR::load(vrow + db * 32 * EB), s[b][tt], oacc[db]);
          }
        }
      }
    }
    if (t + 1 < ntiles) store_tile<DT, D, BN>(st, smem + ((t + 1) & 1) * G::BUF, tid);
    __syncthreads();
  }

  // ---- write-back: deferred normalisation
  const float l_tot = pair_sum(l_run);
  if (row >= p.Sq) return;
  const size_t ridx = size_t(bh) * p.Sq + row;
  if constexpr (!SPLIT) {
    const float inv = l_tot > 0.0f ? p.v_scale / (TR::kPScale * l_tot) : 0.0f;
    float* orow = p.o + ridx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4_t v4 = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2],
                      oacc[db][4 * jj + 3]};
        *reinterpret_cast<f32x4_t*>(orow + db * 32 + jj * 8 + g * 4) = v4 * inv;
      }
    if (g == 0)
      p.lse[ridx] = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
  } else {
    const size_t sidx = size_t(split) * size_t(BH) * p.Sq + ridx;
    const float us = p.v_scale / TR::kPScale;
    float* urow = p.ws_u + sidx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4_t v4 = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2],
                      oacc[db][4 * jj + 3]};
        *reinterpret_cast<f32x4_t*>(urow + db * 32 + jj * 8 + g * 4) = v4 * us;
      }
    if (g == 0) {
      p.ws_m[sidx] = l_tot > 0.0f ? m_run * kLn2 : -__builtin_inff();
      p.ws_l[sidx] = l_tot;
    }
  }
}

// ------------------------------------------------------------------ merge kernel
// One group of D/4 lanes per row, each lane owning 4 consecutive columns.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 4;             // threads per row
  constexpr int RPB = 256 / TPR;         // rows per block
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int col = (threadIdx.x % TPR) * 4;
  if (row >= a.rows) return;
  float M = -__builtin_inff();
  for (int s = 0; s < a.num_splits; ++s) {
    const float m = a.ws_m[int64_t(s) * a.rows + row];
    M = M > m ? M : m;
  }
  float L = 0.0f;
  f32x4_t U = {0.f, 0.f, 0.f, 0.f};
  if (M != -__builtin_inff()) {
    for (int s = 0; s < a.num_splits; ++s) {
      const int64_t i = int64_t(s) * a.rows + row;
      const float m = a.ws_m[i];
      if (m == -__builtin_inff()) continue;
      const float w = expf(m - M);
      L += w * a.ws_l[i];
      U += w * *reinterpret_cast<const f32x4_t*>(a.ws_u + i * D + col);
    }
  }
  const bool empty = !(L > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / L;
  *reinterpret_cast<f32x4_t*>(a.o + row * D + col) = U * inv;
  if (col == 0) a.lse[row] = empty ? -__builtin_inff() : M + logf(L);
}

template <int DT, int D>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  constexpr int BN = block_n(DT, D);
  const int64_t nwg = int64_t(a.B) * a.H * ((a.Sq + kBlockM - 1) / kBlockM) * a.num_splits;
  if (a.split_mode)
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, BN, true>), dim3(unsigned(nwg)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, BN, false>), dim3(unsigned(nwg)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_fwd_t<DT, 64>(a, s);
    case 128: return launch_fwd_t<DT, 128>(a, s);
    case 256: return launch_fwd_t<DT, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int launch_fwd(const FwdArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (a.dtype) {
    case DT_F32: return int(launch_fwd_d<DT_F32>(a, s));
    case DT_BF16: return int(launch_fwd_d<DT_BF16>(a, s));
    case DT_FP8: return int(launch_fwd_d<DT_FP8>(a, s));
  }
  return int(hipErrorInvalidValue);
}

int launch_merge(const MergeArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto blocks = [&](int d) { return unsigned((a.rows + (256 / (d / 4)) - 1) / (256 / (d / 4))); };
  switch (a.d) {
    case 64: hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(blocks(64)), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(blocks(128)), dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(attn_merge_kernel<256>, dim3(blocks(256)), dim3(256), 0, s, a); break;
    default: return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

const char* fwd_kernel_name(int dtype, int d, int split_mode) {
  static const char* names[3][3][2] = {
      {{"attn_fwd_f32_d64_bm128_bn32", "attn_fwd_splitkv_f32_d64_bm128_bn32"},
       {"attn_fwd_f32_d128_bm128_bn32", "attn_fwd_splitkv_f32_d128_bm128_bn32"},
       {"attn_fwd_f32_d256_bm128_bn32", "attn_fwd_splitkv_f32_d256_bm128_bn32"}},
      {{"attn_fwd_bf16_d64_bm128_bn64", "attn_fwd_splitkv_bf16_d64_bm128_bn64"},
       {"attn_fwd_bf16_d128_bm128_bn64", "attn_fwd_splitkv_bf16_d128_bm128_bn64"},
       {"attn_fwd_bf16_d256_bm128_bn64", "attn_fwd_splitkv_bf16_d256_bm128_bn64"}},
      {{"attn_fwd_fp8_d64_bm128_bn64", "attn_fwd_splitkv_fp8_d64_bm128_bn64"},
       {"attn_fwd_fp8_d128_bm128_bn64", "attn_fwd_splitkv_fp8_d128_bm128_bn64"},
       {"attn_fwd_fp8_d256_bm128_bn64", "attn_fwd_splitkv_fp8_d256_bm128_bn64"}}};
  const int di = d == 64 ? 0 : d == 128 ? 1 : 2;
  return names[dtype][di][split_mode ? 1 : 0];
}

}  // namespace attn
