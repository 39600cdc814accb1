// Exact attention kernels for CDNA4 (gfx950): forward, split-KV merge, backward.
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
// output accumulator.  The bf16 and fp8 main loops skip even the tile's row maximum:
// they take the probabilities against the reference as it stands and redo the tile
// against its maximum only when the probabilities' sum shows the reference was too
// low for the format (bf16: a lane sum past 2^32; fp8: a probability past E4M3's 448).
//
// Split mode computes, for one chunk of the keys, the unnormalised state (m, l, u) of
// the split-K section of "AI 大模型之 FlashAttention_02" and stores it in a
// workspace; the merge kernel after the forward kernel combines the chunks.  The
// backward kernels (dQ, dK, dV) close the file.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

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
// Op: one lane's operand of the S^T MFMA (and of the value MFMA); POp: the packed
// probabilities of one 16-key step; kKPL: contraction elements one lane supplies per
// MFMA; kKS: contraction depth of one MFMA (two lane halves); kTau: lazy-rescale
// threshold in log2 units; kDMA: tiles reach LDS by direct buffer-to-LDS loads (else
// through registers).
template <int DT> struct Traits;

template <> struct Traits<DT_BF16> {
  using Op = bf16x8_t;
  using POp = bf16x8_t;
  static constexpr int kBytes = 2, kKPL = 8, kKS = 16;
  static constexpr bool kDMA = true;
  static constexpr float kTau = 8.0f;
  static constexpr float kPScale = 1.0f;
  __device__ static f32x16_t mfma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// FP8 uses gfx950's 32x32x64 MFMA (32 bytes per lane, unit E8M0 block scales = 127):
// the 32x32x16 FP8 MFMA inherited from gfx942 runs at the bf16 rate on this chip, the
// 32x32x64 one at twice that (measured 2.0 vs 4.3 PFLOP/s).
template <> struct Traits<DT_FP8> {
  using Op = i32x8_t;
  using POp = long;
  static constexpr int kBytes = 1, kKPL = 32, kKS = 64;
  static constexpr bool kDMA = true;
  // FP8 probabilities are scaled by 2^kPExp before rounding to E4M3 (max 448) so that
  // most of them sit in the format's normal range.  The reference may lag the row
  // maximum by kTau (log2 units), so probabilities reach 2^(kPExp + kTau) and the two
  // must stay below log2(448) = 8.807.  The split is a trade: kPExp = 4, kTau = 4.75
  // keeps probabilities down to 2^-10 normal (2^-13 as subnormals, absolute error at
  // most 2^-14 against row sums >= 1) and rescales the accumulator only when a row
  // maximum moves by more than 4.75, which after the first tile of a chunk is rare;
  // kTau = 0.75 with kPExp = 8 rescaled on most tiles of short chunks.
  static constexpr int kPExp = 4;
  static constexpr float kTau = 4.75f;
  static constexpr float kPScale = float(1 << kPExp);
  static_assert(kPExp + kTau < 8.807f, "scaled probabilities must stay below E4M3's 448");
  __device__ static f32x16_t mfma(Op a, Op b, f32x16_t c) {
    // formats 0 / 0: E4M3 for both operands; scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

template <> struct Traits<DT_F32> {
  using Op = float;
  using POp = float;
  static constexpr int kBytes = 4, kKPL = 1, kKS = 2;
  static constexpr bool kDMA = false;
  static constexpr float kTau = 8.0f;
  static constexpr float kPScale = 1.0f;
  __device__ static f32x16_t mfma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// Raw buffer loads return zero past num_records, so rows at or beyond the sequence
// end read as zeros without any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// Wait until at most N vector memory operations of this wavefront are in flight.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without the release fence of __syncthreads(): the fence would make
// the compiler wait for every direct-to-LDS load still in flight (vmcnt(0)), including
// the ones meant to stay in flight across the barrier.  Callers wait explicitly for
// the loads whose data must be visible; LDS writes from registers are drained here
// (lgkmcnt(0)); the empty asm statements stop the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ================================================================== direct-to-LDS tiles
// A key or value tile (BN rows of D elements) lands in LDS row-major without padding;
// bank conflicts are avoided by XOR-permuting the 16-byte chunks of each row.
//
// Key tile: the S^T MFMA reads one 16-byte (bf16) or 8-byte (fp8) piece per lane,
// 16 consecutive rows at the same column; the key swizzle gives those rows distinct
// banks.  Value tile (bf16): the transposed LDS read (ds_read_b64_tr_b16) has each
// 16-lane group fetch 4 consecutive rows x 32 bytes; the value swizzle puts the 4 rows
// of a group, and the two groups sharing a cycle, on distinct banks.  Value tile
// (fp8): the transposed read (ds_read_b64_tr_b8) has each 32-lane half fetch rows
// {0..3, 8..11} (+4 in the upper half) x two adjacent 16-byte chunks; the value swizzle
// gives the rows that share a bank row (same row mod 256/ROWB) distinct chunk pairs.
template <int ROWB> __device__ __forceinline__ int swz_k(int r) {
  return ROWB >= 256 ? (r & 15) : ROWB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int DT, int ROWB> __device__ __forceinline__ int swz_v(int r) {
  if constexpr (DT == DT_FP8)
    return ROWB >= 256 ? (((r & 3) | ((r >> 1) & 4)) << 1)
         : ROWB == 128 ? ((((r >> 1) & 1) | ((r >> 2) & 2)) << 1)
                       : ((r >> 2) & 3);
  return ROWB >= 256 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int DT, int D, int BN> struct DmaGeo {
  static constexpr int EB = Traits<DT>::kBytes;
  static constexpr int ROWB = D * EB;                  // bytes per row
  static constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;               // bytes per tile (one stage)
};

// Issue the loads of one tile (rows k0..k0+BN-1) straight into an LDS stage.
template <int DT, int D, int BN, bool VALUE, int NW = kWaves>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, uint8_t* stage, int k0,
                                         int wave, int lane) {
  using G = DmaGeo<DT, D, BN>;
  constexpr int NI = G::TILE / 1024 / NW;              // 1 KiB loads per wavefront
  static_assert(NI >= 1 && G::TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads");
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int blk = wave * NI + j;                     // wave-uniform 1 KiB block
    const int L = blk * 64 + lane;                     // chunk index inside the tile
    const int row = L / G::CPR, chp = L % G::CPR;
    const int ch = chp ^ (VALUE ? swz_v<DT, G::ROWB>(row) : swz_k<G::ROWB>(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + blk * 1024), 16,
                                             (k0 + row) * G::ROWB + ch * 16, 0, 0, 0);
  }
}

// A (batch, head) slice of K or V: base address and size in bytes.  Forward tile
// loads address it through a buffer resource rebased to the tile's first row (scalar
// arithmetic only), so the per-lane offsets stay loop-invariant and the range check,
// which returns zeros past the slice, stays exact.
struct Slice {
  const uint8_t* base;
  uint32_t bytes;
};

template <int DT, int D, int BN, bool VALUE, int NW = kWaves>
__device__ __forceinline__ void dma_tile_at(const Slice& sl, uint8_t* stage, int k0, int wave, int lane) {
  using G = DmaGeo<DT, D, BN>;
  constexpr int NI = G::TILE / 1024 / NW;
  static_assert(NI >= 1 && G::TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads");
  const uint32_t off = uint32_t(k0) * G::ROWB;
  // signed max, not a saturating subtract: the latter has no scalar form, and a buffer
  // resource computed in vector registers costs a loop per load (both values < 2^31)
  const int left = __builtin_amdgcn_readfirstlane(max(int(sl.bytes) - int(off), 0));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(sl.base + off, uint32_t(left));
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int blk = wave * NI + j;
    const int L = blk * 64 + lane;
    const int row = L / G::CPR, chp = L % G::CPR;
    const int ch = chp ^ (VALUE ? swz_v<DT, G::ROWB>(row) : swz_k<G::ROWB>(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + blk * 1024), 16,
                                             row * G::ROWB + ch * 16, 0, 0, 0);
  }
}

// Per-lane LDS offsets (relative to a stage) used by the operand reads.
template <int DT, int D, int BN> struct DmaLane {
  using G = DmaGeo<DT, D, BN>;
  int kx;      // key operand: row c, this lane's half g, swizzle folded in
  int kx2;     // fp8: the second 16-byte chunk of the lane's 32-byte key operand
  int vx[2];   // value operand (bf16: two transposed reads; fp8: one)
  __device__ __forceinline__ DmaLane(int lane) {
    const int c = lane & 31, g = lane >> 5;
    if constexpr (DT == DT_BF16) {
      kx = c * G::ROWB + ((g ^ swz_k<G::ROWB>(c)) << 4);
      kx2 = 0;
      const int q = (lane & 15) >> 2, hi = (lane >> 4) & 1, lo2 = (lane & 3) >> 1;
      const int qhi = G::ROWB >= 256 ? q : (q >> 1);
#pragma unroll
      for (int B = 0; B < 2; ++B)
        vx[B] = (g * 4 + 8 * B + q) * G::ROWB + (qhi << 6) +
                ((((hi << 1) | lo2) ^ ((g + 2 * B) & 3)) << 4) + ((lane & 1) << 3);
    } else {
      // 32-byte operands: head-dim bytes 64*ks + 32*g + [0, 32) of key row c, i.e.
      // chunks 4*ks + 2*g and 4*ks + 2*g + 1, each XOR the row's swizzle (the ks term
      // is XORed in by the reader: it stays inside the chunk field, 64*ks < ROWB)
      const int f = swz_k<G::ROWB>(c);
      kx = c * G::ROWB + (((2 * g) ^ f) << 4);
      kx2 = c * G::ROWB + (((2 * g + 1) ^ f) << 4);
      const int s = (lane & 15) >> 1, hi = (lane >> 4) & 1;
      const int keyin = s < 4 ? g * 4 + s : 8 + g * 4 + (s - 4);
      const int fv = swz_v<DT, G::ROWB>(keyin);
      vx[0] = keyin * G::ROWB + ((hi ^ fv) << 4) + ((lane & 1) << 3);
      vx[1] = 0;
    }
  }
};

// S^T = K Q^T for every 32-key block of a tile held in LDS stage kt.
template <int DT, int D, int BN>
__device__ __forceinline__ void qk_dma(f32x16_t (&s)[BN / 32], const uint8_t* kt,
                                       const typename Traits<DT>::Op (&qop)[D / Traits<DT>::kKS],
                                       const DmaLane<DT, D, BN>& ln) {
  using TR = Traits<DT>;
  using G = DmaGeo<DT, D, BN>;
  using Op = typename TR::Op;
  constexpr int KSTEPS = D / TR::kKS;
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) s[b] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
    for (int b = 0; b < BN / 32; ++b) {
      Op a;
      if constexpr (DT == DT_BF16) {
        // logical chunk 2ks+g -- XOR on the chunk field
        a = *reinterpret_cast<const Op*>(kt + (ln.kx ^ (ks << 5)) + b * 32 * G::ROWB);
      } else {
        // two 16-byte chunks (4ks+2g, 4ks+2g+1): the same head-dim bytes the Q operand
        // of this lane half holds, in the same order
        const uint8_t* base = kt + b * 32 * G::ROWB;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + (ln.kx ^ (ks << 6)));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + (ln.kx2 ^ (ks << 6)));
        a = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      s[b] = TR::mfma(a, qop[ks], s[b]);
    }
  }
}

// O^T += V^T P^T for a tile held in LDS stage vt.  Lane (c, g) needs, for output rows
// d = 32*db + c, the 8 keys {4g..4g+3, 8+4g..8+4g+3} of every 16-key step; the
// transposed reads deliver exactly those from the row-major value tile.
template <int DT, int BN> struct PTile;
template <int DT, int D, int BN>
__device__ __forceinline__ void pv_dma(f32x16_t (&oacc)[D / 32], const PTile<DT, BN>& pt,
                                       const uint8_t* vt, const DmaLane<DT, D, BN>& ln) {
  using TR = Traits<DT>;
  using G = DmaGeo<DT, D, BN>;
  using Op = typename TR::Op;
  constexpr int NDB = D / 32;
  if constexpr (DT == DT_FP8) {
    // One 32x32x64 MFMA per output block: the lane's 32 contraction bytes are the four
    // 16-key steps (b, h) of the tile in the order (0,0) (0,1) (1,0) (1,1), 8 keys each,
    // for the value operand (four transposed reads) and the probabilities alike -- the
    // same pairing of keys as four 32x32x16 MFMAs, so the same sum.
    static_assert(BN == 64, "fp8 tiles are 64 keys: one 64-deep MFMA per output block");
    const i32x8_t pb = __builtin_bit_cast(i32x8_t, (long __attribute__((ext_vector_type(4)))){
        pt.pk[0][0], pt.pk[0][1], pt.pk[1][0], pt.pk[1][1]});
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      i32x2_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int roff = ((i >> 1) * 32 + (i & 1) * 16) * G::ROWB;
        r[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(vt + roff + (ln.vx[0] ^ (db << 5))));
      }
      const i32x8_t a = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
      oacc[db] = TR::mfma(a, pb, oacc[db]);
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const Op pb = pt.pk[b][h];  // bf16: Op == POp
      const int roff = (b * 32 + h * 16) * G::ROWB;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        Op a;
        if constexpr (DT == DT_BF16) {
          const int dx = db << 6;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vt + roff + (ln.vx[0] ^ dx)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vt + roff + (ln.vx[1] ^ dx)));
          typedef short i16x8_t __attribute__((ext_vector_type(8)));
          const i16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          a = __builtin_bit_cast(Op, both);
        }
        oacc[db] = TR::mfma(a, pb, oacc[db]);
      }
    }
  }
}


// Operands of one tile read from LDS into registers ahead of their MFMAs, so that the
// LDS latency is hidden behind other work and the MFMAs can issue back to back with
// VALU work in between.
template <int DT, int D, int BN> struct KOps {
  typename Traits<DT>::Op a[D / 16][BN / 32];
};
template <int DT, int D, int BN> struct VOps {
  typename Traits<DT>::Op a[BN / 32][2][D / 32];
};

template <int DT, int D, int BN>
__device__ __forceinline__ void load_kops(KOps<DT, D, BN>& ko, const uint8_t* kt,
                                          const DmaLane<DT, D, BN>& ln) {
  using G = DmaGeo<DT, D, BN>;
  using Op = typename Traits<DT>::Op;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int x = ln.kx ^ (DT == DT_BF16 ? (ks << 5) : (ks << 4));
#pragma unroll
    for (int b = 0; b < BN / 32; ++b) ko.a[ks][b] = *reinterpret_cast<const Op*>(kt + x + b * 32 * G::ROWB);
  }
}

template <int DT, int D, int BN>
__device__ __forceinline__ void load_vops(VOps<DT, D, BN>& vo, const uint8_t* vt,
                                          const DmaLane<DT, D, BN>& ln) {
  using G = DmaGeo<DT, D, BN>;
  using Op = typename Traits<DT>::Op;
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int roff = (b * 32 + h * 16) * G::ROWB;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        if constexpr (DT == DT_BF16) {
          const int dx = db << 6;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vt + roff + (ln.vx[0] ^ dx)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vt + roff + (ln.vx[1] ^ dx)));
          vo.a[b][h][db] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2_t*)(vt + roff + (ln.vx[0] ^ (db << 5))));
          vo.a[b][h][db] = __builtin_bit_cast(Op, v);
        }
      }
    }
}

// S^T = K Q^T from key operands in registers.
template <int DT, int D, int BN>
__device__ __forceinline__ void qk_regs(f32x16_t (&s)[BN / 32], const KOps<DT, D, BN>& ko,
                                        const typename Traits<DT>::Op (&qop)[D / 16]) {
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) s[b] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int b = 0; b < BN / 32; ++b) s[b] = Traits<DT>::mfma(ko.a[ks][b], qop[ks], s[b]);
}

// O^T += V^T P^T from value operands in registers.
template <int DT, int D, int BN>
__device__ __forceinline__ void pv_regs(f32x16_t (&oacc)[D / 32], const PTile<DT, BN>& pt,
                                        const VOps<DT, D, BN>& vo) {
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = Traits<DT>::mfma(vo.a[b][h][db], pt.pk[b][h], oacc[db]);
}

// ================================================================== register-staged tiles (fp32)
// fp32 tiles go through registers into padded LDS rows: keys row-major, values
// row-major (the fp32 MFMA takes one element per lane, so no transpose is needed).
template <int D, int BN> struct StGeo {
  static constexpr int EB = 4;
  static constexpr int K_STRIDE = D * EB + 4;                        // odd dword stride
  static constexpr int V_STRIDE = D * EB + 16;
  static constexpr int K_BYTES = (BN * K_STRIDE + 15) / 16 * 16;
  static constexpr int V_BYTES = (BN * V_STRIDE + 15) / 16 * 16;
  static constexpr int LDS_BYTES = 2 * (K_BYTES + V_BYTES);
  static constexpr int CPR = D * EB / 16;
  static constexpr int CHUNKS = BN * CPR;
  static constexpr int PER_THREAD = (CHUNKS + kThreads - 1) / kThreads;
};

template <int D, int BN> struct StRegs {
  u32x4_t r[StGeo<D, BN>::PER_THREAD];
};

template <int D, int BN>
__device__ __forceinline__ void st_load(StRegs<D, BN>& st, __amdgpu_buffer_rsrc_t rs, int k0, int tid) {
  using G = StGeo<D, BN>;
#pragma unroll
  for (int r = 0; r < G::PER_THREAD; ++r) {
    const int idx = tid + r * kThreads;
    if (G::CHUNKS % kThreads == 0 || idx < G::CHUNKS) {
      const int row = idx / G::CPR, col = idx % G::CPR;
      st.r[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k0 + row) * (D * G::EB) + col * 16, 0, 0);
    }
  }
}

template <int D, int BN, int STRIDE>
__device__ __forceinline__ void st_store(const StRegs<D, BN>& st, uint8_t* dst, int tid) {
  using G = StGeo<D, BN>;
#pragma unroll
  for (int r = 0; r < G::PER_THREAD; ++r) {
    const int idx = tid + r * kThreads;
    if (G::CHUNKS % kThreads == 0 || idx < G::CHUNKS) {
      const int row = idx / G::CPR, col = idx % G::CPR;
      uint32_t* q = reinterpret_cast<uint32_t*>(dst + row * STRIDE + col * 16);
      if constexpr (STRIDE % 16 == 0) {
        *reinterpret_cast<u32x4_t*>(q) = st.r[r];
      } else {
        q[0] = st.r[r][0]; q[1] = st.r[r][1]; q[2] = st.r[r][2]; q[3] = st.r[r][3];
      }
    }
  }
}

template <int D, int BN>
__device__ __forceinline__ void qk_st(f32x16_t (&s)[BN / 32], const uint8_t* kb,
                                      const float (&qop)[D / 2], int c, int g) {
  using G = StGeo<D, BN>;
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) {
    s[b] = f32x16_t{};
    const uint8_t* krow = kb + (b * 32 + c) * G::K_STRIDE + g * 4;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
      s[b] = Traits<DT_F32>::mfma(*reinterpret_cast<const float*>(krow + ks * 8), qop[ks], s[b]);
  }
}

template <int D, int BN>
__device__ __forceinline__ void pv_st(f32x16_t (&oacc)[D / 32], const f32x16_t (&s)[BN / 32],
                                      const uint8_t* vb, int c, int g) {
  using G = StGeo<D, BN>;
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const int key = b * 32 + (tt >> 2) * 8 + g * 4 + (tt & 3);
      const uint8_t* vrow = vb + key * G::V_STRIDE + c * 4;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = Traits<DT_F32>::mfma(*reinterpret_cast<const float*>(vrow + db * 128),
                                        s[b][tt], oacc[db]);
    }
}

// ================================================================== softmax
// Keys past the chunk / sequence end, and keys above the causal diagonal, become -inf.
template <int BN>
__device__ __forceinline__ void mask_tile(f32x16_t (&s)[BN / 32], int k0, int kend, int row,
                                          int off, bool causal, int g) {
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = k0 + b * 32 + (j >> 2) * 8 + g * 4 + (j & 3);
      const bool vis = key < kend && (!causal || key <= row + off);
      if (!vis) s[b][j] = -__builtin_inff();
    }
}

// Probabilities of a tile in the form the value MFMA consumes: for bf16 and fp8 the
// packed B operands of each 16-key step (pk[b][h] holds elements 8h..8h+7 of score
// block b); for fp32 the scores themselves, overwritten in place.
template <int DT, int BN> struct PTile {
  typename Traits<DT>::POp pk[BN / 32][2];
};
template <int BN> struct PTile<DT_F32, BN> {};

// Online-softmax step for one tile, in three parts so that the key sweep can
// interleave them with the MFMAs of neighbouring tiles:
//
//   softmax_rescale  row maximum; moves the reference maximum (lazily) and rescales
//                    the accumulator and the running sums when it moves;
//   softmax_exp      unnormalised probabilities exp2(s * scale_log2 - m), packed into
//                    the operand form of the value MFMA;
//   softmax_sums     two row sums: l_run of the probabilities as computed (it gives the
//                    log-sum-exp), and c_run of exactly the rounded values that entered
//                    the value MFMA (it normalises O).  With c_run, numerator and
//                    denominator of O agree, so a row dominated by one key returns that
//                    key's value up to accumulation error instead of off by the
//                    rounding of its probability.
template <int DT, int BN, int NDB>
__device__ __forceinline__ float softmax_rescale(const f32x16_t (&s)[BN / 32], f32x16_t (&oacc)[NDB],
                                                 float& m_run, float& l_run, float& c_run, float sl2) {
  using TR = Traits<DT>;
  float mx = -__builtin_inff();
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[b][j]);
  mx = pair_max(mx);
  const float mt = mx * sl2;
  if (__builtin_amdgcn_ballot_w64(mt > m_run + TR::kTau)) {
    const float m_new = __builtin_fmaxf(m_run, mt);
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
    c_run *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
    m_run = m_new;
  }
  return (m_run == -__builtin_inff()) ? 0.0f : m_run;
}

// Probabilities (already scaled by 2^kPExp) -> E4M3 value-MFMA operands.  Each 32-bit
// word takes two conversions (low half, then high half); written as one asm pair with
// an output-only word, so that no register has to be cleared or copied for the half the
// first conversion leaves alone.
__device__ __forceinline__ uint32_t cvt4_fp8(float a, float b, float c, float d) {
  uint32_t w;
  asm("v_cvt_pk_fp8_f32 %0, %1, %2\n\tv_cvt_pk_fp8_f32 %0, %3, %4 op_sel:[0,0,1]"
      : "=&v"(w) : "v"(a), "v"(b), "v"(c), "v"(d));
  return w;
}
template <int BN>
__device__ __forceinline__ void pack_fp8(const f32x16_t (&p)[BN / 32], PTile<DT_FP8, BN>& pt) {
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 8 * h;
      const uint32_t lo = cvt4_fp8(p[b][e + 0], p[b][e + 1], p[b][e + 2], p[b][e + 3]);
      const uint32_t hi = cvt4_fp8(p[b][e + 4], p[b][e + 5], p[b][e + 6], p[b][e + 7]);
      pt.pk[b][h] = (long)(((unsigned long)hi << 32) | lo);
    }
}

template <int DT, int BN>
__device__ __forceinline__ void softmax_exp(f32x16_t (&s)[BN / 32], PTile<DT, BN>& pt, float ms,
                                            float sl2) {
  using TR = Traits<DT>;
  // FP8 probabilities come out scaled by kPScale (an exponent offset of kPExp).
  float mo = ms;
  if constexpr (DT == DT_FP8) mo = ms - float(TR::kPExp);
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) s[b][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][j], sl2, -mo));
  if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int b = 0; b < BN / 32; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x8_t x = {s[b][8 * h + 0], s[b][8 * h + 1], s[b][8 * h + 2], s[b][8 * h + 3],
                     s[b][8 * h + 4], s[b][8 * h + 5], s[b][8 * h + 6], s[b][8 * h + 7]};
        pt.pk[b][h] = __builtin_convertvector(x, bf16x8_t);
      }
  } else if constexpr (DT == DT_FP8) {
    pack_fp8<BN>(s, pt);
  }
}

template <int DT, int BN>
__device__ __forceinline__ void softmax_sums(const f32x16_t (&s)[BN / 32], const PTile<DT, BN>& pt,
                                             float& l_run, float& c_run) {
  using TR = Traits<DT>;
  float ls = 0.0f;
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) ls += s[b][j];
  l_run += ls * (1.0f / TR::kPScale);
  if constexpr (DT == DT_BF16) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float cs = 0.0f;
#pragma unroll
    for (int b = 0; b < BN / 32; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2_t two = {pt.pk[b][h][2 * e], pt.pk[b][h][2 * e + 1]};
          cs = __builtin_amdgcn_fdot2_f32_bf16(two, ones, cs, false);
        }
    c_run += cs;
  } else if constexpr (DT == DT_FP8) {
    // the packed sum comes from fp8_psum (an MFMA), read into c_run after the sweep
  } else {
    c_run += ls;
  }
}

// Main-loop variant for bf16 without a per-tile row maximum.  The probabilities are
// taken against the running reference m_run as it stands, and their exact sum tells
// whether that was safe: the sum stays <= 2^kSumCap unless some score exceeds the
// reference by about kSumCap (log2 units) or there is no reference yet (m_run = -inf
// gives +inf).  Only then (rare: a new score far above everything seen so far) is the
// tile redone the exact way: row maximum, new reference, correction of the
// accumulator and the running sums.  The result is the same exact softmax; the
// unnormalised probabilities are just allowed to reach 2^kSumCap instead of 2^kTau.
constexpr float kSumCap = 4294967296.0f;  // 2^32

template <int BN>
__device__ __forceinline__ float softmax_exp_ref(const f32x16_t (&s)[BN / 32], f32x16_t (&p)[BN / 32],
                                                 float m_ref, float sl2) {
  float ls = 0.0f;
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[b][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][j], sl2, -m_ref));
      ls = (b == 0 && j == 0) ? p[b][j] : ls + p[b][j];
    }
  return ls;
}

// (eoff: exponent offset of the probabilities, kPExp for fp8, 0 otherwise)
template <int BN, int NDB>
__device__ __forceinline__ float softmax_redo(const f32x16_t (&s)[BN / 32], f32x16_t (&p)[BN / 32],
                                              f32x16_t (&oacc)[NDB], float& m_run, float& l_run,
                                              float& c_run, float sl2, float eoff = 0.0f) {
  float mx = -__builtin_inff();
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[b][j]);
  const float m_new = __builtin_fmaxf(m_run, pair_max(mx) * sl2);
  if (m_new != -__builtin_inff()) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
    l_run *= alpha;
    c_run *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
    m_run = m_new;
  }
  return softmax_exp_ref<BN>(s, p, (m_run == -__builtin_inff() ? 0.0f : m_run) - eoff, sl2);
}

// FP8: the column sums of a tile's packed probabilities (one per query, the same in every
// accumulator element of the lane) from one 64-deep MFMA with an all-ones E4M3 block
// (0x38 = 1.0) as the A operand: exact products, fp32 accumulation like the value MFMA.
// The sums accumulate in an accumulator block of their own, next to the value blocks,
// which every rescale of the accumulator scales with them; nothing reads it before the
// end of the sweep, so no step waits on this MFMA.
__device__ __forceinline__ void fp8_psum(const PTile<DT_FP8, 64>& pt, f32x16_t& acc) {
  const i32x8_t ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};
  const i32x8_t pb = __builtin_bit_cast(i32x8_t, (long __attribute__((ext_vector_type(4)))){
      pt.pk[0][0], pt.pk[0][1], pt.pk[1][0], pt.pk[1][1]});
  acc = Traits<DT_FP8>::mfma(ones, pb, acc);
}

// Probabilities -> value-MFMA operands (bf16), and the sum of exactly those values.
template <int BN>
__device__ __forceinline__ float pack_bf16(const f32x16_t (&p)[BN / 32], PTile<DT_BF16, BN>& pt) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  float cs = 0.0f;
#pragma unroll
  for (int b = 0; b < BN / 32; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x8_t x = {p[b][8 * h + 0], p[b][8 * h + 1], p[b][8 * h + 2], p[b][8 * h + 3],
                   p[b][8 * h + 4], p[b][8 * h + 5], p[b][8 * h + 6], p[b][8 * h + 7]};
      pt.pk[b][h] = __builtin_convertvector(x, bf16x8_t);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t two = {pt.pk[b][h][2 * e], pt.pk[b][h][2 * e + 1]};
        cs = __builtin_amdgcn_fdot2_f32_bf16(two, ones, cs, false);
      }
    }
  return cs;
}

template <int DT, int BN, int NDB>
__device__ __forceinline__ void softmax_tile(f32x16_t (&s)[BN / 32], PTile<DT, BN>& pt,
                                             f32x16_t (&oacc)[NDB], float& m_run, float& l_run,
                                             float& c_run, float sl2) {
  const float ms = softmax_rescale<DT, BN, NDB>(s, oacc, m_run, l_run, c_run, sl2);
  softmax_exp<DT, BN>(s, pt, ms, sl2);
  softmax_sums<DT, BN>(s, pt, l_run, c_run);
}

// Wavefronts per SIMD the register budget allows: two (256 registers each) unless a
// wavefront holds a d = 256 accumulator or fp32 operands; three (168 registers) for the
// bf16 d = 64 four-wavefront kernels, whose 32-key tiles leave 32 KB of LDS per workgroup
// and whose VALU-heavy sweep gains from a third wavefront beside each MFMA stream.
constexpr int waves_per_eu(int dt, int d) { return (d >= 256 || dt == DT_F32) ? 1 : 2; }
constexpr int fwd_waves(int dt, int d, int bn, bool two_groups) {
  return (dt == DT_BF16 && d == 64 && bn == 32 && !two_groups) ? 3 : waves_per_eu(dt, d);
}

// ================================================================== tile pipeline
// Uniform interface over the two ways tiles reach LDS.  issue_*: start the loads of a
// tile (direct-to-LDS loads already target the stage); commit_*: registers -> LDS for
// the staged variant, nothing for the direct one.
template <int DT, int D, int BN, int NW, bool DMA = Traits<DT>::kDMA> struct Pipe;

template <int DT, int D, int BN, int NW> struct Pipe<DT, D, BN, NW, true> {
  using G = DmaGeo<DT, D, BN>;
  using Op = typename Traits<DT>::Op;
  static constexpr int STAGE_K = G::TILE, STAGE_V = G::TILE;
  static constexpr int NSTAGE = 4;
  static constexpr int KSTEPS = D / Traits<DT>::kKS;
  // bf16 operands go LDS -> registers ahead of their MFMAs (d = 256 too: one wavefront
  // per SIMD has 512 registers, and the deferred sweep's independent MFMA and VALU work
  // is what overlaps there, +4-6 % measured).
  static constexpr bool kRegOps = DT == DT_BF16;
  // Wait until at most N iterations' worth of tile loads are still in flight.
  static constexpr int NI = G::TILE / 1024 / NW;  // 1 KiB loads per wavefront per tile
  template <int N> __device__ __forceinline__ static void wait_loads() {
    constexpr int n = N * 2 * NI;  // key + value loads per thread per iteration
    static_assert(n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
  }
  DmaLane<DT, D, BN> ln;
  int wave, lane;
  __device__ __forceinline__ Pipe(int w, int l) : ln(l), wave(w), lane(l) {}
  __device__ __forceinline__ void issue_k(__amdgpu_buffer_rsrc_t rs, int k0, uint8_t* dst) {
    dma_tile<DT, D, BN, false, NW>(rs, dst, k0, wave, lane);
  }
  __device__ __forceinline__ void issue_v(__amdgpu_buffer_rsrc_t rs, int k0, uint8_t* dst) {
    dma_tile<DT, D, BN, true, NW>(rs, dst, k0, wave, lane);
  }
  __device__ __forceinline__ void issue_k(const Slice& sl, int k0, uint8_t* dst) {
    dma_tile_at<DT, D, BN, false, NW>(sl, dst, k0, wave, lane);
  }
  __device__ __forceinline__ void issue_v(const Slice& sl, int k0, uint8_t* dst) {
    dma_tile_at<DT, D, BN, true, NW>(sl, dst, k0, wave, lane);
  }
  __device__ __forceinline__ void commit_k(uint8_t*, int) {}
  __device__ __forceinline__ void commit_v(uint8_t*, int) {}
  __device__ __forceinline__ void qk(f32x16_t (&s)[BN / 32], const uint8_t* kt, const Op (&qop)[KSTEPS]) {
    qk_dma<DT, D, BN>(s, kt, qop, ln);
  }
  __device__ __forceinline__ void pv(f32x16_t (&oacc)[D / 32], const f32x16_t (&)[BN / 32],
                                     const PTile<DT, BN>& pt, const uint8_t* vt) {
    pv_dma<DT, D, BN>(oacc, pt, vt, ln);
  }
};

template <int DT, int D, int BN, int NW> struct Pipe<DT, D, BN, NW, false> {
  static_assert(NW == kWaves, "the register-staged path runs four wavefronts");
  using G = StGeo<D, BN>;
  using Op = float;
  static constexpr int STAGE_K = G::K_BYTES, STAGE_V = G::V_BYTES;
  static constexpr int NSTAGE = 2;
  static constexpr int KSTEPS = D / 2;
  static constexpr bool kRegOps = false;
  template <int N> __device__ __forceinline__ static void wait_loads() { wait_vmem(); }
  StRegs<D, BN> rk, rv;
  int c, g;
  __device__ __forceinline__ Pipe(int w, int l) : c(l & 31), g(l >> 5) { (void)w; }
  __device__ __forceinline__ void issue_k(__amdgpu_buffer_rsrc_t rs, int k0, uint8_t*) {
    st_load<D, BN>(rk, rs, k0, threadIdx.x);
  }
  __device__ __forceinline__ void issue_v(__amdgpu_buffer_rsrc_t rs, int k0, uint8_t*) {
    st_load<D, BN>(rv, rs, k0, threadIdx.x);
  }
  __device__ __forceinline__ void issue_k(const Slice& sl, int k0, uint8_t*) {
    st_load<D, BN>(rk, make_rsrc(sl.base, sl.bytes), k0, threadIdx.x);
  }
  __device__ __forceinline__ void issue_v(const Slice& sl, int k0, uint8_t*) {
    st_load<D, BN>(rv, make_rsrc(sl.base, sl.bytes), k0, threadIdx.x);
  }
  __device__ __forceinline__ void commit_k(uint8_t* dst, int tid) { st_store<D, BN, G::K_STRIDE>(rk, dst, tid); }
  __device__ __forceinline__ void commit_v(uint8_t* dst, int tid) { st_store<D, BN, G::V_STRIDE>(rv, dst, tid); }
  __device__ __forceinline__ void qk(f32x16_t (&s)[BN / 32], const uint8_t* kt, const float (&qop)[KSTEPS]) {
    qk_st<D, BN>(s, kt, qop, c, g);
  }
  __device__ __forceinline__ void pv(f32x16_t (&oacc)[D / 32], const f32x16_t (&s)[BN / 32],
                                     const PTile<DT_F32, BN>&, const uint8_t* vt) {
    pv_st<D, BN>(oacc, s, vt, c, g);
  }
};

// ================================================================== instruction interleave
// Within one wavefront an MFMA occupies the matrix pipe for 32 cycles (32x32x16) while
// the wavefront keeps issuing independent VALU instructions, about four of them per
// MFMA.  sched_pairs asks the scheduler for N repetitions of {C1 instructions of
// class M1, C2 of class M2} (class masks of __builtin_amdgcn_sched_group_barrier:
// 0x2 VALU, 0x8 MFMA), so the exponentials of one tile fill the shadow of the MFMAs of
// its neighbours instead of running in a block of their own.
template <int N, int M1, int C1, int M2, int C2>
__device__ __forceinline__ void sched_pairs() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(M1, C1, 0);
    __builtin_amdgcn_sched_group_barrier(M2, C2, 0);
    sched_pairs<N - 1, M1, C1, M2, C2>();
  }
}

// Interleave for the bf16 main loop (no row maximum), whose tile step has two
// scheduling regions (before and after the rare re-reference branch): the S^T MFMAs of
// the next tile with the exponentials and the exact sum, then the value MFMAs with the
// conversion and the consistent sum.
template <int D, int BN>
__device__ __forceinline__ void interleave_exp() {
  constexpr int NKB = BN / 32;
  constexpr int NQ = (D / 16) * NKB;
  constexpr int VE = NKB * 48;                // fma + exp + add per score
  sched_pairs<NQ, 0x8, 1, 0x2, (VE + NQ - 1) / NQ>();
}
template <int D, int BN>
__device__ __forceinline__ void interleave_pv() {
  constexpr int NKB = BN / 32;
  constexpr int NP = NKB * 2 * (D / 32);
  constexpr int VS = NKB * 16;                // converts and dot products
  sched_pairs<NP, 0x8, 1, 0x2, (VS + NP - 1) / NP>();
}

// Interleave for the deferred bf16 main loop: each of the iteration's MFMAs
// (S^T of tile t+2, then P(t) V(t)) is followed by two VALU instructions of the work on
// tile t+1 -- exponentials, row sum, bf16 packing and the sum of the packed values, none
// of which the MFMAs depend on -- and what remains of that work follows the last MFMA.
// (Two per MFMA measured 1.7-3 % faster at d = 64 and 128 than spreading all of it
// evenly, i.e. 4 or 8 per MFMA; one, three, none, or a block of it first were slower.)
template <int D, int BN>
__device__ __forceinline__ void interleave_deferred() {
  constexpr int NKB = BN / 32;
  constexpr int NM = (D / 16) * NKB + NKB * 2 * (D / 32);  // MFMAs per iteration
  constexpr int NV = NKB * (48 + 16);                       // VALU per iteration
  constexpr int NR = NKB * (D / 16) + NKB * 2 * (D / 32) * 2;  // LDS operand reads
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  sched_pairs<NM, 0x8, 1, 0x2, 2>();
  __builtin_amdgcn_sched_group_barrier(0x2, NV, 0);
}

// Largest finite E4M3 value.
constexpr float kFp8Max = 448.0f;

// ================================================================== forward kernel
// MODE kPlain: O and lse of one 128-row query tile per workgroup (four wavefronts).
// MODE kSplit: the unnormalised state of one key chunk of one query tile.
// MODE kPairs (causal): one workgroup of two four-wavefront groups per pair of query
//   tiles t < T = nqt-1-t of one head, which together need (t+1) + (T+1) key-tile
//   units.  Group A sweeps tile t, then the first X key tiles of tile T; group B
//   sweeps the rest of tile T; X is chosen so that both groups sweep the same number
//   of key tiles.  At the end A hands its partial state of tile T to B through LDS and
//   B merges the two (the split-K merge of the pages, inside one workgroup).  Every CU
//   then does the same work with both groups busy to the end, where separate
//   workgroups of very different lengths would leave one alone on its CU.
// MODE kDualPlain / kDualSplit: as kPlain / kSplit, but two four-wavefront groups split
//   the tile's key range in halves and merge the same way (used when the grid has at
//   most one workgroup per CU: the second group gives every SIMD a second wavefront).
enum : int { kPlain = 0, kSplit = 1, kPairs = 2, kDualPlain = 3, kDualSplit = 4 };
constexpr bool two_groups(int mode) { return mode == kPairs || mode == kDualPlain || mode == kDualSplit; }

template <int DT, int D, int BN, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads * (two_groups(MODE) ? 2 : 1),
                                                      kThreads * (two_groups(MODE) ? 2 : 1)),
                          amdgpu_waves_per_eu(fwd_waves(DT, D, BN, two_groups(MODE)),
                                              fwd_waves(DT, D, BN, two_groups(MODE)))))
void attn_fwd_kernel(FwdArgs p) {
  using TR = Traits<DT>;
  using P = Pipe<DT, D, BN, kWaves>;
  using Op = typename TR::Op;
  constexpr bool SPLIT = MODE == kSplit || MODE == kDualSplit;
  constexpr int NG = two_groups(MODE) ? 2 : 1;  // four-wavefront groups per workgroup
  constexpr int EB = TR::kBytes;
  constexpr int KSTEPS = D / TR::kKS;  // MFMAs over d per 32-key block of S^T
  constexpr int NKB = BN / 32;         // 32-key blocks per tile
  constexpr int NDB = D / 32;          // 32-row blocks of O^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int gwave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = NG > 1 ? gwave / kWaves : 0;      // group of this wavefront
  const int wave = NG > 1 ? gwave % kWaves : gwave;  // wavefront within its group
  const int gtid = NG > 1 ? tid % kThreads : tid;    // thread within its group
  const int c = lane & 31, g = lane >> 5;

  // ---- which (batch*head, query tile(s), split) this workgroup owns.
  const int BH = p.B * p.H;
  const int nqt = ceil_div_i(p.Sq, kBlockM);
  int bh, qt, split = 0;
  if (MODE == kPlain && p.cu_q != nullptr) {
    // Ragged batch: workgroup -> (sequence b, head h, r-th query tile of the sequence);
    // the grid is sized for the longest sequence and workgroups past their sequence's
    // end leave at once (before any barrier).  Slice s = b*H + h runs on XCD s % 8 (the
    // dispatcher sends workgroup i to XCD i % 8), all its tiles in a row: the XCDs get
    // the heads of every sequence in equal shares whatever the lengths, and each slice's
    // keys stream through one L2.  (A contiguous range of sequences per XCD, as for
    // dense calls, leaves the XCDs with the short sequences idle.)  The offsets come from
    // device memory: clamped to [0, total] and the lengths to [0, max_seqlen], so that no
    // entry can move an access outside the buffers.  From here on the workgroup sees one
    // (batch, head) slice of length Sq x Sk, as in a dense call with B = H = 1.
    const int nslices = p.B * p.H;
    int r, sh;
    if ((nslices & 7) == 0) {
      const int j = blockIdx.x & 7, i = blockIdx.x >> 3;
      sh = j + 8 * (i / nqt);
      r = i % nqt;
    } else {
      sh = blockIdx.x / nqt;
      r = blockIdx.x % nqt;
    }
    const int b = sh / p.H, h = sh % p.H;
    auto span = [](const int32_t* cu, int b, int total, int maxlen, int& lo) {
      const long long a = cu[b], e = cu[b + 1];
      lo = int(a < 0 ? 0 : a > total ? total : a);
      long long n = e - lo;
      n = n < 0 ? 0 : n;
      n = n > maxlen ? maxlen : n;
      n = n > total - lo ? total - lo : n;
      return int(n);
    };
    int q_lo, k_lo;
    const int q_len = span(p.cu_q, b, p.total_q, p.Sq, q_lo);
    const int k_len = span(p.cu_k, b, p.total_k, p.Sk, k_lo);
    const int nqt_b = ceil_div_i(q_len, kBlockM);
    if (r >= nqt_b) return;
    qt = p.causal ? nqt_b - 1 - r : r;  // causal: longest sweeps first
    bh = 0;
    const int64_t qrow = int64_t(h) * p.total_q + q_lo, krow = int64_t(h) * p.total_k + k_lo;
    p.q = reinterpret_cast<const uint8_t*>(p.q) + qrow * D * EB;
    p.k = reinterpret_cast<const uint8_t*>(p.k) + krow * D * EB;
    p.v = reinterpret_cast<const uint8_t*>(p.v) + krow * D * EB;
    p.o = p.o_bf16 ? reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(p.o) + qrow * D) : p.o + qrow * D;
    p.lse += qrow;
    p.Sq = q_len;
    p.Sk = k_len;
  } else if (MODE == kPairs) {
    // batch*head fastest: all pairs of a head land on one XCD (index mod 8).
    bh = blockIdx.x % BH;
    qt = blockIdx.x / BH;              // the lighter tile t of the pair
  } else if (!SPLIT && p.causal && p.pair_order == 1) {
    // The whole grid is resident at once (two workgroups per CU, dispatched in index
    // order): workgroups i and i + grid/2 share a CU, so they get complementary query
    // tiles (t and nqt-1-t) of the same head and every CU gets the same work.
    bh = blockIdx.x % BH;
    qt = blockIdx.x / BH;
    const int half = (nqt + 1) / 2;
    qt = qt < half ? nqt - 1 - qt : qt - half;
  } else {
    // The dispatcher hands workgroup i to XCD i mod 8.  Renumber so that each XCD
    // works through a contiguous range of the logical order, and order that range as
    // groups of head_group heads with all their query tiles, heads fastest: the
    // workgroups resident on an XCD at one time then share a few heads' key/value
    // streams in that XCD's L2.  Causal sweeps go longest first within each group.
    int x = blockIdx.x;
    const int nwg = gridDim.x;
    if ((nwg & 7) == 0) x = (x & 7) * (nwg >> 3) + (x >> 3);
    const int per_split = BH * nqt;
    split = x / per_split;
    x -= split * per_split;
    const int G = p.head_group;
    const int b = x % G;
    x /= G;
    const int r = x % nqt;
    bh = (x / nqt) * G + b;
    qt = (!SPLIT && p.causal) ? nqt - 1 - r : r;
  }
  const int off = p.Sk - p.Sq;                // causal: key j visible to row i iff j <= i + off

  // Keys a query tile sees: [0, kend_of(tile)) (causal: up to its last row's diagonal).
  auto kend_of = [&](int tile) __attribute__((always_inline)) {
    if (!p.causal) return p.Sk;
    const int last_row = min((tile + 1) * kBlockM, p.Sq) - 1;
    return max(0, min(p.Sk, last_row + off + 1));
  };

  const size_t q_base = size_t(bh) * p.Sq * D;
  const size_t kv_base = size_t(bh) * p.Sk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const uint8_t*>(p.q) + q_base * EB,
                                              uint32_t(p.Sq) * D * EB);
  const Slice rk{reinterpret_cast<const uint8_t*>(p.k) + kv_base * EB, uint32_t(p.Sk) * D * EB};
  const Slice rv{reinterpret_cast<const uint8_t*>(p.v) + kv_base * EB, uint32_t(p.Sk) * D * EB};

  // ---- per-wavefront state of the query tile being swept
  int q0 = 0, r0 = 0, row = 0, wave_last = 0;
  Op qop[KSTEPS];
  // O^T blocks, and for fp8 one more block that accumulates the packed sums
  constexpr int NACC = NDB + (DT == DT_FP8 ? 1 : 0);
  f32x16_t oacc[NACC];
  float m_run, l_run, c_run;  // reference maximum (log2 units), row sum, consistent row sum
  auto ov = [&]() __attribute__((always_inline)) -> f32x16_t(&)[NDB] {
    return *reinterpret_cast<f32x16_t(*)[NDB]>(&oacc[0]);
  };
  // FP8: c_run from the packed-sum block (every lane holds its query's full sum; half
  // of it goes to each of the two lanes whose partial sums pair_sum adds)
  auto take_csum = [&]() __attribute__((always_inline)) {
    if constexpr (DT == DT_FP8) c_run = oacc[NDB][0] * (0.5f / TR::kPScale);
  };
  auto add_psum = [&](const PTile<DT, BN>& pt) __attribute__((always_inline)) {
    if constexpr (DT == DT_FP8) fp8_psum(pt, oacc[NDB]);
  };
  const float sl2 = p.scale_log2;

  // Start query tile `tile`: its rows, its Q operands (B operand of S^T = K Q^T, in
  // registers for the whole sweep; rows past Sq read as zeros) and an empty state.
  auto begin_tile = [&](int tile) __attribute__((always_inline)) {
    q0 = tile * kBlockM;
    r0 = q0 + wave * kRowsPerWave;            // first query row of this wavefront
    row = r0 + c;                             // query row of this lane
    wave_last = min(r0 + kRowsPerWave - 1, p.Sq - 1);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int boff = (row * D + ks * TR::kKS + g * TR::kKPL) * EB;
      if constexpr (DT == DT_BF16) {
        qop[ks] = __builtin_bit_cast(Op, __builtin_amdgcn_raw_buffer_load_b128(rq, boff, 0, 0));
      } else if constexpr (DT == DT_FP8) {
        const u32x4_t lo = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, boff, 0, 0));
        const u32x4_t hi = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, boff + 16, 0, 0));
        qop[ks] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        qop[ks] = __builtin_bit_cast(Op, __builtin_amdgcn_raw_buffer_load_b32(rq, boff, 0, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < NACC; ++i) oacc[i] = f32x16_t{};
    m_run = -__builtin_inff();  // same in lanes c and c+32
    l_run = 0.0f;               // this lane's share of the row sum
    c_run = 0.0f;               // same, of the probabilities as rounded for the MFMA
  };

  P pipe(wave, lane);
  // NS-stage rings for key and value tiles, one pair of rings per group.  Tile j lives
  // in stage j % NS.  The sweep is unrolled, so every LDS access names a compile-time
  // stage and the direct-to-LDS loads still in flight provably do not alias the
  // stages being read (no wait is needed before the operand reads).
  constexpr int NS = P::NSTAGE;
  static_assert(NS >= 2 && NS <= 5, "stage count");
  constexpr int SK = P::STAGE_K * NG, SV = P::STAGE_V * NG;
  // one named array per stage: the wait insertion only tells distinct objects apart
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[SK], ks1[SK];
  __shared__ __attribute__((aligned(1024))) uint8_t ks2[NS > 2 ? SK : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t ks3[NS > 3 ? SK : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t ks4[NS > 4 ? SK : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[SV], vs1[SV];
  __shared__ __attribute__((aligned(1024))) uint8_t vs2[NS > 2 ? SV : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t vs3[NS > 3 ? SV : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t vs4[NS > 4 ? SV : 1];
  const int kgo = grp * P::STAGE_K, vgo = grp * P::STAGE_V;  // this group's half
  auto kst = [&](int j) __attribute__((always_inline)) -> uint8_t* {
    const int i = j % NS;
    return (i == 0 ? ks0 : i == 1 ? ks1 : i == 2 ? ks2 : i == 3 ? ks3 : ks4) + kgo;
  };
  auto vst = [&](int j) __attribute__((always_inline)) -> uint8_t* {
    const int i = j % NS;
    return (i == 0 ? vs0 : i == 1 ? vs1 : i == 2 ? vs2 : i == 3 ? vs3 : vs4) + vgo;
  };
  // The sweep is unrolled by U tiles: a multiple of NS (constant stages) and of 2 (the
  // two score buffers alternate).
  constexpr int U = NS % 2 == 0 ? NS : 2 * NS;
  constexpr bool kDeferred = P::kRegOps && MODE != kPairs;

  // ---- key sweep over keys [kbeg, kend) of the current query tile, in `ntiles`
  // iterations.  Every group of the workgroup passes the same number of barriers
  // (2 + ntiles): iterations past this group's own keys only keep the barrier cadence.
  auto sweep = [&](int kbeg, int kend, int ntiles) __attribute__((always_inline)) {
    // The key and value slices end at kend: the ring's loads past the range (the last
    // iterations' look-ahead) then return zeros without touching memory, instead of
    // fetching the next keys -- another group's or another chunk's -- for nothing.
    const uint32_t kv_end = uint32_t(kend) * uint32_t(D * EB);
    const Slice ksl{rk.base, rk.bytes < kv_end ? rk.bytes : kv_end};
    const Slice vsl{rv.base, rv.bytes < kv_end ? rv.bytes : kv_end};
    // A tile starting at key k0 has work for this wavefront unless it starts past the
    // range, every row of the wavefront is past Sq, or (causal) every key of the tile
    // is above the wavefront's diagonal.
    auto active = [&](int k0) __attribute__((always_inline)) {
      return k0 < kend && r0 < p.Sq && (!p.causal || k0 <= wave_last + off);
    };
    auto needs_mask = [&](int k0) __attribute__((always_inline)) {
      return (k0 + BN > kend) || (p.causal && (k0 + BN - 1 > r0 + off));
    };

    if constexpr (kDeferred) {
      // ---- deferred pipeline (bf16, every head dim; not the causal pair mode, whose two
      // sweeps per group pay the longer prologue twice: measured 2-5 % slower there).
      // Iteration t computes S^T of key tile t+2, adds P(t) V(t) with the probabilities
      // packed in iteration t-1, and turns the scores of tile t+1 into P(t+1): none of
      // the iteration's MFMAs waits for its own exponentials, so the two interleave
      // freely.  Tile j's keys and values
      // live in stage j % 4; iteration t requests key tile t+5 (into the stage of key
      // tile t+1, read in iteration t-1) and value tile t+3 (into the stage of value
      // tile t-1).  In every iteration the newest two iterations' loads may stay in
      // flight: loads complete in order, so key tile t+3 and value tile t+1 (needed
      // next) have then landed.
      static_assert(NS == 4 && U == 4, "the stage plan assumes a four-stage ring");
      f32x16_t sa[NKB], sb[NKB];
      PTile<DT, BN> pa, pb;
      if (ntiles > 0) {
        pipe.issue_k(ksl, kbeg + 0 * BN, kst(0));
        pipe.issue_k(ksl, kbeg + 1 * BN, kst(1));
        pipe.issue_k(ksl, kbeg + 2 * BN, kst(2));
        pipe.issue_v(vsl, kbeg + 0 * BN, vst(0));
        pipe.issue_k(ksl, kbeg + 3 * BN, kst(3));
        pipe.issue_v(vsl, kbeg + 1 * BN, vst(1));
      }
      P::template wait_loads<2>();  // key tiles 0 and 1
      block_sync();
      const bool act0 = ntiles > 0 && active(kbeg);
      if (act0) pipe.qk(sa, kst(0), qop);
      if (ntiles > 1 && active(kbeg + BN)) pipe.qk(sb, kst(1), qop);
      block_sync();  // key tile 0's stage is free again
      if (ntiles > 0) {
        pipe.issue_k(ksl, kbeg + 4 * BN, kst(0));
        pipe.issue_v(vsl, kbeg + 2 * BN, vst(2));
      }
      // tile 0's softmax (registers only) while key tile 2 and value tile 0 land
      if (act0) {
        if (needs_mask(kbeg)) mask_tile<BN>(sa, kbeg, kend, row, off, p.causal, g);
        softmax_tile<DT, BN, NACC>(sa, pa, oacc, m_run, l_run, c_run, sl2);
      }
      P::template wait_loads<2>();  // key tile 2 and value tile 0
      block_sync();

      auto finish_d = [&]() __attribute__((always_inline)) {
        P::template wait_loads<2>();
        block_sync();
      };
      // Tiles t and t+1 full (every row sees every key, every wavefront active): no
      // branch except the rare re-reference.  The next tile's probabilities are packed
      // speculatively and packed again if the reference moves.
      auto step_full = [&](int t, uint8_t* kdst, uint8_t* vdst, const uint8_t* kb, const uint8_t* vb,
                           f32x16_t (&s_cur)[NKB], f32x16_t (&s_next)[NKB], const PTile<DT, BN>& pcur,
                           PTile<DT, BN>& pnext) __attribute__((always_inline)) {
        const int k0 = kbeg + t * BN;
        pipe.issue_k(ksl, k0 + 5 * BN, kdst);
        pipe.issue_v(vsl, k0 + 3 * BN, vdst);
        KOps<DT, D, BN> ko;
        VOps<DT, D, BN> vo;
        load_kops<DT, D, BN>(ko, kb, pipe.ln);
        load_vops<DT, D, BN>(vo, vb, pipe.ln);
        qk_regs<DT, D, BN>(s_next, ko, qop);
        pv_regs<DT, D, BN>(oacc, pcur, vo);
        f32x16_t pr[NKB];
        float ls = softmax_exp_ref<BN>(s_cur, pr, m_run, sl2);
        float cs = pack_bf16<BN>(pr, pnext);
        interleave_deferred<D, BN>();
        // (cs is in the test only so that the packing stays ahead of the branch; it is
        // close to ls and non-finite exactly when ls is)
        if (__builtin_amdgcn_ballot_w64(!(ls + cs <= 2.0f * kSumCap))) {
          ls = softmax_redo<BN, NACC>(s_cur, pr, oacc, m_run, l_run, c_run, sl2);
          cs = pack_bf16<BN>(pr, pnext);
        }
        l_run += ls;
        c_run += cs;
        finish_d();
      };
      // Everything else: the causal diagonal band, the sequence / chunk tail, the last
      // tiles, and the cadence-keeping iterations past the range.
      auto step_edge = [&](int t, uint8_t* kdst, uint8_t* vdst, const uint8_t* kb, const uint8_t* vb,
                           f32x16_t (&s_cur)[NKB], f32x16_t (&s_next)[NKB], const PTile<DT, BN>& pcur,
                           PTile<DT, BN>& pnext) __attribute__((always_inline)) {
        const int k0 = kbeg + t * BN;
        const bool act_t = t < ntiles && active(k0);
        const bool act_1 = t + 1 < ntiles && active(k0 + BN);
        const bool act_2 = t + 2 < ntiles && active(k0 + 2 * BN);
        pipe.issue_k(ksl, k0 + 5 * BN, kdst);
        pipe.issue_v(vsl, k0 + 3 * BN, vdst);
        if (act_2) pipe.qk(s_next, kb, qop);
        if (act_t) pipe.pv(ov(), s_cur, pcur, vb);
        if (act_1) {
          // the main loop's lazy softmax, with the mask where the tile needs one
          if (needs_mask(k0 + BN)) mask_tile<BN>(s_cur, k0 + BN, kend, row, off, p.causal, g);
          f32x16_t pr[NKB];
          float ls = softmax_exp_ref<BN>(s_cur, pr, m_run, sl2);
          if (__builtin_amdgcn_ballot_w64(!(ls <= kSumCap)))
            ls = softmax_redo<BN, NACC>(s_cur, pr, oacc, m_run, l_run, c_run, sl2);
          l_run += ls;
          c_run += pack_bf16<BN>(pr, pnext);
        }
        finish_d();
      };
      // Leading tiles that are full: inside [kbeg, kend), (causal) below the diagonal
      // of the tile's first row, and every wavefront has rows.  Iteration t of the
      // full loop needs tiles t and t+1 full; the count is rounded down to a multiple
      // of U so that both loops start on stage 0 with constant stage indices.
      int nfull = (kend - kbeg) / BN;
      if (p.causal) {
        const int d = q0 + off - kbeg - (BN - 1);
        nfull = min(nfull, d < 0 ? 0 : d / BN + 1);
      }
      if (r0 >= p.Sq) nfull = 0;
      nfull = nfull - 1 < 0 ? 0 : ((nfull - 1) / U) * U;
      auto run = [&](auto full_c, int t0, int t1) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
        for (int t = t0; t < t1; t += U) {
#pragma unroll
          for (int j = 0; j < U; ++j) {
            if (FULL || t + j < t1) {
              uint8_t* kd = kst(j + 1);
              uint8_t* vd = vst(j + 3);
              const uint8_t* kb = kst(j + 2);
              const uint8_t* vb = vst(j);
              if (j % 2 == 0) {
                if constexpr (FULL) step_full(t + j, kd, vd, kb, vb, sb, sa, pa, pb);
                else step_edge(t + j, kd, vd, kb, vb, sb, sa, pa, pb);
              } else {
                if constexpr (FULL) step_full(t + j, kd, vd, kb, vb, sa, sb, pb, pa);
                else step_edge(t + j, kd, vd, kb, vb, sa, sb, pb, pa);
              }
            }
          }
        }
      };
      run(std::true_type{}, 0, nfull);
      run(std::false_type{}, nfull, ntiles);
      wait_vmem();
      block_sync();
    } else {

    // prologue: key tiles 0..NS-1 and value tiles 0..NS-2 in flight, then S^T of tile
    // 0 once key tile 0 has landed.  Loads are issued unconditionally (tiles past the
    // end are never used; past the sequence they read as zeros) so that every
    // iteration has the same number of loads in flight and the partial waits stay
    // exact.
    if (ntiles > 0) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        pipe.issue_k(ksl, kbeg + j * BN, kst(j));
        pipe.commit_k(kst(j), gtid);
        if (j < NS - 1) {
          pipe.issue_v(vsl, kbeg + j * BN, vst(j));
          pipe.commit_v(vst(j), gtid);
        }
      }
    }
    // Key tiles 0 and 1 and value tile 0 are what the first iteration reads; the loads
    // complete in order, so the later NS-2 tiles' worth may stay in flight.
    P::template wait_loads<NS - 2>();
    block_sync();
    f32x16_t sa[NKB], sb[NKB];
    if (ntiles > 0 && active(kbeg)) pipe.qk(sa, kst(0), qop);
    block_sync();

    // Iteration t: S^T of tile t+1 is computed while tile t's softmax runs; then
    // O^T += V^T P^T with tile t's values.  Key tile t+NS and value tile t+NS-1 are
    // requested into the stages that iteration t-1 finished reading; at the end of
    // the iteration only the loads that iteration t+1 needs are waited for.
    auto finish = [&](uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
      pipe.commit_k(kdst, gtid);
      pipe.commit_v(vdst, gtid);
      // Loads complete in order and every iteration issues the same number, so
      // leaving the newest (NS-2) iterations' loads in flight guarantees that key
      // tile t+2 and value tile t+1 have landed.
      P::template wait_loads<NS - 2>();
      block_sync();
    };
    // Main part: tiles visible to every row of the group (no mask, every wavefront
    // active).  One straight-line block per tile.
    auto step_full = [&](int t, uint8_t* kdst, uint8_t* vdst, const uint8_t* kb, const uint8_t* vb,
                         f32x16_t (&s_cur)[NKB], f32x16_t (&s_next)[NKB]) __attribute__((always_inline)) {
      const int k0 = kbeg + t * BN;
      pipe.issue_k(ksl, k0 + NS * BN, kdst);
      pipe.issue_v(vsl, k0 + (NS - 1) * BN, vdst);
      PTile<DT, BN> pt;
      if constexpr (P::kRegOps) {
        // Both operand sets are read first (their LDS latency overlaps the row
        // maximum), then the MFMAs of tile t+1 (S^T) and tile t (values) interleave
        // with the exponentials and sums of tile t.
        KOps<DT, D, BN> ko;
        VOps<DT, D, BN> vo;
        load_kops<DT, D, BN>(ko, kb, pipe.ln);
        load_vops<DT, D, BN>(vo, vb, pipe.ln);
        qk_regs<DT, D, BN>(s_next, ko, qop);
        f32x16_t pr[NKB];
        float ls = softmax_exp_ref<BN>(s_cur, pr, m_run, sl2);
        interleave_exp<D, BN>();
        if (__builtin_amdgcn_ballot_w64(!(ls <= kSumCap)))
          ls = softmax_redo<BN, NACC>(s_cur, pr, oacc, m_run, l_run, c_run, sl2);
        l_run += ls;
        c_run += pack_bf16<BN>(pr, pt);
        pv_regs<DT, D, BN>(oacc, pt, vo);
        interleave_pv<D, BN>();
      } else if constexpr (DT == DT_FP8 && D <= 128) {
        // No row maximum: the probabilities are taken against the reference as it
        // stands, 2^kPExp-scaled.  Their lane sum bounds every one of them, so a sum
        // <= 448 (E4M3's largest value) means they pack without overflow and the
        // reference may stay (it then lags the row maximum by at most
        // log2(448) - kPExp); otherwise -- or with no reference yet -- the tile is
        // redone against its row maximum.  (d = 256 keeps the row maximum: the
        // extra probability tile would spill there.)
        pipe.qk(s_next, kb, qop);
        f32x16_t pr[NKB];
        float ls = softmax_exp_ref<BN>(s_cur, pr, m_run - float(TR::kPExp), sl2);
        if (__builtin_amdgcn_ballot_w64(!(ls <= kFp8Max)))
          ls = softmax_redo<BN, NACC>(s_cur, pr, oacc, m_run, l_run, c_run, sl2, float(TR::kPExp));
        l_run += ls * (1.0f / TR::kPScale);
        pack_fp8<BN>(pr, pt);
        pipe.pv(ov(), s_cur, pt, vb);
        add_psum(pt);
      } else {
        pipe.qk(s_next, kb, qop);
        softmax_tile<DT, BN, NACC>(s_cur, pt, oacc, m_run, l_run, c_run, sl2);
        pipe.pv(ov(), s_cur, pt, vb);
        add_psum(pt);
      }
      finish(kdst, vdst);
    };
    // Remaining tiles: the causal diagonal band, the sequence / chunk tail, the last
    // tile, and the cadence-keeping iterations past the range.
    auto step_edge = [&](int t, uint8_t* kdst, uint8_t* vdst, const uint8_t* kb, const uint8_t* vb,
                         f32x16_t (&s_cur)[NKB], f32x16_t (&s_next)[NKB]) __attribute__((always_inline)) {
      const int k0 = kbeg + t * BN;
      const bool act_cur = active(k0);
      const bool act_next = t + 1 < ntiles && active(k0 + BN);
      pipe.issue_k(ksl, k0 + NS * BN, kdst);
      pipe.issue_v(vsl, k0 + (NS - 1) * BN, vdst);
      if constexpr (P::kRegOps) {
        // bf16: the main loop's lazy softmax (no row maximum unless the reference has
        // to move), with the mask where the tile needs one
        if (act_next) pipe.qk(s_next, kb, qop);
        if (act_cur) {
          if (needs_mask(k0)) mask_tile<BN>(s_cur, k0, kend, row, off, p.causal, g);
          PTile<DT, BN> pt;
          f32x16_t pr[NKB];
          float ls = softmax_exp_ref<BN>(s_cur, pr, m_run, sl2);
          if (__builtin_amdgcn_ballot_w64(!(ls <= kSumCap)))
            ls = softmax_redo<BN, NACC>(s_cur, pr, oacc, m_run, l_run, c_run, sl2);
          l_run += ls;
          c_run += pack_bf16<BN>(pr, pt);
          pipe.pv(ov(), s_cur, pt, vb);
        }
        finish(kdst, vdst);
        return;
      }
      if (act_next) pipe.qk(s_next, kb, qop);
      if (act_cur) {
        if (needs_mask(k0)) mask_tile<BN>(s_cur, k0, kend, row, off, p.causal, g);
        PTile<DT, BN> pt;
        softmax_tile<DT, BN, NACC>(s_cur, pt, oacc, m_run, l_run, c_run, sl2);
        pipe.pv(ov(), s_cur, pt, vb);
        add_psum(pt);
      }
      finish(kdst, vdst);
    };
    // Tiles [0, nfull) are full: below every row's diagonal (causal) and before kend;
    // nfull is rounded down to a multiple of U so that both loops start on stage 0
    // with the first score buffer, unrolled with constant stage indices.  The last tile
    // of the range may be one of them: the S^T its step computes for the next tile then
    // comes from a stage the ring filled with zeros and is never read.
    int nfull = ntiles;
    {
      const int lim_end = (kend - kbeg) / BN;  // tiles ending at or before kend
      nfull = min(nfull, lim_end);
      if (p.causal) {
        // tile t is fully visible to the tile's first row iff k0 + BN - 1 <= q0 + off
        const int d = q0 + off - kbeg - (BN - 1);
        nfull = min(nfull, d < 0 ? 0 : d / BN + 1);
      }
      if (r0 >= p.Sq) nfull = 0;  // wavefronts with no row take the guarded path
      // Both loops pass one barrier per tile, so wavefronts may split at different tiles.
      nfull = nfull < 0 ? 0 : (nfull / U) * U;
    }
    // The full loop runs from tile 0 over a multiple of U tiles, so its unrolled body
    // needs no per-tile bound check.
    auto run = [&](auto full_c, int t0, int t1) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_c)::value;
      for (int t = t0; t < t1; t += U) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
          if (FULL || t + j < t1) {
            uint8_t* kd = kst(j);
            uint8_t* vd = vst(j + NS - 1);
            const uint8_t* kb = kst(j + 1);
            const uint8_t* vb = vst(j);
            if (j % 2 == 0) {
              if constexpr (FULL) step_full(t + j, kd, vd, kb, vb, sa, sb);
              else step_edge(t + j, kd, vd, kb, vb, sa, sb);
            } else {
              if constexpr (FULL) step_full(t + j, kd, vd, kb, vb, sb, sa);
              else step_edge(t + j, kd, vd, kb, vb, sb, sa);
            }
          }
        }
      }
    };
    run(std::true_type{}, 0, nfull);
    run(std::false_type{}, nfull, ntiles);
    // Drain every load before the rings are reused, by this group or the next sweep.
    wait_vmem();
    block_sync();
    }
    take_csum();
  };

  // ---- write-back: deferred normalisation
  auto write_out = [&]() __attribute__((always_inline)) {
    const float l_tot = pair_sum(l_run);
    const float c_tot = pair_sum(c_run);
    if (row >= p.Sq) return;
    const size_t ridx = size_t(bh) * p.Sq + row;
    float* out;
    float sc;
    if constexpr (!SPLIT) {
      out = p.o + ridx * D;
      sc = c_tot > 0.0f ? p.v_scale / (TR::kPScale * c_tot) : 0.0f;
      if (g == 0)
        p.lse[ridx] = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
    } else {
      // u is stored as (l / c) * sum(rounded p * v): u / l is then the chunk's
      // consistent weighted average, while u still equals sum(exp(s - m) v) up to
      // rounding.
      const size_t sidx = size_t(split) * size_t(BH) * p.Sq + ridx;
      out = p.ws_u + sidx * D;
      sc = c_tot > 0.0f ? p.v_scale * l_tot / (TR::kPScale * c_tot) : 0.0f;
      if (g == 0) {
        p.ws_m[sidx] = l_tot > 0.0f ? m_run * kLn2 : -__builtin_inff();
        p.ws_l[sidx] = l_tot;
      }
    }
    if (!SPLIT && p.o_bf16) {
      // the same fp32 values, rounded to bf16 (nearest even) and stored as 8 bytes
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      uint16_t* out16 = reinterpret_cast<uint16_t*>(p.o) + ridx * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x4_t v4 = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2],
                        oacc[db][4 * jj + 3]};
          *reinterpret_cast<u32x2_t*>(out16 + db * 32 + jj * 8 + g * 4) =
              __builtin_bit_cast(u32x2_t, __builtin_convertvector(v4 * sc, bf16x4_t));
        }
      return;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4_t v4 = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2],
                      oacc[db][4 * jj + 3]};
        *reinterpret_cast<f32x4_t*>(out + db * 32 + jj * 8 + g * 4) = v4 * sc;
      }
  };

  // keys of this workgroup's (query tile, chunk)
  int kbeg = 0, kend = p.Sk;
  if (SPLIT) {
    const long long b = (long long)split * p.chunk;
    kbeg = (int)(b < p.Sk ? b : p.Sk);
    const long long e = b + p.chunk;
    kend = (int)(e < p.Sk ? e : p.Sk);
  }
  if constexpr (NG == 1) {
    begin_tile(qt);
    const int kend_q = min(kend, kend_of(qt));
    sweep(kbeg, kend_q, kend_q > kbeg ? ceil_div_i(kend_q - kbeg, BN) : 0);
    write_out();
  } else {
    if constexpr (MODE != kPairs) {
      // Dual: group A takes the first half of the key tiles, B the rest (B's extra
      // iteration, if any, is idle); both end with a partial state of the same tile.
      begin_tile(qt);
      const int kend_q = min(kend, kend_of(qt));
      const int nt = kend_q > kbeg ? ceil_div_i(kend_q - kbeg, BN) : 0;
      const int half = (nt + 1) / 2;
      const int cut = min(kend_q, kbeg + half * BN);
      sweep(grp == 0 ? kbeg : cut, grp == 0 ? cut : kend_q, half);
    } else {
    // Tiles t (lighter) and T (heavier) of the pair, in key tiles of BN.  When nqt is
    // odd the middle tile pairs with itself and the two groups just split its sweep.
    const int t = qt, T = nqt - 1 - qt;
    const int ke_t = kend_of(t), ke_T = kend_of(T);
    const int w_t = t < T ? ceil_div_i(ke_t, BN) : 0;
    const int w_T = ceil_div_i(ke_T, BN);
    // Phase 1: A sweeps tile t, B the first w_t key tiles of T, so that both groups,
    // and all workgroups of the head, stream the keys from 0 in step (one pass through
    // the XCD's L2).  Phase 2: A takes key tiles [w_t, w_t + x) of T and B takes the
    // rest, [w_t + x, w_T), ending on T's diagonal.
    const int mid = w_T - w_t;                  // key tiles of T left after phase 1
    const int x = mid / 2;
    begin_tile(grp == 0 && t < T ? t : T);
    // One sweep call site for both groups and both phases keeps a single copy of the
    // sweep's code, which both groups execute (instruction-cache footprint).
#pragma nounroll
    for (int ph = t < T ? 0 : 1; ph < 2; ++ph) {
      int kb, ke, n;
      if (ph == 0) {
        kb = 0;
        ke = grp == 0 ? ke_t : min(w_t * BN, ke_T);
        n = w_t;
      } else {
        // both groups run mid - x iterations; A's last one may be idle
        kb = (grp == 0 ? w_t : w_t + x) * BN;
        ke = grp == 0 ? (w_t + x) * BN : ke_T;
        n = mid - x;
      }
      sweep(kb, ke, n);
      if (ph == 0 && grp == 0) {
        write_out();
        begin_tile(T);
      }
    }
    }
    // A hands its state of the shared tile to B through LDS (the rings are drained): the
    // 16-byte piece jj of accumulator block db of lane L of wavefront w goes to
    // ks<db>[(jj * 256 + w * 64 + L) * 4] -- consecutive lanes write consecutive 16 bytes,
    // free of bank conflicts -- the running maximum and sums to vs0.
    static_assert(NDB <= NS, "one ring stage array per accumulator block");
    static_assert(P::STAGE_K * NG >= kWaves * 64 * 16 * 4, "stage array holds a block");
    float* hand_m = reinterpret_cast<float*>(vs0);
    const int slot = wave * 64 + lane;
    if (grp == 0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        float* dst = reinterpret_cast<float*>(db == 0 ? ks0 : db == 1 ? ks1 : db == 2 ? ks2 : ks3) + slot * 4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x4_t v4 = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2],
                        oacc[db][4 * jj + 3]};
          *reinterpret_cast<f32x4_t*>(dst + jj * (kWaves * 64 * 4)) = v4;
        }
      }
      hand_m[slot * 3 + 0] = m_run;
      hand_m[slot * 3 + 1] = l_run;
      hand_m[slot * 3 + 2] = c_run;
    }
    block_sync();
    if (grp == 1) {
      const float ma = hand_m[slot * 3 + 0];
      const float la = hand_m[slot * 3 + 1];
      const float ca = hand_m[slot * 3 + 2];
      const float mn = __builtin_fmaxf(ma, m_run);
      const float wa = ma == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(ma - mn);
      const float wb = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const float* src = reinterpret_cast<const float*>(db == 0 ? ks0 : db == 1 ? ks1 : db == 2 ? ks2 : ks3) + slot * 4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(src + jj * (kWaves * 64 * 4));
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[db][4 * jj + e] = wa * v4[e] + wb * oacc[db][4 * jj + e];
        }
      }
      l_run = wa * la + wb * l_run;
      c_run = wa * ca + wb * c_run;
      m_run = mn;
      write_out();
    }
  }
}


// ------------------------------------------------------------------ merge kernel
// One workgroup of 256 threads per row.  Thread t owns the 16-byte column chunk t % CH
// (CH = D/4 chunks per row) for the splits s = t / CH, t / CH + NG, ... (NG = 256 / CH
// split groups).  Each thread merges its splits in one pass with a running maximum --
// the merge of the split-K section of "AI 大模型之 FlashAttention_02" applied one chunk
// at a time (rescale what is accumulated by exp(m_old - m_new) when the maximum moves) --
// so all of a row's state loads are independent and in flight together; the NG group
// states are then combined in LDS in a fixed order (the result does not depend on
// timing).
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_merge_kernel(MergeArgs a) {
  constexpr int CH = D / 4;
  constexpr int NG = 256 / CH;
  __shared__ f32x4_t part_u[NG][CH];
  __shared__ float part_m[NG];
  __shared__ float part_l[NG];
  const int tid = threadIdx.x;
  const int ch = tid % CH, grp = tid / CH;
  const int n = a.num_splits;
  // grid-stride over rows (the grid is capped); the loop bound is uniform per workgroup
  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    float Mt = -__builtin_inff(), Lt = 0.0f;  // natural-log units, as stored
    f32x4_t Ut = {0.f, 0.f, 0.f, 0.f};
    for (int s = grp; s < n; s += NG) {
      const int64_t i = int64_t(s) * a.rows + row;
      const float m = a.ws_m[i];
      const float l = a.ws_l[i];
      const f32x4_t u = *reinterpret_cast<const f32x4_t*>(a.ws_u + i * D + ch * 4);
      if (m == -__builtin_inff()) continue;  // empty chunk: neutral
      if (m > Mt) {
        const float c = Mt == -__builtin_inff() ? 0.0f : expf(Mt - m);
        Lt *= c;
        Ut *= c;
        Mt = m;
      }
      const float w = expf(m - Mt);
      Lt += w * l;
      Ut += w * u;
    }
    part_u[grp][ch] = Ut;
    if (ch == 0) {
      part_m[grp] = Mt;
      part_l[grp] = Lt;
    }
    __syncthreads();
    if (grp == 0) {
      float M = part_m[0];
#pragma unroll
      for (int gi = 1; gi < NG; ++gi) M = __builtin_fmaxf(M, part_m[gi]);
      float L = 0.0f;
      f32x4_t U = {0.f, 0.f, 0.f, 0.f};
      if (M != -__builtin_inff()) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const float mg = part_m[gi];
          const float w = mg == -__builtin_inff() ? 0.0f : expf(mg - M);
          L += w * part_l[gi];
          U += w * part_u[gi][ch];
        }
      }
      const bool empty = !(L > 0.0f);
      const float inv = empty ? 0.0f : 1.0f / L;
      *reinterpret_cast<f32x4_t*>(a.o + row * D + ch * 4) = U * inv;
      if (ch == 0) a.lse[row] = empty ? -__builtin_inff() : M + logf(L);
    }
    __syncthreads();  // part_* are reused by the next row
  }
}

template <int DT, int D>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  constexpr int BN = block_n(DT, D), BN2 = block_n_two_groups(DT, D);
  const int64_t nqt = (a.Sq + kBlockM - 1) / kBlockM;
  if constexpr (pairs_supported(DT, D)) {
    if (a.pair_order == 2 && !a.split_mode && a.causal) {
      const int64_t nwg = int64_t(a.B) * a.H * ((nqt + 1) / 2);
      hipLaunchKernelGGL((attn_fwd_kernel<DT, D, BN2, kPairs>), dim3(unsigned(nwg)), dim3(2 * kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  const int64_t nwg = int64_t(a.B) * a.H * nqt * a.num_splits;
  if constexpr (dual_supported(DT, D)) {
    if (a.pair_order == 3) {
      if (a.split_mode)
        hipLaunchKernelGGL((attn_fwd_kernel<DT, D, BN2, kDualSplit>), dim3(unsigned(nwg)), dim3(2 * kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((attn_fwd_kernel<DT, D, BN2, kDualPlain>), dim3(unsigned(nwg)), dim3(2 * kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (DT == DT_BF16 && D == 64) {
    if (a.chunk > kShortSweep) {  // long sweeps: 64-key tiles, two workgroups per CU
      if (a.split_mode)
        hipLaunchKernelGGL((attn_fwd_kernel<DT, D, 64, kSplit>), dim3(unsigned(nwg)), dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((attn_fwd_kernel<DT, D, 64, kPlain>), dim3(unsigned(nwg)), dim3(kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.split_mode)
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, BN, kSplit>), dim3(unsigned(nwg)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, BN, kPlain>), dim3(unsigned(nwg)), dim3(kThreads), 0, s, a);
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


// ================================================================== backward
// Gradients of exact attention with the probabilities recomputed from the forward's
// lse, never stored: per (batch, head), with S = scale Q K^T masked as in the forward,
//
//   P = exp(S - lse),  dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  D_i = sum_d dO_id O_id,
//   dQ = scale dS K,   dK = scale dS^T Q.
//
// dK and dV sum over queries and dQ over keys -- the "AI 大模型之 FlashAttention_02"
// page, section "Training and deployment: backward consistency of split and reduction",
// notes that the backward reduces across queries, the other direction from the forward.
// Each sum stays inside one workgroup, so there are no atomics and the result does not
// depend on timing:
//
//   attn_bwd_pre_kernel   per query row: D, dO rounded to bf16, lse in log2 units;
//   attn_bwd_dkdv_kernel  one workgroup per 128 keys (four wavefronts of 32 keys, each
//                         key in a lane position like a query row of the forward),
//                         sweeping the query tiles of 32 rows that see those keys;
//   attn_bwd_dq_kernel    one workgroup per 128 query rows, sweeping the visible key
//                         tiles of 32, the forward's layout.
//
// Every product is a 32x32x16 bf16 MFMA with fp32 accumulation; P and dS are rounded
// to bf16 as MFMA operands.  Tiles reach LDS by direct loads into two stages, each tile
// once in the key-operand layout (rows read as the A operand) and, where its transpose
// is needed, once more in the value-operand layout (read with ds_read_b64_tr_b16).

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_bwd_pre_kernel(BwdArgs a) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  constexpr int TPR = D / 4;       // threads per row, four elements each
  constexpr int RPB = 256 / TPR;   // rows per workgroup pass
  const int64_t rows = int64_t(a.B) * a.H * a.Sq;
  const int t = threadIdx.x % TPR;
  // grid-stride over rows; the TPR threads of a row stay together
  for (int64_t r = int64_t(blockIdx.x) * RPB + threadIdx.x / TPR; r < rows;
       r += int64_t(gridDim.x) * RPB) {
    const f32x4_t o4 = *reinterpret_cast<const f32x4_t*>(a.o + r * D + t * 4);
    const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(a.dout + r * D + t * 4);
    float dot = o4[0] * d4[0] + o4[1] * d4[1] + o4[2] * d4[2] + o4[3] * d4[3];
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, TPR);
    *reinterpret_cast<bf16x4_t*>(a.do16 + r * D + t * 4) = __builtin_convertvector(d4, bf16x4_t);
    if (t == 0) {
      a.dsum[r] = dot;
      const float l = a.lse[r];
      a.lse2[r] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
    }
  }
}

// 64 consecutive floats from row i0 of a per-row buffer straight into LDS (lane L's at
// dst[L]; rows past the buffer read as zeros).
__device__ __forceinline__ void dma_floats(__amdgpu_buffer_rsrc_t rs, float* dst, int i0, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 4, (i0 + lane) * 4, 0, 0, 0);
}

__device__ __forceinline__ void pack_tile(const float (&x)[16], PTile<DT_BF16, 32>& pt) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x8_t v = {x[8 * h + 0], x[8 * h + 1], x[8 * h + 2], x[8 * h + 3],
                 x[8 * h + 4], x[8 * h + 5], x[8 * h + 6], x[8 * h + 7]};
    pt.pk[0][h] = __builtin_convertvector(v, bf16x8_t);
  }
}

// Rows of a 32-row block of an output [S][D] from an accumulator X^T (d x rows) held in
// the 32x32 layout: lane (c, g) writes row r0 + c, columns 32*db + 8*jj + 4*g + 0..3.
template <int D>
__device__ __forceinline__ void store_rows(float* out, int r0, int nrows, int c, int g,
                                           const f32x16_t (&acc)[D / 32], float mul) {
  if (r0 + c >= nrows) return;
  float* dst = out + size_t(r0 + c) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4_t v4 = {acc[db][4 * jj + 0], acc[db][4 * jj + 1], acc[db][4 * jj + 2],
                          acc[db][4 * jj + 3]};
      *reinterpret_cast<f32x4_t*>(dst + db * 32 + jj * 8 + g * 4) = v4 * mul;
    }
}

// dV^T and dK^T accumulation of the d = 256 dK/dV kernel.  Its two accumulators (8
// blocks of 16 registers each) fill all 256 accumulation registers, so their MFMAs name
// that register class (inline asm, "+a"); the library is built with MFMA results in VGPRs
// by default, so S and dP stay in the 256 VGPRs.  (Left to itself the compiler put S and
// dP among the accumulators and spilled 154 registers per lane, or, with the accumulators
// pinned, moved two accumulator blocks out and back every tile.)  The compiler does not
// see these instructions as MFMAs, so it inserts none of their hazard waits: each one
// starts with the two wait states a VALU write of its A or B operand needs, and nothing
// else reads or writes the accumulators between agpr_settle calls -- the zeroing before
// the sweep and the reads of the write-back each sit behind one, which waits out the
// MFMA pipeline.  Within the sweep an accumulator block is read again as the MFMA's C
// operand only 7 MFMAs later.
__device__ __forceinline__ void mfma_bf16_agpr(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int N>
__device__ __forceinline__ void agpr_settle(f32x16_t (&x)[N], f32x16_t (&y)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15" : "+a"(x[0]));  // 32 wait states
#pragma unroll
  for (int i = 0; i < N; ++i) {
    asm volatile("" : "+a"(x[i]));
    asm volatile("" : "+a"(y[i]));
  }
}
template <int N>
__device__ __forceinline__ void agpr_settle1(f32x16_t (&x)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15" : "+a"(x[0]));  // 32 wait states
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(x[i]));
}
// pv_dma (bf16) with the accumulation in mfma_bf16_agpr.
template <int D>
__device__ __forceinline__ void pv_dma_agpr(f32x16_t (&oacc)[D / 32], const PTile<DT_BF16, 32>& pt,
                                            const uint8_t* vt, const DmaLane<DT_BF16, D, 32>& ln) {
  using G = DmaGeo<DT_BF16, D, 32>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x8_t pb = pt.pk[0][h];
    const int roff = h * 16 * G::ROWB;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dx = db << 6;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vt + roff + (ln.vx[0] ^ dx)));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vt + roff + (ln.vx[1] ^ dx)));
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      const i16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      mfma_bf16_agpr(oacc[db], __builtin_bit_cast(bf16x8_t, both), pb);
    }
  }
}

// Row-operand offset into a tile stored in the value layout: lane (c, g) reads 16-byte
// chunk 2*ks + g of row c as `tile + (x ^ (ks << 5))`, the same access the key layout
// gives with DmaLane::kx, so one copy of a tile serves both its row reads and its
// transposed reads.
template <int D>
__device__ __forceinline__ int row_lane_offset_vlayout(int lane) {
  constexpr int ROWB = D * 2;
  const int c = lane & 31, g = lane >> 5;
  return c * ROWB + ((g ^ swz_v<DT_BF16, ROWB>(c)) << 4);
}

// One 32x32 block of X Y^T from two LDS tiles read as rows: X rows from `xt` (value
// layout, lane offset xv) as the A operand, Y rows from `yt` (key layout, lane offset ky)
// as the B operand.
template <int D>
__device__ __forceinline__ f32x16_t rows_product_lds(const uint8_t* xt, int xv, const uint8_t* yt, int ky) {
  using Op = Traits<DT_BF16>::Op;
  f32x16_t acc = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const Op a = *reinterpret_cast<const Op*>(xt + (xv ^ (ks << 5)));
    const Op b = *reinterpret_cast<const Op*>(yt + (ky ^ (ks << 5)));
    acc = Traits<DT_BF16>::mfma(a, b, acc);
  }
  return acc;
}

// Same with the B operand already in registers.
template <int D>
__device__ __forceinline__ f32x16_t rows_product_reg(const uint8_t* xt, int xv,
                                                     const Traits<DT_BF16>::Op (&b)[D / 16]) {
  using Op = Traits<DT_BF16>::Op;
  f32x16_t acc = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    acc = Traits<DT_BF16>::mfma(*reinterpret_cast<const Op*>(xt + (xv ^ (ks << 5))), b[ks], acc);
  return acc;
}

// dK and dV of 128 keys per workgroup.  Each wavefront's 32 keys sit in lane position;
// their K rows stay in registers (B operand of S = Q K^T) and their V rows in an LDS
// block loaded once (B operand of dP = dO V^T).  Query tiles of 32 rows stream through
// two LDS stages, Q and dO each stored once in the value layout: read as rows for S and
// dP, transposed for dK^T += Q^T dS and dV^T += dO^T P.  Two workgroups fit a CU (LDS
// and 256 registers per wavefront).  Causal: key tile kt sees the queries from
// kt*128 - (Sk - Sq) on, so workgroups i and i + grid/2, which share a CU, take
// complementary key tiles.
// Wavefronts per SIMD of the backward kernels: the products of one tile form one dependent
// chain per wavefront, so more wavefronts per SIMD fill more of its gaps.  At d = 64 the
// dK/dV kernel fits three in the register file (at most 168 registers; 33 KB of LDS per
// workgroup) and the dQ kernel four (128 registers, 24 KB); d = 128 two (three would spill
// in dQ), d = 256 one.
constexpr int bwd_waves(int d, bool dq) { return d >= 256 ? 1 : d == 64 ? (dq ? 4 : 3) : 2; }

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(bwd_waves(D, false), bwd_waves(D, false))))
void attn_bwd_dkdv_kernel(BwdArgs a) {
  using Op = Traits<DT_BF16>::Op;
  using G = DmaGeo<DT_BF16, D, 32>;
  constexpr int KSTEPS = D / 16;
  constexpr int NDB = D / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  // Work items, longest sweeps first: the two halves of each long key tile merged with
  // the other key tiles by sweep length (without long tiles: the key tiles in order, which
  // is the same rule).
  const int item = blockIdx.x / BH;
  const int L = a.long_tiles;
  int kt = item, part = -1;  // part -1: the whole sweep; 0 / 1: its first / second half
  if (L > 0) {
    const int nkt = ceil_div_i(a.Sk, kBlockM);
    int hi = 0, pj = 0;
    bwd_item(item, L, nkt - L,
             [&](int i) { return (bwd_query_tiles(a.Sq, a.Sk, i, 1) + 1) / 2; },
             [&](int j) { return bwd_query_tiles(a.Sq, a.Sk, L + j, 1); }, &hi, &pj);
    kt = hi >= 0 ? hi : L + pj;
    part = hi >= 0 ? pj : -1;
  }
  const int kw0 = kt * kBlockM + wave * 32;  // first key of this wavefront
  const int key = kw0 + c;                   // this lane's key
  const int off = a.Sk - a.Sq;
  const float sl2 = a.scale_log2;

  const size_t qo = size_t(bh) * a.Sq, ko = size_t(bh) * a.Sk;
  const auto rq = make_rsrc(reinterpret_cast<const uint8_t*>(a.q) + qo * D * 2, uint32_t(a.Sq) * D * 2);
  const auto rdo = make_rsrc(a.do16 + qo * D, uint32_t(a.Sq) * D * 2);
  const auto rk = make_rsrc(reinterpret_cast<const uint8_t*>(a.k) + ko * D * 2, uint32_t(a.Sk) * D * 2);
  const auto rv = make_rsrc(reinterpret_cast<const uint8_t*>(a.v) + ko * D * 2, uint32_t(a.Sk) * D * 2);
  const auto rl = make_rsrc(a.lse2 + qo, uint32_t(a.Sq) * 4);
  const auto rd = make_rsrc(a.dsum + qo, uint32_t(a.Sq) * 4);

  Op kop[KSTEPS];  // this wavefront's keys, B operand of S (zeros past Sk)
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    kop[ks] = __builtin_bit_cast(Op, __builtin_amdgcn_raw_buffer_load_b128(rk, (key * D + ks * 16 + g * 8) * 2, 0, 0));
  f32x16_t dkt[NDB], dvt[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dkt[i] = f32x16_t{};
    dvt[i] = f32x16_t{};
  }
  constexpr bool kAgpr = D >= 256;  // accumulators pinned to the accumulation registers
  if constexpr (kAgpr) agpr_settle(dkt, dvt);
  Pipe<DT_BF16, D, 32, kWaves> pipe(wave, lane);  // direct-to-LDS tile loads
  const DmaLane<DT_BF16, D, 32>& ln = pipe.ln;
  const int xv = row_lane_offset_vlayout<D>(lane);

  // the workgroup's V rows (key layout), then two stages of {Q, dO} (value layout)
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[G::TILE], vb1[G::TILE], vb2[G::TILE], vb3[G::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t q0s[G::TILE], o0s[G::TILE], q1s[G::TILE], o1s[G::TILE];
  __shared__ __attribute__((aligned(256))) float ls0[64], ds0[64], ls1[64], ds1[64];
  const uint8_t* vmine = wave == 0 ? vb0 : wave == 1 ? vb1 : wave == 2 ? vb2 : vb3;

  int ibeg = a.causal ? (max(0, kt * kBlockM - off) / 32) * 32 : 0;
  int ntiles = ibeg < a.Sq ? ceil_div_i(a.Sq - ibeg, 32) : 0;
  if (part >= 0) {  // first or second half of the query tiles
    const int h = (ntiles + 1) / 2;
    if (part == 1) ibeg += h * 32;
    ntiles = part == 0 ? h : ntiles - h;
  }

  auto issue = [&](int i0, uint8_t* qs, uint8_t* os, float* ls, float* ds) __attribute__((always_inline)) {
    pipe.issue_v(rq, i0, qs);
    pipe.issue_v(rdo, i0, os);
    if (wave == 0) dma_floats(rl, ls, i0, lane);
    if (wave == 1) dma_floats(rd, ds, i0, lane);
  };
  auto compute = [&](int i0, const uint8_t* qs, const uint8_t* os, const float* ls, const float* ds)
      __attribute__((always_inline)) {
    const f32x16_t st = rows_product_reg<D>(qs, xv, kop);              // S  [query][key]
    const f32x16_t dp = rows_product_lds<D>(os, xv, vmine, ln.kx);     // dP [query][key]
    float pv[16], sv[16];
    // every (query, key) pair of this wavefront's block visible: no per-element test
    const bool full = i0 + 32 <= a.Sq && kw0 + 32 <= a.Sk && (!a.causal || kw0 + 31 <= i0 + off);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(ls + 8 * b + 4 * g);
      const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(ds + 8 * b + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * b + r;
        const int i = i0 + 8 * b + 4 * g + r;
        const bool vis = full || (i < a.Sq && key < a.Sk && (!a.causal || key <= i + off));
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[e], sl2, -l4[r])) : 0.0f;
        pv[e] = p;
        sv[e] = p * (dp[e] - d4[r]);
      }
    }
    PTile<DT_BF16, 32> pp, ps;
    pack_tile(pv, pp);
    pack_tile(sv, ps);
    if constexpr (kAgpr) {
      pv_dma_agpr<D>(dvt, pp, os, ln);
      pv_dma_agpr<D>(dkt, ps, qs, ln);
    } else {
      pv_dma<DT_BF16, D, 32>(dvt, pp, os, ln);  // dV^T += dO^T P
      pv_dma<DT_BF16, D, 32>(dkt, ps, qs, ln);  // dK^T += Q^T dS
    }
  };

#pragma unroll
  for (int i = 0; i < 4; ++i)
    pipe.issue_k(rv, kt * kBlockM + 32 * i, i == 0 ? vb0 : i == 1 ? vb1 : i == 2 ? vb2 : vb3);
  if (ntiles > 0) issue(ibeg, q0s, o0s, ls0, ds0);
  wait_vmem();
  block_sync();
  for (int t = 0; t < ntiles; t += 2) {
    const int i0 = ibeg + t * 32;
    if (t + 1 < ntiles) issue(i0 + 32, q1s, o1s, ls1, ds1);
    compute(i0, q0s, o0s, ls0, ds0);
    wait_vmem();
    block_sync();
    if (t + 1 < ntiles) {
      if (t + 2 < ntiles) issue(i0 + 64, q0s, o0s, ls0, ds0);
      compute(i0 + 32, q1s, o1s, ls1, ds1);
      wait_vmem();
      block_sync();
    }
  }
  if constexpr (kAgpr) agpr_settle(dkt, dvt);
  if (part == 1) {  // second half: to the workspace, added by attn_bwd_combine_kernel
    const size_t po = size_t(bh) * size_t(L) * kBlockM;
    store_rows<D>(a.pdk + po * D, kw0, a.Sk, c, g, dkt, a.scale);
    store_rows<D>(a.pdv + po * D, kw0, a.Sk, c, g, dvt, 1.0f);
  } else {
    store_rows<D>(a.dk + ko * D, kw0, a.Sk, c, g, dkt, a.scale);
    store_rows<D>(a.dv + ko * D, kw0, a.Sk, c, g, dvt, 1.0f);
  }
}

// dK, dV of the split key tiles and dQ of the split query tiles: first half (already in
// place) + second half (workspace), in that order, so the sum does not depend on timing.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_bwd_combine_kernel(BwdArgs a) {
  // the long query tiles are the last ones: rows [q_first, Sq) of every (batch, head)
  const int q_first = (ceil_div_i(a.Sq, kBlockM) - a.long_qtiles) * kBlockM;
  const int qrows = a.Sq - q_first;
  const int64_t m4 = a.long_qtiles > 0 ? int64_t(a.B) * a.H * qrows * (D / 4) : 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < m4; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / (D / 4), col = (i % (D / 4)) * 4;
    const int64_t bh = r / qrows, qr = r % qrows;
    const size_t o = size_t(bh * a.Sq + q_first + qr) * D + col;
    const size_t w = size_t(bh * int64_t(a.long_qtiles) * kBlockM + qr) * D + col;
    *reinterpret_cast<f32x4_t*>(a.dq + o) += *reinterpret_cast<const f32x4_t*>(a.pdq + w);
  }
}

// dK and dV of the long key tiles: the first half's (in dk, dv) plus the second half's
// (pdk, pdv), in that order.  The dQ launch runs this in the workgroups past its own
// items: the dispatcher starts them last, on the CUs the shortest dQ sweeps leave idle,
// and the dK/dV launch before it has finished both halves.  Each thread keeps kCombineU
// elements' loads in flight at once.
constexpr int kCombineU = 4;
template <int D>
__device__ __forceinline__ void combine_kv(const BwdArgs& a, int64_t first, int64_t stride) {
  const int rows = min(a.Sk, a.long_tiles * kBlockM);  // per (batch, head)
  const int64_t n4 = int64_t(a.B) * a.H * rows * (D / 4);
  for (int64_t base = first; base < n4; base += stride * kCombineU) {
    f32x4_t k0[kCombineU], k1[kCombineU], v0[kCombineU], v1[kCombineU];
    size_t oo[kCombineU];
#pragma unroll
    for (int j = 0; j < kCombineU; ++j) {
      const int64_t i = base + j * stride;
      if (i < n4) {
        const int64_t r = i / (D / 4), col = (i % (D / 4)) * 4;
        const int64_t bh = r / rows, kr = r % rows;
        oo[j] = size_t(bh * a.Sk + kr) * D + col;
        const size_t w = size_t(bh * int64_t(a.long_tiles) * kBlockM + kr) * D + col;
        k0[j] = *reinterpret_cast<const f32x4_t*>(a.dk + oo[j]);
        k1[j] = *reinterpret_cast<const f32x4_t*>(a.pdk + w);
        v0[j] = *reinterpret_cast<const f32x4_t*>(a.dv + oo[j]);
        v1[j] = *reinterpret_cast<const f32x4_t*>(a.pdv + w);
      }
    }
#pragma unroll
    for (int j = 0; j < kCombineU; ++j) {
      if (base + j * stride < n4) {
        *reinterpret_cast<f32x4_t*>(a.dk + oo[j]) = k0[j] + k1[j];
        *reinterpret_cast<f32x4_t*>(a.dv + oo[j]) = v0[j] + v1[j];
      }
    }
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(bwd_waves(D, true), bwd_waves(D, true))))
void attn_bwd_dq_kernel(BwdArgs a) {
  using Op = Traits<DT_BF16>::Op;
  using G = DmaGeo<DT_BF16, D, 32>;
  constexpr int KSTEPS = D / 16;
  constexpr int NDB = D / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = ceil_div_i(a.Sq, kBlockM);
  const int LQ = a.long_qtiles;
  const int nitems = BH * (nqt + LQ);
  if (int(blockIdx.x) >= nitems) {  // the dK/dV combine workgroups (before any barrier)
    combine_kv<D>(a, int64_t(int(blockIdx.x) - nitems) * 256 + tid,
                  int64_t(int(gridDim.x) - nitems) * 256);
    return;
  }
  const int bh = blockIdx.x % BH;
  const int item = blockIdx.x / BH;
  int qt = item, part = -1;  // part -1: the whole sweep; 0 / 1: its first / second half
  if (LQ > 0) {
    // Longest items first: the two halves of each long (last) query tile merged with the
    // other tiles by sweep length.
    int hi = 0, pj = 0;
    bwd_item(item, LQ, nqt - LQ,
             [&](int i) { return (bwd_key_tiles(a.Sq, a.Sk, nqt - 1 - i, 1) + 1) / 2; },
             [&](int j) { return bwd_key_tiles(a.Sq, a.Sk, nqt - 1 - LQ - j, 1); }, &hi, &pj);
    qt = hi >= 0 ? nqt - 1 - hi : nqt - 1 - LQ - pj;
    part = hi >= 0 ? pj : -1;
  } else if (a.causal) {  // longest (last) query tiles first
    qt = nqt - 1 - qt;
  }
  const int r0 = qt * kBlockM + wave * 32;
  const int row = r0 + c;  // this lane's query row
  const int off = a.Sk - a.Sq;
  const float sl2 = a.scale_log2;

  const size_t qo = size_t(bh) * a.Sq, ko = size_t(bh) * a.Sk;
  const auto rq = make_rsrc(reinterpret_cast<const uint8_t*>(a.q) + qo * D * 2, uint32_t(a.Sq) * D * 2);
  const auto rdo = make_rsrc(a.do16 + qo * D, uint32_t(a.Sq) * D * 2);
  const auto rk = make_rsrc(reinterpret_cast<const uint8_t*>(a.k) + ko * D * 2, uint32_t(a.Sk) * D * 2);
  const auto rv = make_rsrc(reinterpret_cast<const uint8_t*>(a.v) + ko * D * 2, uint32_t(a.Sk) * D * 2);

  Op qop[KSTEPS], dop[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int boff = (row * D + ks * 16 + g * 8) * 2;
    qop[ks] = __builtin_bit_cast(Op, __builtin_amdgcn_raw_buffer_load_b128(rq, boff, 0, 0));
    dop[ks] = __builtin_bit_cast(Op, __builtin_amdgcn_raw_buffer_load_b128(rdo, boff, 0, 0));
  }
  const float l2 = row < a.Sq ? a.lse2[qo + row] : __builtin_inff();
  const float dd = row < a.Sq ? a.dsum[qo + row] : 0.0f;
  f32x16_t dqt[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqt[i] = f32x16_t{};
  constexpr bool kAgpr = D >= 256;  // accumulators pinned to the accumulation registers
  if constexpr (kAgpr) agpr_settle1(dqt);
  Pipe<DT_BF16, D, 32, kWaves> pipe(wave, lane);  // direct-to-LDS tile loads
  const DmaLane<DT_BF16, D, 32>& ln = pipe.ln;

  // three stages of {K (value layout), V (key layout)}: tile t+2 is requested while tile t
  // is computed, so a tile's loads have two iterations to land
  __shared__ __attribute__((aligned(1024))) uint8_t kv0[G::TILE], vk0[G::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kv1[G::TILE], vk1[G::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kv2[G::TILE], vk2[G::TILE];
  const int xv = row_lane_offset_vlayout<D>(lane);
  constexpr int LPT = 2 * (G::TILE / 1024 / kWaves);  // loads per wavefront per tile

  int kend = a.Sk;
  if (a.causal) {
    const int last_row = min((qt + 1) * kBlockM, a.Sq) - 1;
    kend = max(0, min(a.Sk, last_row + off + 1));
  }
  // this item's key tiles [kt0, kt0 + ntiles)
  const int nall = ceil_div_i(kend, 32);
  const int kt0 = part == 1 ? nall / 2 : 0;
  const int ntiles = part == 0 ? nall / 2 : nall - kt0;

  auto kvst = [&](int j) __attribute__((always_inline)) -> uint8_t* {
    return j % 3 == 0 ? kv0 : j % 3 == 1 ? kv1 : kv2;
  };
  auto vkst = [&](int j) __attribute__((always_inline)) -> uint8_t* {
    return j % 3 == 0 ? vk0 : j % 3 == 1 ? vk1 : vk2;
  };
  auto issue = [&](int k0, uint8_t* kv, uint8_t* vk) __attribute__((always_inline)) {
    pipe.issue_v(rk, k0, kv);
    pipe.issue_k(rv, k0, vk);
  };
  auto compute = [&](int k0, const uint8_t* kv, const uint8_t* vk) __attribute__((always_inline)) {
    const f32x16_t st = rows_product_reg<D>(kv, xv, qop);  // S^T  [key][query]
    f32x16_t dpt[1];
    qk_dma<DT_BF16, D, 32>(dpt, vk, dop, ln);              // dP^T [key][query]
    float sv[16];
    // every (key, query) pair of this wavefront's block visible: no per-element test
    const bool full = k0 + 32 <= kend && r0 + 32 <= a.Sq && (!a.causal || k0 + 31 <= r0 + off);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kj = k0 + 8 * (e >> 2) + 4 * g + (e & 3);
      const bool vis = full || (kj < kend && row < a.Sq && (!a.causal || kj <= row + off));
      const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[e], sl2, -l2)) : 0.0f;
      sv[e] = p * (dpt[0][e] - dd);
    }
    PTile<DT_BF16, 32> ps;
    pack_tile(sv, ps);
    if constexpr (kAgpr) pv_dma_agpr<D>(dqt, ps, kv, ln);  // dQ^T += K^T dS^T
    else pv_dma<DT_BF16, D, 32>(dqt, ps, kv, ln);
  };

  const int kb = kt0 * 32;  // first key of the sweep
  if (ntiles > 0) issue(kb, kv0, vk0);
  if (ntiles > 1) issue(kb + 32, kv1, vk1);
  // loads complete in order: with tile 1 in flight, at most its LPT loads remain
  if (ntiles > 1) wait_vmcnt<LPT>(); else wait_vmem();
  block_sync();
  for (int t = 0; t < ntiles; t += 3) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int tt = t + j;
      if (tt < ntiles) {
        if (tt + 2 < ntiles) issue(kb + (tt + 2) * 32, kvst(j + 2), vkst(j + 2));
        compute(kb + tt * 32, kvst(j), vkst(j));
        // tile tt+1 has landed once only tile tt+2's loads (if any) are in flight
        if (tt + 2 < ntiles) wait_vmcnt<LPT>(); else wait_vmem();
        block_sync();
      }
    }
  }
  if constexpr (kAgpr) agpr_settle1(dqt);
  if (part == 1) {  // second half: to the workspace, added by attn_bwd_combine_kernel
    const int q_first = (nqt - LQ) * kBlockM;  // first row of the long tiles
    store_rows<D>(a.pdq + size_t(bh) * size_t(LQ) * kBlockM * D, r0 - q_first, a.Sq - q_first, c, g, dqt,
                  a.scale);
  } else {
    store_rows<D>(a.dq + qo * D, r0, a.Sq, c, g, dqt, a.scale);
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = int64_t(a.B) * a.H * a.Sq;
  constexpr int RPB = 256 / (D / 4);
  const int64_t pre = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL(attn_bwd_pre_kernel<D>, dim3(unsigned(pre < 65536 ? pre : 65536)), dim3(256), 0, s, a);
  const int64_t nkv = int64_t(a.B) * a.H * ((a.Sk + kBlockM - 1) / kBlockM + a.long_tiles);
  if (nkv > 0) hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3(unsigned(nkv)), dim3(kThreads), 0, s, a);
  const int64_t nq = int64_t(a.B) * a.H * ((a.Sq + kBlockM - 1) / kBlockM + a.long_qtiles);
  // dK/dV of the split key tiles are combined by workgroups appended to the dQ grid (one
  // per kCombineU x 256 elements, at most 512); the dQ halves by one pass after it.
  int64_t ncomb = 0;
  if (a.long_tiles > 0) {
    const int64_t zr = int64_t(a.long_tiles) * kBlockM < a.Sk ? int64_t(a.long_tiles) * kBlockM : a.Sk;
    const int64_t n4 = int64_t(a.B) * a.H * zr * (D / 4);
    ncomb = (n4 + 256 * kCombineU - 1) / (256 * kCombineU);
    ncomb = ncomb < 512 ? ncomb : 512;
  }
  if (nq > 0) hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3(unsigned(nq + ncomb)), dim3(kThreads), 0, s, a);
  if (a.long_qtiles > 0) {
    const int64_t qf = ((a.Sq + kBlockM - 1) / kBlockM - a.long_qtiles) * int64_t(kBlockM);
    const int64_t n4 = int64_t(a.B) * a.H * (a.Sq - qf) * (D / 4);
    const int64_t nb = (n4 + 255) / 256;
    hipLaunchKernelGGL(attn_bwd_combine_kernel<D>, dim3(unsigned(nb < 65536 ? nb : 65536)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
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
  const dim3 grid(unsigned(a.rows < (int64_t(1) << 20) ? a.rows : (int64_t(1) << 20)));
  switch (a.d) {
    case 64: hipLaunchKernelGGL(attn_merge_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_merge_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(attn_merge_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

int launch_bwd(const BwdArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (a.d) {
    case 64: return int(launch_bwd_d<64>(a, s));
    case 128: return int(launch_bwd_d<128>(a, s));
    case 256: return int(launch_bwd_d<256>(a, s));
  }
  return int(hipErrorInvalidValue);
}

const char* bwd_kernel_name(int d, int which) {
  static const char* names[3][4] = {
      {"attn_bwd_pre_d64", "attn_bwd_dkdv_bf16_d64_bn128_bm32", "attn_bwd_dq_bf16_d64_bm128_bn32", "attn_bwd_combine_d64"},
      {"attn_bwd_pre_d128", "attn_bwd_dkdv_bf16_d128_bn128_bm32", "attn_bwd_dq_bf16_d128_bm128_bn32", "attn_bwd_combine_d128"},
      {"attn_bwd_pre_d256", "attn_bwd_dkdv_bf16_d256_bn128_bm32", "attn_bwd_dq_bf16_d256_bm128_bn32", "attn_bwd_combine_d256"}};
  if ((d != 64 && d != 128 && d != 256) || which < 0 || which > 3) return "";
  return names[d == 64 ? 0 : d == 128 ? 1 : 2][which];
}

// ------------------------------------------------------------------ static scratch
// Workspace of attn_fwd_splitkv_noalloc (for callers that cannot allocate): a fixed
// device array, one copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in, never a device address: kernels get the
// address hipGetSymbolAddress returns for the current device.
__device__ __align__(256) static uint8_t scratch[kNoallocScratchBytes];

void* noalloc_scratch(int* hip_err) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= 64)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *hip_err = int(e);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current: its own copy of the array
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *hip_err = int(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = n;
  return n;
}

const char* fwd_kernel_name(int dtype, int d, int split_mode, int sched, int sweep_keys) {
  if (sched == 2 && pairs_supported(dtype, d))
    return d == 64 ? "attn_fwd_causal_pairs_bf16_d64_bm256_bn64" : "attn_fwd_causal_pairs_bf16_d128_bm256_bn32";
  if (sched == 3 && dual_supported(dtype, d)) {
    if (dtype == DT_FP8)
      return split_mode ? "attn_fwd_splitkv_dual_fp8_d128_bm128_bn64" : "attn_fwd_dual_fp8_d128_bm128_bn64";
    if (d == 64)
      return split_mode ? "attn_fwd_splitkv_dual_bf16_d64_bm128_bn64" : "attn_fwd_dual_bf16_d64_bm128_bn64";
    return split_mode ? "attn_fwd_splitkv_dual_bf16_d128_bm128_bn32" : "attn_fwd_dual_bf16_d128_bm128_bn32";
  }
  static const char* names[3][3][2] = {
      {{"attn_fwd_f32_d64_bm128_bn32", "attn_fwd_splitkv_f32_d64_bm128_bn32"},
       {"attn_fwd_f32_d128_bm128_bn32", "attn_fwd_splitkv_f32_d128_bm128_bn32"},
       {"attn_fwd_f32_d256_bm128_bn32", "attn_fwd_splitkv_f32_d256_bm128_bn32"}},
      {{"attn_fwd_bf16_d64_bm128_bn32", "attn_fwd_splitkv_bf16_d64_bm128_bn32"},
       {"attn_fwd_bf16_d128_bm128_bn32", "attn_fwd_splitkv_bf16_d128_bm128_bn32"},
       {"attn_fwd_bf16_d256_bm128_bn32", "attn_fwd_splitkv_bf16_d256_bm128_bn32"}},
      {{"attn_fwd_fp8_d64_bm128_bn64", "attn_fwd_splitkv_fp8_d64_bm128_bn64"},
       {"attn_fwd_fp8_d128_bm128_bn64", "attn_fwd_splitkv_fp8_d128_bm128_bn64"},
       {"attn_fwd_fp8_d256_bm128_bn64", "attn_fwd_splitkv_fp8_d256_bm128_bn64"}}};
  const int di = d == 64 ? 0 : d == 128 ? 1 : 2;
  if (block_n_for(dtype, d, sweep_keys) == 64 && dtype == DT_BF16)
    return split_mode ? "attn_fwd_splitkv_bf16_d64_bm128_bn64" : "attn_fwd_bf16_d64_bm128_bn64";
  return names[dtype][di][split_mode ? 1 : 0];
}

}  // namespace attn
