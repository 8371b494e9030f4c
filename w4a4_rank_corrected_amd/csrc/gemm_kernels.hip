// Fused W4A4 GEMM + low-rank up-projection (second fused pair of Nunchaku).
//
// [Review] = "SVDQuant: How a Small High-Precision Branch Makes 4-Bit Diffusion
// Practical" (technical review of arXiv:2411.05007v4): sec. 4.2 Eq.(7),
// sec. 6.1 Algorithm 2 steps 4-8 and Fig. 4 second pair.
// [Nunchaku] = "SVDQuant: 4-bit Quantization Enables Efficient Diffusion Model
// Inference on Consumer GPUs", section "Nunchaku": two 4-bit values per byte,
// unpacked with bit operations.
//
// Y[i,j] = sum_g sx[g,i] sw[g,j] isum[i,j,g] + (bf16(Z) L2)[i,j] + bias[j]
//
// Exact per-group integer sums on i8 MFMA: a nibble is unpacked to the byte
// 16*q (mask for the high nibble, shift-and-mask for the low one), so one
// v_mfma_i32_16x16x64_i8 over exactly one 64-channel group yields 256*isum.
// The MFMA accumulator is seeded with the bits of 1.5*2^23, so the result read
// as a float is 1.5*2^23 + 256*isum exactly (|256*isum| <= 802816 < 2^22).  Two
// FMAs then apply the scales:
//   t   = fma(r, sx/256, -1.5*2^23 * sx/256) = isum * sx   (exact: <= 23 bits)
//   acc = fma(t, sw, acc)                                 (one rounding)
// The low-rank branch initialises the accumulators with bf16 MFMAs.
//
// The two FMAs per (output element, group) make the kernel VALU-bound on
// gfx950 (a 16x16x64 i8 MFMA covers 256 element-groups in 16 cycles; their 8
// wave64 FMAs need 32), and only about 40 % of an MFMA's time overlaps VALU
// work, whether the two come from one wave or from different waves (measured
// with a microbenchmark).  The work decomposition therefore aims at keeping
// the VALU busy: three waves per SIMD to cover each other's latencies,
// unpacking each code once per workgroup, few LDS reads of scales, and few
// barriers.
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, 4 SIMDs per CU, wave64),
// parameterised by GemmCfg:
//   a workgroup computes TM x TN tiles of Y (rows x columns) with
//   (TM/WM) x (TN/WN) waves, each owning a WM x WN sub-tile of 16x16 MFMA
//   blocks.  Per 64-channel group it loads the packed activation and weight
//   records (contiguous in the group-major layout) with buffer loads, unpacks
//   them once into LDS (double-buffered), and every wave reads its MFMA
//   operands from there.  Global loads run DEPTH groups ahead in registers.
//   Measured alternatives that were not faster on gfx950: 256 x 256 and
//   128 x 256 tiles (register spills or fewer resident waves), 128 x 64 tiles
//   at three or four waves per SIMD (more staging and LDS traffic per output),
//   and explicit MFMA/FMA interleaving hints (the resident workgroups
//   already interleave).
//
// Schedules (tile = TM x TN outputs over all G groups; slots = the resident
// workgroups of all CUs, three per CU):
//   * one whole tile per workgroup, when the tiles fill whole rounds of slots
//     or their last round is more than a third full;
//   * otherwise the tiles of the last round are split along the channel
//     groups into k pieces each, one piece per workgroup (split workgroups
//     first in the grid, then the full rounds of whole tiles).  A piece
//     stores its sums in a partial slot of the workspace and ends; a
//     reduction kernel launched next on the same stream adds each tile's k
//     slots in piece order, applies the epilogue and stores the tile.  No
//     workgroup waits for or signals another (the kernel boundary orders the
//     slots' stores before their loads), so correctness does not depend on
//     the order or residency in which workgroups are dispatched, and results
//     are deterministic for a shape and CU count.  Device-scope atomics and
//     coherent loads, the alternative inside one kernel, measured 4-5 us per
//     round trip here: the last piece of a 256-row FLUX tile spent 35 us
//     adding eight 64 KB slots.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <unordered_map>
#include <utility>

#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace svdq {
namespace {

using namespace dev;

template <int BYTES>
struct Piece;  // packed code piece: BYTES/4 words of one 32-byte record
template <>
struct Piece<4> {
  uint32_t w[1];
};
template <>
struct Piece<8> {
  uint32_t w[2];
};
template <>
struct Piece<16> {
  uint32_t w[4];
};
template <>
struct Piece<32> {
  uint32_t w[8];
};

template <int BYTES>
__device__ __forceinline__ Piece<BYTES> buffer_piece(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  Piece<BYTES> p;
  if constexpr (BYTES == 32) {
    const u32x4 v0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
    const u32x4 v1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16u, 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) p.w[e] = v0[e], p.w[4 + e] = v1[e];
  } else if constexpr (BYTES == 16) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
    p.w[0] = v[0], p.w[1] = v[1], p.w[2] = v[2], p.w[3] = v[3];
  } else if constexpr (BYTES == 8) {
    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, 0, 0));
    p.w[0] = v.x, p.w[1] = v.y;
  } else {
    p.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, 0);
  }
  return p;
}

// LDS rows hold the 64 bytes of one row of one channel group as four 16-byte
// chunks; chunk j of row `row` sits at chunk position j ^ chunk_swz(row).  With
// this permutation both access patterns are free of bank conflicts whether
// the LDS serves 8 or 16 lanes of a 16-byte access per cycle: the staging
// stores (lanes 2t, 2t+1 write the two halves of row t) and the MFMA operand
// reads (16 consecutive rows at one chunk index).
__device__ __forceinline__ int chunk_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Unpack a piece starting at word w0 of a record into the LDS row `row` (whose
// swizzle is rs): the low nibbles of record word w go to byte 4*(w%4) of chunk
// 2*(w/4), the high nibbles to the same byte of chunk 2*(w/4)+1, each nibble
// becoming the signed byte 16*q.  Activations and weights use the same
// placement, so the channel permutation cancels in the dot product.
template <int BYTES>
__device__ __forceinline__ void unpack_piece(uint8_t* row, int rs, int w0, const Piece<BYTES>& p) {
  constexpr int NW = BYTES / 4;
  uint8_t* lo_dst = row + 16 * ((2 * (w0 >> 2)) ^ rs) + 4 * (w0 & 3);
  uint8_t* hi_dst = row + 16 * ((2 * (w0 >> 2) + 1) ^ rs) + 4 * (w0 & 3);
  uint32_t lo[NW], hi[NW];
#pragma unroll
  for (int e = 0; e < NW; ++e) {
    lo[e] = (p.w[e] << 4) & 0xF0F0F0F0u;
    hi[e] = p.w[e] & 0xF0F0F0F0u;
  }
  if constexpr (NW == 4) {
    *reinterpret_cast<u32x4*>(lo_dst) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<u32x4*>(hi_dst) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  } else if constexpr (NW == 2) {
    *reinterpret_cast<uint2*>(lo_dst) = uint2{lo[0], lo[1]};
    *reinterpret_cast<uint2*>(hi_dst) = uint2{hi[0], hi[1]};
  } else {
    *reinterpret_cast<uint32_t*>(lo_dst) = lo[0];
    *reinterpret_cast<uint32_t*>(hi_dst) = hi[0];
  }
}

// Copy a piece of an 8-bit record (64 codes, one byte each) starting at word w0
// into the LDS row `row` (swizzle rs), chunk by chunk.
__device__ __forceinline__ void copy_piece(uint8_t* row, int rs, int w0, const Piece<32>& p) {
  const int j = w0 >> 2;
  *reinterpret_cast<u32x4*>(row + 16 * (j ^ rs)) = u32x4{p.w[0], p.w[1], p.w[2], p.w[3]};
  *reinterpret_cast<u32x4*>(row + 16 * ((j + 1) ^ rs)) = u32x4{p.w[4], p.w[5], p.w[6], p.w[7]};
}

// f(integral_constant<int, U>) for each U of the sequence, in order (compile-time
// indices for register arrays).
template <int... U, class F>
__device__ __forceinline__ void unrolled(std::integer_sequence<int, U...>, F&& f) {
  (f(std::integral_constant<int, U>{}), ...);
}

// Linear tile index -> (tile row, tile column), so that tiles with nearby
// indices share activation and weight records: bands of 4 tile-rows,
// column-major inside.  Each XCD runs a contiguous range of linear tiles
// (dp_tile) and keeps its few activation rows in L2 while it streams the
// weight columns.  Measured on gfx950: column bands (an XCD keeping an eighth
// of the weight columns) were 1-4 % slower for one tile per workgroup, despite
// 26 % less HBM fetch on FLUX QKV.
__device__ __forceinline__ void band_tile(int t, int tiles_m, int tiles_n, int& ti, int& tj) {
  constexpr int GB = 4;
  const int band = t / (GB * tiles_n);
  const int first = band * GB;
  const int gb = min(tiles_m - first, GB);
  const int in_band = t - band * GB * tiles_n;
  ti = first + in_band % gb;
  tj = in_band / gb;
}

// Workgroup d of `count` one-tile workgroups -> linear tile base + t.
// Workgroups are dealt round-robin to the 8 XCDs, so each XCD gets a contiguous
// range of linear tiles, whose workgroups then share records in its L2.
__device__ __forceinline__ int dp_tile(int d, int count, int base) {
  const int xcd = d & 7, k = d >> 3;
  const int per = count >> 3, extra = count & 7;
  return base + (xcd < extra ? xcd * (per + 1) + k : extra * (per + 1) + (xcd - extra) * per + k);
}

template <int TM_, int TN_, int WM_, int WN_, int WPE_, int DEPTH_, int KG_ = 1>
struct GemmCfg {
  static constexpr int TM = TM_, TN = TN_;  // workgroup tile: rows (tokens) x output columns
  static constexpr int WM = WM_, WN = WN_;  // wave tile
  static constexpr int WPE = WPE_;          // waves per SIMD the register budget must allow
  static constexpr int DEPTH = DEPTH_;      // pipeline steps of global loads in flight
  static constexpr int KG = KG_;            // channel groups per pipeline step (per barrier)
  static constexpr int WAVES_N = TN / WN;
  static constexpr int NT = 64 * (TM / WM) * WAVES_N;
  static constexpr int BI = WM / 16, BJ = WN / 16;
  static constexpr int A_BYTES = TM * 32 / NT;  // packed activation bytes staged per thread per group
  static constexpr int B_BYTES = TN * 32 / NT;  // packed weight bytes staged per thread per group
  static constexpr int ROWB = 64;               // LDS bytes per unpacked 64-channel row
  static constexpr int WG_PER_CU = WPE * 4 / (NT / 64);  // resident workgroups per CU (4 SIMDs)
  static_assert(DEPTH >= 1 && KG >= 1, "pipeline shape");
  static_assert(WG_PER_CU >= 1 && (WPE * 4) % (NT / 64) == 0, "whole workgroups per CU");
  static_assert(A_BYTES == 4 || A_BYTES == 8 || A_BYTES == 16, "activation staging piece");
  static_assert(B_BYTES == 4 || B_BYTES == 8 || B_BYTES == 16, "weight staging piece");
  static_assert(NT >= TM + TN && TM % 64 == 0 && TN % 64 == 0, "scale staging: at most one scale per thread");
  static_assert(BI == 4 && BJ % 2 == 0, "scale reads: one 16-byte row-scale vector, whole fp16 column vectors");
};

// 128 x 128 tile, 4 waves of 64 x 64; three workgroups share a CU (168
// registers per lane), so one workgroup's barrier and LDS-latency phases
// overlap the others' compute, and loads run one group ahead.  Each format
// has one configuration; launches with split tiles use its build with the
// split-K code (SK = true), which fits the same register budget (every kernel
// of the library is checked for zero scratch at build time and before its
// first launch).
using Cfg = GemmCfg<128, 128, 64, 64, 3, 1>;
// INT4, narrow tiles for few rows (when the wide tiles would not fill one
// round of slots): 128 x 64 tiles, 4 waves of 64 x 32, half the work per
// workgroup and group, twice the workgroups; loads run two groups ahead.
using CfgN = GemmCfg<128, 64, 64, 32, 3, 2>;
// 8-bit codes: no per-group VALU work, so a group's compute is short: loads
// run two groups ahead (140 registers).
using Cfg8 = GemmCfg<128, 128, 64, 64, 3, 2>;
// NVFP4 (packed records in LDS, 20 KB per workgroup).
using CfgF4 = GemmCfg<128, 128, 64, 64, 3, 1>;

// Split tiles of a launch: workgroups [0, P) each compute one piece of one of
// the first T linear tiles (k pieces per tile, P = T k); the remaining
// workgroups compute whole tiles.
struct SplitK {
  int P;            // split workgroups: blockIdx < P (0 = none)
  int T;            // split tiles: linear tiles [0, T)
  int k;            // pieces per split tile
  int lr;           // the low-rank product's cost in groups, taken off the last piece
  float* partials;  // [k + 1][T][TM*TN] fp32 (or i32): piece q of tile t in slot q*T + t,
                    // the low-rank product of tile t (8-bit setting) in slot k*T + t
};

// Non-negative E4M3 block-scale byte -> its value as fp16 bits (exact: E4M3
// values are 2^-9 .. 448 with at most 4 significant bits).
// Branch-free: a normal E4M3 value keeps its fields (exponent rebiased from 7
// to 15, mantissa moved up 7 bits); a subnormal one, mant * 2^-9, is
// converted through fp32.
__device__ __forceinline__ uint32_t e4m3_to_f16_bits(uint32_t bits) {
  const uint32_t ex = (bits >> 3) & 15u, mant = bits & 7u;
  const uint32_t normal = ((bits & 0x7Fu) << 7) + 0x2000u;
  const uint32_t sub = __builtin_bit_cast(uint16_t, (_Float16)((float)mant * 0.001953125f));
  return ex ? normal : sub;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Eight FP4 codes (one 32-bit word, the even channel in each byte's low
// nibble) -> the f16 operand code * s, in channel order.  The conversion at
// unit scale is exact, and so is the product: an E2M1 value times an E4M3
// scale has at most 6 significant bits and lies in 2^-10 .. 2688.
__device__ __forceinline__ f16x8 fp4_operand(uint32_t w, _Float16 s) {
  const f16x2 ss = {s, s};
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// The kernel body for three operand formats (FMT):
//  * kFmtInt4: INT4 codes in 32-byte group records with per-group fp16 scales
//    (the exact per-group sums and fp32 scale epilogue described above);
//  * kFmtInt8: the 8-bit setting, per-token activation and per-output-channel
//    weight INT8 codes, one byte each, in 64-byte group-major records
//    [m/64][rows][64], with one fp16 scale per row and per column.  The MFMAs
//    chain over all groups into i32 accumulators (|sum| <= 127^2 m < 2^31 for
//    the m the library accepts) and the scales are applied once, in the
//    epilogue, so no per-group VALU work remains; split-K partials are then
//    i32 sums;
//  * kFmtFp4: the NVFP4 setting, FP4 E2M1 codes in the INT4 record layout and
//    one FP8 E4M3 scale per 16 channels (records [m/64][rows][4] bytes).  A
//    code times its block scale is exact in f16 (at most 6 significant bits,
//    magnitudes 2^-10 .. 2688).  LDS holds the packed code records and the
//    block scales as fp16; each wave dequantizes its MFMA operands in
//    registers (fp4_operand), and the f16 MFMAs accumulate sum_k x^ w^ in
//    fp32; the two power-of-two tensor scales (txw = t_x t_w) are applied
//    once in the epilogue, exactly.
template <class C, bool OUT_BF16, int FMT, bool SK = true>
__device__ __forceinline__ void gemm_up_body(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ ascale,
    const float* __restrict__ z, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, int b, int n, int G, int rank, int tiles_m, int tiles_n,
    void* __restrict__ yout, SplitK sk, float txw) {
  constexpr bool W8 = FMT == kFmtInt8, F4 = FMT == kFmtFp4;
  // INT4 starts the accumulators from the low-rank product; the 8-bit and
  // NVFP4 settings apply their scales after the main loop and then add it.
  constexpr bool POST = W8 || F4;
  static_assert(!W8 || (2 * C::A_BYTES == 32 && 2 * C::B_BYTES == 32), "8-bit records: 32-byte staging pieces");
  static_assert(!F4 || (C::A_BYTES == 16 && C::B_BYTES == 16), "FP4 records: 16-byte staging pieces");
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN, NT = C::NT;
  constexpr int BI = C::BI, BJ = C::BJ;
  constexpr int ROWB = F4 ? 32 : C::ROWB;  // LDS bytes per row and group (packed records for FP4)
  constexpr int KG = C::KG;
  // per buffer: KG groups of TM (TN) rows
  __shared__ __align__(16) uint8_t As[2][KG * TM * ROWB];
  __shared__ __align__(16) uint8_t Bs[2][KG * TN * ROWB];
  // FP4: per buffer and group, the four block scales (fp16) of each of the TM
  // activation rows, then of the TN weight columns
  __shared__ __align__(16) uint16_t F4s[2][F4 ? KG * (TM + TN) * 4 : 4];
  // per buffer and group: [sx/256 (TM floats) | sw (TN fp16)], each in the
  // order in which a lane reads its rows and columns (see store_stage); no
  // per-group scales with 8-bit or FP4 codes
  constexpr int SSC = TM + TN / 2;
  __shared__ __align__(16) float Ssc[2][POST ? 4 : KG * SSC];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r = lane & 15, c = lane >> 4;
  // this lane's 16-byte chunk of an MFMA operand row in LDS (rows of a block
  // start at multiples of 16, so the row's swizzle is that of r)
  const int cs = 16 * (c ^ chunk_swz(r));
  // FP4: 32-byte packed rows, word j at position j ^ 4 in rows with bit 3 set
  // (the operand reads of 16 rows then hit 64 distinct banks); this lane reads
  // word 4 kh + c of its rows (channels 32 kh + 8c .. +7, block 2 kh + c/2)
  const int f4w0 = c ^ (4 * ((r >> 3) & 1)), f4w1 = (4 + c) ^ (4 * ((r >> 3) & 1));
  constexpr int REC = W8 ? 64 : 32;  // record bytes of one row in one group
  constexpr int AB = W8 ? 2 * C::A_BYTES : C::A_BYTES, BB = W8 ? 2 * C::B_BYTES : C::B_BYTES;
  const int a_row = tid * AB / REC, a_w0 = (tid * AB % REC) / 4;
  const int b_col = tid * BB / REC, b_w0 = (tid * BB % REC) / 4;
  const uint32_t a_bytes = (uint32_t)b * REC, b_bytes = (uint32_t)n * REC;
  const i32x4 magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  f32x4 acc[BI][BJ];
  i32x4 iacc[BI][BJ];  // 8-bit setting: integer sums over all groups

  // ---- low-rank branch: acc = bf16(Z) L2 over K = rank in chunks of 32 -------
  // 16-byte loads when every row of l2 / z starts 16-byte aligned
  const bool l2_vec = (rank % 8) == 0 && ((uintptr_t)l2t & 15u) == 0;
  const bool z_vec = (rank % 4) == 0 && ((uintptr_t)z & 15u) == 0;
  auto lowrank = [&](int i0, int j0) {
    for (int kc = 0; kc < rank; kc += 32) {
      const int t0 = kc + 8 * c;  // this lane's 8 entries of the rank dimension
      bf16x8 P[BJ];
#pragma unroll
      for (int bj = 0; bj < BJ; ++bj) {
        const int j = j0 + WN * wn + 16 * bj + r;
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (j < n) {
          if (l2_vec && t0 + 8 <= rank) {
            wv = ldg16(l2t + (size_t)j * rank + t0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = t0 + 2 * e;
              const uint32_t lo = t < rank ? l2t[(size_t)j * rank + t] : 0u;
              const uint32_t hi = t + 1 < rank ? l2t[(size_t)j * rank + t + 1] : 0u;
              wv[e] = lo | (hi << 16);
            }
          }
        }
        P[bj] = __builtin_bit_cast(bf16x8, wv);
      }
#pragma unroll
      for (int bi = 0; bi < BI; ++bi) {
        const int i = i0 + WM * wm + 16 * bi + r;
        float zv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (i < b) {
          const float* zr = z + (size_t)i * rank + t0;
          if (z_vec && t0 + 8 <= rank) {
            const f32x4 z0 = *reinterpret_cast<const f32x4*>(zr);
            const f32x4 z1 = *reinterpret_cast<const f32x4*>(zr + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              zv[e] = z0[e];
              zv[4 + e] = z1[e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) zv[e] = t0 + e < rank ? zr[e] : 0.0f;
          }
        }
        const bf16x8 Q = __builtin_bit_cast(
            bf16x8, u32x4{pack_bf16x2(zv[0], zv[1]), pack_bf16x2(zv[2], zv[3]),
                          pack_bf16x2(zv[4], zv[5]), pack_bf16x2(zv[6], zv[7])});
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P[bj], Q, acc[bi][bj], 0, 0, 0);
      }
    }
  };

  // ---- main branch over groups [g0, g1) of the tile at (i0, j0) --------------
  // Staging: per group every thread issues the same three buffer loads: one
  // piece of an activation record, one piece of a weight record, one fp16
  // scale.  The per-group base lives in the (scalar) buffer descriptor, whose
  // size bound makes rows >= b and columns >= n read as zero.  A pipeline step
  // stages KG consecutive groups.
  struct Stage {
    Piece<AB> a[KG];
    Piece<BB> w[KG];
    uint32_t s[KG];   // INT4: this thread's group scale; FP4: the activation row's two block scales
    uint32_t s2[KG];  // FP4: the weight column's two block scales
  };
  // `pre` runs once the first groups' loads are in flight (the low-rank
  // branch: its own loads and MFMAs then overlap those loads' latency).
  auto main_branch = [&](int i0, int j0, int g0, int g1, auto&& pre) {
    const uint32_t a_voff = (uint32_t)(i0 + a_row) * REC + 4u * a_w0;
    const uint32_t b_voff = (uint32_t)(j0 + b_col) * REC + 4u * b_w0;
    // activation scale of row i0+tid, weight scale of column j0+tid-TM, or an
    // out-of-range offset (reads 0) for the threads that stage no scale
    const uint32_t s_voff = tid < TM ? (uint32_t)(i0 + tid) * 2u
                                     : (tid < TM + TN ? (uint32_t)(j0 + tid - TM) * 2u : 0x7FFFFFF0u);
    const int NG = g1 - g0;            // groups in this segment
    if (NG <= 0) {                     // the up-projection alone (no channel groups)
      pre();
      return;
    }
    const int S = (NG + KG - 1) / KG;  // pipeline steps
    // Step k's groups g0 + KG k + q.  A group past the segment's end reads as
    // zero (size-0 descriptors: zero codes and scales add nothing); a step past
    // the last one is never computed.
    auto load_stage = [&](int k, Stage& st) {
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        const int gi = KG * k + q;
        const bool live = gi < NG;
        const int g = g0 + (live ? gi : NG - 1);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(qx + (size_t)g * a_bytes, live ? a_bytes : 0u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(qw + (size_t)g * b_bytes, live ? b_bytes : 0u);
        st.a[q] = buffer_piece<AB>(ra, a_voff);
        st.w[q] = buffer_piece<BB>(rb, b_voff);
        if constexpr (F4) {
          // the two block scales of this thread's 32 codes: bytes 2h, 2h+1 of
          // the row's 4-byte scale record (h = the record half it stages)
          const uint8_t* as8 = reinterpret_cast<const uint8_t*>(ascale);
          const uint8_t* ws8 = reinterpret_cast<const uint8_t*>(wscale);
          const __amdgpu_buffer_rsrc_t rsa = make_rsrc(as8 + (size_t)g * b * 4, live ? (uint32_t)b * 4u : 0u);
          const __amdgpu_buffer_rsrc_t rsw = make_rsrc(ws8 + (size_t)g * n * 4, live ? (uint32_t)n * 4u : 0u);
          st.s[q] = __builtin_amdgcn_raw_buffer_load_b16(rsa, (uint32_t)(i0 + a_row) * 4u + 2u * (a_w0 >> 2), 0, 0);
          st.s2[q] = __builtin_amdgcn_raw_buffer_load_b16(rsw, (uint32_t)(j0 + b_col) * 4u + 2u * (b_w0 >> 2), 0, 0);
        } else if constexpr (!W8) {
          // wave-uniform choice (waves 0 .. TM/64-1 stage activation scales), so
          // the descriptor stays in scalar registers
          const __amdgpu_buffer_rsrc_t rs =
              wave_u < TM / 64 ? make_rsrc(ascale + (size_t)g * b, live ? (uint32_t)b * 2u : 0u)
                               : make_rsrc(wscale + (size_t)g * n, live ? (uint32_t)n * 2u : 0u);
          st.s[q] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_voff, 0, 0);
        }
      }
    };
    // Scales go to one LDS array per buffer and group: [sx/256 (TM floats) |
    // sw (TN fp16)].  Thread t < TM stages row i0+t's activation scale, thread
    // TM+u column j0+u's weight scale (the choice is wave-uniform).  Both are
    // permuted so that a lane's values are contiguous: row l = 16 bi + r of a
    // wave's row block sits at BI r + bi (one 16-byte read gives a lane its BI
    // rows), column l = 16 bj + 4 c + v of a wave's column block at
    // 4 BJ c + 4 bj + v (BJ/2 16-byte reads give a lane its 4 BJ columns).
    // FP4: a 16-byte code piece (words w0 .. w0+3 of the record) is copied to
    // its row (swizzled as above), and its two E4M3 block scales (blocks
    // w0/2 and w0/2 + 1: bytes 0 and 1 of sc) go to the row's scale slots as
    // fp16, with one 32-bit store
    auto stage_fp4 = [&](uint8_t* row, int ridx, int w0, const Piece<16>& pc, uint32_t sc, uint16_t* srow) {
      *reinterpret_cast<u32x4*>(row + 4 * (w0 ^ (4 * ((ridx >> 3) & 1)))) = u32x4{pc.w[0], pc.w[1], pc.w[2], pc.w[3]};
      reinterpret_cast<uint32_t*>(srow)[w0 >> 2] =
          e4m3_to_f16_bits(sc & 0xFFu) | (e4m3_to_f16_bits((sc >> 8) & 0xFFu) << 16);
    };
    auto store_stage = [&](int buf, const Stage& st) {
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        uint8_t* as = &As[buf][(q * TM + a_row) * ROWB];
        uint8_t* bs = &Bs[buf][(q * TN + b_col) * ROWB];
        if constexpr (F4) {
          uint16_t* fs = &F4s[buf][q * (TM + TN) * 4];
          stage_fp4(as, a_row, a_w0, st.a[q], st.s[q], fs + a_row * 4);
          stage_fp4(bs, b_col, b_w0, st.w[q], st.s2[q], fs + (TM + b_col) * 4);
        } else if constexpr (W8) {
          copy_piece(as, chunk_swz(a_row), a_w0, st.a[q]);
          copy_piece(bs, chunk_swz(b_col), b_w0, st.w[q]);
        } else {
          unpack_piece<AB>(as, chunk_swz(a_row), a_w0, st.a[q]);
          unpack_piece<BB>(bs, chunk_swz(b_col), b_w0, st.w[q]);
          // one 32-bit store per thread: sx/256 (exact), or the fp16 pair of
          // columns (l, l ^ 1), which lanes u and u ^ 1 both write
          const uint32_t sv = st.s[q];
          const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)sv, 0xB1, 0xF, 0xF, false);  // lane ^ 1
          const bool act = wave_u < TM / 64;
          const int la = tid % WM, lw = (tid - TM) % WN;
          const int pa = tid - la + BI * (la & 15) + (la >> 4);
          const int pw = TM + ((tid - TM - lw + 4 * BJ * ((lw & 15) >> 2) + 4 * (lw >> 4) + (lw & 3)) >> 1);
          const uint32_t va = __float_as_uint(f16_to_f32((uint16_t)sv) * 0.00390625f);
          const uint32_t vw = (lw & 1) ? (nb | (sv << 16)) : (sv | (nb << 16));
          // waves past the TM + TN scale threads (narrow tiles) stage none
          if (TM + TN == NT || wave_u < (TM + TN) / 64)
            reinterpret_cast<uint32_t*>(&Ssc[buf][q * SSC])[act ? pa : pw] = act ? va : vw;
        }
      }
    };
    // One group q of a buffer.  INT4: for each 16-row block bi, BJ MFMAs (one
    // per 16-column block), whose results are applied by 8 * BJ FMAs.  8-bit:
    // the MFMAs accumulate into the integer sums directly.
    auto compute_group = [&](int buf, int q) {
      const uint8_t* as = &As[buf][q * TM * ROWB];
      const uint8_t* bs = &Bs[buf][q * TN * ROWB];
      if constexpr (F4) {
        const uint32_t* aw = reinterpret_cast<const uint32_t*>(as);
        const uint32_t* bw = reinterpret_cast<const uint32_t*>(bs);
        const _Float16* fs = reinterpret_cast<const _Float16*>(&F4s[buf][q * (TM + TN) * 4]);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {  // channels 0-31, then 32-63 of the group
          const int wo = kh ? f4w1 : f4w0, blk = 2 * kh + (c >> 1);
          f16x8 Pb[BJ];
#pragma unroll
          for (int bj = 0; bj < BJ; ++bj) {
            const int row = WN * wn + 16 * bj + r;
            Pb[bj] = fp4_operand(bw[row * 8 + wo], fs[(TM + row) * 4 + blk]);
          }
#pragma unroll
          for (int bi = 0; bi < BI; ++bi) {
            const int row = WM * wm + 16 * bi + r;
            const f16x8 Qa = fp4_operand(aw[row * 8 + wo], fs[row * 4 + blk]);
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
              acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Pb[bj], Qa, acc[bi][bj], 0, 0, 0);
          }
        }
      } else if constexpr (W8) {
        u32x4 Pb[BJ];
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj)
          Pb[bj] = *reinterpret_cast<const u32x4*>(bs + (WN * wn + 16 * bj + r) * ROWB + cs);
#pragma unroll
        for (int bi = 0; bi < BI; ++bi) {
          const u32x4 Qa = *reinterpret_cast<const u32x4*>(as + (WM * wm + 16 * bi + r) * ROWB + cs);
#pragma unroll
          for (int bj = 0; bj < BJ; ++bj)
            iacc[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                __builtin_bit_cast(i32x4, Pb[bj]), __builtin_bit_cast(i32x4, Qa), iacc[bi][bj], 0, 0, 0);
        }
      } else {
        typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
        const float* sc = &Ssc[buf][q * SSC];
        u32x4 Pb[BJ];
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj)
          Pb[bj] = *reinterpret_cast<const u32x4*>(bs + (WN * wn + 16 * bj + r) * ROWB + cs);
        // this lane's BI row scales sx/256 and 4 BJ column scales sw (fp16,
        // applied by mixed-precision FMAs: the conversion is exact)
        const f32x4 sx4 = *reinterpret_cast<const f32x4*>(sc + WM * wm + BI * r);
        f16x8 sw8[BJ / 2];
#pragma unroll
        for (int h = 0; h < BJ / 2; ++h)
          sw8[h] = *reinterpret_cast<const f16x8*>(reinterpret_cast<const _Float16*>(sc + TM) + WN * wn +
                                                   4 * BJ * c + 8 * h);
        const int rbase = WM * wm + r;
        // The wave's BI activation fragments are all read up front (the
        // compiler would otherwise read each just before its block's MFMAs and
        // wait out the LDS latency BI times per group): measured 2-4 % faster
        // on FLUX QKV and PixArt fc1.  An FMA needs its block's MFMA results;
        // the register budget holds one block's results, and the other waves
        // of the SIMD cover the MFMA latency.
        u32x4 Qall[BI];
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
          Qall[bi] = *reinterpret_cast<const u32x4*>(as + (rbase + 16 * bi) * ROWB + cs);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bi = 0; bi < BI; ++bi) {
          const float sxq = sx4[bi];
          const float sng = -kMagic * sx4[bi];  // exact: 3 * 2^14 * sx
          i32x4 d[BJ];
#pragma unroll
          for (int bj = 0; bj < BJ; ++bj)
            d[bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, Pb[bj]),
                                                          __builtin_bit_cast(i32x4, Qall[bi]), magic, 0, 0, 0);
#pragma unroll
          for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float t = __builtin_fmaf(__int_as_float(d[bj][v]), sxq, sng);
              acc[bi][bj][v] = __builtin_fmaf(t, (float)sw8[bj >> 1][4 * (bj & 1) + v], acc[bi][bj][v]);
            }
        }
      }
    };

    // Pipeline over D = C::DEPTH register stages: LDS buffer k & 1 holds step
    // k's groups while they are computed, register stage j % D holds step j's
    // for k < j <= k + D (the later ones still loading).  A step computes its
    // groups, moves step k + 1's from their register stage into the other LDS
    // buffer, starts loading step k + 1 + D's into the freed stage, and ends
    // with one barrier, so loads have D steps to arrive.  Loads and stores are
    // unconditional (past the last step they re-read the last group into a
    // buffer nobody reads), so no branch sits inside a step and each wait
    // covers exactly one step.  The trailing barrier also frees the LDS
    // buffers for the next segment.  The loop is unrolled over lcm(D, 2) steps
    // so that stage and buffer indices are compile-time constants.
    constexpr int D = C::DEPTH;
    constexpr int UNR = D % 2 == 0 ? D : 2 * D;
    Stage st[D];
#pragma unroll
    for (int u = 0; u < D; ++u) load_stage(u, st[u]);
    pre();
    store_stage(0, st[0]);
    load_stage(D, st[0]);
    __syncthreads();
    auto step = [&](int k, auto U) {
      constexpr int u = decltype(U)::value;  // k % UNR
#pragma unroll
      for (int q = 0; q < KG; ++q) compute_group(u & 1, q);
      store_stage((u & 1) ^ 1, st[(u + 1) % D]);
      load_stage(k + 1 + D, st[(u + 1) % D]);
      __syncthreads();
    };
    int k = 0;
    for (; k + UNR - 1 < S; k += UNR)
      unrolled(std::make_integer_sequence<int, UNR>{}, [&](auto U) { step(k + decltype(U)::value, U); });
    unrolled(std::make_integer_sequence<int, UNR - 1>{}, [&](auto U) {
      if (k + decltype(U)::value < S) step(k + decltype(U)::value, U);
    });
  };

  // ---- epilogue: bias, cast, one store of Y ---------------------------------
  // lane holds Y[i][j..j+3]: i = row (l & 15) of block bi, j = 4 (l >> 4) of block bj
  auto store_tile = [&](int i0, int j0) {
    const bool vec_ok = (n & 3) == 0 && ((uintptr_t)yout & (OUT_BF16 ? 7u : 15u)) == 0;
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj) {
      const int j = j0 + WN * wn + 16 * bj + 4 * c;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (j + v < n) bv[v] = __uint_as_float((uint32_t)bias[j + v] << 16);
      }
#pragma unroll
      for (int bi = 0; bi < BI; ++bi) {
        const int i = i0 + WM * wm + 16 * bi + r;
        if (i >= b) continue;
        f32x4 o = acc[bi][bj];
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] += bv[v];
        if (OUT_BF16) {
          uint16_t* y = reinterpret_cast<uint16_t*>(yout) + (size_t)i * n + j;
          if (vec_ok && j + 3 < n) {
            *reinterpret_cast<uint2*>(y) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (j + v < n) y[v] = bf16_bits(o[v]);
          }
        } else {
          float* y = reinterpret_cast<float*>(yout) + (size_t)i * n + j;
          if (vec_ok && j + 3 < n) {
            *reinterpret_cast<f32x4*>(y) = o;
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (j + v < n) y[v] = o[v];
          }
        }
      }
    }
  };

  auto zero_acc = [&]() {
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < BJ; ++bj) {
        if constexpr (W8)
          iacc[bi][bj] = i32x4{0, 0, 0, 0};
        else
          acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };
  auto zero_acc_f32 = [&]() {
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < BJ; ++bj) acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // 8-bit setting, after all groups: acc = isum * (sx sw); the product of the
  // two fp16 scales is exact in fp32, so each element takes the rounding of the
  // conversion and of one multiplication
  auto scale_sums = [&](int i0, int j0) {
    if constexpr (F4) {  // a power of two: exact
#pragma unroll
      for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj) acc[bi][bj] *= txw;
      return;
    }
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj) {
      const int j = j0 + WN * wn + 16 * bj + 4 * c;
      float sw[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) sw[v] = j + v < n ? f16_to_f32(wscale[j + v]) : 0.0f;
#pragma unroll
      for (int bi = 0; bi < BI; ++bi) {
        const int i = i0 + WM * wm + 16 * bi + r;
        const float sx = i < b ? f16_to_f32(ascale[i]) : 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[bi][bj][v] = (float)iacc[bi][bj][v] * (sx * sw[v]);
      }
    }
  };

  // ---- this workgroup's work: a whole tile, or one piece of a split tile ----
  // Split pieces come first in the grid.  A piece stores its raw sums (fp32,
  // or i32 in the 8-bit setting) in its partial slot and ends; the reduction
  // kernel launched after this one adds each tile's k slots in piece order
  // and applies the epilogue.  The kernel boundary orders the slots' stores
  // before their loads, so no workgroup waits for or signals another, and the
  // result does not depend on dispatch order (deterministic for a shape and
  // CU count).  The piece with the tile's last groups carries the low-rank
  // product in its sums (INT4), or, in the 8-bit setting (integer sums),
  // stores it alone in slot k of the tile (NVFP4 tiles are never split).
  const int T = tiles_m * tiles_n;
  const bool split = SK && (int)blockIdx.x < sk.P;
  int t, g0 = 0, g1 = G;
  if (split) {
    // pieces of equal time: the tile's work counts the low-rank product (done
    // by the last piece) as lr groups, so the last piece gets lr fewer
    t = (int)blockIdx.x / sk.k;
    const int j = (int)blockIdx.x - t * sk.k;
    const int Ge = G + sk.lr;
    g0 = (int)((long long)j * Ge / sk.k);
    g1 = j + 1 == sk.k ? G : (int)((long long)(j + 1) * Ge / sk.k);
  } else {
    t = dp_tile((int)blockIdx.x - sk.P, T - sk.T, sk.T);
  }
  int ti, tj;
  band_tile(t, tiles_m, tiles_n, ti, tj);
  const int i0 = ti * TM, j0 = tj * TN;
  zero_acc();
  main_branch(i0, j0, g0, g1, [&] {
    // the tile's last groups carry the low-rank branch
    if constexpr (!POST)
      if (g1 == G) lowrank(i0, j0);
  });
  if constexpr (SK) {
    if (split) {
      // Slot layout, in 16-byte units: [wave][block k = bi BJ + bj][lane], so
      // each store of a wave writes 1 KB contiguous (the reduction kernel
      // maps units back to outputs the same way); the byte offset
      // wave*BI*BJ KB + k KB + 16 lane is split into a per-lane base, a scalar
      // 4 KB multiple and an instruction immediate below 4 KB.  Slots are
      // piece-major: piece q of split tile t in slot q*T + t.
      static_assert(BI * BJ % 4 == 0 && NT == 256, "partial layout: blocks of 1 KB, 4 per 4 KB");
      const uint32_t part_voff = (uint32_t)(wave * BI * BJ * 1024 + lane * 16);
      auto partial_offset = [](int q) { return (uint32_t)((q & 3) * 1024); };
      auto partial_soffset = [](int q) { return (q >> 2) * 4096; };
      auto store_slot = [&](int slot, auto&& val) {
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(sk.partials + (size_t)slot * (TM * TN), TM * TN * 4);
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
          for (int bj = 0; bj < BJ; ++bj)
            __builtin_amdgcn_raw_buffer_store_b128(val(bi, bj), rp, part_voff + partial_offset(bi * BJ + bj),
                                                   partial_soffset(bi * BJ + bj), 0);
      };
      const int piece = (int)blockIdx.x - t * sk.k;
      if constexpr (W8)
        store_slot(piece * sk.T + t, [&](int bi, int bj) { return __builtin_bit_cast(u32x4, iacc[bi][bj]); });
      else
        store_slot(piece * sk.T + t, [&](int bi, int bj) { return __builtin_bit_cast(u32x4, acc[bi][bj]); });
      if constexpr (!POST) {
        return;
      } else {
        // the piece with the tile's last groups: its low-rank product alone,
        // in slot k of the tile (one lowrank call site below keeps the
        // register allocation of the epilogue shared)
        if (g1 != G || rank <= 0) return;
        zero_acc_f32();
      }
    }
  }
  if constexpr (POST) {
    if (!split) scale_sums(i0, j0);
    lowrank(i0, j0);
    if constexpr (SK) {
      if (split) {
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(sk.partials + ((size_t)sk.k * sk.T + t) * (TM * TN), TM * TN * 4);
        const uint32_t part_voff = (uint32_t)(wave * BI * BJ * 1024 + lane * 16);
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
          for (int bj = 0; bj < BJ; ++bj)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[bi][bj]), rp,
                                                   part_voff + (uint32_t)(((bi * BJ + bj) & 3) * 1024),
                                                   ((bi * BJ + bj) >> 2) * 4096, 0);
        return;
      }
    }
  }
  store_tile(i0, j0);
}

template <class C, bool OUT_BF16, bool SK>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void gemm_w4a4_up_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ ascale,
    const float* __restrict__ z, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, int b, int n, int G, int rank, int tiles_m, int tiles_n,
    void* __restrict__ yout, SplitK sk, float txw) {
  gemm_up_body<C, OUT_BF16, kFmtInt4, SK>(qx, ascale, z, qw, wscale, l2t, bias, b, n, G, rank, tiles_m, tiles_n,
                                          yout, sk, txw);
}

template <class C, bool OUT_BF16, bool SK>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void gemm_w8a8_up_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ ascale,
    const float* __restrict__ z, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, int b, int n, int G, int rank, int tiles_m, int tiles_n,
    void* __restrict__ yout, SplitK sk, float txw) {
  gemm_up_body<C, OUT_BF16, kFmtInt8, SK>(qx, ascale, z, qw, wscale, l2t, bias, b, n, G, rank, tiles_m, tiles_n,
                                          yout, sk, txw);
}

template <class C, bool OUT_BF16, bool SK>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void gemm_fp4_up_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ ascale,
    const float* __restrict__ z, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, int b, int n, int G, int rank, int tiles_m, int tiles_n,
    void* __restrict__ yout, SplitK sk, float txw) {
  gemm_up_body<C, OUT_BF16, kFmtFp4, SK>(qx, ascale, z, qw, wscale, l2t, bias, b, n, G, rank, tiles_m, tiles_n,
                                         yout, sk, txw);
}

// Reduction of the split tiles: thread u handles 16-byte unit u of every slot
// of its tile (4 consecutive outputs of one row, in the slot layout the pieces
// store), adds the k pieces' units in piece order (i32 in the 8-bit setting,
// exact), applies the epilogue the whole tiles apply (8-bit: the per-row and
// per-column scales, then the tile's low-rank slot), adds the bias and stores
// Y.  All k loads are issued before the first add.  (NVFP4 tiles are never
// split.)
template <class C, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ partials, int T, int k, int tiles_m, int tiles_n, int b, int n,
    const uint16_t* __restrict__ ascale, const uint16_t* __restrict__ wscale, int lowrank_slot,
    const uint16_t* __restrict__ bias, void* __restrict__ yout) {
  static_assert(C::NT == 256 && kMaxPiecesAll <= 16, "unit layout of the slots");
  constexpr int WU = C::BI * C::BJ * 64;    // units per wave
  static_assert(FMT == kFmtInt4 || FMT == kFmtInt8, "INT4 and 8-bit tiles only");
  constexpr int UNITS = C::TM * C::TN / 4;  // 16-byte units per slot
  const int u = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int t = u / UNITS, w = u - t * UNITS;
  if (t >= T) return;
  const int wave = w / WU, blk = (w / 64) % (C::BI * C::BJ), lane = w & 63;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int bi = blk / C::BJ, bj = blk % C::BJ;
  int ti, tj;
  band_tile(t, tiles_m, tiles_n, ti, tj);
  const int i = ti * C::TM + C::WM * wm + 16 * bi + (lane & 15);
  const int j = tj * C::TN + C::WN * wn + 16 * bj + 4 * (lane >> 4);
  if (i >= b || j >= n) return;
  const f32x4* slots = reinterpret_cast<const f32x4*>(partials);
  const size_t stride = (size_t)T * UNITS, base = (size_t)t * UNITS + w;
  f32x4 v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (q < k) v[q] = slots[base + (size_t)q * stride];
  f32x4 o;
  if constexpr (FMT == kFmtInt8) {
    i32x4 s = __builtin_bit_cast(i32x4, v[0]);
#pragma unroll
    for (int q = 1; q < 16; ++q)
      if (q < k) s += __builtin_bit_cast(i32x4, v[q]);
    const float sx = f16_to_f32(ascale[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)s[e] * (sx * (j + e < n ? f16_to_f32(wscale[j + e]) : 0.0f));
  } else {
    o = v[0];
#pragma unroll
    for (int q = 1; q < 16; ++q)
      if (q < k) o += v[q];
  }
  if (lowrank_slot) o += slots[base + (size_t)k * stride];
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  if (bias) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e < n) bv[e] = __uint_as_float((uint32_t)bias[j + e] << 16);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] += bv[e];
  const bool vec_ok = (n & 3) == 0 && ((uintptr_t)yout & (OUT_BF16 ? 7u : 15u)) == 0 && j + 3 < n;
  if (OUT_BF16) {
    uint16_t* y = reinterpret_cast<uint16_t*>(yout) + (size_t)i * n + j;
    if (vec_ok) {
      *reinterpret_cast<uint2*>(y) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < n) y[e] = bf16_bits(o[e]);
    }
  } else {
    float* y = reinterpret_cast<float*>(yout) + (size_t)i * n + j;
    if (vec_ok) {
      *reinterpret_cast<f32x4*>(y) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < n) y[e] = o[e];
    }
  }
}

int g_num_cus = 0;
// Weight-side operands of one launch (INT4 or 8-bit layer).
struct Operands {
  const uint8_t* qw;
  const uint16_t* wscale;
  const uint16_t* l2;
  const uint16_t* bias;
  int n, rank;
};

// A GEMM kernel that uses scratch memory (register spills) is refused before
// its first launch: spills cost bandwidth, and a spill around a divergent
// region once produced wrong results in a GEMM build.  The build checks the
// same; this guards a library rebuilt with another compiler.  Queried once per
// kernel and process.
int scratch_free(const void* kernel) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> seen;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = seen.find(kernel);
  if (it != seen.end()) return it->second;
  hipFuncAttributes attr{};
  const hipError_t e = hipFuncGetAttributes(&attr, kernel);
  const int status = e != hipSuccess ? (int)e : (attr.localSizeBytes != 0 ? kErrKernelScratch : 0);
  seen[kernel] = status;
  return status;
}

template <class K, class... Args>
int launch_checked(K kernel, int grid, int threads, hipStream_t st, Args... args) {
  const int ok = scratch_free(reinterpret_cast<const void*>(kernel));
  if (ok != 0) return ok;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, st, args...);
  return (int)hipGetLastError();
}

template <bool OUT_BF16, int FMT>
int launch_typed(const uint8_t* qx, const uint16_t* ascale, const float* z, const Operands& L, int b,
                 void* y, const GemmPlan& plan, void* ws, hipStream_t st, float txw = 1.0f) {
  SplitK sk{0, 0, 1, 0, nullptr};
  if (plan.split) {
    sk.P = plan.split_grid;
    sk.T = plan.split_tiles;
    sk.k = plan.pieces;
    // about one memory round trip of its loads, measured at 4-6 us, the time
    // of 4 groups at three workgroups per CU; (k - 1) lr < G - k holds since
    // every piece has at least kMinPieceGroups groups
    sk.lr = L.rank > 0 ? kLowRankPieceGroups : 0;
    sk.partials = reinterpret_cast<float*>(ws);
  }
#define SVDQ_GEMM_ARGS qx, ascale, z, L.qw, L.wscale, L.l2, L.bias, b, L.n, plan.G, L.rank, plan.tiles_m, \
                       plan.tiles_n, y, sk, txw
  int st_gemm;
  if constexpr (FMT == kFmtInt8) {
    st_gemm = plan.split
                  ? launch_checked(gemm_w8a8_up_kernel<Cfg8, OUT_BF16, true>, plan.grid, Cfg8::NT, st, SVDQ_GEMM_ARGS)
                  : launch_checked(gemm_w8a8_up_kernel<Cfg8, OUT_BF16, false>, plan.grid, Cfg8::NT, st, SVDQ_GEMM_ARGS);
  } else if constexpr (FMT == kFmtFp4) {
    // the planner never splits NVFP4 tiles (its split build exceeds the
    // register budget of three workgroups per CU)
    if (plan.split) return (int)hipErrorInvalidValue;
    st_gemm = launch_checked(gemm_fp4_up_kernel<CfgF4, OUT_BF16, false>, plan.grid, CfgF4::NT, st, SVDQ_GEMM_ARGS);
  } else if (plan.tile_n == CfgN::TN) {
    st_gemm = plan.split
                  ? launch_checked(gemm_w4a4_up_kernel<CfgN, OUT_BF16, true>, plan.grid, CfgN::NT, st, SVDQ_GEMM_ARGS)
                  : launch_checked(gemm_w4a4_up_kernel<CfgN, OUT_BF16, false>, plan.grid, CfgN::NT, st, SVDQ_GEMM_ARGS);
  } else {
    st_gemm = plan.split
                  ? launch_checked(gemm_w4a4_up_kernel<Cfg, OUT_BF16, true>, plan.grid, Cfg::NT, st, SVDQ_GEMM_ARGS)
                  : launch_checked(gemm_w4a4_up_kernel<Cfg, OUT_BF16, false>, plan.grid, Cfg::NT, st, SVDQ_GEMM_ARGS);
  }
#undef SVDQ_GEMM_ARGS
  if (st_gemm != 0 || !plan.split) return st_gemm;
  const int lr_slot = FMT == kFmtInt8 && L.rank > 0 ? 1 : 0;
  auto reduce = [&](auto cfg) {
    using C = decltype(cfg);
    constexpr int UNITS = C::TM * C::TN / 4;
    return launch_checked(splitk_reduce_kernel<C, FMT, OUT_BF16>, (int)(((long long)sk.T * UNITS + 255) / 256),
                          256, st, (const float*)sk.partials, sk.T, sk.k, plan.tiles_m, plan.tiles_n, b, L.n,
                          ascale, L.wscale, lr_slot, L.bias, y);
  };
  if constexpr (FMT == kFmtFp4) {
    return st_gemm;
  } else if constexpr (FMT == kFmtInt8) {
    return reduce(Cfg8{});
  } else {
    return plan.tile_n == CfgN::TN ? reduce(CfgN{}) : reduce(Cfg{});
  }
}

}  // namespace

// The launch plan (gemm_plan) is host logic in plan.cpp; the kernel builds
// here must match the tiling and residencies it plans for.
static_assert(Cfg::TM == kGemmTileM && Cfg::TN == kGemmTileN && CfgN::TM == kGemmTileM &&
                  CfgN::TN == kGemmTileNNarrow && CfgN::WG_PER_CU == Cfg::WG_PER_CU,
              "tile shapes");
static_assert(Cfg::TM == Cfg8::TM && Cfg::TN == Cfg8::TN && Cfg::TM == CfgF4::TM && Cfg::TN == CfgF4::TN,
              "one tiling for every setting");
static_assert(Cfg::WG_PER_CU == kGemmWgPerCu[kFmtInt4] && Cfg8::WG_PER_CU == kGemmWgPerCu[kFmtInt8] &&
                  CfgF4::WG_PER_CU == kGemmWgPerCu[kFmtFp4],
              "resident workgroups per CU of each build");

int device_cus() {
  if (g_num_cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      g_num_cus = std::min(v, kMaxCUs);
    else
      g_num_cus = kMaxCUs;
  }
  return g_num_cus;
}

int launch_gemm_up(const uint8_t* qx, const uint16_t* ascale, const float* z, const svdq_layer& L,
                   int b, void* y, int y_dtype, void* ws, void* stream) {
  const GemmPlan plan = gemm_plan(b, L.n, L.m, device_cus());
  const Operands o{L.qw, L.wscale, L.l2, L.bias, L.n, L.rank};
  hipStream_t st = (hipStream_t)stream;
  if (y_dtype == SVDQ_OUT_BF16) return launch_typed<true, kFmtInt4>(qx, ascale, z, o, b, y, plan, ws, st);
  return launch_typed<false, kFmtInt4>(qx, ascale, z, o, b, y, plan, ws, st);
}

int launch_gemm8_up(const int8_t* qx, const uint16_t* ascale, const float* z, const svdq_w8a8_layer& L,
                    int b, void* y, int y_dtype, void* ws, void* stream) {
  const GemmPlan plan = gemm_plan(b, L.n, L.m, device_cus(), kFmtInt8);
  const Operands o{reinterpret_cast<const uint8_t*>(L.qw), L.wscale, L.l2, L.bias, L.n, L.rank};
  const uint8_t* a = reinterpret_cast<const uint8_t*>(qx);
  hipStream_t st = (hipStream_t)stream;
  if (y_dtype == SVDQ_OUT_BF16) return launch_typed<true, kFmtInt8>(a, ascale, z, o, b, y, plan, ws, st);
  return launch_typed<false, kFmtInt8>(a, ascale, z, o, b, y, plan, ws, st);
}

int launch_gemm_fp4_up(const uint8_t* qx, const uint8_t* ascale, const float* z, const svdq_fp4_layer& L, int b,
                       void* y, int y_dtype, void* ws, void* stream) {
  const GemmPlan plan = gemm_plan(b, L.n, L.m, device_cus(), kFmtFp4);
  const Operands o{L.qw, reinterpret_cast<const uint16_t*>(L.wscale), L.l2, L.bias, L.n, L.rank};
  const uint16_t* as = reinterpret_cast<const uint16_t*>(ascale);
  const float txw = L.t_x * L.t_w;  // powers of two: exact
  hipStream_t st = (hipStream_t)stream;
  if (y_dtype == SVDQ_OUT_BF16) return launch_typed<true, kFmtFp4>(qx, as, z, o, b, y, plan, ws, st, txw);
  return launch_typed<false, kFmtFp4>(qx, as, z, o, b, y, plan, ws, st, txw);
}

// The low-rank up-projection alone, y = bf16(z) L2 (the unfused path's
// separate kernel): the GEMM kernel with no channel groups and no bias.
int launch_lowrank_up(const float* z, const svdq_layer& L, int b, void* y, int y_dtype, void* stream) {
  const GemmPlan plan = gemm_plan(b, L.n, 0, device_cus());  // G = 0: one tile per workgroup
  const Operands o{nullptr, nullptr, L.l2, nullptr, L.n, L.rank};
  hipStream_t st = (hipStream_t)stream;
  if (y_dtype == SVDQ_OUT_BF16) return launch_typed<true, kFmtInt4>(nullptr, nullptr, z, o, b, y, plan, nullptr, st);
  return launch_typed<false, kFmtInt4>(nullptr, nullptr, z, o, b, y, plan, nullptr, st);
}

}  // namespace svdq
