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
// wave64 FMAs need 32).  The work decomposition therefore aims at keeping the
// VALU busy: many waves per SIMD so MFMAs co-issue with other waves' FMAs,
// unpacking each code once per workgroup, and few barriers.
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, 4 SIMDs per CU, wave64),
// parameterised by GemmCfg:
//   a workgroup computes a TM x TN tile of Y (rows x columns) with
//   (TM/WM) x (TN/WN) waves, each owning a WM x WN sub-tile of 16x16 MFMA
//   blocks.  Per stage of KG channel groups it loads the packed activation and
//   weight records (contiguous in the group-major layout) with buffer loads,
//   unpacks them once into LDS (double-buffered), and every wave reads its MFMA
//   operands from there.  Global loads run two stages ahead in registers.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace svdq {
namespace {

using namespace dev;

template <int TM_, int TN_, int WM_, int WN_, int KG_, int WPE_>
struct GemmCfg {
  static constexpr int TM = TM_, TN = TN_;  // workgroup tile: rows (tokens) x output columns
  static constexpr int WM = WM_, WN = WN_;  // wave tile
  static constexpr int KG = KG_;            // channel groups per LDS stage
  static constexpr int WPE = WPE_;          // waves per SIMD the register budget must allow
  static constexpr int WAVES_N = TN / WN;
  static constexpr int NT = 64 * (TM / WM) * WAVES_N;
  static constexpr int BI = WM / 16, BJ = WN / 16;
  static constexpr int A_BYTES = TM * 32 / NT;  // packed activation bytes staged per thread per group
  static constexpr int B_BYTES = TN * 32 / NT;  // packed weight bytes staged per thread per group
  static constexpr int ROWB = 64 + 16;          // LDS bytes per unpacked 64-channel row (+16 pad)
  static constexpr int STAGE_A = KG * TM * ROWB, STAGE_B = KG * TN * ROWB;
  static_assert(A_BYTES == 4 || A_BYTES == 8 || A_BYTES == 16, "activation staging piece");
  static_assert(B_BYTES == 4 || B_BYTES == 8 || B_BYTES == 16, "weight staging piece");
  static_assert(NT >= TM + TN && TM % 64 == 0 && (TM + TN) % 64 == 0, "scale staging");
};

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

template <int BYTES>
__device__ __forceinline__ Piece<BYTES> buffer_piece(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  Piece<BYTES> p;
  if constexpr (BYTES == 16) {
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

// Unpack a piece starting at word w0 of a record into the LDS row `row`: the
// low nibbles of record word w go to byte 32*(w/4) + 4*(w%4), the high nibbles
// 16 bytes further, each nibble becoming the signed byte 16*q.  Activations and
// weights use the same placement, so the channel permutation cancels in the
// dot product.
template <int BYTES>
__device__ __forceinline__ void unpack_piece(uint8_t* row, int w0, const Piece<BYTES>& p) {
  constexpr int NW = BYTES / 4;
  uint8_t* lo_dst = row + 32 * (w0 >> 2) + 4 * (w0 & 3);
  uint32_t lo[NW], hi[NW];
#pragma unroll
  for (int e = 0; e < NW; ++e) {
    lo[e] = (p.w[e] << 4) & 0xF0F0F0F0u;
    hi[e] = p.w[e] & 0xF0F0F0F0u;
  }
  if constexpr (NW == 4) {
    *reinterpret_cast<u32x4*>(lo_dst) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<u32x4*>(lo_dst + 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  } else if constexpr (NW == 2) {
    *reinterpret_cast<uint2*>(lo_dst) = uint2{lo[0], lo[1]};
    *reinterpret_cast<uint2*>(lo_dst + 16) = uint2{hi[0], hi[1]};
  } else {
    *reinterpret_cast<uint32_t*>(lo_dst) = lo[0];
    *reinterpret_cast<uint32_t*>(lo_dst + 16) = hi[0];
  }
}

// Workgroup -> tile.  Workgroups are dealt round-robin to the 8 XCDs, so give
// each XCD a contiguous range of tiles, ordered in bands of 4 tile-rows
// (column-major inside a band) so that concurrently running workgroups of one
// XCD share activation and weight tiles in its L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& ti, int& tj) {
  const int T = tiles_m * tiles_n;
  const int xcd = bid & 7, k = bid >> 3;
  const int per = T >> 3, extra = T & 7;
  const int t = xcd < extra ? xcd * (per + 1) + k : extra * (per + 1) + (xcd - extra) * per + k;
  constexpr int GM = 4;
  const int band = t / (GM * tiles_n);
  const int first = band * GM;
  const int gm = min(tiles_m - first, GM);
  const int in_band = t - band * GM * tiles_n;
  ti = first + in_band % gm;
  tj = in_band / gm;
}

template <class C, bool OUT_BF16>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void gemm_w4a4_up_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ ascale,
    const float* __restrict__ z, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, int b, int n, int G, int rank, int tiles_m, int tiles_n,
    void* __restrict__ yout) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN, KG = C::KG;
  constexpr int BI = C::BI, BJ = C::BJ, ROWB = C::ROWB;
  __shared__ __align__(16) uint8_t As[2][C::STAGE_A];
  __shared__ __align__(16) uint8_t Bs[2][C::STAGE_B];
  __shared__ __align__(16) float Sxq[2][KG][TM];  // sx / 256
  __shared__ __align__(16) float Sng[2][KG][TM];  // -1.5*2^23 * sx / 256
  __shared__ __align__(16) float Sw[2][KG][TN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r = lane & 15, c = lane >> 4;
  int ti, tj;
  tile_of(blockIdx.x, tiles_m, tiles_n, ti, tj);
  const int i0 = ti * TM, j0 = tj * TN;

  f32x4 acc[BI][BJ];
#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj) acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- low-rank branch: acc = bf16(Z) L2 over K = rank in chunks of 32 -------
  // 16-byte loads when every row of l2 / z starts 16-byte aligned
  const bool l2_vec = (rank % 8) == 0 && ((uintptr_t)l2t & 15u) == 0;
  const bool z_vec = (rank % 4) == 0 && ((uintptr_t)z & 15u) == 0;
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

  // ---- main branch: exact per-group i8 MFMA + fp32 scale epilogue ----------
  // Staging: per group every thread issues the same three buffer loads: one
  // piece of an activation record, one piece of a weight record, one fp16
  // scale.  The per-group base lives in the (scalar) buffer descriptor, whose
  // size bound makes rows >= b and columns >= n read as zero.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  constexpr int AB = C::A_BYTES, BB = C::B_BYTES;
  const int a_row = tid * AB / 32, a_w0 = (tid * AB % 32) / 4;
  const int b_col = tid * BB / 32, b_w0 = (tid * BB % 32) / 4;
  const uint32_t a_voff = (uint32_t)(i0 + a_row) * 32u + 4u * a_w0;
  const uint32_t b_voff = (uint32_t)(j0 + b_col) * 32u + 4u * b_w0;
  // activation scale of row i0+tid, weight scale of column j0+tid-TM, or an
  // out-of-range offset (reads 0) for the threads that stage no scale
  const uint32_t s_voff = tid < TM ? (uint32_t)(i0 + tid) * 2u
                                   : (tid < TM + TN ? (uint32_t)(j0 + tid - TM) * 2u : 0x7FFFFFF0u);
  const uint32_t a_bytes = (uint32_t)b * 32u, b_bytes = (uint32_t)n * 32u;

  struct Stage {
    Piece<AB> a[KG];
    Piece<BB> w[KG];
    uint32_t s[KG];
  };
  const int S = (G + KG - 1) / KG;  // stages
  auto load_stage = [&](int st_idx, Stage& st) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int g = min(st_idx * KG + kg, G - 1);
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(qx + (size_t)g * a_bytes, a_bytes);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(qw + (size_t)g * b_bytes, b_bytes);
      // wave-uniform choice (waves 0 .. TM/64-1 stage activation scales), so the
      // descriptor stays in scalar registers
      const __amdgpu_buffer_rsrc_t rs =
          wave_u < TM / 64 ? make_rsrc(ascale + (size_t)g * b, (uint32_t)b * 2u)
                           : make_rsrc(wscale + (size_t)g * n, (uint32_t)n * 2u);
      st.a[kg] = buffer_piece<AB>(ra, a_voff);
      st.w[kg] = buffer_piece<BB>(rb, b_voff);
      st.s[kg] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_voff, 0, 0);
    }
  };
  auto store_stage = [&](int buf, const Stage& st) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      unpack_piece<AB>(&As[buf][(kg * TM + a_row) * ROWB], a_w0, st.a[kg]);
      unpack_piece<BB>(&Bs[buf][(kg * TN + b_col) * ROWB], b_w0, st.w[kg]);
      const float sv = f16_to_f32((uint16_t)st.s[kg]);
      if (wave_u < TM / 64) {
        const float q = sv * 0.00390625f;  // sx / 256 (exact)
        Sxq[buf][kg][tid] = q;
        Sng[buf][kg][tid] = -kMagic * q;   // exact: 3 * 2^14 * sx
      } else if (wave_u < (TM + TN) / 64) {
        Sw[buf][kg][tid - TM] = sv;
      }
    }
  };

  const i32x4 magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  // One group: for each 16-row block bi, BJ MFMAs (one per 16-column block) and
  // 8*BJ FMAs.  The MFMAs of block bi are issued next to the FMAs of block bi-1
  // (software pipeline).  The empty asm statements take the updated
  // accumulators as operands: they emit nothing but pin each block's FMAs in
  // place, so the compiler cannot sink them past later MFMAs (which would keep
  // every MFMA result live at once).
  auto compute_group = [&](const uint8_t* Ab, const uint8_t* Bb, const float* sxq_s,
                           const float* sng_s, const float* sw_s) {
    u32x4 Pb[BJ];
    f32x4 sw4[BJ];
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj) {
      const int cc = WN * wn + 16 * bj;
      Pb[bj] = *reinterpret_cast<const u32x4*>(&Bb[(cc + r) * ROWB + 16 * c]);
      sw4[bj] = *reinterpret_cast<const f32x4*>(&sw_s[cc + 4 * c]);
    }
    const int rbase = WM * wm + r;
    u32x4 Qa = *reinterpret_cast<const u32x4*>(&Ab[rbase * ROWB + 16 * c]);
    i32x4 d[2][BJ];
    float sxq[2], sng[2];
#pragma unroll
    for (int bi = 0; bi <= BI; ++bi) {
      const int cur = bi & 1, prev = cur ^ 1;
      u32x4 Qn = Qa;
      if (bi < BI) {
        const int rr = rbase + 16 * bi;
        sxq[cur] = sxq_s[rr];
        sng[cur] = sng_s[rr];
        if (bi + 1 < BI) Qn = *reinterpret_cast<const u32x4*>(&Ab[(rr + 16) * ROWB + 16 * c]);
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj)
          d[cur][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              __builtin_bit_cast(i32x4, Pb[bj]), __builtin_bit_cast(i32x4, Qa), magic, 0, 0, 0);
      }
      if (bi > 0) {
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float t = __builtin_fmaf(__int_as_float(d[prev][bj][v]), sxq[prev], sng[prev]);
            acc[bi - 1][bj][v] = __builtin_fmaf(t, sw4[bj][v], acc[bi - 1][bj][v]);
          }
          asm volatile("" : "+v"(acc[bi - 1][bj]));
        }
      }
      Qa = Qn;
    }
  };
  auto compute = [&](int buf, int st_idx) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      if (KG == 1 || st_idx * KG + kg < G)
        compute_group(&As[buf][kg * TM * ROWB], &Bs[buf][kg * TN * ROWB], Sxq[buf][kg], Sng[buf][kg],
                      Sw[buf][kg]);
    }
  };

  // pipeline: LDS[s & 1] holds stage s; register stage st[(s + 1) & 1] holds
  // stage s + 1; stage st[s & 1] has stage s + 2 in flight.  Loads and stores
  // in the loop are unconditional (past the end they re-read the last group
  // into a buffer nobody reads), so no branch sits between a load and its use
  // and each wait covers exactly one stage.
  Stage st0, st1;
  load_stage(0, st0);
  load_stage(min(1, S - 1), st1);
  store_stage(0, st0);
  load_stage(min(2, S - 1), st0);
  __syncthreads();
  int s = 0;
  for (; s + 1 < S; s += 2) {
    compute(0, s);
    store_stage(1, st1);
    load_stage(min(s + 3, S - 1), st1);
    __syncthreads();
    compute(1, s + 1);
    store_stage(0, st0);
    load_stage(min(s + 4, S - 1), st0);
    __syncthreads();
  }
  if (s < S) compute(0, s);

  // ---- epilogue: bias, cast, one store of Y ---------------------------------
  // lane holds Y[i][j..j+3]: i = row (l & 15) of block bi, j = 4 (l >> 4) of block bj
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
}

template <class C>
int launch_cfg(const uint8_t* qx, const uint16_t* ascale, const float* z, const svdq_layer& L, int b,
               void* y, int y_dtype, hipStream_t st) {
  const int G = L.m / 64;
  const int tiles_n = (L.n + C::TN - 1) / C::TN;
  const int tiles_m = (b + C::TM - 1) / C::TM;
  dim3 grid((unsigned)(tiles_n * tiles_m));
  if (y_dtype == SVDQ_OUT_BF16)
    hipLaunchKernelGGL((gemm_w4a4_up_kernel<C, true>), grid, dim3(C::NT), 0, st, qx, ascale, z, L.qw,
                       L.wscale, L.l2, L.bias, b, L.n, G, L.rank, tiles_m, tiles_n, y);
  else
    hipLaunchKernelGGL((gemm_w4a4_up_kernel<C, false>), grid, dim3(C::NT), 0, st, qx, ascale, z, L.qw,
                       L.wscale, L.l2, L.bias, b, L.n, G, L.rank, tiles_m, tiles_n, y);
  return (int)hipGetLastError();
}

// 128 x 128 tile, 4 waves of 64 x 64; two workgroups share a CU, so one
// workgroup's barrier and LDS-latency phases overlap the others' compute.
using CfgBig = GemmCfg<128, 128, 64, 64, 1, 2>;

}  // namespace

int launch_gemm_up(const uint8_t* qx, const uint16_t* ascale, const float* z, const svdq_layer& L,
                   int b, void* y, int y_dtype, void* stream) {
  return launch_cfg<CfgBig>(qx, ascale, z, L, b, y, y_dtype, (hipStream_t)stream);
}

}  // namespace svdq
