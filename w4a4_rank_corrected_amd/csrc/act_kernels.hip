// Activation-side kernels: calibration statistic, the fused activation
// quantization + low-rank down-projection (first fused pair of Nunchaku), the
// per-token INT8 quantizer of the 8-bit setting, and the ordered reduction of
// split partial sums.
//
// [Review] = "SVDQuant: How a Small High-Precision Branch Makes 4-Bit Diffusion
// Practical" (technical review of arXiv:2411.05007v4).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace svdq {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// calibration: amax[k] = max_i |x[i][k]|  ([Review] sec. 3.1, Eq.(4) statistics)
// |x| >= 0, so the IEEE bit patterns order like unsigned integers and an
// integer atomic max is exact and order-independent.
// ---------------------------------------------------------------------------
__global__ void fill_zero_kernel(float* p, int count) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.0f;
}

__global__ __launch_bounds__(256) void calibrate_kernel(const uint16_t* __restrict__ x, int b, int m,
                                                        float* __restrict__ amax, int rows_per_block) {
  const int chunk = blockIdx.x * blockDim.x + threadIdx.x;  // 8 channels per thread
  if (chunk * 8 >= m) return;
  const int r0 = blockIdx.y * rows_per_block;
  const int r1 = min(b, r0 + rows_per_block);
  float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0; r < r1; ++r) {
    u32x4 w = ldg16(x + (size_t)r * m + chunk * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx[2 * e] = fmaxf(mx[2 * e], fabsf(bf16_lo(w[e])));
      mx[2 * e + 1] = fmaxf(mx[2 * e + 1], fabsf(bf16_hi(w[e])));
    }
  }
  if (r0 >= r1) return;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    atomicMax(reinterpret_cast<unsigned int*>(amax) + chunk * 8 + e, __float_as_uint(mx[e]));
}

// ---------------------------------------------------------------------------
// Fused activation quantization + low-rank down-projection
// ([Review] sec. 6.1 Algorithm 2 steps 1-3; Fig. 4 first pair; Eq.(1), Eq.(3)).
//
// Workgroup = 4 waves over 64 rows (one 16-row strip per wave) and a
// contiguous range of gps channel groups (one split), walked in chunks of
// `chunk` groups (at most about 40 KB of LDS): the workgroup stages a chunk's 1/lambda and L1 slices in LDS
// (shared by the four waves), then each wave processes the chunk for its strip.
// Activations stream through a register ring D groups ahead, across chunk
// boundaries, and each wave owns its rows' Z (no cross-wave reduction).  In one wave, lane l owns row (l & 15) and, in each 64-channel
// group, channels 8c..8c+7 and 32+8c..32+8c+7 with c = l >> 4: exactly the
// bf16 MFMA A-operand layout, so the smoothed bf16 tile feeds both the
// quantizer and the down-projection.  Global loads go through buffer
// descriptors whose size covers exactly what may be read, so rows >= b,
// ranks >= rank and loads past the last group read zero without touching
// memory.
//
// Per element:  x~ = bf16(fl32(x * inv))
// Per row/group: s = fp16(fl32(amax / 7)) (saturated), r = fl32(1 / s)
// Per element:  q = clamp(round_even(x~ / s), -7, 7), computed without a divide:
//   p = fl(x~ r); e = fma(-p, s, x~) (exact remainder); q1 = fma(e, r, p)
//   q1 equals the correctly rounded quotient fl32(x~ / s) for every bf16 x~ and
//   fp16 s the kernel can meet (one Newton correction; proven on the host by
//   exhaustive enumeration in the tests), so round_even(q1) matches the
//   definition.
// ---------------------------------------------------------------------------
constexpr int kL1Pitch = kActL1Pitch;  // dynamic LDS: gps groups of act_lds_group_bytes(TB)

// TB: 16-column blocks of Z (rank <= 16 * TB; 0 = no low-rank branch);
// SMOOTH: multiply by 1/lambda (inv != nullptr); Q: the codes and scales
// emitted (kActQuantNone: the down-projection alone, the unfused path's and the
// 8-bit setting's separate kernel; kActQuantInt4; kActQuantFp4).

// FP8 E4M3 rounding of x >= 0 (nearest, ties to even, saturated at 448): the
// quantum is 2^(e-3) in the binade [2^e, 2^(e+1)) for e >= -6, 2^-9 below.
__device__ __forceinline__ float e4m3_round(float x) {
  if (!(x < 448.0f)) return 448.0f;
  const int e = max((int)((__float_as_uint(x) >> 23) & 0xFF) - 127, -6);
  const float down = __uint_as_float((uint32_t)(127 - (e - 3)) << 23);  // 2^-(e-3), exact
  const float up = __uint_as_float((uint32_t)(127 + (e - 3)) << 23);    // 2^(e-3)
  return fminf(__builtin_rintf(x * down) * up, 448.0f);
}

// Bit pattern of a non-negative E4M3 value.
__device__ __forceinline__ uint32_t e4m3_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  const int e = (int)((u >> 23) & 0xFF) - 127;
  if (v == 0.0f) return 0u;
  if (e >= -6) return ((uint32_t)(e + 7) << 3) | ((u >> 20) & 7u);
  return (uint32_t)(v * 512.0f);  // subnormal: v = m 2^-9, m = 1..7 (exact)
}

// Quantizes one row-group piece of the smoothed tile and stores its codes and
// scale (INT4 or NVFP4; nothing for kActQuantNone).  v: this lane's 16
// smoothed bf16 values (channels 8c..8c+7 and 32+8c..32+8c+7 of group g of
// row `row`), in the lane layout of the act-quant kernels: lanes l, l ^ 16,
// l ^ 32, l ^ 48 hold the same row.  q_off / s_off: this lane's byte offsets
// of its code words and of the row's scale in the group's records.
template <int Q>
__device__ __forceinline__ void quant_store(const float (&v)[16], int g, int b, int row, int c, uint32_t q_off,
                                            uint32_t s_off, uint8_t* __restrict__ qx,
                                            uint16_t* __restrict__ ascale, float tx) {
  if constexpr (Q == kActQuantFp4) {
    // NVFP4: blocks of 16 channels; this lane holds half of block c >> 1
    // (v[0..7]) and half of block 2 + (c >> 1) (v[8..15]), lane l ^ 16 the
    // other halves.  sb = E4M3(fl32(amax / 6) / t), S = sb t (t a power of
    // two), codes E2M1_RNE_sat(fl32(v / S)) with the quotient's sign.
    float am[2] = {0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 16; ++e) am[e >> 3] = fmaxf(am[e >> 3], fabsf(v[e]));
    uint32_t w[2];
    uint32_t sbits[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float a = fmaxf(am[h], __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(am[h]), 0x401F)));
      const float u = a / 6.0f;                    // IEEE division (correctly rounded)
      const float sb = e4m3_round(u * (1.0f / tx));  // 1/t and the product are exact
      sbits[h] = e4m3_bits(sb);
      const float S = sb * tx;                      // exact
      const float rc = S > 0.0f ? 1.0f / S : 0.0f;
      const float S8 = 8.0f * S;
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float vv = v[8 * h + e];
        const float pq = vv * rc;
        const float rem = __builtin_fmaf(-pq, S, vv);
        const float q1 = __builtin_fmaf(rem, rc, pq);
        y[e] = S > 0.0f ? __builtin_copysignf(fabsf(vv) <= S8 ? q1 : 8.0f, vv) : 0.0f;
      }
      // two codes per byte, the even channel in the low nibble (RNE on the
      // E2M1 grid, saturating: the hardware conversion at unit scale)
      uint32_t word = 0u;
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[0], y[1], 1.0f, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[2], y[3], 1.0f, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[4], y[5], 1.0f, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[6], y[7], 1.0f, 3);
      w[h] = word;
    }
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qx + (size_t)g * b * 32, (uint32_t)b * 32u);
    __builtin_amdgcn_raw_buffer_store_b32(w[0], rq, q_off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(w[1], rq, q_off + 16u, 0, 0);
    // block scales: record [m/64][b][4] bytes, byte j = block j; the lanes
    // with even c store blocks c/2 and 2 + c/2 (odd c: an offset past the
    // end, dropped)
    uint8_t* sc8 = reinterpret_cast<uint8_t*>(ascale);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sc8 + (size_t)g * b * 4, (uint32_t)b * 4u);
    const uint32_t s8_off = (c & 1) == 0 ? (uint32_t)row * 4u + (uint32_t)(c >> 1) : 0x7FFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbits[0], rs, s8_off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbits[1], rs, s8_off + 2u, 0, 0);
  }
  if constexpr (Q == kActQuantInt4) {
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(v[e]));
    am = max4_rows(am);
    float s32 = am / 7.0f;                 // IEEE division (correctly rounded)
    s32 = fminf(s32, 65504.0f);            // saturate instead of rounding to inf
    const _Float16 s16 = (_Float16)s32;    // round to nearest even
    const float sf = (float)s16;
    const float rc = sf > 0.0f ? 1.0f / sf : 0.0f;
    // rb[e]: the bits of q + 1.5 * 2^23, whose low byte is the code in two's
    // complement (the addition rounds to the nearest integer, ties to even)
    uint32_t rb[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pq = v[e] * rc;
      const float rem = __builtin_fmaf(-pq, sf, v[e]);
      const float q1 = __builtin_fmaf(rem, rc, pq);
      const float q = __builtin_amdgcn_fmed3f(q1, -7.0f, 7.0f);
      rb[e] = __float_as_uint(q + kMagic);
    }
    // Nibble e of a word (bits 4e..4e+3) is code e: byte permutes gather the
    // even codes' and the odd codes' low bytes into two words, then one
    // bitfield insert takes the low nibbles of the first and the shifted low
    // nibbles of the second.
    auto pack8 = [](const uint32_t* c8) {
      const uint32_t e01 = __builtin_amdgcn_perm(c8[2], c8[0], 0x0c0c0400u);  // bytes: c0, c2, 0, 0
      const uint32_t e23 = __builtin_amdgcn_perm(c8[6], c8[4], 0x04000c0cu);  // bytes: 0, 0, c4, c6
      const uint32_t o01 = __builtin_amdgcn_perm(c8[3], c8[1], 0x0c0c0400u);
      const uint32_t o23 = __builtin_amdgcn_perm(c8[7], c8[5], 0x04000c0cu);
      return ((e01 | e23) & 0x0F0F0F0Fu) | (((o01 | o23) << 4) & 0xF0F0F0F0u);
    };
    const uint32_t w0 = pack8(rb), w1 = pack8(rb + 8);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qx + (size_t)g * b * 32, (uint32_t)b * 32u);
    __builtin_amdgcn_raw_buffer_store_b32(w0, rq, q_off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(w1, rq, q_off + 16u, 0, 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(ascale + (size_t)g * b, (uint32_t)b * 2u);
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, s16), rs, s_off, 0, 0);
  }
}

template <int TB, bool SMOOTH, int Q>
__global__ __launch_bounds__(256) void act_quant_down_kernel(
    const uint16_t* __restrict__ x, int b, int m, int G, const float* __restrict__ inv,
    const uint16_t* __restrict__ l1t, int rank, uint8_t* __restrict__ qx,
    uint16_t* __restrict__ ascale, float* __restrict__ zout, int gps, float tx) {
  constexpr int NB = TB > 0 ? TB : 1;
  constexpr int GB = act_lds_group_bytes(TB);
  constexpr int chunk = act_chunk(TB);
  __shared__ __align__(16) uint8_t lds[chunk * GB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int split = blockIdx.y;
  const int g_begin = split * gps;
  const int g_end = min(G, g_begin + gps);
  const int ng = g_end - g_begin;

  // Staging of 1/lambda and the L1 slices of groups [cb, ce) in LDS: each
  // part's loads all go out before its LDS writes.  A wave's loads complete
  // in issue order, so the first chunk's staging loads are issued before the
  // activation loads: the waves then wait only for the staging data before
  // the barrier, and start on their first group while the rest of the
  // activations are still arriving.
  constexpr int SP = TB > 0 ? (chunk * TB * 16 * 8 + 255) / 256 : 1;  // L1 pieces per thread
  auto inv_load = [&](int cb, int ce) {
    static_assert(chunk * 16 <= 256, "one 1/lambda piece per thread");
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(inv + (size_t)cb * 64, (uint32_t)(ce - cb) * 256u);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (uint32_t)tid * 16u, 0, 0));
  };
  auto inv_store = [&](const u32x4& v) {
    if (tid < chunk * 16) *reinterpret_cast<u32x4*>(lds + (tid >> 4) * GB + 16 * (tid & 15)) = v;
  };
  // L1 rows t < 16 TB (zero beyond rank), 8 pieces of 16 B per (group, t)
  auto l1_load = [&](int cb, int ce, u32x4 (&v)[SP]) {
    const int n = ce - cb;
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(l1t + (size_t)cb * 64, (uint32_t)((rank - 1) * m + n * 64) * 2u);
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      const int k = tid + 256 * i;
      const int q = k & 7, t = (k >> 3) % (TB * 16), j = (k >> 3) / (TB * 16);
      const uint32_t off = (t < rank && j < n) ? (uint32_t)(t * m + j * 64 + 8 * q) * 2u : 0xFFFFFFF0u;
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, off, 0, 0));
    }
  };
  auto l1_store = [&](const u32x4 (&v)[SP]) {
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      const int k = tid + 256 * i;
      const int q = k & 7, t = (k >> 3) % (TB * 16), j = (k >> 3) / (TB * 16);
      if (k < chunk * TB * 16 * 8) *reinterpret_cast<u32x4*>(lds + j * GB + 256 + (t * kL1Pitch + 8 * q) * 2) = v[i];
    }
  };
  auto stage = [&](int cb, int ce) {
    if constexpr (SMOOTH) inv_store(inv_load(cb, ce));
    if constexpr (TB > 0) {
      u32x4 v[SP];
      l1_load(cb, ce, v);
      l1_store(v);
    }
  };

  // Activations D groups ahead in a register ring (below).  Builds with a
  // one-group ring, for the largest ranks, keep the activation load first and
  // stage every chunk behind a leading barrier: peeling the first chunk costs
  // them registers.  Every wave runs the same barrier sequence: the first chunk
  // (kStageFirst) is staged without a leading barrier, the others with one.
  constexpr int D = act_depth(TB);
  constexpr bool kStageFirst = D > 1;

  // this wave's strip; a wave past the end only helps stage and takes part in
  // the barriers
  const int row0 = blockIdx.x * 64 + wave * 16;
  if (row0 >= b) {
    for (int cb = g_begin; cb < g_end; cb += chunk) {
      if (!kStageFirst || cb != g_begin) __syncthreads();
      stage(cb, min(cb + chunk, g_end));
      __syncthreads();
    }
    return;
  }
  const int row = row0 + r;
  const int rows_here = min(16, b - row0);
  const uint32_t x_bytes = (uint32_t)((rows_here - 1) * m + 64) * 2u;  // per group, from its base
  const uint32_t x_off = (uint32_t)(r * m + 8 * c) * 2u;              // + 64 for channels 32+8c..
  auto load_x = [&](int g, u32x4& xa, u32x4& xb) {
    const bool live = g < g_end;
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(x + (size_t)row0 * m + (size_t)(live ? g : g_begin) * 64, live ? x_bytes : 0u);
    xa = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off, 0, 0));
    xb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off + 64u, 0, 0));
  };

  f32x4 acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // code records and scales of group g are written through descriptors that
  // end at row b, so stores of rows >= b (and of lanes c != 0 for the scale)
  // are dropped by the hardware range check: straight-line code per group
  const uint32_t q_off = (uint32_t)row * 32u + 4u * c;
  const uint32_t s_off = c == 0 ? (uint32_t)row * 2u : 0xFFFFFFF0u;
  auto process = [&](int g, int j, const u32x4& xa, const u32x4& xb) {
    const uint8_t* gl = lds + j * GB;
    float v[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(xa[e]);
      v[2 * e + 1] = bf16_hi(xa[e]);
      v[8 + 2 * e] = bf16_lo(xb[e]);
      v[8 + 2 * e + 1] = bf16_hi(xb[e]);
    }
    if constexpr (SMOOTH) {
      const float* iv = reinterpret_cast<const float*>(gl);
      const f32x4 i0 = *reinterpret_cast<const f32x4*>(iv + 8 * c);
      const f32x4 i1 = *reinterpret_cast<const f32x4*>(iv + 8 * c + 4);
      const f32x4 i2 = *reinterpret_cast<const f32x4*>(iv + 32 + 8 * c);
      const f32x4 i3 = *reinterpret_cast<const f32x4*>(iv + 36 + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] *= i0[e];
        v[4 + e] *= i1[e];
        v[8 + e] *= i2[e];
        v[12 + e] *= i3[e];
      }
    }
    // materialise X~ once as bf16 (packed pairs feed the MFMA)
    uint32_t xt[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      xt[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
      v[2 * q] = bf16_lo(xt[q]);
      v[2 * q + 1] = bf16_hi(xt[q]);
    }
    quant_store<Q>(v, g, b, row, c, q_off, s_off, qx, ascale, tx);
    if constexpr (TB > 0) {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{xt[0], xt[1], xt[2], xt[3]});
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, u32x4{xt[4], xt[5], xt[6], xt[7]});
      const uint16_t* lr = reinterpret_cast<const uint16_t*>(gl + 256) + r * kL1Pitch + 8 * c;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(lr + tb * 16 * kL1Pitch);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(lr + tb * 16 * kL1Pitch + 32);
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, b0), acc[tb], 0, 0, 0);
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, b1), acc[tb], 0, 0, 0);
      }
    }
  };

  // x D groups ahead in a register ring: slot u holds the groups g with
  // (g - g_begin) % D == u.  chunk is a multiple of D, so every chunk starts
  // at slot 0 and only the split's last chunk ends early.
  u32x4 xa[D], xb[D];
  if constexpr (kStageFirst) {
    const int ce = min(g_begin + chunk, g_end);
    u32x4 iv = {0u, 0u, 0u, 0u}, lv[SP];
    if constexpr (SMOOTH) iv = inv_load(g_begin, ce);
    if constexpr (TB > 0) l1_load(g_begin, ce, lv);
#pragma unroll
    for (int u = 0; u < D; ++u) load_x(g_begin + u, xa[u], xb[u]);
    if constexpr (SMOOTH) inv_store(iv);
    if constexpr (TB > 0) l1_store(lv);
    __syncthreads();
  } else {
#pragma unroll
    for (int u = 0; u < D; ++u) load_x(g_begin + u, xa[u], xb[u]);
  }
  for (int cb = g_begin; cb < g_end; cb += chunk) {
    const int ce = min(cb + chunk, g_end);
    if (!kStageFirst || cb != g_begin) {
      __syncthreads();  // every wave is done with the previous chunk
      stage(cb, ce);
      __syncthreads();
    }
    int g = cb;
    for (; g + D <= ce; g += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        process(g + u, g + u - cb, xa[u], xb[u]);
        load_x(g + u + D, xa[u], xb[u]);
      }
    }
#pragma unroll
    for (int u = 0; u + 1 < D; ++u)
      if (g + u < ce) process(g + u, g + u - cb, xa[u], xb[u]);
  }

  if constexpr (TB > 0) {
    // this split's Z for the strip (MFMA D layout: row 4c+v, column l & 15)
    float* zs = zout + (size_t)split * b * rank;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = tb * 16 + r;
      if (t < rank) {
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int zr = row0 + 4 * c + vv;
          if (zr < b) zs[(size_t)zr * rank + t] = acc[tb][vv];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same computation for many rows (a few thousand): a workgroup of 8
// waves owns 16 rows, and the waves split the channel groups (wave w takes
// groups w, w + 8, w + 16, ...), so each row's Z is complete inside one
// workgroup: the waves' partial Z tiles are added in LDS in wave order and
// stored once (no split partials in memory, no reduction launch).  Each wave
// streams its groups through a register ring D groups ahead: the activation
// piece, its L1 operand pieces (16 B per Z block and channel half; L1 is small
// and stays in L2) and the group's 64 values of 1/lambda (one dword per lane,
// passed through a 256-byte LDS slot of the wave to reach the lanes that use
// them).  The waves never wait for each other before the final reduction.
// Per element and per row/group the arithmetic is the act-quant kernel's
// (quant_store); Z is summed over groups in a fixed order for a shape.
// ---------------------------------------------------------------------------
constexpr int kWideWaves = kWideWavesPlan;
template <int TB, bool SMOOTH, int Q>
__global__ __launch_bounds__(64 * kWideWaves) void act_quant_wide_kernel(
    const uint16_t* __restrict__ x, int b, int m, int G, const float* __restrict__ inv,
    const uint16_t* __restrict__ l1t, int rank, uint8_t* __restrict__ qx,
    uint16_t* __restrict__ ascale, float* __restrict__ zout, float tx) {
  constexpr int NW = kWideWaves;
  constexpr int NB = TB > 0 ? TB : 1;
  constexpr int D = 2;
  __shared__ __align__(16) float s_inv[NW][64];
  __shared__ __align__(16) float s_z[TB > 0 ? NW * 16 * 16 * TB : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + r;
  const int rows_here = min(16, b - row0);
  const uint32_t x_bytes = (uint32_t)((rows_here - 1) * m + 64) * 2u;
  const uint32_t x_off = (uint32_t)(r * m + 8 * c) * 2u;
  const uint32_t l1_bytes = TB > 0 ? (uint32_t)((rank - 1) * m + 64) * 2u : 0u;
  const int nj = wave < G ? (G - wave + NW - 1) / NW : 0;  // groups of this wave

  struct Stage {
    u32x4 xa, xb;
    u32x4 la[NB], lb[NB];  // L1 rows tb*16 + r, channels 8c.. and 32 + 8c..
    uint32_t iv;           // 1/lambda of channel `lane` of the group
  };
  auto load = [&](int j, Stage& st) {
    const bool live = j < nj;
    const int g = live ? wave + NW * j : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)row0 * m + (size_t)g * 64, live ? x_bytes : 0u);
    st.xa = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off, 0, 0));
    st.xb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off + 64u, 0, 0));
    if constexpr (TB > 0) {
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(l1t + (size_t)g * 64, live ? l1_bytes : 0u);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int t = tb * 16 + r;
        const uint32_t off = t < rank ? (uint32_t)(t * m + 8 * c) * 2u : 0xFFFFFFF0u;
        st.la[tb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, off, 0, 0));
        st.lb[tb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, off + 64u, 0, 0));
      }
    }
    if constexpr (SMOOTH) {
      const __amdgpu_buffer_rsrc_t ri = make_rsrc(inv + (size_t)g * 64, live ? 256u : 0u);
      st.iv = __builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)lane * 4u, 0, 0);
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t q_off = (uint32_t)row * 32u + 4u * c;
  const uint32_t s_off = c == 0 ? (uint32_t)row * 2u : 0xFFFFFFF0u;

  auto process = [&](int j, const Stage& st) {
    const int g = wave + NW * j;
    float v[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(st.xa[e]);
      v[2 * e + 1] = bf16_hi(st.xa[e]);
      v[8 + 2 * e] = bf16_lo(st.xb[e]);
      v[8 + 2 * e + 1] = bf16_hi(st.xb[e]);
    }
    if constexpr (SMOOTH) {
      // the wave's own slot: LDS accesses of one wave complete in order, so
      // the previous group's reads finish before this write lands
      s_inv[wave][lane] = __uint_as_float(st.iv);
      const float* iv = s_inv[wave];
      const f32x4 i0 = *reinterpret_cast<const f32x4*>(iv + 8 * c);
      const f32x4 i1 = *reinterpret_cast<const f32x4*>(iv + 8 * c + 4);
      const f32x4 i2 = *reinterpret_cast<const f32x4*>(iv + 32 + 8 * c);
      const f32x4 i3 = *reinterpret_cast<const f32x4*>(iv + 36 + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] *= i0[e];
        v[4 + e] *= i1[e];
        v[8 + e] *= i2[e];
        v[12 + e] *= i3[e];
      }
    }
    uint32_t xt[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      xt[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
      v[2 * q] = bf16_lo(xt[q]);
      v[2 * q + 1] = bf16_hi(xt[q]);
    }
    quant_store<Q>(v, g, b, row, c, q_off, s_off, qx, ascale, tx);
    if constexpr (TB > 0) {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{xt[0], xt[1], xt[2], xt[3]});
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, u32x4{xt[4], xt[5], xt[6], xt[7]});
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, st.la[tb]), acc[tb], 0, 0, 0);
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, st.lb[tb]), acc[tb], 0, 0, 0);
      }
    }
  };

  if (row0 < b) {
    Stage st[D];
#pragma unroll
    for (int u = 0; u < D; ++u) load(u, st[u]);
    int j = 0;
    for (; j + D <= nj; j += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        process(j + u, st[u]);
        load(j + u + D, st[u]);
      }
    }
#pragma unroll
    for (int u = 0; u + 1 < D; ++u)
      if (j + u < nj) process(j + u, st[u]);
  }

  if constexpr (TB > 0) {
    // partial Z of each wave (MFMA D layout: row 4c + v, column 16 tb + r),
    // then Z[row0 + i][t] = sum over waves in order
    constexpr int ZC = 16 * TB;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) s_z[(wave * 16 + 4 * c + vv) * ZC + tb * 16 + r] = acc[tb][vv];
    __syncthreads();
    for (int e = tid; e < 16 * ZC; e += 64 * NW) {
      const int i = e / ZC, t = e - i * ZC;
      float zsum = s_z[i * ZC + t];
#pragma unroll
      for (int w = 1; w < NW; ++w) zsum += s_z[(w * 16 + i) * ZC + t];
      if (row0 + i < b && t < rank) zout[(size_t)(row0 + i) * rank + t] = zsum;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-token INT8 codes of X~ (the 8-bit setting: [Review] sec. 8, with the
// quantizer of Eq.(1) and 127 in place of 7).  A row's scale needs the maximum
// over all of its m channels, so one wave owns one row: lane l handles the
// 8-channel pieces p = l, l + 64, ... (each wave step reads 1 KB of the row,
// coalesced).  Pass 1 smooths the pieces to bf16, keeping them in registers
// when the row fits in RP pieces per lane, and reduces max |x~| over the wave;
// then s = fp16(fl32(amax / 127)) (saturated) and r = fl32(1 / s).  Pass 2
// quantizes with the same division-free quotient as the INT4 kernel (checked
// exhaustively on the host for codes up to 127 as well):
//   p = fl(x~ r); e = fma(-p, s, x~); q = med3(fma(e, r, p), -127, 127)
// and stores 8 codes per lane: piece p lies in channel group p / 8, at byte
// 8 (p % 8) of the row's 64-byte record [m/64][b][64].
// ---------------------------------------------------------------------------
template <int RP>  // pieces per lane kept in registers (0: smooth the row again in pass 2)
__global__ __launch_bounds__(256) void act8_quant_kernel(const uint16_t* __restrict__ x, int b, int m,
                                                         const float* __restrict__ inv, int8_t* __restrict__ qx,
                                                         uint16_t* __restrict__ ascale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= b) return;  // no barriers below
  const int P = m >> 3;
  const uint16_t* xr = x + (size_t)row * m;
  auto smooth = [&](int p) -> u32x4 {
    const u32x4 w = ldg16(xr + 8 * p);
    if (!inv) return w;  // x~ = x
    const f32x4 i0 = *reinterpret_cast<const f32x4*>(inv + 8 * p);
    const f32x4 i1 = *reinterpret_cast<const f32x4*>(inv + 8 * p + 4);
    return u32x4{pack_bf16x2(bf16_lo(w[0]) * i0[0], bf16_hi(w[0]) * i0[1]),
                 pack_bf16x2(bf16_lo(w[1]) * i0[2], bf16_hi(w[1]) * i0[3]),
                 pack_bf16x2(bf16_lo(w[2]) * i1[0], bf16_hi(w[2]) * i1[1]),
                 pack_bf16x2(bf16_lo(w[3]) * i1[2], bf16_hi(w[3]) * i1[3])};
  };
  auto piece_max = [](const u32x4& v, float am) {
#pragma unroll
    for (int e = 0; e < 4; ++e) am = fmaxf(am, fmaxf(fabsf(bf16_lo(v[e])), fabsf(bf16_hi(v[e]))));
    return am;
  };
  float sf = 0.0f, rc = 0.0f;
  auto set_scale = [&](float am) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    float s32 = am / 127.0f;               // IEEE division (correctly rounded)
    s32 = fminf(s32, 65504.0f);            // saturate instead of rounding to inf
    const _Float16 s16 = (_Float16)s32;    // round to nearest even
    sf = (float)s16;
    rc = sf > 0.0f ? 1.0f / sf : 0.0f;
    if (lane == 0) ascale[row] = __builtin_bit_cast(uint16_t, s16);
  };
  auto quant = [&](int p, const u32x4& v) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float val = (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
      const float pq = val * rc;
      const float rem = __builtin_fmaf(-pq, sf, val);
      const float q = __builtin_amdgcn_fmed3f(__builtin_fmaf(rem, rc, pq), -127.0f, 127.0f);
      w[e >> 2] |= (__float_as_uint(q + kMagic) & 0xFFu) << (8 * (e & 3));
    }
    *reinterpret_cast<uint2*>(qx + ((size_t)(p >> 3) * b + row) * 64 + 8 * (p & 7)) = uint2{w[0], w[1]};
  };
  if constexpr (RP > 0) {
    u32x4 v[RP];
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < RP; ++k) {  // loads unconditional (clamped), so all are in flight together
      const int p = 64 * k + lane;
      v[k] = smooth(p < P ? p : P - 1);
      if (p < P) am = piece_max(v[k], am);
    }
    set_scale(am);
#pragma unroll
    for (int k = 0; k < RP; ++k)
      if (64 * k + lane < P) quant(64 * k + lane, v[k]);
  } else {
    float am = 0.0f;
    for (int p = lane; p < P; p += 64) am = piece_max(smooth(p), am);
    set_scale(am);
    for (int p = lane; p < P; p += 64) quant(p, smooth(p));
  }
}

// z[i][t] = the splits' partial sums zpart[s][i][t] added in one fixed order:
// chunk c (c = 0..15) sums the splits s = c, c + 16, c + 32, ... in turn, then
// the chunks' sums are added in chunk order (with at most 16 splits this is
// simply split 0, then 1, 2, ...).  The kernels below all add in exactly this
// order, so which of them runs (it depends on alignment) changes no bit.
constexpr int kZChunks = 16;

// At most 16 splits (one per chunk: the order is split 0, 1, 2, ...): each
// thread handles 4 consecutive elements (16-byte loads and stores) and issues
// all of its loads before adding them.
__global__ void z_reduce_kernel(const float* __restrict__ zpart, int splits, size_t count,
                                float* __restrict__ z) {
  const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (idx >= count) return;
  f32x4 v[kZChunks];
#pragma unroll
  for (int u = 0; u < kZChunks; ++u)
    if (u < splits) v[u] = *reinterpret_cast<const f32x4*>(zpart + (size_t)u * count + idx);
  f32x4 s = v[0];
#pragma unroll
  for (int u = 1; u < kZChunks; ++u)
    if (u < splits) s += v[u];
  *reinterpret_cast<f32x4*>(z + idx) = s;
}

// More than 16 splits (few rows, many channel groups): a workgroup takes 16
// units of 4 consecutive elements, and thread (unit u, chunk c) issues the
// loads of its chunk's splits at once, so the partials cost one or two memory
// latencies instead of one per 16 splits.
__global__ __launch_bounds__(256) void z_reduce_chunked_kernel(const float* __restrict__ zpart, int splits,
                                                               size_t count, float* __restrict__ z) {
  __shared__ f32x4 part[kZChunks][16];
  const int u = threadIdx.x & 15, c = threadIdx.x >> 4;
  const size_t idx = ((size_t)blockIdx.x * 16 + u) * 4;
  const bool live = idx < count && c < splits;
  f32x4 q = f32x4{0.f, 0.f, 0.f, 0.f};
  if (live) {
    constexpr int B = 4;  // loads in flight per batch
    for (int s0 = c; s0 < splits; s0 += B * kZChunks) {
      f32x4 v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int sp = s0 + j * kZChunks;
        if (sp < splits) v[j] = *reinterpret_cast<const f32x4*>(zpart + (size_t)sp * count + idx);
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int sp = s0 + j * kZChunks;
        if (sp < splits) q = sp == c ? v[j] : q + v[j];
      }
    }
  }
  part[c][u] = q;
  __syncthreads();
  if (c == 0 && idx < count) {
    f32x4 zs = part[0][u];
    for (int k = 1; k < kZChunks && k < splits; ++k) zs += part[k][u];
    *reinterpret_cast<f32x4*>(z + idx) = zs;
  }
}

// The same sums one element per thread (counts or pointers that do not allow
// 16-byte accesses).
__global__ void z_reduce1_kernel(const float* __restrict__ zpart, int splits, size_t count,
                                 float* __restrict__ z) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= count) return;
  float zs = 0.0f;
  for (int c = 0; c < kZChunks && c < splits; ++c) {
    float q = zpart[(size_t)c * count + idx];
    for (int sp = c + kZChunks; sp < splits; sp += kZChunks) q += zpart[(size_t)sp * count + idx];
    zs = c == 0 ? q : zs + q;
  }
  z[idx] = zs;
}

}  // namespace

const char* hip_error_name(int err) { return hipGetErrorName((hipError_t)err); }

int launch_calibrate(const uint16_t* x, int b, int m, float* amax, int accumulate, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (!accumulate) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((m + 255) / 256), dim3(256), 0, st, amax, m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  if (b == 0) return 0;
  const int chunks = m / 8;
  const int rows_per_block = 64;
  dim3 grid((chunks + 255) / 256, (b + rows_per_block - 1) / rows_per_block);
  hipLaunchKernelGGL(calibrate_kernel, grid, dim3(256), 0, st, x, b, m, amax, rows_per_block);
  return (int)hipGetLastError();
}

int launch_act_quant_down(const uint16_t* x, int b, int m, int rank, const float* smooth_inv,
                          const uint16_t* l1, uint8_t* qx, uint16_t* ascale, float* zpart,
                          const ActPlan& plan, int qmode, float tx, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int G = m / 64;
  dim3 grid(plan.strips, plan.splits);
  const int tb = act_blocks(rank);
  if (plan.wide) {  // 16 rows per workgroup, waves over the groups; Z written directly
#define SVDQ_WIDE_Q(TBV, SM, QV)                                                                        \
  hipLaunchKernelGGL((act_quant_wide_kernel<TBV, SM, QV>), dim3(plan.strips), dim3(64 * kWideWaves), 0, st, \
                     x, b, m, G, smooth_inv, l1, rank, qx, ascale, zpart, tx)
#define SVDQ_WIDE_S(TBV, QV)          \
  do {                                \
    if (smooth_inv)                   \
      SVDQ_WIDE_Q(TBV, true, QV);     \
    else                              \
      SVDQ_WIDE_Q(TBV, false, QV);    \
  } while (0)
#define SVDQ_WIDE(TBV)                                 \
  do {                                                 \
    if (qmode == kActQuantInt4)                        \
      SVDQ_WIDE_S(TBV, kActQuantInt4);                 \
    else if (qmode == kActQuantFp4)                    \
      SVDQ_WIDE_S(TBV, kActQuantFp4);                  \
    else                                               \
      SVDQ_WIDE_S(TBV, kActQuantNone);                 \
  } while (0)
    if (tb == 0)
      SVDQ_WIDE(0);
    else if (tb == 1)
      SVDQ_WIDE(1);
    else if (tb == 2)
      SVDQ_WIDE(2);
    else if (tb == 3)
      SVDQ_WIDE(3);
    else if (tb == 4)
      SVDQ_WIDE(4);
    else
      return (int)hipErrorInvalidValue;  // the plan allows the wide kernel up to rank 64
#undef SVDQ_WIDE
#undef SVDQ_WIDE_S
#undef SVDQ_WIDE_Q
    return (int)hipGetLastError();
  }
#define SVDQ_ACT_Q(TBV, SM, QV)                                                                    \
  hipLaunchKernelGGL((act_quant_down_kernel<TBV, SM, QV>), grid, dim3(256), 0, st, x, b, m, G,     \
                     smooth_inv, l1, rank, qx, ascale, zpart, plan.groups_per_split, tx)
#define SVDQ_ACT_S(TBV, QV)           \
  do {                                \
    if (smooth_inv)                   \
      SVDQ_ACT_Q(TBV, true, QV);      \
    else                              \
      SVDQ_ACT_Q(TBV, false, QV);     \
  } while (0)
#define SVDQ_ACT(TBV)                                  \
  do {                                                 \
    if (qmode == kActQuantInt4)                           \
      SVDQ_ACT_S(TBV, kActQuantInt4);                     \
    else if (qmode == kActQuantFp4)                       \
      SVDQ_ACT_S(TBV, kActQuantFp4);                      \
    else                                               \
      SVDQ_ACT_S(TBV, kActQuantNone);                     \
  } while (0)
  if (tb == 0)
    SVDQ_ACT(0);
  else if (tb == 1)
    SVDQ_ACT(1);
  else if (tb == 2)
    SVDQ_ACT(2);
  else if (tb == 3)
    SVDQ_ACT(3);
  else if (tb == 4)
    SVDQ_ACT(4);
  else if (tb == 8)
    SVDQ_ACT(8);
  else
    SVDQ_ACT(16);
#undef SVDQ_ACT
#undef SVDQ_ACT_S
#undef SVDQ_ACT_Q
  return (int)hipGetLastError();
}

// y[i] = y[i] + t[i] in fp32, stored back in the tensors' type (bf16: round to
// nearest even).  Eight elements per thread.
namespace {
template <bool BF16>
__global__ void add_kernel(void* __restrict__ y, const void* __restrict__ t, size_t count) {
  const size_t i0 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 >= count) return;
  if (BF16) {
    uint16_t* yy = reinterpret_cast<uint16_t*>(y);
    const uint16_t* tt = reinterpret_cast<const uint16_t*>(t);
    if (i0 + 8 <= count) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(yy + i0);
      const u32x4 c = *reinterpret_cast<const u32x4*>(tt + i0);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(bf16_lo(a[e]) + bf16_lo(c[e]), bf16_hi(a[e]) + bf16_hi(c[e]));
      *reinterpret_cast<u32x4*>(yy + i0) = o;
    } else {
      for (size_t i = i0; i < count; ++i)
        yy[i] = bf16_bits(__uint_as_float((uint32_t)yy[i] << 16) + __uint_as_float((uint32_t)tt[i] << 16));
    }
  } else {
    float* yy = reinterpret_cast<float*>(y);
    const float* tt = reinterpret_cast<const float*>(t);
    if (i0 + 8 <= count) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(yy + i0 + 4 * h);
        const f32x4 c = *reinterpret_cast<const f32x4*>(tt + i0 + 4 * h);
        *reinterpret_cast<f32x4*>(yy + i0 + 4 * h) = a + c;
      }
    } else {
      for (size_t i = i0; i < count; ++i) yy[i] += tt[i];
    }
  }
}
}  // namespace

int launch_add(void* y, const void* t, size_t count, int y_dtype, void* stream) {
  const unsigned blocks = (unsigned)((count + 8 * 256 - 1) / (8 * 256));
  if (y_dtype == SVDQ_OUT_BF16)
    hipLaunchKernelGGL(add_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, y, t, count);
  else
    hipLaunchKernelGGL(add_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, y, t, count);
  return (int)hipGetLastError();
}

int launch_act8_quant(const uint16_t* x, int b, int m, const float* smooth_inv, int8_t* qx, uint16_t* ascale,
                      void* stream) {
  if (b == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)((b + 3) / 4));
  const int per_lane = (m / 8 + 63) / 64;  // pieces of the row per lane
  if (per_lane <= 4)
    hipLaunchKernelGGL(act8_quant_kernel<4>, grid, dim3(256), 0, st, x, b, m, smooth_inv, qx, ascale);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(act8_quant_kernel<8>, grid, dim3(256), 0, st, x, b, m, smooth_inv, qx, ascale);
  else if (per_lane <= 24)
    hipLaunchKernelGGL(act8_quant_kernel<24>, grid, dim3(256), 0, st, x, b, m, smooth_inv, qx, ascale);
  else
    hipLaunchKernelGGL(act8_quant_kernel<0>, grid, dim3(256), 0, st, x, b, m, smooth_inv, qx, ascale);
  return (int)hipGetLastError();
}

int launch_z_reduce(const float* zpart, int splits, int b, int rank, float* z, void* stream) {
  const size_t count = (size_t)b * rank;
  // 16-byte accesses when every split's slice and z start 16-byte aligned
  // (the workspace is 256-byte aligned; each slice is count floats)
  const bool vec = count % 4 == 0 && ((uintptr_t)zpart & 15u) == 0 && ((uintptr_t)z & 15u) == 0;
  if (vec && splits <= kZChunks)
    hipLaunchKernelGGL(z_reduce_kernel, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, zpart, splits, count, z);
  else if (vec)
    hipLaunchKernelGGL(z_reduce_chunked_kernel, dim3((unsigned)((count / 4 + 15) / 16)), dim3(256), 0,
                       (hipStream_t)stream, zpart, splits, count, z);
  else
    hipLaunchKernelGGL(z_reduce1_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, zpart, splits, count, z);
  return (int)hipGetLastError();
}

}  // namespace svdq
