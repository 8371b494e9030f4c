// Activation-side kernels: calibration statistic, the fused activation
// quantization + low-rank down-projection (first fused pair of Nunchaku), and
// the ordered reduction of split partial sums.
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
// `chunk` groups (1..6, at most about 40 KB of LDS): the workgroup stages a chunk's 1/lambda and L1 slices in LDS
// (shared by the four waves), then each wave processes the chunk for its strip.
// Activations stream through registers two groups ahead, across chunk
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

template <int TB>  // 16-column blocks of Z (rank <= 16 * TB); 0 = no low-rank branch
__global__ __launch_bounds__(256) void act_quant_down_kernel(
    const uint16_t* __restrict__ x, int b, int m, int G, const float* __restrict__ inv,
    const uint16_t* __restrict__ l1t, int rank, uint8_t* __restrict__ qx,
    uint16_t* __restrict__ ascale, float* __restrict__ zout, int gps, int chunk) {
  constexpr int NB = TB > 0 ? TB : 1;
  constexpr int GB = act_lds_group_bytes(TB);
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int split = blockIdx.y;
  const int g_begin = split * gps;
  const int g_end = min(G, g_begin + gps);
  const int ng = g_end - g_begin;

  // stage 1/lambda and the L1 slices of groups [cb, ce) in LDS
  auto stage = [&](int cb, int ce) {
    const int n = ce - cb;
    const __amdgpu_buffer_rsrc_t ri =
        make_rsrc(inv ? inv + (size_t)cb * 64 : nullptr, inv ? (uint32_t)n * 256u : 0u);
    for (int k = tid; k < n * 16; k += 256) {  // 16 chunks of 16 B per group
      const int j = k >> 4, q = k & 15;
      *reinterpret_cast<u32x4*>(lds + j * GB + 16 * q) =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (uint32_t)(j * 256 + 16 * q), 0, 0));
    }
    if constexpr (TB > 0) {
      // L1 rows t < 16 TB (zero beyond rank), 8 chunks of 16 B per (group, t)
      const __amdgpu_buffer_rsrc_t rl =
          make_rsrc(l1t + (size_t)cb * 64, (uint32_t)((rank - 1) * m + n * 64) * 2u);
      for (int k = tid; k < n * TB * 16 * 8; k += 256) {
        const int q = k & 7, t = (k >> 3) % (TB * 16), j = (k >> 3) / (TB * 16);
        const uint32_t off = t < rank ? (uint32_t)(t * m + j * 64 + 8 * q) * 2u : 0xFFFFFFF0u;
        *reinterpret_cast<u32x4*>(lds + j * GB + 256 + (t * kL1Pitch + 8 * q) * 2) =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, off, 0, 0));
      }
    }
  };

  // this wave's strip (a wave past the end still takes part in the barriers)
  const int row0 = blockIdx.x * 64 + wave * 16;
  const bool strip_live = row0 < b;
  const int row = row0 + r;
  const bool valid = row < b;
  const int rows_here = strip_live ? min(16, b - row0) : 1;
  const uint32_t x_bytes = (uint32_t)((rows_here - 1) * m + 64) * 2u;  // per group, from its base
  const uint32_t x_off = (uint32_t)(r * m + 8 * c) * 2u;              // + 64 for channels 32+8c..
  auto load_x = [&](int g, u32x4& xa, u32x4& xb) {
    const bool live = g < g_end && strip_live;
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(x + (size_t)(live ? row0 : 0) * m + (size_t)(live ? g : 0) * 64, live ? x_bytes : 0u);
    xa = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off, 0, 0));
    xb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off + 64u, 0, 0));
  };

  f32x4 acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](int g, int j, const u32x4& xa, const u32x4& xb) {
    if (!strip_live) return;
    const uint8_t* gl = lds + j * GB;
    float v[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(xa[e]);
      v[2 * e + 1] = bf16_hi(xa[e]);
      v[8 + 2 * e] = bf16_lo(xb[e]);
      v[8 + 2 * e + 1] = bf16_hi(xb[e]);
    }
    if (inv) {
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
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(v[e]));
    am = max4_rows(am);
    float s32 = am / 7.0f;                 // IEEE division (correctly rounded)
    s32 = fminf(s32, 65504.0f);            // saturate instead of rounding to inf
    const _Float16 s16 = (_Float16)s32;    // round to nearest even
    const float sf = (float)s16;
    const float rc = sf > 0.0f ? 1.0f / sf : 0.0f;
    uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pq = v[e] * rc;
      const float rem = __builtin_fmaf(-pq, sf, v[e]);
      const float q1 = __builtin_fmaf(rem, rc, pq);
      const float q = __builtin_amdgcn_fmed3f(q1, -7.0f, 7.0f);
      const uint32_t nib = __float_as_uint(q + kMagic) & 0xFu;
      if (e < 8)
        w0 |= nib << (4 * e);
      else
        w1 |= nib << (4 * (e - 8));
    }
    if (valid) {
      uint8_t* rec = qx + ((size_t)g * b + row) * 32;
      *reinterpret_cast<uint32_t*>(rec + 4 * c) = w0;
      *reinterpret_cast<uint32_t*>(rec + 16 + 4 * c) = w1;
      if (c == 0) ascale[(size_t)g * b + row] = __builtin_bit_cast(uint16_t, s16);
    }
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

  // x two groups ahead: register stage 0 holds the even groups of the split
  // (counted from g_begin), stage 1 the odd ones
  u32x4 xa[2], xb[2];
  load_x(g_begin, xa[0], xb[0]);
  load_x(g_begin + 1, xa[1], xb[1]);
  for (int cb = g_begin; cb < g_end; cb += chunk) {
    const int ce = min(cb + chunk, g_end);
    __syncthreads();  // every wave is done with the previous chunk
    stage(cb, ce);
    __syncthreads();
    int g = cb;
    if ((g - g_begin) & 1) {  // an odd-sized chunk left the next group odd
      process(g, 0, xa[1], xb[1]);
      load_x(g + 2, xa[1], xb[1]);
      ++g;
    }
    for (; g + 1 < ce; g += 2) {
      process(g, g - cb, xa[0], xb[0]);
      load_x(g + 2, xa[0], xb[0]);
      process(g + 1, g + 1 - cb, xa[1], xb[1]);
      load_x(g + 3, xa[1], xb[1]);
    }
    if (g < ce) {
      process(g, g - cb, xa[0], xb[0]);
      load_x(g + 2, xa[0], xb[0]);
    }
  }
  if (!strip_live) return;

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

// z[i][t] = sum over splits s (in order) of zpart[s][i][t].  Loads are issued
// eight splits at a time; the additions keep the split order.
__global__ void z_reduce_kernel(const float* __restrict__ zpart, int splits, size_t count,
                                float* __restrict__ z) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= count) return;
  float s = zpart[idx];
  int k = 1;
  for (; k + 8 <= splits; k += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = zpart[(size_t)(k + u) * count + idx];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; k < splits; ++k) s += zpart[(size_t)k * count + idx];
  z[idx] = s;
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
                          const ActPlan& plan, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int G = m / 64;
  dim3 grid(plan.strips, plan.splits);
  const int tb = act_blocks(rank);
#define SVDQ_ACT(TBV)                                                                            \
  hipLaunchKernelGGL(act_quant_down_kernel<TBV>, grid, dim3(256),                                \
                     (size_t)plan.chunk * act_lds_group_bytes(TBV), st, x, b, m, G, smooth_inv,   \
                     l1, rank, qx, ascale, zpart, plan.groups_per_split, plan.chunk)
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
  return (int)hipGetLastError();
}

int launch_z_reduce(const float* zpart, int splits, int b, int rank, float* z, void* stream) {
  const size_t count = (size_t)b * rank;
  hipLaunchKernelGGL(z_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, zpart, splits, count, z);
  return (int)hipGetLastError();
}

}  // namespace svdq
