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
// Workgroup = 4 waves over a strip of 16 rows and a contiguous range of channel
// groups (one split); the waves take the groups round-robin.  In one wave, lane
// l owns row (l & 15) and, in each 64-channel group, channels 8c..8c+7 and
// 32+8c..32+8c+7 with c = l >> 4: exactly the bf16 MFMA A-operand layout, so
// the smoothed bf16 tile feeds both the quantizer and the down-projection.
//
// Per element:  x~ = bf16(fl32(x * inv))
// Per row/group: s = fp16(fl32(amax / 7)) (saturated), r = fl32(1 / s)
// Per element:  q = clamp(round_even(x~ / s), -7, 7), computed without a divide:
//   p = fl(x~ r); e = fma(-p, s, x~) (exact remainder); q1 = fma(e, r, p)
//   q1 equals the correctly rounded quotient fl32(x~ / s) for every bf16 x~ and
//   fp16 s (one Newton correction; proven on the host by exhaustive
//   enumeration in the tests), so round_even(q1) matches the definition.
// ---------------------------------------------------------------------------
template <int TB>  // 16-column blocks of Z (rank <= 16 * TB); 0 = no low-rank branch
__global__ __launch_bounds__(256) void act_quant_down_kernel(
    const uint16_t* __restrict__ x, int b, int m, int G, const float* __restrict__ inv,
    const uint16_t* __restrict__ l1t, int rank, uint8_t* __restrict__ qx,
    uint16_t* __restrict__ ascale, float* __restrict__ zpart, int gps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const int row = blockIdx.x * 16 + r;
  const bool valid = row < b;
  const int split = blockIdx.y;
  const int g_begin = split * gps;
  const int g_end = min(G, g_begin + gps);

  f32x4 acc[TB > 0 ? TB : 1];
#pragma unroll
  for (int t = 0; t < (TB > 0 ? TB : 1); ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xrow = x + (size_t)(valid ? row : 0) * m;
  for (int g = g_begin + wave; g < g_end; g += 4) {
    const int k0 = g * 64 + 8 * c;  // first 8 channels of this lane; second 8 at k0 + 32
    u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
    if (valid) {
      xa = ldg16(xrow + k0);
      xb = ldg16(xrow + k0 + 32);
    }
    float v[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(xa[e]);
      v[2 * e + 1] = bf16_hi(xa[e]);
      v[8 + 2 * e] = bf16_lo(xb[e]);
      v[8 + 2 * e + 1] = bf16_hi(xb[e]);
    }
    if (inv) {
      const f32x4 i0 = *reinterpret_cast<const f32x4*>(inv + k0);
      const f32x4 i1 = *reinterpret_cast<const f32x4*>(inv + k0 + 4);
      const f32x4 i2 = *reinterpret_cast<const f32x4*>(inv + k0 + 32);
      const f32x4 i3 = *reinterpret_cast<const f32x4*>(inv + k0 + 36);
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
    for (int p = 0; p < 8; ++p) {
      xt[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
      v[2 * p] = bf16_lo(xt[p]);
      v[2 * p + 1] = bf16_hi(xt[p]);
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
      const float p = v[e] * rc;
      const float rem = __builtin_fmaf(-p, sf, v[e]);
      const float q1 = __builtin_fmaf(rem, rc, p);
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
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int t = tb * 16 + r;
        u32x4 b0 = {0u, 0u, 0u, 0u}, b1 = {0u, 0u, 0u, 0u};
        if (t < rank) {
          b0 = ldg16(l1t + (size_t)t * m + k0);
          b1 = ldg16(l1t + (size_t)t * m + k0 + 32);
        }
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, b0), acc[tb], 0, 0, 0);
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, b1), acc[tb], 0, 0, 0);
      }
    }
  }

  if constexpr (TB > 0) {
    // ordered cross-wave sum (wave 0 + 1 + 2 + 3), one 16-column block at a time
    __shared__ f32x4 red[4][64];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      red[wave][lane] = acc[tb];
      __syncthreads();
      if (wave == 0) {
        f32x4 s = red[0][lane];
        s += red[1][lane];
        s += red[2][lane];
        s += red[3][lane];
        const int t = tb * 16 + r;
        if (t < rank) {
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const int zr = blockIdx.x * 16 + 4 * c + vv;  // MFMA D layout: row 4c+v, column l&15
            if (zr < b) zpart[((size_t)split * b + zr) * rank + t] = s[vv];
          }
        }
      }
      __syncthreads();
    }
  }
}

// z[i][t] = sum over splits s (in order) of zpart[s][i][t]
__global__ void z_reduce_kernel(const float* __restrict__ zpart, int splits, size_t count,
                                float* __restrict__ z) {
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= count) return;
  float s = zpart[idx];
  for (int k = 1; k < splits; ++k) s += zpart[(size_t)k * count + idx];
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
  const int tb = (rank + 15) / 16;
#define SVDQ_ACT(TBV)                                                                              \
  hipLaunchKernelGGL(act_quant_down_kernel<TBV>, grid, dim3(256), 0, st, x, b, m, G, smooth_inv, l1, \
                     rank, qx, ascale, zpart, plan.groups_per_split)
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
  else if (tb <= 8)
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
