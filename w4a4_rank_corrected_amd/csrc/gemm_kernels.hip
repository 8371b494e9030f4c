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
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace svdq {
namespace {

using namespace dev;

constexpr int TM = 128;       // output rows (tokens) per workgroup
constexpr int TN = 128;       // output columns per workgroup
constexpr int ROWB = 64 + 16; // LDS bytes per unpacked 64-channel row (+16 pad: conflict-free b128 reads)

__device__ __forceinline__ void unpack_store(uint8_t* dst, u32x4 w) {
  // 8 nibbles per word -> the low nibbles go to the first 16 bytes, the high
  // nibbles to the next 16, each as the signed byte 16*q.  Both operands use
  // the same placement, so the channel permutation cancels in the dot product.
  u32x4 lo, hi;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = (w[e] << 4) & 0xF0F0F0F0u;
    hi[e] = w[e] & 0xF0F0F0F0u;
  }
  *reinterpret_cast<u32x4*>(dst) = lo;
  *reinterpret_cast<u32x4*>(dst + 16) = hi;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_w4a4_up_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ ascale,
    const float* __restrict__ z, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, int b, int n, int G, int rank, int tiles_n,
    void* __restrict__ yout) {
  __shared__ __align__(16) uint8_t As[2][TM * ROWB];
  __shared__ __align__(16) uint8_t Bs[2][TN * ROWB];
  __shared__ __align__(16) float Sxq[2][TM];  // sx / 256
  __shared__ __align__(16) float Sng[2][TM];  // -1.5*2^23 * sx / 256
  __shared__ __align__(16) float Sw[2][TN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, c = lane >> 4;
  const int tile_j = blockIdx.x % tiles_n, tile_i = blockIdx.x / tiles_n;
  const int i0 = tile_i * TM, j0 = tile_j * TN;

  f32x4 acc[4][4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- low-rank branch: acc = bf16(Z) L2 over K = rank in chunks of 32 -------
  for (int kc = 0; kc < rank; kc += 32) {
    bf16x8 P[4], Q[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int j = j0 + 64 * wn + 16 * bj + r;
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = kc + 8 * c + 2 * e;
        uint32_t lo = 0u, hi = 0u;
        if (j < n && t < rank) lo = l2t[(size_t)j * rank + t];
        if (j < n && t + 1 < rank) hi = l2t[(size_t)j * rank + t + 1];
        wv[e] = lo | (hi << 16);
      }
      P[bj] = __builtin_bit_cast(bf16x8, u32x4{wv[0], wv[1], wv[2], wv[3]});
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const int i = i0 + 64 * wm + 16 * bi + r;
      float zv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = kc + 8 * c + e;
        zv[e] = (i < b && t < rank) ? z[(size_t)i * rank + t] : 0.0f;
      }
      Q[bi] = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16x2(zv[0], zv[1]), pack_bf16x2(zv[2], zv[3]),
                        pack_bf16x2(zv[4], zv[5]), pack_bf16x2(zv[6], zv[7])});
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P[bj], Q[bi], acc[bi][bj], 0, 0, 0);
  }

  // ---- main branch: exact per-group i8 MFMA + fp32 scale epilogue ----------
  const int srow = tid >> 1, shalf = tid & 1;  // staging: one 16-byte half record per thread
  const bool a_ok = i0 + srow < b;
  const bool b_ok = j0 + srow < n;
  const uint8_t* a_src = qx + ((size_t)(i0 + srow)) * 32 + 16 * shalf;
  const uint8_t* b_src = qw + ((size_t)(j0 + srow)) * 32 + 16 * shalf;
  const size_t a_gstride = (size_t)b * 32, b_gstride = (size_t)n * 32;

  auto load_stage = [&](int g, u32x4& av, u32x4& bv, float& sc) {
    av = a_ok ? ldg16(a_src + (size_t)g * a_gstride) : u32x4{0u, 0u, 0u, 0u};
    bv = b_ok ? ldg16(b_src + (size_t)g * b_gstride) : u32x4{0u, 0u, 0u, 0u};
    if (tid < TM) {
      const int i = i0 + tid;
      sc = i < b ? f16_to_f32(ascale[(size_t)g * b + i]) : 0.0f;
    } else {
      const int j = j0 + tid - TM;
      sc = j < n ? f16_to_f32(wscale[(size_t)g * n + j]) : 0.0f;
    }
  };
  auto store_stage = [&](int buf, const u32x4& av, const u32x4& bv, float sc) {
    unpack_store(&As[buf][srow * ROWB + 32 * shalf], av);
    unpack_store(&Bs[buf][srow * ROWB + 32 * shalf], bv);
    if (tid < TM) {
      const float q = sc * 0.00390625f;  // sx / 256 (exact)
      Sxq[buf][tid] = q;
      Sng[buf][tid] = -kMagic * q;       // exact: 3 * 2^14 * sx
    } else {
      Sw[buf][tid - TM] = sc;
    }
  };

  const i32x4 magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  if (G > 0) {
    u32x4 av, bv;
    float sc;
    load_stage(0, av, bv, sc);
    store_stage(0, av, bv, sc);
  }
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int cur = g & 1;
    u32x4 nav, nbv;
    float nsc = 0.0f;
    const bool more = g + 1 < G;
    if (more) load_stage(g + 1, nav, nbv, nsc);

    u32x4 Qa[4], Pb[4];
    float sxq[4], sng[4];
    f32x4 sw4[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const int rr = 64 * wm + 16 * bi + r;
      Qa[bi] = *reinterpret_cast<const u32x4*>(&As[cur][rr * ROWB + 16 * c]);
      sxq[bi] = Sxq[cur][rr];
      sng[bi] = Sng[cur][rr];
    }
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int cc = 64 * wn + 16 * bj;
      Pb[bj] = *reinterpret_cast<const u32x4*>(&Bs[cur][(cc + r) * ROWB + 16 * c]);
      sw4[bj] = *reinterpret_cast<const f32x4*>(&Sw[cur][cc + 4 * c]);
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            __builtin_bit_cast(i32x4, Pb[bj]), __builtin_bit_cast(i32x4, Qa[bi]), magic, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float t = __builtin_fmaf(__int_as_float(d[v]), sxq[bi], sng[bi]);
          acc[bi][bj][v] = __builtin_fmaf(t, sw4[bj][v], acc[bi][bj][v]);
        }
      }
    }
    if (more) store_stage(cur ^ 1, nav, nbv, nsc);
    __syncthreads();
  }

  // ---- epilogue: bias, cast, one store of Y ---------------------------------
  // lane holds Y[i][j..j+3]: i = row (l & 15) of block bi, j = 4 (l >> 4) of block bj
  // 4-element vector stores need n % 4 == 0 and a base aligned to 4 elements
  const bool vec_ok = (n & 3) == 0 && ((uintptr_t)yout & (OUT_BF16 ? 7u : 15u)) == 0;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const int i = i0 + 64 * wm + 16 * bi + r;
    if (i >= b) continue;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int j = j0 + 64 * wn + 16 * bj + 4 * c;
      f32x4 o = acc[bi][bj];
      if (bias) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (j + v < n) o[v] += __uint_as_float((uint32_t)bias[j + v] << 16);
      }
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

}  // namespace

int launch_gemm_up(const uint8_t* qx, const uint16_t* ascale, const float* z, const svdq_layer& L,
                   int b, void* y, int y_dtype, void* stream) {
  const int G = L.m / 64;
  const int tiles_n = (L.n + TN - 1) / TN;
  const int tiles_m = (b + TM - 1) / TM;
  dim3 grid((unsigned)(tiles_n * tiles_m));
  hipStream_t st = (hipStream_t)stream;
  if (y_dtype == SVDQ_OUT_BF16)
    hipLaunchKernelGGL(gemm_w4a4_up_kernel<true>, grid, dim3(256), 0, st, qx, ascale, z,
                       L.qw, L.wscale, L.l2, L.bias, b, L.n, G, L.rank, tiles_n, y);
  else
    hipLaunchKernelGGL(gemm_w4a4_up_kernel<false>, grid, dim3(256), 0, st, qx, ascale, z,
                       L.qw, L.wscale, L.l2, L.bias, b, L.n, G, L.rank, tiles_n, y);
  return (int)hipGetLastError();
}

}  // namespace svdq
