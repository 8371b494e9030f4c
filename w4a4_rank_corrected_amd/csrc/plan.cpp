// Launch plan of the GEMM kernels (host logic; the kernels are in
// gemm_kernels.hip, which checks its builds against the tiling and
// residencies declared in internal.h).
#include <algorithm>

#include "internal.h"

namespace svdq {

// Plan of the GEMM launch.  With T tiles of G groups and S = CUs * (resident
// workgroups per CU of the kernel) slots, one tile per workgroup runs
// ceil(T / S) rounds, the last one a fraction f of slots full, idle for
// I = (1 - f) * G group-iterations per slot.  Stream-K is chosen when
// I >= 16 (splitting a tile costs a few group-iterations) and T < S, f <= 1/4
// or I >= 40: then the tiles beyond the first floor(T / S) - 1 full rounds
// (between S and 2S of them, or all T when T < 2S) go to min(S, their
// iterations / 8) stream-K workgroups, dispatched first, and the full rounds
// follow one tile per workgroup.  Otherwise one tile per workgroup: a last
// round more than a quarter full finishes faster on its emptier CUs, which
// measured better than splitting short tiles (FLUX QKV, G = 48, at three
// workgroups per CU: I = 30) but not long ones (FLUX fc2, G = 192, at two per
// CU: I = 60).  Every setting first tries its three-per-CU kernel (one tile
// per workgroup only); if that residency calls for stream-K, the two-per-CU
// kernel is planned by the same rule.  NVFP4 uses stream-K only for T < S.  The
// workspace bound assumes the largest gfx950 part (256 CUs) and the largest
// stream-K residency, so it does not depend on the device or the format.
namespace {
void plan_rounds(GemmPlan& p, long long slots, bool split_last_round) {
  const long long T = (long long)p.tiles_m * p.tiles_n;
  const long long full = T / slots, rest = T - full * slots;  // rest / slots = f
  const long long idle = (slots - rest) * p.G;               // (1 - f) G, in units of 1/slots
  p.streamk = T * p.G >= 16 && idle >= 16 * slots &&
              (full == 0 || (split_last_round && rest > 0 && (4 * rest <= slots || idle >= 40 * slots)));
  p.sk_tiles = 0;
  p.sk_grid = 0;
  if (p.streamk) {
    const long long dp = full >= 2 ? (full - 1) * slots : 0;
    p.sk_tiles = (int)(T - dp);
    p.sk_grid = (int)std::max(1LL, std::min(slots, (long long)p.sk_tiles * p.G / 8));
    p.grid = (int)(p.sk_grid + dp);
    // the kernel splits the iterations in 32-bit arithmetic: U * P < 2^32
    if ((unsigned long long)p.sk_tiles * (unsigned long long)p.G * (unsigned long long)p.sk_grid >= (1ull << 32)) {
      p.streamk = 0;
      p.sk_tiles = p.sk_grid = 0;
    }
  }
  if (!p.streamk) p.grid = (int)T;
}
}  // namespace

GemmPlan gemm_plan(int b, int n, int m, int cus, int fmt) {
  constexpr int kMaxSkWgPerCu =
      std::max({kGemmWgPerCu[kFmtInt4][1], kGemmWgPerCu[kFmtInt8][1], kGemmWgPerCu[kFmtFp4][1]});
  const int ncu = cus > 0 ? cus : kMaxCUs;
  GemmPlan p;
  p.G = m / 64;
  p.tiles_m = (b + kGemmTileM - 1) / kGemmTileM;
  p.tiles_n = (n + kGemmTileN - 1) / kGemmTileN;
  p.wg_per_cu = kGemmWgPerCu[fmt][0];
  // NVFP4 splits only tiles that do not fill one round: its two-per-CU build,
  // whose operand dequantization then runs at two waves per SIMD, measured
  // slower than one tile per workgroup at three per CU (FLUX fc2 and single
  // out: 7-8 %)
  const bool split_last_round = fmt != kFmtFp4;
  plan_rounds(p, (long long)p.wg_per_cu * ncu, split_last_round);
  if (p.streamk) {
    p.wg_per_cu = kGemmWgPerCu[fmt][1];
    plan_rounds(p, (long long)p.wg_per_cu * ncu, split_last_round);
  }
  const long long T = (long long)p.tiles_m * p.tiles_n;
  const long long max_sk = std::max(1LL, std::min((long long)kMaxSkWgPerCu * kMaxCUs, T * p.G / 8));
  p.partial_bytes = (size_t)(2 * max_sk) * kGemmTileM * kGemmTileN * 4;  // two partial slots per workgroup
  p.ws_bytes = p.streamk || cus <= 0 ? p.partial_bytes + (size_t)std::max(1LL, T) * 8 : 0;
  return p;
}

}  // namespace svdq
