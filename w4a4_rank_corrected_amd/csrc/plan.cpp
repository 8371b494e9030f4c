// Launch plan of the GEMM kernels (host logic; the kernels are in
// gemm_kernels.hip, which checks its builds against the tiling and
// residencies declared in internal.h).
#include <algorithm>

#include "internal.h"

namespace svdq {

// Plan of the GEMM launch.  With T tiles of G groups and S = CUs * (resident
// workgroups per CU) slots, one tile per workgroup runs T / S full rounds and
// a last round of R = T mod S tiles, which leaves S - R slots idle for a whole
// tile's time.  Those R tiles are split instead, each into k pieces along the
// channel groups (one piece per workgroup, each of at least kMinPieceGroups
// groups), so the last round takes about 1/k of a tile's time:
//   * after full rounds, k = floor(S / R) capped at kMaxPieces, and only when
//     k >= kMinPieces: halves cost more in partial sums than they save
//     (measured on FLUX QKV and PixArt fc1);
//   * when every tile is in the last round (T < S, a few hundred rows), k =
//     floor(S / T) capped at kMaxPiecesAll, from k = 2: otherwise most CUs
//     idle (FLUX projections at 256 rows).
// NVFP4 tiles are never split: that build of its kernel does not fit the
// register budget of three workgroups per CU without spilling.
// Each piece stores its sums in a partial slot of the workspace and a
// reduction kernel adds them (plus, in the 8-bit setting, one slot per tile
// for the low-rank product).  Split workgroups come first in the
// grid, then the full rounds of whole tiles.  The workspace bound assumes the
// largest gfx950 part (256 CUs), so it does not depend on the device or the
// format.
GemmPlan gemm_plan(int b, int n, int m, int cus, int fmt) {
  const int ncu = cus > 0 ? cus : kMaxCUs;
  GemmPlan p;
  p.G = m / 64;
  p.tiles_m = (b + kGemmTileM - 1) / kGemmTileM;
  p.wg_per_cu = kGemmWgPerCu[fmt];
  const long long slots = (long long)p.wg_per_cu * ncu;
  // INT4 tiles narrow to 128 x 64 when the wide ones would not fill a round
  const long long T128 = (long long)p.tiles_m * ((n + kGemmTileN - 1) / kGemmTileN);  // wide tiles
  p.tile_n = fmt == kFmtInt4 && T128 < slots ? kGemmTileNNarrow : kGemmTileN;
  p.tiles_n = (n + p.tile_n - 1) / p.tile_n;
  const long long T = (long long)p.tiles_m * p.tiles_n;
  const long long full = T / slots, rest = T - full * slots;
  const long long cap = full == 0 ? kMaxPiecesAll : kMaxPieces, kmin = full == 0 ? 2 : kMinPieces;
  const long long k = rest > 0 ? std::min<long long>({slots / rest, cap, p.G / kMinPieceGroups}) : 0;
  p.split = fmt != kFmtFp4 && rest > 0 && k >= kmin;  // NVFP4: never (register budget)
  p.split_tiles = p.split ? (int)rest : 0;
  p.pieces = p.split ? (int)k : 1;
  p.split_grid = p.split_tiles * p.pieces;
  p.grid = (int)(p.split_grid + (T - p.split_tiles));
  // workspace: one slot per split workgroup (at most one round of slots on
  // the largest part) plus one low-rank slot per split tile (at most half a
  // round: k >= 2); none when m has too few groups to split on any device
  const int max_wg_per_cu = std::max({kGemmWgPerCu[kFmtInt4], kGemmWgPerCu[kFmtInt8], kGemmWgPerCu[kFmtFp4]});
  const long long round = (long long)max_wg_per_cu * kMaxCUs;
  const long long kcap = std::min<long long>(kMaxPiecesAll, p.G / kMinPieceGroups);
  // counted in wide tiles of 64 KB: a narrow plan's k * T narrow slots of 32 KB
  // stay within it, on any device (k * T <= one round, T <= 2 * T128)
  const long long max_slots = kcap >= 2 ? std::min(round, T128 * kcap) + std::min(T128, round / 2) : 0;
  p.partial_bytes = (size_t)max_slots * kGemmTileM * kGemmTileN * 4;
  p.ws_bytes = p.partial_bytes;
  return p;
}

}  // namespace svdq
