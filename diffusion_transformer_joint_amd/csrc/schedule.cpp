// Host policy for covering the query tiles of one launch with workgroups.
//
// The attention kernel runs one 256-row query tile of one (batch, head) per
// workgroup and one workgroup per compute unit.  With T tiles and C units the
// last round is partial unless C divides T (8,704 tokens x 24 heads: 816 tiles
// on 256 units is 3.19 rounds).  The remedy: run the first F' full rounds as
// whole tiles and cut each of the remaining L tiles into S key/value ranges, so
// the last round holds L*S <= C-ish short pieces; the pieces' fp32 partial
// softmax states are merged exactly afterwards.  (F', S) minimises the time
//   F' (r + o) + ceil(L*S / C) (r / S + o) + (merge traffic of L*S partials)
// against ceil(T / C) (r + o) without a split, where r is the loop time of a
// whole tile and o what every work item pays outside its loop.  Both were
// measured on MI355X with per-workgroup timestamps (bf16, head_dim 128): ~2 us
// per 64-key step of a 256-row tile, and ~8 us per item for Q staging, the
// first tile, the epilogue and the change of workgroup on the CU.  With o in
// the model, a call whose last round is large (4,608 tokens: 432 tiles, 1.69
// rounds) runs unsplit: cutting 176 tiles into 4 pieces saves less loop time
// than the 704 items and the merge of their partials cost.
#include <cmath>

#include "kernels.h"

namespace flux {

Schedule plan_schedule(int tiles, int kv_tiles, int num_cus, int max_pieces, int head_dim) {
  Schedule best{tiles, 0, 1, tiles};
  if (tiles <= 0 || num_cus <= 0) return best;
  const double C = num_cus;
  // Loop time of one whole tile, per-item cost, and HBM cost of one partial
  // (written and read back: 256 rows x head_dim fp32 + (m, l)).
  const double tile_s = 2.0e-6 * head_dim / 128.0;  // one 64-key step of a 256-row tile
  const double item_s = 8.0e-6;
  const double round_s = kv_tiles * tile_s;
  const double piece_bytes = 2.0 * 256.0 * (head_dim * 4.0 + 8.0);
  const double hbm = 6.0e12;
  double best_cost = std::ceil(tiles / C) * (round_s + item_s);
  const int F = tiles / num_cus;
  for (int Fp = F; Fp >= 0 && Fp >= F - 1; --Fp) {
    const int L = tiles - Fp * num_cus;
    if (L <= 0) continue;
    const int smax = kv_tiles < 16 ? kv_tiles : 16;
    for (int S = 2; S <= smax; ++S) {
      const long pieces = (long)L * S;
      if (pieces > max_pieces) break;
      const double cost =
          Fp * (round_s + item_s) + std::ceil(pieces / C) * (round_s / S + item_s) + pieces * piece_bytes / hbm;
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = Schedule{Fp * num_cus, L, S, Fp * num_cus + (int)pieces};
      }
    }
  }
  return best;
}

// Dense single-range launches: the split above, or a persistent split in
// which each of the C workgroups runs an equal slice of the T x kv_tiles tile
// positions (partials in at most 2 C slots).  Measured with T >= C (8,704
// tokens x 24 heads: 816 tiles) the persistent split loses (-8%) although its
// loop takes no more shader cycles per tile: the chip is power-limited under
// this loop, and with every CU busy to the end the clock drops (1.57 against
// 1.67 GHz), which outweighs the better balance.  With T < C (one GPU's 3-head
// share: 102 tiles) it wins (+10%) over cutting every tile into 5 pieces and
// running them in two rounds.  So: persistent when T < C and every slice gets
// at least two positions (mode 0), always where the workspace allows (mode 2),
// or never (mode 1).
Schedule plan_schedule_dense(int tiles, int kv_tiles, int num_cus, int max_pieces, int head_dim, int mode) {
  const Schedule base = plan_schedule(tiles, kv_tiles, num_cus, max_pieces, head_dim);
  if (mode == 1 || tiles <= 0 || kv_tiles <= 0 || num_cus < 2 || 2 * num_cus > max_pieces) return base;
  Schedule s{0, 0, 1, num_cus};
  s.sk_nkv = kv_tiles;
  s.sk_tiles = tiles;
  s.sk_cus = num_cus;
  if (mode == 2) return s;
  const long W = (long)tiles * kv_tiles;
  return (tiles < num_cus && W >= 2L * num_cus) ? s : base;
}

}  // namespace flux
