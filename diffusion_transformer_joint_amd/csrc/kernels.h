// Kernel argument blocks and launchers of the joint RoPE attention library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {

struct AttnArgs {
  const uint16_t* q;      // [B][N][H][D] bf16 bits
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;            // [B][N][H][D] bf16 bits
  const uint32_t* rope;   // [N][D/2] (cos, sin) as packed fp16, cos in the low half
  int batch_tokens;       // tokens between consecutive batch entries of q, k, v, o
  int heads;
  int batch;
  float c;                // softmax scale * log2(e)
  // Work split (see Schedule): blocks [0, whole) run whole query tiles; the
  // other blocks run one of `split` K/V ranges of the remaining tiles and write
  // fp32 partials that attn_merge combines.
  int whole;
  int split;
  int sk_nkv, sk_tiles, sk_cus;  // persistent split (see Schedule); sk_nkv = 0: off
  float* part_o;          // [slot][256][D] un-normalized O of each partial
  float2* part_ml;        // [slot][256] (running max in the exp2 domain, row sum)
  // Tile-sparse launches only: kept 64-key tiles of each 256-row query tile,
  // ascending, kv_list[tile * list_stride + i] for i < kv_count[tile].
  const int* kv_list;
  const int* kv_count;
  int list_stride;
  // Optional (tile-sparse): dispatch order of the tiles; whole tiles run in
  // this order and the last ones in it are split.
  const int* tile_order;
  // Optional: natural-log log-sum-exp of each row of scale * S, [B][H][N]
  // (single-range launches).
  float* lse;
  // Optional clock measurement: [0] += shader cycles, [1] += wall-clock ticks
  // of every workgroup (ClockProbe).
  unsigned long long* clk;
  // Token ranges of the launch (bf16 kernel): range r attends over tokens
  // [rng_tok0[r], rng_tok0[r] + rng_len[r]) of the sequence (q, k, v, o and
  // rope point at token 0) and owns the launch's tiles [rng_tile0[r],
  // rng_tile0[r + 1]).  Joint attention is one range; segment-local mode puts
  // up to kMaxRanges segments into one launch.
  static constexpr int kMaxRanges = 16;
  int nranges;
  int rng_tok0[kMaxRanges];
  int rng_len[kMaxRanges];
  int rng_tile0[kMaxRanges + 1];
};

// How one launch covers T query tiles of 256 rows with K/V ranges of n_kv
// 64-key tiles on C compute units (one workgroup per CU): `whole_tiles` tiles
// are run whole, the remaining `split_tiles` are cut into `split` K/V ranges
// each, so that the last round of workgroups fills the machine.
struct Schedule {
  int whole_tiles;
  int split_tiles;
  int split;
  int grid;
  // Persistent split instead (sk_nkv > 0): grid = sk_cus workgroups, each
  // runs an equal slice of the sk_tiles x sk_nkv tile positions.
  int sk_nkv = 0;
  int sk_tiles = 0;
  int sk_cus = 0;
};
Schedule plan_schedule(int tiles, int kv_tiles, int num_cus, int max_pieces, int head_dim);
// Dense single-range bf16 launches: plan_schedule's split or the persistent
// one (mode 0: by cost, 1: never persistent, 2: persistent where possible).
Schedule plan_schedule_dense(int tiles, int kv_tiles, int num_cus, int max_pieces, int head_dim, int mode);

struct Fp8Args {
  const uint8_t* q;       // [B][N][H][D] e4m3 codes
  const uint8_t* k;
  const uint8_t* v;
  const float* scales;    // [3][B][H]: q, k, v scales
  uint16_t* o;            // [B][N][H][D] bf16 bits
  const uint32_t* rope;   // [N][D/2] packed fp16 (cos, sin)
  int n_tokens;
  int batch_tokens;
  int heads;
  int batch;
  int q_tiles;
  float c;
  int whole;
  int split;
  float* part_o;
  float2* part_ml;
  unsigned long long* clk;  // optional clock measurement (as AttnArgs::clk)
};

// Per-pair rotary frequencies theta^(-2j/d_a), computed on the host in double
// and passed to the table kernel by value (no device copy).
struct RopeFreq {
  double f[64];  // head_dim / 2 <= 64 pairs
};

// (cos, sin) of pos[n][axis(p)] * freq[p] for every token n and pair p, as
// packed fp16 (cos in the low half).
hipError_t launch_rope_table(const int32_t* pos, const RopeFreq& freq, uint32_t* table, int n_tokens,
                             int head_dim, int d0, int d1, hipStream_t stream);
// The same angles as fp32 (cos, sin) pairs, for the pooled tile-mask rule.
hipError_t launch_rope_table_f32(const int32_t* pos, const RopeFreq& freq, float2* table, int n_tokens,
                                 int head_dim, int d0, int d1, hipStream_t stream);

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, const Schedule& sch, hipStream_t stream);

// Backward of the bf16 joint attention (attn_bwd.hip).
struct BwdArgs {
  const uint16_t* q;      // [B][N][H][D] bf16 bits (unrotated)
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;    // forward output
  const uint16_t* dout;   // upstream gradient
  const float* lse;       // [B][H][N] natural-log log-sum-exp of scale * S
  float* dr;              // [B][H][N] workspace: rowsum(dout * out)
  uint16_t* qr;           // [B][N][H][D] workspace: bf16 R(q)
  uint16_t* kr;           // [B][N][H][D] workspace: bf16 R(k)
  uint16_t* dq;           // [B][N][H][D] bf16
  uint16_t* dk;
  uint16_t* dv;
  const uint32_t* rope;   // [N][D/2] packed fp16 (cos, sin)
  int n_tokens;
  int heads;
  int batch;
  float c;                // scale * log2(e)
  float scale;
};
hipError_t launch_attn_bwd(const BwdArgs& a, int head_dim, hipStream_t stream);
// Exact merge of split partials: O = sum_i 2^(m_i - m) O_i / sum_i 2^(m_i - m) l_i.
hipError_t launch_attn_merge(const AttnArgs& a, int head_dim, const Schedule& sch, hipStream_t stream);
hipError_t launch_attn_fp8(const Fp8Args& a, int head_dim, const Schedule& sch, hipStream_t stream);

// Tile-sparse support (block_sparse.hip).  Means of the rotated rows of x over
// tiles of `tile` tokens: fp32 [B][H][ceil(N/tile)][D].
hipError_t launch_tile_means(const uint16_t* x, const float2* rope, float* out, int n_tokens, int batch_tokens,
                             int heads, int batch, int head_dim, int tile, hipStream_t stream);
// Mask rows (b, h, query tile) of pooled scores c * <qbar, kbar> against the
// threshold row max + log2_tau: uint8 [rows][KT].
hipError_t launch_block_select(const float* qbar, const float* kbar, uint8_t* mask, int rows, int QT, int KT,
                               int head_dim, float c, float log2_tau, hipStream_t stream);
// Score-bound tile mask: for each (b, h, query tile) row of mask [B][H][QT][KT],
// key tile t is kept when max over the tile's queries i of (i's largest score
// over t - L_i) >= log2_tau, L_i = i's largest score over the 4 key tiles
// aligned with the query tile (scores c <R q, R k> in the exp2 domain, bf16
// operands as in the attention kernel).
struct BoundArgs {
  const uint16_t* q;      // [B][batch_tokens][H][D] bf16 bits
  const uint16_t* k;
  const uint32_t* rope;   // [N][D/2] packed fp16 (cos, sin)
  uint8_t* mask;          // [B][H][QT][KT]
  int n_tokens;
  int batch_tokens;
  int heads;
  int batch;
  int kt;                 // ceil(N / 64)
  float c;                // scale * log2(e)
  float log2_tau;
  int whole;              // set by launch_tile_bound: query tiles run over all key tiles,
  int split;              // and pieces per remaining query tile (key-tile ranges)
};
// Dynamic LDS of the per-wave reductions (8 x KT floats): KT <= 2048.
constexpr size_t kBoundMaxLds = 64 * 1024;
hipError_t launch_tile_bound(const BoundArgs& a, int head_dim, int num_cus, hipStream_t stream);
// Kept key tiles of each mask row (ascending) into list[row * stride + i], count[row].
hipError_t launch_mask_to_list(const uint8_t* mask, int* list, int* count, int rows, int KT, int stride,
                               hipStream_t stream);
// Query tiles ordered by kept count, descending (ties by index): order[rows].
// hipErrorInvalidValue when rows > 32768 (the caller keeps the natural order).
hipError_t launch_tile_order(const int* count, int* order, int rows, int KT, hipStream_t stream);

}  // namespace flux
