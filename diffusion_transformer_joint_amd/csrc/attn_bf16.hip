// bf16 joint RoPE attention for gfx950 (MI355X).
//
// Computes O = softmax(scale * R(q) R(k)^T) V for one (batch, head, 256-row
// query tile) per workgroup, non-causal, over the whole joint sequence of
// text, noisy-image and reference tokens ("Welcome FLUX.3 Image Klein in
// Diffusers", Architecture: the joint blocks attend over the concatenated
// streams).  Rotary embedding is applied while Q and K tiles are loaded
// ("Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell GPUs", How it
// works: rotary embeddings fused into the surrounding kernels).
//
// Work decomposition
//   workgroup = 8 waves x 32 query rows = 256 rows (two waves per SIMD); K/V
//   streamed in 64-key tiles, double-buffered in LDS (K rotated on the way
//   in, rows padded).
//   S^T = K Q^T is computed so that each lane owns one query (lane % 32) and
//   16 keys per 32-key block: the softmax row reductions are in-lane plus one
//   exchange between the two wave halves.
//   O^T += V^T P^T reuses the S^T accumulator registers directly as the P^T
//   operand (rounded to bf16); V^T fragments come from row-major V in LDS
//   through the gfx950 transpose read.
//   Software pipeline over tiles: iteration t issues one fixed-order stream of
//   MFMAs, S(t) = QK(t) then O += PV(t-1), and places the independent VALU
//   work between them (RoPE and LDS stores of the next tiles beside QK, P(t)
//   beside PV), so that each wave keeps its own matrix unit busy while it
//   computes the softmax.
//   Online softmax (Milakov & Gimelshein 2018) against a reference max that
//   rarely moves: the first tile of a K/V range sets it to the row max; later
//   tiles form p = exp2(c s - m) directly and only move m (rescaling O and l)
//   when a row's tile sum reaches 2^32.  The result is the same softmax.
//
// Layouts: q, k, v, o [B][N][H][D] bf16; rope [N][D/2] packed fp16 (cos, sin).
#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace flux {

template <int D>
struct Bf16Cfg {
  static constexpr int BM = 256;           // query rows per workgroup
  static constexpr int BN = 64;            // keys per K/V tile
  static constexpr int NT = 512;           // threads per workgroup (8 waves x 32 rows)
  static constexpr int KSTEPS = D / 16;    // 16-wide d steps of Q K^T
  static constexpr int DB = D / 32;        // 32-wide d blocks of O
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int RPP = NT / CPR;     // rows staged per pass
  static constexpr int NPASS = BN / RPP;   // staging passes per tile
  static constexpr int KTILEB = BN * (2 * D + 16);  // bytes per K tile in LDS
  static constexpr int VTILEB = BN * (2 * D + 64);  // bytes per V tile in LDS
};

// One work item: query tile tile_g (in the launch's tile order) over its K/V
// positions [kvx0, kvx1), or, with kvx0 < 0, over piece `piece` of `a.split`
// (slot >= 0) or all of them (slot < 0).  slot >= 0: the fp32 partial state
// goes to workspace slot `slot`; otherwise O is written.
template <int D, bool SPARSE>
__device__ __forceinline__ void fwd_tile(const AttnArgs& a, char (&ksm)[2][Bf16Cfg<D>::KTILEB],
                                         char (&vsm)[2][Bf16Cfg<D>::VTILEB], int tile_g, int slot, int piece,
                                         int kvx0, int kvx1) {
  using C = Bf16Cfg<D>;
  const int H = a.heads;
  // The token range this tile belongs to: N tokens from token tok0.
  int rg = 0;
  while (rg + 1 < a.nranges && tile_g >= a.rng_tile0[rg + 1]) ++rg;
  const int N = a.rng_len[rg], tok0 = a.rng_tok0[rg];
  const int tile = tile_g - a.rng_tile0[rg];
  const int q_tiles = (N + C::BM - 1) / C::BM;
  const int n_tiles = (N + C::BN - 1) / C::BN;
  const uint32_t* const rope = a.rope + (size_t)tok0 * (D / 2);
  // The 64-key tiles this query tile attends to, by position p: all of them
  // (p itself), or in a tile-sparse launch the kept list.  A split piece runs
  // positions [kv0, kv1).  Positions past the range map to a tile past N,
  // whose loads read zeros.
  const int* kvlist = SPARSE ? a.kv_list + (size_t)tile_g * a.list_stride : nullptr;
  const int cnt = SPARSE ? a.kv_count[tile_g] : n_tiles;
  int kv0 = 0, kv1 = cnt;
  if (kvx0 >= 0) {
    kv0 = kvx0;
    kv1 = kvx1;
  } else if (slot >= 0) {
    kv0 = piece * cnt / a.split;
    kv1 = (piece + 1) * cnt / a.split;
  }
  auto kvt = [&](int p) -> int {
    if constexpr (SPARSE) return p < kv1 ? kvlist[p] : n_tiles;
    else return p;
  };
  // In the main loop a sparse range reads its list entries through vector
  // loads two iterations ahead (a scalar load would make the loop's LDS waits
  // drain completely): kv_roll = tiles at positions t, t+1, t+2.
  int kv_roll[3] = {0, 0, 0};
  uint32_t kv_ahead = 0;  // list entry of position t+3, loaded during iteration t
  const __amdgpu_buffer_rsrc_t rlist = make_rsrc(kvlist, SPARSE ? (uint32_t)kv1 * 4u : 0u);
  const int qt = tile % q_tiles;
  const int bh = tile / q_tiles;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t tok_stride = (size_t)H * D;  // elements between consecutive tokens
  const size_t bat = ((size_t)b * a.batch_tokens + tok0) * tok_stride;  // this batch entry's range
  const uint16_t* qbase = a.q + bat + (size_t)h * D;
  const uint16_t* kbase = a.k + bat + (size_t)h * D;
  const uint16_t* vbase = a.v + bat + (size_t)h * D;
  const float c = a.c;

  // Running max folded into the score MFMA: an extra k-step multiplies a
  // column of ones in K by -m in Q, so the accumulator holds c*s - m and
  // p = exp2(acc).  m is kept bf16-representable, so this is exact.  Lanes of
  // the first half-wave carry k index 0 of the step, the others zeros.  That
  // product does not depend on the K tile: `fold` (-m in every row of each
  // query's column) is formed once per change of m and fed as the
  // accumulator input of the first score MFMA of each block.
  const bf16x8 zero8 = {};
  bf16x8 kone = zero8, qm = zero8;
  if (g == 0) kone[0] = (__bf16)1.0f;
  f32x16 fold = {};

  // ---- staging of K/V tiles: global -> registers -> (K rotated) -> LDS.
  // Each thread owns NPASS (row, 16-byte chunk) slots of a tile, split into two
  // halves with separate lifetimes so that the loads of tile j+2 can be issued
  // as soon as the matching half of tile j+1 has been written to LDS.
  const int st_chunk = tid % C::CPR;
  const int st_row0 = tid / C::CPR;
  u32x4 kraw[C::NPASS], vraw[C::NPASS];
  u32x4 kcs[C::NPASS];  // table entries of the 4 pairs of each slot
  // Buffer loads relative to the tile's first row: rows at or past N read as
  // zero (their keys are masked to -inf before the softmax), and tiles past
  // the last one are staged as zeros into a buffer that is never read.  The
  // per-thread offsets are loop invariant; the tile offset goes into the
  // (scalar) resource base.
  uint32_t kv_off[C::NPASS], rp_off[C::NPASS];
#pragma unroll
  for (int p = 0; p < C::NPASS; ++p) {
    const int r = st_row0 + p * C::RPP;
    kv_off[p] = (uint32_t)(r * tok_stride * 2 + st_chunk * 16);
    rp_off[p] = (uint32_t)(r * (D / 2) * 4 + st_chunk * 16);
  }
  // Range of a resource starting at row kt0: whole token rows up to the end
  // of the range.  Row r of a tile sits at byte r * tok_stride * 2 (+ its
  // chunk offset, below 2D), so the rows from N on fall outside the range
  // and rows before it inside.  Branch-free (max, multiply): a branch here
  // would split the loop body into several blocks, and the per-slot order
  // fixed by the scheduling barriers only holds within a block.
  auto tile_bytes = [&](int kt0) -> uint32_t {
    return (uint32_t)max(N - kt0, 0) * (uint32_t)(tok_stride * 2);
  };
  auto load_k = [&](int kt0) {
    const uint32_t rp_bytes = (uint32_t)max(N - kt0, 0) * (uint32_t)(D / 2 * 4);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)kt0 * tok_stride, tile_bytes(kt0));
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rope + (size_t)kt0 * (D / 2), rp_bytes);
#pragma unroll
    for (int p = 0; p < C::NPASS; ++p) {
      kraw[p] = buffer_load_b128(rk, kv_off[p]);
      kcs[p] = buffer_load_b128(rr, rp_off[p]);
    }
  };
  auto load_v = [&](int kt0) {
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)kt0 * tok_stride, tile_bytes(kt0));
#pragma unroll
    for (int p = 0; p < C::NPASS; ++p) vraw[p] = buffer_load_b128(rv, kv_off[p]);
  };
  auto store_k = [&](int buf) {
    FLUX_LDS char* kl = (FLUX_LDS char*)ksm[buf];
#pragma unroll
    for (int p = 0; p < C::NPASS; ++p)
      lds_write_b128(kl + k_off<D>(st_row0 + p * C::RPP, st_chunk), rope_chunk(kraw[p], kcs[p]));
  };
  auto store_v = [&](int buf) {
    FLUX_LDS char* vl = (FLUX_LDS char*)vsm[buf];
#pragma unroll
    for (int p = 0; p < C::NPASS; ++p) lds_write_b128(vl + v_off<D>(st_row0 + p * C::RPP, st_chunk), vraw[p]);
  };

  // ---- Q fragments (B operand of S^T = K Q^T), rotated, held in registers.
  // The Q tile is staged like a K tile: coalesced loads of whole rows (16
  // threads per row) and their angles, rotation, LDS (rows 0-127 in the K
  // buffers, 128-255 in the V buffers, K row layout), then each lane reads its
  // fragments.  Loading the fragments directly would touch 32 rows per
  // instruction and keep the workgroup's memory pipeline busy ~4x longer.
  // The first K/V tile's loads are issued behind the Q loads.  Rows at or past
  // N read as zero (buffer range check) and rotate to zero.
  const int qrow = qt * C::BM + wave * 32 + l32;
  bf16x8 qf[C::KSTEPS];
  {
    constexpr int QCH = C::BM * C::CPR / C::NT;  // chunks per thread
    static_assert(QCH * C::NT == C::BM * C::CPR && (QCH / 2) * C::RPP == C::BM / 2, "Q staging split");
    static_assert((C::BM / 2) * (2 * D + 16) <= 2 * C::KTILEB && (C::BM / 2) * (2 * D + 16) <= 2 * C::VTILEB,
                  "Q staging fits the K and V buffers");
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase + (size_t)qt * C::BM * tok_stride, tile_bytes(qt * C::BM));
    const __amdgpu_buffer_rsrc_t rqa =
        make_rsrc(rope + (size_t)qt * C::BM * (D / 2), (uint32_t)((N - qt * C::BM) * (D / 2) * 4));
    u32x4 qraw[QCH];
    u32x4 qcs[QCH];
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int r = st_row0 + i * C::RPP;
      qraw[i] = buffer_load_b128(rq, (uint32_t)(r * tok_stride * 2 + st_chunk * 16));
      qcs[i] = buffer_load_b128(rqa, (uint32_t)(r * (D / 2) * 4 + st_chunk * 16));
    }
    if (kv0 < kv1) {
      load_k(kvt(kv0) * C::BN);
      load_v(kvt(kv0) * C::BN);
    }
    auto qrow_lds = [&](int r) -> FLUX_LDS char* {
      return r < C::BM / 2 ? (FLUX_LDS char*)&ksm[0][0] + k_off<D>(r, 0)
                           : (FLUX_LDS char*)&vsm[0][0] + k_off<D>(r - C::BM / 2, 0);
    };
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int r = st_row0 + i * C::RPP;
      lds_write_b128(qrow_lds(r) + 16 * st_chunk, rope_chunk_scaled(qraw[i], qcs[i], c));
    }
    __syncthreads();
    const FLUX_LDS char* ql = qrow_lds(wave * 32 + l32);
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) qf[t] = __builtin_bit_cast(bf16x8, lds_read_b128(ql + 16 * (2 * t + g)));
    __syncthreads();  // the K/V buffers are reused below
  }

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = (f32x16){};
  float m_ref = 0.f;   // reference max of c*score, exp2 domain, bf16-representable
  float lsum = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int grp = lane >> 4, li = lane & 15;

  // S^T block kb (32 keys x the wave's 32 queries) of a K tile in LDS.  All
  // K fragments of the block are read before the MFMA chain starts.
  auto qk = [&](const FLUX_LDS char* kl, int kb) -> f32x16 {
    const int krow = 32 * kb + krow_perm(l32);
    bf16x8 kf[C::KSTEPS];
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t)
      kf[t] = __builtin_bit_cast(bf16x8, lds_read_b128(kl + k_off<D>(krow, 2 * t + g)));
    f32x16 s = mfma_bf16(kone, qm, (f32x16){});
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) s = mfma_bf16(kf[t], qf[t], s);
    return s;
  };
  // Keys past N (last tile only) get score -inf.
  auto mask = [&](int kt0, int kb, f32x16& s) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kt0 + 32 * kb + 16 * (e >> 3) + 8 * g + (e & 7);
      if (key >= N) s[e] = -INFINITY;
    }
  };
  // Running reference m (exp2 domain, bf16-representable; s holds
  // c*score - m through the folded MFMA column).  The first block of a K/V range
  // sets m to its row max.  Later blocks do not look at the max: p = exp2(s) is
  // formed directly and the block's row sum checked afterwards.  Only when a
  // row's block sum reaches 2^32 (or is not finite) does the rare path move m up
  // to the block max, rescale O, l and the pending score blocks, and recompute
  // P.  Between moves p <= 2^32, so O and l stay far inside the fp32 range; the
  // result is the same softmax.
  auto rebase = [&](float m_new, f32x16& s) {
    const float shift = m_ref - m_new;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] += shift;
  };
  auto set_ref = [&](float m_new) {
    m_ref = m_new;
    if (g == 0) qm[0] = (__bf16)(-m_new);
    fold = mfma_bf16(kone, qm, (f32x16){});
  };
  auto block_max = [&](const f32x16& s) -> float {
    float mt = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s[e]);
    return fmaxf(mt, swap_halves(mt));
  };
  auto rescale_o = [&](float alpha) {
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
  };
  // P^T fragment of one 16-key slice (hh) of block s; the row sum of the
  // bf16-rounded values goes to bsum.  The dot operand is built as a bf16x2
  // directly: a bit-cast vector element here made the compiler feed one
  // register to every dot instruction.
  auto make_p = [&](const f32x16& s, int hh, float& bsum) -> u32x4 {
    u32x4 pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(s[8 * hh + 2 * i]);
      const float p1 = __builtin_amdgcn_exp2f(s[8 * hh + 2 * i + 1]);
      bf16x2 pp;
      pp[0] = (__bf16)p0;
      pp[1] = (__bf16)p1;
      pf[i] = __builtin_bit_cast(uint32_t, pp);
      bsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, bsum, false);
    }
    return pf;
  };
  auto block_ok = [&](float bsum) -> bool { return __ballot(!(bsum < 0x1p32f)) == 0; };
  // O^T += V^T P^T for the 16-key slice (kb, hh).
  auto pv = [&](const FLUX_LDS char* vl, int kb, int hh, const u32x4& pf) {
    const int krow0 = 32 * kb + 16 * hh + 8 * (grp >> 1) + (li >> 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int d = 32 * db + 16 * (grp & 1) + 4 * (li & 3);
      const int cb = (d & 7) * 2;
      const u32x2 lo = lds_read_tr16(vl + v_off<D>(krow0, d >> 3) + cb);
      const u32x2 hi = lds_read_tr16(vl + v_off<D>(krow0 + 4, d >> 3) + cb);
      const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
      o[db] = mfma_bf16(__builtin_bit_cast(bf16x8, vv), __builtin_bit_cast(bf16x8, pf), o[db]);
    }
  };

  // Software pipeline over 64-key tiles.  Iteration t:
  //   MFMA:  S(t) = QK(t) (both 32-key blocks), then O += PV(t-1) with P(t-1)
  //          from the previous iteration;
  //   VALU:  P(t) = exp2(S(t)) with its row sums, beside the wave's own PV
  //          MFMAs; RoPE + LDS store of K(t+1) and store of V(t) beside QK;
  //          global loads of K(t+2) and V(t+1).
  //   barrier.
  // K(t) is read in iteration t and V(t) in iteration t+1, so K(t+1) and V(t)
  // are written into the buffers that K(t-1) and V(t-2) held: two buffers each.
  if (kv0 < kv1) {  // (a tile-sparse range may be empty: O = 0)
  store_k(0);  // K and V of the first tile were loaded with Q
  load_k(kvt(kv0 + 1) * C::BN);
  __syncthreads();

  u32x4 pp[4];  // P(t-1): fragments (block 0, keys 0-15), (0, 16-31), (1, 0-15), (1, 16-31)
  // The first tile of the range (no PV yet): its row max sets m.
  auto step_first = [&](auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm[0];
    const int kt0 = kvt(kv0) * C::BN;

    f32x16 s0 = qk(kl, 0);
    f32x16 s1 = qk(kl, 1);
    if (LAST) {
      mask(kt0, 0, s0);
      mask(kt0, 1, s1);
    }
    {
      const float m_new = bf16_round(m_ref + fmaxf(block_max(s0), block_max(s1)));
      rebase(m_new, s0);
      rebase(m_new, s1);
      set_ref(m_new);
    }
    float b = 0.f;
    pp[0] = make_p(s0, 0, b);
    pp[1] = make_p(s0, 1, b);
    pp[2] = make_p(s1, 0, b);
    pp[3] = make_p(s1, 1, b);
    if (!block_ok(b)) {  // rare: move m up to this tile's max
      const float m_new = fmaxf(m_ref, bf16_round(m_ref + fmaxf(block_max(s0), block_max(s1))));
      rescale_o(__builtin_amdgcn_exp2f(m_ref - m_new));
      rebase(m_new, s0);
      rebase(m_new, s1);
      set_ref(m_new);
      b = 0.f;
      pp[0] = make_p(s0, 0, b);
      pp[1] = make_p(s0, 1, b);
      pp[2] = make_p(s1, 0, b);
      pp[3] = make_p(s1, 1, b);
    }
    lsum += b;
    store_k(1);
    store_v(0);
    load_k(kvt(kv0 + 2) * C::BN);
    load_v(kvt(kv0 + 1) * C::BN);
    __syncthreads();
  };

  // Every tile after the first of the range: one MFMA stream (S(t) = QK(t),
  // then O += PV(t-1)) in a fixed order, each MFMA followed by the LDS operand
  // read NPF MFMAs ahead and a slice of independent VALU work: RoPE + store of
  // K(t+1) and store of V(t) beside QK, P(t) beside PV once the P(t-1)
  // fragment it replaces has been consumed.
  auto p_pair = [&](float x0, float x1, float& bsum) -> uint32_t {
    bf16x2 q2;
    q2[0] = (__bf16)__builtin_amdgcn_exp2f(x0);
    q2[1] = (__bf16)__builtin_amdgcn_exp2f(x1);
    bsum = __builtin_amdgcn_fdot2_f32_bf16(q2, ones, bsum, false);
    return __builtin_bit_cast(uint32_t, q2);
  };
  auto step_main = [&](int t, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int i = t - kv0;
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm[i & 1];
    const FLUX_LDS char* vl = (const FLUX_LDS char*)vsm[(i + 1) & 1];  // V(t-1)
    FLUX_LDS char* kw = (FLUX_LDS char*)ksm[(i + 1) & 1];              // K(t+1)
    FLUX_LDS char* vw = (FLUX_LDS char*)vsm[i & 1];                    // V(t)
    const int kt0 = (SPARSE ? kv_roll[0] : t) * C::BN;
    // MFMA j < NK: S(t), K fragment j; NK <= j < NL: PV(t-1), V fragment j - NK.
    constexpr int NK = 2 * C::KSTEPS, NL = NK + 4 * C::DB;
    auto ld = [&](int j) -> u32x4 {
      if (j < NK) {
        const int kb = j / C::KSTEPS, tt = j % C::KSTEPS;
        return lds_read_b128(kl + k_off<D>(32 * kb + krow_perm(l32), 2 * tt + g));
      }
      const int v = j - NK, kb = v / (2 * C::DB), hh = (v / C::DB) & 1, db = v % C::DB;
      const int krow0 = 32 * kb + 16 * hh + 8 * (grp >> 1) + (li >> 2);
      const int d = 32 * db + 16 * (grp & 1) + 4 * (li & 3);
      const u32x2 lo = lds_read_tr16(vl + v_off<D>(krow0, d >> 3) + (d & 7) * 2);
      const u32x2 hi = lds_read_tr16(vl + v_off<D>(krow0 + 4, d >> 3) + (d & 7) * 2);
      return (u32x4){lo[0], lo[1], hi[0], hi[1]};
    };
    // Slot plan (slot j follows MFMA j): RoPE of the 4 * NPASS pairs of K(t+1)
    // in every other slot from 0, store of V(t) in slots 1 and 3, loads of
    // V(t+1) in slot 5 and of K(t+2) once its registers are free; P(t) slice q
    // in the four slots after P(t-1) slice q has been consumed.  With D = 128
    // the last slice is formed early, in slots NK + 2 and NK + 3 (right after
    // the mask of s1), into spare registers that replace P(t-1) slice 3 after
    // the stream: the tail after the last MFMA is then short.
    constexpr int NPF = 3;                           // operand reads ahead
    constexpr int ROPE_END = 2 * 4 * C::NPASS;       // slots 0, 2, .., ROPE_END - 2
    constexpr int VST0 = 1, VST1 = 3, LVS = 5, LKS = ROPE_END > NK ? ROPE_END : NK;
    u32x4 fb[NPF];
#pragma unroll
    for (int j = 0; j < NPF; ++j) fb[j] = ld(j);
    f32x16 s0, s1;
    u32x4 kr[C::NPASS];
    u32x4 pn;  // P(t) slice 3 (D = 128)
    float b = 0.f;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NL>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const u32x4 x = fb[j % NPF];
      if constexpr (j + NPF < NL) fb[j % NPF] = ld(j + NPF);
      if constexpr (j < C::KSTEPS) {
        s0 = mfma_bf16(__builtin_bit_cast(bf16x8, x), qf[j], j == 0 ? fold : s0);
      } else if constexpr (j < NK) {
        s1 = mfma_bf16(__builtin_bit_cast(bf16x8, x), qf[j - C::KSTEPS], j == C::KSTEPS ? fold : s1);
      } else {
        constexpr int v = j - NK, q4 = v / C::DB, db = v % C::DB;
        o[db] = mfma_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, pp[q4]), o[db]);
      }
      if constexpr (j < ROPE_END && j % 2 == 0) {  // RoPE of K(t+1), one pair
        constexpr int p = (j / 2) >> 2, e = (j / 2) & 3;
        kr[p][e] = rope_pair(kraw[p][e], kcs[p][e]);
        if constexpr (e == 3) lds_write_b128(kw + k_off<D>(st_row0 + p * C::RPP, st_chunk), kr[p]);
      }
      if constexpr (j == VST0 || j == VST1) {     // V(t)
        constexpr int p = j == VST0 ? 0 : 1;
        lds_write_b128(vw + v_off<D>(st_row0 + p * C::RPP, st_chunk), vraw[p]);
      }
      if constexpr (SPARSE && j == 0) kv_ahead = buffer_load_b32(rlist, (uint32_t)(t + 3) * 4u);
      if constexpr (j == LVS) load_v((SPARSE ? kv_roll[1] : t + 1) * C::BN);
      if constexpr (j == LKS) load_k((SPARSE ? kv_roll[2] : t + 2) * C::BN);
      if constexpr (j >= NK) {
        constexpr int v = j - NK;
        if (LAST && v == 0) mask(kt0, 0, s0);
        if (LAST && v == 2) mask(kt0, 1, s1);
        if constexpr (D == 128 && (v == 2 || v == 3)) {  // P(t) slice 3, early
#pragma unroll
          for (int ee = 0; ee < 2; ++ee) {
            const int e2 = (v - 2) * 2 + ee;
            pn[e2] = p_pair(s1[8 + 2 * e2], s1[8 + 2 * e2 + 1], b);
          }
        }
        if constexpr (v >= C::DB) {                 // P(t) slice q replaces P(t-1) slice q
          constexpr int q = (v - C::DB) / C::DB, e = (v - C::DB) % C::DB;
          const f32x16& sq = q < 2 ? s0 : s1;
          constexpr int hh = q & 1;
#pragma unroll
          for (int ee = 0; ee < 4 / C::DB; ++ee) {
            const int e2 = e * (4 / C::DB) + ee;
            pp[q][e2] = p_pair(sq[8 * hh + 2 * e2], sq[8 * hh + 2 * e2 + 1], b);
          }
        }
      }
      // Within the slot: its MFMA first, then its VALU work, so that the
      // VALU issues while the MFMA runs.
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      if constexpr (D == 128) pp[3][e2] = pn[e2];
      else pp[3][e2] = p_pair(s1[8 + 2 * e2], s1[8 + 2 * e2 + 1], b);
    }
    if (!block_ok(b)) {  // rare: move m up to this tile's max
      const float m_new = fmaxf(m_ref, bf16_round(m_ref + fmaxf(block_max(s0), block_max(s1))));
      rescale_o(__builtin_amdgcn_exp2f(m_ref - m_new));
      rebase(m_new, s0);
      rebase(m_new, s1);
      set_ref(m_new);
      b = 0.f;
      pp[0] = make_p(s0, 0, b);
      pp[1] = make_p(s0, 1, b);
      pp[2] = make_p(s1, 0, b);
      pp[3] = make_p(s1, 1, b);
    }
    lsum += b;
    if constexpr (SPARSE) {
      kv_roll[0] = kv_roll[1];
      kv_roll[1] = kv_roll[2];
      kv_roll[2] = t + 3 < kv1 ? __builtin_amdgcn_readfirstlane((int)kv_ahead) : n_tiles;
    }
    __syncthreads();
  };

  // positions before full_end hold full tiles; the last one may be ragged
  const int full_end = (N % C::BN != 0 && kvt(kv1 - 1) == n_tiles - 1) ? kv1 - 1 : kv1;
  if constexpr (SPARSE) {
    kv_roll[0] = kvt(kv0 + 1);
    kv_roll[1] = kvt(kv0 + 2);
    kv_roll[2] = kvt(kv0 + 3);
  }
  if (kv0 < full_end) {
    step_first(std::false_type{});
    for (int t = kv0 + 1; t < full_end; ++t) step_main(t, std::false_type{});
    if (full_end < kv1) step_main(full_end, std::true_type{});
  } else {
    step_first(std::true_type{});
  }
  {
    const FLUX_LDS char* vl = (const FLUX_LDS char*)vsm[(kv1 - 1 - kv0) & 1];
    pv(vl, 0, 0, pp[0]);
    pv(vl, 0, 1, pp[1]);
    pv(vl, 1, 0, pp[2]);
    pv(vl, 1, 1, pp[3]);
  }
  }  // kv0 < kv1

  // ---- epilogue.  A K/V range of a split tile stores its fp32 partial state.
  const float ltot = lsum + swap_halves(lsum);
  if (slot >= 0) {
    const int r = wave * 32 + l32;
    float* po = a.part_o + ((size_t)slot * C::BM + r) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const f32x4 w = {o[db][4 * aa], o[db][4 * aa + 1], o[db][4 * aa + 2], o[db][4 * aa + 3]};
        *(f32x4*)(po + 32 * db + 8 * aa + 4 * g) = w;
      }
    if (g == 0) a.part_ml[(size_t)slot * C::BM + r] = make_float2(kv0 < kv1 ? m_ref : -INFINITY, ltot);
    return;
  }
  // ---- epilogue: O = O^T / l, bf16, stored row-major.
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;  // 0: an empty tile-sparse range
  if (a.lse != nullptr && g == 0 && qrow < N)
    a.lse[((size_t)b * H + h) * N + qrow] = (m_ref + __builtin_log2f(ltot)) * 0.6931471805599453f;
  if (qrow < N) {
    uint16_t* orow = a.o + bat + (size_t)qrow * tok_stride + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int d = 32 * db + 8 * aa + 4 * g;
        u32x2 w;
        w[0] = pack_bf16(o[db][4 * aa + 0] * inv, o[db][4 * aa + 1] * inv);
        w[1] = pack_bf16(o[db][4 * aa + 2] * inv, o[db][4 * aa + 3] * inv);
        *(u32x2*)(orow + d) = w;
      }
  }
}

// One work item per workgroup: whole tiles first (XCD-contiguous, or in the
// given order), then the split pieces of the last round.
template <int D, bool SPARSE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(AttnArgs a) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) char ksm[2][C::KTILEB];
  __shared__ __attribute__((aligned(16))) char vsm[2][C::VTILEB];
  int tile_g, slot = -1, piece = 0;
  if ((int)blockIdx.x < a.whole) {
    tile_g = a.tile_order != nullptr ? a.tile_order[blockIdx.x] : xcd_tile_order(blockIdx.x, a.whole);
  } else {
    // pieces of neighbouring tiles on one XCD, like the whole tiles
    slot = xcd_tile_order(blockIdx.x - a.whole, gridDim.x - a.whole);
    tile_g = a.whole + slot / a.split;
    if (a.tile_order != nullptr) tile_g = a.tile_order[tile_g];
    piece = slot % a.split;
  }
  const ClockProbe probe(a.clk);
  fwd_tile<D, SPARSE>(a, ksm, vsm, tile_g, slot, piece, -1, -1);
  probe.finish();
}

// Persistent split (one workgroup per CU, dense): the launch's tiles x K/V
// positions, flattened, are cut into gridDim.x equal slices; a slice runs the
// pieces of the tiles it covers one after the other.  A piece that is not a
// whole tile stores its partial state in slot 2c (the slice's first tile) or
// 2c + 1 (its last), and attn_merge_sk_kernel combines them.  Slices of one
// XCD are adjacent.
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_persistent_kernel(AttnArgs a) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) char ksm[2][C::KTILEB];
  __shared__ __attribute__((aligned(16))) char vsm[2][C::VTILEB];
  const int nkv = a.sk_nkv;
  const int cu = xcd_tile_order(blockIdx.x, gridDim.x);
  const long W = (long)a.sk_tiles * nkv;
  const long hi = W * (cu + 1) / gridDim.x;
  long pos = W * cu / gridDim.x;
  const int first = (int)(pos / nkv);
  const ClockProbe probe(a.clk);
  while (pos < hi) {
    const int tile_g = (int)(pos / nkv);
    const long next = hi < (long)(tile_g + 1) * nkv ? hi : (long)(tile_g + 1) * nkv;
    const int k0 = (int)(pos - (long)tile_g * nkv), k1 = (int)(next - (long)tile_g * nkv);
    const int slot = (k0 != 0 || k1 != nkv) ? 2 * cu + (tile_g == first ? 0 : 1) : -1;
    fwd_tile<D, false>(a, ksm, vsm, tile_g, slot, 0, k0, k1);
    pos = next;
    if (pos < hi) __syncthreads();  // the next piece reuses the LDS buffers
  }
  probe.finish();
}

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, const Schedule& sch, hipStream_t stream) {
  AttnArgs args = a;
  args.whole = sch.whole_tiles;
  args.split = sch.split;
  args.sk_nkv = sch.sk_nkv;
  args.sk_tiles = sch.sk_tiles;
  args.sk_cus = sch.sk_cus;
  const bool sparse = a.kv_list != nullptr;
  if (sch.sk_nkv > 0 && !sparse) {
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_fwd_bf16_persistent_kernel<128>, dim3(sch.grid), dim3(Bf16Cfg<128>::NT), 0, stream, args);
    else if (head_dim == 64)
      hipLaunchKernelGGL(attn_fwd_bf16_persistent_kernel<64>, dim3(sch.grid), dim3(Bf16Cfg<64>::NT), 0, stream, args);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (head_dim == 128 && !sparse)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), dim3(sch.grid), dim3(Bf16Cfg<128>::NT), 0, stream, args);
  else if (head_dim == 128)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), dim3(sch.grid), dim3(Bf16Cfg<128>::NT), 0, stream, args);
  else if (head_dim == 64 && !sparse)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false>), dim3(sch.grid), dim3(Bf16Cfg<64>::NT), 0, stream, args);
  else if (head_dim == 64)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true>), dim3(sch.grid), dim3(Bf16Cfg<64>::NT), 0, stream, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace flux
