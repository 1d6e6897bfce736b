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
//   workgroup = 8 waves x 32 query rows = 256 rows (two waves per SIMD, so one
//   wave's softmax can run while the other issues MFMAs); K/V streamed in
//   64-key tiles, double-buffered in LDS (K rotated on the way in, rows padded).
//   S^T = K Q^T is computed so that each lane owns one query (lane % 32) and
//   16 keys per 32-key block: the softmax row reductions are in-lane plus one
//   exchange between the two wave halves.
//   O^T += V^T P^T reuses the S^T accumulator registers directly as the P^T
//   operand (rounded to bf16); V^T fragments come from row-major V in LDS
//   through the gfx950 transpose read.
//   Online softmax (Milakov & Gimelshein 2018) with a lazily updated running
//   max: the reference max only moves when a row's tile max exceeds it by more
//   than 2^8 in the exp2 domain, which keeps every p <= 256 and skips most
//   rescales of the output accumulators; the result is the same softmax.
//
// Layouts: q, k, v, o [B][N][H][D] bf16; rope [N][D/2] float2 (cos, sin).
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

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(AttnArgs a) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) char ksm[2][C::KTILEB];
  __shared__ __attribute__((aligned(16))) char vsm[2][C::VTILEB];

  const int N = a.n_tokens, H = a.heads;
  const int n_tiles = (N + C::BN - 1) / C::BN;
  int tile, kv0 = 0, kv1 = n_tiles, slot = -1;
  if ((int)blockIdx.x < a.whole) {
    tile = xcd_tile_order(blockIdx.x, a.whole);
  } else {
    slot = blockIdx.x - a.whole;
    tile = a.whole + slot / a.split;
    const int piece = slot % a.split;
    kv0 = piece * n_tiles / a.split;
    kv1 = (piece + 1) * n_tiles / a.split;
  }
  const int qt = tile % a.q_tiles;
  const int bh = tile / a.q_tiles;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t tok_stride = (size_t)H * D;  // elements between consecutive tokens
  const uint16_t* qbase = a.q + (size_t)b * N * tok_stride + (size_t)h * D;
  const uint16_t* kbase = a.k + (size_t)b * N * tok_stride + (size_t)h * D;
  const uint16_t* vbase = a.v + (size_t)b * N * tok_stride + (size_t)h * D;
  const float c = a.c;

  // ---- Q fragments (B operand of S^T = K Q^T), rotated, held in registers.
  const int qrow = qt * C::BM + wave * 32 + l32;
  bf16x8 qf[C::KSTEPS];
#pragma unroll
  for (int t = 0; t < C::KSTEPS; ++t) {
    const int d0 = 16 * t + 8 * g;
    u32x4 x = {0, 0, 0, 0};
    f32x4 cs01 = {1.f, 0.f, 1.f, 0.f}, cs23 = {1.f, 0.f, 1.f, 0.f};
    if (qrow < N) {
      x = global_load_b128(qbase + (size_t)qrow * tok_stride + d0);
      const f32x4* rp = (const f32x4*)(a.rope + (size_t)qrow * (D / 2) + d0 / 2);
      cs01 = rp[0];
      cs23 = rp[1];
    }
    qf[t] = __builtin_bit_cast(bf16x8, rope_chunk_scaled(x, cs01, cs23, c));
  }
  // Running max folded into the score MFMA: an extra k-step multiplies a
  // column of ones in K by -m in Q, so the accumulator holds c*s - m and
  // p = exp2(acc).  m is kept bf16-representable, so this is exact.  Lanes of
  // the first half-wave carry k index 0 of the step, the others zeros.
  const bf16x8 zero8 = {};
  bf16x8 kone = zero8, qm = zero8;
  if (g == 0) kone[0] = (__bf16)1.0f;

  // ---- staging of K/V tiles: global -> registers -> (K rotated) -> LDS.
  // Each thread owns NPASS (row, 16-byte chunk) slots of a tile, split into two
  // halves with separate lifetimes so that the loads of tile j+2 can be issued
  // as soon as the matching half of tile j+1 has been written to LDS.
  const int st_chunk = tid % C::CPR;
  const int st_row0 = tid / C::CPR;
  constexpr int HALF = C::NPASS / 2;
  u32x4 kraw[C::NPASS], vraw[C::NPASS];
  f32x4 kcs[C::NPASS][2];
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
    rp_off[p] = (uint32_t)(r * (D / 2) * 8 + st_chunk * 32);
  }
  auto stage_load = [&](int kt0, int p) {
    const int rows = N - kt0;
    const uint32_t kv_bytes = rows > 0 ? (uint32_t)((rows - 1) * tok_stride * 2 + 2 * D) : 0u;
    const uint32_t rp_bytes = rows > 0 ? (uint32_t)(rows * (D / 2) * 8) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)kt0 * tok_stride, kv_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)kt0 * tok_stride, kv_bytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.rope + (size_t)kt0 * (D / 2), rp_bytes);
    kraw[p] = buffer_load_b128(rk, kv_off[p]);
    vraw[p] = buffer_load_b128(rv, kv_off[p]);
    kcs[p][0] = __builtin_bit_cast(f32x4, buffer_load_b128(rr, rp_off[p]));
    kcs[p][1] = __builtin_bit_cast(f32x4, buffer_load_b128(rr, rp_off[p] + 16));
  };
  auto stage_store = [&](int buf, int p) {
    FLUX_LDS char* kl = (FLUX_LDS char*)ksm[buf];
    FLUX_LDS char* vl = (FLUX_LDS char*)vsm[buf];
    const int r = st_row0 + p * C::RPP;
    lds_write_b128(kl + k_off<D>(r, st_chunk), rope_chunk(kraw[p], kcs[p][0], kcs[p][1]));
    lds_write_b128(vl + v_off<D>(r, st_chunk), vraw[p]);
  };

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

#pragma unroll
  for (int p = 0; p < C::NPASS; ++p) stage_load(kv0 * C::BN, p);
#pragma unroll
  for (int p = 0; p < C::NPASS; ++p) stage_store(0, p);
#pragma unroll
  for (int p = 0; p < C::NPASS; ++p) stage_load((kv0 + 1) * C::BN, p);
  __syncthreads();

  // Per tile j (buffer j&1 holds tile j, buffer (j+1)&1 receives tile j+1):
  //   1. S0 = QK(block 0)              || RoPE + LDS store of half of tile j+1
  //   2. S1 = QK(block 1)              || P(block 0); loads of that half of tile j+2
  //   3. O += PV(block 0, keys 0-15)   || P(block 1, keys 0-15)
  //   4. O += PV(block 0, keys 16-31)  || P(block 1, keys 16-31)
  //   5. O += PV(block 1)              || RoPE + store of the other half of tile j+1;
  //                                      its loads for tile j+2
  // No max reduction sits between a score block and its P: the block row
  // sums are checked after P is formed (see make_p / block_ok).
  // One tile step; LAST selects the masked variant for a ragged final tile.
  auto tile_step = [&](int j, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int buf = (j - kv0) & 1;
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm[buf];
    const FLUX_LDS char* vl = (const FLUX_LDS char*)vsm[buf];
    const int kt0 = j * C::BN;

    // 1. S0 = QK(block 0) || RoPE + store of the first half of tile j+1.
    f32x16 s0 = qk(kl, 0);
#pragma unroll
    for (int p = 0; p < HALF; ++p) stage_store(buf ^ 1, p);
    sched_interleave<C::KSTEPS, 4>();
    if (LAST) mask(kt0, 0, s0);
    if (j == kv0) {  // first block of the range: m = its row max
      const float m_new = bf16_round(m_ref + block_max(s0));
      rebase(m_new, s0);
      set_ref(m_new);
    }

    // 2. S1 = QK(block 1) || P of block 0; loads of the first half of tile j+2.
    f32x16 s1 = qk(kl, 1);
    float b0 = 0.f, b1 = 0.f;
    u32x4 p00 = make_p(s0, 0, b0);
    u32x4 p01 = make_p(s0, 1, b0);
#pragma unroll
    for (int p = 0; p < HALF; ++p) stage_load((j + 2) * C::BN, p);
    sched_interleave<C::KSTEPS, 6>();
    if (LAST) mask(kt0, 1, s1);
    if (!block_ok(b0)) {  // rare: move m up to block 0's max (s1 used the old m too)
      const float m_new = fmaxf(m_ref, bf16_round(m_ref + block_max(s0)));
      rescale_o(__builtin_amdgcn_exp2f(m_ref - m_new));
      rebase(m_new, s0);
      rebase(m_new, s1);
      set_ref(m_new);
      b0 = 0.f;
      p00 = make_p(s0, 0, b0);
      p01 = make_p(s0, 1, b0);
    }
    lsum += b0;

    // 3.-5. O += PV(block 0) || P of block 1; O += PV(block 1) || RoPE + store
    // of the second half of tile j+1 and its loads for tile j+2.
    pv(vl, 0, 0, p00);
    u32x4 p10 = make_p(s1, 0, b1);
    pv(vl, 0, 1, p01);
    u32x4 p11 = make_p(s1, 1, b1);
    if (!block_ok(b1)) {  // rare: O already holds PV(block 0) at the old m
      const float m_new = fmaxf(m_ref, bf16_round(m_ref + block_max(s1)));
      rescale_o(__builtin_amdgcn_exp2f(m_ref - m_new));
      rebase(m_new, s1);
      set_ref(m_new);
      b1 = 0.f;
      p10 = make_p(s1, 0, b1);
      p11 = make_p(s1, 1, b1);
    }
    lsum += b1;
    pv(vl, 1, 0, p10);
    pv(vl, 1, 1, p11);
#pragma unroll
    for (int p = HALF; p < C::NPASS; ++p) stage_store(buf ^ 1, p);
#pragma unroll
    for (int p = HALF; p < C::NPASS; ++p) stage_load((j + 2) * C::BN, p);
    sched_interleave<4 * C::DB, 5>();
    __syncthreads();
  };

  const int full_end = min(kv1, N / C::BN);  // tiles before this one are full
  for (int j = kv0; j < full_end; ++j) tile_step(j, std::false_type{});
  if (full_end < kv1) tile_step(full_end, std::true_type{});

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
    if (g == 0) a.part_ml[(size_t)slot * C::BM + r] = make_float2(m_ref, ltot);
    return;
  }
  // ---- epilogue: O = O^T / l, bf16, stored row-major.
  const float inv = 1.0f / ltot;
  if (qrow < N) {
    uint16_t* orow = a.o + (size_t)b * N * tok_stride + (size_t)qrow * tok_stride + (size_t)h * D;
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

// One thread per (split tile, row, 8 output dims): combines the `split`
// partial states of its row exactly and writes bf16.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int per_tile = 256 * (D / 8);
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int st = idx / per_tile;
  const int rem = idx - st * per_tile;
  const int r = rem / (D / 8), d0 = (rem % (D / 8)) * 8;
  const int tile = a.whole + st;
  const int qt = tile % a.q_tiles, bh = tile / a.q_tiles;
  const int h = bh % a.heads, b = bh / a.heads;
  const int row = qt * 256 + r;
  if (row >= a.n_tokens) return;
  const int slot0 = st * a.split;
  float m = -INFINITY;
  for (int i = 0; i < a.split; ++i) m = fmaxf(m, a.part_ml[(size_t)(slot0 + i) * 256 + r].x);
  float l = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < a.split; ++i) {
    const float2 ml = a.part_ml[(size_t)(slot0 + i) * 256 + r];
    const float w = __builtin_amdgcn_exp2f(ml.x - m);
    l += w * ml.y;
    const float* po = a.part_o + ((size_t)(slot0 + i) * 256 + r) * D + d0;
    const f32x4 x0 = *(const f32x4*)po, x1 = *(const f32x4*)(po + 4);
    acc[0] += w * x0[0]; acc[1] += w * x0[1]; acc[2] += w * x0[2]; acc[3] += w * x0[3];
    acc[4] += w * x1[0]; acc[5] += w * x1[1]; acc[6] += w * x1[2]; acc[7] += w * x1[3];
  }
  const float inv = 1.0f / l;
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = pack_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  const size_t tok_stride = (size_t)a.heads * D;
  *(u32x4*)(a.o + (size_t)b * a.n_tokens * tok_stride + (size_t)row * tok_stride + (size_t)h * D + d0) = out;
}

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, const Schedule& sch, hipStream_t stream) {
  AttnArgs args = a;
  args.q_tiles = (a.n_tokens + 255) / 256;
  args.whole = sch.whole_tiles;
  args.split = sch.split;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, dim3(sch.grid), dim3(Bf16Cfg<128>::NT), 0, stream, args);
  else if (head_dim == 64)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, dim3(sch.grid), dim3(Bf16Cfg<64>::NT), 0, stream, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs& a, int head_dim, const Schedule& sch, hipStream_t stream) {
  if (sch.split_tiles == 0) return hipSuccess;
  AttnArgs args = a;
  args.q_tiles = (a.n_tokens + 255) / 256;
  args.whole = sch.whole_tiles;
  args.split = sch.split;
  const int threads = sch.split_tiles * 256 * (head_dim / 8);
  const int blocks = (threads + 255) / 256;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(blocks), dim3(256), 0, stream, args);
  else if (head_dim == 64)
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(blocks), dim3(256), 0, stream, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace flux
