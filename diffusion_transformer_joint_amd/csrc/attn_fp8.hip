// e4m3 joint RoPE attention for gfx950 (MI355X).
//
// FP8 variant of the joint attention: query, key and value arrive as OCP e4m3
// codes with one scale per (tensor, batch, head) ("Optimizing FLUX 3 Image
// Klein inference on NVIDIA Blackwell GPUs", How it works: quantized attention
// with query, key and value in FP8).  The result is the attention of the
// dequantized inputs (codes x scale), bf16 out.
//
// Where quantization happens (the pages do not say): the rotary embedding is
// part of this path, so Q and K are rotated here.  Codes are widened to fp16
// (exactly), rotated with packed fp16 arithmetic, halved and rounded back to
// e4m3; rotation is linear, so the scales
// never enter the loop (a rotated pair component is at most sqrt(2) times the
// pair's largest code, so halving keeps it under 448).  Scores are fp8 MFMA
// sums of those codes times 4 * s_q * s_k.  P stays bf16 (e4m3 P costs ~2%
// relative error); V codes are widened exactly to bf16 (every e4m3 value is a
// bf16 value) and s_v is applied to the output.
//
// Work decomposition, LDS pipeline, softmax and split/merge are those of the
// bf16 kernel; only the score MFMA (32x32x64 e4m3, K tile in LDS as codes) and
// the staging conversions differ.
#include <type_traits>

#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"

namespace flux {

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int D>
struct Fp8Cfg {
  static constexpr int BM = 256;             // query rows per workgroup
  static constexpr int BN = 64;              // keys per K/V tile
  static constexpr int NT = 512;             // threads (8 waves x 32 rows)
  static constexpr int KS8 = D / 64;         // 64-wide k-steps of the fp8 score MFMA
  static constexpr int DB = D / 32;          // 32-wide d blocks of O
  static constexpr int CPR8 = D / 16;        // 16-code chunks per row
  static constexpr int NCH = BN * CPR8;      // chunks per tile (<= NT)
  static constexpr int K8ROW = D + 16;       // LDS bytes per K code row (16-byte skew)
  static constexpr int K8TILEB = BN * K8ROW;
  static constexpr int VTILEB = BN * (2 * D + 64);  // V tile as bf16, rows as in the bf16 kernel
};

// One pair of codes widened to fp16, p = (x0, x1), rotated by its table
// entry cs = (cos, sin): x0 (cos, sin) + x1 (-sin, cos), as packed fp16
// products (the swap and the sign are operand modifiers).  Every e4m3 value
// and every rotated value (|y| <= 448 sqrt 2) is an fp16 normal number; the
// fp16 product and sum round at 2^-11, far below the e4m3 rounding (2^-4)
// that follows.
__device__ __forceinline__ f16x2 rot_pair_f16(f16x2 p, f16x2 cs) {
  const f16x2 sc = {-cs[1], cs[0]};
  const f16x2 a = {p[0], p[0]}, b = {p[1], p[1]};
  return __builtin_elementwise_fma(a, cs, b * sc);
}

// One dword of codes (two pairs) rotated by table entries w0, w1 and halved
// back to e4m3: one exact widening per pair, two packed fp16 operations per
// pair, one scaled conversion per pair (scale 2: the halving costs nothing).
__device__ __forceinline__ uint32_t rope_dword_e4m3(uint32_t x, uint32_t w0, uint32_t w1) {
  const f16x2 y0 = rot_pair_f16(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x, 1.0f, false),
                                __builtin_bit_cast(f16x2, w0));
  const f16x2 y1 = rot_pair_f16(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x, 1.0f, true),
                                __builtin_bit_cast(f16x2, w1));
  s16x2 r = __builtin_bit_cast(s16x2, x);  // both halves are overwritten
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, y0, 2.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, y1, 2.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}

// The 8 pairs of 16 codes x (dword-packed) rotated by their table entries
// w[0] (pairs 0-3) and w[1] (pairs 4-7), halved, as e4m3 codes.
__device__ __forceinline__ u32x4 rope16_e4m3(u32x4 x, const u32x4 (&w)[2]) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = rope_dword_e4m3(x[i], w[i >> 1][2 * (i & 1)], w[i >> 1][2 * (i & 1) + 1]);
  return y;
}

// 16 codes to 16 bf16 (exact): two 16-byte halves.  One gfx950 conversion
// per code pair (scale 1).
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4 x, u32x4* lo, u32x4* hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4& dst = i < 2 ? *lo : *hi;
    dst[(i & 1) * 2 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[i], 1.0f, false));
    dst[(i & 1) * 2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[i], 1.0f, true));
  }
}

// One work item per workgroup: a whole query tile, or one K/V piece of a
// split tile of the last round.
template <int D>
__device__ __forceinline__ void fp8_tile(const Fp8Args& a, char (&ksm)[2][Fp8Cfg<D>::K8TILEB],
                                         char (&vsm)[2][Fp8Cfg<D>::VTILEB]) {
  using C = Fp8Cfg<D>;

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
  const size_t tok_stride = (size_t)H * D;  // codes between consecutive tokens
  const size_t bat = (size_t)b * a.batch_tokens * tok_stride;
  const uint8_t* qbase = a.q + bat + (size_t)h * D;
  const uint8_t* kbase = a.k + bat + (size_t)h * D;
  const uint8_t* vbase = a.v + bat + (size_t)h * D;
  const float s_q = a.scales[(0 * a.batch + b) * H + h];
  const float s_k = a.scales[(1 * a.batch + b) * H + h];
  const float s_v = a.scales[(2 * a.batch + b) * H + h];
  const float sc = 4.0f * s_q * s_k * a.c;  // score (exp2 domain) per unit of code dot product

  // ---- Q fragments: 32 codes per lane per 64-wide k-step, rotated and halved.
  const int qrow = qt * C::BM + wave * 32 + l32;
  i32x8 qf[C::KS8];
#pragma unroll
  for (int t = 0; t < C::KS8; ++t) {
    u32x4 y[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int d0 = 64 * t + 32 * g + 16 * hf;
      u32x4 x = {0, 0, 0, 0};
      constexpr uint32_t kIdentity = 0x3C00u;  // cos 1, sin 0 (fp16)
      u32x4 cs[2] = {{kIdentity, kIdentity, kIdentity, kIdentity}, {kIdentity, kIdentity, kIdentity, kIdentity}};
      if (qrow < N) {
        x = global_load_b128(qbase + (size_t)qrow * tok_stride + d0);
        const u32x4* rp = (const u32x4*)(a.rope + (size_t)qrow * (D / 2) + d0 / 2);
        cs[0] = rp[0];
        cs[1] = rp[1];
      }
      y[hf] = rope16_e4m3(x, cs);
    }
    const uint32_t w[8] = {y[0][0], y[0][1], y[0][2], y[0][3], y[1][0], y[1][1], y[1][2], y[1][3]};
    qf[t] = __builtin_bit_cast(i32x8, w);
  }

  // ---- staging: one 16-code chunk of K and of V per thread and tile.
  // Thread-to-row maps chosen so that each 16-lane phase of an LDS store
  // covers every bank once (64 banks of 4 bytes):
  //   K: a thread stages one 16-code chunk; a phase holds 16 / CPR8 rows
  //      spaced KSP apart, whose padded rows (D + 16 bytes) then start 64 /
  //      (16 / CPR8) banks apart.
  //   V: a thread stages 8 codes of each of two rows (two 8-byte loads) and
  //      stores each as one 16-byte bf16 chunk; per store a phase covers one
  //      whole row (D = 128) or two rows 2 apart (D = 64), whose padded rows
  //      (2 D + 64 bytes) start 32 banks apart.
  const bool st_on = C::NCH >= C::NT || tid < C::NCH;  // every thread stages when D = 128
  const int ph = tid >> 4, pl = tid & 15;  // 16-lane phase, lane in the phase
  constexpr int KRP = 16 / C::CPR8, KSP = D == 128 ? 8 : 4;
  const int k_row = (ph % KSP) + KSP * KRP * (ph / KSP) + KSP * (pl / C::CPR8), k_c = pl % C::CPR8;
  constexpr int VCPR = D / 8, VRP = 16 / VCPR;  // 8-code chunks per row, rows per phase and store
  const int v_row = 2 * VRP * ph + 2 * (pl / VCPR), v_c = pl % VCPR;  // rows v_row, v_row + 1
  const uint32_t k_gl = (uint32_t)(k_row * tok_stride + k_c * 16);
  const uint32_t rp_off = (uint32_t)(k_row * (D / 2) * 4 + k_c * 32);
  const uint32_t k_lds = (uint32_t)(k_row * C::K8ROW + k_c * 16);
  const uint32_t v_gl = (uint32_t)(v_row * tok_stride + v_c * 8);
  const uint32_t v_lds0 = (uint32_t)v_off<D>(v_row, v_c), v_lds1 = (uint32_t)v_off<D>(v_row + 1, v_c);
  u32x4 kraw, vraw;
  u32x4 kcs[2];
  auto stage_load_k = [&](int kt0) {
    if (!st_on) return;
    const int rows = N - kt0;
    const uint32_t kv_bytes = rows > 0 ? (uint32_t)((rows - 1) * tok_stride + D) : 0u;
    const uint32_t rp_bytes = rows > 0 ? (uint32_t)(rows * (D / 2) * 4) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)kt0 * tok_stride, kv_bytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.rope + (size_t)kt0 * (D / 2), rp_bytes);
    kraw = buffer_load_b128(rk, k_gl);
#pragma unroll
    for (int i = 0; i < 2; ++i) kcs[i] = buffer_load_b128(rr, rp_off + 16 * i);
  };
  auto stage_load_v = [&](int kt0) {
    if (!st_on) return;
    const int rows = N - kt0;
    const uint32_t kv_bytes = rows > 0 ? (uint32_t)((rows - 1) * tok_stride + D) : 0u;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)kt0 * tok_stride, kv_bytes);
    const u32x2 v0 = buffer_load_b64(rv, v_gl), v1 = buffer_load_b64(rv, v_gl + (uint32_t)tok_stride);
    vraw = (u32x4){v0[0], v0[1], v1[0], v1[1]};
  };
  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = (f32x16){};
  float m_ref = 0.f;  // reference of the scaled score (exp2 domain): p = exp2(s * sc - m_ref)
  float lsum = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int grp = lane >> 4, li = lane & 15;

  auto kfrag = [&](const FLUX_LDS char* kl, int kb, int t) -> i32x8 {
    const FLUX_LDS char* p = kl + (32 * kb + krow_perm(l32)) * C::K8ROW + 64 * t + 32 * g;
    const u32x4 x0 = lds_read_b128(p), x1 = lds_read_b128(p + 16);
    const uint32_t w[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    return __builtin_bit_cast(i32x8, w);
  };
  auto qk = [&](const FLUX_LDS char* kl, int kb) -> f32x16 {
    i32x8 kf[C::KS8];
#pragma unroll
    for (int t = 0; t < C::KS8; ++t) kf[t] = kfrag(kl, kb, t);
    f32x16 s = {};
#pragma unroll
    for (int t = 0; t < C::KS8; ++t) s = mfma_fp8(kf[t], qf[t], s);
    return s;
  };
  auto mask = [&](int kt0, int kb, f32x16& s) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kt0 + 32 * kb + 16 * (e >> 3) + 8 * g + (e & 7);
      if (key >= N) s[e] = -INFINITY;
    }
  };
  // Reference m as in the bf16 kernel: the first tile of the range sets it to
  // the row max; later tiles form p directly and only move it when a row's
  // tile sum reaches 2^32 (or is not finite).
  auto block_max = [&](const f32x16& s) -> float {
    float mt = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s[e]);
    return fmaxf(mt, swap_halves(mt)) * sc;
  };
  auto rescale_o = [&](float alpha) {
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
  };
  auto p_pair = [&](float x0, float x1, float& bsum) -> uint32_t {
    bf16x2 q2;
    q2[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(x0, sc, -m_ref));
    q2[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(x1, sc, -m_ref));
    bsum = __builtin_amdgcn_fdot2_f32_bf16(q2, ones, bsum, false);
    return __builtin_bit_cast(uint32_t, q2);
  };
  auto make_p = [&](const f32x16& s, int hh, float& bsum) -> u32x4 {
    u32x4 pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = p_pair(s[8 * hh + 2 * i], s[8 * hh + 2 * i + 1], bsum);
    return pf;
  };
  auto block_ok = [&](float bsum) -> bool { return __ballot(!(bsum < 0x1p32f)) == 0; };
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
  auto store_k = [&](int buf) {
    if (!st_on) return;
    FLUX_LDS char* kl = (FLUX_LDS char*)ksm[buf];
    lds_write_b128(kl + k_lds, rope16_e4m3(kraw, kcs));
  };
  auto store_v = [&](int buf) {
    if (!st_on) return;
    FLUX_LDS char* vl = (FLUX_LDS char*)vsm[buf];
    u32x4 lo, hi;
    e4m3x16_to_bf16(vraw, &lo, &hi);
    lds_write_b128(vl + v_lds0, lo);
    lds_write_b128(vl + v_lds1, hi);
  };

  // Software pipeline over 64-key tiles, as in the bf16 kernel.  Iteration t:
  //   MFMA:  S(t) = QK(t) (fp8), then O += PV(t-1) (bf16) with P(t-1);
  //   VALU:  RoPE + requantization and LDS store of K(t+1), widening and store
  //          of V(t) beside them; P(t) beside PV; global loads of the next tiles.
  //   barrier.
  // K(t+1) and V(t) go into the buffers that K(t-1) and V(t-2) held.
  stage_load_k(kv0 * C::BN);
  store_k(0);
  stage_load_k((kv0 + 1) * C::BN);
  stage_load_v(kv0 * C::BN);
  __syncthreads();

  u32x4 pp[4];  // P(t-1): fragments (block 0, keys 0-15), (0, 16-31), (1, 0-15), (1, 16-31)
  auto rare_move = [&](f32x16& s0, f32x16& s1, float& b) {
    const float m_new = fmaxf(m_ref, bf16_round(fmaxf(block_max(s0), block_max(s1))));
    rescale_o(__builtin_amdgcn_exp2f(m_ref - m_new));
    m_ref = m_new;
    b = 0.f;
    pp[0] = make_p(s0, 0, b);
    pp[1] = make_p(s0, 1, b);
    pp[2] = make_p(s1, 0, b);
    pp[3] = make_p(s1, 1, b);
  };
  // The first tile of the range (no PV yet): its row max sets m.
  auto step_first = [&](auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm[0];
    const int kt0 = kv0 * C::BN;
    f32x16 s0 = qk(kl, 0);
    f32x16 s1 = qk(kl, 1);
    if (LAST) {
      mask(kt0, 0, s0);
      mask(kt0, 1, s1);
    }
    m_ref = bf16_round(fmaxf(block_max(s0), block_max(s1)));
    float b = 0.f;
    pp[0] = make_p(s0, 0, b);
    pp[1] = make_p(s0, 1, b);
    pp[2] = make_p(s1, 0, b);
    pp[3] = make_p(s1, 1, b);
    if (!block_ok(b)) rare_move(s0, s1, b);
    lsum += b;
    store_k(1);
    store_v(0);
    stage_load_k((kv0 + 2) * C::BN);
    stage_load_v((kv0 + 1) * C::BN);
    __syncthreads();
  };
  // Every later tile: one fixed-order MFMA stream (QK(t), then PV(t-1)), each
  // MFMA followed by its operand reads NPF MFMAs ahead and a slice of VALU work.
  auto step_main = [&](int t, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int i = t - kv0;
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm[i & 1];
    const FLUX_LDS char* vl = (const FLUX_LDS char*)vsm[(i + 1) & 1];  // V(t-1)
    const int kt0 = t * C::BN;
    constexpr int NK = 2 * C::KS8, NV = 4 * C::DB, NL = NK + NV;
    auto vfrag = [&](int v) -> u32x4 {
      const int kb = v / (2 * C::DB), hh = (v / C::DB) & 1, db = v % C::DB;
      const int krow0 = 32 * kb + 16 * hh + 8 * (grp >> 1) + (li >> 2);
      const int d = 32 * db + 16 * (grp & 1) + 4 * (li & 3);
      const u32x2 lo = lds_read_tr16(vl + v_off<D>(krow0, d >> 3) + (d & 7) * 2);
      const u32x2 hi = lds_read_tr16(vl + v_off<D>(krow0 + 4, d >> 3) + (d & 7) * 2);
      return (u32x4){lo[0], lo[1], hi[0], hi[1]};
    };
    // K fragments are read two MFMAs ahead, V fragments NPF ahead.
    constexpr int NPF = 3;
    i32x8 fk[2];
    u32x4 fv[NPF];
    fk[0] = kfrag(kl, 0, 0);
    if constexpr (NK > 1) fk[1] = kfrag(kl, 1 / C::KS8, 1 % C::KS8);
    FLUX_LDS char* kw = (FLUX_LDS char*)ksm[(i + 1) & 1];  // K(t+1)
    FLUX_LDS char* vw = (FLUX_LDS char*)vsm[i & 1];        // V(t)
    u32x4 ky, vlo, vhi;
    f32x16 s0 = (f32x16){}, s1 = (f32x16){};
    float b = 0.f;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NL>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < NK) {
        const i32x8 x = fk[j % 2];
        if constexpr (j + 2 < NK) fk[j % 2] = kfrag(kl, (j + 2) / C::KS8, (j + 2) % C::KS8);
        if constexpr (j < C::KS8) s0 = mfma_fp8(x, qf[j], s0);
        else s1 = mfma_fp8(x, qf[j - C::KS8], s1);
      } else {
        constexpr int v = j - NK, q4 = v / C::DB, db = v % C::DB;
        const u32x4 x = fv[v % NPF];
        o[db] = mfma_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, pp[q4]), o[db]);
      }
      // V fragment v is read in slot NK + v - NPF (or before the first PV MFMA)
      constexpr int vn = j - NK + NPF;
      if constexpr (j >= NK - 1 && j < NK) {
#pragma unroll
        for (int v0 = 0; v0 < NPF; ++v0) fv[v0] = vfrag(v0);
      } else if constexpr (j >= NK && vn < NV) {
        fv[vn % NPF] = vfrag(vn);
      }
      // staging: RoPE of K(t+1), one dword of codes per slot, beside the
      // 64-cycle score MFMAs (K(t+1) goes to the buffer K(t-1) held, which
      // is no longer read), then its store; V(t) widened and stored beside
      // the first output MFMA; loads of K(t+2) and V(t+1) behind them.
      constexpr int RS = 4;                  // dwords of codes per staged chunk
      constexpr int R0 = NK >= RS ? 0 : NK;  // first staging slot
      if constexpr (j >= R0 && j < R0 + RS) {
        if (st_on) ky[j - R0] = rope_dword_e4m3(kraw[j - R0], kcs[(j - R0) >> 1][2 * ((j - R0) & 1)], kcs[(j - R0) >> 1][2 * ((j - R0) & 1) + 1]);
        if constexpr (j == R0 + RS - 1) {
          if (st_on) lds_write_b128(kw + k_lds, ky);
        }
      }
      constexpr int RV = NK > R0 + RS ? NK : R0 + RS;  // V(t) staging slot
      if constexpr (j == RV) {
        if (st_on) {
          e4m3x16_to_bf16(vraw, &vlo, &vhi);
          lds_write_b128(vw + v_lds0, vlo);
          lds_write_b128(vw + v_lds1, vhi);
        }
      }
      if constexpr (j == RV + 1) stage_load_k((t + 2) * C::BN);
      if constexpr (j == RV + 2) stage_load_v((t + 1) * C::BN);
      if constexpr (j >= NK) {
        constexpr int v = j - NK;
        if (LAST && v == 0) mask(kt0, 0, s0);
        if (LAST && v == 1) mask(kt0, 1, s1);
        if constexpr (v >= C::DB) {  // P(t) slice q replaces P(t-1) slice q
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
    for (int e2 = 0; e2 < 4; ++e2) pp[3][e2] = p_pair(s1[8 + 2 * e2], s1[8 + 2 * e2 + 1], b);
    if (!block_ok(b)) rare_move(s0, s1, b);  // rare
    lsum += b;
    __syncthreads();
  };

  const int full_end = min(kv1, N / C::BN);  // tiles before this one are full
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

  const float ltot = lsum + swap_halves(lsum);
  if (slot >= 0) {
    const int r = wave * 32 + l32;
    float* po = a.part_o + ((size_t)slot * C::BM + r) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const f32x4 w = {o[db][4 * aa] * s_v, o[db][4 * aa + 1] * s_v, o[db][4 * aa + 2] * s_v, o[db][4 * aa + 3] * s_v};
        *(f32x4*)(po + 32 * db + 8 * aa + 4 * g) = w;
      }
    if (g == 0) a.part_ml[(size_t)slot * C::BM + r] = make_float2(m_ref, ltot);
    return;
  }
  const float inv = s_v / ltot;
  if (qrow < N) {
    uint16_t* orow = a.o + (size_t)b * a.batch_tokens * tok_stride + (size_t)qrow * tok_stride + (size_t)h * D;
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

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(Fp8Args a) {
  using C = Fp8Cfg<D>;
  __shared__ __attribute__((aligned(16))) char ksm[2][C::K8TILEB];
  __shared__ __attribute__((aligned(16))) char vsm[2][C::VTILEB];
  const ClockProbe probe(a.clk);
  fp8_tile<D>(a, ksm, vsm);
  probe.finish();
}

hipError_t launch_attn_fp8(const Fp8Args& a, int head_dim, const Schedule& sch, hipStream_t stream) {
  Fp8Args args = a;
  args.q_tiles = (a.n_tokens + 255) / 256;
  args.whole = sch.whole_tiles;
  args.split = sch.split;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<128>, dim3(sch.grid), dim3(Fp8Cfg<128>::NT), 0, stream, args);
  else if (head_dim == 64)
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<64>, dim3(sch.grid), dim3(Fp8Cfg<64>::NT), 0, stream, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace flux
