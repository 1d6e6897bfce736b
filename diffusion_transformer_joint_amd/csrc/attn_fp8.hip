// e4m3 joint RoPE attention for gfx950 (MI355X).
//
// FP8 variant of the joint attention: query, key and value arrive as OCP e4m3
// codes with one scale per (tensor, batch, head) ("Optimizing FLUX 3 Image
// Klein inference on NVIDIA Blackwell GPUs", How it works: quantized attention
// with query, key and value in FP8).  The result is the attention of the
// dequantized inputs (codes x scale), bf16 out.
//
// Where quantization happens (the pages do not say): the rotary embedding is
// part of this path, so Q and K are rotated here.  Codes are widened to fp32,
// rotated, halved and rounded back to e4m3; rotation is linear, so the scales
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

typedef float f32x2 __attribute__((ext_vector_type(2)));

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

// Four e4m3 codes (one dword) to floats.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* f) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// Four floats to e4m3 codes (one dword), round to nearest even.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Rotate the 8 pairs of 16 codes x (dword-packed) by (cos, sin) in cs[0..3]
// (two pairs per f32x4) and return the halved result as e4m3 codes.
__device__ __forceinline__ u32x4 rope16_e4m3(u32x4 x, const f32x4* cs) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[4];
    e4m3x4_to_f32(x[i], f);
    // pairs (f0, f1) and (f2, f3); angles 2i and 2i+1 of the chunk
    const float c0 = 0.5f * cs[i][0], s0 = 0.5f * cs[i][1];
    const float c1 = 0.5f * cs[i][2], s1 = 0.5f * cs[i][3];
    y[i] = f32x4_to_e4m3(f[0] * c0 - f[1] * s0, f[0] * s0 + f[1] * c0, f[2] * c1 - f[3] * s1, f[2] * s1 + f[3] * c1);
  }
  return y;
}

// 16 codes to 16 bf16 (exact): two 16-byte halves.
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4 x, u32x4* lo, u32x4* hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[4];
    e4m3x4_to_f32(x[i], f);
    u32x4& dst = i < 2 ? *lo : *hi;
    dst[(i & 1) * 2 + 0] = pack_bf16(f[0], f[1]);
    dst[(i & 1) * 2 + 1] = pack_bf16(f[2], f[3]);
  }
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(Fp8Args a) {
  using C = Fp8Cfg<D>;
  __shared__ __attribute__((aligned(16))) char ksm[2][C::K8TILEB];
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
      f32x4 cs[4] = {{1.f, 0.f, 1.f, 0.f}, {1.f, 0.f, 1.f, 0.f}, {1.f, 0.f, 1.f, 0.f}, {1.f, 0.f, 1.f, 0.f}};
      if (qrow < N) {
        x = global_load_b128(qbase + (size_t)qrow * tok_stride + d0);
        const f32x4* rp = (const f32x4*)(a.rope + (size_t)qrow * (D / 2) + d0 / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = rp[i];
      }
      y[hf] = rope16_e4m3(x, cs);
    }
    const uint32_t w[8] = {y[0][0], y[0][1], y[0][2], y[0][3], y[1][0], y[1][1], y[1][2], y[1][3]};
    qf[t] = __builtin_bit_cast(i32x8, w);
  }

  // ---- staging: one 16-code chunk of K and of V per thread and tile.
  const bool st_on = tid < C::NCH;
  const int st_row = tid / C::CPR8, st_c = tid % C::CPR8;
  const uint32_t kv_off = (uint32_t)(st_row * tok_stride + st_c * 16);
  const uint32_t rp_off = (uint32_t)(st_row * (D / 2) * 8 + st_c * 64);
  u32x4 kraw, vraw;
  f32x4 kcs[4];
  auto stage_load = [&](int kt0) {
    if (!st_on) return;
    const int rows = N - kt0;
    const uint32_t kv_bytes = rows > 0 ? (uint32_t)((rows - 1) * tok_stride + D) : 0u;
    const uint32_t rp_bytes = rows > 0 ? (uint32_t)(rows * (D / 2) * 8) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)kt0 * tok_stride, kv_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)kt0 * tok_stride, kv_bytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.rope + (size_t)kt0 * (D / 2), rp_bytes);
    kraw = buffer_load_b128(rk, kv_off);
    vraw = buffer_load_b128(rv, kv_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) kcs[i] = __builtin_bit_cast(f32x4, buffer_load_b128(rr, rp_off + 16 * i));
  };
  auto stage_store = [&](int buf) {
    if (!st_on) return;
    FLUX_LDS char* kl = (FLUX_LDS char*)ksm[buf];
    FLUX_LDS char* vl = (FLUX_LDS char*)vsm[buf];
    lds_write_b128(kl + st_row * C::K8ROW + st_c * 16, rope16_e4m3(kraw, kcs));
    u32x4 lo, hi;
    e4m3x16_to_bf16(vraw, &lo, &hi);
    lds_write_b128(vl + v_off<D>(st_row, 2 * st_c), lo);
    lds_write_b128(vl + v_off<D>(st_row, 2 * st_c + 1), hi);
  };

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = (f32x16){};
  float m_ref = -INFINITY;  // running max of the scaled score, exp2 domain
  float lsum = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int grp = lane >> 4, li = lane & 15;

  auto qk = [&](const FLUX_LDS char* kl, int kb) -> f32x16 {
    const int krow = 32 * kb + krow_perm(l32);
    i32x8 kf[C::KS8];
#pragma unroll
    for (int t = 0; t < C::KS8; ++t) {
      const FLUX_LDS char* p = kl + krow * C::K8ROW + 64 * t + 32 * g;
      const u32x4 x0 = lds_read_b128(p), x1 = lds_read_b128(p + 16);
      const uint32_t w[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      kf[t] = __builtin_bit_cast(i32x8, w);
    }
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
  // Lazy running max in the exp2 domain: moves only when a row's block max
  // exceeds it by more than 8 (p stays <= 256).
  auto update_max = [&](const f32x16& s, float* alpha) -> bool {
    float mt = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s[e]);
    mt = fmaxf(mt, swap_halves(mt));
    const float ms = mt * sc;
    const bool need = ms > m_ref + 8.0f;
    *alpha = 1.0f;
    if (__ballot(need) == 0) return false;
    *alpha = need ? __builtin_amdgcn_exp2f(m_ref - ms) : 1.0f;
    m_ref = need ? ms : m_ref;
    return true;
  };
  auto rescale_o = [&](float alpha) {
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
  };
  auto make_p = [&](const f32x16& s, int hh) -> u32x4 {
    u32x4 pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hh + 2 * i], sc, -m_ref));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hh + 2 * i + 1], sc, -m_ref));
      bf16x2 pp;
      pp[0] = (__bf16)p0;
      pp[1] = (__bf16)p1;
      pf[i] = __builtin_bit_cast(uint32_t, pp);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
    }
    return pf;
  };
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

  stage_load(kv0 * C::BN);
  stage_store(0);
  stage_load((kv0 + 1) * C::BN);
  __syncthreads();

  // Per tile: S0 = QK(block 0) || store of tile j+1; S1 = QK(block 1) || P of
  // block 0 and loads of tile j+2; O += PV(block 0) || P of block 1;
  // O += PV(block 1).  Same buffer discipline as the bf16 kernel.
  auto tile_step = [&](int j, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int buf = (j - kv0) & 1;
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm[buf];
    const FLUX_LDS char* vl = (const FLUX_LDS char*)vsm[buf];
    const int kt0 = j * C::BN;
    float alpha;

    f32x16 s0 = qk(kl, 0);
    stage_store(buf ^ 1);
    if (LAST) mask(kt0, 0, s0);
    if (update_max(s0, &alpha)) rescale_o(alpha);

    f32x16 s1 = qk(kl, 1);
    const u32x4 p00 = make_p(s0, 0);
    const u32x4 p01 = make_p(s0, 1);
    stage_load((j + 2) * C::BN);
    sched_interleave<C::KS8, 8>();
    if (LAST) mask(kt0, 1, s1);
    if (update_max(s1, &alpha)) {
      rescale_o(alpha);
      // P of block 0 was formed with the old reference: rescale it too.
      u32x4 q0 = p00, q1 = p01;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q0[i] = pack_bf16(bf16lo(q0[i]) * alpha, bf16hi(q0[i]) * alpha);
        q1[i] = pack_bf16(bf16lo(q1[i]) * alpha, bf16hi(q1[i]) * alpha);
      }
      pv(vl, 0, 0, q0);
      pv(vl, 0, 1, q1);
    } else {
      pv(vl, 0, 0, p00);
      pv(vl, 0, 1, p01);
    }
    const u32x4 p10 = make_p(s1, 0);
    const u32x4 p11 = make_p(s1, 1);
    pv(vl, 1, 0, p10);
    pv(vl, 1, 1, p11);
    sched_interleave<2 * C::DB, 4>();
    __syncthreads();
  };

  const int full_end = min(kv1, N / C::BN);
  for (int j = kv0; j < full_end; ++j) tile_step(j, std::false_type{});
  if (full_end < kv1) tile_step(full_end, std::true_type{});

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
