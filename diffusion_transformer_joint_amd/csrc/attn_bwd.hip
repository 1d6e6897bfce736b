// Backward of the bf16 joint RoPE attention for gfx950 (MI355X).
//
// The adjacent training workload of the path (LoRA fine-tuning of the base
// model, "FLUX.3 Image Klein Brings 2-Second AI Image Generation to
// Diffusers", Summary).  Gradients of O = softmax(scale R(q) R(k)^T) V with
// the row-sum form of the softmax gradient (FlashAttention, Dao et al. 2022):
//   P = exp2(c Q~ K~^T - lse2),  c = scale log2(e),  lse2 = lse / ln 2
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - Dr),  Dr = rowsum(dO O)
//   dQ~ = scale dS K~,  dK~ = scale dS^T Q~,  dq = R^T dQ~,  dk = R^T dK~
// The forward's log-sum-exp (lse) is taken as given; P is recomputed.
//
// Two kernels, no atomics:
//   attn_bwd_dq_kernel   - query-stationary: a wave holds 32 queries (c Q~ and
//                          dO as MFMA B operands); per 64-key tile it forms
//                          S^T = K~ Q~^T and dP^T = V dO^T (lane = query), then
//                          dS^T and dQ~^T += K~^T dS^T (K~ through the LDS
//                          transpose read).
//   attn_bwd_dkdv_kernel - key-stationary: a wave holds 32 keys (c K~ and V as
//                          B operands); per 64-query tile it forms S = Q~ K~^T
//                          and dP = dO V^T (lane = key), then dV^T += dO^T P
//                          and dK~^T += Q~^T dS (dO and Q~ through the
//                          transpose read).
// Both: 4 waves per workgroup (one per SIMD), 128 rows; the 32x32x16 bf16
// MFMA with fp32 accumulation; RoPE applied while tiles are staged and
// transposed back (R^T) on the gradients in the epilogue.
#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"

namespace flux {

namespace {

template <int D>
struct BwdCfg {
  static constexpr int ROWS = 128;         // rows (queries or keys) per workgroup
  static constexpr int T = 64;             // streamed tile
  static constexpr int NT = 256;           // 4 waves
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int ROWB = 2 * D + 16;  // LDS bytes per staged row
  static constexpr int TILEB = T * ROWB;
  static constexpr int CH = T * CPR / NT;  // chunks per thread per staged tile
};

// R^T on a pair: rotation by the negative angle.
__device__ __forceinline__ void rot_back(float& x0, float& x1, float2 cs) {
  const float a = x0 * cs.x + x1 * cs.y;
  const float b = x1 * cs.x - x0 * cs.y;
  x0 = a;
  x1 = b;
}

}  // namespace

// Dr[b][h][i] = sum_d dO[b][i][h][d] * O[b][i][h][d], fp32.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // (b, i, h)
  const int total = a.batch * a.n_tokens * a.heads;
  if (idx >= total) return;
  const int h = idx % a.heads, i = (idx / a.heads) % a.n_tokens, b = idx / (a.heads * a.n_tokens);
  const size_t off = (size_t)idx * D;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 x = *(const u32x4*)(a.dout + off + 8 * c);
    const u32x4 y = *(const u32x4*)(a.out + off + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf16lo(x[e]) * bf16lo(y[e]) + bf16hi(x[e]) * bf16hi(y[e]);
  }
  a.dr[((size_t)b * a.heads + h) * a.n_tokens + i] = s;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dq_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char ksm[C::TILEB];  // K~ tile (rotated)
  __shared__ __attribute__((aligned(16))) char vsm[C::TILEB];  // V tile
  const int N = a.n_tokens, H = a.heads;
  const int q_tiles = (N + C::ROWS - 1) / C::ROWS;
  const int qt = blockIdx.x % q_tiles, bh = blockIdx.x / q_tiles;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const size_t ts = (size_t)H * D;                          // elements between tokens
  const size_t base = (size_t)b * N * ts + (size_t)h * D;
  const float c = a.c;

  // queries of this lane: c R(q) and dO as B fragments; lse2 and Dr
  const int qrow = qt * C::ROWS + wave * 32 + l32;
  const bool qok = qrow < N;
  bf16x8 qf[C::KSTEPS], of[C::KSTEPS];
#pragma unroll
  for (int t = 0; t < C::KSTEPS; ++t) {
    const int d0 = 16 * t + 8 * g;
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    f32x4 cs01 = {1.f, 0.f, 1.f, 0.f}, cs23 = {1.f, 0.f, 1.f, 0.f};
    if (qok) {
      x = global_load_b128(a.q + base + (size_t)qrow * ts + d0);
      y = global_load_b128(a.dout + base + (size_t)qrow * ts + d0);
      const f32x4* rp = (const f32x4*)(a.rope + (size_t)qrow * (D / 2) + d0 / 2);
      cs01 = rp[0];
      cs23 = rp[1];
    }
    qf[t] = __builtin_bit_cast(bf16x8, rope_chunk_scaled(x, cs01, cs23, c));
    of[t] = __builtin_bit_cast(bf16x8, y);
  }
  const size_t row_bh = ((size_t)b * H + h) * N;
  const float lse2 = qok ? a.lse[row_bh + qrow] * 1.4426950408889634f : 0.f;
  const float dr = qok ? a.dr[row_bh + qrow] : 0.f;

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = (f32x16){};

  const int n_tiles = (N + C::T - 1) / C::T;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int k0 = kt * C::T;
    __syncthreads();
    // stage K~ (rotated) and V rows of the tile; rows past N are zero
#pragma unroll
    for (int i = 0; i < C::CH; ++i) {
      const int ch = tid + i * C::NT, r = ch / C::CPR, cc = ch % C::CPR;
      u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
      f32x4 cs01 = {1.f, 0.f, 1.f, 0.f}, cs23 = {1.f, 0.f, 1.f, 0.f};
      if (k0 + r < N) {
        x = global_load_b128(a.k + base + (size_t)(k0 + r) * ts + 8 * cc);
        y = global_load_b128(a.v + base + (size_t)(k0 + r) * ts + 8 * cc);
        const f32x4* rp = (const f32x4*)(a.rope + (size_t)(k0 + r) * (D / 2) + 4 * cc);
        cs01 = rp[0];
        cs23 = rp[1];
      }
      lds_write_b128((FLUX_LDS char*)ksm + r * C::ROWB + 16 * cc, rope_chunk(x, cs01, cs23));
      lds_write_b128((FLUX_LDS char*)vsm + r * C::ROWB + 16 * cc, y);
    }
    __syncthreads();
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm;
    const FLUX_LDS char* vl = (const FLUX_LDS char*)vsm;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int krow = 32 * kb + krow_perm(l32);
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int t = 0; t < C::KSTEPS; ++t) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, lds_read_b128(kl + krow * C::ROWB + 16 * (2 * t + g)));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, lds_read_b128(vl + krow * C::ROWB + 16 * (2 * t + g)));
        s = mfma_bf16(kf, qf[t], s);
        dp = mfma_bf16(vf, of[t], dp);
      }
      // dS^T (keys x this lane's query), bf16, as the B operand of the next MFMA
      u32x4 dsf[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ds2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 8 * hh + 2 * i + u;
            const int key = k0 + 32 * kb + 16 * (e >> 3) + 8 * g + (e & 7);
            const float p = (key < N && qok) ? __builtin_amdgcn_exp2f(s[e] - lse2) : 0.f;
            ds2[u] = p * (dp[e] - dr);
          }
          dsf[hh][i] = pack_bf16(ds2[0], ds2[1]);
        }
      // dQ~^T += K~^T dS^T
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int krow0 = 32 * kb + 16 * hh + 8 * (grp >> 1) + (li >> 2);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int d = 32 * db + 16 * (grp & 1) + 4 * (li & 3);
          const u32x2 lo = lds_read_tr16(kl + krow0 * C::ROWB + 2 * d);
          const u32x2 hi = lds_read_tr16(kl + (krow0 + 4) * C::ROWB + 2 * d);
          const u32x4 kk = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = mfma_bf16(__builtin_bit_cast(bf16x8, kk), __builtin_bit_cast(bf16x8, dsf[hh]), acc[db]);
        }
      }
    }
  }

  // epilogue: dq = R^T (scale dQ~), bf16
  if (qok) {
    uint16_t* orow = a.dq + base + (size_t)qrow * ts;
    const float2* rp = a.rope + (size_t)qrow * (D / 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int d = 32 * db + 8 * aa + 4 * g;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * aa + e] * a.scale;
        rot_back(x[0], x[1], rp[d / 2]);
        rot_back(x[2], x[3], rp[d / 2 + 1]);
        u32x2 w;
        w[0] = pack_bf16(x[0], x[1]);
        w[1] = pack_bf16(x[2], x[3]);
        *(u32x2*)(orow + d) = w;
      }
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char qsm[C::TILEB];  // Q~ tile (rotated)
  __shared__ __attribute__((aligned(16))) char osm[C::TILEB];  // dO tile
  __shared__ float lse_s[C::T], dr_s[C::T];
  const int N = a.n_tokens, H = a.heads;
  const int k_tiles = (N + C::ROWS - 1) / C::ROWS;
  const int kt = blockIdx.x % k_tiles, bh = blockIdx.x / k_tiles;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const size_t ts = (size_t)H * D;
  const size_t base = (size_t)b * N * ts + (size_t)h * D;
  const size_t row_bh = ((size_t)b * H + h) * N;
  const float c = a.c;

  // keys of this lane: c R(k) and V as B fragments
  const int krow = kt * C::ROWS + wave * 32 + l32;
  const bool kok = krow < N;
  bf16x8 kf[C::KSTEPS], vf[C::KSTEPS];
#pragma unroll
  for (int t = 0; t < C::KSTEPS; ++t) {
    const int d0 = 16 * t + 8 * g;
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    f32x4 cs01 = {1.f, 0.f, 1.f, 0.f}, cs23 = {1.f, 0.f, 1.f, 0.f};
    if (kok) {
      x = global_load_b128(a.k + base + (size_t)krow * ts + d0);
      y = global_load_b128(a.v + base + (size_t)krow * ts + d0);
      const f32x4* rp = (const f32x4*)(a.rope + (size_t)krow * (D / 2) + d0 / 2);
      cs01 = rp[0];
      cs23 = rp[1];
    }
    kf[t] = __builtin_bit_cast(bf16x8, rope_chunk_scaled(x, cs01, cs23, c));
    vf[t] = __builtin_bit_cast(bf16x8, y);
  }

  f32x16 dv[C::DB], dk[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dv[db] = (f32x16){};
    dk[db] = (f32x16){};
  }

  const int n_q = (N + C::T - 1) / C::T;
  for (int qt = 0; qt < n_q; ++qt) {
    const int q0 = qt * C::T;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::CH; ++i) {
      const int ch = tid + i * C::NT, r = ch / C::CPR, cc = ch % C::CPR;
      u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
      f32x4 cs01 = {1.f, 0.f, 1.f, 0.f}, cs23 = {1.f, 0.f, 1.f, 0.f};
      if (q0 + r < N) {
        x = global_load_b128(a.q + base + (size_t)(q0 + r) * ts + 8 * cc);
        y = global_load_b128(a.dout + base + (size_t)(q0 + r) * ts + 8 * cc);
        const f32x4* rp = (const f32x4*)(a.rope + (size_t)(q0 + r) * (D / 2) + 4 * cc);
        cs01 = rp[0];
        cs23 = rp[1];
      }
      lds_write_b128((FLUX_LDS char*)qsm + r * C::ROWB + 16 * cc, rope_chunk(x, cs01, cs23));
      lds_write_b128((FLUX_LDS char*)osm + r * C::ROWB + 16 * cc, y);
    }
    if (tid < C::T) {
      const bool ok = q0 + tid < N;
      lse_s[tid] = ok ? a.lse[row_bh + q0 + tid] * 1.4426950408889634f : INFINITY;  // past N: p = 0
      dr_s[tid] = ok ? a.dr[row_bh + q0 + tid] : 0.f;
    }
    __syncthreads();
    const FLUX_LDS char* ql = (const FLUX_LDS char*)qsm;
    const FLUX_LDS char* ol = (const FLUX_LDS char*)osm;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qr = 32 * qb + krow_perm(l32);
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int t = 0; t < C::KSTEPS; ++t) {
        const bf16x8 qfr = __builtin_bit_cast(bf16x8, lds_read_b128(ql + qr * C::ROWB + 16 * (2 * t + g)));
        const bf16x8 ofr = __builtin_bit_cast(bf16x8, lds_read_b128(ol + qr * C::ROWB + 16 * (2 * t + g)));
        s = mfma_bf16(qfr, kf[t], s);
        dp = mfma_bf16(ofr, vf[t], dp);
      }
      // element e: query 32qb + 16(e/8) + 8g + e%8 of the tile, this lane's key
      u32x4 pf[2], dsf[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p2[2], ds2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 8 * hh + 2 * i + u;
            const int ql_ = 32 * qb + 16 * (e >> 3) + 8 * g + (e & 7);
            const float p = __builtin_amdgcn_exp2f(s[e] - lse_s[ql_]);
            p2[u] = p;
            ds2[u] = p * (dp[e] - dr_s[ql_]);
          }
          pf[hh][i] = pack_bf16(p2[0], p2[1]);
          dsf[hh][i] = pack_bf16(ds2[0], ds2[1]);
        }
      // dV^T += dO^T P,  dK~^T += Q~^T dS
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r0 = 32 * qb + 16 * hh + 8 * (grp >> 1) + (li >> 2);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int d = 32 * db + 16 * (grp & 1) + 4 * (li & 3);
          const u32x2 olo = lds_read_tr16(ol + r0 * C::ROWB + 2 * d);
          const u32x2 ohi = lds_read_tr16(ol + (r0 + 4) * C::ROWB + 2 * d);
          const u32x2 qlo = lds_read_tr16(ql + r0 * C::ROWB + 2 * d);
          const u32x2 qhi = lds_read_tr16(ql + (r0 + 4) * C::ROWB + 2 * d);
          const u32x4 oo = {olo[0], olo[1], ohi[0], ohi[1]};
          const u32x4 qq = {qlo[0], qlo[1], qhi[0], qhi[1]};
          dv[db] = mfma_bf16(__builtin_bit_cast(bf16x8, oo), __builtin_bit_cast(bf16x8, pf[hh]), dv[db]);
          dk[db] = mfma_bf16(__builtin_bit_cast(bf16x8, qq), __builtin_bit_cast(bf16x8, dsf[hh]), dk[db]);
        }
      }
    }
  }

  // epilogue: dk = R^T (scale dK~), dv, bf16
  if (kok) {
    uint16_t* krow_k = a.dk + base + (size_t)krow * ts;
    uint16_t* krow_v = a.dv + base + (size_t)krow * ts;
    const float2* rp = a.rope + (size_t)krow * (D / 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int d = 32 * db + 8 * aa + 4 * g;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dk[db][4 * aa + e] * a.scale;
        rot_back(x[0], x[1], rp[d / 2]);
        rot_back(x[2], x[3], rp[d / 2 + 1]);
        u32x2 w, wv;
        w[0] = pack_bf16(x[0], x[1]);
        w[1] = pack_bf16(x[2], x[3]);
        wv[0] = pack_bf16(dv[db][4 * aa + 0], dv[db][4 * aa + 1]);
        wv[1] = pack_bf16(dv[db][4 * aa + 2], dv[db][4 * aa + 3]);
        *(u32x2*)(krow_k + d) = w;
        *(u32x2*)(krow_v + d) = wv;
      }
  }
}

hipError_t launch_attn_bwd(const BwdArgs& a, int head_dim, hipStream_t stream) {
  const int total = a.batch * a.n_tokens * a.heads;
  const int tiles = a.batch * a.heads * ((a.n_tokens + 127) / 128);
  if (head_dim == 128) {
    hipLaunchKernelGGL(attn_bwd_prep_kernel<128>, dim3((total + 255) / 256), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, dim3(tiles), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, dim3(tiles), dim3(256), 0, stream, a);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(attn_bwd_prep_kernel<64>, dim3((total + 255) / 256), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, dim3(tiles), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, dim3(tiles), dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace flux
