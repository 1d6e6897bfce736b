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
// Two launches, no atomics:
//   attn_bwd_prep_kernel - one pass over the rows: Dr, and bf16 Q~ = R(q),
//                          K~ = R(k) into workspace, so that the tiles the
//                          streaming workgroups read (each is read once per
//                          128-row workgroup of the head) need no rotation.
//   attn_bwd_kernel      - all three gradients, one workgroup kind per index
//                          range:
//     bwd_dkv<true>  (dK)  key-stationary: S, dP, dS, dK~^T += Q~^T dS;
//     bwd_dq             query-stationary: a wave holds 32 queries (c Q~ and
//                          dO as B operands); per 64-key tile it forms
//                          S^T = K~ Q~^T and dP^T = V dO^T (lane = query),
//                          then dS^T and dQ~^T += K~^T dS^T (K~ through the
//                          transpose read);
//     bwd_dkv<false> (dV)  key-stationary: S, P, dV^T += dO^T P.
//   dK and dV are separate workgroups: that recomputes S once more (8 instead
//   of 7 N x N x D products in all) but lets each run two waves per SIMD; a
//   fused body needs both 32-key accumulators and both stationary operands in
//   registers, more than half the register file.
// The streaming workgroups: 4 waves per workgroup (32 rows each, 128 rows), two
// workgroups per CU; the 32x32x16 bf16 MFMA with fp32 accumulation; 64-row
// tiles stream from global memory straight into double-buffered LDS (buffer
// loads with the LDS destination, issued one tile ahead, one barrier per
// tile); the stationary operands are rotated from q, k in registers and the
// gradients rotated back (R^T) in the epilogue; workgroups of one head are
// kept on one XCD so that its L2 serves the streamed tiles.
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
  static constexpr int ROWB = 2 * D;       // LDS bytes per staged row (unpadded)
  static constexpr int TILEB = T * ROWB;
  static constexpr int CH = T * CPR / NT;  // chunks per thread per staged tile
};

// Staged tiles are read both one row per lane (b128: a 16-lane phase reads 16
// rows at one chunk) and transposed (ds_read_b64_tr_b16: a 32-lane phase reads
// 4 consecutive rows x 64 bytes).  Chunk c of row r sits at chunk
// c ^ swz(r) of the row; swz makes both patterns, and the 16-lane row writes,
// touch every bank once.
template <int D> __device__ __forceinline__ int swz(int r);
template <> __device__ __forceinline__ int swz<128>(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// 128-byte rows: two rows per bank cycle, so bit 0 of the row already picks
// the half; bits 1..3 pick the chunk within it.
template <> __device__ __forceinline__ int swz<64>(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// R^T on a pair (rotation by the negative angle), table entry w.
__device__ __forceinline__ void rot_back(float& x0, float& x1, uint32_t w) {
  float a, b;
  rot_pair_back(x0, x1, w, a, b);
  x0 = a;
  x1 = b;
}

__device__ __forceinline__ f32x4 lds_read_f32x4(const FLUX_LDS float* p) {
  return *(const FLUX_LDS f32x4*)p;
}

// Per-lane LDS offsets of the two read patterns of a staged tile (relative to
// the tile and to the 32-row block; the block adds 32 * ROWB).
template <int D>
struct TileOffsets {
  using C = BwdCfg<D>;
  int row[C::KSTEPS];  // b128: row krow_perm(l32), chunk 2t + g
  int tr[C::DB][2];    // transposed: rows 8(grp/2) + li/4 (+4), bytes 64 db + 32 (grp&1) + 8 (li&3)
  __device__ __forceinline__ TileOffsets(int lane) {
    const int g = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
    const int r = krow_perm(l32), sw = swz<D>(r);
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) row[t] = r * C::ROWB + 16 * ((2 * t + g) ^ sw);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int rr = 8 * (grp >> 1) + (li >> 2) + 4 * hi, sr = swz<D>(rr);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int cc = 4 * db + 2 * (grp & 1) + ((li & 3) >> 1);
        tr[db][hi] = rr * C::ROWB + 16 * (cc ^ sr) + 8 * (li & 1);
      }
    }
  }
};

// One streamed 64-row tile of one tensor, loaded straight into LDS
// (buffer_load ... lds): each wave instruction fills 1 KB of LDS linearly
// (16 bytes per lane at M0 + 16 lane), so the swizzle is applied to the
// global side: the lane that fills LDS chunk pc of tile row r fetches
// logical chunk pc ^ swz(r) of that row.
template <int D>
struct TileDma {
  using C = BwdCfg<D>;
  static constexpr int NI = C::TILEB / (C::NT * 16);  // instructions per tile
  uint32_t voff[NI];
  int wave_off;
  __device__ __forceinline__ TileDma(int tid, uint32_t row_bytes) {
    const int w = tid >> 6, l = tid & 63;
    wave_off = __builtin_amdgcn_readfirstlane(w * 1024);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int p = i * C::NT * 16 + w * 1024 + 16 * l;
      const int r = p / C::ROWB, pc = (p % C::ROWB) / 16;
      voff[i] = (uint32_t)r * row_bytes + 16u * (uint32_t)(pc ^ swz<D>(r));
    }
  }
  // rows from byte offset soff of the resource into the tile at lds
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t res, FLUX_LDS char* lds, uint32_t soff) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (FLUX_LDS void*)(lds + i * C::NT * 16 + wave_off), 16, voff[i],
                                              soff, 0, 0);
  }
};

// Wait for this wave's outstanding vector-memory loads (incl. LDS DMA).
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

enum BwdKind { KIND_DK = 0, KIND_DV = 1, KIND_DQ = 2 };

// One 64-row streamed tile against one wave's 32 stationary rows (lane =
// stationary row), in two 32-row halves u.  Per half:
//   S = A(ra) st0 and, except for dV, dP = A(rb) st1 (A: streamed rows from
//   LDS, st: stationary B fragments; c is already in st0), element e of lane l
//   holding streamed row 32 u + 16 (e / 8) + 8 (l / 32) + e % 8 of the tile;
//   p = exp2(S - lse log2 e);  B = p (dV) or p (dP - Dr) (dK, dq), bf16;
//   acc[db] += A(ta)^T B, A(ta) through the transpose read.
// lse and Dr come per streamed row from LDS (dK, dV) or per lane (dq).  MASK
// (dq): streamed rows at or past lim get p = 0.  LDS operands are read NPF
// MFMAs ahead; the first reads of each phase are issued in the one before.
template <int D, int KIND, bool MASK>
__device__ __forceinline__ void tile_pass(const FLUX_LDS char* ra, const FLUX_LDS char* rb, const FLUX_LDS char* ta,
                                          const FLUX_LDS float* lse_t, const FLUX_LDS float* dr_t, float lse_l,
                                          float dr_l, int lim, const bf16x8* st0, const bf16x8* st1,
                                          const TileOffsets<D>& off, int g, f32x16* acc) {
  using C = BwdCfg<D>;
  constexpr bool TWO = KIND != KIND_DV;  // dP needed
  constexpr bool ROWSTATS = KIND != KIND_DQ;
  constexpr int NPF = 2;
  constexpr int OSTEPS = 2 * C::DB;      // output MFMAs per half: (hh, db)
  constexpr float L2E = 1.4426950408889634f;
  auto rrow = [&](const FLUX_LDS char* t, int u, int k) {
    return __builtin_bit_cast(bf16x8, lds_read_b128(t + 32 * u * C::ROWB + off.row[k]));
  };
  auto rtr = [&](int u, int j) {
    const int hh = j / C::DB, db = j % C::DB;
    const FLUX_LDS char* p = ta + (32 * u + 16 * hh) * C::ROWB;
    const u32x2 lo = lds_read_tr16(p + off.tr[db][0]);
    const u32x2 hi = lds_read_tr16(p + off.tr[db][1]);
    return __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
  };
  bf16x8 pa[NPF], pb[NPF], pt[NPF];
  static_for<0, NPF>([&](auto K) {
    pa[K] = rrow(ra, 0, K);
    if constexpr (TWO) pb[K] = rrow(rb, 0, K);
  });
  static_for<0, 2>([&](auto U) {
    constexpr int u = decltype(U)::value;
    f32x16 s = {}, dp = {};
    f32x4 ls[4], ds[4];  // lse, Dr of rows 32 u + 16 hh + 8 g + 4 q + 0..3 at [2 hh + q]
    static_for<0, C::KSTEPS>([&](auto K) {
      constexpr int k = decltype(K)::value;
      s = mfma_bf16(pa[k % NPF], st0[k], s);
      if constexpr (TWO) dp = mfma_bf16(pb[k % NPF], st1[k], dp);
      if constexpr (k + NPF < C::KSTEPS) {
        pa[k % NPF] = rrow(ra, u, k + NPF);
        if constexpr (TWO) pb[k % NPF] = rrow(rb, u, k + NPF);
      } else {
        constexpr int j = k + NPF - C::KSTEPS;
        pt[j] = rtr(u, j);
        if constexpr (ROWSTATS && j == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) ls[q] = lds_read_f32x4(lse_t + 32 * u + 16 * (q >> 1) + 8 * g + 4 * (q & 1));
        }
        if constexpr (KIND == KIND_DK && j == NPF - 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) ds[q] = lds_read_f32x4(dr_t + 32 * u + 16 * (q >> 1) + 8 * g + 4 * (q & 1));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    u32x4 bfr[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v2[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int e = 8 * hh + 2 * i + w, r8 = 2 * i + w;  // row 32 u + 16 hh + 8 g + r8
          const float lse = ROWSTATS ? ls[2 * hh + (r8 >> 2)][r8 & 3] : lse_l;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(lse, -L2E, s[e]));
          if constexpr (MASK) p = 32 * u + 16 * hh + 8 * g + r8 < lim ? p : 0.f;
          if constexpr (KIND == KIND_DV)
            v2[w] = p;
          else
            v2[w] = p * (dp[e] - (ROWSTATS ? ds[2 * hh + (r8 >> 2)][r8 & 3] : dr_l));
        }
        bfr[hh][i] = pack_bf16(v2[0], v2[1]);
      }
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, OSTEPS>([&](auto J) {
      constexpr int j = decltype(J)::value;
      acc[j % C::DB] = mfma_bf16(pt[j % NPF], __builtin_bit_cast(bf16x8, bfr[j / C::DB]), acc[j % C::DB]);
      if constexpr (j + NPF < OSTEPS) {
        pt[j % NPF] = rtr(u, j + NPF);
      } else if constexpr (u == 0) {
        constexpr int k = j + NPF - OSTEPS;  // first row operands of the second half
        pa[k] = rrow(ra, 1, k);
        if constexpr (TWO) pb[k] = rrow(rb, 1, k);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

}  // namespace

// Per row (b, i, h): Dr = sum_d dO * O (fp32), bf16 R(q) and R(k).  One thread
// per 16-byte chunk; the D/8 threads of a row reduce Dr by shuffles.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = gid / CPR, cc = gid % CPR;  // row = (b N + i) H + h
  const int total = a.batch * a.n_tokens * a.heads;
  const bool ok = row < total;  // whole rows are in or out: CPR divides the block
  float s = 0.f;
  int i = 0, h = 0, b = 0;
  if (ok) {
    h = row % a.heads;
    i = (row / a.heads) % a.n_tokens;
    b = row / (a.heads * a.n_tokens);
    const size_t off = (size_t)row * D + 8 * cc;
    const u32x4 cs = *(const u32x4*)(a.rope + (size_t)i * (D / 2) + 4 * cc);
    *(u32x4*)(a.qr + off) = rope_chunk(global_load_b128(a.q + off), cs);
    *(u32x4*)(a.kr + off) = rope_chunk(global_load_b128(a.k + off), cs);
    const u32x4 x = global_load_b128(a.dout + off);
    const u32x4 y = global_load_b128(a.out + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf16lo(x[e]) * bf16lo(y[e]) + bf16hi(x[e]) * bf16hi(y[e]);
  }
#pragma unroll
  for (int m = CPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, CPR);
  if (ok && cc == 0) a.dr[((size_t)b * a.heads + h) * a.n_tokens + i] = s;
}

// dq of the 128 queries of workgroup tile blk; smem holds the K~ and V tile
// buffers (4 x 64 rows).
template <int D>
__device__ __forceinline__ void bwd_dq(const BwdArgs& a, int blk, FLUX_LDS char* sm0, FLUX_LDS char* sm1) {
  using C = BwdCfg<D>;
  // buffer b: K~ tile (rotated) at smb, V tile at smb + TILEB
  const int N = a.n_tokens, H = a.heads;
  const int q_tiles = (N + C::ROWS - 1) / C::ROWS;
  const int qt = blk % q_tiles, bh = blk / q_tiles;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t ts = (size_t)H * D;                          // elements between tokens
  const size_t base = (size_t)b * N * ts + (size_t)h * D;
  const float c = a.c;

  // K~ and V tiles stream straight from global memory into LDS; rows past N
  // read as zero through the buffer range check
  const uint32_t bytes = (uint32_t)(((size_t)(N - 1) * ts + D) * 2);
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(a.kr + base, bytes);
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(a.v + base, bytes);
  const TileDma<D> dma(tid, (uint32_t)(ts * 2));
  const uint32_t tile_bytes = (uint32_t)(C::T * ts * 2);
  dma.issue(kres, sm0, 0);
  dma.issue(vres, sm0 + C::TILEB, 0);

  // queries of this lane: c R(q) and dO as B fragments; lse2 and Dr.  Rows
  // past N carry zeros (finite p and dS; never stored).
  const int qrow = qt * C::ROWS + wave * 32 + l32;
  const bool qok = qrow < N;
  bf16x8 qf[C::KSTEPS], of[C::KSTEPS];
#pragma unroll
  for (int t = 0; t < C::KSTEPS; ++t) {
    const int d0 = 16 * t + 8 * g;
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    u32x4 cs = {0, 0, 0, 0};  // rows past N: zeros rotate to zeros
    if (qok) {
      x = global_load_b128(a.q + base + (size_t)qrow * ts + d0);
      y = global_load_b128(a.dout + base + (size_t)qrow * ts + d0);
      cs = *(const u32x4*)(a.rope + (size_t)qrow * (D / 2) + d0 / 2);
    }
    qf[t] = __builtin_bit_cast(bf16x8, rope_chunk_scaled(x, cs, c));
    of[t] = __builtin_bit_cast(bf16x8, y);
  }
  const size_t row_bh = ((size_t)b * H + h) * N;
  const float lse = qok ? a.lse[row_bh + qrow] : 0.f;
  const float dr = qok ? a.dr[row_bh + qrow] : 0.f;
  const TileOffsets<D> off(lane);

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = (f32x16){};

  // one 64-key tile from LDS buffer BUF; MASK: the tile holds keys >= N
  auto tile = [&](auto BUF, auto MASK, int k0) {
    const FLUX_LDS char* kl = decltype(BUF)::value ? sm1 : sm0;
    const FLUX_LDS char* vl = kl + C::TILEB;
    tile_pass<D, KIND_DQ, decltype(MASK)::value>(kl, vl, kl, nullptr, nullptr, lse, dr, N - k0, qf, of, off, g, acc);
  };

  // Tiles alternate between the two LDS buffers; the next tile's loads are
  // issued before the current tile's MFMAs and waited for at the barrier
  // that ends it.  Pairs of full tiles run in the loop, so the accumulators
  // stay in place; the last one or two tiles (one of them partial) follow.
  const int n_tiles = (N + C::T - 1) / C::T;
  const int n_full = N / C::T;  // tiles without keys past N
  FLUX_LDS char* const k0s = sm0;
  FLUX_LDS char* const k1s = sm1;
  FLUX_LDS char* const v0s = sm0 + C::TILEB;
  FLUX_LDS char* const v1s = sm1 + C::TILEB;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  dma_wait();
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= n_full; kt += 2) {
    dma.issue(kres, k1s, (uint32_t)(kt + 1) * tile_bytes);
    dma.issue(vres, v1s, (uint32_t)(kt + 1) * tile_bytes);
    tile(B0{}, std::false_type{}, kt * C::T);
    dma_wait();
    __syncthreads();
    if (kt + 2 < n_tiles) {
      dma.issue(kres, k0s, (uint32_t)(kt + 2) * tile_bytes);
      dma.issue(vres, v0s, (uint32_t)(kt + 2) * tile_bytes);
    }
    tile(B1{}, std::false_type{}, (kt + 1) * C::T);
    dma_wait();
    __syncthreads();
  }
  if (kt < n_full) {  // one full tile left (buffer 0), maybe a partial one after it
    if (kt + 1 < n_tiles) {
      dma.issue(kres, k1s, (uint32_t)(kt + 1) * tile_bytes);
      dma.issue(vres, v1s, (uint32_t)(kt + 1) * tile_bytes);
    }
    tile(B0{}, std::false_type{}, kt * C::T);
    dma_wait();
    __syncthreads();
    if (kt + 1 < n_tiles) tile(B1{}, std::true_type{}, (kt + 1) * C::T);
  } else if (kt < n_tiles) {  // the partial tile (buffer 0)
    tile(B0{}, std::true_type{}, kt * C::T);
  }

  // epilogue: dq = R^T (scale dQ~), bf16
  if (qok) {
    uint16_t* orow = a.dq + base + (size_t)qrow * ts;
    const uint32_t* rp = a.rope + (size_t)qrow * (D / 2);
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

// Key-stationary gradients, one kernel per tensor (DK: dK, else dV).  A wave
// holds 32 keys as B operands (c K~, and V for dK); per 64-query tile it forms
// S = Q~ K~^T (and dP = dO V^T for dK) with lane = key, then
//   dV^T += dO^T P           (dO through the transpose read), or
//   dK~^T += Q~^T dS         (Q~ through the transpose read).
// Queries past N stream in as zero rows with lse = Dr = 0: p = 1, dS = 0, and
// their dO and Q~ rows are zero, so they add nothing.  Keys past N only touch
// their own (unstored) accumulator columns.
template <int D, bool DK>
__device__ __forceinline__ void bwd_dkv(const BwdArgs& a, int blk, FLUX_LDS char* sm0, FLUX_LDS char* sm1) {
  using C = BwdCfg<D>;
  // buffer b: Q~ tile (rotated) at smb, dO tile at + TILEB, natural-log lse of
  // the tile's queries at + 2 TILEB, their Dr (dK) after that
  const int N = a.n_tokens, H = a.heads;
  const int k_tiles = (N + C::ROWS - 1) / C::ROWS;
  const int kt = blk % k_tiles, bh = blk / k_tiles;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t ts = (size_t)H * D;
  const size_t base = (size_t)b * N * ts + (size_t)h * D;
  const size_t row_bh = ((size_t)b * H + h) * N;
  const float c = a.c;

  const uint32_t bytes = (uint32_t)(((size_t)(N - 1) * ts + D) * 2);
  const __amdgpu_buffer_rsrc_t qres = make_rsrc(a.qr + base, bytes);
  const __amdgpu_buffer_rsrc_t ores = make_rsrc(a.dout + base, bytes);
  const __amdgpu_buffer_rsrc_t lres = make_rsrc(a.lse + row_bh, (uint32_t)N * 4);
  const __amdgpu_buffer_rsrc_t dres = make_rsrc(a.dr + row_bh, (uint32_t)N * 4);
  const TileDma<D> dma(tid, (uint32_t)(ts * 2));
  const uint32_t tile_bytes = (uint32_t)(C::T * ts * 2);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  FLUX_LDS char* const qs[2] = {sm0, sm1};
  FLUX_LDS char* const os[2] = {sm0 + C::TILEB, sm1 + C::TILEB};
  FLUX_LDS float* const ls[2] = {(FLUX_LDS float*)(sm0 + 2 * C::TILEB), (FLUX_LDS float*)(sm1 + 2 * C::TILEB)};
  FLUX_LDS float* const dss[2] = {ls[0] + C::T, ls[1] + C::T};
  // tile qt into buffer bf: Q~ and dO rows, lse (wave 0) and Dr (wave 1, dK)
  auto issue = [&](int bf, int qt) {
    dma.issue(qres, qs[bf], (uint32_t)qt * tile_bytes);
    dma.issue(ores, os[bf], (uint32_t)qt * tile_bytes);
    if (wv == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lres, (FLUX_LDS void*)ls[bf], 4, 4u * lane, (uint32_t)qt * C::T * 4, 0, 0);
    if (DK && wv == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(dres, (FLUX_LDS void*)dss[bf], 4, 4u * lane, (uint32_t)qt * C::T * 4, 0,
                                              0);
  };
  issue(0, 0);

  // keys of this lane: c R(k) (and V) as B fragments
  const int krow = kt * C::ROWS + wave * 32 + l32;
  const bool kok = krow < N;
  bf16x8 kf[C::KSTEPS], vf[DK ? C::KSTEPS : 1];
#pragma unroll
  for (int t = 0; t < C::KSTEPS; ++t) {
    const int d0 = 16 * t + 8 * g;
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    u32x4 cs = {0, 0, 0, 0};  // rows past N: zeros rotate to zeros
    if (kok) {
      x = global_load_b128(a.k + base + (size_t)krow * ts + d0);
      if constexpr (DK) y = global_load_b128(a.v + base + (size_t)krow * ts + d0);
      cs = *(const u32x4*)(a.rope + (size_t)krow * (D / 2) + d0 / 2);
    }
    kf[t] = __builtin_bit_cast(bf16x8, rope_chunk_scaled(x, cs, c));
    if constexpr (DK) vf[t] = __builtin_bit_cast(bf16x8, y);
  }
  const TileOffsets<D> off(lane);

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = (f32x16){};

  auto tile = [&](auto BUF) {
    constexpr int bf = decltype(BUF)::value;
    tile_pass<D, DK ? KIND_DK : KIND_DV, false>(qs[bf], os[bf], DK ? qs[bf] : os[bf], ls[bf], dss[bf], 0.f, 0.f, 0,
                                                kf, vf, off, g, acc);
  };

  // double-buffered query tiles, as in the dq kernel (no partial-tile case:
  // rows past N are zeros that add nothing)
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const int n_q = (N + C::T - 1) / C::T;
  dma_wait();
  __syncthreads();
  int qt = 0;
  for (; qt + 2 <= n_q; qt += 2) {
    issue(1, qt + 1);
    tile(B0{});
    dma_wait();
    __syncthreads();
    if (qt + 2 < n_q) issue(0, qt + 2);
    tile(B1{});
    dma_wait();
    __syncthreads();
  }
  if (qt < n_q) tile(B0{});

  // epilogue: dk = R^T (scale dK~) or dv, bf16
  if (kok) {
    uint16_t* orow = (DK ? a.dk : a.dv) + base + (size_t)krow * ts;
    const uint32_t* rp = a.rope + (size_t)krow * (D / 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int d = 32 * db + 8 * aa + 4 * g;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * aa + e];
        if constexpr (DK) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] *= a.scale;
          rot_back(x[0], x[1], rp[d / 2]);
          rot_back(x[2], x[3], rp[d / 2 + 1]);
        }
        u32x2 w;
        w[0] = pack_bf16(x[0], x[1]);
        w[1] = pack_bf16(x[2], x[3]);
        *(u32x2*)(orow + d) = w;
      }
  }
}

// All three gradients in one launch: workgroups [0, G) compute dK, [G, 2G)
// dq and [2G, 3G) dV for the G = B H ceil(N / 128) row tiles.  The dispatcher
// hands out workgroups in index order, so the shorter dV workgroups (two of
// the products instead of three) fill the last round instead of leaving
// each gradient's partial last round idle.  One LDS block serves whichever
// body runs.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  // the two tile buffers are separate LDS objects, so that reads of one are
  // known not to alias the loads in flight into the other
  __shared__ __attribute__((aligned(16))) char smem0[2 * C::TILEB + 2 * C::T * (int)sizeof(float)];
  __shared__ __attribute__((aligned(16))) char smem1[2 * C::TILEB + 2 * C::T * (int)sizeof(float)];
  FLUX_LDS char* const s0 = (FLUX_LDS char*)smem0;
  FLUX_LDS char* const s1 = (FLUX_LDS char*)smem1;
  const int G = gridDim.x / 3;
  const int seg = blockIdx.x / G, i = blockIdx.x - seg * G;
  const int blk = xcd_tile_order(i, G);
  if (seg == 0)
    bwd_dkv<D, true>(a, blk, s0, s1);
  else if (seg == 1)
    bwd_dq<D>(a, blk, s0, s1);
  else
    bwd_dkv<D, false>(a, blk, s0, s1);
}

// Explicit instantiations: without them hipcc does not always emit the host
// launch stubs of kernels launched from the template below.
template __global__ void attn_bwd_prep_kernel<128>(BwdArgs);
template __global__ void attn_bwd_prep_kernel<64>(BwdArgs);
template __global__ void attn_bwd_kernel<128>(BwdArgs);
template __global__ void attn_bwd_kernel<64>(BwdArgs);

template <int D>
static void launch_bwd_kernels(const BwdArgs& a, hipStream_t stream) {
  const long long chunks = (long long)a.batch * a.n_tokens * a.heads * (D / 8);
  const int tiles = a.batch * a.heads * ((a.n_tokens + 127) / 128);
  hipLaunchKernelGGL(attn_bwd_prep_kernel<D>, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(attn_bwd_kernel<D>, dim3(3 * tiles), dim3(256), 0, stream, a);
}

hipError_t launch_attn_bwd(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 128)
    launch_bwd_kernels<128>(a, stream);
  else if (head_dim == 64)
    launch_bwd_kernels<64>(a, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace flux
