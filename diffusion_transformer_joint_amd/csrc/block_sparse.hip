// Tile-sparse attention support: the tile masks and the lists of kept key
// tiles.
//
// Sparse attention skips the work for less important token pairs according to
// a sparsity threshold tau ("Optimizing FLUX 3 Image Klein inference on NVIDIA
// Blackwell GPUs", How it works; What you can do: tau).  Granularity and
// importance measure are this library's reading: 256-token query tiles x
// 64-token key tiles, and two rules (c = scale * log2 e, exp2 domain):
//   score bound (tile_bound_kernel): key tile t is skipped for query tile Q
//     when, for every query i of Q, i's largest score over t is below
//     L_i + log2(tau), with L_i i's largest score over the 4 key tiles aligned
//     with Q (a lower bound of its row maximum); every skipped pair then has
//     weight below tau times its row's largest, which bounds the distance
//     from dense attention;
//   pooled score (tile_mean_kernel, block_select_kernel), an alternative
//     without that guarantee: the pooled score of a tile pair is
//     c * <mean of the tile's rotated q, mean of the tile's rotated k>; a key
//     tile is kept when its pooled score is at least the query tile's largest
//     plus log2(tau).
#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"

namespace flux {

// Mean over the tokens of each tile of the rotated rows of x (bf16
// [B][batch_tokens][H][D]), fp32 out [B][H][T][D].  One workgroup of 256
// threads per (b, h, tile): thread = (rotary pair, token group).
template <int D>
__global__ __launch_bounds__(256) void tile_mean_kernel(const uint16_t* __restrict__ x,
                                                        const float2* __restrict__ rope, float* __restrict__ out,
                                                        int n_tokens, int batch_tokens, int heads, int tile, int T) {
  constexpr int P = D / 2;       // rotary pairs
  constexpr int G = 256 / P;     // token groups
  __shared__ float red[256][2];
  const int t = blockIdx.x % T, bh = blockIdx.x / T;
  const int h = bh % heads, b = bh / heads;
  const int p = threadIdx.x % P, grp = threadIdx.x / P;
  const int r0 = t * tile, r1 = min(r0 + tile, n_tokens);
  float s0 = 0.f, s1 = 0.f;
  for (int r = r0 + grp; r < r1; r += G) {
    const uint32_t w = ((const uint32_t*)(x + (((size_t)b * batch_tokens + r) * heads + h) * D))[p];
    const float2 cs = rope[(size_t)r * P + p];
    const float x0 = bf16lo(w), x1 = bf16hi(w);
    s0 += x0 * cs.x - x1 * cs.y;
    s1 += x0 * cs.y + x1 * cs.x;
  }
  red[threadIdx.x][0] = s0;
  red[threadIdx.x][1] = s1;
  __syncthreads();
  if (grp == 0) {
    for (int k = 1; k < G; ++k) {
      s0 += red[k * P + p][0];
      s1 += red[k * P + p][1];
    }
    const float inv = 1.0f / (float)(r1 - r0);
    float* o = out + (((size_t)b * heads + h) * T + t) * D;
    o[2 * p] = s0 * inv;
    o[2 * p + 1] = s1 * inv;
  }
}

// Mask row of one (b, h, query tile): pooled scores against every key tile,
// their max, and the threshold decision.  256 threads; scores in dynamic LDS.
template <int D>
__global__ __launch_bounds__(256) void block_select_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                           uint8_t* __restrict__ mask, int QT, int KT, float c,
                                                           float log2_tau) {
  extern __shared__ float sc[];  // [KT]
  __shared__ float qv[D];
  __shared__ float wmax[4];
  const int row = blockIdx.x;  // (b*H + h)*QT + qt
  const int bh = row / QT;
  const float* q = qbar + (size_t)row * D;
  const float* kb = kbar + (size_t)bh * KT * D;
  for (int d = threadIdx.x; d < D; d += 256) qv[d] = q[d];
  __syncthreads();
  float mx = -INFINITY;
  for (int kt = threadIdx.x; kt < KT; kt += 256) {
    const float* kr = kb + (size_t)kt * D;
    float s = 0.f;
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(qv[d], kr[d], s);
    s *= c;
    sc[kt] = s;
    mx = fmaxf(mx, s);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float thr = mx + log2_tau;
  for (int kt = threadIdx.x; kt < KT; kt += 256) mask[(size_t)row * KT + kt] = sc[kt] >= thr ? 1 : 0;
}

// Score-bound rule for one (b, h, 256-row query tile) per workgroup: 8 waves
// x 32 queries.  Q and K are rotated, scaled and rounded exactly as in the
// attention kernel (same table, same bf16 operands), the scores are bf16
// MFMA sums in fp32.  The workgroup first walks the 4 key tiles aligned with
// its query tile, each query keeping its largest score L, then every key tile
// t, each wave reducing max over its queries of (tile max - L) into
// red[wave][t]; at the end red's column maxima decide the mask row.  K tiles
// are double-buffered in LDS, one barrier per tile.  Keys past N are masked
// in the one tile that holds them only; the per-query values of 32 tiles
// are collected in LDS (one store per tile) and each lane then reduces one
// tile's 32 values, instead of a shuffle reduction per tile.
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void tile_bound_kernel(BoundArgs a) {
  constexpr int BN = 64, NT = 512, KSTEPS = D / 16, CPR = D / 8, RPP = NT / CPR, NPASS = BN / RPP;
  constexpr int KTILEB = BN * LdsRows<D>::K;
  __shared__ __attribute__((aligned(16))) char ksm[2][KTILEB];
  __shared__ __attribute__((aligned(16))) float vbuf[8][32][32];  // [wave][tile % 32][query]
  extern __shared__ float red[];  // [8][KT]
  const int N = a.n_tokens, H = a.heads, KT = a.kt;
  const int QT = (N + 255) / 256;
  // Work item: a whole query tile, or one piece (a range of key tiles) of a
  // query tile of the last round; the mask bits of a key tile depend only on
  // that tile and the aligned ones, so pieces need no merge.
  int tile, kt_lo = 0, kt_hi = KT;
  if ((int)blockIdx.x < a.whole) {
    tile = xcd_tile_order(blockIdx.x, a.whole);
  } else {
    const int slot = blockIdx.x - a.whole;
    tile = a.whole + slot / a.split;
    const int piece = slot % a.split;
    kt_lo = piece * KT / a.split;
    kt_hi = (piece + 1) * KT / a.split;
  }
  const int qt = tile % QT, bh = tile / QT;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t tok_stride = (size_t)H * D;
  const uint16_t* qbase = a.q + (size_t)b * a.batch_tokens * tok_stride + (size_t)h * D;
  const uint16_t* kbase = a.k + (size_t)b * a.batch_tokens * tok_stride + (size_t)h * D;

  // Q fragments of this lane's query, rotated, times c, bf16 (rows past N: 0)
  const int qrow = qt * 256 + wave * 32 + l32;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    const int ch = 2 * t + g;
    u32x4 x = {0, 0, 0, 0}, w = {0, 0, 0, 0};
    if (qrow < N) {
      x = global_load_b128(qbase + (size_t)qrow * tok_stride + 8 * ch);
      w = global_load_b128(a.rope + (size_t)qrow * (D / 2) + 4 * ch);
    }
    qf[t] = __builtin_bit_cast(bf16x8, rope_chunk_scaled(x, w, a.c));
  }

  // key tile of position p: the 4 aligned tiles first, then kt_lo .. kt_hi - 1
  const int t_al0 = 4 * qt, n_al = min(4, KT - t_al0);
  auto tile_of = [&](int p) { return p < n_al ? t_al0 + p : kt_lo + p - n_al; };
  const int n_rng = kt_hi - kt_lo;
  const int n_pos = n_al + n_rng;
  const int st_chunk = tid % CPR, st_row0 = tid / CPR;
  u32x4 kraw[NPASS], kcs[NPASS];
  auto load_k = [&](int kt0) {
    const int rows = N - kt0;
    const uint32_t kbytes = rows > 0 ? (uint32_t)((rows - 1) * tok_stride * 2 + 2 * D) : 0u;
    const uint32_t rbytes = rows > 0 ? (uint32_t)(rows * (D / 2) * 4) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)kt0 * tok_stride, kbytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.rope + (size_t)kt0 * (D / 2), rbytes);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int r = st_row0 + p * RPP;
      kraw[p] = buffer_load_b128(rk, (uint32_t)(r * tok_stride * 2 + st_chunk * 16));
      kcs[p] = buffer_load_b128(rr, (uint32_t)(r * (D / 2) * 4 + st_chunk * 16));
    }
  };
  auto store_k = [&](int buf) {
    FLUX_LDS char* kl = (FLUX_LDS char*)ksm[buf];
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
      lds_write_b128(kl + k_off<D>(st_row0 + p * RPP, st_chunk), rope_chunk(kraw[p], kcs[p]));
  };
  auto store_rotated = [&](int buf, const u32x4 (&kr)[NPASS]) {
    FLUX_LDS char* kl = (FLUX_LDS char*)ksm[buf];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) lds_write_b128(kl + k_off<D>(st_row0 + p * RPP, st_chunk), kr[p]);
  };

  load_k(tile_of(0) * BN);
  store_k(0);
  if (n_pos > 1) load_k(tile_of(1) * BN);
  __syncthreads();
  float low = -INFINITY;  // L of this lane's query
  // Lane j < n of the wave: the maximum over the wave's 32 queries of the
  // values stored for range tile t0 + j (slot j of vbuf) goes to
  // red[wave][kt_lo + t0 + j].
  auto flush = [&](int t0, int n) {
    if (lane < n) {
      const float* row = &vbuf[wave][lane][0];
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const float4 x = *(const float4*)(row + i);
        m = fmaxf(m, fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)));
      }
      red[wave * KT + kt_lo + t0 + lane] = m;
    }
  };
  for (int p = 0; p < n_pos; ++p) {
    const int t = tile_of(p), kt0 = t * BN;
    const FLUX_LDS char* kl = (const FLUX_LDS char*)ksm[p & 1];
    // the previous 32 tiles' values were stored before the last barrier
    if (p > n_al && ((p - n_al) & 31) == 0) flush(p - n_al - 32, 32);
    // The score MFMAs of this tile in a fixed order, each with the LDS read
    // of the K fragment two MFMAs ahead and, in every other slot, the
    // rotation of one pair of the next K tile (loaded one iteration ahead).
    constexpr int NM = 2 * KSTEPS, NPAIR = NPASS * 4;
    static_assert(2 * NPAIR <= NM, "one rotated pair per two MFMAs");
    auto kfrag = [&](int j) {
      return __builtin_bit_cast(bf16x8, lds_read_b128(kl + k_off<D>(32 * (j / KSTEPS) + l32, 2 * (j % KSTEPS) + g)));
    };
    f32x16 s[2] = {(f32x16){}, (f32x16){}};
    u32x4 kr[NPASS];
    bf16x8 fk[2] = {kfrag(0), kfrag(1)};
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const bf16x8 x = fk[j % 2];
      if constexpr (j + 2 < NM) fk[j % 2] = kfrag(j + 2);
      s[j / KSTEPS] = mfma_bf16(x, qf[j % KSTEPS], s[j / KSTEPS]);
      if constexpr (j % 2 == 0 && j / 2 < NPAIR) {
        constexpr int pi = j / 2;
        kr[pi / 4][pi % 4] = rope_pair(kraw[pi / 4][pi % 4], kcs[pi / 4][pi % 4]);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // The other buffer was last read in the previous tile, before the
    // barrier; after the last tile nothing reads it, so the store is
    // unconditional.
    store_rotated((p + 1) & 1, kr);
    float mx = -INFINITY;
    if (kt0 + BN <= N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    } else {
      // element e of lane l: key 32 kb + 8 (e / 4) + 4 g + e % 4 of the tile
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt0 + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
          mx = fmaxf(mx, key < N ? s[kb][e] : -INFINITY);
        }
    }
    mx = fmaxf(mx, swap_halves(mx));  // this query's largest score over the tile
    if (p < n_al) {
      low = fmaxf(low, mx);
    } else if (g == 0) {
      vbuf[wave][(p - n_al) & 31][l32] = qrow < N ? mx - low : -INFINITY;
    }
    if (p + 2 < n_pos) load_k(tile_of(p + 2) * BN);
    __syncthreads();
  }
  {
    const int done = n_rng & ~31;  // range tiles already reduced into red
    if (done < n_rng) flush(done, n_rng - done);
    else if (n_rng > 0) flush(n_rng - 32, 32);
  }
  __syncthreads();
  uint8_t* mrow = a.mask + (size_t)tile * KT;
  for (int t = kt_lo + tid; t < kt_hi; t += NT) {
    float m = red[t];
#pragma unroll
    for (int w = 1; w < 8; ++w) m = fmaxf(m, red[w * KT + t]);
    mrow[t] = m >= a.log2_tau ? 1 : 0;
  }
}

// Kept key tiles of each mask row, ascending, and their count: one wave per
// row, 64 entries per step, positions from a ballot prefix count.
__global__ __launch_bounds__(256) void mask_to_list_kernel(const uint8_t* __restrict__ mask, int* __restrict__ list,
                                                           int* __restrict__ count, int rows, int KT, int stride) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole waves leave together
  const uint8_t* m = mask + (size_t)row * KT;
  int* l = list + (size_t)row * stride;
  int n = 0;
  for (int k0 = 0; k0 < KT; k0 += 64) {
    const int kt = k0 + lane;
    const bool keep = kt < KT && m[kt] != 0;
    const uint64_t bits = __ballot(keep);
    const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0));
    if (keep) l[n + before] = kt;
    n += __popcll(bits);
  }
  if (lane == 0) count[row] = n;
}

// Dispatch order of a tile-sparse launch: query tiles by kept count,
// longest first (ties by index, so the order and with it the split of the
// last round are deterministic).  One workgroup sorts the keys
// (KT - count) << IB | index with a bitonic network.  Up to 1024 rows each
// thread holds one key in a register: the compare-exchange steps with
// partners inside the wave (distance < 64) use shuffles, only the longer ones
// go through LDS with a barrier; larger row counts sort in LDS throughout.
__global__ __launch_bounds__(1024) void tile_order_kernel(const int* __restrict__ count, int* __restrict__ order,
                                                          int rows, int KT, int P, int IB) {
  extern __shared__ uint32_t key[];  // [max(P, 1024)], P = power of two >= rows
  const int tid = threadIdx.x;
  auto make_key = [&](int i) -> uint32_t {
    return i < rows ? ((uint32_t)(KT - count[i]) << IB) | (uint32_t)i : 0xffffffffu;
  };
  if (P <= 1024) {
    uint32_t x = tid < P ? make_key(tid) : 0xffffffffu;
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        uint32_t y;
        if (j >= 64) {
          key[tid] = x;
          __syncthreads();
          y = key[tid ^ j];
          __syncthreads();
        } else {
          y = (uint32_t)__shfl_xor((int)x, j);
        }
        const bool lower = (tid & j) == 0, up = (tid & k) == 0;
        // the lower element of an ascending pair keeps the smaller key
        x = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
      }
    }
    if (tid < rows) order[tid] = (int)(x & ((1u << IB) - 1u));
    return;
  }
  for (int i = tid; i < P; i += 1024) key[i] = make_key(i);
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t a = key[i], b = key[l];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            key[i] = b;
            key[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < rows; i += 1024) order[i] = (int)(key[i] & ((1u << IB) - 1u));
}

hipError_t launch_tile_means(const uint16_t* x, const float2* rope, float* out, int n_tokens, int batch_tokens,
                             int heads, int batch, int head_dim, int tile, hipStream_t stream) {
  const int T = (n_tokens + tile - 1) / tile;
  const dim3 grid(batch * heads * T);
  if (head_dim == 128)
    hipLaunchKernelGGL(tile_mean_kernel<128>, grid, dim3(256), 0, stream, x, rope, out, n_tokens, batch_tokens,
                       heads, tile, T);
  else if (head_dim == 64)
    hipLaunchKernelGGL(tile_mean_kernel<64>, grid, dim3(256), 0, stream, x, rope, out, n_tokens, batch_tokens,
                       heads, tile, T);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_tile_order(const int* count, int* order, int rows, int KT, hipStream_t stream) {
  int P = 1, IB = 0;
  while (P < rows) P <<= 1;
  while ((1 << IB) < P) ++IB;
  if (P > 32768 || ((uint64_t)KT << IB) >= (1ull << 32)) return hipErrorInvalidValue;
  // the register path stores one key per thread (1024) in its LDS steps
  const size_t lds = (size_t)(P > 1024 ? P : 1024) * sizeof(uint32_t);
  hipLaunchKernelGGL(tile_order_kernel, dim3(1), dim3(1024), lds, stream, count, order, rows, KT, P, IB);
  return hipGetLastError();
}

hipError_t launch_block_select(const float* qbar, const float* kbar, uint8_t* mask, int rows, int QT, int KT,
                               int head_dim, float c, float log2_tau, hipStream_t stream) {
  const size_t lds = (size_t)KT * sizeof(float);
  if (head_dim == 128)
    hipLaunchKernelGGL(block_select_kernel<128>, dim3(rows), dim3(256), lds, stream, qbar, kbar, mask, QT, KT, c,
                       log2_tau);
  else if (head_dim == 64)
    hipLaunchKernelGGL(block_select_kernel<64>, dim3(rows), dim3(256), lds, stream, qbar, kbar, mask, QT, KT, c,
                       log2_tau);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_tile_bound(const BoundArgs& args, int head_dim, int num_cus, hipStream_t stream) {
  BoundArgs a = args;
  const int QT = (a.n_tokens + 255) / 256;
  const int tiles = a.batch * a.heads * QT;
  // Full rounds of whole query tiles; the tiles of a partial last round are
  // cut into key-tile ranges (at most 8 pieces, at least 8 key tiles each) so
  // that the round fills the compute units.
  const int C = num_cus > 0 ? num_cus : 1;
  const int rest = tiles % C;
  int split = rest > 0 ? C / rest : 1;
  split = split < 8 ? split : 8;
  split = split < a.kt / 8 ? split : a.kt / 8;
  if (split < 2) split = 1;
  a.whole = split > 1 ? tiles - rest : tiles;
  a.split = split;
  const dim3 grid((unsigned)(a.whole + (tiles - a.whole) * split));
  const size_t lds = (size_t)8 * a.kt * sizeof(float);
  if (lds > kBoundMaxLds) return hipErrorInvalidValue;
  if (head_dim == 128)
    hipLaunchKernelGGL(tile_bound_kernel<128>, grid, dim3(512), lds, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(tile_bound_kernel<64>, grid, dim3(512), lds, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_mask_to_list(const uint8_t* mask, int* list, int* count, int rows, int KT, int stride,
                               hipStream_t stream) {
  hipLaunchKernelGGL(mask_to_list_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, mask, list, count, rows, KT,
                     stride);
  return hipGetLastError();
}

}  // namespace flux
