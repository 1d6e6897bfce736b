// Exact merge of split K/V ranges for gfx950 (MI355X).
//
// A query tile whose K/V range was cut into pieces (the split of the last
// round, or the persistent split) leaves one fp32 partial softmax state per
// piece: un-normalized O, the reference max m (exp2 domain) and the row sum
// l.  Merging is the exact recombination of online softmax (Milakov &
// Gimelshein 2018): with m = max m_i,
//     O = sum_i 2^(m_i - m) O_i / sum_i 2^(m_i - m) l_i,
// then bf16 out (and the natural-log log-sum-exp (m + log2 l) ln 2 when
// requested).  Joint attention over the concatenated token sequence ("Welcome
// FLUX.3 Image Klein in Diffusers", Architecture) is unchanged by the split.
#include "device_common.h"
#include "kernels.h"

namespace flux {

// Merge of a persistent-split launch: D/8 blocks per query tile, each block
// 256 / (D/8) rows of the tile with D/8 threads per row (8 dims each).  A tile
// that lies inside one slice was stored by the attention kernel and is left
// alone; otherwise the partial states of the slices covering it are combined
// in one pass with a running maximum (slice c keeps its piece of the tile in
// slot 2c when the tile is its first one, else in 2c + 1; empty slices hold
// none).  The slice arithmetic is block-uniform, so it stays out of the
// per-element work.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_sk_kernel(AttnArgs a) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;  // threads per row, rows per block
  const long ncu = a.sk_cus, nkv = a.sk_nkv;
  const long W = (long)a.sk_tiles * nkv;
  const int T = blockIdx.x / TPR, sub = blockIdx.x % TPR;
  const long t0 = (long)T * nkv, t1 = t0 + nkv;
  auto start = [&](long c) -> long { return W * c / ncu; };
  const long c0 = ((t0 + 1) * ncu + W - 1) / W - 1;  // the slice holding position t0
  if (start(c0 + 1) >= t1) return;                    // the whole tile lies in one slice
  const int r = sub * RPB + (int)threadIdx.x / TPR, d0 = ((int)threadIdx.x % TPR) * 8;
  const int N = a.rng_len[0];
  const int q_tiles = (N + 255) / 256;
  const int qt = T % q_tiles, bh = T / q_tiles;
  const int h = bh % a.heads, b = bh / a.heads;
  const int row = qt * 256 + r;
  if (row >= N) return;
  float m = -INFINITY, l = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (long cc = c0; cc < ncu && start(cc) < t1; ++cc) {
    const long s0 = start(cc);
    if (s0 == start(cc + 1)) continue;  // empty slice
    const long slot = 2 * cc + (s0 / nkv == T ? 0 : 1);
    const float2 ml = a.part_ml[slot * 256 + r];
    if (!(ml.y > 0.f)) continue;
    const float mn = fmaxf(m, ml.x);
    const float wa = __builtin_amdgcn_exp2f(m - mn), wb = __builtin_amdgcn_exp2f(ml.x - mn);
    const float* po = a.part_o + ((size_t)slot * 256 + r) * D + d0;
    const f32x4 x0 = *(const f32x4*)po, x1 = *(const f32x4*)(po + 4);
    l = l * wa + ml.y * wb;
    acc[0] = acc[0] * wa + x0[0] * wb; acc[1] = acc[1] * wa + x0[1] * wb;
    acc[2] = acc[2] * wa + x0[2] * wb; acc[3] = acc[3] * wa + x0[3] * wb;
    acc[4] = acc[4] * wa + x1[0] * wb; acc[5] = acc[5] * wa + x1[1] * wb;
    acc[6] = acc[6] * wa + x1[2] * wb; acc[7] = acc[7] * wa + x1[3] * wb;
    m = mn;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (a.lse != nullptr && d0 == 0)
    a.lse[((size_t)b * a.heads + h) * N + row] = (m + __builtin_log2f(l)) * 0.6931471805599453f;
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = pack_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  const size_t tok_stride = (size_t)a.heads * D;
  *(u32x4*)(a.o + ((size_t)b * a.batch_tokens + a.rng_tok0[0] + row) * tok_stride + (size_t)h * D + d0) = out;
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
  const int tile_g = a.tile_order != nullptr ? a.tile_order[a.whole + st] : a.whole + st;
  int rg = 0;
  while (rg + 1 < a.nranges && tile_g >= a.rng_tile0[rg + 1]) ++rg;
  const int N = a.rng_len[rg], tok0 = a.rng_tok0[rg];
  const int tile = tile_g - a.rng_tile0[rg];
  const int q_tiles = (N + 255) / 256;
  const int qt = tile % q_tiles, bh = tile / q_tiles;
  const int h = bh % a.heads, b = bh / a.heads;
  const int row = qt * 256 + r;
  if (row >= N) return;
  const int slot0 = st * a.split;
  float m = -INFINITY;
  for (int i = 0; i < a.split; ++i) m = fmaxf(m, a.part_ml[(size_t)(slot0 + i) * 256 + r].x);
  float l = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < a.split; ++i) {
    const float2 ml = a.part_ml[(size_t)(slot0 + i) * 256 + r];
    const float w = ml.y > 0.f ? __builtin_amdgcn_exp2f(ml.x - m) : 0.f;  // empty ranges weigh 0
    l += w * ml.y;
    const float* po = a.part_o + ((size_t)(slot0 + i) * 256 + r) * D + d0;
    const f32x4 x0 = *(const f32x4*)po, x1 = *(const f32x4*)(po + 4);
    acc[0] += w * x0[0]; acc[1] += w * x0[1]; acc[2] += w * x0[2]; acc[3] += w * x0[3];
    acc[4] += w * x1[0]; acc[5] += w * x1[1]; acc[6] += w * x1[2]; acc[7] += w * x1[3];
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;  // 0: no kept keys (tile-sparse)
  if (a.lse != nullptr && d0 == 0)
    a.lse[((size_t)b * a.heads + h) * N + row] = (m + __builtin_log2f(l)) * 0.6931471805599453f;
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = pack_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  const size_t tok_stride = (size_t)a.heads * D;
  *(u32x4*)(a.o + ((size_t)b * a.batch_tokens + tok0 + row) * tok_stride + (size_t)h * D + d0) = out;
}

hipError_t launch_attn_merge(const AttnArgs& a, int head_dim, const Schedule& sch, hipStream_t stream) {
  if (sch.sk_nkv > 0) {
    AttnArgs args = a;
    args.sk_nkv = sch.sk_nkv;
    args.sk_tiles = sch.sk_tiles;
    args.sk_cus = sch.sk_cus;
    const dim3 grid((unsigned)(sch.sk_tiles * (head_dim / 8)));
    if (sch.sk_cus < 2 || sch.sk_tiles < 1) return hipSuccess;
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_merge_sk_kernel<128>, grid, dim3(256), 0, stream, args);
    else if (head_dim == 64)
      hipLaunchKernelGGL(attn_merge_sk_kernel<64>, grid, dim3(256), 0, stream, args);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (sch.split_tiles == 0) return hipSuccess;
  AttnArgs args = a;
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
