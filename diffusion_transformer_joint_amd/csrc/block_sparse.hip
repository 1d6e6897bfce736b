// Tile-sparse attention support: the pooled-score tile mask and the lists of
// kept key tiles.
//
// Sparse attention skips the work for less important token pairs according to
// a sparsity threshold tau ("Optimizing FLUX 3 Image Klein inference on NVIDIA
// Blackwell GPUs", How it works; What you can do: tau).  The importance
// measure and granularity are this library's reading: 256-token query tiles x
// 64-token key tiles; the pooled score of a tile pair is
// c * <mean of the tile's rotated q, mean of the tile's rotated k>
// (c = scale * log2 e); a key tile is kept when its pooled score is at least
// the query tile's largest plus log2(tau).
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

hipError_t launch_mask_to_list(const uint8_t* mask, int* list, int* count, int rows, int KT, int stride,
                               hipStream_t stream) {
  hipLaunchKernelGGL(mask_to_list_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, mask, list, count, rows, KT,
                     stride);
  return hipGetLastError();
}

}  // namespace flux
