// RoPE angle table: (cos, sin) per token and rotary pair.
//
// Rotary embedding (RoFormer, Su et al. 2021) as used by the FLUX 3 Image Klein
// transformer ("Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell
// GPUs", How it works).  Multi-axis form: head_dim is cut into three slices of
// widths (d0, d1, d2); pair j of slice a is rotated by pos[n][a] * theta^(-2j/d_a).
// The per-pair frequencies are computed on the host in double and passed by
// value; here each angle is formed in double.
//
// Two storage forms:
//   packed fp16 (the attention kernels): one dword per pair, cos in the low
//     half and sin in the high half, rounded to nearest: 4 bytes per pair,
//     error at most 2^-12 (plus ~1e-7 from the fp32 evaluation) in each, a
//     small fraction of the bf16 rounding that follows the rotation;
//   float2 (the tile-mask rule, whose pooled scores decide kept tiles and are
//     compared with an exact rule): (cos, sin) evaluated in double, stored
//     as fp32.
#include "kernels.h"

namespace flux {

template <bool PACKED16>
__global__ void rope_table_kernel(const int32_t* __restrict__ pos, const RopeFreq freq,
                                  void* __restrict__ table, int n_tokens, int half, int p0, int p1) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_tokens * half) return;
  const int n = idx / half, p = idx - n * half;
  const int axis = p < p0 ? 0 : (p < p0 + p1 ? 1 : 2);
  const double ang = (double)pos[3 * n + axis] * freq.f[p];
  if constexpr (PACKED16) {
    // The angle is reduced to [-pi, pi] in double and evaluated in fp32:
    // error ~1e-7, far below the fp16 rounding (2^-12) that follows.
    constexpr double kTwoPi = 6.283185307179586476925286766559;
    const float r = (float)(ang - kTwoPi * rint(ang * (1.0 / kTwoPi)));
    float s, c;
    sincosf(r, &s, &c);
    const uint32_t ch = __builtin_bit_cast(uint16_t, (_Float16)c);
    const uint32_t sh = __builtin_bit_cast(uint16_t, (_Float16)s);
    static_cast<uint32_t*>(table)[idx] = ch | (sh << 16);
  } else {
    double s, c;
    sincos(ang, &s, &c);
    static_cast<float2*>(table)[idx] = make_float2((float)c, (float)s);
  }
}

template <bool PACKED16>
static hipError_t launch_table(const int32_t* pos, const RopeFreq& freq, void* table, int n_tokens, int head_dim,
                               int d0, int d1, hipStream_t stream) {
  const int half = head_dim / 2;
  const int total = n_tokens * half;
  const int threads = 256;
  hipLaunchKernelGGL(rope_table_kernel<PACKED16>, dim3((total + threads - 1) / threads), dim3(threads), 0, stream,
                     pos, freq, table, n_tokens, half, d0 / 2, d1 / 2);
  return hipGetLastError();
}

hipError_t launch_rope_table(const int32_t* pos, const RopeFreq& freq, uint32_t* table, int n_tokens,
                             int head_dim, int d0, int d1, hipStream_t stream) {
  return launch_table<true>(pos, freq, table, n_tokens, head_dim, d0, d1, stream);
}

hipError_t launch_rope_table_f32(const int32_t* pos, const RopeFreq& freq, float2* table, int n_tokens,
                                 int head_dim, int d0, int d1, hipStream_t stream) {
  return launch_table<false>(pos, freq, table, n_tokens, head_dim, d0, d1, stream);
}

}  // namespace flux
