// RoPE angle table: (cos, sin) per token and rotary pair.
//
// Rotary embedding (RoFormer, Su et al. 2021) as used by the FLUX 3 Image Klein
// transformer ("Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell
// GPUs", How it works).  Multi-axis form: head_dim is cut into three slices of
// widths (d0, d1, d2); pair j of slice a is rotated by pos[n][a] * theta^(-2j/d_a).
// The per-pair frequencies are computed once per plan on the host in double;
// here each angle is formed and evaluated in double, then stored as float.
#include "kernels.h"

namespace flux {

__global__ void rope_table_kernel(const int32_t* __restrict__ pos, const double* __restrict__ freq,
                                  float2* __restrict__ table, int n_tokens, int half, int p0, int p1) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_tokens * half) return;
  const int n = idx / half, p = idx - n * half;
  const int axis = p < p0 ? 0 : (p < p0 + p1 ? 1 : 2);
  const double ang = (double)pos[3 * n + axis] * freq[p];
  double s, c;
  sincos(ang, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

hipError_t launch_rope_table(const int32_t* pos, const double* freq, float2* table, int n_tokens,
                             int head_dim, int d0, int d1, hipStream_t stream) {
  const int half = head_dim / 2;
  const int total = n_tokens * half;
  const int threads = 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + threads - 1) / threads), dim3(threads), 0, stream,
                     pos, freq, table, n_tokens, half, d0 / 2, d1 / 2);
  return hipGetLastError();
}

}  // namespace flux
