// Pieces shared by the bf16 and e4m3 attention kernels: LDS row layout,
// key-row permutation of the score MFMA, RoPE of a 16-byte bf16 chunk and the
// MFMA/VALU interleave hint.
#pragma once
#include "device_common.h"

namespace flux {

// LDS rows are padded instead of swizzled so that every fragment read is one
// per-lane base address plus a compile-time offset.
//   K rows: 2D + 16 bytes.  A 16-lane phase of the b128 fragment read touches
//   16 distinct rows at one column; the 16-byte skew per row puts them in 16
//   different 16-byte bank groups.
//   V rows: 2D + 64 bytes.  A 32-lane phase of the transpose read touches 4
//   consecutive rows x 64 bytes; the 64-byte skew makes those 256 bytes
//   cover every bank once.
template <int D> struct LdsRows {
  static constexpr int K = 2 * D + 16;
  static constexpr int V = 2 * D + 64;
};

template <int D>
__device__ __forceinline__ int k_off(int r, int c) { return r * LdsRows<D>::K + (c << 4); }

template <int D>
__device__ __forceinline__ int v_off(int r, int c) { return r * LdsRows<D>::V + (c << 4); }

// Key-row permutation for the S^T MFMA: swapping bits 2 and 3 of the MFMA row
// makes accumulator element e of lane l hold key 16(e/8) + 8(l/32) + e%8 of its
// 32-key block, i.e. 8 consecutive keys per P^T fragment.
__device__ __forceinline__ int krow_perm(int r) {
  return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Scheduling hint for the current basic block: MFMAs alternate with groups of
// up to VPM VALU instructions, LDS reads are issued ahead of them.
template <int NMFMA, int VPM>
__device__ __forceinline__ void sched_interleave() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0); // VALU
  }
}

// Rotate the 4 adjacent bf16 pairs of one 16-byte chunk by (cos, sin).
__device__ __forceinline__ u32x4 rope_chunk(u32x4 x, f32x4 cs01, f32x4 cs23) {
  u32x4 y;
  float c[4] = {cs01[0], cs01[2], cs23[0], cs23[2]};
  float s[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x0 = bf16lo(x[i]), x1 = bf16hi(x[i]);
    y[i] = pack_bf16(x0 * c[i] - x1 * s[i], x0 * s[i] + x1 * c[i]);
  }
  return y;
}

// Same rotation, result multiplied by k before rounding (Q carries the
// softmax scale times log2(e)).
__device__ __forceinline__ u32x4 rope_chunk_scaled(u32x4 x, f32x4 cs01, f32x4 cs23, float k) {
  u32x4 y;
  float c[4] = {cs01[0], cs01[2], cs23[0], cs23[2]};
  float s[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x0 = bf16lo(x[i]), x1 = bf16hi(x[i]);
    y[i] = pack_bf16((x0 * c[i] - x1 * s[i]) * k, (x0 * s[i] + x1 * c[i]) * k);
  }
  return y;
}

}  // namespace flux
