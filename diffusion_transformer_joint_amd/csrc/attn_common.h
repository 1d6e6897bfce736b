// Pieces shared by the attention kernels: LDS row layout, key-row
// permutation of the score MFMA, RoPE from the packed fp16 table and the
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

// RoPE table entries are packed fp16 pairs: cos in the low half, sin in the
// high half (rope_table.hip).  The rotation's products take the fp16 values
// as operands of mixed-precision FMAs (v_fma_mix_f32 widens them exactly), so
// the half-size table costs no conversion instructions; a zero addend keeps
// a plain product in FMA form for that.  The halves are read through 16-bit
// integers: a bit cast of one vector element to a two-half vector made the
// compiler narrow a 16-byte table load to its first dword and use that entry
// for every pair.
__device__ __forceinline__ float cs_cos(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float cs_sin(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// (x0 c - x1 s, x0 s + x1 c) in fp32 from the table entry w.
__device__ __forceinline__ void rot_pair(float x0, float x1, uint32_t w, float& y0, float& y1) {
  const float c = cs_cos(w), s = cs_sin(w);
  y0 = __builtin_fmaf(x0, c, __builtin_fmaf(-x1, s, 0.f));
  y1 = __builtin_fmaf(x0, s, __builtin_fmaf(x1, c, 0.f));
}

// The inverse rotation (x0 c + x1 s, x1 c - x0 s).
__device__ __forceinline__ void rot_pair_back(float x0, float x1, uint32_t w, float& y0, float& y1) {
  const float c = cs_cos(w), s = cs_sin(w);
  y0 = __builtin_fmaf(x0, c, __builtin_fmaf(x1, s, 0.f));
  y1 = __builtin_fmaf(x1, c, __builtin_fmaf(-x0, s, 0.f));
}

// One bf16 pair rotated and rounded back to bf16.
__device__ __forceinline__ uint32_t rope_pair(uint32_t x, uint32_t w) {
  float y0, y1;
  rot_pair(bf16lo(x), bf16hi(x), w, y0, y1);
  return pack_bf16(y0, y1);
}

// The 4 adjacent bf16 pairs of one 16-byte chunk, with their 4 table entries.
__device__ __forceinline__ u32x4 rope_chunk(u32x4 x, u32x4 w) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = rope_pair(x[i], w[i]);
  return y;
}

// Same rotation, result multiplied by k before rounding (Q carries the
// softmax scale times log2(e)).
__device__ __forceinline__ u32x4 rope_chunk_scaled(u32x4 x, u32x4 w, float k) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y0, y1;
    rot_pair(bf16lo(x[i]), bf16hi(x[i]), w[i], y0, y1);
    y[i] = pack_bf16(y0 * k, y1 * k);
  }
  return y;
}

}  // namespace flux
