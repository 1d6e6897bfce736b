// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, bf16 packing, LDS transpose reads and XCD-aware tile order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace flux {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FLUX_LDS __attribute__((address_space(3)))

// 32x32x16 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%32][8(l/32)..+8]
// and B[8(l/32)..+8][l%32]; result element e of lane l is
// C[8(e/4) + 4(l/32) + e%4][l%32].
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x64 fp8(e4m3) x fp8(e4m3) MFMA, fp32 accumulate.  Lane l supplies 32
// codes of row l%32 of A and of column l%32 of B; the k split between lanes l
// and l+32 only has to agree between A and B.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest even) and pack: a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Inside each group of 16
// lanes, lane i receives half-word (i % 4) of the 8 bytes addressed by lanes
// 4e + i/4, e = 0..3, as its element e.
__device__ __forceinline__ u32x2 lds_read_tr16(const FLUX_LDS void* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FLUX_LDS i16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 lds_read_b128(const FLUX_LDS void* p) {
  return *(const FLUX_LDS u32x4*)p;
}

__device__ __forceinline__ void lds_write_b128(FLUX_LDS void* p, u32x4 v) {
  *(FLUX_LDS u32x4*)p = v;
}

__device__ __forceinline__ u32x4 global_load_b128(const void* p) {
  return *(const u32x4*)p;
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return 0 (hardware range check), which zero-fills rows past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}

__device__ __forceinline__ u32x2 buffer_load_b64(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voffset, 0, 0));
}

__device__ __forceinline__ uint32_t buffer_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voffset, 0, 0));
}

__device__ __forceinline__ float bf16_round(float x) {
  return (float)(__bf16)x;
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 in order: a loop
// that is unrolled however large its body is, with a compile-time index.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Value of lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32);
}

// Optional clock measurement of a workgroup: shader-clock cycles
// (s_memtime) and constant-rate wall-clock ticks (s_memrealtime) from the
// workgroup's start to the end of its first wave are added to dst[0] and
// dst[1] by one thread; their ratio over a launch is the average shader clock
// the launch's workgroups ran at.  The start values are subtracted at once
// (unsigned sums wrap, so the totals come out right) and nothing stays live
// across the kernel.  dst == nullptr: off (one uniform branch each).
struct ClockProbe {
  unsigned long long* dst;
  __device__ __forceinline__ explicit ClockProbe(unsigned long long* d) : dst(d) {
    if (dst != nullptr && threadIdx.x == 0) {
      const uint64_t c0 = __builtin_amdgcn_s_memtime();
      const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
      atomicAdd(dst, (unsigned long long)(0ull - c0));
      atomicAdd(dst + 1, (unsigned long long)(0ull - r0));
    }
  }
  __device__ __forceinline__ void finish() const {
    if (dst != nullptr && threadIdx.x == 0) {
      const uint64_t c1 = __builtin_amdgcn_s_memtime();
      const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
      atomicAdd(dst, (unsigned long long)c1);
      atomicAdd(dst + 1, (unsigned long long)r1);
    }
  }
};

// Tiles are dispatched round-robin over the 8 XCDs (block i runs on XCD i % 8).
// Remap so that each XCD receives a contiguous range of logical tiles: tiles of
// one head then share that XCD's L2.  A bijection on [0, total).
__device__ __forceinline__ int xcd_tile_order(int i, int total) {
  const int nx = 8;
  int per = total / nx, rem = total % nx;
  int x = i % nx, k = i / nx;
  return x * per + (x < rem ? x : rem) + k;
}

}  // namespace flux
