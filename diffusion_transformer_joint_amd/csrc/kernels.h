// Kernel argument blocks and launchers of the joint RoPE attention library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {

struct AttnArgs {
  const uint16_t* q;      // [B][N][H][D] bf16 bits
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;            // [B][N][H][D] bf16 bits
  const float2* rope;     // [N][D/2] (cos, sin)
  int n_tokens;
  int heads;
  int batch;
  int q_tiles;            // filled by the launcher
  float c;                // softmax scale * log2(e)
};

struct Fp8Args {
  const uint8_t* q;       // [B][N][H][D] e4m3 codes
  const uint8_t* k;
  const uint8_t* v;
  const float* scales;    // [3][B][H]
  uint16_t* o;            // [B][N][H][D] bf16 bits
  const float2* rope;     // [N][D/2]
  int n_tokens;
  int heads;
  int batch;
  int q_tiles;
  float c;
};

// (cos, sin) of pos[n][axis(p)] * freq[p] for every token n and pair p.
hipError_t launch_rope_table(const int32_t* pos, const double* freq, float2* table, int n_tokens,
                             int head_dim, int d0, int d1, hipStream_t stream);

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_attn_fp8(const Fp8Args& a, int head_dim, hipStream_t stream);

}  // namespace flux
