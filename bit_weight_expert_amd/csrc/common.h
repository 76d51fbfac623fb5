// Internal helpers shared by the HIP sources of the library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// Weight formats and epilogues (values match the public enums).
enum { FMT_NVFP4 = 0, FMT_MXFP4 = 1, FMT_GPTQ = 2 };
enum { EPI_SWIGLU = 0, EPI_RELU2 = 1, EPI_NONE = 2, EPI_DOWN = 3 };
// Workgroups of the multi-workgroup sort (its count table is kAlignGroups x E ints).
constexpr int kAlignGroups = 16;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float -> bf16 bits, round to nearest even (inputs here are finite or NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  const bf16x2 r = __builtin_convertvector(v, bf16x2);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// Parameters of one weight family as the kernels see them.
struct WeightArgs {
  const uint8_t* qweight;      // NVFP4/MXFP4: [E][N][K/2]; GPTQ: int32 words [E][K/8][N]
  const uint8_t* scales;       // e4m3 / e8m0 bytes, or fp16 [E][K/G][N]
  const uint32_t* zeros;       // GPTQ zero words [E][K/G][N/8]
  const float* global_scale;   // NVFP4 [E]
  const uint16_t* bias;        // bf16 [E][N] or null
  int group;
  const uint8_t* scales_kc;    // scales by K chunk, or null: NVFP4 e4m3 [E][K/64][N][4],
                               // MXFP4 e8m0 [E][ceil(K/128)][N][4]
  const uint8_t* qweight_kc;   // codes by K chunk, or null: NVFP4 [E][K/64][N][32] (needs
                               // scales_kc), MXFP4 [E][ceil(K/128)][N][64]
  const int32_t* g_idx;        // GPTQ group map [E][K], or null; only the identity is valid here
};

// Kernel choice for blocks of 16/32 rows (values match the public enum).
enum { KERNEL_AUTO = 0, KERNEL_SPLITK = 1, KERNEL_WIDE = 2 };

}  // namespace moe
