// MXFP8 quantiser for the GEMM inputs of the MXFP4 x MXFP8 layer.
//
// The variant is the MoE with MXFP8 activations that the "gpt-oss-120b MXFP4
// + --enable-expert-parallel crashes" page names as the alternative to bf16
// activations (sections "Actual behavior" and "Why the mxfp8 workaround is
// not a fix").  The page names the format only; the encoding is the OCP
// microscaling one: per block of 32 consecutive values of a row the shared
// e8m0 exponent is floor(log2(amax)) - 8 (8 = exponent of e4m3's largest
// normal 448), and each element is value / 2^exponent rounded to the nearest
// e4m3 value, ties to even, saturating at 448.  An all-zero block takes
// exponent -127 (byte 0); a block holding a NaN or an infinity gets the NaN
// exponent 0xFF and NaN elements.
//
// Layout written (what the MX GEMM kernel reads): codes [rows][lda] with
// lda = K rounded up to 128 and zeros past K; scales [rows][lds] with
// lds = K/32 rounded up to 16 and zeros past K/32.  Optionally the
// dequantised values as bf16 [rows][K] (exact: an e4m3 value times a power of
// two has at most 4 significant bits), which may overwrite the input.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace {

// |v| < 2^9 (or infinite) -> e4m3fn byte, round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t mag;
  if (!(a < 448.f)) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal step 2^-9 (8 steps = 2^-6 is code 8)
    mag = (uint32_t)rintf(a * 512.f);
  } else {
    int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // -6 .. 8
    uint32_t m = (uint32_t)rintf(ldexpf(a, 3 - E));           // 8 .. 16
    if (m == 16u) {
      ++E;
      m = 8u;
    }
    mag = min((uint32_t)(((E + 7) << 3) | (int)(m - 8u)), 0x7Eu);
  }
  return sign | mag;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t mag = code & 0x7Fu;
  const float v = mag < 8u ? (float)mag * 0.001953125f
                           : ldexpf((float)(8u + (mag & 7u)), (int)((mag >> 3) & 15u) - 10);
  return (code & 0x80u) ? -v : v;
}

// One thread per 32-value block of a row, and per padding block / scale byte.
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const uint16_t* src, int rows, int K,
                                                          int lda, int lds, uint8_t* codes,
                                                          uint8_t* scales, uint16_t* deq) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long)rows * lds) return;
  const int r = (int)(t / lds);
  const int b = (int)(t - (long)r * lds);
  const int kb = K / 32;
  if (b >= kb) {
    if (codes != nullptr && b < lda / 32) {
      uint4* c = reinterpret_cast<uint4*>(codes + (size_t)r * lda + 32 * b);
      c[0] = make_uint4(0, 0, 0, 0);
      c[1] = make_uint4(0, 0, 0, 0);
    }
    if (scales != nullptr) scales[(size_t)r * lds + b] = 0;
    return;
  }
  const uint4* s = reinterpret_cast<const uint4*>(src + (size_t)r * K + 32 * b);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = s[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  float x[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    amax = fmaxf(amax, fabsf(x[i]));
    finite = finite && (fabsf(x[i]) <= 3.4028235e38f);  // false for NaN and infinities
  }
  // shared exponent: floor(log2 amax) - 8, clamped to [-127, 127]; subnormal
  // or zero amax clamps to -127
  const int ea = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = ea == 0 ? -127 : max(ea - 127 - 8, -127);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t code = finite ? e4m3_encode(ldexpf(x[4 * i + j], -e)) : 0x7Fu;
      word |= code << (8 * j);
    }
    q[i] = word;
  }
  if (codes != nullptr) {
    uint4* c = reinterpret_cast<uint4*>(codes + (size_t)r * lda + 32 * b);
    c[0] = make_uint4(q[0], q[1], q[2], q[3]);
    c[1] = make_uint4(q[4], q[5], q[6], q[7]);
  }
  if (scales != nullptr) scales[(size_t)r * lds + b] = (uint8_t)(finite ? e + 127 : 255);
  if (deq != nullptr) {
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c0 = (q[i / 2] >> (16 * (i & 1))) & 0xFFu;
      const uint32_t c1 = (q[i / 2] >> (16 * (i & 1) + 8)) & 0xFFu;
      const float v0 = finite ? ldexpf(e4m3_value(c0), e) : __builtin_nanf("");
      const float v1 = finite ? ldexpf(e4m3_value(c1), e) : __builtin_nanf("");
      o[i] = moe::pack_bf16x2(v0, v1);
    }
    uint4* d = reinterpret_cast<uint4*>(deq + (size_t)r * K + 32 * b);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
}

}  // namespace

extern "C" hipError_t moe_launch_mxfp8_quant(const uint16_t* src, int rows, int K, int lda,
                                             int lds, uint8_t* codes, uint8_t* scales,
                                             uint16_t* deq, hipStream_t st) {
  const long n = (long)rows * lds;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src,
                     rows, K, lda, lds, codes, scales, deq);
  return hipGetLastError();
}
