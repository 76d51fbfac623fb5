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

// Four values (|v| < 2^9) -> four e4m3fn bytes, round to nearest even,
// saturating at 448: the hardware conversion after a clamp to [-448, 448]
// (an exhaustive check over every bf16 value below 2^9 in magnitude found it
// equal to the rounding written out: nearest even on the e4m3 grid, subnormal
// step 2^-9, ties to even, larger magnitudes to 448).
__device__ __forceinline__ uint32_t e4m3_encode4(float v0, float v1, float v2, float v3) {
  const float c0 = __builtin_amdgcn_fmed3f(v0, -448.f, 448.f);
  const float c1 = __builtin_amdgcn_fmed3f(v1, -448.f, 448.f);
  const float c2 = __builtin_amdgcn_fmed3f(v2, -448.f, 448.f);
  const float c3 = __builtin_amdgcn_fmed3f(v3, -448.f, 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t mag = code & 0x7Fu;
  const float v = mag < 8u ? (float)mag * 0.001953125f
                           : ldexpf((float)(8u + (mag & 7u)), (int)((mag >> 3) & 15u) - 10);
  return (code & 0x80u) ? -v : v;
}

// Four lanes per 32-value block (8 values, 16 bytes of input, each), so that a
// wave's loads and code stores cover contiguous runs of 1 KB and 512 bytes;
// the block's amax and finiteness are combined over the four lanes.  Padding
// blocks (K/32 <= b < lds) take zero codes (b < lda/32) and zero scale bytes.
// The four lanes of a block are one aligned quad, so a quad takes every
// branch together.
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const uint16_t* src, int rows, int K,
                                                          int lda, int lds, uint8_t* codes,
                                                          uint8_t* scales, uint16_t* deq) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= 4L * rows * lds) return;
  const long blk = t >> 2;
  const int q = (int)(t & 3);
  const int r = (int)(blk / lds);
  const int b = (int)(blk - (long)r * lds);
  const int kb = K / 32;
  if (b >= kb) {
    if (codes != nullptr && b < lda / 32)
      *reinterpret_cast<uint2*>(codes + (size_t)r * lda + 32 * b + 8 * q) = make_uint2(0, 0);
    if (scales != nullptr && q == 0) scales[(size_t)r * lds + b] = 0;
    return;
  }
  const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)r * K + 32 * b + 8 * q);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
  int finite = 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    amax = fmaxf(amax, fabsf(x[i]));
    finite &= (fabsf(x[i]) <= 3.4028235e38f) ? 1 : 0;  // 0 for NaN and infinities
  }
  // the quad's lanes are active together (see above)
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  finite &= __shfl_xor(finite, 1);
  finite &= __shfl_xor(finite, 2);
  // shared exponent: floor(log2 amax) - 8, clamped to [-127, 127]; subnormal
  // or zero amax clamps to -127
  const int ea = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = ea == 0 ? -127 : max(ea - 127 - 8, -127);
  uint32_t c[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    c[i] = finite ? e4m3_encode4(ldexpf(x[4 * i], -e), ldexpf(x[4 * i + 1], -e),
                                 ldexpf(x[4 * i + 2], -e), ldexpf(x[4 * i + 3], -e))
                  : 0x7F7F7F7Fu;
  if (codes != nullptr)
    *reinterpret_cast<uint2*>(codes + (size_t)r * lda + 32 * b + 8 * q) = make_uint2(c[0], c[1]);
  if (scales != nullptr && q == 0) scales[(size_t)r * lds + b] = (uint8_t)(finite ? e + 127 : 255);
  if (deq != nullptr) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c0 = (c[i / 2] >> (16 * (i & 1))) & 0xFFu;
      const uint32_t c1 = (c[i / 2] >> (16 * (i & 1) + 8)) & 0xFFu;
      const float v0 = finite ? ldexpf(e4m3_value(c0), e) : __builtin_nanf("");
      const float v1 = finite ? ldexpf(e4m3_value(c1), e) : __builtin_nanf("");
      o[i] = moe::pack_bf16x2(v0, v1);
    }
    *reinterpret_cast<uint4*>(deq + (size_t)r * K + 32 * b + 8 * q) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

extern "C" hipError_t moe_launch_mxfp8_quant(const uint16_t* src, int rows, int K, int lda,
                                             int lds, uint8_t* codes, uint8_t* scales,
                                             uint16_t* deq, hipStream_t st) {
  const long n = 4L * rows * lds;  // four lanes per block
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src,
                     rows, K, lda, lds, codes, scales, deq);
  return hipGetLastError();
}
