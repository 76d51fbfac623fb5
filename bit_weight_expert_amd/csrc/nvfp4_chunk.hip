// NVFP4 scales and codes re-laid by 64-deep K chunk, and MXFP4 scales and
// codes by 128-deep K chunk, once, when the weights are loaded.
//
// The checkpoint layout keeps each weight row's e4m3 group scales (one per 16
// along K) together: [E][N][K/16].  The 64/128-row GEMM kernel reads, for each
// 64-deep chunk, the four scales of that chunk for 256 consecutive rows; in
// the checkpoint layout those are 4 bytes every K/16 bytes, one memory request
// per row.  Laid out as [E][K/64][N][4] they are one contiguous kilobyte that
// the kernel copies into on-chip memory with the chunk's codes.
//
// The codes ([E][N][K/2], 32 bytes per row per chunk) have the same problem
// at a larger grain: one chunk of a 32-row block is 32 pieces of 32 bytes, a
// quarter of a cache line each, and the other three quarters are evicted
// before the next chunks use them.  Laid out as [E][K/64][N][32] a block's
// chunk is one contiguous kilobyte.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// One thread per (expert, chunk, row): one aligned 4-byte word moved.
__global__ __launch_bounds__(256) void nvfp4_scales_by_chunk_kernel(const uint32_t* __restrict__ in,
                                                                    int N, int KC,
                                                                    uint32_t* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  const int e = blockIdx.z;
  if (n >= N) return;
  // in: row (e, n) holds KC words (4 scales each); out: [e][c][n]
  out[((size_t)e * KC + c) * N + n] = in[((size_t)e * N + n) * KC + c];
}


// One thread per (expert, chunk, row): 32 aligned bytes moved.
__global__ __launch_bounds__(256) void nvfp4_codes_by_chunk_kernel(const uint4* __restrict__ in,
                                                                   int N, int KC,
                                                                   uint4* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  const int e = blockIdx.z;
  if (n >= N) return;
  // in: row (e, n) holds 2*KC 16-byte units; out: [e][c][n] two units
  const uint4* src = in + (((size_t)e * N + n) * KC + c) * 2;
  uint4* dst = out + (((size_t)e * KC + c) * N + n) * 2;
  dst[0] = src[0];
  dst[1] = src[1];
}


// MXFP4 codes by 128-deep K chunk for the MX kernel: [E][ceil(K/128)][N][64];
// the part of the last chunk past K (K % 128 == 64) is zero.  One thread per
// (expert, chunk, row): four 16-byte units.
__global__ __launch_bounds__(256) void mxfp4_codes_by_chunk_kernel(const uint4* __restrict__ in,
                                                                   int N, int K, int KC,
                                                                   uint4* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  const int e = blockIdx.z;
  if (n >= N) return;
  const int units = K / 32;  // 16-byte units per row
  const uint4* src = in + ((size_t)e * N + n) * units;
  uint4* dst = out + (((size_t)e * KC + c) * N + n) * 4;
#pragma unroll
  for (int u = 0; u < 4; ++u) dst[u] = 4 * c + u < units ? src[4 * c + u] : make_uint4(0, 0, 0, 0);
}

// MXFP4 e8m0 scales by 128-deep K chunk: [E][ceil(K/128)][N][4], byte j of
// row n's word of chunk c = the scale of 32-group 4c + j (0 past K/32).  One
// thread per (expert, chunk, row); the checkpoint bytes are read one by one
// (K/32 need not be a multiple of 4).
__global__ __launch_bounds__(256) void mxfp4_scales_by_chunk_kernel(const uint8_t* __restrict__ in,
                                                                    int N, int G, int KC,
                                                                    uint32_t* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  const int e = blockIdx.z;
  if (n >= N) return;
  const uint8_t* row = in + ((size_t)e * N + n) * G;
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * c + j < G) w |= (uint32_t)row[4 * c + j] << (8 * j);
  out[((size_t)e * KC + c) * N + n] = w;
}

}  // namespace

extern "C" hipError_t moe_launch_mxfp4_scales_by_chunk(const uint8_t* scales, int E, int N, int K,
                                                       uint8_t* out, hipStream_t st) {
  const int g = K / 32, kc = (K + 127) / 128;
  hipLaunchKernelGGL(mxfp4_scales_by_chunk_kernel, dim3((N + 255) / 256, kc, E), dim3(256), 0, st,
                     scales, N, g, kc, reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_nvfp4_scales_by_chunk(const uint8_t* scales, int E, int N, int K,
                                                       uint8_t* out, hipStream_t st) {
  const int kc = K / 64;
  hipLaunchKernelGGL(nvfp4_scales_by_chunk_kernel, dim3((N + 255) / 256, kc, E), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(scales), N, kc,
                     reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_nvfp4_codes_by_chunk(const uint8_t* qweight, int E, int N, int K,
                                                      uint8_t* out, hipStream_t st) {
  const int kc = K / 64;
  hipLaunchKernelGGL(nvfp4_codes_by_chunk_kernel, dim3((N + 255) / 256, kc, E), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(qweight), N, kc, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_mxfp4_codes_by_chunk(const uint8_t* qweight, int E, int N, int K,
                                                      uint8_t* out, hipStream_t st) {
  const int kc = (K + 127) / 128;
  hipLaunchKernelGGL(mxfp4_codes_by_chunk_kernel, dim3((N + 255) / 256, kc, E), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(qweight), N, K, kc, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}
