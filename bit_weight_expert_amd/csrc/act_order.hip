// GPTQ act-order ("desc_act") support.
//
// A GPTQ checkpoint quantised in activation order keeps its rows in the
// model's input-channel order and gives each row k its quantisation group
// g_idx[k] (the per-expert gate_proj/up_proj/down_proj tensors of the
// OneCompression "GPT-OSS (mixed_gptq)" page, section 1, list g_idx next to
// qweight, qzeros and scales).  The GEMM kernels read groups as contiguous
// runs of group_size rows, so act-order weights are brought into that form
// once, when they are loaded:
//
//   gptq_sort_kernel        per expert, the stable order of the rows by group
//                           (k_perm), after checking that every group holds
//                           exactly group_size rows
//   gptq_repack_rows_kernel the packed 4-bit rows in that order
//
// after which row k of the stored weight multiplies input channel k_perm[k]
// and the scales and zero points apply unchanged.  At run time the GEMM input
// rows are gathered through the same permutation (permute_slots_kernel): one
// row per flat slot, permuted by the slot's own expert.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// One workgroup per expert.  LDS: g_idx of the expert, then the group counts.
__global__ __launch_bounds__(1024) void gptq_sort_kernel(const int32_t* __restrict__ g_idx, int K,
                                                         int G, int32_t* __restrict__ k_perm,
                                                         int32_t* __restrict__ status) {
  extern __shared__ int32_t sort_lds[];
  __shared__ int bad;
  const int e = blockIdx.x;
  const int ng = K / G;
  int32_t* gl = sort_lds;
  int32_t* cnt = sort_lds + K;
  const int32_t* ge = g_idx + (size_t)e * K;
  int32_t* pe = k_perm + (size_t)e * K;
  if (threadIdx.x == 0) bad = 0;
  for (int g = threadIdx.x; g < ng; g += blockDim.x) cnt[g] = 0;
  __syncthreads();
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    const int v = ge[k];
    gl[k] = v;
    if (v < 0 || v >= ng)
      bad = 1;
    else
      atomicAdd(&cnt[v], 1);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < ng; g += blockDim.x)
    if (cnt[g] != G) bad = 1;
  __syncthreads();
  if (bad) {
    // not a valid act-order map: report it and leave the identity order
    for (int k = threadIdx.x; k < K; k += blockDim.x) pe[k] = k;
    if (threadIdx.x == 0) status[e] = 1;
    return;
  }
  // group g fills positions g*G .. g*G+G-1 with its rows in ascending k; the
  // count check above bounds c by G
  for (int g = threadIdx.x; g < ng; g += blockDim.x) {
    int c = 0;
    int32_t* dst = pe + (size_t)g * G;
    for (int k = 0; k < K; ++k)
      if (gl[k] == g) dst[c++] = k;
  }
  if (threadIdx.x == 0) status[e] = 0;
}

// qweight int32 [E][K/8][N], nibble i of word [r][n] holds row 8r+i.  One
// thread per output word: out[e][r][n] nibble i = row k_perm[8r+i] of column n.
__global__ __launch_bounds__(256) void gptq_repack_rows_kernel(const uint32_t* __restrict__ q,
                                                               const int32_t* __restrict__ k_perm,
                                                               int K, int N,
                                                               uint32_t* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int e = blockIdx.z;
  if (n >= N) return;
  const int32_t* pe = k_perm + (size_t)e * K + 8 * r;
  const uint32_t* qe = q + (size_t)e * (K / 8) * N;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = min((unsigned)pe[i], (unsigned)(K - 1));
    const uint32_t src = qe[(size_t)(k >> 3) * N + n];
    w |= ((src >> (4 * (k & 7))) & 0xFu) << (4 * i);
  }
  out[((size_t)e * (K / 8) + r) * N + n] = w;
}

// One workgroup per flat slot f: dst[f][k] = src[f / top_k][k_perm[e][k]] with
// e = topk_ids[f].  The source row is staged in LDS before anything is
// written, so dst may be src when top_k is 1 (each workgroup owns its row).
// Slots whose expert is outside [0, E) are skipped (no GEMM block reads them).
constexpr int kPermThreads = 128;

__global__ __launch_bounds__(kPermThreads) void permute_slots_kernel(
    const uint16_t* src, int top_k, int K, int E, const int32_t* __restrict__ k_perm,
    const int32_t* __restrict__ topk_ids, uint16_t* dst) {
  extern __shared__ uint16_t perm_row[];
  const int f = blockIdx.x;
  const int e = topk_ids[f];
  if (e < 0 || e >= E) return;
  const uint4* s = reinterpret_cast<const uint4*>(src + (size_t)(f / top_k) * K);
  uint4* lrow = reinterpret_cast<uint4*>(perm_row);
  const int nv = K / 8;
  for (int i = threadIdx.x; i < nv; i += kPermThreads) lrow[i] = s[i];
  __syncthreads();
  const int4* pe = reinterpret_cast<const int4*>(k_perm + (size_t)e * K);
  uint4* d = reinterpret_cast<uint4*>(dst + (size_t)f * K);
  const unsigned kmax = (unsigned)(K - 1);
  for (int i = threadIdx.x; i < nv; i += kPermThreads) {
    const int4 p0 = pe[2 * i];
    const int4 p1 = pe[2 * i + 1];
    auto at = [&](int k) { return (uint32_t)perm_row[min((unsigned)k, kmax)]; };
    uint4 v;
    v.x = at(p0.x) | (at(p0.y) << 16);
    v.y = at(p0.z) | (at(p0.w) << 16);
    v.z = at(p1.x) | (at(p1.y) << 16);
    v.w = at(p1.z) | (at(p1.w) << 16);
    d[i] = v;
  }
}

}  // namespace

extern "C" hipError_t moe_launch_gptq_sort(const int32_t* qweight, const int32_t* g_idx, int E,
                                           int K, int N, int G, int32_t* qweight_sorted,
                                           int32_t* k_perm, int32_t* status, hipStream_t st) {
  const size_t lds = (size_t)(K + K / G) * sizeof(int32_t);
  hipLaunchKernelGGL(gptq_sort_kernel, dim3(E), dim3(1024), lds, st, g_idx, K, G, k_perm, status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gptq_repack_rows_kernel, dim3((N + 255) / 256, K / 8, E), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(qweight), k_perm, K, N,
                     reinterpret_cast<uint32_t*>(qweight_sorted));
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_permute_slots(const uint16_t* src, int n_slots, int top_k, int K,
                                               int E, const int32_t* k_perm,
                                               const int32_t* topk_ids, uint16_t* dst,
                                               hipStream_t st) {
  if (n_slots == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_slots_kernel, dim3(n_slots), dim3(kPermThreads),
                     (size_t)K * sizeof(uint16_t), st, src, top_k, K, E, k_perm, topk_ids, dst);
  return hipGetLastError();
}
