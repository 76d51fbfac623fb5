// Grouped W4A16 GEMMs (GEMM1 with gate/up weights, GEMM2 with down weights)
// and the k-row sum, for gfx950.
//
// Work decomposition.  One workgroup = one aligned block of BM sorted slots
// (all of one expert, "moe_align_block_size" in the NVFP4 repro) x BN = 128
// output columns.  Four waves split the columns, 32 per wave, so every
// 4-bit weight is fetched and dequantised exactly once per workgroup and no
// LDS is spent on the weights.  The A rows (x for GEMM1, gathered through
// sorted_id / top_k; the intermediate for GEMM2, one row per slot) are
// staged through LDS in K-chunks of 128 and shared by the four waves.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16).  Lane l works on column l%16 of a
// 16-column fragment and on k-group g = l/16.  Within a 128-wide K chunk the
// lane owns the 32 consecutive k in [32g, 32g+32): one 16-byte load of
// e2m1 codes (or four GPTQ words), dequantised in registers and consumed by
// four MFMA steps, step s taking k in [32g+8s, 32g+8s+8).  The A fragment of
// step s is read from LDS with the same k assignment, so the reduction covers
// every k exactly once (the order of a reduction is free).
//
// Dequantisation (exact in bf16 for NVFP4 and MXFP4):
//   NVFP4  e2m1 -> f32 with the gfx950 fp4 convert (scale 1), times the
//          e4m3 block scale in f32, rounded to bf16 (exact: 2 x 4 significant
//          bits); the per-expert global scale multiplies the fp32 accumulator.
//   MXFP4  the fp4 -> bf16 convert applies the e8m0 power of two itself.
//   GPTQ   (q - z) * s evaluated exactly in f32 as fma(q, s, -z*s), then
//          rounded once to bf16.
//
// Tails.  K need only be a multiple of 32: a lane whose 32-k range lies past
// K loads nothing and contributes zeros, and the A tile is zero-filled there.
// N need only be a multiple of 16 (32 when gated): whole fragments past N are
// skipped.  No padded buffer is read or written (hidden 2880 = 22*128 + 64).
//
// Epilogue.  GEMM1: + bias, then swigluoai over the (gate, up) pair -- lane
// fragments 0/1 of a wave hold weight rows 2c and 2c+1, so the pair meets in
// one lane -- or ReLU^2.  GEMM2: (acc * global + bias) * topk_w[sorted_id],
// the routing weight looked up by the same sorted slot id the row is stored
// under (the bug on "moe_wna16_marlin_gemm applies wrong per-row topk
// weights" was a row index that did not match the slot).
#include "common.h"

namespace moe {

constexpr int kWaves = 4;
constexpr int kWN = 32;                // columns per wave
constexpr int kBN = kWaves * kWN;      // columns per workgroup
constexpr int kBK = 128;               // K chunk
constexpr int kLdsRow = kBK / 8 + 1;   // uint4 per LDS row (one uint4 of padding)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ uint4 deq_nvfp4(uint32_t w, float s) {
  uint4 r;
  f32x2 p;
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  r.x = pack_bf16x2(p[0] * s, p[1] * s);
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  r.y = pack_bf16x2(p[0] * s, p[1] * s);
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  r.z = pack_bf16x2(p[0] * s, p[1] * s);
  p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  r.w = pack_bf16x2(p[0] * s, p[1] * s);
  return r;
}

__device__ __forceinline__ uint4 deq_mxfp4(uint32_t w, float s) {
  uint4 r;
  bf16x2 p;
  p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  __builtin_memcpy(&r.x, &p, 4);
  p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  __builtin_memcpy(&r.y, &p, 4);
  p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  __builtin_memcpy(&r.z, &p, 4);
  p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  __builtin_memcpy(&r.w, &p, 4);
  return r;
}

__device__ __forceinline__ uint4 deq_gptq(uint32_t w, float s, float zs) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf((float)((w >> (4 * i)) & 15u), s, -zs);
  uint4 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  r.z = pack_bf16x2(v[4], v[5]);
  r.w = pack_bf16x2(v[6], v[7]);
  return r;
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

// Raw weight data of one lane for one 16-column fragment and one K chunk.
struct BRaw {
  uint4 q;       // 32 codes (NVFP4/MXFP4) or 4 GPTQ words
  float s0, s1;  // NVFP4: scales of the two 16-k groups; MXFP4: s0 = 2^(e-127); GPTQ: s0 = s, s1 = z*s
};

template <int FMT>
__device__ __forceinline__ void load_b(BRaw& b, const WeightArgs& W, int e, int n, int N, int K,
                                       int k) {
  if (FMT == FMT_NVFP4) {
    const size_t row = (size_t)e * N + n;
    b.q = *reinterpret_cast<const uint4*>(W.qweight + row * (K / 2) + k / 2);
    const uint16_t sb = *reinterpret_cast<const uint16_t*>(W.scales + row * (K / 16) + k / 16);
    b.s0 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0);
    b.s1 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 1);
  } else if (FMT == FMT_MXFP4) {
    const size_t row = (size_t)e * N + n;
    b.q = *reinterpret_cast<const uint4*>(W.qweight + row * (K / 2) + k / 2);
    const uint32_t sb = W.scales[row * (K / 32) + k / 32];
    b.s0 = __uint_as_float(sb << 23);
    b.s1 = 0.f;
  } else {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(W.qweight);
    const size_t base = ((size_t)e * (K / 8) + k / 8) * N + n;
    b.q.x = qw[base];
    b.q.y = qw[base + N];
    b.q.z = qw[base + 2 * (size_t)N];
    b.q.w = qw[base + 3 * (size_t)N];
    const int grp = k / W.group;
    const size_t gi = (size_t)e * (K / W.group) + grp;
    const float s = half_bits_to_f32(reinterpret_cast<const uint16_t*>(W.scales)[gi * N + n]);
    const uint32_t z = (W.zeros[gi * (N / 8) + n / 8] >> (4 * (n & 7))) & 15u;
    b.s0 = s;
    b.s1 = (float)z * s;
  }
}

template <int FMT>
__device__ __forceinline__ uint4 deq_step(const BRaw& b, int s) {
  const uint32_t w = (s == 0) ? b.q.x : (s == 1) ? b.q.y : (s == 2) ? b.q.z : b.q.w;
  if (FMT == FMT_NVFP4) return deq_nvfp4(w, s < 2 ? b.s0 : b.s1);
  if (FMT == FMT_MXFP4) return deq_mxfp4(w, b.s0);
  return deq_gptq(w, b.s0, b.s1);
}

template <int FMT, int EPI, int BM>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(
    const uint16_t* __restrict__ A, int a_div, int n_slots, int K, int N, int E, WeightArgs W,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ expert_ids,
    const int32_t* __restrict__ num_post_pad, const float* __restrict__ topk_w, int mul_tw,
    float alpha, float beta, float limit, uint16_t* __restrict__ out, int out_ld) {
  constexpr int MI = BM / 16;
  __shared__ uint4 As[BM][kLdsRow];

  const int mb = blockIdx.x, nt = blockIdx.y;
  if (mb * BM >= num_post_pad[0]) return;
  const int e = expert_ids[mb];
  if (e < 0 || e >= E) return;  // unused block, or an expert this call does not hold

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int n0w = nt * kBN + wave * kWN;
  int ncol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ncol[j] = (EPI == EPI_SWIGLU) ? n0w + 2 * c16 + j : n0w + 16 * j + c16;
  const bool wave_on = n0w < N;  // N % 32 == 0 when gated, % 16 otherwise
  const bool frag_on[2] = {n0w < N, n0w + 16 < N || (EPI == EPI_SWIGLU && n0w < N)};

  // the A rows this thread stages: rows tid/16 + 16*it, 16-byte segment tid%16
  const int seg = tid & 15;
  const uint16_t* arow[MI];
#pragma unroll
  for (int it = 0; it < MI; ++it) {
    const int sid = sorted_ids[mb * BM + (tid >> 4) + 16 * it];
    arow[it] = (sid < n_slots) ? A + (size_t)(sid / a_div) * K : nullptr;
  }

  f32x4 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    // stage A
#pragma unroll
    for (int it = 0; it < MI; ++it) {
      const int k = k0 + seg * 8;
      uint4 v = {0u, 0u, 0u, 0u};
      if (arow[it] != nullptr && k < K) v = *reinterpret_cast<const uint4*>(arow[it] + k);
      As[(tid >> 4) + 16 * it][seg] = v;
    }
    // fetch this lane's weights for the chunk
    const int kl = k0 + 32 * g;
    BRaw b[2];
    const bool k_on = kl < K;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (frag_on[j] && k_on) {
        load_b<FMT>(b[j], W, e, ncol[j], N, K, kl);
      } else {
        b[j].q = uint4{0u, 0u, 0u, 0u};
        b[j].s0 = 0.f;
        b[j].s1 = 0.f;
      }
    }
    __syncthreads();
    if (wave_on) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 bf[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = as_bf16x8(deq_step<FMT>(b[j], s));
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const bf16x8 af = as_bf16x8(As[i * 16 + c16][g * 4 + s]);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  if (!wave_on) return;

  // epilogue: lane holds rows i*16 + 4g + r, column c16 of fragments 0/1
  const float gsc = (FMT == FMT_NVFP4) ? W.global_scale[e] : 1.f;
  float bias[2] = {0.f, 0.f};
  if (W.bias != nullptr) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (frag_on[j]) bias[j] = bf16_bits_to_f32(W.bias[(size_t)e * N + ncol[j]]);
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sid = sorted_ids[mb * BM + i * 16 + 4 * g + r];
      if (sid >= n_slots) continue;
      uint16_t* orow = out + (size_t)sid * out_ld;
      if (EPI == EPI_SWIGLU) {
        float gate = acc[i][0][r] * gsc + bias[0];
        float up = acc[i][1][r] * gsc + bias[1];
        gate = fminf(gate, limit);
        up = fminf(fmaxf(up, -limit), limit);
        const float a = gate / (1.f + expf(-alpha * gate)) * (up + beta);
        orow[n0w / 2 + c16] = f32_to_bf16_bits(a);
      } else {
        float tw = 1.f;
        if (EPI == EPI_DOWN && mul_tw) tw = topk_w[sid];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (!frag_on[j]) continue;
          float v = acc[i][j][r] * gsc + bias[j];
          if (EPI == EPI_RELU2) {
            v = fmaxf(v, 0.f);
            v = v * v;
          } else if (EPI == EPI_DOWN) {
            v = v * tw;
          }
          orow[ncol[j]] = f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// out[t][:] = sum_j y[t*k + j][:] for valid ids, fp32, j ascending.
__global__ void __launch_bounds__(256) moe_sum_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ ids, int T,
                                                      int top_k, int H, int E,
                                                      uint16_t* __restrict__ out) {
  const int per_row = H / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const int e = ids[(size_t)t * top_k + j];
    if (e < 0 || e >= E) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(y + ((size_t)t * top_k + j) * H + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += __uint_as_float(w[q] << 16);
      acc[2 * q + 1] += __uint_as_float(w[q] & 0xffff0000u);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + c * 8) = o;
}

template <int FMT, int EPI>
static hipError_t launch_bm(int block_m, dim3 grid, hipStream_t st, const uint16_t* A, int a_div,
                            int n_slots, int K, int N, int E, const WeightArgs& W, const int32_t* sid,
                            const int32_t* eid, const int32_t* npp, const float* tw, int mul,
                            float alpha, float beta, float limit, uint16_t* out, int out_ld) {
#define MOE_LAUNCH(BMV)                                                                         \
  grouped_gemm_kernel<FMT, EPI, BMV><<<grid, dim3(256), 0, st>>>(A, a_div, n_slots, K, N, E, W, sid, \
                                                                 eid, npp, tw, mul, alpha, beta, \
                                                                 limit, out, out_ld)
  switch (block_m) {
    case 16: MOE_LAUNCH(16); break;
    case 32: MOE_LAUNCH(32); break;
    case 64: MOE_LAUNCH(64); break;
    default: MOE_LAUNCH(128); break;
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(int epi, int block_m, dim3 grid, hipStream_t st, const uint16_t* A,
                             int a_div, int n_slots, int K, int N, int E, const WeightArgs& W,
                             const int32_t* sid, const int32_t* eid, const int32_t* npp,
                             const float* tw, int mul, float alpha, float beta, float limit,
                             uint16_t* out, int out_ld) {
  switch (epi) {
    case EPI_SWIGLU:
      return launch_bm<FMT, EPI_SWIGLU>(block_m, grid, st, A, a_div, n_slots, K, N, E, W, sid, eid, npp,
                                        tw, mul, alpha, beta, limit, out, out_ld);
    case EPI_RELU2:
      return launch_bm<FMT, EPI_RELU2>(block_m, grid, st, A, a_div, n_slots, K, N, E, W, sid, eid, npp,
                                       tw, mul, alpha, beta, limit, out, out_ld);
    case EPI_NONE:
      return launch_bm<FMT, EPI_NONE>(block_m, grid, st, A, a_div, n_slots, K, N, E, W, sid, eid, npp,
                                      tw, mul, alpha, beta, limit, out, out_ld);
    default:
      return launch_bm<FMT, EPI_DOWN>(block_m, grid, st, A, a_div, n_slots, K, N, E, W, sid, eid, npp,
                                      tw, mul, alpha, beta, limit, out, out_ld);
  }
}

}  // namespace moe

// Launch one grouped GEMM.  cap = capacity of sorted_ids (grid covers every block
// that could be used; blocks past num_post_pad exit at once).
extern "C" hipError_t moe_launch_gemm(int fmt, int epi, int block_m, int cap, const uint16_t* A,
                                      int a_div, int n_slots, int K, int N, int E,
                                      const moe::WeightArgs* W, const int32_t* sid,
                                      const int32_t* eid, const int32_t* npp, const float* tw,
                                      int mul, float alpha, float beta, float limit, uint16_t* out,
                                      int out_ld, hipStream_t st) {
  const dim3 grid(cap / block_m, (N + moe::kBN - 1) / moe::kBN);
  if (grid.x == 0) return hipSuccess;
  switch (fmt) {
    case moe::FMT_NVFP4:
      return moe::launch_fmt<moe::FMT_NVFP4>(epi, block_m, grid, st, A, a_div, n_slots, K, N, E, *W,
                                             sid, eid, npp, tw, mul, alpha, beta, limit, out,
                                             out_ld);
    case moe::FMT_MXFP4:
      return moe::launch_fmt<moe::FMT_MXFP4>(epi, block_m, grid, st, A, a_div, n_slots, K, N, E, *W,
                                             sid, eid, npp, tw, mul, alpha, beta, limit, out,
                                             out_ld);
    default:
      return moe::launch_fmt<moe::FMT_GPTQ>(epi, block_m, grid, st, A, a_div, n_slots, K, N, E, *W,
                                            sid, eid, npp, tw, mul, alpha, beta, limit, out,
                                            out_ld);
  }
}

extern "C" hipError_t moe_launch_sum(const uint16_t* y, const int32_t* ids, int T, int top_k, int H,
                                     int E, uint16_t* out, hipStream_t st) {
  const size_t n = (size_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  moe::moe_sum_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(y, ids, T, top_k, H,
                                                                             E, out);
  return hipGetLastError();
}
