// Top-k routing and the per-expert slot sort (moe_align) for gfx950.
//
// Routing: one wave64 per token.  Each lane holds up to 16 of the token's E
// scores in registers; the k winners are found by k rounds of a wave-wide
// argmax (descending score, ties to the lower expert id), so the selection is
// a pure comparison of float32 scores, identical on every lane.
//   softmax      topk(softmax(logits)) with optional renormalisation
//                ("moe_wna16_marlin_gemm applies wrong per-row topk weights",
//                repro, routing step).
//   sigmoid+bias sigmoid evaluated in double and rounded once to float,
//                score = sigmoid + bias in float, weights = selected unbiased
//                sigmoids renormalised; n_group = 1 makes the grouped top-k a
//                plain top-k (Nemotron-3-Nano page, Analysis item 3).
//
// Align: one workgroup of 1024 threads.  Counts per expert with LDS atomics
// (order-free), pads each count to block_m, and places every slot at
//   offset[e] + (number of earlier slots with the same expert),
// which makes the sort stable and the output unique.  The within-wave rank
// comes from ballots over the bits of the expert id (lanes with an equal id
// share every bit), the cross-wave part from a per-wave count table in LDS.
#include "common.h"

namespace moe {

constexpr int kRouteMaxPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int KIND>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int top_k, const float* __restrict__ ebias,
                                                    int renorm, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + (size_t)t * E;

  float score[kRouteMaxPerLane];  // what selection compares
  float base[kRouteMaxPerLane];   // logit (softmax) or unbiased sigmoid
  float lmax = -INFINITY;
#pragma unroll
  for (int c = 0; c < kRouteMaxPerLane; ++c) {
    const int e = c * 64 + lane;
    float v = -INFINITY, s = -INFINITY;
    if (e < E) {
      const float l = row[e];
      if (KIND == 0) {
        v = l;
        s = l;
        lmax = fmaxf(lmax, l);
      } else {
        v = (float)(1.0 / (1.0 + exp(-(double)l)));
        s = v + ebias[e];
      }
    }
    score[c] = (s != s) ? -INFINITY : s;  // NaN never wins a comparison
    base[c] = v;
  }

  // softmax denominator over all E (fp32; fixed shuffle order -> deterministic)
  float denom = 1.f;
  if (KIND == 0) {
    for (int o = 32; o > 0; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kRouteMaxPerLane; ++c)
      if (c * 64 + lane < E) s += expf(base[c] - lmax);
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    denom = s;
  }

  unsigned taken = 0;  // bit c: entry c of this lane already selected
  int my_id = -1;
  float my_base = 0.f;
  for (int r = 0; r < top_k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < kRouteMaxPerLane; ++c) {
      const int e = c * 64 + lane;
      if (e < E && !((taken >> c) & 1u) && better(score[c], e, bv, bi)) {
        bv = score[c];
        bi = e;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // owner marks it taken and broadcasts the weight basis
    float sel_base = 0.f;
    const int owner = bi & 63, oc = bi >> 6;
#pragma unroll
    for (int c = 0; c < kRouteMaxPerLane; ++c)
      if (c == oc && lane == owner) {
        taken |= 1u << c;
        sel_base = base[c];
      }
    sel_base = __shfl(sel_base, owner);
    if (lane == r) {
      my_id = bi;
      my_base = sel_base;
    }
  }

  float p = 0.f;
  if (lane < top_k) p = (KIND == 0) ? expf(my_base - lmax) / denom : my_base;
  if (renorm) {
    float s = (lane < top_k) ? p : 0.f;
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    p = p / s;
  }
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    w[(size_t)t * top_k + lane] = p;
  }
}

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kAlignMaxE = 1024;

// Exclusive prefix sum of one int per thread over the 1024-thread block.
__device__ int block_exclusive_scan(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wave_tot[wid] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wid; ++i) before += wave_tot[i];
  __syncthreads();
  return before + incl - v;
}

__global__ void __launch_bounds__(kAlignThreads) align_kernel(
    const int32_t* __restrict__ topk_ids, int n_slots, int E, int block_m, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_post_pad) {
  __shared__ int cnt[kAlignMaxE];
  __shared__ int off[kAlignMaxE];
  __shared__ int placed[kAlignMaxE];
  __shared__ int wave_cnt[kAlignWaves][kAlignMaxE];
  __shared__ int wave_tot[kAlignWaves];
  __shared__ int total_s;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;

  for (int e = tid; e < E; e += kAlignThreads) {
    cnt[e] = 0;
    placed[e] = 0;
  }
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) wave_cnt[i / E][i % E] = 0;
  __syncthreads();
  for (int f = tid; f < n_slots; f += kAlignThreads) {
    const int e = topk_ids[f];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // padded segment offsets (E <= 1024: one expert per thread)
  const int my_pad = (tid < E) ? (cnt[tid] + block_m - 1) / block_m * block_m : 0;
  const int my_off = block_exclusive_scan(my_pad, wave_tot);
  if (tid < E) off[tid] = my_off;
  if (tid == E - 1) total_s = my_off + my_pad;
  __syncthreads();
  const int total = total_s;
  if (tid == 0) num_post_pad[0] = total;

  // expert of every block; -1 past the used length
  const int nblocks = cap / block_m;
  if (tid < E) {
    for (int b = my_off / block_m; b < (my_off + my_pad) / block_m; ++b) expert_ids[b] = tid;
  }
  for (int b = total / block_m + tid; b < nblocks; b += kAlignThreads) expert_ids[b] = -1;
  // sentinel in each expert's padding and past the used length
  if (tid < E) {
    for (int i = my_off + cnt[tid]; i < my_off + my_pad; ++i) sorted_ids[i] = n_slots;
  }
  for (int i = total + tid; i < cap; i += kAlignThreads) sorted_ids[i] = n_slots;

  // stable placement, one 1024-slot chunk at a time
  for (int c0 = 0; c0 < n_slots; c0 += kAlignThreads) {
    const int f = c0 + tid;
    int e = (f < n_slots) ? topk_ids[f] : -1;
    const bool valid = (e >= 0 && e < E);
    if (!valid) e = 0;
    unsigned long long same = __ballot(valid);
    for (int bit = 0; bit < 10; ++bit) {
      const unsigned long long m = __ballot((e >> bit) & 1);
      same &= ((e >> bit) & 1) ? m : ~m;
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank_in_wave = __popcll(same & lt);
    const bool leader = valid && ((same >> lane) >> 1) == 0ull;  // last lane of its group
    if (leader) wave_cnt[wid][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int before = placed[e];
      for (int w2 = 0; w2 < wid; ++w2) before += wave_cnt[w2][e];
      sorted_ids[off[e] + before + rank_in_wave] = f;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&placed[e], __popcll(same));
      wave_cnt[wid][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace moe

extern "C" hipError_t moe_launch_route(const float* logits, int T, int E, int top_k, int kind,
                                       const float* ebias, int renorm, int32_t* ids, float* w,
                                       hipStream_t stream) {
  const dim3 grid((T + 3) / 4), block(256);
  if (kind == 0)
    moe::route_kernel<0><<<grid, block, 0, stream>>>(logits, T, E, top_k, ebias, renorm, ids, w);
  else
    moe::route_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, top_k, ebias, renorm, ids, w);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_align(const int32_t* ids, int n_slots, int E, int block_m, int cap,
                                       int32_t* sorted_ids, int32_t* expert_ids, int32_t* npp,
                                       hipStream_t stream) {
  moe::align_kernel<<<1, moe::kAlignThreads, 0, stream>>>(ids, n_slots, E, block_m, cap, sorted_ids,
                                                          expert_ids, npp);
  return hipGetLastError();
}
