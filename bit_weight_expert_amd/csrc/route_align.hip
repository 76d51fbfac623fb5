// Top-k routing and the per-expert slot sort (moe_align) for gfx950.
//
// Routing: one wave64 per token, selection by pure comparison of float32
// scores (descending, ties to the lower expert id), identical on every lane.
//   softmax      topk(softmax(logits)) with optional renormalisation
//                ("moe_wna16_marlin_gemm applies wrong per-row topk weights",
//                repro, routing step).
//   sigmoid+bias sigmoid evaluated in double and rounded once to float,
//                score = sigmoid + bias in float, weights = selected unbiased
//                sigmoids renormalised; n_group = 1 makes the grouped top-k a
//                plain top-k (Nemotron-3-Nano page, Analysis item 3).
// Each lane holds up to 16 scores (E <= 1024; one or two for E <= 128) and
// the k winners come out of k rounds of a wave-wide argmax, in output order.
// The wave-wide max, sum and argmax are butterflies whose first four steps
// are DPP moves inside rows of 16 lanes (a rank count over broadcast scores,
// one v_readlane per expert and score, made each wave a serial chain of ~500
// lane reads at E = 128: 15-24 us per launch).
//
// Align: one workgroup of 1024 threads.  Pads each expert's count to block_m
// and places every slot at
//   offset[e] + (number of earlier slots with the same expert),
// which makes the sort stable and the output unique.  Each wave owns one
// contiguous run of slots and makes two passes over it (count, then place),
// with one block-wide step between them; the within-wave rank comes from
// ballots over the bits of the expert id (lanes with an equal id share every
// bit), the cross-wave part from a per-wave count table in LDS.
//
// For small batches moe_forward runs both in one workgroup (route_align_kernel):
// the routed ids go through LDS straight into the sort, saving a launch.
#include "common.h"

namespace moe {

constexpr int kRouteMaxPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Value held by this lane's partner in step S of a wave-wide all-reduce:
// steps 0, 1 swap lanes within a quad (lane ^ 1, lane ^ 2), steps 2, 3
// mirror within 8 and 16 lanes (each pairs two groups already reduced), all
// four as DPP moves; steps 4, 5 are lane ^ 16 and lane ^ 32.
template <int S>
__device__ __forceinline__ int wave_partner(int v) {
  if (S == 0) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  if (S == 1) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  if (S == 2) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if (S == 3) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  return __shfl_xor(v, S == 4 ? 16 : 32);
}

template <int S>
__device__ __forceinline__ float wave_partner_f(float v) {
  return __int_as_float(wave_partner<S>(__float_as_int(v)));
}

#define MOE_WAVE_STEPS(X) X(0) X(1) X(2) X(3) X(4) X(5)

__device__ __forceinline__ float wave_max(float v) {
#define MOE_STEP(S) v = fmaxf(v, wave_partner_f<S>(v));
  MOE_WAVE_STEPS(MOE_STEP)
#undef MOE_STEP
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#define MOE_STEP(S) v = v + wave_partner_f<S>(v);
  MOE_WAVE_STEPS(MOE_STEP)
#undef MOE_STEP
  return v;
}

// (value, expert id) of the best entry over the wave, on every lane (the
// order of better() is total on distinct ids, so all lanes agree)
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
#define MOE_STEP(S)                                                \
  {                                                                \
    const float ov = wave_partner_f<S>(bv);                        \
    const int oi = wave_partner<S>(bi);                            \
    if (better(ov, oi, bv, bi)) {                                  \
      bv = ov;                                                     \
      bi = oi;                                                     \
    }                                                              \
  }
  MOE_WAVE_STEPS(MOE_STEP)
#undef MOE_STEP
}

// Score used for selection and the weight basis of expert e's logit l.
template <int KIND>
__device__ __forceinline__ void route_score(float l, const float* ebias, int e, float& score,
                                            float& base) {
  if (KIND == 0) {
    score = l;
    base = l;
  } else {
    base = (float)(1.0 / (1.0 + exp(-(double)l)));
    score = base + ebias[e];
  }
  if (score != score) score = -INFINITY;  // NaN never wins a comparison
}

// Route token t with the calling wave.  Writes ids/w[t*top_k + j] (and, if
// lds_ids is not null, the ids to lds_ids[t*top_k + j]).
template <int KIND>
__device__ __forceinline__ void route_wave(const float* __restrict__ logits, int t, int E, int top_k,
                                           const float* __restrict__ ebias, int renorm,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int32_t* lds_ids) {
  const int lane = threadIdx.x & 63;
  const float* row = logits + (size_t)t * E;
  if (E <= 128) {
    // up to two scores per lane: experts lane and lane + 64
    float sc[2], bs[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int e = c * 64 + lane;
      sc[c] = -INFINITY;
      bs[c] = -INFINITY;
      if (e < E) route_score<KIND>(row[e], ebias, e, sc[c], bs[c]);
    }
    // softmax denominator over all E in fp32: per-lane pair sums, then a
    // butterfly (both partners of a step add the same two values, so every
    // lane ends with the same bits)
    float denom = 1.f, lmax = -INFINITY;
    if (KIND == 0) {
      lmax = wave_max(fmaxf(bs[0], bs[1]));
      const float ex0 = (lane < E) ? expf(bs[0] - lmax) : 0.f;
      const float ex1 = (64 + lane < E) ? expf(bs[1] - lmax) : 0.f;
      denom = wave_sum(ex0 + ex1);
    }
    // top_k rounds of a wave-wide argmax: round r finds output position r
    // (the r-th best score, ties to the lower expert id); lane r keeps it
    unsigned taken = 0;  // bit c: entry c of this lane already selected
    int my_id = -1;
    float my_base = 0.f;
    for (int r = 0; r < top_k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int e = c * 64 + lane;
        if (e < E && !((taken >> c) & 1u) && better(sc[c], e, bv, bi)) {
          bv = sc[c];
          bi = e;
        }
      }
      wave_argmax(bv, bi);
      const int win = __builtin_amdgcn_readfirstlane(bi);
      const int owner = win & 63, oc = win >> 6;
      float sel = 0.f;
      if (lane == owner) {
        taken |= 1u << oc;
        sel = oc ? bs[1] : bs[0];
      }
      sel = readlane_f(sel, owner);
      if (lane == r) {
        my_id = win;
        my_base = sel;
      }
    }
    const float p = lane >= top_k ? 0.f : (KIND == 0) ? expf(my_base - lmax) / denom : my_base;
    float norm = 1.f;
    if (renorm) {
      // sum in output order (position 0 .. k-1)
      float s = 0.f;
      for (int r = 0; r < top_k; ++r) s += readlane_f(p, r);
      norm = s;
    }
    if (lane < top_k) {
      const size_t f = (size_t)t * top_k + lane;
      ids[f] = my_id;
      w[f] = renorm ? p / norm : p;
      if (lds_ids != nullptr) lds_ids[f] = my_id;
    }
    return;
  }

  float score[kRouteMaxPerLane];  // what selection compares
  float base[kRouteMaxPerLane];   // logit (softmax) or unbiased sigmoid
  float lmax = -INFINITY;
#pragma unroll
  for (int c = 0; c < kRouteMaxPerLane; ++c) {
    const int e = c * 64 + lane;
    float s = -INFINITY, v = -INFINITY;
    if (e < E) {
      route_score<KIND>(row[e], ebias, e, s, v);
      if (KIND == 0) lmax = fmaxf(lmax, v);
    }
    score[c] = s;
    base[c] = v;
  }

  // softmax denominator over all E (fp32; fixed butterfly -> deterministic)
  float denom = 1.f;
  if (KIND == 0) {
    lmax = wave_max(lmax);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kRouteMaxPerLane; ++c)
      if (c * 64 + lane < E) s += expf(base[c] - lmax);
    denom = wave_sum(s);
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
    wave_argmax(bv, bi);
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
    const size_t f = (size_t)t * top_k + lane;
    ids[f] = my_id;
    w[f] = p;
    if (lds_ids != nullptr) lds_ids[f] = my_id;
  }
}

template <int KIND>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int top_k, const float* __restrict__ ebias,
                                                    int renorm, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  route_wave<KIND>(logits, t, E, top_k, ebias, renorm, ids, w, nullptr);
}

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kAlignMaxE = 1024;

// LDS of the sort.
struct AlignLds {
  int wave_cnt[kAlignWaves][kAlignMaxE];  // per-wave counts, then per-wave cursors
  int wave_tot[kAlignWaves];
  int total;
};

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

constexpr int kIdBatch = 8;  // 64-slot groups whose ids are loaded together

// Lanes of this wave holding the same expert id as this lane (ballots over
// the id's nbits bits), among the lanes where `valid` holds.
__device__ __forceinline__ unsigned long long match_expert(int e, bool valid, int nbits) {
  unsigned long long same = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const unsigned long long m = __ballot((e >> bit) & 1);
    same &= ((e >> bit) & 1) ? m : ~m;
  }
  return same;
}

// Run of slots [s0, s1) that wave `wid` owns inside a workgroup's range [r0, r1).
__device__ __forceinline__ void wave_run(int r0, int r1, int wid, int& s0, int& s1) {
  const int run = ((r1 - r0 + kAlignWaves - 1) / kAlignWaves + 63) / 64 * 64;
  s0 = min(r0 + wid * run, r1);
  s1 = min(s0 + run, r1);
}

// Pass 1: the wave counts its run per expert into its own LDS row (per
// 64-slot group one lane per expert adds the group's count, so no atomics).
// Ids are loaded kIdBatch groups at a time (one memory latency per batch).
__device__ __forceinline__ void count_run(const int32_t* topk_ids, int s0, int s1, int E, int nbits,
                                          int* row) {
  const int lane = threadIdx.x & 63;
  for (int b0 = s0; b0 < s1; b0 += 64 * kIdBatch) {
    int ev[kIdBatch];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int f = b0 + 64 * u + lane;
      ev[u] = (f < s1) ? topk_ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      if (b0 + 64 * u >= s1) break;  // past the run (uniform over the wave)
      int e = ev[u];
      const bool valid = (e >= 0 && e < E);
      if (!valid) e = 0;
      const unsigned long long same = match_expert(e, valid, nbits);
      if (valid && ((same >> lane) >> 1) == 0ull) row[e] += __popcll(same);  // last lane of its group
    }
  }
}

// Pass 2: the wave walks its run again and places each slot at its expert's
// cursor plus its rank among the group's lanes of that expert.  The cursor is
// read by every lane of a group before the group's last lane advances it (one
// wave's LDS accesses stay in order).
__device__ __forceinline__ void place_run(const int32_t* topk_ids, int s0, int s1, int E, int nbits,
                                          int* cursor, int32_t* __restrict__ sorted_ids) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = s0; b0 < s1; b0 += 64 * kIdBatch) {
    int ev[kIdBatch];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int f = b0 + 64 * u + lane;
      ev[u] = (f < s1) ? topk_ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      if (b0 + 64 * u >= s1) break;  // past the run (uniform over the wave)
      const int f = b0 + 64 * u + lane;
      int e = ev[u];
      const bool valid = (e >= 0 && e < E);
      if (!valid) e = 0;
      const unsigned long long same = match_expert(e, valid, nbits);
      const int at = cursor[e];
      if (valid) sorted_ids[at + __popcll(same & lt)] = f;
      if (valid && ((same >> lane) >> 1) == 0ull) cursor[e] = at + __popcll(same);
    }
  }
}

// Expert of every block (-1 past the used length) and the sentinel in each
// expert's padding and past the used length; thread e < E holds expert e's
// padded offset, count and padded count.
__device__ __forceinline__ void align_tables(int n_slots, int E, int block_m, int cap, int total,
                                             int my_off, int my_cnt, int my_pad,
                                             int32_t* __restrict__ sorted_ids,
                                             int32_t* __restrict__ expert_ids,
                                             int32_t* __restrict__ num_post_pad) {
  const int tid = threadIdx.x;
  if (tid == 0) num_post_pad[0] = total;
  const int nblocks = cap / block_m;
  if (tid < E) {
    for (int b = my_off / block_m; b < (my_off + my_pad) / block_m; ++b) expert_ids[b] = tid;
  }
  for (int b = total / block_m + tid; b < nblocks; b += kAlignThreads) expert_ids[b] = -1;
  if (tid < E) {
    for (int i = my_off + my_cnt; i < my_off + my_pad; ++i) sorted_ids[i] = n_slots;
  }
  for (int i = total + tid; i < cap; i += kAlignThreads) sorted_ids[i] = n_slots;
}

// The sort itself, for the whole 1024-thread workgroup; topk_ids may point to
// global memory or to LDS.  Each of the 16 waves owns one contiguous run of
// slots: pass 1 counts it, then per expert the total, the padded segment
// offsets (a block scan) and, in wave order, where each wave's share of the
// segment starts; pass 2 places.  Runs are in wave order and groups in slot
// order, so equal experts keep slot order.
__device__ __forceinline__ void align_block(const int32_t* topk_ids, int n_slots, int E, int block_m,
                                            int cap, int32_t* __restrict__ sorted_ids,
                                            int32_t* __restrict__ expert_ids,
                                            int32_t* __restrict__ num_post_pad, AlignLds& L) {
  const int tid = threadIdx.x, wid = tid >> 6;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  int s0, s1;
  wave_run(0, n_slots, wid, s0, s1);

  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) L.wave_cnt[i / E][i % E] = 0;
  __syncthreads();
  count_run(topk_ids, s0, s1, E, nbits, L.wave_cnt[wid]);
  __syncthreads();

  // per expert (E <= 1024: one per thread): count, padded segment offsets
  int my_cnt = 0;
  if (tid < E)
    for (int w = 0; w < kAlignWaves; ++w) my_cnt += L.wave_cnt[w][tid];
  const int my_pad = (tid < E) ? (my_cnt + block_m - 1) / block_m * block_m : 0;
  const int my_off = block_exclusive_scan(my_pad, L.wave_tot);
  if (tid == E - 1) L.total = my_off + my_pad;
  if (tid < E) {
    // each wave's share of the segment starts after the earlier waves' shares
    int at = my_off;
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = L.wave_cnt[w][tid];
      L.wave_cnt[w][tid] = at;
      at += c;
    }
  }
  __syncthreads();
  align_tables(n_slots, E, block_m, cap, L.total, my_off, my_cnt, my_pad, sorted_ids, expert_ids,
               num_post_pad);
  place_run(topk_ids, s0, s1, E, nbits, L.wave_cnt[wid], sorted_ids);
}

__global__ void __launch_bounds__(kAlignThreads) align_kernel(
    const int32_t* __restrict__ topk_ids, int n_slots, int E, int block_m, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_post_pad) {
  __shared__ AlignLds L;
  align_block(topk_ids, n_slots, E, block_m, cap, sorted_ids, expert_ids, num_post_pad, L);
}

// The same sort over kAlignGroups workgroups for large batches: workgroup g
// owns the g-th contiguous range of slots (its 16 waves a run each).  The
// count launch writes each workgroup's per-expert counts to counts[g][E]; the
// place launch re-counts its range per wave, adds the earlier workgroups'
// counts from the table to each cursor and places; workgroup 0 also writes
// the block table, the sentinels and the padded length.  Same output as the
// single workgroup (slot order is kept across ranges, waves and groups).
__device__ __forceinline__ void group_range(int n_slots, int g, int& r0, int& r1) {
  const int R = ((n_slots + kAlignGroups - 1) / kAlignGroups + 63) / 64 * 64;
  r0 = min(g * R, n_slots);
  r1 = min(r0 + R, n_slots);
}

__global__ void __launch_bounds__(kAlignThreads) align_count_kernel(
    const int32_t* __restrict__ topk_ids, int n_slots, int E, int32_t* __restrict__ counts) {
  __shared__ AlignLds L;
  const int tid = threadIdx.x, wid = tid >> 6, g = blockIdx.x;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  int r0, r1, s0, s1;
  group_range(n_slots, g, r0, r1);
  wave_run(r0, r1, wid, s0, s1);
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) L.wave_cnt[i / E][i % E] = 0;
  __syncthreads();
  count_run(topk_ids, s0, s1, E, nbits, L.wave_cnt[wid]);
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    int c = 0;
    for (int w = 0; w < kAlignWaves; ++w) c += L.wave_cnt[w][e];
    counts[g * E + e] = c;
  }
}

__global__ void __launch_bounds__(kAlignThreads) align_place_kernel(
    const int32_t* __restrict__ topk_ids, int n_slots, int E, int block_m, int cap,
    const int32_t* __restrict__ counts, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ num_post_pad) {
  __shared__ AlignLds L;
  const int tid = threadIdx.x, wid = tid >> 6, g = blockIdx.x;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  int r0, r1, s0, s1;
  group_range(n_slots, g, r0, r1);
  wave_run(r0, r1, wid, s0, s1);
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) L.wave_cnt[i / E][i % E] = 0;
  __syncthreads();
  count_run(topk_ids, s0, s1, E, nbits, L.wave_cnt[wid]);
  // per expert: total over all ranges, and the count of the ranges before g
  int my_cnt = 0, before = 0;
  if (tid < E) {
    for (int h = 0; h < kAlignGroups; ++h) {
      const int c = counts[h * E + tid];
      my_cnt += c;
      before += h < g ? c : 0;
    }
  }
  const int my_pad = (tid < E) ? (my_cnt + block_m - 1) / block_m * block_m : 0;
  const int my_off = block_exclusive_scan(my_pad, L.wave_tot);  // (its barriers order pass 1 too)
  if (tid == E - 1) L.total = my_off + my_pad;
  if (tid < E) {
    int at = my_off + before;
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = L.wave_cnt[w][tid];
      L.wave_cnt[w][tid] = at;
      at += c;
    }
  }
  __syncthreads();
  if (g == 0)
    align_tables(n_slots, E, block_m, cap, L.total, my_off, my_cnt, my_pad, sorted_ids, expert_ids,
                 num_post_pad);
  place_run(topk_ids, s0, s1, E, nbits, L.wave_cnt[wid], sorted_ids);
}

// Routing and the sort in one workgroup (small batches): the 16 waves route
// tokens wave, wave + 16, ...; the ids reach the sort through LDS.
constexpr int kFusedMaxSlots = 4096;

template <int KIND>
__global__ void __launch_bounds__(kAlignThreads) route_align_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, const float* __restrict__ ebias,
    int renorm, int32_t* __restrict__ ids, float* __restrict__ w, int block_m, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_post_pad) {
  __shared__ AlignLds L;
  __shared__ int32_t lds_ids[kFusedMaxSlots];
  for (int t = threadIdx.x >> 6; t < T; t += kAlignWaves)
    route_wave<KIND>(logits, t, E, top_k, ebias, renorm, ids, w, lds_ids);
  __syncthreads();
  align_block(lds_ids, T * top_k, E, block_m, cap, sorted_ids, expert_ids, num_post_pad, L);
}

// Route + align for at most 16 tokens, 64 slots and 128 experts in one small
// workgroup (one wave per token): each wave routes its token (ids into LDS),
// then wave 0 sorts with one slot per lane -- equal ids found by ballots over the id
// bits (lanes with an equal id agree on every bit), each group's last lane
// writes its expert's count, the padded offsets are one wave-wide scan over
// the experts (two per lane), and each slot lands at its expert's offset plus
// its rank among the lanes of its group, which are in slot order.  Same
// outputs as route_kernel + align_kernel, bit for bit (the routing is the same
// code; the sort's result is unique).
constexpr int kSmallSlots = 64;
constexpr int kSmallMaxE = 128;

template <int KIND>
__global__ void __launch_bounds__(1024) route_align_small_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, const float* __restrict__ ebias,
    int renorm, int32_t* __restrict__ ids, float* __restrict__ w, int block_m, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_post_pad) {
  __shared__ int32_t lds_ids[kSmallSlots];
  __shared__ int32_t cnt[kSmallMaxE];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (wid < T) route_wave<KIND>(logits, wid, E, top_k, ebias, renorm, ids, w, lds_ids);
  if (wid == 0) {
    cnt[lane] = 0;
    cnt[lane + 64] = 0;
  }
  __syncthreads();
  if (wid != 0) return;
  const int n = T * top_k;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  int e = lane < n ? lds_ids[lane] : -1;
  const bool valid = e >= 0 && e < E;
  if (!valid) e = 0;
  const unsigned long long same = match_expert(e, valid, nbits);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & lt);
  if (valid && ((same >> lane) >> 1) == 0ull) cnt[e] = __popcll(same);  // group's last lane
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the counts are in LDS
  // experts lane and lane + 64: padded counts, exclusive offsets in expert order
  const int c0 = lane < E ? cnt[lane] : 0, c1 = lane + 64 < E ? cnt[lane + 64] : 0;
  const int p0 = (c0 + block_m - 1) / block_m * block_m, p1 = (c1 + block_m - 1) / block_m * block_m;
  int i0 = p0, i1 = p1;
  for (int o = 1; o < 64; o <<= 1) {
    const int u0 = __shfl_up(i0, o), u1 = __shfl_up(i1, o);
    if (lane >= o) {
      i0 += u0;
      i1 += u1;
    }
  }
  const int tot0 = __shfl(i0, 63);
  const int off0 = i0 - p0, off1 = tot0 + i1 - p1;
  const int total = tot0 + __shfl(i1, 63);
  __builtin_amdgcn_wave_barrier();
  cnt[lane] = off0;  // the counts are read; the table now holds offsets
  cnt[lane + 64] = off1;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xc07f);
  if (lane < n && valid) sorted_ids[cnt[e] + rank] = lane;
  // per expert (two per lane): block table, sentinels in the padding
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ex = lane + 64 * h;
    const int c = h ? c1 : c0, p = h ? p1 : p0, off = h ? off1 : off0;
    if (ex < E && p > 0) {
      for (int b = off / block_m; b < (off + p) / block_m; ++b) expert_ids[b] = ex;
      for (int i = off + c; i < off + p; ++i) sorted_ids[i] = n;
    }
  }
  for (int b = total / block_m + lane; b < cap / block_m; b += 64) expert_ids[b] = -1;
  for (int i = total + lane; i < cap; i += 64) sorted_ids[i] = n;
  if (lane == 0) num_post_pad[0] = total;
}

// Tile plan of the mixed tiling (uneven slots per expert): over the aligned
// blocks of bs rows (16, 32 or 64), every
// expert's first floor(blocks * bs / 128) runs of 128 rows become tiles of
// the streaming kernel, listed as (first row, expert) in block order (the
// last run may end in the expert's padding rows); the other blocks keep
// their expert in dec_eids for the kernel of bs-row blocks, the listed ones get -1
// there.  One workgroup; the block table (sorted by expert, -1 past the used
// length) is staged in LDS and each block finds its expert's run by binary
// search.  tiles has room for nblocks * bs / 128 entries; n_tiles[0] = their
// number.
constexpr int kPlanMaxBlocks = 4096;

__global__ void __launch_bounds__(kAlignThreads) tile_plan_kernel(
    const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ num_post_pad, int bs,
    int nblocks, int32_t* __restrict__ dec_eids, int2* __restrict__ tiles,
    int32_t* __restrict__ n_tiles) {
  __shared__ int32_t eid[kPlanMaxBlocks];
  __shared__ int wave_tot[kAlignWaves];
  __shared__ int running;
  const int tid = threadIdx.x;
  const int nb = min(num_post_pad[0] / bs, nblocks);  // blocks in use
  const int per = 128 / bs;                           // blocks per tile
  for (int b = tid; b < nb; b += kAlignThreads) eid[b] = expert_ids[b];
  __syncthreads();
  int carry = 0;
  for (int b0 = 0; b0 < nblocks; b0 += kAlignThreads) {
    const int b = b0 + tid;
    int e = -1;
    bool first = false, covered = false;
    if (b < nb) {
      e = eid[b];
      int lo = 0, hi = b;  // first block of expert e
      while (lo < hi) {
        const int m = (lo + hi) >> 1;
        if (eid[m] < e) lo = m + 1; else hi = m;
      }
      const int start = lo;
      lo = b + 1;
      hi = nb;  // one past its last block
      while (lo < hi) {
        const int m = (lo + hi) >> 1;
        if (eid[m] <= e) lo = m + 1; else hi = m;
      }
      const int full = (lo - start) / per * per;
      covered = b - start < full;
      first = covered && (b - start) % per == 0;
    }
    if (b < nblocks) dec_eids[b] = covered ? -1 : (b < nb ? e : -1);
    const int pos = carry + block_exclusive_scan(first ? 1 : 0, wave_tot);
    if (first) tiles[pos] = int2{b * bs, e};
    // the last thread's position plus its own flag is the running count
    if (tid == kAlignThreads - 1) running = pos + (first ? 1 : 0);
    __syncthreads();
    carry = running;
    __syncthreads();
  }
  if (tid == 0) n_tiles[0] = carry;
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

extern "C" hipError_t moe_launch_align_large(const int32_t* ids, int n_slots, int E, int block_m,
                                             int cap, int32_t* counts, int32_t* sorted_ids,
                                             int32_t* expert_ids, int32_t* npp, hipStream_t stream) {
  moe::align_count_kernel<<<moe::kAlignGroups, moe::kAlignThreads, 0, stream>>>(ids, n_slots, E, counts);
  moe::align_place_kernel<<<moe::kAlignGroups, moe::kAlignThreads, 0, stream>>>(
      ids, n_slots, E, block_m, cap, counts, sorted_ids, expert_ids, npp);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_align(const int32_t* ids, int n_slots, int E, int block_m, int cap,
                                       int32_t* sorted_ids, int32_t* expert_ids, int32_t* npp,
                                       hipStream_t stream) {
  moe::align_kernel<<<1, moe::kAlignThreads, 0, stream>>>(ids, n_slots, E, block_m, cap, sorted_ids,
                                                          expert_ids, npp);
  return hipGetLastError();
}

// Route + align in one launch for at most one token per wave of the fused
// workgroup (measured: 8.7 us instead of 8.3 + 4.6 at one token; at 64 tokens
// the single workgroup's serial routing takes 31 us against 10 + 5 for the
// two kernels); otherwise the two kernels.  Returns what the launches return.
extern "C" hipError_t moe_launch_route_align(const float* logits, int T, int E, int top_k, int kind,
                                             const float* ebias, int renorm, int32_t* ids, float* w,
                                             int block_m, int cap, int32_t* sorted_ids,
                                             int32_t* expert_ids, int32_t* npp,
                                             hipStream_t stream) {
  if (T <= moe::kAlignWaves && T * top_k <= moe::kSmallSlots && E <= moe::kSmallMaxE) {
    const dim3 block(64 * T);  // one wave per token
    if (kind == 0)
      moe::route_align_small_kernel<0><<<1, block, 0, stream>>>(
          logits, T, E, top_k, ebias, renorm, ids, w, block_m, cap, sorted_ids, expert_ids, npp);
    else
      moe::route_align_small_kernel<1><<<1, block, 0, stream>>>(
          logits, T, E, top_k, ebias, renorm, ids, w, block_m, cap, sorted_ids, expert_ids, npp);
    return hipGetLastError();
  }
  if (T <= moe::kAlignWaves && T * top_k <= moe::kFusedMaxSlots) {
    if (kind == 0)
      moe::route_align_kernel<0><<<1, moe::kAlignThreads, 0, stream>>>(
          logits, T, E, top_k, ebias, renorm, ids, w, block_m, cap, sorted_ids, expert_ids, npp);
    else
      moe::route_align_kernel<1><<<1, moe::kAlignThreads, 0, stream>>>(
          logits, T, E, top_k, ebias, renorm, ids, w, block_m, cap, sorted_ids, expert_ids, npp);
    return hipGetLastError();
  }
  hipError_t e = moe_launch_route(logits, T, E, top_k, kind, ebias, renorm, ids, w, stream);
  if (e == hipSuccess) e = moe_launch_align(ids, T * top_k, E, block_m, cap, sorted_ids, expert_ids, npp, stream);
  return e;
}

// Tile plan of the mixed tiling (tile_plan_kernel); nblocks <= 4096.
extern "C" hipError_t moe_launch_tile_plan(const int32_t* expert_ids, const int32_t* npp, int bs,
                                           int nblocks, int32_t* dec_eids, int2* tiles,
                                           int32_t* n_tiles, hipStream_t stream) {
  if (nblocks > moe::kPlanMaxBlocks || (bs != 16 && bs != 32 && bs != 64)) return hipErrorInvalidValue;
  moe::tile_plan_kernel<<<1, moe::kAlignThreads, 0, stream>>>(expert_ids, npp, bs, nblocks, dec_eids,
                                                             tiles, n_tiles);
  return hipGetLastError();
}
