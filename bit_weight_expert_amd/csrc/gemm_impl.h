#pragma once
// Grouped W4A16 GEMMs (GEMM1 with the gate/up weights, GEMM2 with the down
// weights) for gfx950: the kernels and their launch rules.
//
// Both GEMMs run over the aligned blocks of moe_align: block b holds up to
// BM sorted slots that all route to expert e = expert_ids[b] ("moe_align_block_size"
// in the NVFP4 repro); its A rows are x[sorted_id / top_k] for GEMM1 and the
// intermediate row of the slot itself for GEMM2 (the top_k = 1 view).
//
// Three kernels share the weight decoders and the routing-weight epilogue rule:
//   prefill  many rows per expert (blocks of 64/128 slots).  Workgroup = BM
//            rows x 256 weight rows; four waves split the weight rows, so
//            every weight is dequantised once per workgroup.  A rows and the
//            4-bit codes stream through a 4-deep LDS ring filled by gfx950
//            LDS-DMA, the tile's scales for the whole K sit in LDS, MFMA is
//            v_mfma_f32_32x32x16_bf16 (details at the kernel).
//   wide     a few to a few dozen rows per expert (blocks of 16/32 slots)
//            when (block, 128-column tile) pairs fill the chip: four waves
//            of 32 columns over the whole K share each A chunk through LDS,
//            the codes stream per wave through a register ring (details at
//            the kernel).
//   decode   a few rows per expert and too few tiles for the wide kernel:
//            Workgroup = 16*MI rows x 16*NF columns with v_mfma_f32_16x16x32:
//            lane l works on column l%16 of a 16-column fragment and on
//            k-group g = l/16; each wave owns one or more 256-wide K chunks
//            (up to 12 waves for one row block, 8 for two), reads its codes
//            and A straight from global memory, and the waves add their
//            partial sums through LDS in wave order (deterministic); the
//            epilogue is then spread over the waves.
// Both handle K tails exactly (K need only be a multiple of 32; no MFMA step
// is spent on padding) and N tails per fragment: no padded buffer is read or
// written (hidden 2880 = 45*64 = 11*256 + 64).
//
// Dequantisation:
//   NVFP4  e2m1 -> f32 with the gfx950 fp4 convert (unit scale), times the
//          e4m3 block scale in f32, packed to bf16 (exact: 2 x 4 significant
//          bits); the per-expert global scale multiplies the fp32 result.
//   MXFP4  the fp4 -> bf16 convert applies the e8m0 power of two itself.
//   GPTQ   (q - z) * s evaluated exactly in f32 as fma(q, s, -z*s), then
//          rounded once to bf16.
//
// Epilogues.  GEMM1: + bias, then swigluoai over the (gate, up) pair -- a
// wave's fragments 2j and 2j+1 hold weight rows 2c and 2c+1 of the same pair,
// so the pair meets in one lane -- or ReLU^2, or nothing.  GEMM2:
// (acc * global + bias) * topk_w[sorted_id]: the routing weight is looked up
// with the very slot id the row is stored under (the bug on
// "moe_wna16_marlin_gemm applies wrong per-row topk weights" was an epilogue
// row index that did not match the slot the weight belonged to).
#include <type_traits>

#include "common.h"

namespace moe {

// --------------------------------------------------------------------------
// weight chunk of one lane for one 16-column fragment
// --------------------------------------------------------------------------

template <int FMT, int C>
struct BChunk {
  static constexpr int kSteps = C / 32;  // MFMA steps (8 k each) in the lane's C/4 range
  // raw scale words exactly as loaded (decoded only when a step uses them, so
  // a prefetched chunk never makes the wave wait for its loads early):
  //   NVFP4  C=256: two u16 (4 group scales); C=128: one u16; else one u8
  //   MXFP4  C=256: two u8 (2 group scales); else one u8
  //   GPTQ   [0] = fp16 scale bits, [1] = the packed zero-point word
  static constexpr int kRaw = FMT == FMT_GPTQ ? 2 : (C == 256 ? 2 : 1);
  uint32_t q[kSteps];
  uint32_t sr[kRaw];
  int zsh;  // GPTQ: bit offset of this column's zero point in sr[1]
};

// Scale operand of the fp4 -> bf16 convert for an e8m0 byte: the byte in the
// fp32 exponent field.  The convert applies only that field, read as e8m0 (so
// in-bounds probes on gfx950 found): byte 0x00 (a float 0) scales by 2^-127,
// giving exact bf16 subnormals, and 0xFF (a float infinity) gives NaN, the
// OCP decode of both bytes.
__device__ __forceinline__ float e8m0_operand(uint32_t byte) {
  return __uint_as_float((byte & 0xffu) << 23);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

template <int FMT, int C>
__device__ __forceinline__ void zero_chunk(BChunk<FMT, C>& b) {
#pragma unroll
  for (int i = 0; i < BChunk<FMT, C>::kSteps; ++i) b.q[i] = 0u;
#pragma unroll
  for (int i = 0; i < BChunk<FMT, C>::kRaw; ++i) b.sr[i] = 0u;
  b.zsh = 0;
}

// Codes and scale bytes of weight row n of expert e from k = kl on (NVFP4 and
// MXFP4), in whichever layout the family holds: the checkpoint rows ([E][N][K/2]
// codes, [E][N][K/G] scales) or the copies by K chunk ([E][KC][N][CH/2] codes,
// [E][KC][N][4] scales, CH = 64 for NVFP4 and 128 for MXFP4, KC = ceil(K/CH)).
// A lane's range never crosses a chunk: it is at most 64 deep and aligned.
template <int FMT>
__device__ __forceinline__ const uint8_t* codes_at(const WeightArgs& W, int e, int n, int N, int K,
                                                   int kl) {
  if (W.qweight_kc != nullptr) {
    constexpr int CH = FMT == FMT_NVFP4 ? 64 : 128;
    const int kcn = (K + CH - 1) / CH;
    return W.qweight_kc + (((size_t)e * kcn + kl / CH) * N + n) * (CH / 2) + (kl % CH) / 2;
  }
  return W.qweight + ((size_t)e * N + n) * (size_t)(K / 2) + kl / 2;
}
template <int FMT>
__device__ __forceinline__ const uint8_t* scales_at(const WeightArgs& W, int e, int n, int N, int K,
                                                    int kl) {
  constexpr int G = FMT == FMT_NVFP4 ? 16 : 32;
  if (W.scales_kc != nullptr) {
    constexpr int CH = 4 * G;
    const int kcn = (K + CH - 1) / CH;
    return W.scales_kc + (((size_t)e * kcn + kl / CH) * N + n) * 4 + (kl % CH) / G;
  }
  return W.scales + ((size_t)e * N + n) * (size_t)(K / G) + kl / G;
}

// Load the lane's k range [kl, kl + C/4) of weight row n of expert e.
template <int FMT, int C>
__device__ __forceinline__ void load_chunk(BChunk<FMT, C>& b, const WeightArgs& W, int e, int n,
                                           int N, int K, int kl) {
  constexpr int S = BChunk<FMT, C>::kSteps;
  if (FMT == FMT_NVFP4 || FMT == FMT_MXFP4) {
    const uint8_t* p = codes_at<FMT>(W, e, n, N, K, kl);
    if (S >= 4) {
#pragma unroll
      for (int v = 0; v < S / 4; ++v) {
        const uint4 t = *reinterpret_cast<const uint4*>(p + 16 * v);
        b.q[4 * v] = t.x;
        b.q[4 * v + 1] = t.y;
        b.q[4 * v + 2] = t.z;
        b.q[4 * v + 3] = t.w;
      }
    } else if (S == 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(p);
      b.q[0] = t.x;
      b.q[1] = t.y;
    } else {
      b.q[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    const uint8_t* sp = scales_at<FMT>(W, e, n, N, K, kl);
    if (FMT == FMT_NVFP4) {
      // K % 32 == 0 makes K/16 even, so scale pairs are 2-byte aligned
      if (C == 256) {
        b.sr[0] = *reinterpret_cast<const uint16_t*>(sp);
        b.sr[1] = *reinterpret_cast<const uint16_t*>(sp + 2);
      } else if (C == 128) {
        b.sr[0] = *reinterpret_cast<const uint16_t*>(sp);
      } else {
        b.sr[0] = *sp;
      }
    } else {
      b.sr[0] = sp[0];
      if (C == 256) b.sr[1] = sp[1];
    }
  } else {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(W.qweight);
    const size_t base = ((size_t)e * (K / 8) + kl / 8) * N + n;
#pragma unroll
    for (int i = 0; i < S; ++i) b.q[i] = qw[base + (size_t)i * N];
    const size_t gi = (size_t)e * (K / W.group) + kl / W.group;
    b.sr[0] = reinterpret_cast<const uint16_t*>(W.scales)[gi * N + n];
    b.sr[1] = W.zeros[gi * (N / 8) + n / 8];
    b.zsh = 4 * (n & 7);
  }
}

// The codes part of load_chunk only (the raw scale words are filled separately).
template <int FMT, int C>
__device__ __forceinline__ void load_codes(BChunk<FMT, C>& b, const WeightArgs& W, int e, int n,
                                           int N, int K, int kl) {
  constexpr int S = BChunk<FMT, C>::kSteps;
  if (FMT == FMT_NVFP4 || FMT == FMT_MXFP4) {
    const uint8_t* p = codes_at<FMT>(W, e, n, N, K, kl);
    if (S >= 4) {
#pragma unroll
      for (int v = 0; v < S / 4; ++v) {
        const uint4 t = *reinterpret_cast<const uint4*>(p + 16 * v);
        b.q[4 * v] = t.x;
        b.q[4 * v + 1] = t.y;
        b.q[4 * v + 2] = t.z;
        b.q[4 * v + 3] = t.w;
      }
    } else if (S == 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(p);
      b.q[0] = t.x;
      b.q[1] = t.y;
    } else {
      b.q[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  } else {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(W.qweight);
    const size_t base = ((size_t)e * (K / 8) + kl / 8) * N + n;
#pragma unroll
    for (int i = 0; i < S; ++i) b.q[i] = qw[base + (size_t)i * N];
  }
}

// 8 dequantised bf16 weights of MFMA step st.
// Eight GPTQ codes of one word (code i in bits 4i .. 4i+3) as code * s + zs.
// The even codes are masked into the word's four bytes and the odd ones
// shifted there first.  A byte 0..15 read as e4m3 is that integer times 2^-9
// (subnormals up to 7, then the first binade), so one scaled fp8 convert
// with scale 2^9 turns two bytes into two exact integer floats; the products
// are exact in fp32.  (The masks are opaque to the compiler: knowing the
// bits of lo and hi, it would fold each byte read back into a nibble extract.)
__device__ __forceinline__ void gptq_deq8(uint32_t w, float s, float zs, float (&v)[8]) {
  uint32_t lo, hi;
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w));
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w >> 4));
  const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, false);  // codes 0, 2
  const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, true);   // codes 4, 6
  const f32x2 o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, false);  // codes 1, 3
  const f32x2 o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, true);   // codes 5, 7
  v[0] = fmaf(e0[0], s, zs);
  v[1] = fmaf(o0[0], s, zs);
  v[2] = fmaf(e0[1], s, zs);
  v[3] = fmaf(o0[1], s, zs);
  v[4] = fmaf(e1[0], s, zs);
  v[5] = fmaf(o1[0], s, zs);
  v[6] = fmaf(e1[1], s, zs);
  v[7] = fmaf(o1[1], s, zs);
}

template <int FMT, int C>
__device__ __forceinline__ bf16x8 deq_step(const BChunk<FMT, C>& b, int st) {
  const uint32_t w = b.q[st];
  uint4 r;
  if (FMT == FMT_NVFP4) {
    const int grp = (st * 8) / 16;  // 16-k group inside the lane's range
    const uint32_t raw = (C == 256) ? b.sr[grp >> 1] : b.sr[0];
    const float s = (grp & 1) ? __builtin_amdgcn_cvt_f32_fp8((int)raw, 1)
                              : __builtin_amdgcn_cvt_f32_fp8((int)raw, 0);
    f32x2 p;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    r.x = pack_bf16x2(p[0] * s, p[1] * s);
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    r.y = pack_bf16x2(p[0] * s, p[1] * s);
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    r.z = pack_bf16x2(p[0] * s, p[1] * s);
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    r.w = pack_bf16x2(p[0] * s, p[1] * s);
  } else if (FMT == FMT_MXFP4) {
    const int grp = (st * 8) / 32;
    const uint32_t raw = (C == 256) ? b.sr[grp] : b.sr[0];
    const float s = e8m0_operand(raw);
    bf16x2 p;
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    __builtin_memcpy(&r.x, &p, 4);
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    __builtin_memcpy(&r.y, &p, 4);
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    __builtin_memcpy(&r.z, &p, 4);
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    __builtin_memcpy(&r.w, &p, 4);
  } else {
    const float s = half_bits_to_f32((uint16_t)b.sr[0]);
    const float zs = (float)((b.sr[1] >> b.zsh) & 15u) * s;
    float v[8];
    gptq_deq8(w, s, -zs, v);
    r.x = pack_bf16x2(v[0], v[1]);
    r.y = pack_bf16x2(v[2], v[3]);
    r.z = pack_bf16x2(v[4], v[5]);
    r.w = pack_bf16x2(v[6], v[7]);
  }
  bf16x8 o;
  __builtin_memcpy(&o, &r, 16);
  return o;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// sigmoid(x) with the hardware exp2 and reciprocal (about 1 ulp each; the result
// is rounded to bf16 afterwards).  x -> -inf gives 0, x -> +inf gives 1.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// The activations of the GEMM1 epilogue.  The clamps are selects, not
// fminf/fmaxf: those return the other operand when one is NaN, which would
// turn a NaN pre-activation (a NaN scale, say) into a finite output.  Here a
// NaN stays NaN, as it does in the plain definition.
// swigluoai: g = min(gate, limit), u = clamp(up, -limit, limit),
// a = g * sigmoid(alpha * g) * (u + beta).
__device__ __forceinline__ float act_swigluoai(float gate, float up, float alpha, float beta,
                                               float limit) {
  const float g = gate > limit ? limit : gate;
  const float u = up > limit ? limit : (up < -limit ? -limit : up);
  return g * sigmoid_fast(alpha * g) * (u + beta);
}
// ReLU^2: max(h, 0)^2.
__device__ __forceinline__ float act_relu2(float h) {
  const float r = h < 0.f ? 0.f : h;
  return r * r;
}

// GPTQ weights passed with a group map: the kernels read groups as runs of
// `group` consecutive rows, so only the identity map (row k in group
// k / group) describes weights they can multiply.  Every workgroup checks its
// expert's map after its K loop (K ints, from L2) and all its threads agree
// on the result; any other map poisons the workgroup's outputs with NaN, a
// visible failure instead of silently misgrouped scales.  Act-order maps go
// through the load-time group sort instead.  Called by every thread of the
// workgroup (the condition on g_idx is the same for all of them).
template <int FMT>
__device__ __forceinline__ bool gidx_bad(const WeightArgs& W, int e, int K, int tid, int nthreads) {
  int bad = 0;
  if (FMT == FMT_GPTQ && W.g_idx != nullptr) {
    const int32_t* g = W.g_idx + (size_t)e * K;
    for (int k = tid; k < K; k += nthreads) bad |= g[k] != k / W.group;
    bad = __syncthreads_or(bad);
  }
  return bad != 0;
}

// Per-expert multiplier of the accumulators: the NVFP4 global scale (1 for the
// other formats), or NaN for a poisoned tile.
template <int FMT>
__device__ __forceinline__ float acc_scale(const WeightArgs& W, int e, bool poison) {
  const float g = (FMT == FMT_NVFP4) ? W.global_scale[e] : 1.f;
  return poison ? __builtin_nanf("") : g;
}

// --------------------------------------------------------------------------
// epilogue for one wave's fragment accumulators
// --------------------------------------------------------------------------

struct EpiArgs {
  const int32_t* sorted_ids;  // block's slot ids start at sorted_ids[row0]
  int row0;
  int n_slots;
  int N;
  const float* topk_w;
  int mul_tw;
  float alpha, beta, limit;
  uint16_t* out;
  int out_ld;
};

// Weight row of fragment j (of NF) of a wave whose first row is n0.
template <int EPI>
__device__ __forceinline__ int frag_row(int n0, int j, int c16) {
  return (EPI == EPI_SWIGLU) ? n0 + 32 * (j >> 1) + 2 * c16 + (j & 1) : n0 + 16 * j + c16;
}

// Is fragment j valid (N % 16 == 0; gated N % 32 == 0)?
template <int EPI>
__device__ __forceinline__ bool frag_on(int n0, int j, int N) {
  return (EPI == EPI_SWIGLU) ? (n0 + 32 * (j >> 1) < N) : (n0 + 16 * j < N);
}

// acc[i][j]: rows i*16 + 4g + r, fragment j (NF fragments from weight row n0).
template <int EPI, int FMT, int MI, int NF>
__device__ __forceinline__ void epilogue(const f32x4 (&acc)[MI][NF], const EpiArgs& a,
                                         const WeightArgs& W, int e, int n0, int lane,
                                         bool poison = false) {
  const int c16 = lane & 15, g = lane >> 4;
  const float gsc = acc_scale<FMT>(W, e, poison);
  // bias: unconditional loads (another valid word when there is none)
  const bool has_bias = W.bias != nullptr;
  const uint16_t* bbase = has_bias ? W.bias : reinterpret_cast<const uint16_t*>(W.qweight != nullptr ? W.qweight : W.qweight_kc);
  const int bmul = has_bias ? 1 : 0;
  float bias[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int row = frag_on<EPI>(n0, j, a.N) ? frag_row<EPI>(n0, j, c16) : n0;
    const float b = bf16_bits_to_f32(bbase[((size_t)e * a.N + row) * bmul]);
    bias[j] = has_bias ? b : 0.f;
  }
  // slot ids, then routing weights, each as one batch of unconditional loads
  // (a load inside the per-row branch would be waited for at once)
  int sids[MI][4];
  float tws[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) sids[i][r] = a.sorted_ids[a.row0 + i * 16 + 4 * g + r];
  // (GEMM2: the output row is scaled; GEMM1: the accumulator, i.e. the
  // input row -- the routing weight applied on the input)
  const bool use_tw = a.mul_tw;
  const float* tbase = use_tw ? a.topk_w : reinterpret_cast<const float*>(a.sorted_ids);
  const int tmul = use_tw ? 1 : 0;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) tws[i][r] = tbase[min(sids[i][r], a.n_slots - 1) * tmul];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sid = sids[i][r];
      if (sid >= a.n_slots) continue;
      uint16_t* orow = a.out + (size_t)sid * a.out_ld;
      const float tw = use_tw ? tws[i][r] : 1.f;
      const float gin = (EPI == EPI_DOWN) ? gsc : gsc * tw;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int p = 0; p < NF / 2; ++p) {
          if (!frag_on<EPI>(n0, 2 * p, a.N)) continue;
          const float gate = acc[i][2 * p][r] * gin + bias[2 * p];
          const float up = acc[i][2 * p + 1][r] * gin + bias[2 * p + 1];
          const float v = act_swigluoai(gate, up, a.alpha, a.beta, a.limit);
          orow[n0 / 2 + 16 * p + c16] = f32_to_bf16_bits(v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          if (!frag_on<EPI>(n0, j, a.N)) continue;
          float v = acc[i][j][r] * gin + bias[j];
          if (EPI == EPI_RELU2) {
            v = act_relu2(v);
          } else if (EPI == EPI_DOWN) {
            v = v * tw;
          }
          orow[n0 + 16 * j + c16] = f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// prefill kernel
// --------------------------------------------------------------------------
//
// Workgroup tile: BM rows (slots of one expert block) x BN = 4*NF*32 weight
// rows; four waves (one per SIMD) split the weight rows (NF 32-column
// fragments each) and every wave covers all BM rows, so each weight is
// dequantised exactly once per workgroup.  MFMA is v_mfma_f32_32x32x16_bf16:
// per instruction it does twice the work of the 16x16 shape for the same
// operand registers, which leaves room to keep the next step's A fragments
// and dequantised weights in flight without spilling.
//
// K is walked in 64-wide chunks through a 4-deep LDS ring holding, per chunk,
// the A rows (bf16, gathered by slot) and the 4-bit weight codes, both copied
// global -> LDS by the gfx950 LDS-DMA loads; the scales of the tile's rows
// for the whole K sit in LDS from the start.  The DMA loads are issued from
// inline assembly so the compiler never inserts waits for them; the pipeline
// keeps its own count (every chunk issues the same number of DMA instructions
// per wave and loads retire in order), so a chunk is waited for only when it
// is needed and three more stay in flight.
//
// Lane mapping (lane l, c = l % 32, h = l / 32): in a 64-wide chunk the lane
// owns k in [32h, 32h + 32); MFMA step s (0..3) takes k = 32h + 8s .. +8 of
// it for both operands (a reduction's order is free).  The lane's A rows are
// i*32 + c, its weight row is that of column c of each fragment, and its 32
// codes of a chunk are one 16-byte LDS read.

struct GemmArgs {
  const uint16_t* A;
  int a_div;       // A row = sorted_id / a_div
  uint64_t a_mul;  // ceil(2^32 / a_div): sorted_id / a_div == (sorted_id * a_mul) >> 32 for ids < 2^24
  int n_slots;     // sentinel
  int K, N, E;
  int n_mblocks, n_ntiles;
  int group_m;     // prefill tile order: expert blocks per group
  int block_m;     // rows per aligned block (expert_ids has one entry per block)
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* num_post_pad;
  // prefill kernel only, optional: a list of 128-row tiles (first row in
  // sorted_ids, expert) with its length in n_tiles[0], instead of the
  // aligned blocks (mixed tiling: an expert's full 128-row runs)
  const int2* tiles;
  const int32_t* n_tiles;
};

// First row (in sorted_ids) and expert of prefill tile mb: aligned block mb,
// or entry mb of the tile list.
__device__ __forceinline__ void tile_rows(const GemmArgs& ga, int mb, int bm, int& row0, int& e) {
  if (ga.tiles != nullptr) {
    const int2 t = ga.tiles[mb];
    row0 = t.x;
    e = t.y;
  } else {
    row0 = mb * bm;
    e = ga.expert_ids[mb];
  }
}

// A row of a sorted slot.  Padding slots read row 0 instead: their products
// land only in accumulator rows that the epilogue never stores (an MFMA row
// depends on its own A row only), so no zero-fill or branch is needed.
__device__ __forceinline__ const uint16_t* a_row(const GemmArgs& ga, int sid) {
  const int row = (int)(((uint64_t)(uint32_t)sid * ga.a_mul) >> 32);
  return ga.A + (size_t)(sid < ga.n_slots ? row : 0) * ga.K;
}

// Weights of the wave's NF fragments for the chunk starting at k0 (lane range k0 + g*C/4).
// Rows of fragments past N were clamped to a valid row by the caller: their
// products land only in columns the epilogue never stores.
template <int FMT, int C, int NF>
__device__ __forceinline__ void load_frags(BChunk<FMT, C> (&b)[NF], const WeightArgs& W, int e,
                                           const int (&nrow)[NF], int N, int K, int k0, int g) {
#pragma unroll
  for (int j = 0; j < NF; ++j) load_chunk<FMT, C>(b[j], W, e, nrow[j], N, K, k0 + g * (C / 4));
}

constexpr int kPfBK = 64;                  // K chunk
// Waves per SIMD of the prefill kernel (row split): two for MXFP4, whose
// dequant is one convert per two weights (measured 3-4% faster at the
// gpt-oss-120b shape), one otherwise (the doubled dequant of NVFP4 / GPTQ
// costs more than the overlap gains: GPTQ measured 13% slower).
template <int FMT>
constexpr int pf_rs() { return FMT == FMT_MXFP4 ? 2 : 1; }
// K split (KS = 2): eight waves, waves w and w + 4 take the same rows and
// columns and alternate MFMA steps (two of the four of each chunk), so no
// dequant or LDS read is done twice; their sums meet through LDS at the end.
template <int FMT>
constexpr int pf_ks() { return FMT == FMT_MXFP4 ? 1 : 2; }
constexpr int kPfScaleBytes = 60 * 1024;   // LDS for the tile's scales over all of K

// SK = 1 (NVFP4 with scales laid out by K chunk, [E][K/64][N][4]): each
// chunk's scales (4 bytes per weight row, contiguous over the tile's rows)
// travel through the ring with its codes, so no scale tile stays resident;
// with 3 stages the workgroup needs 76 KB of LDS and two share a CU, one's
// prologue and epilogue overlapping the other's K loop.  SK = 2: the
// codes are laid out by K chunk too ([E][K/64][N][32]), so the copy of one
// 32-row block of a chunk reads one contiguous kilobyte.  (Measured: 256-row
// tiles -- two blocks of one expert, 256 accumulators per lane, so one
// workgroup per CU -- ran 4-10% slower at the gpt-oss shapes despite half the
// dequantisation per MFMA: with one wave per SIMD, a third of the time had
// neither the matrix core nor the VALU busy.)
template <int BM, int NF, int SK = 0>
struct Pf {
  static constexpr int MI = BM / 32;
  static constexpr int BN = 128 * NF;
  static constexpr int kABytes = BM * kPfBK * 2;            // A rows of one chunk
  static constexpr int kBBytes = BN * kPfBK / 2;            // weight codes of one chunk
  static constexpr int kSBytes = SK ? BN * 4 : 0;           // streamed scales of one chunk
  static constexpr int kAIssue = kABytes / 1024 / 4;         // DMA instructions per wave per chunk
  static constexpr int kBIssue = kBBytes / 1024 / 4;
  static constexpr int kSIssue = SK ? 1 : 0;                 // 64 lanes x 4 bytes per wave
  static constexpr int kIssue = kAIssue + kBIssue + kSIssue;
  static constexpr int kStage = kABytes + kBBytes + kSBytes;
  static constexpr int kStages = SK ? 3 : 4;                 // LDS ring depth
  // the last BM * 8 bytes hold the row table of the epilogue (inside the
  // scale area when the scales are resident: written after their last read)
  static constexpr int kRowTab = BM * 8;
  static constexpr int kLds = kStages * kStage + (SK ? kRowTab : kPfScaleBytes);
  static_assert(kAIssue >= 1 && kBIssue >= 1, "tile too small for the DMA split");
  static_assert(!SK || kSBytes == 4 * 256, "one 256-byte scale run per wave");
  static_assert(kLds <= 160 * 1024, "LDS");
  static_assert((kStages - 1) * kIssue < 64, "vmcnt range");
};

// Bytes of LDS the scales of one BN-row tile take for the whole K.
__host__ __device__ inline int pf_scale_bytes(int fmt, int K, int group, int bn) {
  if (fmt == FMT_NVFP4) return bn * (K / 16);
  if (fmt == FMT_MXFP4) return bn * (K / 32);
  return (K / group) * (bn * 2 + bn / 2);  // fp16 scales + packed zero points
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// One global -> LDS DMA instruction: lane l copies 16 bytes from g to
// lds_base + 16*l (lds_base must be wave-uniform).  Issued as inline assembly
// so the compiler does not track it; the kernel waits with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory");
}

// Same with 4 bytes per lane: lane l copies g[0..3] to lds_base + 4*l.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory");
}

// The same two DMA instructions, pinned between MFMAs: `after` and `before`
// are read-write register operands the instruction leaves untouched, so the
// compiler keeps it after the last reader of `after` and before the first
// reader of `before` (an asm statement with only a memory clobber may drift
// past MFMAs, which touch no memory).
__device__ __forceinline__ void dma16_pinned(const void* g, uint32_t lds_base, uint32_t& after,
                                             uint32_t& before) {
  asm volatile("s_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %2, off"
               : "+v"(after), "+v"(before)
               : "v"(g), "s"(lds_base)
               : "memory");
}
__device__ __forceinline__ void dma4_pinned(const void* g, uint32_t lds_base, uint32_t& after,
                                            uint32_t& before) {
  asm volatile("s_mov_b32 m0, %3\n\tglobal_load_lds_dword %2, off"
               : "+v"(after), "+v"(before)
               : "v"(g), "s"(lds_base)
               : "memory");
}

// s_waitcnt vmcnt(N): all but the N most recent vector-memory loads of this wave have landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "I"(N) : "memory");
}

// Workgroup barrier that does not wait for the wave's outstanding loads
// (__syncthreads waits for all of them, which would drain the ring).
// The LDS reads issued before it are waited for first, so no DMA started
// after the barrier can overwrite data a read has not yet taken.
__device__ __forceinline__ void pf_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tile of a workgroup.  Only the blocks moe_align actually filled are
// scheduled: their number is read from num_post_pad, and the 8 XCDs (which
// receive workgroups round-robin) each get a contiguous run of them.  Inside
// a run, tiles go in groups of group_m expert blocks: the blocks of a group
// cycle fastest, then the column tiles, so the workgroups that run at the
// same time on one XCD share both their weight tiles (the blocks of one
// expert) and their A blocks (across column tiles) in that XCD's L2.
__device__ __forceinline__ bool prefill_tile(const GemmArgs& a, int bm, int& mb, int& nt) {
  const int nmb = min(a.tiles != nullptr ? a.n_tiles[0] : a.num_post_pad[0] / bm, a.n_mblocks);
  const int total = nmb * a.n_ntiles;
  const int per_xcd = (total + 7) / 8;
  const int pid = blockIdx.x;
  const int idx = pid >> 3;
  const int lid = (pid & 7) * per_xcd + idx;
  if (idx >= per_xcd || lid >= total) return false;
  const int gsize = a.group_m * a.n_ntiles;
  const int grp = lid / gsize;
  const int rem = lid - grp * gsize;
  const int h = min(a.group_m, nmb - grp * a.group_m);
  nt = rem / h;
  mb = grp * a.group_m + rem % h;
  return true;
}

// Position (16-byte unit) of the codes of tile row r, half h inside its
// 32-row block of a chunk's weight tile.  Gated tiles store even rows (the
// gate halves of the pairs) before odd ones, so the 8 lanes that one LDS
// cycle serves always hit 8 different bank groups.
template <int EPI>
__device__ __forceinline__ int pf_bpos(int r, int h) {
  const int s = (EPI == EPI_SWIGLU) ? ((r & 31) >> 1) + 16 * (r & 1) : (r & 31);
  return (r >> 5) * 64 + 32 * h + s;
}
// Tile row stored at position p (0..63) of 32-row block b (inverse of pf_bpos).
template <int EPI>
__device__ __forceinline__ int pf_brow(int b, int p) {
  const int s = p & 31;
  return 32 * b + ((EPI == EPI_SWIGLU) ? 2 * (s & 15) + (s >> 4) : s);
}

// Source of a lane's streamed scale word (SK != 0): chunk kc reads
// p + (kc >> gsh) * stride.  NVFP4: one [N][4] row per 64-deep chunk; MXFP4:
// one per 128-deep chunk (gsh = 1); GPTQ: the checkpoint's fp16 scale row
// and packed zero-point row of the chunk's group (gsh = log2(group / 64)),
// lanes 0..31 two scales each, lanes 32..39 one zero word each.
struct SkSrc {
  const uint8_t* p;
  uint32_t stride;
  int gsh;
};

// DMA instruction d (0 <= d < kIssue) of one wave's share of chunk kc, into
// the ring stage at stage_lds: first the A rows, then the weight codes, then
// (SK) the chunk's 4-byte scale runs of tile rows 64*wave .. 64*wave+63.
// PIN places it between MFMAs (dma16_pinned).
template <int FMT, int BM, int NF, int SK, bool PIN>
__device__ __forceinline__ void pf_issue_one(int d, uint32_t stage_lds,
                                             const uint16_t* const (&arow)[Pf<BM, NF, SK>::kAIssue],
                                             const uint8_t* const (&brow)[Pf<BM, NF, SK>::kBIssue],
                                             const SkSrc& sk, int kc, int wave_u, int N,
                                             uint32_t& after, uint32_t& before) {
  using P = Pf<BM, NF, SK>;
  const int k0 = kc * kPfBK;
  const void* src;
  uint32_t dst;
  if (d < P::kAIssue) {  // instruction q = 4d + wave: A rows 8q .. 8q+7
    src = arow[d] + k0;
    dst = stage_lds + (uint32_t)(8 * (4 * d + wave_u)) * 128u;
  } else if (d < P::kAIssue + P::kBIssue) {
    const int p = d - P::kAIssue;
    dst = stage_lds + P::kABytes + (uint32_t)(4 * p + wave_u) * 1024u;
    if (FMT == FMT_GPTQ)
      src = brow[p] + (size_t)k0 / 8 * N * 4;  // 256 words of the [8][BN] word tile
    else if (SK == 2 && FMT == FMT_NVFP4)
      src = brow[p] + (size_t)kc * N * 32;     // one 32-row block, codes by 64-deep chunk
    else if (SK == 2)
      src = brow[p] + (size_t)(kc >> 1) * N * 64 + 32 * (kc & 1);  // MXFP4 codes by 128-deep chunk
    else
      src = brow[p] + k0 / 2;                  // one 32-row block
  } else {
    // the chunk's scale words (MXFP4: one row per 128-deep chunk, fetched for
    // both of its 64-deep halves; GPTQ: one row per group)
    src = sk.p + (size_t)(kc >> sk.gsh) * sk.stride;
    dst = stage_lds + P::kABytes + P::kBBytes + (uint32_t)wave_u * 256u;
  }
  const bool word = SK && d == P::kIssue - 1;
  if (PIN) {
    if (word) dma4_pinned(src, dst, after, before);
    else dma16_pinned(src, dst, after, before);
  } else {
    if (word) dma4(src, dst);
    else dma16(src, dst);
  }
}

// All of one wave's DMA of chunk kc into the ring stage at stage_lds.
template <int FMT, int BM, int NF, int SK>
__device__ __forceinline__ void pf_issue(uint32_t stage_lds, const uint16_t* const (&arow)[Pf<BM, NF, SK>::kAIssue],
                                         const uint8_t* const (&brow)[Pf<BM, NF, SK>::kBIssue],
                                         const SkSrc& sk, int kc, int wave_u, int N) {
  uint32_t unused = 0;
#pragma unroll
  for (int d = 0; d < Pf<BM, NF, SK>::kIssue; ++d)
    pf_issue_one<FMT, BM, NF, SK, false>(d, stage_lds, arow, brow, sk, kc, wave_u, N, unused, unused);
}

// Weight codes of one fragment for one chunk (one code word per MFMA step)
// and its group scale(s): NVFP4 two e4m3 scales (k 0..15 and 16..31 of the
// lane's range), MXFP4 one power of two, GPTQ scale and -zero*scale.
struct PfB {
  uint4 q;
  float s0, s1;
};

template <int FMT>
__device__ __forceinline__ bf16x8 pf_deq(uint32_t w, float s, float zs) {
  uint4 r;
  if (FMT == FMT_NVFP4) {
    f32x2 p;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    r.x = pack_bf16x2(p[0] * s, p[1] * s);
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    r.y = pack_bf16x2(p[0] * s, p[1] * s);
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    r.z = pack_bf16x2(p[0] * s, p[1] * s);
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    r.w = pack_bf16x2(p[0] * s, p[1] * s);
  } else if (FMT == FMT_MXFP4) {
    bf16x2 p;
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    __builtin_memcpy(&r.x, &p, 4);
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    __builtin_memcpy(&r.y, &p, 4);
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    __builtin_memcpy(&r.z, &p, 4);
    p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    __builtin_memcpy(&r.w, &p, 4);
  } else {
    float v[8];
    gptq_deq8(w, s, zs, v);
    r.x = pack_bf16x2(v[0], v[1]);
    r.y = pack_bf16x2(v[2], v[3]);
    r.z = pack_bf16x2(v[4], v[5]);
    r.w = pack_bf16x2(v[6], v[7]);
  }
  bf16x8 o;
  __builtin_memcpy(&o, &r, 16);
  return o;
}

// Dequantised weights of MFMA step s from a fragment's raw chunk.
template <int FMT>
__device__ __forceinline__ bf16x8 pf_deq_step(const PfB& b, int s) {
  const uint32_t w = s == 0 ? b.q.x : s == 1 ? b.q.y : s == 2 ? b.q.z : b.q.w;
  if (FMT == FMT_NVFP4) return pf_deq<FMT>(w, s < 2 ? b.s0 : b.s1, 0.f);
  return pf_deq<FMT>(w, b.s0, b.s1);
}

// LDS reads of the fragment weights of chunk kc (codes from the ring stage
// at bstage, scales from the resident scale tile).  rl[j] is the lane's tile
// row of fragment j.
template <int FMT, int EPI, int NF, int SK = 0>
__device__ __forceinline__ void pf_read_b(PfB (&b)[NF], const uint8_t* bstage, const uint8_t* sc,
                                          const int (&rl)[NF], int kc, int h, int K, int group,
                                          int bn) {
  const int k0 = kc * kPfBK;
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int r = rl[j];
    if (FMT == FMT_GPTQ) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(bstage);
      b[j].q.x = w[(4 * h + 0) * bn + r];
      b[j].q.y = w[(4 * h + 1) * bn + r];
      b[j].q.z = w[(4 * h + 2) * bn + r];
      b[j].q.w = w[(4 * h + 3) * bn + r];
      float s, z;
      if (SK) {
        // the stage's run of wave r/64: 64 fp16 scales, then 8 zero words
        const uint8_t* run = sc + (r >> 6) * 256;
        s = half_bits_to_f32(*reinterpret_cast<const uint16_t*>(run + (r & 63) * 2));
        z = (float)((*reinterpret_cast<const uint32_t*>(run + 128 + ((r & 63) >> 3) * 4) >> (4 * (r & 7))) & 15u);
      } else {
        const int grp = (k0 + 32 * h) / group;
        s = half_bits_to_f32(reinterpret_cast<const uint16_t*>(sc)[grp * bn + r]);
        const uint32_t* zw = reinterpret_cast<const uint32_t*>(sc + (K / group) * bn * 2);
        z = (float)((zw[grp * (bn / 8) + (r >> 3)] >> (4 * (r & 7))) & 15u);
      }
      b[j].s0 = s;
      b[j].s1 = -z * s;
    } else {
      b[j].q = *reinterpret_cast<const uint4*>(bstage + 16 * pf_bpos<EPI>(r, h));
      if (FMT == FMT_NVFP4) {
        // SK: sc is the stage's [BN][4] scale run of this chunk
        const uint32_t s2 = SK ? *reinterpret_cast<const uint16_t*>(sc + r * 4 + 2 * h)
                               : *reinterpret_cast<const uint16_t*>(sc + r * (K / 16) + k0 / 16 + 2 * h);
        b[j].s0 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 0);
        b[j].s1 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 1);
      } else {
        // SK: the stage's [BN][4] e8m0 bytes of the 128-deep chunk holding kc
        b[j].s0 = e8m0_operand(SK ? sc[r * 4 + 2 * (kc & 1) + h] : sc[r * (K / 32) + k0 / 32 + h]);
        b[j].s1 = 0.f;
      }
    }
  }
}

// Physical 16-byte slot of logical slot q in A row r of a 128-byte-row LDS
// stage: q ^ ((r / 2) % 8).  A 16-byte read serves 16 lanes (16 rows) per LDS
// cycle, and two rows fill the 64 banks; with this swizzle the 16 rows of a
// cycle cover 16 distinct 4-bank groups (q ^ (r % 8) gave rows r and r + 8 the
// same group: a two-way conflict on every A read).
__device__ __forceinline__ int a_slot(int q, int r) { return q ^ ((r >> 1) & 7); }

// A fragments of MFMA step s of a chunk: rows i*32 + c, k = 32h + 8s .. +8.
// A rows are 128 bytes in LDS, logical 16-byte slot q of row r stored at a_slot(q, r).
// (MA <= MI: only the first MA fragments, the rest of a tile being padding rows.)
template <int MI, int MA = MI>
__device__ __forceinline__ void pf_read_a(uint4 (&a)[MI], const uint8_t* astage, int c, int h, int s) {
#pragma unroll
  for (int i = 0; i < MA; ++i) {
    const int r = i * 32 + c;
    a[i] = *reinterpret_cast<const uint4*>(astage + r * 128 + 16 * a_slot(4 * h + s, r));
  }
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

template <int MI, int NF, int MA = MI>
__device__ __forceinline__ void pf_mfma(f32x16 (&acc)[MI][NF], const uint4 (&a)[MI], const bf16x8 (&b)[NF]) {
#pragma unroll
  for (int i = 0; i < MA; ++i) {
    const bf16x8 af = as_bf16x8(a[i]);
#pragma unroll
    for (int j = 0; j < NF; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b[j], acc[i][j], 0, 0, 0);
  }
}

// One MFMA step (as pf_mfma) with one wave's DMA of chunk kc dealt between
// its rows.  Issued back to back, a wave's 5..7 DMA instructions sit in
// front of the MFMAs that follow them in the wave's in-order issue; dealt
// between rows they overlap the matrix core's work (measured ~5% faster on
// both GEMMs).  The A fragments serve as the pins, so `a` reads as modified
// afterwards (callers reload it).
template <int FMT, int BM, int NF, int SK, int MI, int MA = MI>
__device__ __forceinline__ void pf_mfma_issue(f32x16 (&acc)[MI][NF], uint4 (&a)[MI], const bf16x8 (&b)[NF],
                                              uint32_t stage_lds,
                                              const uint16_t* const (&arow)[Pf<BM, NF, SK>::kAIssue],
                                              const uint8_t* const (&brow)[Pf<BM, NF, SK>::kBIssue],
                                              const SkSrc& sk, int kc, int wave_u, int N) {
  using P = Pf<BM, NF, SK>;
  constexpr int kPer = (P::kIssue + MA - 1) / MA;  // DMA instructions after each active row
  uint32_t last = 0;
#pragma unroll
  for (int i = 0; i < MA; ++i) {
    const bf16x8 af = as_bf16x8(a[i]);
#pragma unroll
    for (int j = 0; j < NF; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int d = kPer * i; d < kPer * (i + 1) && d < P::kIssue; ++d)
      pf_issue_one<FMT, BM, NF, SK, true>(d, stage_lds, arow, brow, sk, kc, wave_u, N, a[i].x,
                                          i + 1 < MA ? a[i + 1 < MA ? i + 1 : i].x : last);
  }
}

// DMA of a region of `bytes` bytes into LDS at lds_base, described as rows of
// row_bytes bytes (all sizes multiples of 16): LDS byte o comes from
// src + (o / row_bytes) * ld + o % row_bytes, for the first valid_row_bytes
// of each row only (the rest is left unfilled and never read).
// Instructions are dealt to the four waves round-robin; lanes outside the
// region are switched off.  Only the prologue uses it, before the ring starts.
__device__ __forceinline__ void pf_dma_region(uint32_t lds_base, const uint8_t* src, size_t ld,
                                              int row_bytes, int valid_row_bytes, int bytes,
                                              int wave_u, int lane) {
  const int nq = (bytes + 1023) / 1024;
  for (int q = wave_u; q < nq; q += 4) {
    const int o = q * 1024 + 16 * lane;
    const int in_row = o % row_bytes;
    if (o < bytes && in_row < valid_row_bytes)
      dma16(src + (size_t)(o / row_bytes) * ld + in_row, lds_base + q * 1024);
  }
}

// Weight row of fragment j (32 columns) for lane column c, and whether the
// column exists (N % 16 == 0; gated N % 32 == 0, rows 2i / 2i+1 = gate / up
// of output column i meet in one lane through fragments 2p / 2p+1).
template <int EPI>
__device__ __forceinline__ int frag32_row(int n0, int j, int c) {
  return (EPI == EPI_SWIGLU) ? n0 + 64 * (j >> 1) + 2 * c + (j & 1) : n0 + 32 * j + c;
}

// Epilogue of the 32x32 accumulators: lane (c, h) holds column c of every
// fragment and rows 8*(v/4) + 4h + v%4 (v = 0..15) of every 32-row fragment.
// rows: null, or the block's (slot id, routing weight bits) pairs in LDS,
// indexed by the row within the block; rloc0 is this wave's first such row.
template <int EPI, int FMT, int MI, int NF>
__device__ __forceinline__ void epilogue32(const f32x16 (&acc)[MI][NF], const EpiArgs& a,
                                           const WeightArgs& W, int e, int n0, int lane,
                                           const int2* rows = nullptr, int rloc0 = 0,
                                           bool poison = false) {
  const int c = lane & 31, h = lane >> 5;
  const float gsc = acc_scale<FMT>(W, e, poison);
  // bias: unconditional loads (another valid word when there is none)
  const bool has_bias = W.bias != nullptr;
  const uint16_t* bbase = has_bias ? W.bias : reinterpret_cast<const uint16_t*>(W.qweight != nullptr ? W.qweight : W.qweight_kc);
  const int bmul = has_bias ? 1 : 0;
  float bias[NF];
  bool on[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = frag32_row<EPI>(n0, j, c);
    on[j] = n < a.N;
    const float b = bf16_bits_to_f32(bbase[((size_t)e * a.N + (on[j] ? n : n0)) * bmul]);
    bias[j] = has_bias ? b : 0.f;
  }
  // routing weights: one unconditional load per row, all issued before any
  // is used (a load inside the per-row branch would be waited for at once,
  // one memory latency per row); sentinel rows read a valid unused weight
  // (GEMM2: the output row is scaled; GEMM1: the accumulator, i.e. the
  // input row -- the routing weight applied on the input)
  const bool use_tw = a.mul_tw;
  const float* tbase = use_tw ? a.topk_w : reinterpret_cast<const float*>(a.sorted_ids);
  const int tmul = use_tw ? 1 : 0;
  // slot ids one row group ahead of their use, so each group's loads overlap
  // the previous group's stores
  int sid_next[16];
  if (rows == nullptr) {
#pragma unroll
    for (int v = 0; v < 16; ++v) sid_next[v] = a.sorted_ids[a.row0 + 8 * (v >> 2) + 4 * h + (v & 3)];
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    int sid[16];
    float tws[16];
    if (rows != nullptr) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int2 r = rows[rloc0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3)];
        sid[v] = r.x;
        tws[v] = __int_as_float(r.y);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) sid[v] = sid_next[v];
#pragma unroll
      for (int v = 0; v < 16; ++v)
        tws[v] = tbase[min(sid[v], a.n_slots - 1) * tmul];
      if (i + 1 < MI) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          sid_next[v] = a.sorted_ids[a.row0 + (i + 1) * 32 + 8 * (v >> 2) + 4 * h + (v & 3)];
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (sid[v] >= a.n_slots) continue;
      uint16_t* orow = a.out + (size_t)sid[v] * a.out_ld;
      const float tw = use_tw ? tws[v] : 1.f;
      const float gin = (EPI == EPI_DOWN) ? gsc : gsc * tw;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int p = 0; p < NF / 2; ++p) {
          if (!on[2 * p]) continue;
          const float gate = acc[i][2 * p][v] * gin + bias[2 * p];
          const float up = acc[i][2 * p + 1][v] * gin + bias[2 * p + 1];
          const float y = act_swigluoai(gate, up, a.alpha, a.beta, a.limit);
          orow[n0 / 2 + 32 * p + c] = f32_to_bf16_bits(y);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          if (!on[j]) continue;
          float y = acc[i][j][v] * gin + bias[j];
          if (EPI == EPI_RELU2) {
            y = act_relu2(y);
          } else if (EPI == EPI_DOWN) {
            y = y * tw;
          }
          orow[n0 + 32 * j + c] = f32_to_bf16_bits(y);
        }
      }
    }
  }
}

// K tail (K % 64 == 32): two 16-wide MFMA steps with A and weights loaded
// straight from global memory (lane k range k0 + 16h .. +16).
template <int FMT, int EPI, int MI, int NF>
__device__ __forceinline__ void pf_tail32(f32x16 (&acc)[MI][NF], const GemmArgs& ga, const WeightArgs& W,
                                          int e, int row0, int n0, int c, int h, int k0) {
  BChunk<FMT, 64> bt[NF];  // C = 64: the lane's 16 k in two 8-k steps
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = min(frag32_row<EPI>(n0, j, c), ga.N - 1);
    load_chunk<FMT, 64>(bt[j], W, e, n, ga.N, ga.K, k0 + 16 * h);
  }
  uint4 a0[MI], a1[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const uint16_t* p = a_row(ga, ga.sorted_ids[row0 + i * 32 + c]) + k0 + 16 * h;
    a0[i] = *reinterpret_cast<const uint4*>(p);
    a1[i] = *reinterpret_cast<const uint4*>(p + 8);
  }
  bf16x8 b0[NF], b1[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    b0[j] = deq_step<FMT, 64>(bt[j], 0);
    b1[j] = deq_step<FMT, 64>(bt[j], 1);
  }
  pf_mfma<MI, NF>(acc, a0, b0);
  pf_mfma<MI, NF>(acc, a1, b1);
}

template <int FMT, int EPI, int BM, int NF, int RS, int KS, int SK>
__global__ void __launch_bounds__(256 * RS * KS, SK ? 2 : 1) gemm_prefill_kernel(GemmArgs ga, WeightArgs W, EpiArgs ea) {
  using P = Pf<BM, NF, SK>;
  constexpr int kStages = P::kStages;
  static_assert(kStages == 3 || kStages == 4, "the K loop is unrolled for 3 or 4 stages");
  static_assert(!SK || (RS == 1 && KS == 1 && (FMT != FMT_GPTQ || SK == 1)),
                "streamed scales: one wave per SIMD per workgroup; GPTQ codes as stored");
  // RS = 2: eight waves, two per SIMD; waves w and w + 4 take the same
  // columns and one half of the rows each (both dequantise the same codes),
  // so one wave's dequant and LDS reads overlap the other's MFMAs.  Only the
  // first four waves issue the DMA.
  constexpr int MI = P::MI / RS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[P::kLds];
  uint8_t* const scale_lds = smem + kStages * P::kStage;  // resident scales (SK = 0)

  int mb, nt;
  if (!prefill_tile(ga, BM, mb, nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_u = wave_all & 3;            // column group, and DMA share
  const int rpart = RS == 2 ? wave_all >> 2 : 0;  // row part (RS = 2)
  const int kp = KS == 2 ? wave_all >> 2 : 0;     // K part (KS = 2): MFMA steps 2kp, 2kp+1
  const bool dma_wave = (wave_all >> 2) == 0;
  const int aoff = rpart * MI * 32 * 128;     // this wave's rows in an A stage
  const int K = ga.K, N = ga.N;

  // slot ids of the A rows this lane copies, requested before anything waits:
  // DMA instruction q = 4p + wave covers rows 8q .. 8q+7, lane l row 8q + l/8
  int rowb, e;  // the tile's first row in sorted_ids, its expert
  tile_rows(ga, mb, BM, rowb, e);
  // 32-row fragments holding a real slot: a tile's real slots come first (the
  // sort pads each expert's run at its end), so fragment i is live when its
  // first slot is
  int nact = 1;
#pragma unroll
  for (int i = 1; i < BM / 32; ++i) nact += ga.sorted_ids[rowb + 32 * i] < ga.n_slots ? 1 : 0;
  int sid[P::kAIssue];
#pragma unroll
  for (int p = 0; p < P::kAIssue; ++p) sid[p] = ga.sorted_ids[rowb + 8 * (4 * p + wave_u) + (lane >> 3)];
  if (e < 0 || e >= ga.E) return;
  // slot id of block row tid, for the epilogue: requested now, first used
  // after the K loop, so its latency hides behind the loop
  const int row_sid = ga.sorted_ids[rowb + min(tid, BM - 1)];

  const int nt0 = nt * P::BN;             // first weight row of the tile
  const int rows = min(P::BN, N - nt0);   // valid weight rows of the tile
  const int n0 = nt0 + wave_u * NF * 32;  // first weight row of this wave

  // DMA sources.  A: lane l of instruction q writes physical slot l%8 of row
  // r = 8q + l/8, so it fetches logical slot a_slot(l%8, r) (see pf_read_a).
  const uint16_t* arow[P::kAIssue];
#pragma unroll
  for (int p = 0; p < P::kAIssue; ++p) {
    const int r = 8 * (4 * p + wave_u) + (lane >> 3);
    arow[p] = a_row(ga, sid[p]) + 8 * a_slot(lane & 7, r);
  }
  // Weight codes.  NVFP4/MXFP4: instruction q fills 32-row block q, lane l
  // the half l/32 of tile row pf_brow(q, l) (rows past N re-read the last
  // row).  GPTQ: instruction q covers words 256q .. 256q+255 of the chunk's
  // [8 k-words][BN columns] tile, lane l four consecutive columns.
  const uint8_t* brow[P::kBIssue];
#pragma unroll
  for (int p = 0; p < P::kBIssue; ++p) {
    const int q = 4 * p + wave_u;
    if (FMT == FMT_GPTQ) {
      const int w = q * 256 + 4 * lane;
      const int col = min(nt0 + w % P::BN, N - 4);
      brow[p] = W.qweight + (((size_t)e * (K / 8) + w / P::BN) * N + col) * 4;
    } else {
      const int n = min(nt0 + pf_brow<EPI>(q, lane), N - 1);
      brow[p] = SK == 2 ? (FMT == FMT_NVFP4
                               ? W.qweight_kc + ((size_t)e * (K / 64) * N + n) * 32 + 16 * (lane >> 5)
                               : W.qweight_kc + ((size_t)e * ((K + 127) / 128) * N + n) * 64 +
                                     16 * (lane >> 5))
                        : W.qweight + ((size_t)e * N + n) * (K / 2) + 16 * (lane >> 5);
    }
  }

  // the tile's scales for the whole K (resident in LDS), then ring stages
  // 0..3 <- chunks 0..3 (chunks past the end re-read the last one)
  const uint32_t ring = lds_addr(smem);
  const uint32_t sc_lds = ring + kStages * P::kStage;
  // SK: this lane's scale-run source for chunk 0 (the wave's tile rows
  // 64*wave .. 64*wave+63; rows past N re-read the last row)
  SkSrc skc{nullptr, 0u, 0};
  if constexpr (SK != 0 && FMT == FMT_GPTQ) {
    const int ng = K / W.group, c0 = nt0 + 64 * wave_u;
    skc.gsh = 31 - __builtin_clz((unsigned)(W.group / 64));
    if (lane < 32) {
      skc.p = W.scales + ((size_t)e * ng * N + min(c0 + 2 * lane, N - 2)) * 2;
      skc.stride = (uint32_t)N * 2;
    } else {
      skc.p = reinterpret_cast<const uint8_t*>(W.zeros) +
              ((size_t)e * ng * (N / 8) + min(c0 / 8 + min(lane - 32, 7), N / 8 - 1)) * 4;
      skc.stride = (uint32_t)N / 2;
    }
  } else if constexpr (SK != 0) {
    const int chunks = FMT == FMT_NVFP4 ? K / 64 : (K + 127) / 128;
    skc.p = W.scales_kc + ((size_t)e * chunks * N + min(nt0 + 64 * wave_u + lane, N - 1)) * 4;
    skc.stride = (uint32_t)N * 4;
    skc.gsh = FMT == FMT_NVFP4 ? 0 : 1;
  }
  const int nchunks = K / kPfBK;  // (K < 64: only the 32-wide tail, no LDS)
  if (nchunks == 0 || !dma_wave || SK) {
  } else if (FMT == FMT_NVFP4) {
    const int nb = rows * (K / 16);
    pf_dma_region(sc_lds, W.scales + ((size_t)e * N + nt0) * (K / 16), 0, nb, nb, nb, wave_u, lane);
  } else if (FMT == FMT_MXFP4) {
    const int nb = rows * (K / 32);
    pf_dma_region(sc_lds, W.scales + ((size_t)e * N + nt0) * (K / 32), 0, nb, nb, nb, wave_u, lane);
  } else {
    // fp16 scales [groups][BN] and packed zero points [groups][BN/8]; columns
    // past N are left unfilled (N % 32 == 0 keeps every piece 16-byte aligned)
    const int ng = K / W.group;
    pf_dma_region(sc_lds, W.scales + ((size_t)e * ng * N + nt0) * 2, (size_t)N * 2, P::BN * 2,
                  rows * 2, ng * P::BN * 2, wave_u, lane);
    pf_dma_region(sc_lds + ng * P::BN * 2,
                  reinterpret_cast<const uint8_t*>(W.zeros) + ((size_t)e * ng * (N / 8) + nt0 / 8) * 4,
                  (size_t)N / 2, P::BN / 2, rows / 2, ng * P::BN / 2, wave_u, lane);
  }
  if (nchunks > 0 && dma_wave) {
#pragma unroll
    for (int s = 0; s < kStages; ++s)
      pf_issue<FMT, BM, NF, SK>(ring + s * P::kStage, arow, brow, skc, min(s, nchunks - 1), wave_u, N);
  }

  // tile rows of this lane's fragments (columns past N read row 0)
  int rl[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = frag32_row<EPI>(n0, j, c);
    rl[j] = n < N ? n - nt0 : 0;
  }

  f32x16 acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // live fragments among this wave's MI (wave-uniform: the slot ids are the
  // same for all lanes)
  const int nact_w = __builtin_amdgcn_readfirstlane(min(max(nact - rpart * MI, 0), MI));

  if (KS == 2 && nchunks > 0) {
    wait_vmcnt<(kStages - 1) * P::kIssue>();
    pf_barrier();
    const int s0 = 2 * kp, s1 = 2 * kp + 1;
    PfB b[NF];
    uint4 a0[MI], a1[MI];
    bf16x8 q0[NF], q1[NF];
    pf_read_b<FMT, EPI, NF, SK>(b, smem + P::kABytes, SK ? smem + P::kABytes + P::kBBytes : scale_lds, rl,
                                0, h, K, W.group, P::BN);
    pf_read_a<MI>(a0, smem + aoff, c, h, s0);
#pragma unroll
    for (int j = 0; j < NF; ++j) q0[j] = pf_deq_step<FMT>(b[j], s0);
    for (int kc = 0; kc < nchunks; ++kc) {
      const uint8_t* st = smem + (kc % kStages) * P::kStage + aoff;
      pf_read_a<MI>(a1, st, c, h, s1);
#pragma unroll
      for (int j = 0; j < NF; ++j) q1[j] = pf_deq_step<FMT>(b[j], s1);
      pf_mfma<MI, NF>(acc, a0, q0);
      // chunk kc+1 has landed and every wave is past its reads of chunk kc
      wait_vmcnt<(kStages - 2) * P::kIssue>();
      pf_barrier();
      if (dma_wave)
        pf_issue<FMT, BM, NF, SK>(ring + (kc % kStages) * P::kStage, arow, brow, skc,
                                  min(kc + kStages, nchunks - 1), wave_u, N);
      const uint8_t* nx = smem + ((kc + 1) % kStages) * P::kStage;
      pf_read_b<FMT, EPI, NF, SK>(b, nx + P::kABytes, SK ? nx + P::kABytes + P::kBBytes : scale_lds, rl,
                                  min(kc + 1, nchunks - 1), h, K,
                              W.group, P::BN);
      pf_read_a<MI>(a0, nx + aoff, c, h, s0);
      pf_mfma<MI, NF>(acc, a1, q1);
#pragma unroll
      for (int j = 0; j < NF; ++j) q0[j] = pf_deq_step<FMT>(b[j], s0);
    }
  } else if (nchunks > 0) {
    // scales and chunk 0 have landed (chunks 1..3 may still be in flight)
    wait_vmcnt<(kStages - 1) * P::kIssue>();
    pf_barrier();
    // the K loop with the wave's first MA row fragments (MA < MI: the tile's
    // later 32-row fragments hold only padding rows, whose MFMAs and A reads
    // are skipped); one copy of the loop per MA, chosen once per tile
    auto kloop = [&](auto ma_tag) {
      constexpr int MA = decltype(ma_tag)::value;
      // chunk 0: weights, step-0 A fragments and dequant
      PfB b[NF];
      uint4 a0[MI], a1[MI];
      bf16x8 q0[NF], q1[NF];
      pf_read_b<FMT, EPI, NF, SK>(b, smem + P::kABytes, SK ? smem + P::kABytes + P::kBBytes : scale_lds, rl,
                                  0, h, K, W.group, P::BN);
      pf_read_a<MI, MA>(a0, smem + aoff, c, h, 0);
#pragma unroll
      for (int j = 0; j < NF; ++j) q0[j] = pf_deq_step<FMT>(b[j], 0);
      // one chunk, in ring stage ST = kc % kStages (a constant, so every LDS
      // read of the chunk is a lane offset plus an immediate)
      auto chunk = [&](int kc, auto st_tag) {
        const int ST = st_tag, NX = ST + 1 < kStages ? ST + 1 : 0;
        const uint8_t* st = smem + ST * P::kStage + aoff;
        // steps 0..2: each overlaps the next step's A reads and dequant
        pf_read_a<MI, MA>(a1, st, c, h, 1);
#pragma unroll
        for (int j = 0; j < NF; ++j) q1[j] = pf_deq_step<FMT>(b[j], 1);
        pf_mfma<MI, NF, MA>(acc, a0, q0);
        pf_read_a<MI, MA>(a0, st, c, h, 2);
#pragma unroll
        for (int j = 0; j < NF; ++j) q0[j] = pf_deq_step<FMT>(b[j], 2);
        pf_mfma<MI, NF, MA>(acc, a1, q1);
        pf_read_a<MI, MA>(a1, st, c, h, 3);
#pragma unroll
        for (int j = 0; j < NF; ++j) q1[j] = pf_deq_step<FMT>(b[j], 3);
        pf_mfma<MI, NF, MA>(acc, a0, q0);
        // step 3 overlaps chunk kc+1's reads: chunk kc+1 has landed (all but the
        // two newest chunks' DMA are done) and every wave is past its reads of
        // chunk kc, whose stage is refilled with chunk kc+kStages
        wait_vmcnt<(kStages - 2) * P::kIssue>();
        pf_barrier();
        const uint8_t* nx = smem + NX * P::kStage;
        if constexpr (SK != 0) {
          // every wave copies (one per SIMD): its DMA goes between step 3's rows
          pf_read_b<FMT, EPI, NF, SK>(b, nx + P::kABytes, nx + P::kABytes + P::kBBytes, rl,
                                      min(kc + 1, nchunks - 1), h, K, W.group, P::BN);
          pf_read_a<MI, MA>(a0, nx + aoff, c, h, 0);
          pf_mfma_issue<FMT, BM, NF, SK, MI, MA>(acc, a1, q1, ring + ST * P::kStage, arow, brow, skc,
                                                 min(kc + kStages, nchunks - 1), wave_u, N);
        } else {
          if (dma_wave)
            pf_issue<FMT, BM, NF, SK>(ring + ST * P::kStage, arow, brow, skc,
                                      min(kc + kStages, nchunks - 1), wave_u, N);
          pf_read_b<FMT, EPI, NF, SK>(b, nx + P::kABytes, scale_lds, rl, min(kc + 1, nchunks - 1), h, K,
                                      W.group, P::BN);
          pf_read_a<MI, MA>(a0, nx + aoff, c, h, 0);
          pf_mfma<MI, NF, MA>(acc, a1, q1);
        }
#pragma unroll
        for (int j = 0; j < NF; ++j) q0[j] = pf_deq_step<FMT>(b[j], 0);
      };
      // kStages chunks per trip, then the last nchunks % kStages
      int kc = 0;
      for (; kc + kStages <= nchunks; kc += kStages) {
        chunk(kc, std::integral_constant<int, 0>{});
        chunk(kc + 1, std::integral_constant<int, 1>{});
        chunk(kc + 2, std::integral_constant<int, 2>{});
        if constexpr (kStages == 4) chunk(kc + 3, std::integral_constant<int, 3 % kStages>{});
      }
      if (kc < nchunks) chunk(kc++, std::integral_constant<int, 0>{});
      if (kc < nchunks) chunk(kc++, std::integral_constant<int, 1>{});
      if constexpr (kStages == 4)
        if (kc < nchunks) chunk(kc++, std::integral_constant<int, 2>{});
    };
    if ((SK != 0 && n0 >= N) || nact_w == 0) {
      // every weight row of this wave lies past N (the last column tile), or
      // all its rows are padding: only its share of the copies, which leaves
      // its SIMD to the other workgroup (or wave) on it
      for (int kc = 0; kc < nchunks; ++kc) {
        wait_vmcnt<(kStages - 2) * P::kIssue>();
        pf_barrier();
        if (SK != 0 || dma_wave)
          pf_issue<FMT, BM, NF, SK>(ring + (kc % kStages) * P::kStage, arow, brow, skc,
                                    min(kc + kStages, nchunks - 1), wave_u, N);
      }
    } else if (nact_w >= MI) {
      kloop(std::integral_constant<int, MI>{});
    } else if constexpr (MI >= 2) {
      if (nact_w == 1) kloop(std::integral_constant<int, 1>{});
      else if constexpr (MI >= 3) {
        if (nact_w == 2) kloop(std::integral_constant<int, 2>{});
        else if constexpr (MI >= 4) kloop(std::integral_constant<int, 3>{});
      }
    }
  }
  // no DMA may land in LDS after this workgroup is gone
  wait_vmcnt<0>();
  const bool poison = gidx_bad<FMT>(W, e, K, tid, 256 * RS * KS);

  const int row0 = rowb + rpart * MI * 32;
  if (K % kPfBK && kp == 0) pf_tail32<FMT, EPI, MI, NF>(acc, ga, W, e, row0, n0, c, h, nchunks * kPfBK);

  // (slot id, routing weight) of every block row, in the last KB of LDS
  // (beyond what the K-split exchange uses); one load of the weights per tile
  int2* rowtab = reinterpret_cast<int2*>(smem + P::kLds - P::kRowTab);
  {
    const bool use_tw = ea.mul_tw;
    const float tw = use_tw ? ea.topk_w[min(row_sid, ea.n_slots - 1)] : 1.f;
    pf_barrier();  // every wave is past its reads of the ring and the scale tile
    if (tid < BM) rowtab[tid] = int2{row_sid, __float_as_int(tw)};
  }

  if constexpr (KS == 2) {
    // the two K parts meet: each wave hands over the half of the rows the
    // other finalises (lane-major in LDS, the ring is free now), then adds
    // the other's half of its own rows and runs the epilogue on them
    constexpr int HM = MI / 2;
    constexpr int kRed = HM * NF * 16 * 64;  // floats per wave
    float* red = reinterpret_cast<float*>(smem);
    float* mine = red + (size_t)(wave_u * 2 + kp) * kRed;
    const float* theirs = red + (size_t)(wave_u * 2 + (1 - kp)) * kRed;
    f32x16 acch[HM][NF];
    if (kp == 0) {
#pragma unroll
      for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) mine[((i * NF + j) * 16 + v) * 64 + lane] = acc[HM + i][j][v];
    } else {
#pragma unroll
      for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) mine[((i * NF + j) * 16 + v) * 64 + lane] = acc[i][j][v];
    }
    pf_barrier();
    if (kp == 0) {
#pragma unroll
      for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acch[i][j][v] = acc[i][j][v] + theirs[((i * NF + j) * 16 + v) * 64 + lane];
    } else {
#pragma unroll
      for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acch[i][j][v] = theirs[((i * NF + j) * 16 + v) * 64 + lane] + acc[HM + i][j][v];
    }
    if (n0 >= N) return;
    EpiArgs a = ea;
    a.row0 = row0 + kp * HM * 32;
    epilogue32<EPI, FMT, HM, NF>(acch, a, W, e, n0, lane, rowtab, a.row0 - rowb, poison);
    return;
  }

  pf_barrier();  // the row table is complete
  if (n0 >= N) return;
  EpiArgs a = ea;
  a.row0 = row0;
  epilogue32<EPI, FMT, MI, NF>(acc, a, W, e, n0, lane, rowtab, row0 - rowb, poison);
}

// --------------------------------------------------------------------------
// decode kernel
// --------------------------------------------------------------------------
//
// A few rows per expert: the weight stream is the whole cost.  Workgroup =
// one row block (16*MI slots) x 16*NF weight rows (NF = 2 or 4), with
// nw = 1, 2 or 4 waves that split K into contiguous runs of 128-wide chunks.
// The tile's scales (contiguous in memory for NVFP4/MXFP4) are copied once
// into LDS with full-width loads, so the per-chunk loads are only the 4-bit
// codes and the A fragments.  Each wave walks its run with kDcDepth chunks of
// those in flight in registers (a ring of slots, every load issued
// unconditionally so the compiler can count exactly what is outstanding), so
// the HBM stream never stops for a chunk's multiply; the waves' partial sums
// are added through LDS in wave order (deterministic) and the epilogue is
// spread over the waves.  The host picks nw so that the launch has enough
// waves in flight when few experts are routed.

constexpr int kDcBK = 128;    // K chunk
constexpr int kDcDepth = 4;   // chunks in flight per wave
// LDS scale tile of one workgroup of R weight rows: NVFP4 [R rows][K/16]
// e4m3 bytes, MXFP4 [R rows][K/32] e8m0 bytes, GPTQ [K/G][R columns] fp16
// scales followed by [K/G][R/8] packed zero-point words.  With the scales by
// K chunk the NVFP4/MXFP4 tile keeps that layout, [KC][R rows][4 bytes]
// (64-deep chunks for NVFP4, 128-deep for MXFP4), so it copies in runs of
// 4R bytes; the MXFP4 size covers both layouts.
__host__ __device__ inline int dc_scale_bytes(int fmt, int K, int group, int R) {
  if (fmt == FMT_NVFP4) return R * (K / 16);
  if (fmt == FMT_MXFP4) return 4 * R * ((K + 127) / 128);
  return (K / group) * (R * 2 + R / 2);
}

// Copy the tile's scales (weight rows n0 .. n0 + R - 1, those below N) into LDS.
template <int FMT, int R>
__device__ __forceinline__ void dc_stage_scales(uint8_t* sc, const WeightArgs& W, int e, int n0,
                                                int N, int K, int tid, int nthreads) {
  const int rows = min(R, N - n0);  // a multiple of 16
  if ((FMT == FMT_NVFP4 || FMT == FMT_MXFP4) && W.scales_kc != nullptr) {
    // [KC][R][4]: chunk c's 4 * rows bytes from its [N][4] row run
    constexpr int CH = FMT == FMT_NVFP4 ? 64 : 128;
    const int kcn = (K + CH - 1) / CH;
    const uint8_t* src = W.scales_kc + ((size_t)e * kcn * N + n0) * 4;
    for (int u = tid; u < kcn * (R / 4); u += nthreads) {
      const int c = u / (R / 4), x = 16 * (u % (R / 4));
      if (x < 4 * rows)
        *reinterpret_cast<uint4*>(sc + c * 4 * R + x) =
            *reinterpret_cast<const uint4*>(src + (size_t)c * N * 4 + x);
    }
  } else if (FMT == FMT_NVFP4 || FMT == FMT_MXFP4) {
    const int per_row = (FMT == FMT_NVFP4) ? K / 16 : K / 32;
    const uint8_t* src = W.scales + ((size_t)e * N + n0) * per_row;
    const int units = rows * per_row / 16;  // rows * per_row is a multiple of 16
    for (int u = tid; u < units; u += nthreads)
      reinterpret_cast<uint4*>(sc)[u] = reinterpret_cast<const uint4*>(src)[u];
  } else {
    const int ng = K / W.group;
    const uint8_t* s16 = W.scales + ((size_t)e * ng * N + n0) * 2;
    for (int u = tid; u < ng * (rows / 8); u += nthreads) {  // 16-byte pieces of fp16 scales
      const int gr = u / (rows / 8), q = u % (rows / 8);
      reinterpret_cast<uint4*>(sc + gr * R * 2)[q] =
          *reinterpret_cast<const uint4*>(s16 + (size_t)gr * N * 2 + 16 * q);
    }
    const uint32_t* z = W.zeros + (size_t)e * ng * (N / 8) + n0 / 8;
    uint32_t* zl = reinterpret_cast<uint32_t*>(sc + ng * R * 2);
    for (int u = tid; u < ng * (rows / 8); u += nthreads) {  // one zero-point word per 8 columns
      const int gr = u / (rows / 8), q = u % (rows / 8);
      zl[gr * (R / 8) + q] = z[(size_t)gr * (N / 8) + q];
    }
  }
}

// NVFP4/MXFP4: the scale tile (contiguous in memory) copied by LDS-DMA, so
// that its loads go out ahead of the weight stream and need no registers;
// the kernel waits for them with wait_vmcnt, counting the loads it issued
// after them.
template <int FMT, int R>
__device__ __forceinline__ void dc_dma_scales(uint8_t* sc, const WeightArgs& W, int e, int n0,
                                              int N, int K, int rows, int wave, int nw, int lane) {
  if (W.scales_kc != nullptr) {
    // [KC][R][4] (see dc_scale_bytes): 16-byte piece o of the tile is chunk
    // o / 4R, bytes o % 4R of its row run (rows past N left unfilled)
    constexpr int CH = FMT == FMT_NVFP4 ? 64 : 128;
    const int kcn = (K + CH - 1) / CH;
    const uint8_t* src = W.scales_kc + ((size_t)e * kcn * N + n0) * 4;
    const int bytes = kcn * 4 * R;
    const uint32_t base = lds_addr(sc);
    for (int q = __builtin_amdgcn_readfirstlane(wave); q * 1024 < bytes; q += nw) {
      const int o = q * 1024 + 16 * lane;
      const int c = o / (4 * R), x = o % (4 * R);
      if (o < bytes && x < 4 * rows) dma16(src + (size_t)c * N * 4 + x, base + q * 1024);
    }
    return;
  }
  const int per_row = (FMT == FMT_NVFP4) ? K / 16 : K / 32;
  const uint8_t* src = W.scales + ((size_t)e * N + n0) * per_row;
  const int bytes = rows * per_row;  // a multiple of 16
  const uint32_t base = lds_addr(sc);
  for (int q = __builtin_amdgcn_readfirstlane(wave); q * 1024 < bytes; q += nw) {
    const int o = q * 1024 + 16 * lane;
    if (o < bytes) dma16(src + o, base + q * 1024);
  }
}

// LDS bytes before the partial-sum area (the scale tile, 16-byte aligned end).
__host__ __device__ inline int dc_scale_region(int fmt, int K, int group, int R) {
  return (dc_scale_bytes(fmt, K, group, R) + 15) & ~15;
}

// Raw scale words of one fragment for the lane's k range [kl, kl + C/4), from
// the LDS tile (r = the fragment row's index inside the tile; kc: the tile
// has the by-chunk layout).
template <int FMT, int C, int R>
__device__ __forceinline__ void dc_fill_scales(BChunk<FMT, C>& b, const uint8_t* sc, int r, int K,
                                               int group, int kl, bool kc) {
  if (FMT == FMT_NVFP4) {
    const uint8_t* sp = kc ? sc + ((kl / 64) * R + r) * 4 + (kl % 64) / 16 : sc + r * (K / 16) + kl / 16;
    if (C == 256) {
      b.sr[0] = *reinterpret_cast<const uint16_t*>(sp);
      b.sr[1] = *reinterpret_cast<const uint16_t*>(sp + 2);
    } else if (C == 128) {
      b.sr[0] = *reinterpret_cast<const uint16_t*>(sp);
    } else {
      b.sr[0] = *sp;
    }
  } else if (FMT == FMT_MXFP4) {
    const uint8_t* sp = kc ? sc + ((kl / 128) * R + r) * 4 + (kl % 128) / 32 : sc + r * (K / 32) + kl / 32;
    b.sr[0] = sp[0];
    if (C == 256) b.sr[1] = sp[1];
  } else {
    const int gr = kl / group;
    b.sr[0] = reinterpret_cast<const uint16_t*>(sc)[gr * R + r];
    b.sr[1] = reinterpret_cast<const uint32_t*>(sc + (K / group) * R * 2)[gr * (R / 8) + (r >> 3)];
    b.zsh = 4 * (r & 7);
  }
}

// One wave's share of a K chunk: the weight codes of NF fragments, and
// separately its A fragments (A comes from L2 and needs a shallower ring).
template <int FMT, int C, int NF>
struct DcB {
  BChunk<FMT, C> b[NF];
};
template <int C, int MI>
struct DcA {
  uint4 a[MI][C / 32];
};

template <int FMT, int C, int NF>
__device__ __forceinline__ void dc_load_b(DcB<FMT, C, NF>& d, const WeightArgs& W, const GemmArgs& ga,
                                          const int (&nrow)[NF], int e, int k0, int g) {
#pragma unroll
  for (int j = 0; j < NF; ++j) load_codes<FMT, C>(d.b[j], W, e, nrow[j], ga.N, ga.K, k0 + g * (C / 4));
}
// The same with the lane's k offset given.
template <int FMT, int C, int NF>
__device__ __forceinline__ void dc_load_b(DcB<FMT, C, NF>& d, const WeightArgs& W, const GemmArgs& ga,
                                          const int (&nrow)[NF], int e, int kl) {
#pragma unroll
  for (int j = 0; j < NF; ++j) load_codes<FMT, C>(d.b[j], W, e, nrow[j], ga.N, ga.K, kl);
}

// Padding slots read A row 0 (a_row), so every lane loads and no branch is
// needed; their products only reach accumulator rows the epilogue skips.
template <int C, int MI>
__device__ __forceinline__ void dc_load_a(DcA<C, MI>& d, const uint16_t* const (&arow)[MI], int k0,
                                          int g) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int s = 0; s < C / 32; ++s)
      d.a[i][s] = *reinterpret_cast<const uint4*>(arow[i] + k0 + g * (C / 4) + 8 * s);
}

template <int FMT, int C, int MI, int NF, int R = 16 * NF>
__device__ __forceinline__ void dc_compute(f32x4 (&acc)[MI][NF], const DcB<FMT, C, NF>& db,
                                           const DcA<C, MI>& da, const uint8_t* sc,
                                           const int (&rl)[NF], int K, int group, int g, int k0,
                                           bool kc) {
  BChunk<FMT, C> b[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    b[j] = db.b[j];
    dc_fill_scales<FMT, C, R>(b[j], sc, rl[j], K, group, k0 + g * (C / 4), kc);
  }
#pragma unroll
  for (int s = 0; s < C / 32; ++s) {
    bf16x8 bf[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) bf[j] = deq_step<FMT, C>(b[j], s);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const bf16x8 af = as_bf16x8(da.a[i][s]);
#pragma unroll
      for (int j = 0; j < NF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
    }
  }
}

// One unpipelined chunk of width C (the K tail).
template <int FMT, int C, int MI, int NF, int R = 16 * NF>
__device__ __forceinline__ void dc_chunk(f32x4 (&acc)[MI][NF], const WeightArgs& W,
                                         const GemmArgs& ga, const uint16_t* const (&arow)[MI],
                                         const int (&nrow)[NF], const int (&rl)[NF],
                                         const uint8_t* sc, int e, int k0, int g) {
  DcB<FMT, C, NF> db;
  DcA<C, MI> da;
  dc_load_b(db, W, ga, nrow, e, k0, g);
  dc_load_a(da, arow, k0, g);
  dc_compute<FMT, C, MI, NF, R>(acc, db, da, sc, rl, ga.K, W.group, g, k0, W.scales_kc != nullptr);
}

template <int FMT, int EPI, int MI, int NF>
__global__ void __launch_bounds__(256) gemm_decode_kernel(GemmArgs ga, WeightArgs W, EpiArgs ea) {
  constexpr int BM = 16 * MI;
  extern __shared__ __attribute__((aligned(16))) uint8_t dc_smem[];  // scale tile, then [nw][MI][NF][64] partials

  const int mb = blockIdx.x / ga.n_ntiles, nt = blockIdx.x % ga.n_ntiles;
  if (mb * BM >= ga.num_post_pad[0]) return;
  const int e = ga.expert_ids[mb * BM / ga.block_m];  // BM divides block_m
  if (e < 0 || e >= ga.E) return;

  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = nt * 16 * NF;
  const int K = ga.K;
  uint8_t* const sc = dc_smem;

  const uint16_t* arow[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) arow[i] = a_row(ga, ga.sorted_ids[mb * BM + i * 16 + c16]);
  int nrow[NF], rl[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    nrow[j] = frag_on<EPI>(n0, j, ga.N) ? frag_row<EPI>(n0, j, c16) : n0;
    rl[j] = nrow[j] - n0;
  }

  f32x4 acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's run of full chunks [c0, c0 + n).  Weight codes run kDcDepth
  // chunks ahead; A fragments as far for one 16-row block (they are issued
  // with the codes of the same chunk, so waiting for one chunk's A never
  // waits for younger codes), two for two blocks (registers).  The scale
  // tile's loads go out first (NVFP4/MXFP4).
  constexpr int kADepth = (MI == 1) ? 4 : 2;
  const int nfull = K / kDcBK;
  const int c0 = nfull * wave / nw, n = nfull * (wave + 1) / nw - c0;
  const int last = max(c0 + n - 1, 0);
  const int srows = min(16 * NF, ga.N - n0);
  DcB<FMT, kDcBK, NF> b0, b1, b2, b3;
  DcA<kDcBK, MI> a0, a1, a2, a3;
  if (n > 0 && FMT != FMT_GPTQ) {
    // (n is the same on all lanes of a wave, and every wave reaches exactly
    // one of the two barriers)
    dc_dma_scales<FMT, 16 * NF>(sc, W, e, n0, ga.N, K, srows, wave, nw, lane);
    dc_load_b(b0, W, ga, nrow, e, c0 * kDcBK, g);
    dc_load_a(a0, arow, c0 * kDcBK, g);
    dc_load_b(b1, W, ga, nrow, e, min(c0 + 1, last) * kDcBK, g);
    dc_load_a(a1, arow, min(c0 + 1, last) * kDcBK, g);
    dc_load_b(b2, W, ga, nrow, e, min(c0 + 2, last) * kDcBK, g);
    if (kADepth == 4) dc_load_a(a2, arow, min(c0 + 2, last) * kDcBK, g);
    dc_load_b(b3, W, ga, nrow, e, min(c0 + 3, last) * kDcBK, g);
    if (kADepth == 4) dc_load_a(a3, arow, min(c0 + 3, last) * kDcBK, g);
    // the scale DMAs are older than these prologue loads: wait for them only
    constexpr int kPro = kDcDepth * NF * (kDcBK / 128) + kADepth * MI * (kDcBK / 32);
    wait_vmcnt<kPro>();
    pf_barrier();
  } else if (n > 0) {
    dc_load_b(b0, W, ga, nrow, e, c0 * kDcBK, g);
    dc_load_a(a0, arow, c0 * kDcBK, g);
    dc_load_b(b1, W, ga, nrow, e, min(c0 + 1, last) * kDcBK, g);
    dc_load_a(a1, arow, min(c0 + 1, last) * kDcBK, g);
    dc_load_b(b2, W, ga, nrow, e, min(c0 + 2, last) * kDcBK, g);
    if (kADepth == 4) dc_load_a(a2, arow, min(c0 + 2, last) * kDcBK, g);
    dc_load_b(b3, W, ga, nrow, e, min(c0 + 3, last) * kDcBK, g);
    if (kADepth == 4) dc_load_a(a3, arow, min(c0 + 3, last) * kDcBK, g);
    dc_stage_scales<FMT, 16 * NF>(sc, W, e, n0, ga.N, K, tid, 64 * nw);
    __syncthreads();
  } else {
    dc_stage_scales<FMT, 16 * NF>(sc, W, e, n0, ga.N, K, tid, 64 * nw);
    __syncthreads();
  }
  const int group = W.group;
  const bool kc = W.scales_kc != nullptr;  // scale tile in the by-chunk layout
  // groups of four chunks in straight-line code (no exit between the
  // phases, so every prefetch is issued where it is written); chunk
  // c0 + i + d sits in b<d> and a<d % kADepth>; once multiplied its slots
  // take chunk + 4 (codes) and chunk + kADepth (A); past the run the last
  // chunk is fetched again and never used
  const int n4 = n & ~3;
  for (int i = 0; i < n4; i += kDcDepth) {
#define MOE_DC_PHASE(D, BS, AS)                                                                    \
    {                                                                                              \
      dc_compute(acc, BS, AS, sc, rl, K, group, g, (c0 + i + D) * kDcBK, kc);                      \
      dc_load_b(BS, W, ga, nrow, e, min(c0 + i + D + 4, last) * kDcBK, g);                         \
      dc_load_a(AS, arow, min(c0 + i + D + kADepth, last) * kDcBK, g);                             \
    }
    MOE_DC_PHASE(0, b0, a0)
    MOE_DC_PHASE(1, b1, a1)
    MOE_DC_PHASE(2, b2, (kADepth == 4 ? a2 : a0))
    MOE_DC_PHASE(3, b3, (kADepth == 4 ? a3 : a1))
#undef MOE_DC_PHASE
  }
  // the run's last n % 4 chunks are already in the ring
  const int rem = n - n4;
  if (rem > 0) {
    dc_compute(acc, b0, a0, sc, rl, K, group, g, (c0 + n4) * kDcBK, kc);
    if (kADepth == 2 && rem > 2) dc_load_a(a0, arow, (c0 + n4 + 2) * kDcBK, g);
  }
  if (rem > 1) dc_compute(acc, b1, a1, sc, rl, K, group, g, (c0 + n4 + 1) * kDcBK, kc);
  if (rem > 2)
    dc_compute(acc, b2, (kADepth == 4 ? a2 : a0), sc, rl, K, group, g, (c0 + n4 + 2) * kDcBK, kc);
  // K tail (K % 128: a 64- and/or a 32-wide piece) on the last wave
  if (wave == nw - 1) {
    int k0 = nfull * kDcBK;
    if (K - k0 >= 64) {
      dc_chunk<FMT, 64, MI, NF>(acc, W, ga, arow, nrow, rl, sc, e, k0, g);
      k0 += 64;
    }
    if (K - k0 >= 32) dc_chunk<FMT, 32, MI, NF>(acc, W, ga, arow, nrow, rl, sc, e, k0, g);
  }

  const bool poison = gidx_bad<FMT>(W, e, K, tid, 64 * nw);
  EpiArgs a = ea;
  a.row0 = mb * BM;
  if (nw == 1) {
    epilogue<EPI, FMT, MI, NF>(acc, a, W, e, n0, lane, poison);
    return;
  }
  // add the waves' partial sums in wave order
  f32x4* red = reinterpret_cast<f32x4*>(dc_smem + dc_scale_region(FMT, K, group, 16 * NF));
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) red[((wave * MI + i) * NF + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  // wave w finishes fragment groups w, w + nw, ...: one fragment (plain) or one
  // gate/up pair (gated) each
  constexpr int GF = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int kGroups = NF / GF;
  for (int grp = wave; grp < kGroups; grp += nw) {
    f32x4 fin[MI][GF];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < GF; ++q) {
        const int j = grp * GF + q;
        f32x4 sum = red[(i * NF + j) * 64 + lane];
        for (int w2 = 1; w2 < nw; ++w2) {
          const f32x4 t = red[((w2 * MI + i) * NF + j) * 64 + lane];
          sum[0] += t[0];
          sum[1] += t[1];
          sum[2] += t[2];
          sum[3] += t[3];
        }
        fin[i][q] = sum;
      }
    // the fragment group as its own "wave" starting at weight row n0 + 16*GF*grp
    epilogue<EPI, FMT, MI, GF>(fin, a, W, e, n0 + 16 * GF * grp, lane, poison);
  }
}

// --------------------------------------------------------------------------
// wide decode kernel
// --------------------------------------------------------------------------
//
// For a few to a few dozen rows per expert with enough (expert, column tile)
// pairs to fill the chip.  Workgroup = 16*MI rows x 128 weight rows over the
// whole K: four waves of 32 weight rows each, so every A chunk (16*MI rows x
// 128 k, bf16) is fetched once per workgroup instead of once per 32 columns.
// Each thread loads 16 bytes of it per 16 rows into a register ring as deep
// as the codes ring, writes it to one of two LDS stages a chunk ahead of
// use, and all four waves read their MFMA fragments from there (16-byte
// slots of a row XOR-swizzled by the row, so a fragment read is free of bank
// conflicts).  One barrier per chunk.  The codes stream per wave into a
// 4-deep register ring; the tile's scales sit in LDS (NVFP4/MXFP4 copied by
// LDS-DMA ahead of the stream).  The compiler counts every load but the
// scale DMA, which the kernel waits for itself.

constexpr int kWdCols = 128;  // weight rows per workgroup (4 waves x 32)
constexpr int kWdBK = 128;    // K chunk
constexpr int kWdDepth = 4;   // chunks in flight per wave

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Everything the epilogue reads besides the accumulators, loaded at the start
// so that its latency hides behind the weight stream: the slot ids of the
// lane's rows (i*16 + 4g + r), their routing weights, the lane's bias values
// and the NVFP4 global scale.  The routing weight scales GEMM2's output row,
// or GEMM1's accumulator when it is applied on the input instead.
template <int MI, int NF>
struct EpiPre {
  int sid[MI][4];
  float tw[MI][4];
  float bias[NF];
  float gsc;
};

// Every load is unconditional: a load inside a branch makes the compiler
// wait for it at the branch's end.  Without a bias (or routing weights) the
// load reads some other valid global word and the epilogue ignores it; rows
// with the sentinel slot id read some valid routing weight, also unused.
// (Both candidate bases are kernel-argument pointers, so the load stays a
// global one: a flat load would make every later wait a full drain.)

// Part 1: slot ids, bias, global scale.
template <int EPI, int FMT, int MI, int NF>
__device__ __forceinline__ void epi_prefetch_ids(EpiPre<MI, NF>& p, const EpiArgs& a,
                                                 const WeightArgs& W, int e, int n0, int lane) {
  const int c16 = lane & 15, g = lane >> 4;
  p.gsc = (FMT == FMT_NVFP4) ? W.global_scale[e] : 1.f;
  const bool has_bias = W.bias != nullptr;
  const uint16_t* bbase = has_bias ? W.bias : reinterpret_cast<const uint16_t*>(W.qweight != nullptr ? W.qweight : W.qweight_kc);
  const int bmul = has_bias ? 1 : 0;
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int row = frag_on<EPI>(n0, j, a.N) ? frag_row<EPI>(n0, j, c16) : n0;
    p.bias[j] = bf16_bits_to_f32(bbase[((size_t)e * a.N + row) * bmul]);
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) p.sid[i][r] = a.sorted_ids[a.row0 + i * 16 + 4 * g + r];
}

// Part 2: routing weights (GEMM2), once the slot ids are in.
template <int EPI, int MI, int NF>
__device__ __forceinline__ void epi_prefetch_tw(EpiPre<MI, NF>& p, const EpiArgs& a) {
  const bool use = a.mul_tw;
  const float* tbase = use ? a.topk_w : reinterpret_cast<const float*>(a.sorted_ids);
  const int tmul = use ? 1 : 0;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) p.tw[i][r] = tbase[min(p.sid[i][r], a.n_slots - 1) * tmul];
}

// The epilogue of the 16x16 fragments with prefetched metadata (same
// arithmetic as epilogue()).
template <int EPI, int MI, int NF>
__device__ __forceinline__ void epilogue_pre(const f32x4 (&acc)[MI][NF], const EpiPre<MI, NF>& p,
                                             const EpiArgs& a, const WeightArgs& W, int n0,
                                             int lane) {
  const int c16 = lane & 15;
  float bias[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) bias[j] = (W.bias != nullptr) ? p.bias[j] : 0.f;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sid = p.sid[i][r];
      if (sid >= a.n_slots) continue;
      uint16_t* orow = a.out + (size_t)sid * a.out_ld;
      const float tw = a.mul_tw ? p.tw[i][r] : 1.f;
      const float gin = (EPI == EPI_DOWN) ? p.gsc : p.gsc * tw;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int q = 0; q < NF / 2; ++q) {
          if (!frag_on<EPI>(n0, 2 * q, a.N)) continue;
          const float gate = acc[i][2 * q][r] * gin + bias[2 * q];
          const float up = acc[i][2 * q + 1][r] * gin + bias[2 * q + 1];
          const float v = act_swigluoai(gate, up, a.alpha, a.beta, a.limit);
          orow[n0 / 2 + 16 * q + c16] = f32_to_bf16_bits(v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          if (!frag_on<EPI>(n0, j, a.N)) continue;
          float v = acc[i][j][r] * gin + bias[j];
          if (EPI == EPI_RELU2) {
            v = act_relu2(v);
          } else if (EPI == EPI_DOWN) {
            v = v * tw;
          }
          orow[n0 + 16 * j + c16] = f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// A pieces of one chunk held by one thread: 16 bytes per 16 rows.  Piece q of
// thread t is row 16q + t/16, 16-byte slot t%16 of the chunk.
template <int MI>
struct WdA {
  u32x4 v[MI];  // native vectors (HIP's uint4 struct copies would keep the ring in memory)
};

// The last chunk may pass K (K % 128 != 0): its A pieces past K are stored as
// zeros and read from a clamped address, so the weights the same lanes load
// there (also from clamped addresses: real, finite values) add nothing.
template <int MI>
__device__ __forceinline__ void wd_load_a(WdA<MI>& r, const uint16_t* const (&prow)[MI], int k0,
                                          int slot, int K) {
#pragma unroll
  for (int q = 0; q < MI; ++q)
    r.v[q] = *reinterpret_cast<const u32x4*>(prow[q] + min(k0 + 8 * slot, K - 8));
}

// LDS stage: [16*MI rows][16 slots of 16 bytes], the slot XOR-swizzled by the
// row so that the 16 rows of a fragment read hit distinct banks.
template <int MI>
__device__ __forceinline__ void wd_store_a(uint8_t* stage, const WdA<MI>& r, int tid, int k0, int K) {
  // (k0 passes through an empty asm so that the select below, which needs
  // the loaded value, cannot be hoisted ahead of the loads issued before)
  asm volatile("" : "+v"(k0));
  const bool live = k0 + 8 * (tid & 15) < K;
#pragma unroll
  for (int q = 0; q < MI; ++q) {
    const int row = 16 * q + (tid >> 4), slot = tid & 15;
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(stage + row * 256 + ((slot ^ (row & 15)) << 4)) = live ? r.v[q] : z;
  }
}

// Multiply one chunk: the wave's codes of NF fragments (dequantised with the
// scales of the LDS tile) by the A fragments read step by step from the stage
// (row i*16 + c16, k = 32g + 8s .. +8).  kl = the lane's clamped k offset.
template <int FMT, int MI, int NF>
__device__ __forceinline__ void wd_compute(f32x4 (&acc)[MI][NF], const DcB<FMT, kWdBK, NF>& db,
                                           const uint8_t* stage, const uint8_t* sc,
                                           const int (&rl)[NF], int K, int group, int g, int c16,
                                           int kl, bool kc) {
  BChunk<FMT, kWdBK> b[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    b[j] = db.b[j];
    dc_fill_scales<FMT, kWdBK, kWdCols>(b[j], sc, rl[j], K, group, kl, kc);
  }
#pragma unroll
  for (int s = 0; s < kWdBK / 32; ++s) {
    bf16x8 bf[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) bf[j] = deq_step<FMT, kWdBK>(b[j], s);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = i * 16 + c16, slot = 4 * g + s;
      const bf16x8 af =
          as_bf16x8(*reinterpret_cast<const uint4*>(stage + row * 256 + ((slot ^ c16) << 4)));
#pragma unroll
      for (int j = 0; j < NF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
    }
  }
}

template <int FMT, int EPI, int MI>
__global__ void __launch_bounds__(256, (MI == 1 ? 4 : 3)) gemm_wide_kernel(GemmArgs ga, WeightArgs W, EpiArgs ea) {
  constexpr int BM = 16 * MI, NF = 2, C = kWdBK, D = kWdDepth;
  constexpr int kStage = BM * C * 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t wd_smem[];  // scale tile, 2 A stages

  const int mb = blockIdx.x / ga.n_ntiles, nt = blockIdx.x % ga.n_ntiles;
  const int npp = ga.num_post_pad[0];
  const int e = ga.expert_ids[mb * BM / ga.block_m];  // BM divides block_m
  if (mb * BM >= npp || e < 0 || e >= ga.E) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = nt * kWdCols, n0w = n0 + 32 * wave;
  const int K = ga.K, group = W.group;
  uint8_t* const sc = wd_smem;
  uint8_t* const stages = wd_smem + dc_scale_region(FMT, K, group, kWdCols);

  // chunks of 128 (the last may be partial); a lane's 32-wide k range is
  // entirely inside K or entirely past it (K % 32 == 0); past it the lane
  // loads codes and scales of its last valid range (clamped) and the A it
  // meets there is zero
  const int n = (K + C - 1) / C;
  const int last = n - 1;
  const int kmax = K - C / 4;  // largest lane offset
  const int srows = min(kWdCols, ga.N - n0);

  // prologue, in issue order: the scale DMA (it needs only the expert), the
  // slot ids and the epilogue's metadata, the codes of chunks 0 .. D-1, then
  // (once the slot ids are in -- which, loads retiring in order, also means
  // the DMA has landed) the A pieces of chunks 0 .. D-1.
  if (FMT != FMT_GPTQ) dc_dma_scales<FMT, kWdCols>(sc, W, e, n0, ga.N, K, srows, wave, 4, lane);
  const bool kc = W.scales_kc != nullptr;  // scale tile in the by-chunk layout
  int psid[MI];  // slots of the A rows this thread copies
#pragma unroll
  for (int q = 0; q < MI; ++q) psid[q] = ga.sorted_ids[mb * BM + 16 * q + (tid >> 4)];
  const int slot = tid & 15;
  int nrow[NF], rl[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    nrow[j] = frag_on<EPI>(n0w, j, ga.N) ? frag_row<EPI>(n0w, j, c16) : n0;
    rl[j] = nrow[j] - n0;
  }
  EpiArgs ep = ea;
  ep.row0 = mb * BM;
  EpiPre<MI, NF> pre;
  epi_prefetch_ids<EPI, FMT, MI, NF>(pre, ep, W, e, n0w, lane);
  f32x4 acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  DcB<FMT, C, NF> b[D];
  WdA<MI> r[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
    dc_load_b(b[d], W, ga, nrow, e, min(min(d, last) * C + g * (C / 4), kmax));
  const uint16_t* prow[MI];
#pragma unroll
  for (int q = 0; q < MI; ++q) prow[q] = a_row(ga, psid[q]);
  // the slot ids are waited for here, before any A load is issued
#pragma unroll
  for (int q = 0; q < MI; ++q) asm volatile("" : : "v"(prow[q]) : "memory");
  epi_prefetch_tw<EPI, MI, NF>(pre, ep);
#pragma unroll
  for (int d = 0; d < D; ++d) wd_load_a(r[d], prow, min(d, last) * C, slot, K);
  if (FMT == FMT_GPTQ) dc_stage_scales<FMT, kWdCols>(sc, W, e, n0, ga.N, K, tid, 256);
  wd_store_a(stages, r[0], tid, 0, K);
  pf_barrier();

  // phase c (ring slot d = c % D): multiply chunk c (codes in b[d], A in
  // stage c % 2); refill the slot with chunk c + D; then move chunk c + 1's
  // A from its ring slot into the other stage (read by every wave in phase
  // c - 1, which the previous barrier closed) and barrier.  Past the end the
  // last chunk is fetched again and never used.  The first group of D
  // phases is written out before the loop: the loads in flight when it
  // starts differ from those at the loop's back edge, and a shared loop
  // entry would make the compiler's waits drain the ring every iteration.
#define MOE_WD_PHASE(c, d)                                                                         \
  {                                                                                                \
    wd_compute<FMT, MI, NF>(acc, b[d], stages + ((c) & 1) * kStage, sc, rl, K, group, g, c16,      \
                            min((c) * C + g * (C / 4), kmax), kc);                                 \
    dc_load_b(b[d], W, ga, nrow, e, min(min((c) + D, last) * C + g * (C / 4), kmax));              \
    wd_load_a(r[d], prow, min((c) + D, last) * C, slot, K);                                        \
    asm volatile("" ::: "memory"); /* the loads above go out before the store waits */             \
    wd_store_a(stages + (((c) + 1) & 1) * kStage, r[((d) + 1) % D], tid, ((c) + 1) * C, K);        \
    pf_barrier();                                                                                  \
  }
  const int nd = n - n % D;
  if (nd > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) MOE_WD_PHASE(d, d)
  }
  for (int i = D; i < nd; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) MOE_WD_PHASE(i + d, d)
  }
#undef MOE_WD_PHASE
  // the last n % D chunks are already in the rings
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    if (nd + d < n) {  // the same for the whole workgroup
      const int c = nd + d;
      wd_compute<FMT, MI, NF>(acc, b[d], stages + (c & 1) * kStage, sc, rl, K, group, g, c16,
                              min(c * C + g * (C / 4), kmax), kc);
      wd_store_a(stages + ((c + 1) & 1) * kStage, r[(d + 1) % D], tid, (c + 1) * C, K);
      pf_barrier();
    }
  }
  if (gidx_bad<FMT>(W, e, K, tid, 256)) pre.gsc = __builtin_nanf("");
  epilogue_pre<EPI, MI, NF>(acc, pre, ep, W, n0w, lane);
}

// --------------------------------------------------------------------------
// launch
// --------------------------------------------------------------------------

// Decode launch: 32-row weight tiles (64-row ones measured no faster at
// 64 tokens); K split over nw waves per workgroup when few units would leave
// the chip short of waves.
template <int FMT, int EPI, int MI, int NF>
static void launch_decode_nf(GemmArgs ga, const WeightArgs& W, const EpiArgs& ea, long units,
                             hipStream_t st) {
  ga.n_ntiles = (ga.N + 16 * NF - 1) / (16 * NF);
  const int nw = units >= 4096 ? 1 : units >= 2048 ? 2 : 4;
  const size_t lds = (size_t)dc_scale_region(FMT, ga.K, W.group, 16 * NF) +
                     (nw > 1 ? (size_t)nw * MI * NF * 64 * sizeof(f32x4) : 0);
  gemm_decode_kernel<FMT, EPI, MI, NF>
      <<<dim3(ga.n_mblocks * ga.n_ntiles), dim3(64 * nw), lds, st>>>(ga, W, ea);
}

// LDS of the wide kernel: the 128-row scale tile and two A stages.
static inline size_t wide_lds(int fmt, int K, int group, int MI) {
  return (size_t)dc_scale_region(fmt, K, group, kWdCols) + 2 * (size_t)(16 * MI) * kWdBK * 2;
}
constexpr size_t kWdMaxLds = 64 * 1024;
// Wide kernel when the (expert block, 128-column tile) pairs alone give the
// chip enough workgroups; otherwise the split-K kernel.  The caller's kernel
// argument can force either (KERNEL_WIDE where its LDS fits).
constexpr long kWdMinTiles = 640;

template <int FMT, int EPI, int MI>
static void launch_decode(GemmArgs ga, const WeightArgs& W, const EpiArgs& ea, int blocks_est,
                          int kernel, hipStream_t st) {
  const long wide_tiles = (long)blocks_est * ((ga.N + kWdCols - 1) / kWdCols);
  const size_t lds = wide_lds(FMT, ga.K, W.group, MI);
  const bool want_wide = kernel == KERNEL_WIDE || (kernel == KERNEL_AUTO && wide_tiles >= kWdMinTiles);
  if (want_wide && lds <= kWdMaxLds) {
    ga.n_ntiles = (ga.N + kWdCols - 1) / kWdCols;
    gemm_wide_kernel<FMT, EPI, MI>
        <<<dim3(ga.n_mblocks * ga.n_ntiles), dim3(256), lds, st>>>(ga, W, ea);
    return;
  }
  launch_decode_nf<FMT, EPI, MI, 2>(ga, W, ea, (long)blocks_est * ((ga.N + 31) / 32), st);
}

// The streaming (prefill) kernel reads each chunk's scales with its codes
// (no resident scale tile, any K): NVFP4/MXFP4 given the scales by K chunk,
// GPTQ with groups of 64 * 2^j rows (a chunk then lies in one group, whose
// scale and zero-point rows the checkpoint stores contiguous over N).
static inline bool prefill_streams(int fmt, int group, bool scales_kc) {
  return fmt == FMT_GPTQ ? group >= 64 && (group & (group - 1)) == 0 : scales_kc;
}
// The streaming kernel's tiles fit: scales streamed, or the tile's scales for
// the whole K in its LDS (the resident-scale variant); GPTQ zero-point rows in
// 16-byte pieces.  Otherwise 64/128-row blocks run the split-K kernel on
// 32-row sub-blocks.
static inline bool prefill_fits(int fmt, int K, int N, int group, bool streams) {
  if (fmt == FMT_GPTQ && N % 32 != 0) return false;
  return streams || pf_scale_bytes(fmt, K, group, Pf<128, 2>::BN) <= kPfScaleBytes;
}

template <int FMT, int EPI>
hipError_t launch_epi(int block_m, int cap, GemmArgs ga, const WeightArgs& W, EpiArgs ea,
                             int kernel, hipStream_t st) {
  ga.n_mblocks = cap / block_m;
  if (block_m <= 32) {
    // at most one block per routed expert is expected in this regime: the
    // number of routed experts bounds the blocks that hold slots
    const int blocks_est = ga.E < ga.n_slots ? ga.E : ga.n_slots;
    if (block_m == 16)
      launch_decode<FMT, EPI, 1>(ga, W, ea, blocks_est, kernel, st);
    else
      launch_decode<FMT, EPI, 2>(ga, W, ea, blocks_est, kernel, st);
  } else {
    // widest tile whose scales fit the kernel's LDS; otherwise the split-K kernel
    const bool streams = prefill_streams(FMT, W.group, W.scales_kc != nullptr);
    if (!prefill_fits(FMT, ga.K, ga.N, W.group, streams)) {
      if (ga.tiles != nullptr) return hipErrorInvalidValue;
      // very long K (scales too large for LDS), or GPTQ zero-point rows that
      // are not 16-byte multiples: the split-K kernel over 32-row sub-blocks
      // of the aligned blocks
      ga.n_mblocks = cap / 32;
      launch_decode<FMT, EPI, 2>(ga, W, ea, ga.n_mblocks, kernel, st);
      return hipGetLastError();
    }
    ga.n_ntiles = (ga.N + Pf<128, 2>::BN - 1) / Pf<128, 2>::BN;
    ga.group_m = 4;  // measured flat between 1 and 16 at the gpt-oss-20b shape
    const dim3 grid((ga.n_mblocks * ga.n_ntiles + 7) / 8 * 8);
    constexpr int kThreads = 256 * pf_rs<FMT>() * pf_ks<FMT>();
    if constexpr (FMT == FMT_GPTQ) {
      if (streams) {
        // scale and zero-point rows streamed: two 256-thread workgroups per CU
        if (block_m == 64)
          gemm_prefill_kernel<FMT, EPI, 64, 2, 1, 1, 1><<<grid, dim3(256), 0, st>>>(ga, W, ea);
        else
          gemm_prefill_kernel<FMT, EPI, 128, 2, 1, 1, 1><<<grid, dim3(256), 0, st>>>(ga, W, ea);
        return hipGetLastError();
      }
    } else {
      if (streams) {
        // scales (and codes) by K chunk: two 256-thread workgroups per CU
        if (W.qweight_kc != nullptr) {
          if (block_m == 64)
            gemm_prefill_kernel<FMT, EPI, 64, 2, 1, 1, 2><<<grid, dim3(256), 0, st>>>(ga, W, ea);
          else
            gemm_prefill_kernel<FMT, EPI, 128, 2, 1, 1, 2><<<grid, dim3(256), 0, st>>>(ga, W, ea);
        } else if (block_m == 64) {
          gemm_prefill_kernel<FMT, EPI, 64, 2, 1, 1, 1><<<grid, dim3(256), 0, st>>>(ga, W, ea);
        } else {
          gemm_prefill_kernel<FMT, EPI, 128, 2, 1, 1, 1><<<grid, dim3(256), 0, st>>>(ga, W, ea);
        }
        return hipGetLastError();
      }
    }
    if (block_m == 64) {
      gemm_prefill_kernel<FMT, EPI, 64, 2, pf_rs<FMT>(), pf_ks<FMT>(), 0>
          <<<grid, dim3(kThreads), 0, st>>>(ga, W, ea);
    } else {
      gemm_prefill_kernel<FMT, EPI, 128, 2, pf_rs<FMT>(), pf_ks<FMT>(), 0>
          <<<grid, dim3(kThreads), 0, st>>>(ga, W, ea);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
