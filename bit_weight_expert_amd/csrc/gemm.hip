// Grouped W4A16 GEMMs (GEMM1 with the gate/up weights, GEMM2 with the down
// weights) and the k-row sum, for gfx950.
//
// Both GEMMs run over the aligned blocks of moe_align: block b holds up to
// BM sorted slots that all route to expert e = expert_ids[b] ("moe_align_block_size"
// in the NVFP4 repro); its A rows are x[sorted_id / top_k] for GEMM1 and the
// intermediate row of the slot itself for GEMM2 (the top_k = 1 view).
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16).  Lane l works on column l%16 of a
// 16-column fragment and on k-group g = l/16.  A K chunk of width C is split
// in four: the lane owns the C/4 consecutive k at [k0 + g*C/4, k0 + (g+1)*C/4),
// holds their 4-bit codes in registers and dequantises 8 of them per MFMA
// step; step s reads the A fragment with the same k assignment, so every k
// is reduced exactly once (the order of a reduction is free).  C = 256/128
// for full chunks; the K tail is cut into 128/64/32-wide chunks, so K need
// only be a multiple of 32 and no MFMA step is spent on padding.  No padded
// buffer is read or written (hidden 2880 = 11*256 + 64 = 22*128 + 64).
//
// Two kernels share the chunk loaders, the dequantisers and the epilogue:
//   prefill  many rows per expert.  Workgroup = BM (64/128) rows x 128
//            columns; four waves split the columns, 32 each, so every weight
//            is fetched and dequantised once per workgroup and no LDS is spent
//            on weights.  A is staged by LDS-DMA into a double-buffered,
//            XOR-swizzled LDS tile (128-wide chunks); the next chunk's A and
//            weight codes (raw scale words included, decoded only when used,
//            so no wait for the load is forced early) are in flight while the
//            current chunk is multiplied.  Tiles are ordered expert-block-major
//            within groups of 4 column tiles and handed out so that each XCD
//            works on a contiguous run, keeping a weight tile and an A block
//            in one XCD's L2 while they are reused.
//   decode   a few rows per expert: the weight stream is the whole cost.
//            Workgroup = 16*MI rows x 16*NF columns; each wave owns one or
//            more 256-wide K chunks (up to 12 waves for one row block, 8 for
//            two), reads A straight from global memory, and the waves add
//            their partial sums through LDS in wave order (deterministic);
//            the epilogue is then spread over the waves.
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

// Load the lane's k range [kl, kl + C/4) of weight row n of expert e.
template <int FMT, int C>
__device__ __forceinline__ void load_chunk(BChunk<FMT, C>& b, const WeightArgs& W, int e, int n,
                                           int N, int K, int kl) {
  constexpr int S = BChunk<FMT, C>::kSteps;
  if (FMT == FMT_NVFP4 || FMT == FMT_MXFP4) {
    const size_t row = (size_t)e * N + n;
    const uint8_t* p = W.qweight + row * (size_t)(K / 2) + kl / 2;
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
    if (FMT == FMT_NVFP4) {
      // K % 32 == 0 makes K/16 even, so scale pairs are 2-byte aligned
      const uint8_t* sp = W.scales + row * (size_t)(K / 16) + kl / 16;
      if (C == 256) {
        b.sr[0] = *reinterpret_cast<const uint16_t*>(sp);
        b.sr[1] = *reinterpret_cast<const uint16_t*>(sp + 2);
      } else if (C == 128) {
        b.sr[0] = *reinterpret_cast<const uint16_t*>(sp);
      } else {
        b.sr[0] = *sp;
      }
    } else {
      const uint8_t* sp = W.scales + row * (size_t)(K / 32) + kl / 32;
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

// 8 dequantised bf16 weights of MFMA step st.
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
    const float s = __uint_as_float((raw & 0xffu) << 23);
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
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf((float)((w >> (4 * i)) & 15u), s, -zs);
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
                                         const WeightArgs& W, int e, int n0, int lane) {
  const int c16 = lane & 15, g = lane >> 4;
  const float gsc = (FMT == FMT_NVFP4) ? W.global_scale[e] : 1.f;
  float bias[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    bias[j] = 0.f;
    if (W.bias != nullptr && frag_on<EPI>(n0, j, a.N))
      bias[j] = bf16_bits_to_f32(W.bias[(size_t)e * a.N + frag_row<EPI>(n0, j, c16)]);
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sid = a.sorted_ids[a.row0 + i * 16 + 4 * g + r];
      if (sid >= a.n_slots) continue;
      uint16_t* orow = a.out + (size_t)sid * a.out_ld;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int p = 0; p < NF / 2; ++p) {
          if (!frag_on<EPI>(n0, 2 * p, a.N)) continue;
          float gate = acc[i][2 * p][r] * gsc + bias[2 * p];
          float up = acc[i][2 * p + 1][r] * gsc + bias[2 * p + 1];
          gate = fminf(gate, a.limit);
          up = fminf(fmaxf(up, -a.limit), a.limit);
          const float v = gate * sigmoid_fast(a.alpha * gate) * (up + a.beta);
          orow[n0 / 2 + 16 * p + c16] = f32_to_bf16_bits(v);
        }
      } else {
        float tw = 1.f;
        if (EPI == EPI_DOWN && a.mul_tw) tw = a.topk_w[sid];
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          if (!frag_on<EPI>(n0, j, a.N)) continue;
          float v = acc[i][j][r] * gsc + bias[j];
          if (EPI == EPI_RELU2) {
            v = fmaxf(v, 0.f);
            v = v * v;
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

// Fragments (16 columns each) per wave of the prefill kernel.  Two (32-column
// waves, 128-column workgroups) at both block sizes: with four the software
// pipeline of a 128-row block (next fragments' codes and raw scales in flight
// while the current ones are multiplied) no longer fits in 256 VGPRs and spills.
#ifndef MOE_PF_NF
#define MOE_PF_NF 2
#endif
constexpr int kPfWaves = 4;
template <int BM, int FMT>
struct PfShape {
  static constexpr int NF = MOE_PF_NF;
  static constexpr int BN = kPfWaves * NF * 16;  // columns per workgroup
};
constexpr int kPfBK = 128;                    // K chunk staged in LDS
constexpr int kPfSlots = kPfBK / 8;           // 16-byte slots per LDS row
constexpr int kPfGroupN = 4;                  // column tiles per group in the tile order

struct GemmArgs {
  const uint16_t* A;
  int a_div;    // A row = sorted_id / a_div
  int n_slots;  // sentinel
  int K, N, E;
  int n_mblocks, n_ntiles;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* num_post_pad;
};

// A row of a sorted slot.  Padding slots read row 0 instead: their products
// land only in accumulator rows that the epilogue never stores (an MFMA row
// depends on its own A row only), so no zero-fill or branch is needed.
__device__ __forceinline__ const uint16_t* a_row(const GemmArgs& ga, int sid) {
  return ga.A + (size_t)(sid < ga.n_slots ? sid / ga.a_div : 0) * ga.K;
}

// LDS rows hold 16 slots of 16 bytes; slot q of row r is stored at q ^ (r % 16),
// so the 16 rows that one MFMA A fragment reads hit 16 different bank groups.
__device__ __forceinline__ int swz(int r, int q) { return q ^ (r & 15); }

// Logical tile of a workgroup: each XCD (workgroups are dealt to the 8 XCDs
// round-robin) gets a contiguous run of logical tiles; logical tiles run over
// groups of kPfGroupN column tiles, expert blocks ascending inside a group.
__device__ __forceinline__ bool prefill_tile(const GemmArgs& a, int& mb, int& nt) {
  const int total = a.n_mblocks * a.n_ntiles;
  const int per_xcd = (total + 7) / 8;
  const int pid = blockIdx.x;
  const int lid = (pid & 7) * per_xcd + (pid >> 3);
  if (lid >= total) return false;
  const int group_tiles = a.n_mblocks * kPfGroupN;
  const int grp = lid / group_tiles;
  const int rem = lid - grp * group_tiles;
  const int width = min(kPfGroupN, a.n_ntiles - grp * kPfGroupN);
  mb = rem / width;
  nt = grp * kPfGroupN + rem % width;
  return true;
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

// MFMA steps of one C-wide chunk: A fragments from the swizzled LDS tile.
template <int FMT, int C, int MI, int NF>
__device__ __forceinline__ void pf_compute(f32x4 (&acc)[MI][NF], const uint4 (*As)[kPfSlots],
                                           const BChunk<FMT, C> (&b)[NF], int c16, int g) {
  // Software-pipelined: the weights of step s+1 are dequantised (VALU) while
  // the MFMAs of step s run, so the matrix core and the vector ALU can work at
  // the same time.
  constexpr int S = C / 32;
  bf16x8 bcur[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) bcur[j] = deq_step<FMT, C>(b[j], 0);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    bf16x8 bnext[NF];
    if (s + 1 < S) {
#pragma unroll
      for (int j = 0; j < NF; ++j) bnext[j] = deq_step<FMT, C>(b[j], s + 1);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const bf16x8 af = as_bf16x8(As[i * 16 + c16][(g * S + s) ^ c16]);
#pragma unroll
      for (int j = 0; j < NF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bcur[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < S) {
#pragma unroll
      for (int j = 0; j < NF; ++j) bcur[j] = bnext[j];
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Stage one 128-wide A chunk straight from global memory into LDS (gfx950
// global_load_lds_dwordx4: lane l of a wave writes 16 bytes at base + 16*l).
// Pass p of wave w fills rows 16p + 4w .. 16p + 4w + 3; lane l writes physical
// slot l%16 of row 16p + 4w + l/16, so it fetches that row's logical slot
// (l%16) ^ (row%16) -- arow[p] already points there.
template <int NP>
__device__ __forceinline__ void pf_issue_a(uint4 (*As)[kPfSlots], const uint16_t* const (&arow)[NP],
                                           int k0, int wave) {
#pragma unroll
  for (int p = 0; p < NP; ++p)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(arow[p] + k0),
                                     (lds_void*)(&As[16 * p + 4 * wave][0]), 16, 0, 0);
}

// Wait for every outstanding global load of this wave (the A chunk's LDS DMA
// included), then for the whole workgroup.
__device__ __forceinline__ void pf_sync() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
}

// The K tail (K % 128, a multiple of 32) as one CW-wide chunk staged in As, unpipelined.
template <int FMT, int CW, int BM, int NF>
__device__ __forceinline__ void pf_tail(f32x4 (&acc)[BM / 16][NF], uint4 (*As)[kPfSlots],
                                        const GemmArgs& ga, const WeightArgs& W, int e, int mb,
                                        const int (&nrow)[NF], bool wave_on,
                                        int k0, int tid, int c16, int g) {
  constexpr int segs = CW / 8;
  for (int idx = tid; idx < BM * segs; idx += 256) {
    const int r = idx / segs, sg = idx % segs;
    As[r][swz(r, sg)] = *reinterpret_cast<const uint4*>(a_row(ga, ga.sorted_ids[mb * BM + r]) + k0 + sg * 8);
  }
  BChunk<FMT, CW> bt[NF];
  if (wave_on) load_frags<FMT, CW, NF>(bt, W, e, nrow, ga.N, ga.K, k0, g);
  __syncthreads();
  if (wave_on) pf_compute<FMT, CW, BM / 16, NF>(acc, As, bt, c16, g);
  __syncthreads();
}

template <int FMT, int EPI, int BM>
__global__ void __launch_bounds__(256, 2) gemm_prefill_kernel(GemmArgs ga, WeightArgs W, EpiArgs ea) {
  constexpr int MI = BM / 16;
  constexpr int NF = PfShape<BM, FMT>::NF;
  constexpr int kPasses = BM / 16;  // 16 rows staged per pass (4 per wave)
  // two separate LDS objects (not one [2][..] array), so the compiler can see
  // that the LDS-DMA filling one buffer never aliases the reads of the other
  // and need not wait for the DMA before every LDS read
  __shared__ uint4 As0[BM][kPfSlots];
  __shared__ uint4 As1[BM][kPfSlots];

  int mb, nt;
  if (!prefill_tile(ga, mb, nt)) return;
  if (mb * BM >= ga.num_post_pad[0]) return;
  const int e = ga.expert_ids[mb];
  if (e < 0 || e >= ga.E) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = nt * PfShape<BM, FMT>::BN + wave * NF * 16;
  const bool wave_on = n0 < ga.N;

  // A rows this lane stages (see pf_issue_a)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint16_t* arow[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int r = 16 * p + 4 * wave_u + (lane >> 4);
    arow[p] = a_row(ga, ga.sorted_ids[mb * BM + r]) + 8 * ((lane & 15) ^ (r & 15));
  }
  int nrow[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) nrow[j] = frag_on<EPI>(n0, j, ga.N) ? frag_row<EPI>(n0, j, c16) : 0;

  f32x4 acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nfull = ga.K / kPfBK;
  BChunk<FMT, kPfBK> b0[NF], b1[NF];

  // two chunks per trip: even chunks use LDS buffer 0 and b0, odd ones buffer 1 and b1;
  // each chunk's MFMAs overlap the loads of the next
  if (nfull > 0) {
    pf_issue_a<kPasses>(As0, arow, 0, wave_u);
    if (wave_on) load_frags<FMT, kPfBK, NF>(b0, W, e, nrow, ga.N, ga.K, 0, g);
  }
  pf_sync();
  for (int c = 0; c < nfull; c += 2) {
    const bool m1 = c + 1 < nfull;
    if (m1) {
      pf_issue_a<kPasses>(As1, arow, (c + 1) * kPfBK, wave_u);
      if (wave_on) load_frags<FMT, kPfBK, NF>(b1, W, e, nrow, ga.N, ga.K, (c + 1) * kPfBK, g);
    }
    if (wave_on) pf_compute<FMT, kPfBK, MI, NF>(acc, As0, b0, c16, g);
    pf_sync();
    if (!m1) break;
    const bool m2 = c + 2 < nfull;
    if (m2) {
      pf_issue_a<kPasses>(As0, arow, (c + 2) * kPfBK, wave_u);
      if (wave_on) load_frags<FMT, kPfBK, NF>(b0, W, e, nrow, ga.N, ga.K, (c + 2) * kPfBK, g);
    }
    if (wave_on) pf_compute<FMT, kPfBK, MI, NF>(acc, As1, b1, c16, g);
    pf_sync();
  }

  int k0 = nfull * kPfBK;
  if (ga.K - k0 >= 64) {
    pf_tail<FMT, 64, BM, NF>(acc, As0, ga, W, e, mb, nrow, wave_on, k0, tid, c16, g);
    k0 += 64;
  }
  if (ga.K - k0 >= 32) pf_tail<FMT, 32, BM, NF>(acc, As0, ga, W, e, mb, nrow, wave_on, k0, tid, c16, g);

  if (!wave_on) return;
  EpiArgs a = ea;
  a.row0 = mb * BM;
  epilogue<EPI, FMT, MI, NF>(acc, a, W, e, n0, lane);
}

// --------------------------------------------------------------------------
// decode kernel
// --------------------------------------------------------------------------

constexpr int kDcBK = 256;

// One wave's share of a K chunk: weights of NF fragments plus its A fragments.
template <int FMT, int C, int MI, int NF>
struct DcChunk {
  BChunk<FMT, C> b[NF];
  uint4 a[MI][C / 32];
};

// A rows of padding slots are not read (their lanes keep stale values, which
// only reach accumulator rows the epilogue skips).
template <int FMT, int C, int MI, int NF>
__device__ __forceinline__ void dc_load(DcChunk<FMT, C, MI, NF>& d, const WeightArgs& W,
                                        const GemmArgs& ga, const uint16_t* const (&arow)[MI],
                                        const bool (&aon)[MI], const int (&nrow)[NF], int e, int k0,
                                        int g) {
  load_frags<FMT, C, NF>(d.b, W, e, nrow, ga.N, ga.K, k0, g);
#pragma unroll
  for (int i = 0; i < MI; ++i)
    if (aon[i]) {
#pragma unroll
      for (int s = 0; s < C / 32; ++s)
        d.a[i][s] = *reinterpret_cast<const uint4*>(arow[i] + k0 + g * (C / 4) + 8 * s);
    }
}

template <int FMT, int C, int MI, int NF>
__device__ __forceinline__ void dc_compute(f32x4 (&acc)[MI][NF], const DcChunk<FMT, C, MI, NF>& d) {
#pragma unroll
  for (int s = 0; s < C / 32; ++s) {
    bf16x8 bf[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) bf[j] = deq_step<FMT, C>(d.b[j], s);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const bf16x8 af = as_bf16x8(d.a[i][s]);
#pragma unroll
      for (int j = 0; j < NF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
    }
  }
}

template <int FMT, int C, int MI, int NF>
__device__ __forceinline__ void dc_chunk(f32x4 (&acc)[MI][NF], const WeightArgs& W,
                                         const GemmArgs& ga, const uint16_t* const (&arow)[MI],
                                         const bool (&aon)[MI], const int (&nrow)[NF], int e,
                                         int k0, int g) {
  DcChunk<FMT, C, MI, NF> d;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int s = 0; s < C / 32; ++s) d.a[i][s] = uint4{0u, 0u, 0u, 0u};
  dc_load(d, W, ga, arow, aon, nrow, e, k0, g);
  dc_compute(acc, d);
}

// Workgroup = 16*MI rows x 16*NF columns and one wave per 256-wide K chunk
// (blockDim.x / 64 waves, at most MAXT / 64): every chunk of the tile is in
// flight at once, which is what a weight-streaming GEMV needs.  The waves'
// partial sums are added through LDS in wave order (deterministic).
template <int FMT, int EPI, int MI, int NF, int MAXT>
__global__ void __launch_bounds__(MAXT) gemm_decode_kernel(GemmArgs ga, WeightArgs W, EpiArgs ea) {
  constexpr int BM = 16 * MI;
  extern __shared__ f32x4 red[];  // [nw][MI][NF][64]

  const int mb = blockIdx.x / ga.n_ntiles, nt = blockIdx.x % ga.n_ntiles;
  if (mb * BM >= ga.num_post_pad[0]) return;
  const int e = ga.expert_ids[mb];
  if (e < 0 || e >= ga.E) return;

  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = nt * NF * 16;

  const uint16_t* arow[MI];
  bool aon[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int sid = ga.sorted_ids[mb * BM + i * 16 + c16];
    aon[i] = sid < ga.n_slots;
    arow[i] = a_row(ga, sid);
  }
  int nrow[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) nrow[j] = frag_on<EPI>(n0, j, ga.N) ? frag_row<EPI>(n0, j, c16) : 0;

  f32x4 acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nfull = ga.K / kDcBK;
  for (int c = wave; c < nfull; c += nw)
    dc_chunk<FMT, kDcBK, MI, NF>(acc, W, ga, arow, aon, nrow, e, c * kDcBK, g);
  // tail (K % 256) in 128/64/32-wide pieces, one wave each, after the last chunk owner
  int k0 = nfull * kDcBK;
  int tw = nfull % nw;
  if (ga.K - k0 >= 128) {
    if (wave == tw) dc_chunk<FMT, 128, MI, NF>(acc, W, ga, arow, aon, nrow, e, k0, g);
    k0 += 128;
    tw = (tw + 1) % nw;
  }
  if (ga.K - k0 >= 64) {
    if (wave == tw) dc_chunk<FMT, 64, MI, NF>(acc, W, ga, arow, aon, nrow, e, k0, g);
    k0 += 64;
    tw = (tw + 1) % nw;
  }
  if (ga.K - k0 >= 32) {
    if (wave == tw) dc_chunk<FMT, 32, MI, NF>(acc, W, ga, arow, aon, nrow, e, k0, g);
  }

  // reduce the partial sums in wave order
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) red[((wave * MI + i) * NF + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  // wave w finishes fragment groups w, w + nw, ...: one fragment (plain) or one
  // gate/up pair (gated) each
  constexpr int GF = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int kGroups = NF / GF;
  EpiArgs a = ea;
  a.row0 = mb * BM;
  for (int grp = wave; grp < kGroups; grp += nw) {
    f32x4 fin[MI][GF];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < GF; ++q) {
        const int j = grp * GF + q;
        f32x4 s = red[(i * NF + j) * 64 + lane];
        for (int w2 = 1; w2 < nw; ++w2) {
          const f32x4 t = red[((w2 * MI + i) * NF + j) * 64 + lane];
          s[0] += t[0];
          s[1] += t[1];
          s[2] += t[2];
          s[3] += t[3];
        }
        fin[i][q] = s;
      }
    // the fragment group as its own "wave" starting at weight row n0 + 16*GF*grp
    epilogue<EPI, FMT, MI, GF>(fin, a, W, e, n0 + 16 * GF * grp, lane);
  }
}

// --------------------------------------------------------------------------
// k-row sum
// --------------------------------------------------------------------------

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

// --------------------------------------------------------------------------
// launch
// --------------------------------------------------------------------------

template <int FMT, int EPI, int MI, int NF, int MAXT>
static void launch_decode_nw(const GemmArgs& ga, const WeightArgs& W, const EpiArgs& ea,
                             hipStream_t st) {
  const int chunks = ga.K / kDcBK + (ga.K % kDcBK ? 1 : 0);
  const int nw = chunks < MAXT / 64 ? chunks : MAXT / 64;
  const size_t lds = (size_t)nw * MI * NF * 64 * sizeof(f32x4);
  gemm_decode_kernel<FMT, EPI, MI, NF, MAXT>
      <<<dim3(ga.n_mblocks * ga.n_ntiles), dim3(64 * nw), lds, st>>>(ga, W, ea);
}

template <int FMT, int EPI, int MI>
static void launch_decode(int nf, const GemmArgs& ga, const WeightArgs& W, const EpiArgs& ea,
                          hipStream_t st) {
  constexpr int kMaxT = MI == 1 ? 768 : 512;
  if (nf == 2)
    launch_decode_nw<FMT, EPI, MI, 2, kMaxT>(ga, W, ea, st);
  else
    launch_decode_nw<FMT, EPI, MI, 4, kMaxT>(ga, W, ea, st);
}

template <int FMT, int EPI>
static hipError_t launch_epi(int block_m, int cap, GemmArgs ga, const WeightArgs& W, EpiArgs ea,
                             hipStream_t st) {
  ga.n_mblocks = cap / block_m;
  if (block_m <= 32) {
    // few rows per expert: split K inside the workgroup.  Narrow (32-column)
    // tiles when 64-column ones would leave fewer than two workgroups per CU
    // (at most one block per routed expert is expected in this regime).
    const int blocks_est = ga.E < ga.n_slots ? ga.E : ga.n_slots;
#ifdef MOE_DC_NF
    const int nf = MOE_DC_NF;
#else
    const int nf = (long)blocks_est * ((ga.N + 63) / 64) < 512 ? 2 : 4;
#endif
    ga.n_ntiles = (ga.N + 16 * nf - 1) / (16 * nf);
    if (block_m == 16)
      launch_decode<FMT, EPI, 1>(nf, ga, W, ea, st);
    else
      launch_decode<FMT, EPI, 2>(nf, ga, W, ea, st);
  } else {
    const int bn = block_m == 64 ? PfShape<64, FMT>::BN : PfShape<128, FMT>::BN;
    ga.n_ntiles = (ga.N + bn - 1) / bn;
    const int total = ga.n_mblocks * ga.n_ntiles;
    const dim3 grid((total + 7) / 8 * 8);
    if (block_m == 64)
      gemm_prefill_kernel<FMT, EPI, 64><<<grid, dim3(256), 0, st>>>(ga, W, ea);
    else
      gemm_prefill_kernel<FMT, EPI, 128><<<grid, dim3(256), 0, st>>>(ga, W, ea);
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(int epi, int block_m, int cap, const GemmArgs& ga, const WeightArgs& W,
                             const EpiArgs& ea, hipStream_t st) {
  switch (epi) {
    case EPI_SWIGLU: return launch_epi<FMT, EPI_SWIGLU>(block_m, cap, ga, W, ea, st);
    case EPI_RELU2: return launch_epi<FMT, EPI_RELU2>(block_m, cap, ga, W, ea, st);
    case EPI_NONE: return launch_epi<FMT, EPI_NONE>(block_m, cap, ga, W, ea, st);
    default: return launch_epi<FMT, EPI_DOWN>(block_m, cap, ga, W, ea, st);
  }
}

}  // namespace moe

// Launch one grouped GEMM.  cap = capacity of sorted_ids (the grid covers every
// block that could be used; blocks past num_post_pad exit at once).
extern "C" hipError_t moe_launch_gemm(int fmt, int epi, int block_m, int cap, const uint16_t* A,
                                      int a_div, int n_slots, int K, int N, int E,
                                      const moe::WeightArgs* W, const int32_t* sid,
                                      const int32_t* eid, const int32_t* npp, const float* tw,
                                      int mul, float alpha, float beta, float limit, uint16_t* out,
                                      int out_ld, hipStream_t st) {
  if (cap / block_m == 0) return hipSuccess;
  moe::GemmArgs ga{A, a_div, n_slots, K, N, E, 0, 0, sid, eid, npp};
  moe::EpiArgs ea{sid, 0, n_slots, N, tw, mul, alpha, beta, limit, out, out_ld};
  switch (fmt) {
    case moe::FMT_NVFP4: return moe::launch_fmt<moe::FMT_NVFP4>(epi, block_m, cap, ga, *W, ea, st);
    case moe::FMT_MXFP4: return moe::launch_fmt<moe::FMT_MXFP4>(epi, block_m, cap, ga, *W, ea, st);
    default: return moe::launch_fmt<moe::FMT_GPTQ>(epi, block_m, cap, ga, *W, ea, st);
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
