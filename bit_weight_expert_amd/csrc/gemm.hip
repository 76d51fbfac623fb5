// Grouped-GEMM launch dispatch, the MX-scaled kernel (MXFP8 activations x
// MXFP4 weights) and the k-row sum.  The W4A16 kernels and their launch
// rules are in gemm_impl.h; each (format, epilogue) pair of them is
// instantiated in its own translation unit (gemm_inst.hip, built once per
// pair), so the library builds in parallel.
#include "gemm_impl.h"

namespace moe {

#define MOE_LAUNCH_EPI_DECL(F, E)                                                              \
  extern template hipError_t launch_epi<F, E>(int, int, GemmArgs, const WeightArgs&, EpiArgs, int, \
                                              hipStream_t);
#define MOE_LAUNCH_EPI_DECL_FMT(F) \
  MOE_LAUNCH_EPI_DECL(F, EPI_SWIGLU) MOE_LAUNCH_EPI_DECL(F, EPI_RELU2) \
  MOE_LAUNCH_EPI_DECL(F, EPI_NONE) MOE_LAUNCH_EPI_DECL(F, EPI_DOWN)
MOE_LAUNCH_EPI_DECL_FMT(FMT_NVFP4)
MOE_LAUNCH_EPI_DECL_FMT(FMT_MXFP4)
MOE_LAUNCH_EPI_DECL_FMT(FMT_GPTQ)
#undef MOE_LAUNCH_EPI_DECL_FMT
#undef MOE_LAUNCH_EPI_DECL
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
// MXFP8 activations x MXFP4 weights: MX-scaled MFMA kernel (blocks of 64/128)
// --------------------------------------------------------------------------
//
// The A operand is MXFP8 as the quantiser writes it: e4m3 codes [rows][lda]
// (lda = K rounded up to 128, zero past K) and e8m0 scales [rows][lds]
// (lds = K/32 rounded up to 16, zero past K/32).  The weights are the MXFP4
// layout as is.  v_mfma_scale_f32_32x32x64_f8f6f4 multiplies e4m3 by e2m1 and
// applies both e8m0 scales per 32-deep block, so nothing is dequantised.
//
// Operand layout of one 64-deep step (measured on gfx950 with one-hot
// operands): lane (c, g), c = lane % 32, g = lane / 32, supplies
//   A  row c: k = 16g .. 16g+15 in bytes 0..15 and 32+16g .. 32+16g+15 in
//      bytes 16..31, and the scale of row c's 32-block g;
//   B  weight row c: k = 32g .. 32g+31 (16 bytes of codes), and the scale of
//      that row's block g.
// The accumulators have the layout of the bf16 32x32 MFMA (epilogue32).
//
// Tile: BM rows x 256 weight rows, four waves side by side over the weight
// rows (two 32-row fragments each), all BM rows per wave -- or, for 128-row
// blocks with streamed scales, a 2 x 2 grid of 64 rows x 128 weight rows per
// wave (each fragment then read from LDS by two waves).  K moves in chunks
// of 128 through an LDS ring filled by LDS-DMA (A: 128 bytes per row,
// 16-byte slot q of row r at a_slot(q, r); weights: 64 bytes per row at the
// row's position, slot q at q ^ ((position / 4) % 4)).  With the weight
// scales by K chunk both scale tiles stream with the chunks (2-deep ring, two
// workgroups per CU); otherwise they stay in LDS for the whole K (3-deep
// ring, eight waves, one workgroup per CU).

struct MxA {
  const uint8_t* codes;   // e4m3 [rows][lda]
  const uint8_t* scales;  // e8m0 [rows][lds]
  int lda, lds;
};

constexpr int kMxBK = 128;
constexpr int kMxStages = 3;
constexpr int kMxScaleBytes = 56 * 1024;
constexpr int kMxScaleIssue = 6;  // A-scale DMA instructions per wave (BM * lds <= 1536 pieces)

// RS = 2: eight waves, waves w and w + 4 take the same weight rows and one
// half of the A rows each, so one wave's LDS reads and waits overlap the
// other's MFMAs on the same SIMD.  NS: ring stages.  SS: both scale tiles
// stream with the chunks instead of staying resident (weights by K chunk:
// each stage holds the chunk's [BN][4] weight scale bytes and [BM][4] A
// scale bytes), so the workgroup waits for nothing but its first chunk and
// takes far less LDS.
template <int BM, int RS = 1, int NS = kMxStages, bool SS = false, int WR = 1>
struct Mx {
  static constexpr int NW = 4 * RS;                   // waves
  static constexpr int MI = BM / 32 / RS / WR;        // 32-row tiles per wave
  static constexpr int NF = 2 * WR;                   // 32-row weight fragments per wave
  static constexpr int BN = 4 / WR * NF * 32;
  static_assert(RS == 1 || WR == 1, "row split or a 2 x 2 wave grid, not both");
  static constexpr int kABytes = BM * kMxBK;
  static constexpr int kBBytes = BN * kMxBK / 2;
  static constexpr int kWsBytes = SS ? BN * 4 : 0;    // streamed weight scales of one chunk
  static constexpr int kAsBytes = SS ? 128 * 4 : 0;   // streamed A scales (room for 128 rows)
  static constexpr int kAIssue = kABytes / 1024 / NW;  // DMA instructions per wave per chunk
  static constexpr int kBIssue = kBBytes / 1024 / NW;
  static constexpr int kSIssue = SS ? 0 : (4 * kMxScaleIssue + NW - 1) / NW;  // A-scale DMA per wave
  static constexpr int kIssue = kAIssue + kBIssue + (SS ? 1 : 0);  // SS: one scale piece per wave
  static constexpr int kStage = kABytes + kBBytes + kWsBytes + kAsBytes;
  static constexpr int kLds = NS * kStage + (SS ? 0 : kMxScaleBytes);
  static_assert(kAIssue >= 1 && kBIssue >= 1, "tile too small for the DMA split");
  static_assert(NS >= 2 && (NS - 1) * kIssue < 64, "ring depth / vmcnt range");
  static_assert(kLds <= 160 * 1024, "LDS");
};

// LDS bytes of both scale tiles (weights: BN rows of K/32; A: BM rows of lds,
// rounded up to whole DMA instructions).
__host__ __device__ inline int mx_scale_bytes(int K, int bm, int lds) {
  const int b = (256 * (K / 32) + 1023) / 1024 * 1024;
  return b + (bm * lds + 1023) / 1024 * 1024;
}

// Position (0..255) of tile row r in the weight stage: 32-row blocks, gated
// tiles with the gate rows (even) before the up rows, so the eight lanes that
// one LDS cycle serves read eight consecutive positions.
template <int EPI>
__device__ __forceinline__ int mx_bpos(int r) {
  const int s = r & 31;
  return (r & ~31) + ((EPI == EPI_SWIGLU) ? (s >> 1) + 16 * (s & 1) : s);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16e __attribute__((ext_vector_type(16)));

// Operands of one 64-deep step: A fragments of the MI row tiles, weight
// fragments of the NF column fragments.
template <int MI, int NF>
struct MxOps {
  i32x8 a[MI];
  i32x8 b[NF];
};

// LDS reads of step ST (0 or 1) of the chunk in stage `stg` (A rows from r0;
// only the first MA row tiles: the rest hold padding rows only).
template <int MI, int NF, int ST, int MA = MI>
__device__ __forceinline__ void mx_read(MxOps<MI, NF>& o, const uint8_t* stg, int abytes,
                                        const int (&bpos)[NF], int c, int g, int r0) {
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int p = bpos[j];
    const uint4 v = *reinterpret_cast<const uint4*>(stg + abytes + p * 64 +
                                                    16 * ((2 * ST + g) ^ ((p >> 2) & 3)));
    o.b[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < MA; ++i) {
    const int r = r0 + 32 * i + c;
    const uint8_t* row = stg + r * 128;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * a_slot(4 * ST + g, r));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + 16 * a_slot(4 * ST + 2 + g, r));
    o.a[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

// The MA x NF MFMAs of one step (the live row tiles); byte 2*ST of each scale
// word is the lane's block.
template <int MI, int NF, int ST, int MA = MI>
__device__ __forceinline__ void mx_mfma(f32x16e (&acc)[MI][NF], const MxOps<MI, NF>& o,
                                        const int (&sa)[MI], const int (&sb)[NF]) {
#pragma unroll
  for (int i = 0; i < MA; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[i], o.b[j], acc[i][j], 0, 4,
                                                                   2 * ST, sa[i], 2 * ST, sb[j]);
}

// Scale words of chunk kc: A dword of blocks 4kc..4kc+3 shifted so bytes 0 / 2
// are this lane's blocks of steps 0 / 1; weight bytes likewise (blocks past
// K/32 read as 2^0: their A codes are zero).  kcs: the weight scale tile is
// [chunk][256 rows][4] (scales by K chunk; blocks past K/32 are zero bytes,
// a finite 2^-127 against zero A codes).
template <int MI, int NF>
__device__ __forceinline__ void mx_scales(int (&sa)[MI], int (&sb)[NF], const uint8_t* sca, int lds,
                                          const uint8_t* scb, int kb, const int (&rl)[NF], int c,
                                          int g, int kc, int r0, bool kcs) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
    sa[i] = (int)(*reinterpret_cast<const uint32_t*>(sca + (r0 + 32 * i + c) * lds + 4 * kc) >> (8 * g));
  const int b0 = 4 * kc + g, b1 = 4 * kc + 2 + g;
  if (kcs) {
#pragma unroll
    for (int j = 0; j < NF; ++j)
      sb[j] = (int)((*reinterpret_cast<const uint32_t*>(scb + kc * 1024 + rl[j] * 4) >> (8 * g)) &
                    0x00FF00FFu);
    return;
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const uint8_t* sr = scb + rl[j] * kb;
    const int s0 = sr[min(b0, kb - 1)];
    const int s1 = sr[min(b1, kb - 1)];
    sb[j] = (b0 < kb ? s0 : 127) | ((b1 < kb ? s1 : 127) << 16);
  }
}

template <int EPI, int BM, int RS, int NS, bool SS, int WR = 1>
__global__ void __launch_bounds__(256 * RS, SS && RS == 1 ? 2 : 1)
    gemm_mx_kernel(GemmArgs ga, MxA ma, WeightArgs W, EpiArgs ea) {
  using P = Mx<BM, RS, NS, SS, WR>;
  constexpr int MI = P::MI, NF = P::NF, NW = P::NW;
  __shared__ __attribute__((aligned(16))) uint8_t smem[P::kLds];

  int mb, nt;
  if (!prefill_tile(ga, BM, mb, nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int c = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // DMA share (0 .. NW-1)
  const int wave_u = wave & 3;                                 // DMA role
  // WR = 1: the four waves side by side over the weight rows; WR = 2: a 2 x 2
  // grid (half the A rows x half the weight rows each), so each A and each
  // weight fragment is read from LDS by two waves instead of A by four
  const int wave_r = WR == 2 ? (wave & 1) : 0;
  const int wave_c = WR == 2 ? (wave_u >> 1) : wave_u;          // weight-row group
  const int r0 = ((wave >> 2) * WR + wave_r) * MI * 32;        // this wave's first A row
  const int K = ga.K, N = ga.N, kb = K / 32;

  // slot ids of the A rows this lane copies (instruction q = NW*p + wave covers
  // rows 8q .. 8q+7) and of the A scale rows (resident tile: instruction
  // q = NW*i + wave covers 16-byte pieces 64q .. 64q+63 of the [BM][lds] tile;
  // streamed: waves 1 and 2 (mod 4) copy rows 0..63 and 64..127, one 4-byte
  // piece per lane), all requested before anything waits
  const int parts = ma.lds / 16;
  const int na = BM * parts;
  int sid[P::kAIssue], ssid[SS ? 1 : P::kSIssue];
#pragma unroll
  for (int p = 0; p < P::kAIssue; ++p) sid[p] = ga.sorted_ids[mb * BM + 8 * (NW * p + wave) + (lane >> 3)];
  if constexpr (SS) {
    ssid[0] = ga.sorted_ids[mb * BM + min((wave_u == 2 ? 64 : 0) + lane, BM - 1)];
  } else {
#pragma unroll
    for (int i = 0; i < P::kSIssue; ++i) {
      const int pc = min((NW * i + wave) * 64 + lane, na - 1);  // lanes past the end repeat the last piece
      ssid[i] = ga.sorted_ids[mb * BM + pc / parts];
    }
  }
  // 32-row tiles holding a real slot: a block's real slots come first (the
  // sort pads each expert's run at its end), so tile i is live when its first
  // slot is; this wave's live tiles among its MI (wave-uniform)
  int nact = 1;
#pragma unroll
  for (int i = 1; i < BM / 32; ++i) nact += ga.sorted_ids[mb * BM + 32 * i] < ga.n_slots ? 1 : 0;
  const int e = ga.expert_ids[mb];
  if (e < 0 || e >= ga.E) return;
  const int nact_w = __builtin_amdgcn_readfirstlane(min(max(nact - r0 / 32, 0), MI));

  const int nt0 = nt * P::BN;
  const int rows = min(P::BN, N - nt0);
  const int n0 = nt0 + wave_c * NF * 32;
  const int nchunks = (K + kMxBK - 1) / kMxBK;

  // DMA sources.  A: lane l writes physical slot l%8 of row r = 8q + l/8, so it
  // fetches logical slot a_slot(l%8, r).
  const uint8_t* arow[P::kAIssue];
#pragma unroll
  for (int p = 0; p < P::kAIssue; ++p) {
    const int r = 8 * (NW * p + wave) + (lane >> 3);
    const int s = sid[p];
    const int row = s < ga.n_slots ? (int)(((uint64_t)(uint32_t)s * ga.a_mul) >> 32) : 0;
    arow[p] = ma.codes + (size_t)row * ma.lda + 16 * a_slot(lane & 7, r);
  }
  // Weights: instruction q fills positions 16q .. 16q+15, lane l the physical
  // slot l%4 of position 16q + l/4 (rows past N re-read the last row; offsets
  // past the row's K/2 bytes re-read its last 16, multiplied by zero A codes).
  // codes by chunk ([E][ceil(K/128)][N][64], zero past K): one contiguous
  // kilobyte per instruction instead of 16 half cache lines
  const bool ck = W.qweight_kc != nullptr;
  const uint8_t* brow[P::kBIssue];
  int bls[P::kBIssue];
#pragma unroll
  for (int p = 0; p < P::kBIssue; ++p) {
    const int pos = 16 * (NW * p + wave) + (lane >> 2);
    const int n = min(nt0 + pf_brow<EPI>(pos >> 5, pos & 31), N - 1);
    brow[p] = ck ? W.qweight_kc + ((size_t)e * nchunks * N + n) * 64
                 : W.qweight + ((size_t)e * N + n) * (K / 2);
    bls[p] = 16 * ((lane & 3) ^ ((pos >> 2) & 3));
  }
  // Streamed scales (SS): this wave's piece of each chunk's scales.  Waves 0
  // and 3 (mod 4): the weight scales of all 256 tile rows, 16 bytes (four
  // rows) per lane (rows past N re-read the last four; the two waves write the
  // same bytes); waves 1 and 2: A rows 0..63 / 64..127, 4 bytes per lane
  // (rows past the tile re-read its last row).  Eight waves copy it twice.
  const uint8_t* ssrc = nullptr;
  uint32_t sdst = 0, sstride = 0;
  const uint32_t ring = lds_addr(smem);
  if constexpr (SS) {
    if (wave_u == 0 || wave_u == 3) {
      const int r = min(nt0 + 4 * lane, N - 4);
      ssrc = W.scales_kc + ((size_t)e * nchunks * N + r) * 4;
      sstride = (uint32_t)N * 4;
      sdst = P::kABytes + P::kBBytes;
    } else {
      const int s = ssid[0];
      const int row = s < ga.n_slots ? (int)(((uint64_t)(uint32_t)s * ga.a_mul) >> 32) : 0;
      ssrc = ma.scales + (size_t)row * ma.lds;
      sstride = 4;
      sdst = P::kABytes + P::kBBytes + P::kWsBytes + (wave_u == 2 ? 256 : 0);
    }
  }

  const uint8_t* scb = smem + NS * P::kStage;
  const int scb_bytes = SS ? 0 : (256 * kb + 1023) / 1024 * 1024;
  const uint8_t* sca = scb + scb_bytes;
  const bool kcs = W.scales_kc != nullptr;
  if constexpr (!SS) {
    // resident scale tiles: the weight scales of the tile rows (contiguous;
    // by K chunk: one kilobyte, [256 rows][4], per 128-deep chunk), then the
    // A scale rows
    const uint32_t scb_lds = ring + NS * P::kStage;
    const uint32_t sca_lds = scb_lds + scb_bytes;
    if (kcs) {
      const uint8_t* src = W.scales_kc + ((size_t)e * nchunks * N + nt0) * 4;
      for (int q = wave; q < nchunks; q += NW)
        if (16 * lane < 4 * rows) dma16(src + (size_t)q * N * 4 + 16 * lane, scb_lds + q * 1024);
    }
    const int nb = kcs ? 0 : rows * kb;   // a multiple of 16 (N % 16 == 0)
    const uint8_t* src = W.scales + ((size_t)e * N + nt0) * kb;
    for (int q = wave; q * 1024 < nb; q += NW)
      if (q * 1024 + 16 * lane < nb) dma16(src + q * 1024 + 16 * lane, scb_lds + q * 1024);
#pragma unroll
    for (int i = 0; i < P::kSIssue; ++i) {
      const int q = NW * i + wave;
      if (q * 64 >= na) break;
      const int pc = min(q * 64 + lane, na - 1);
      const int s = ssid[i];
      const int row = s < ga.n_slots ? (int)(((uint64_t)(uint32_t)s * ga.a_mul) >> 32) : 0;
      dma16(ma.scales + (size_t)row * ma.lds + 16 * (pc % parts), sca_lds + q * 1024);
    }
  }
  auto issue = [&](uint32_t stage, int kc) {
#pragma unroll
    for (int p = 0; p < P::kAIssue; ++p)
      dma16(arow[p] + kc * kMxBK, stage + (uint32_t)(NW * p + wave) * 1024u);
#pragma unroll
    for (int p = 0; p < P::kBIssue; ++p)
      dma16(brow[p] + (ck ? (size_t)kc * N * 64 + bls[p] : (size_t)min(kc * (kMxBK / 2) + bls[p], K / 2 - 16)),
            stage + P::kABytes + (uint32_t)(NW * p + wave) * 1024u);
    if constexpr (SS) {
      if (wave_u == 0 || wave_u == 3)
        dma16(ssrc + (size_t)kc * sstride, stage + sdst);
      else
        dma4(ssrc + (size_t)kc * sstride, stage + sdst);
    }
  };
#pragma unroll
  for (int s = 0; s < NS; ++s) issue(ring + s * P::kStage, min(s, nchunks - 1));

  // this lane's weight positions and scale rows
  int bpos[NF], rl[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = frag32_row<EPI>(n0, j, c);
    rl[j] = n < N ? n - nt0 : 0;
    bpos[j] = mx_bpos<EPI>(rl[j]);
  }

  f32x16e acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // scale words of chunk kc (from its stage, or the resident tiles)
  auto scales = [&](int (&sa)[MI], int (&sb)[NF], int kc) {
    if constexpr (SS) {
      const uint8_t* st = smem + (kc % NS) * P::kStage + P::kABytes + P::kBBytes;
#pragma unroll
      for (int i = 0; i < MI; ++i)
        sa[i] = (int)(*reinterpret_cast<const uint32_t*>(st + P::kWsBytes + (r0 + 32 * i + c) * 4) >> (8 * g));
#pragma unroll
      for (int j = 0; j < NF; ++j)
        sb[j] = (int)((*reinterpret_cast<const uint32_t*>(st + rl[j] * 4) >> (8 * g)) & 0x00FF00FFu);
    } else {
      mx_scales<MI, NF>(sa, sb, sca, ma.lds, scb, kb, rl, c, g, kc, r0, kcs);
    }
  };

  // scales and chunk 0 have landed.  Both 64-deep steps of every chunk run
  // (past K the A codes are zero), so the loop has no branch; each step's
  // LDS reads are issued while the other step's MFMAs run.  Only the wave's
  // first MA row tiles are multiplied (MA < MI: the later 32-row tiles hold
  // only padding rows); one copy of the loop per MA, chosen once per tile.
  wait_vmcnt<(NS - 1) * P::kIssue>();
  pf_barrier();
  auto kloop = [&](auto ma_tag) {
    constexpr int MA = decltype(ma_tag)::value;
    MxOps<MI, NF> o0, o1;
    int sa[MI], sb[NF];
    scales(sa, sb, 0);
    mx_read<MI, NF, 0, MA>(o0, smem, P::kABytes, bpos, c, g, r0);
    for (int kc = 0; kc < nchunks; ++kc) {
      const uint8_t* stg = smem + (kc % NS) * P::kStage;
      mx_read<MI, NF, 1, MA>(o1, stg, P::kABytes, bpos, c, g, r0);
      mx_mfma<MI, NF, 0, MA>(acc, o0, sa, sb);
      // chunk kc+1 has landed (only the NS-2 younger chunks may be in flight)
      // and every wave is past its reads of chunk kc, whose stage takes chunk
      // kc+NS
      wait_vmcnt<(NS - 2) * P::kIssue>();
      pf_barrier();
      issue(ring + (kc % NS) * P::kStage, min(kc + NS, nchunks - 1));
      int na_[MI], nb_[NF];
      const int kn = min(kc + 1, nchunks - 1);
      scales(na_, nb_, kn);
      mx_read<MI, NF, 0, MA>(o0, smem + (kn % NS) * P::kStage, P::kABytes, bpos, c, g, r0);
      mx_mfma<MI, NF, 1, MA>(acc, o1, sa, sb);
#pragma unroll
      for (int i = 0; i < MI; ++i) sa[i] = na_[i];
#pragma unroll
      for (int j = 0; j < NF; ++j) sb[j] = nb_[j];
    }
  };
  if (n0 >= N || nact_w == 0) {
    // every weight row of this wave lies past N (the last column tile), or
    // all its rows are padding: only its share of the copies, which leaves
    // its SIMD to the other waves
    for (int kc = 0; kc < nchunks; ++kc) {
      wait_vmcnt<(NS - 2) * P::kIssue>();
      pf_barrier();
      issue(ring + (kc % NS) * P::kStage, min(kc + NS, nchunks - 1));
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
  // no DMA may land in LDS after this workgroup is gone
  wait_vmcnt<0>();

  if (n0 >= N) return;
  EpiArgs a = ea;
  a.row0 = mb * BM + r0;
  f32x16 accv[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) accv[i][j][v] = acc[i][j][v];
  epilogue32<EPI, FMT_MXFP4, MI, NF>(accv, a, W, e, n0, lane);
}

template <int FMT>
static hipError_t launch_fmt(int epi, int block_m, int cap, const GemmArgs& ga, const WeightArgs& W,
                             const EpiArgs& ea, int kernel, hipStream_t st) {
  switch (epi) {
    case EPI_SWIGLU: return launch_epi<FMT, EPI_SWIGLU>(block_m, cap, ga, W, ea, kernel, st);
    case EPI_RELU2: return launch_epi<FMT, EPI_RELU2>(block_m, cap, ga, W, ea, kernel, st);
    case EPI_NONE: return launch_epi<FMT, EPI_NONE>(block_m, cap, ga, W, ea, kernel, st);
    default: return launch_epi<FMT, EPI_DOWN>(block_m, cap, ga, W, ea, kernel, st);
  }
}

}  // namespace moe

// Launch one grouped GEMM.  cap = capacity of sorted_ids (the grid covers every
// block that could be used; blocks past num_post_pad exit at once).
// tiles (optional, block_m = 128): the streaming kernel over a list of
// 128-row tiles with its length in n_tiles[0] (room for cap / 128 entries)
// instead of the aligned blocks; moe_prefill_tiles_ok must hold.
extern "C" hipError_t moe_launch_gemm(int fmt, int epi, int block_m, int cap, const uint16_t* A,
                                      int a_div, int n_slots, int K, int N, int E,
                                      const moe::WeightArgs* W, const int32_t* sid,
                                      const int32_t* eid, const int32_t* npp, const float* tw,
                                      int mul, float alpha, float beta, float limit, uint16_t* out,
                                      int out_ld, int kernel, const int2* tiles,
                                      const int32_t* n_tiles, hipStream_t st) {
  if (cap / block_m == 0) return hipSuccess;
  if (tiles != nullptr && block_m != 128) return hipErrorInvalidValue;
  const uint64_t a_mul = ((1ull << 32) + (uint64_t)a_div - 1) / (uint64_t)a_div;
  moe::GemmArgs ga{A, a_div, a_mul, n_slots, K, N, E, 0, 0, 1, block_m, sid, eid, npp, tiles, n_tiles};
  moe::EpiArgs ea{sid, 0, n_slots, N, tw, mul, alpha, beta, limit, out, out_ld};
  switch (fmt) {
    case moe::FMT_NVFP4: return moe::launch_fmt<moe::FMT_NVFP4>(epi, block_m, cap, ga, *W, ea, kernel, st);
    case moe::FMT_MXFP4: return moe::launch_fmt<moe::FMT_MXFP4>(epi, block_m, cap, ga, *W, ea, kernel, st);
    default: return moe::launch_fmt<moe::FMT_GPTQ>(epi, block_m, cap, ga, *W, ea, kernel, st);
  }
}

// Grouped GEMM with MXFP8 activations and MXFP4 weights, blocks of 64 or 128
// rows.  Returns hipErrorInvalidValue when the scale tiles do not fit.
extern "C" hipError_t moe_launch_gemm_mx(int epi, int block_m, int cap, const uint8_t* a_codes,
                                         const uint8_t* a_scales, int lda, int lds, int a_div,
                                         int n_slots, int K, int N, int E, const moe::WeightArgs* W,
                                         const int32_t* sid, const int32_t* eid, const int32_t* npp,
                                         const float* tw, int mul, float alpha, float beta,
                                         float limit, uint16_t* out, int out_ld, hipStream_t st) {
  if (cap / block_m == 0) return hipSuccess;
  // the weight scales by K chunk stream with the chunks; otherwise both scale
  // tiles stay resident and must fit
  const bool ss = W->scales_kc != nullptr;
  const int nchunks = (K + moe::kMxBK - 1) / moe::kMxBK;
  if (ss ? (lds % 4 != 0 || lds < 4 * nchunks)
         : (moe::mx_scale_bytes(K, block_m, lds) > moe::kMxScaleBytes ||
            block_m * (lds / 16) > 4 * moe::kMxScaleIssue * 64))
    return hipErrorInvalidValue;
  const uint64_t a_mul = ((1ull << 32) + (uint64_t)a_div - 1) / (uint64_t)a_div;
  // tile order: groups of 4 expert blocks (128-row), 8 (64-row: measured at the
  // gpt-oss-120b shape, T = 512 / 1024: MX GEMM1 -5%, the MXFP8 layer -4%)
  moe::GemmArgs ga{nullptr, a_div, a_mul, n_slots, K, N, E, cap / block_m, 0, block_m == 64 ? 8 : 4,
                   block_m, sid, eid, npp};
  ga.n_ntiles = (N + moe::Mx<128>::BN - 1) / moe::Mx<128>::BN;
  moe::MxA ma{a_codes, a_scales, lda, lds};
  moe::EpiArgs ea{sid, 0, n_slots, N, tw, mul, alpha, beta, limit, out, out_ld};
  const dim3 grid((ga.n_mblocks * ga.n_ntiles + 7) / 8 * 8);
  // resident scales: eight waves, one workgroup per CU (152 KB of LDS).
  // Streamed scales: four waves and a 2-deep ring, 67 KB, two workgroups per
  // CU (measured at the gpt-oss-120b shape, T = 8192: MX GEMM1 795 -> 655 us;
  // eight waves with 3 stages 799 us, four waves with 3 stages 838 us)
  constexpr int kMxRS = 2;
  constexpr int kSsRS = 1, kSsNS = 2;
#define MOE_MX_LAUNCH(EPI)                                                                       \
  do {                                                                                           \
    if (ss && block_m == 64)                                                                     \
      moe::gemm_mx_kernel<EPI, 64, kSsRS, kSsNS, true><<<grid, dim3(256 * kSsRS), 0, st>>>(ga, ma, *W, ea); \
    else if (ss)                                                                                 \
      moe::gemm_mx_kernel<EPI, 128, kSsRS, kSsNS, true, 2><<<grid, dim3(256 * kSsRS), 0, st>>>(ga, ma, *W, ea); \
    else if (block_m == 64)                                                                      \
      moe::gemm_mx_kernel<EPI, 64, kMxRS, moe::kMxStages, false><<<grid, dim3(256 * kMxRS), 0, st>>>(ga, ma, *W, ea); \
    else                                                                                         \
      moe::gemm_mx_kernel<EPI, 128, kMxRS, moe::kMxStages, false><<<grid, dim3(256 * kMxRS), 0, st>>>(ga, ma, *W, ea); \
  } while (0)
  switch (epi) {
    case moe::EPI_SWIGLU: MOE_MX_LAUNCH(moe::EPI_SWIGLU); break;
    case moe::EPI_RELU2: MOE_MX_LAUNCH(moe::EPI_RELU2); break;
    case moe::EPI_NONE: MOE_MX_LAUNCH(moe::EPI_NONE); break;
    default: MOE_MX_LAUNCH(moe::EPI_DOWN); break;
  }
#undef MOE_MX_LAUNCH
  return hipGetLastError();
}

extern "C" int moe_prefill_tiles_ok(int fmt, int K, int N, int group, int scales_kc) {
  return moe::prefill_fits(fmt, K, N, group, moe::prefill_streams(fmt, group, scales_kc != 0)) ? 1 : 0;
}

extern "C" hipError_t moe_launch_sum(const uint16_t* y, const int32_t* ids, int T, int top_k, int H,
                                     int E, uint16_t* out, hipStream_t st) {
  const size_t n = (size_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  moe::moe_sum_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(y, ids, T, top_k, H,
                                                                             E, out);
  return hipGetLastError();
}
