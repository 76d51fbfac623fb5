// C-ABI of the fused W4A16 MoE library: host-side validation and dispatch.
// Every entry point checks its arguments before enqueueing anything and
// returns a status; nothing here allocates, synchronises or reads device
// memory.
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "../../include/moe_w4a16.h"
#include "common.h"

extern "C" hipError_t moe_launch_route(const float*, int, int, int, int, const float*, int,
                                       int32_t*, float*, hipStream_t);
extern "C" hipError_t moe_launch_align(const int32_t*, int, int, int, int, int32_t*, int32_t*,
                                       int32_t*, hipStream_t);
extern "C" hipError_t moe_launch_align_large(const int32_t*, int, int, int, int, int32_t*, int32_t*,
                                             int32_t*, int32_t*, hipStream_t);
extern "C" hipError_t moe_launch_route_align(const float*, int, int, int, int, const float*, int,
                                             int32_t*, float*, int, int, int32_t*, int32_t*,
                                             int32_t*, hipStream_t);
extern "C" hipError_t moe_launch_gemm(int, int, int, int, const uint16_t*, int, int, int, int, int,
                                      const moe::WeightArgs*, const int32_t*, const int32_t*,
                                      const int32_t*, const float*, int, float, float, float,
                                      uint16_t*, int, int, const int2*, const int32_t*, hipStream_t);
extern "C" int moe_prefill_tiles_ok(int, int, int, int, int);
extern "C" hipError_t moe_launch_tile_plan(const int32_t*, const int32_t*, int, int, int32_t*, int2*,
                                           int32_t*, hipStream_t);
extern "C" hipError_t moe_launch_sum(const uint16_t*, const int32_t*, int, int, int, int,
                                     uint16_t*, hipStream_t);
extern "C" hipError_t moe_launch_gptq_sort(const int32_t*, const int32_t*, int, int, int, int,
                                           int32_t*, int32_t*, int32_t*, hipStream_t);
extern "C" hipError_t moe_launch_mxfp8_quant(const uint16_t*, int, int, int, int, uint8_t*, uint8_t*,
                                             uint16_t*, hipStream_t);
extern "C" hipError_t moe_launch_gemm_mx(int, int, int, const uint8_t*, const uint8_t*, int, int, int,
                                         int, int, int, int, const moe::WeightArgs*, const int32_t*,
                                         const int32_t*, const int32_t*, const float*, int, float,
                                         float, float, uint16_t*, int, hipStream_t);
extern "C" hipError_t moe_launch_nvfp4_scales_by_chunk(const uint8_t*, int, int, int, uint8_t*,
                                                       hipStream_t);
extern "C" hipError_t moe_launch_nvfp4_codes_by_chunk(const uint8_t*, int, int, int, uint8_t*,
                                                       hipStream_t);
extern "C" hipError_t moe_launch_mxfp4_codes_by_chunk(const uint8_t*, int, int, int, uint8_t*,
                                                      hipStream_t);
extern "C" hipError_t moe_launch_mxfp4_scales_by_chunk(const uint8_t*, int, int, int, uint8_t*,
                                                       hipStream_t);
extern "C" hipError_t moe_launch_permute_slots(const uint16_t*, int, int, int, int, const int32_t*,
                                               const int32_t*, uint16_t*, hipStream_t);

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxPermK = 8192;  // act-order: K of a permuted family (LDS staging)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_block_m(int b) { return b == 16 || b == 32 || b == 64 || b == 128; }

size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Validate one weight family for logical [N][K] and build the kernel view.
// allow_perm: the caller gathers the GEMM input through w->k_perm itself.
moe_status_t check_weights(const moe_wq_t* w, int N, int K, moe::WeightArgs* out,
                           bool allow_perm = false) {
  if (w == nullptr) return MOE_ERR_NULL;
  // chunked-only NVFP4/MXFP4 family: both copies by K chunk and no checkpoint layout
  const bool kc_only = (w->fmt == MOE_W_NVFP4 || w->fmt == MOE_W_MXFP4) && w->qweight == nullptr &&
                       w->scales == nullptr && w->qweight_kc != nullptr && w->scales_kc != nullptr;
  if (!kc_only && (w->qweight == nullptr || w->scales == nullptr)) return MOE_ERR_NULL;
  if (K <= 0 || N <= 0 || K % 32 != 0 || N % 16 != 0) return MOE_ERR_SHAPE;
  switch (w->fmt) {
    case MOE_W_NVFP4:
      if (w->group_size != 16) return MOE_ERR_UNSUPPORTED;
      if (w->global_scale == nullptr) return MOE_ERR_NULL;
      break;
    case MOE_W_MXFP4:
      if (w->group_size != 32) return MOE_ERR_UNSUPPORTED;
      break;
    case MOE_W_INT4_GPTQ:
      if (w->group_size != 32 && w->group_size != 64 && w->group_size != 128)
        return MOE_ERR_UNSUPPORTED;
      if (K % w->group_size != 0) return MOE_ERR_SHAPE;
      if (w->zeros == nullptr) return MOE_ERR_NULL;
      if (w->k_perm != nullptr) {
        if (!allow_perm) return MOE_ERR_UNSUPPORTED;
        // group-sorted weights: their rows are already in group order
        if (w->g_idx != nullptr) return MOE_ERR_UNSUPPORTED;
        if (K > kMaxPermK) return MOE_ERR_SHAPE;
        if (!aligned16(w->k_perm)) return MOE_ERR_ALIGN;
      }
      // a group map is checked on the device against the identity
      if (w->g_idx != nullptr && (reinterpret_cast<uintptr_t>(w->g_idx) & 3u)) return MOE_ERR_ALIGN;
      break;
    default:
      return MOE_ERR_UNSUPPORTED;
  }
  if (w->fmt != MOE_W_INT4_GPTQ && (w->k_perm != nullptr || w->g_idx != nullptr))
    return MOE_ERR_UNSUPPORTED;
  if (w->scales_kc != nullptr) {
    // NVFP4 [E][K/64][N][4]; MXFP4 [E][ceil(K/128)][N][4]
    if (w->fmt == MOE_W_INT4_GPTQ) return MOE_ERR_UNSUPPORTED;
    if (w->fmt == MOE_W_NVFP4 && K % 64 != 0) return MOE_ERR_SHAPE;
    if (!aligned16(w->scales_kc)) return MOE_ERR_ALIGN;
  }
  if (w->qweight_kc != nullptr) {
    // NVFP4: with scales_kc (format and K % 64 checked above); MXFP4: alone (the
    // MX kernels) or with scales_kc (also the streaming bf16 kernel)
    if (w->fmt == MOE_W_NVFP4 ? w->scales_kc == nullptr : w->fmt != MOE_W_MXFP4)
      return MOE_ERR_UNSUPPORTED;
    if (!aligned16(w->qweight_kc)) return MOE_ERR_ALIGN;
  }
  if (!aligned16(w->qweight) || !aligned16(w->scales)) return MOE_ERR_ALIGN;
  if (w->fmt == MOE_W_INT4_GPTQ && !aligned16(w->zeros)) return MOE_ERR_ALIGN;
  if (w->bias != nullptr && (reinterpret_cast<uintptr_t>(w->bias) & 1u)) return MOE_ERR_ALIGN;
  out->qweight = static_cast<const uint8_t*>(w->qweight);
  out->scales = static_cast<const uint8_t*>(w->scales);
  out->zeros = static_cast<const uint32_t*>(w->zeros);
  out->global_scale = w->global_scale;
  out->bias = w->bias;
  out->scales_kc = w->scales_kc;
  out->qweight_kc = w->qweight_kc;
  out->g_idx = w->g_idx;
  out->group = w->group_size;
  return MOE_OK;
}

bool valid_kernel(moe_kernel_t k) {
  return k == MOE_KERNEL_AUTO || k == MOE_KERNEL_SPLITK || k == MOE_KERNEL_WIDE;
}

int epi_of(moe_act_t act) {
  switch (act) {
    case MOE_ACT_SWIGLUOAI: return moe::EPI_SWIGLU;
    case MOE_ACT_RELU2: return moe::EPI_RELU2;
    case MOE_ACT_NONE: return moe::EPI_NONE;
    default: return -1;
  }
}

constexpr int kMixedMaxBlocks = 4096;  // the tile-plan kernel's block table in LDS

// The sort granularity moe_forward (and moe_forward_mxfp8) uses, by the
// average slots per expert.
// The streaming kernel's 64-row tiles beat the 16/32-row decode kernels from
// 9 slots per expert on (measured at the gpt-oss-20b shape: T = 128 160 ->
// 127 us, T = 256 193 -> 147 us; the gpt-oss-120b skewed layer at T = 1024,
// 32 per expert, 416 -> 381 us against the mixed tiling), and 128-row tiles
// beat 64-row ones from 57 on (T = 512, 64 per expert: 212 -> 197 us; at 56
// the 64-row tiles are 8% faster).  Up to 8 the decode kernels, which split K,
// keep the chip busy where the tiles would be too few.  (Also measured: 64-row
// blocks for uneven loads, pairs of them as 128-row tiles and the odd ones as
// a second, 64-row launch, ran slower than 128-row blocks throughout.)
int forward_block_m(int T, int top_k, int E) {
  const long avg = ((long)T * top_k + E - 1) / E;
  if (avg <= 8) return 16;
  if (avg <= 56) return 64;
  return 128;
}

struct WsLayout {
  size_t ids, w, sorted, eids, npp, cnt, dec, tiles, ntiles, act, y, total;
};

// Slots from which moe_forward sorts with the multi-workgroup kernels
// (measured: the single workgroup is as fast up to about this size).
constexpr int kAlignLargeMin = 8192;
// Mixed tiling (few slots per expert on average): from this many slots on,
// experts' full 128-row runs go to the streaming kernel (a tile list made on
// the device after the sort) and the rest to the 16/32-row decode kernels.
constexpr int kMixedMinSlots = 1024;

WsLayout ws_layout(int T, int E, int top_k, int hidden, int inter, int block_m) {
  WsLayout L;
  const size_t n = (size_t)T * top_k;
  const size_t cap = moe_align_capacity(T, top_k, E, block_m);
  size_t o = 0;
  L.ids = o; o = round_up(o + n * 4, 256);
  L.w = o; o = round_up(o + n * 4, 256);
  L.sorted = o; o = round_up(o + cap * 4, 256);
  L.eids = o; o = round_up(o + (cap / block_m) * 4, 256);
  L.npp = o; o = round_up(o + 4, 256);
  L.cnt = o; o = round_up(o + (size_t)moe::kAlignGroups * E * 4, 256);
  L.dec = o; o = round_up(o + (cap / block_m) * 4, 256);           // mixed tiling: decode blocks
  L.tiles = o; o = round_up(o + (cap / 128 + 1) * 8, 256);         // mixed tiling: 128-row tiles
  L.ntiles = o; o = round_up(o + 4, 256);
  L.act = o; o = round_up(o + n * (size_t)inter * 2, 256);
  L.y = o; o = round_up(o + n * (size_t)hidden * 2, 256);
  L.total = o;
  return L;
}

// MXFP8 operand layout: codes row stride K rounded up to 128, scales row
// stride K/32 rounded up to 16 (zero padded by the quantiser).
int mx_lda(int K) { return (K + 127) / 128 * 128; }
int mx_lds(int K) { return (K / 32 + 15) / 16 * 16; }

// Scale tiles of the MX GEMM kernel must fit its LDS (56 KB), and the A
// scale tile its 4 x 6 DMA instructions of 64 16-byte pieces.
// The MX kernel takes this family at this K: its weight scales by K chunk
// stream with the chunks (any K); otherwise both scale tiles must fit the
// kernel's 56 KB of resident LDS.
bool mx_fits(const moe::WeightArgs& W, int K, int block_m) {
  if (W.scales_kc != nullptr) return true;
  const int b = (256 * (K / 32) + 1023) / 1024 * 1024;
  return b + (block_m * mx_lds(K) + 1023) / 1024 * 1024 <= 56 * 1024 &&
         block_m * (mx_lds(K) / 16) <= 4 * 6 * 64;
}

struct MxWsLayout {
  WsLayout base;
  size_t xq, xs, aq, as, total;
};

MxWsLayout mx_ws_layout(int T, int E, int top_k, int hidden, int inter, int block_m) {
  MxWsLayout L;
  L.base = ws_layout(T, E, top_k, hidden, inter, block_m);
  const size_t n = (size_t)T * top_k;
  size_t o = L.base.total;
  L.xq = o; o = round_up(o + (size_t)T * mx_lda(hidden), 256);
  L.xs = o; o = round_up(o + (size_t)T * mx_lds(hidden), 256);
  L.aq = o; o = round_up(o + n * mx_lda(inter), 256);
  L.as = o; o = round_up(o + n * mx_lds(inter), 256);
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

size_t moe_align_capacity(int T, int top_k, int E, int block_m) {
  if (T <= 0 || top_k <= 0 || E <= 0 || block_m <= 0) return 0;
  const size_t n = (size_t)T * top_k;
  const size_t hit = n < (size_t)E ? n : (size_t)E;
  return round_up(n + hit * (size_t)(block_m - 1), (size_t)block_m);
}

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "required pointer is NULL";
    case MOE_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case MOE_ERR_UNSUPPORTED: return "unsupported format/activation/option";
    case MOE_ERR_ALIGN: return "pointer not sufficiently aligned";
    case MOE_ERR_HIP: return "HIP launch error";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_TOO_LARGE: return "problem needs more than the fixed scratch of moe_forward_noalloc";
  }
  return "unknown status";
}

moe_status_t moe_route(const float* logits, int T, int E, int top_k, moe_route_t kind,
                       const float* expert_bias, int renormalize, int32_t* topk_ids, float* topk_w,
                       moe_stream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || top_k < 1 || top_k > E || top_k > kMaxTopK)
    return MOE_ERR_SHAPE;
  if (kind != MOE_ROUTE_SOFTMAX && kind != MOE_ROUTE_SIGMOID_BIAS) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr) return MOE_ERR_NULL;
  if (kind == MOE_ROUTE_SIGMOID_BIAS && expert_bias == nullptr) return MOE_ERR_NULL;
  return hip_status(moe_launch_route(logits, T, E, top_k, (int)kind, expert_bias, renormalize ? 1 : 0,
                                     topk_ids, topk_w, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_align(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
                       int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post_pad,
                       moe_stream_t stream) {
  if (T < 0 || top_k < 1 || E <= 0 || E > kMaxE || !valid_block_m(block_m)) return MOE_ERR_SHAPE;
  if ((long long)T * top_k >= (1LL << 24)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (topk_ids == nullptr || sorted_ids == nullptr || expert_ids == nullptr ||
      num_post_pad == nullptr)
    return MOE_ERR_NULL;
  const int cap = (int)moe_align_capacity(T, top_k, E, block_m);
  return hip_status(moe_launch_align(topk_ids, T * top_k, E, block_m, cap, sorted_ids, expert_ids,
                                     num_post_pad, static_cast<hipStream_t>(stream)));
}

// Routing and the sort of moe_forward: fused in one workgroup for small
// batches, the multi-workgroup sort (counts in the workspace) for large ones.
hipError_t route_and_sort(const float* logits, int T, int E, int top_k, int kind,
                          const float* ebias, int renorm, int32_t* ids, float* tw, int block_m,
                          int cap, int32_t* sorted, int32_t* eids, int32_t* npp, int32_t* counts,
                          hipStream_t s) {
  const int n = T * top_k;
  if (n < kAlignLargeMin)
    return moe_launch_route_align(logits, T, E, top_k, kind, ebias, renorm, ids, tw, block_m, cap,
                                  sorted, eids, npp, s);
  hipError_t e = moe_launch_route(logits, T, E, top_k, kind, ebias, renorm, ids, tw, s);
  if (e == hipSuccess)
    e = moe_launch_align_large(ids, n, E, block_m, cap, counts, sorted, eids, npp, s);
  return e;
}

size_t moe_align_large_scratch_bytes(int E) {
  return E > 0 && E <= kMaxE ? (size_t)moe::kAlignGroups * E * 4 : 0;
}

moe_status_t moe_align_large(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
                             int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post_pad,
                             int32_t* counts, moe_stream_t stream) {
  if (T < 0 || top_k < 1 || E <= 0 || E > kMaxE || !valid_block_m(block_m)) return MOE_ERR_SHAPE;
  if ((long long)T * top_k >= (1LL << 24)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (topk_ids == nullptr || sorted_ids == nullptr || expert_ids == nullptr ||
      num_post_pad == nullptr || counts == nullptr)
    return MOE_ERR_NULL;
  const int cap = (int)moe_align_capacity(T, top_k, E, block_m);
  return hip_status(moe_launch_align_large(topk_ids, T * top_k, E, block_m, cap, counts, sorted_ids,
                                           expert_ids, num_post_pad,
                                           static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route_align(const float* logits, int T, int E, int top_k, moe_route_t kind,
                             const float* expert_bias, int renormalize, int block_m,
                             int32_t* topk_ids, float* topk_w, int32_t* sorted_ids,
                             int32_t* expert_ids, int32_t* num_post_pad, moe_stream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || top_k < 1 || top_k > E || top_k > kMaxTopK ||
      !valid_block_m(block_m))
    return MOE_ERR_SHAPE;
  if ((long long)T * top_k >= (1LL << 24)) return MOE_ERR_SHAPE;
  if (kind != MOE_ROUTE_SOFTMAX && kind != MOE_ROUTE_SIGMOID_BIAS) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr || sorted_ids == nullptr ||
      expert_ids == nullptr || num_post_pad == nullptr)
    return MOE_ERR_NULL;
  if (kind == MOE_ROUTE_SIGMOID_BIAS && expert_bias == nullptr) return MOE_ERR_NULL;
  const int cap = (int)moe_align_capacity(T, top_k, E, block_m);
  return hip_status(moe_launch_route_align(logits, T, E, top_k, (int)kind, expert_bias,
                                           renormalize ? 1 : 0, topk_ids, topk_w, block_m, cap,
                                           sorted_ids, expert_ids, num_post_pad,
                                           static_cast<hipStream_t>(stream)));
}

static moe_status_t gemm_common_checks(int size_m, int top_k, int E, int block_m) {
  if (size_m < 0 || top_k < 1 || E <= 0 || E > kMaxE || !valid_block_m(block_m))
    return MOE_ERR_SHAPE;
  if ((long long)size_m * top_k >= (1LL << 24)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status_t moe_w4a16_gemm1_ex(const uint16_t* x, int size_m, int top_k, int K, int N, int E,
                                const moe_wq_t* w13, moe_act_t act, float alpha, float beta,
                                float limit, const float* topk_w, int mul_topk_weights,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_post_pad, int block_m, uint16_t* out,
                                moe_kernel_t kernel, moe_stream_t stream) {
  moe_status_t st = gemm_common_checks(size_m, top_k, E, block_m);
  if (st != MOE_OK) return st;
  const int epi = epi_of(act);
  if (epi < 0 || !valid_kernel(kernel)) return MOE_ERR_UNSUPPORTED;
  moe::WeightArgs W;
  st = check_weights(w13, N, K, &W);
  if (st != MOE_OK) return st;
  if (epi == moe::EPI_SWIGLU && N % 32 != 0) return MOE_ERR_SHAPE;
  if (size_m == 0) return MOE_OK;
  if (x == nullptr || sorted_ids == nullptr || expert_ids == nullptr || num_post_pad == nullptr ||
      out == nullptr)
    return MOE_ERR_NULL;
  if (mul_topk_weights && topk_w == nullptr) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
  const int cap = (int)moe_align_capacity(size_m, top_k, E, block_m);
  const int out_ld = (epi == moe::EPI_SWIGLU) ? N / 2 : N;
  return hip_status(moe_launch_gemm((int)w13->fmt, epi, block_m, cap, x, top_k, size_m * top_k, K, N, E,
                                    &W, sorted_ids, expert_ids, num_post_pad, topk_w,
                                    mul_topk_weights ? 1 : 0, alpha, beta, limit, out, out_ld,
                                    (int)kernel, nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_w4a16_gemm1(const uint16_t* x, int size_m, int top_k, int K, int N, int E,
                             const moe_wq_t* w13, moe_act_t act, float alpha, float beta,
                             float limit, const float* topk_w, int mul_topk_weights,
                             const int32_t* sorted_ids, const int32_t* expert_ids,
                             const int32_t* num_post_pad, int block_m, uint16_t* out,
                             moe_stream_t stream) {
  return moe_w4a16_gemm1_ex(x, size_m, top_k, K, N, E, w13, act, alpha, beta, limit, topk_w,
                            mul_topk_weights, sorted_ids, expert_ids, num_post_pad, block_m, out,
                            MOE_KERNEL_AUTO, stream);
}

moe_status_t moe_w4a16_gemm2_ex(const uint16_t* a, int size_m, int top_k, int K, int N, int E,
                                const moe_wq_t* w2, const float* topk_w, int mul_topk_weights,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_post_pad, int block_m, uint16_t* y,
                                moe_kernel_t kernel, moe_stream_t stream) {
  moe_status_t st = gemm_common_checks(size_m, top_k, E, block_m);
  if (st != MOE_OK) return st;
  if (!valid_kernel(kernel)) return MOE_ERR_UNSUPPORTED;
  moe::WeightArgs W;
  st = check_weights(w2, N, K, &W);
  if (st != MOE_OK) return st;
  if (size_m == 0) return MOE_OK;
  if (a == nullptr || sorted_ids == nullptr || expert_ids == nullptr || num_post_pad == nullptr ||
      y == nullptr)
    return MOE_ERR_NULL;
  if (mul_topk_weights && topk_w == nullptr) return MOE_ERR_NULL;
  if (!aligned16(a) || !aligned16(y)) return MOE_ERR_ALIGN;
  const int cap = (int)moe_align_capacity(size_m, top_k, E, block_m);
  return hip_status(moe_launch_gemm((int)w2->fmt, moe::EPI_DOWN, block_m, cap, a, top_k, size_m * top_k,
                                    K, N, E, &W, sorted_ids, expert_ids, num_post_pad, topk_w,
                                    mul_topk_weights ? 1 : 0, 0.f, 0.f, 0.f, y, N, (int)kernel, nullptr, nullptr,
                                    static_cast<hipStream_t>(stream)));
}

moe_status_t moe_w4a16_gemm2(const uint16_t* a, int size_m, int top_k, int K, int N, int E,
                             const moe_wq_t* w2, const float* topk_w, int mul_topk_weights,
                             const int32_t* sorted_ids, const int32_t* expert_ids,
                             const int32_t* num_post_pad, int block_m, uint16_t* y,
                             moe_stream_t stream) {
  return moe_w4a16_gemm2_ex(a, size_m, top_k, K, N, E, w2, topk_w, mul_topk_weights, sorted_ids,
                            expert_ids, num_post_pad, block_m, y, MOE_KERNEL_AUTO, stream);
}

moe_status_t moe_gptq_act_order_sort(const int32_t* qweight, const int32_t* g_idx, int E, int K,
                                     int N, int group_size, int32_t* qweight_sorted,
                                     int32_t* k_perm, int32_t* status, moe_stream_t stream) {
  if (E <= 0 || E > kMaxE || K <= 0 || N <= 0 || K > kMaxPermK) return MOE_ERR_SHAPE;
  if (group_size != 32 && group_size != 64 && group_size != 128) return MOE_ERR_UNSUPPORTED;
  if (K % group_size != 0) return MOE_ERR_SHAPE;
  if (qweight == nullptr || g_idx == nullptr || qweight_sorted == nullptr || k_perm == nullptr ||
      status == nullptr)
    return MOE_ERR_NULL;
  if (qweight_sorted == qweight) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe_launch_gptq_sort(qweight, g_idx, E, K, N, group_size, qweight_sorted,
                                         k_perm, status, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_nvfp4_scales_by_chunk(const uint8_t* scales, int E, int N, int K, uint8_t* out,
                                       moe_stream_t stream) {
  if (E <= 0 || E > kMaxE || N <= 0 || K <= 0 || K % 64 != 0) return MOE_ERR_SHAPE;
  if (scales == nullptr || out == nullptr) return MOE_ERR_NULL;
  if (!aligned16(scales) || !aligned16(out)) return MOE_ERR_ALIGN;
  if (out == scales) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe_launch_nvfp4_scales_by_chunk(scales, E, N, K, out,
                                                     static_cast<hipStream_t>(stream)));
}

moe_status_t moe_nvfp4_codes_by_chunk(const uint8_t* qweight, int E, int N, int K, uint8_t* out,
                                      moe_stream_t stream) {
  if (E <= 0 || E > kMaxE || N <= 0 || K <= 0 || K % 64 != 0) return MOE_ERR_SHAPE;
  if (qweight == nullptr || out == nullptr) return MOE_ERR_NULL;
  if (!aligned16(qweight) || !aligned16(out)) return MOE_ERR_ALIGN;
  if (out == qweight) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe_launch_nvfp4_codes_by_chunk(qweight, E, N, K, out,
                                                    static_cast<hipStream_t>(stream)));
}

moe_status_t moe_mxfp4_scales_by_chunk(const uint8_t* scales, int E, int N, int K, uint8_t* out,
                                       moe_stream_t stream) {
  if (E <= 0 || E > kMaxE || N <= 0 || K <= 0 || K % 32 != 0) return MOE_ERR_SHAPE;
  if (scales == nullptr || out == nullptr) return MOE_ERR_NULL;
  if (!aligned16(out)) return MOE_ERR_ALIGN;
  if (out == scales) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe_launch_mxfp4_scales_by_chunk(scales, E, N, K, out,
                                                     static_cast<hipStream_t>(stream)));
}

moe_status_t moe_mxfp4_codes_by_chunk(const uint8_t* qweight, int E, int N, int K, uint8_t* out,
                                      moe_stream_t stream) {
  if (E <= 0 || E > kMaxE || N <= 0 || K <= 0 || K % 32 != 0) return MOE_ERR_SHAPE;
  if (qweight == nullptr || out == nullptr) return MOE_ERR_NULL;
  if (!aligned16(qweight) || !aligned16(out)) return MOE_ERR_ALIGN;
  if (out == qweight) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe_launch_mxfp4_codes_by_chunk(qweight, E, N, K, out,
                                                    static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute_slots(const uint16_t* src, int size_m, int top_k, int K, int E,
                               const int32_t* k_perm, const int32_t* topk_ids, uint16_t* dst,
                               moe_stream_t stream) {
  if (size_m < 0 || top_k < 1 || E <= 0 || E > kMaxE || K <= 0 || K % 8 != 0 || K > kMaxPermK)
    return MOE_ERR_SHAPE;
  if ((long long)size_m * top_k >= (1LL << 24)) return MOE_ERR_SHAPE;
  if (size_m == 0) return MOE_OK;
  if (src == nullptr || k_perm == nullptr || topk_ids == nullptr || dst == nullptr)
    return MOE_ERR_NULL;
  if (dst == src && top_k != 1) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst) || !aligned16(k_perm)) return MOE_ERR_ALIGN;
  return hip_status(moe_launch_permute_slots(src, size_m * top_k, top_k, K, E, k_perm, topk_ids,
                                             dst, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_mxfp8_quantize(const uint16_t* x, int rows, int K, uint8_t* codes, uint8_t* scales,
                                uint16_t* dequant, moe_stream_t stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (x == nullptr || (codes == nullptr && scales == nullptr && dequant == nullptr))
    return MOE_ERR_NULL;
  if (!aligned16(x) || (codes && !aligned16(codes)) || (dequant && !aligned16(dequant)))
    return MOE_ERR_ALIGN;
  return hip_status(moe_launch_mxfp8_quant(x, rows, K, mx_lda(K), mx_lds(K), codes, scales,
                                           dequant, static_cast<hipStream_t>(stream)));
}

static moe_status_t mx_gemm_checks(const moe_wq_t* w, int N, int K, int block_m,
                                   moe::WeightArgs* W) {
  moe_status_t st = check_weights(w, N, K, W);
  if (st != MOE_OK) return st;
  if (w->fmt != MOE_W_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (block_m != 64 && block_m != 128) return MOE_ERR_UNSUPPORTED;
  if (!mx_fits(*W, K, block_m)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t moe_mx_gemm1(const uint8_t* x_codes, const uint8_t* x_scales, int size_m, int top_k,
                          int K, int N, int E, const moe_wq_t* w13, moe_act_t act, float alpha,
                          float beta, float limit, const int32_t* sorted_ids,
                          const int32_t* expert_ids, const int32_t* num_post_pad, int block_m,
                          uint16_t* out, moe_stream_t stream) {
  moe_status_t st = gemm_common_checks(size_m, top_k, E, block_m);
  if (st != MOE_OK) return st;
  const int epi = epi_of(act);
  if (epi < 0) return MOE_ERR_UNSUPPORTED;
  moe::WeightArgs W;
  st = mx_gemm_checks(w13, N, K, block_m, &W);
  if (st != MOE_OK) return st;
  if (epi == moe::EPI_SWIGLU && N % 32 != 0) return MOE_ERR_SHAPE;
  if (size_m == 0) return MOE_OK;
  if (x_codes == nullptr || x_scales == nullptr || sorted_ids == nullptr || expert_ids == nullptr ||
      num_post_pad == nullptr || out == nullptr)
    return MOE_ERR_NULL;
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(out)) return MOE_ERR_ALIGN;
  const int cap = (int)moe_align_capacity(size_m, top_k, E, block_m);
  const int out_ld = (epi == moe::EPI_SWIGLU) ? N / 2 : N;
  return hip_status(moe_launch_gemm_mx(epi, block_m, cap, x_codes, x_scales, mx_lda(K), mx_lds(K),
                                       top_k, size_m * top_k, K, N, E, &W, sorted_ids, expert_ids,
                                       num_post_pad, nullptr, 0, alpha, beta, limit, out, out_ld,
                                       static_cast<hipStream_t>(stream)));
}

moe_status_t moe_mx_gemm2(const uint8_t* a_codes, const uint8_t* a_scales, int size_m, int K, int N,
                          int E, const moe_wq_t* w2, const float* topk_w, int mul_topk_weights,
                          const int32_t* sorted_ids, const int32_t* expert_ids,
                          const int32_t* num_post_pad, int block_m, uint16_t* y,
                          moe_stream_t stream) {
  moe_status_t st = gemm_common_checks(size_m, 1, E, block_m);
  if (st != MOE_OK) return st;
  moe::WeightArgs W;
  st = mx_gemm_checks(w2, N, K, block_m, &W);
  if (st != MOE_OK) return st;
  if (size_m == 0) return MOE_OK;
  if (a_codes == nullptr || a_scales == nullptr || sorted_ids == nullptr || expert_ids == nullptr ||
      num_post_pad == nullptr || y == nullptr)
    return MOE_ERR_NULL;
  if (mul_topk_weights && topk_w == nullptr) return MOE_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(y)) return MOE_ERR_ALIGN;
  const int cap = (int)moe_align_capacity(size_m, 1, E, block_m);
  return hip_status(moe_launch_gemm_mx(moe::EPI_DOWN, block_m, cap, a_codes, a_scales, mx_lda(K),
                                       mx_lds(K), 1, size_m, K, N, E, &W, sorted_ids, expert_ids,
                                       num_post_pad, topk_w, mul_topk_weights ? 1 : 0, 0.f, 0.f,
                                       0.f, y, N, static_cast<hipStream_t>(stream)));
}

size_t moe_forward_mxfp8_workspace_bytes(int T, int E, int top_k, int hidden, int inter) {
  if (T <= 0 || E <= 0 || top_k <= 0 || hidden <= 0 || inter <= 0) return 0;
  return mx_ws_layout(T, E, top_k, hidden, inter, forward_block_m(T, top_k, E)).total;
}

moe_status_t moe_forward_mxfp8(const uint16_t* x, const float* logits, int T, int E, int top_k,
                               int hidden, int inter, moe_route_t kind, const float* expert_bias,
                               int renormalize, const moe_wq_t* w13, const moe_wq_t* w2,
                               moe_act_t act, float alpha, float beta, float limit,
                               int mul_topk_weights, void* workspace, size_t workspace_bytes,
                               uint16_t* out, moe_stream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || top_k < 1 || top_k > E || top_k > kMaxTopK)
    return MOE_ERR_SHAPE;
  if ((long long)T * top_k >= (1LL << 24)) return MOE_ERR_SHAPE;
  if (kind != MOE_ROUTE_SOFTMAX && kind != MOE_ROUTE_SIGMOID_BIAS) return MOE_ERR_UNSUPPORTED;
  const int epi = epi_of(act);
  if (epi != moe::EPI_SWIGLU && epi != moe::EPI_RELU2) return MOE_ERR_UNSUPPORTED;
  const int n1 = (epi == moe::EPI_SWIGLU) ? 2 * inter : inter;
  moe::WeightArgs W13, W2;
  moe_status_t st = check_weights(w13, n1, hidden, &W13);
  if (st != MOE_OK) return st;
  st = check_weights(w2, hidden, inter, &W2);
  if (st != MOE_OK) return st;
  if (w13->fmt != MOE_W_MXFP4 || w2->fmt != MOE_W_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (epi == moe::EPI_SWIGLU && n1 % 32 != 0) return MOE_ERR_SHAPE;
  if (mul_topk_weights < 0 || mul_topk_weights > 1) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (x == nullptr || logits == nullptr || out == nullptr || workspace == nullptr) return MOE_ERR_NULL;
  if (kind == MOE_ROUTE_SIGMOID_BIAS && expert_bias == nullptr) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return MOE_ERR_ALIGN;
  const int block_m = forward_block_m(T, top_k, E);
  const MxWsLayout L = mx_ws_layout(T, E, top_k, hidden, inter, block_m);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.base.ids);
  float* tw = reinterpret_cast<float*>(ws + L.base.w);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.base.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(ws + L.base.eids);
  int32_t* npp = reinterpret_cast<int32_t*>(ws + L.base.npp);
  uint16_t* actb = reinterpret_cast<uint16_t*>(ws + L.base.act);
  uint16_t* yb = reinterpret_cast<uint16_t*>(ws + L.base.y);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + L.xs);
  uint8_t* aq = reinterpret_cast<uint8_t*>(ws + L.aq);
  uint8_t* as = reinterpret_cast<uint8_t*>(ws + L.as);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = T * top_k;
  const int cap = (int)moe_align_capacity(T, top_k, E, block_m);
  const int mul = mul_topk_weights;

  hipError_t e = route_and_sort(logits, T, E, top_k, (int)kind, expert_bias, renormalize ? 1 : 0,
                                ids, tw, block_m, cap, sorted, eids, npp, reinterpret_cast<int32_t*>(ws + L.base.cnt), s);
  if (block_m >= 64 && mx_fits(W13, hidden, block_m) && mx_fits(W2, inter, block_m)) {
    // MX-scaled MFMA: both GEMMs read e4m3 codes and e8m0 scales
    if (e == hipSuccess)
      e = moe_launch_mxfp8_quant(x, T, hidden, mx_lda(hidden), mx_lds(hidden), xq, xs, nullptr, s);
    if (e == hipSuccess)
      e = moe_launch_gemm_mx(epi, block_m, cap, xq, xs, mx_lda(hidden), mx_lds(hidden), top_k, n,
                             hidden, n1, E, &W13, sorted, eids, npp, tw, 0, alpha, beta, limit,
                             actb, inter, s);
    if (e == hipSuccess)
      e = moe_launch_mxfp8_quant(actb, n, inter, mx_lda(inter), mx_lds(inter), aq, as, nullptr, s);
    if (e == hipSuccess)
      e = moe_launch_gemm_mx(moe::EPI_DOWN, block_m, cap, aq, as, mx_lda(inter), mx_lds(inter), 1,
                             n, inter, hidden, E, &W2, sorted, eids, npp, tw, mul, 0.f, 0.f, 0.f,
                             yb, hidden, s);
  } else {
    // few rows per expert: the operands are taken at their MXFP8 values
    // (quantised and dequantised to bf16, exactly) by the bf16 kernels
    if (e == hipSuccess)
      e = moe_launch_mxfp8_quant(x, T, hidden, mx_lda(hidden), mx_lds(hidden), nullptr, nullptr,
                                 yb, s);
    if (e == hipSuccess)
      e = moe_launch_gemm((int)w13->fmt, epi, block_m, cap, yb, top_k, n, hidden, n1, E, &W13,
                          sorted, eids, npp, tw, 0, alpha, beta, limit, actb, inter,
                          moe::KERNEL_AUTO, nullptr, nullptr, s);
    if (e == hipSuccess)
      e = moe_launch_mxfp8_quant(actb, n, inter, mx_lda(inter), mx_lds(inter), nullptr, nullptr,
                                 actb, s);
    if (e == hipSuccess)
      e = moe_launch_gemm((int)w2->fmt, moe::EPI_DOWN, block_m, cap, actb, 1, n, inter, hidden, E,
                          &W2, sorted, eids, npp, tw, mul, 0.f, 0.f, 0.f, yb, hidden,
                          moe::KERNEL_AUTO, nullptr, nullptr, s);
  }
  if (e == hipSuccess) e = moe_launch_sum(yb, ids, T, top_k, hidden, E, out, s);
  return hip_status(e);
}

int moe_forward_block_m(int T, int top_k, int E) {
  if (T <= 0 || top_k <= 0 || E <= 0) return 16;
  return forward_block_m(T, top_k, E);
}

size_t moe_forward_workspace_bytes(int T, int E, int top_k, int hidden, int inter) {
  if (T <= 0 || E <= 0 || top_k <= 0 || hidden <= 0 || inter <= 0) return 0;
  return ws_layout(T, E, top_k, hidden, inter, forward_block_m(T, top_k, E)).total;
}

}  // extern "C"

// The layer on a given workspace (moe_forward_ex, moe_forward_noalloc).
static moe_status_t forward_run(const uint16_t* x, const float* logits, int T, int E, int top_k,
                                int hidden, int inter, moe_route_t kind, const float* expert_bias,
                                int renormalize, const moe_wq_t* w13, const moe_wq_t* w2,
                                moe_act_t act, float alpha, float beta, float limit,
                                int mul_topk_weights, void* workspace, size_t workspace_bytes,
                                uint16_t* out, moe_kernel_t kernel, moe_stream_t stream) {
  if (T < 0 || E <= 0 || E > kMaxE || top_k < 1 || top_k > E || top_k > kMaxTopK)
    return MOE_ERR_SHAPE;
  if ((long long)T * top_k >= (1LL << 24)) return MOE_ERR_SHAPE;
  if (kind != MOE_ROUTE_SOFTMAX && kind != MOE_ROUTE_SIGMOID_BIAS) return MOE_ERR_UNSUPPORTED;
  if (!valid_kernel(kernel)) return MOE_ERR_UNSUPPORTED;
  const int epi = epi_of(act);
  if (epi != moe::EPI_SWIGLU && epi != moe::EPI_RELU2) return MOE_ERR_UNSUPPORTED;
  const int n1 = (epi == moe::EPI_SWIGLU) ? 2 * inter : inter;
  moe::WeightArgs W13, W2;
  moe_status_t st = check_weights(w13, n1, hidden, &W13, true);
  if (st != MOE_OK) return st;
  st = check_weights(w2, hidden, inter, &W2, true);
  if (st != MOE_OK) return st;
  if (epi == moe::EPI_SWIGLU && n1 % 32 != 0) return MOE_ERR_SHAPE;
  if (mul_topk_weights < 0 || mul_topk_weights > 2) return MOE_ERR_UNSUPPORTED;
  if (mul_topk_weights == 2 && top_k != 1) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || logits == nullptr || out == nullptr || workspace == nullptr) return MOE_ERR_NULL;
  if (kind == MOE_ROUTE_SIGMOID_BIAS && expert_bias == nullptr) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return MOE_ERR_ALIGN;
  const int block_m = forward_block_m(T, top_k, E);
  const WsLayout L = ws_layout(T, E, top_k, hidden, inter, block_m);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* tw = reinterpret_cast<float*>(ws + L.w);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(ws + L.eids);
  int32_t* npp = reinterpret_cast<int32_t*>(ws + L.npp);
  uint16_t* actb = reinterpret_cast<uint16_t*>(ws + L.act);
  uint16_t* yb = reinterpret_cast<uint16_t*>(ws + L.y);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = T * top_k;
  const int cap = (int)moe_align_capacity(T, top_k, E, block_m);

  hipError_t e = route_and_sort(logits, T, E, top_k, (int)kind, expert_bias, renormalize ? 1 : 0,
                                ids, tw, block_m, cap, sorted, eids, npp, reinterpret_cast<int32_t*>(ws + L.cnt), s);
  // Mixed tiling: the 128-row tiles (prefill kernel, tile list) and the rest
  // of the blocks (decode kernels, dec_eids: -1 for blocks in a tile).
  const bool mixed = block_m <= 32 && n >= kMixedMinSlots && cap / block_m <= kMixedMaxBlocks &&
                     moe_prefill_tiles_ok((int)w13->fmt, hidden, n1, w13->group_size, w13->scales_kc != nullptr) &&
                     moe_prefill_tiles_ok((int)w2->fmt, inter, hidden, w2->group_size, w2->scales_kc != nullptr);
  int32_t* dec_eids = reinterpret_cast<int32_t*>(ws + L.dec);
  int2* tiles = reinterpret_cast<int2*>(ws + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  const int tile_cap = cap / 128 * 128;
  if (e == hipSuccess && mixed)
    e = moe_launch_tile_plan(eids, npp, block_m, cap / block_m, dec_eids, tiles, ntiles, s);
  const int32_t* blk_eids = mixed ? dec_eids : eids;
  // Act-order families: GEMM1 reads one gathered input row per slot from the
  // y buffer (free until GEMM2), in the top_k = 1 view; GEMM2's input rows are
  // permuted in place.
  const uint16_t* g1_in = x;
  int g1_topk = top_k;
  if (e == hipSuccess && w13->k_perm != nullptr) {
    e = moe_launch_permute_slots(x, n, top_k, hidden, E, w13->k_perm, ids, yb, s);
    g1_in = yb;
    g1_topk = 1;
  }
  // routing weight on GEMM2's output rows (mode 1) or GEMM1's input rows (mode 2)
  if (e == hipSuccess && mixed && tile_cap > 0)
    e = moe_launch_gemm((int)w13->fmt, epi, 128, tile_cap, g1_in, g1_topk, n, hidden, n1, E, &W13,
                        sorted, eids, npp, tw, mul_topk_weights == 2 ? 1 : 0, alpha, beta, limit,
                        actb, inter, (int)kernel, tiles, ntiles, s);
  if (e == hipSuccess)
    e = moe_launch_gemm((int)w13->fmt, epi, block_m, cap, g1_in, g1_topk, n, hidden, n1, E, &W13,
                        sorted, blk_eids, npp, tw, mul_topk_weights == 2 ? 1 : 0, alpha, beta, limit,
                        actb, inter, (int)kernel, nullptr, nullptr, s);
  if (e == hipSuccess && w2->k_perm != nullptr)
    e = moe_launch_permute_slots(actb, n, 1, inter, E, w2->k_perm, ids, actb, s);
  if (e == hipSuccess && mixed && tile_cap > 0)
    e = moe_launch_gemm((int)w2->fmt, moe::EPI_DOWN, 128, tile_cap, actb, 1, n, inter, hidden, E,
                        &W2, sorted, eids, npp, tw, mul_topk_weights == 1 ? 1 : 0, 0.f, 0.f, 0.f,
                        yb, hidden, (int)kernel, tiles, ntiles, s);
  if (e == hipSuccess)
    e = moe_launch_gemm((int)w2->fmt, moe::EPI_DOWN, block_m, cap, actb, 1, n, inter, hidden, E, &W2,
                        sorted, blk_eids, npp, tw, mul_topk_weights == 1 ? 1 : 0, 0.f, 0.f, 0.f, yb,
                        hidden, (int)kernel, nullptr, nullptr, s);
  if (e == hipSuccess) e = moe_launch_sum(yb, ids, T, top_k, hidden, E, out, s);
  return hip_status(e);
}

// Fixed scratch of moe_forward_noalloc: the same workspace moe_forward takes,
// in one array per GPU (each GPU holds its own copy, from the library's load
// until the process ends).  On the host `scratch` only stands in for the
// device array; its device address comes from hipGetSymbolAddress, looked up
// once per device, with that device current, and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[MOE_FORWARD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's scratch (set up on the first call on
// that device; later calls read the kept address).
moe_status_t scratch_of_current_device(uint8_t** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  uint8_t* a = g_scratch[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return MOE_ERR_HIP;
    a = static_cast<uint8_t*>(q);
    g_scratch[dev].store(a, std::memory_order_release);  // the same address on every lookup
  }
  *p = a;
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status_t moe_forward_ex(const uint16_t* x, const float* logits, int T, int E, int top_k,
                            int hidden, int inter, moe_route_t kind, const float* expert_bias,
                            int renormalize, const moe_wq_t* w13, const moe_wq_t* w2, moe_act_t act,
                            float alpha, float beta, float limit, int mul_topk_weights,
                            void* workspace, size_t workspace_bytes, uint16_t* out,
                            moe_kernel_t kernel, moe_stream_t stream) {
  return forward_run(x, logits, T, E, top_k, hidden, inter, kind, expert_bias, renormalize, w13, w2,
                     act, alpha, beta, limit, mul_topk_weights, workspace, workspace_bytes, out,
                     kernel, stream);
}

moe_status_t moe_forward_noalloc(const uint16_t* x, const float* logits, int T, int E, int top_k,
                                 int hidden, int inter, moe_route_t kind, const float* expert_bias,
                                 int renormalize, const moe_wq_t* w13, const moe_wq_t* w2,
                                 moe_act_t act, float alpha, float beta, float limit,
                                 int mul_topk_weights, uint16_t* out, moe_stream_t stream) {
  uint8_t* ws = nullptr;
  const moe_status_t st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  const moe_status_t r = forward_run(x, logits, T, E, top_k, hidden, inter, kind, expert_bias,
                                     renormalize, w13, w2, act, alpha, beta, limit,
                                     mul_topk_weights, ws, MOE_FORWARD_NOALLOC_SCRATCH_BYTES, out,
                                     MOE_KERNEL_AUTO, stream);
  return r == MOE_ERR_WORKSPACE ? MOE_ERR_TOO_LARGE : r;
}

moe_status_t moe_forward(const uint16_t* x, const float* logits, int T, int E, int top_k,
                         int hidden, int inter, moe_route_t kind, const float* expert_bias,
                         int renormalize, const moe_wq_t* w13, const moe_wq_t* w2, moe_act_t act,
                         float alpha, float beta, float limit, int mul_topk_weights,
                         void* workspace, size_t workspace_bytes, uint16_t* out,
                         moe_stream_t stream) {
  return moe_forward_ex(x, logits, T, E, top_k, hidden, inter, kind, expert_bias, renormalize, w13,
                        w2, act, alpha, beta, limit, mul_topk_weights, workspace, workspace_bytes,
                        out, MOE_KERNEL_AUTO, stream);
}

}  // extern "C"
