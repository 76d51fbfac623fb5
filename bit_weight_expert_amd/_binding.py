"""ctypes marshalling for libmoe_w4a16.so.  Argument checking beyond what the
library does itself is limited to dtype/device/contiguity of tensors."""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe_w4a16.so"

FMT = {"nvfp4": 0, "mxfp4": 1, "gptq": 2}
ACT = {"swigluoai": 0, "relu2": 1, "none": 2}
ROUTE = {"softmax": 0, "sigmoid_bias": 1}
KERNEL = {"auto": 0, "splitk": 1, "wide": 2}   # kernel for blocks of 16/32 rows


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({_status_str(status)})")


class _Wq(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int),
        ("group_size", ctypes.c_int),
        ("qweight", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p),
        ("global_scale", ctypes.c_void_p),
        ("g_idx", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("k_perm", ctypes.c_void_p),
        ("scales_kc", ctypes.c_void_p),
        ("qweight_kc", ctypes.c_void_p),
    ]


_lib = None


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """Load the HIP library (built in-tree by bit_weight_expert_amd.build)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run python -m bit_weight_expert_amd.build")
        L = ctypes.CDLL(path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        wq = ctypes.POINTER(_Wq)
        L.moe_align_capacity.argtypes = [i, i, i, i]
        L.moe_align_capacity.restype = sz
        L.moe_forward_workspace_bytes.argtypes = [i, i, i, i, i]
        L.moe_forward_workspace_bytes.restype = sz
        L.moe_forward_block_m.argtypes = [i, i, i]
        L.moe_forward_block_m.restype = i
        L.moe_status_str.argtypes = [i]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_route.argtypes = [vp, i, i, i, i, vp, i, vp, vp, vp]
        L.moe_route.restype = i
        L.moe_align.argtypes = [vp, i, i, i, i, vp, vp, vp, vp]
        L.moe_align.restype = i
        L.moe_route_align.argtypes = [vp, i, i, i, i, vp, i, i, vp, vp, vp, vp, vp, vp]
        L.moe_route_align.restype = i
        L.moe_w4a16_gemm1.argtypes = [vp, i, i, i, i, i, wq, i, f, f, f, vp, i, vp, vp, vp, i, vp, vp]
        L.moe_w4a16_gemm1.restype = i
        L.moe_w4a16_gemm1_ex.argtypes = L.moe_w4a16_gemm1.argtypes[:-1] + [i, vp]
        L.moe_w4a16_gemm1_ex.restype = i
        L.moe_w4a16_gemm2.argtypes = [vp, i, i, i, i, i, wq, vp, i, vp, vp, vp, i, vp, vp]
        L.moe_w4a16_gemm2.restype = i
        L.moe_w4a16_gemm2_ex.argtypes = L.moe_w4a16_gemm2.argtypes[:-1] + [i, vp]
        L.moe_w4a16_gemm2_ex.restype = i
        L.moe_forward.argtypes = [vp, vp, i, i, i, i, i, i, vp, i, wq, wq, i, f, f, f, i, vp, sz,
                                  vp, vp]
        L.moe_forward.restype = i
        L.moe_forward_ex.argtypes = L.moe_forward.argtypes[:-1] + [i, vp]
        L.moe_forward_ex.restype = i
        L.moe_forward_noalloc.argtypes = [vp, vp, i, i, i, i, i, i, vp, i, wq, wq, i, f, f, f, i,
                                          vp, vp]
        L.moe_forward_noalloc.restype = i
        L.moe_gptq_act_order_sort.argtypes = [vp, vp, i, i, i, i, vp, vp, vp, vp]
        L.moe_gptq_act_order_sort.restype = i
        L.moe_permute_slots.argtypes = [vp, i, i, i, i, vp, vp, vp, vp]
        L.moe_permute_slots.restype = i
        L.moe_nvfp4_scales_by_chunk.argtypes = [vp, i, i, i, vp, vp]
        L.moe_nvfp4_scales_by_chunk.restype = i
        L.moe_nvfp4_codes_by_chunk.argtypes = [vp, i, i, i, vp, vp]
        L.moe_nvfp4_codes_by_chunk.restype = i
        L.moe_mxfp4_codes_by_chunk.argtypes = [vp, i, i, i, vp, vp]
        L.moe_mxfp4_codes_by_chunk.restype = i
        L.moe_mxfp4_scales_by_chunk.argtypes = [vp, i, i, i, vp, vp]
        L.moe_mxfp4_scales_by_chunk.restype = i
        L.moe_align_large.argtypes = [vp, i, i, i, i, vp, vp, vp, vp, vp]
        L.moe_align_large.restype = i
        L.moe_align_large_scratch_bytes.argtypes = [i]
        L.moe_align_large_scratch_bytes.restype = ctypes.c_size_t
        L.moe_mxfp8_quantize.argtypes = [vp, i, i, vp, vp, vp, vp]
        L.moe_mxfp8_quantize.restype = i
        L.moe_mx_gemm1.argtypes = [vp, vp, i, i, i, i, i, wq, i, f, f, f, vp, vp, vp, i, vp, vp]
        L.moe_mx_gemm1.restype = i
        L.moe_mx_gemm2.argtypes = [vp, vp, i, i, i, i, wq, vp, i, vp, vp, vp, i, vp, vp]
        L.moe_mx_gemm2.restype = i
        L.moe_forward_mxfp8_workspace_bytes.argtypes = [i, i, i, i, i]
        L.moe_forward_mxfp8_workspace_bytes.restype = sz
        L.moe_forward_mxfp8.argtypes = [vp, vp, i, i, i, i, i, i, vp, i, wq, wq, i, f, f, f, i, vp,
                                        sz, vp, vp]
        L.moe_forward_mxfp8.restype = i
        _lib = L
    return _lib


def _status_str(s: int) -> str:
    try:
        return lib().moe_status_str(s).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoeError(status, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous {dtype} CUDA tensor, got {t.dtype} "
                        f"on {t.device} (contiguous={t.is_contiguous()})")
    return t


@dataclasses.dataclass
class QuantWeights:
    """Device-resident 4-bit weights of all experts; logical W_e is [N][K]."""
    fmt: str
    group: int
    N: int
    K: int
    qweight: torch.Tensor | None          # None in a chunked-only family (see chunked_only)
    scales: torch.Tensor | None
    zeros: torch.Tensor | None = None
    global_scale: torch.Tensor | None = None
    bias: torch.Tensor | None = None
    k_perm: torch.Tensor | None = None     # GPTQ act-order, from moe_gptq_act_order_sort
    scales_kc: torch.Tensor | None = None  # NVFP4 scales by K chunk, from moe_nvfp4_scales_by_chunk
    qweight_kc: torch.Tensor | None = None  # codes by K chunk: moe_nvfp4_codes_by_chunk (with scales_kc)
    #                                          or moe_mxfp4_codes_by_chunk (MX kernels)
    g_idx: torch.Tensor | None = None      # GPTQ group map int32 [E, K] (identity only, checked on device)

    @classmethod
    def from_arrays(cls, fmt, group, N, K, qweight, scales, zeros=None, global_scale=None,
                    bias=None, device="cuda"):
        """Upload host arrays (numpy) holding the storage bytes."""
        def up(a, dt):
            if a is None:
                return None
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
        sdt = np.float16 if fmt == "gptq" else np.uint8
        return cls(fmt=fmt, group=group, N=N, K=K,
                   qweight=up(qweight, np.int32 if fmt == "gptq" else np.uint8),
                   scales=up(scales, sdt), zeros=up(zeros, np.int32),
                   global_scale=up(global_scale, np.float32), bias=up(bias, np.int16))

    def struct(self) -> _Wq:
        return _Wq(FMT[self.fmt], self.group, _ptr(self.qweight), _ptr(self.scales),
                   _ptr(self.zeros), _ptr(self.global_scale), _ptr(self.g_idx), _ptr(self.bias),
                   _ptr(self.k_perm), _ptr(self.scales_kc), _ptr(self.qweight_kc))

    @property
    def E(self) -> int:
        return (self.qweight if self.qweight is not None else self.qweight_kc).shape[0]

    def chunked_only(self) -> "QuantWeights":
        """NVFP4/MXFP4: the same family holding only the copies by K chunk
        (codes and scales; made here if absent), which every kernel reads
        instead of the checkpoint layout: one copy of the codes on the device."""
        import dataclasses
        if self.fmt not in ("nvfp4", "mxfp4"):
            raise ValueError("only NVFP4 and MXFP4 have a layout by K chunk")
        kc = self
        if self.fmt == "nvfp4":
            if kc.scales_kc is None:
                kc = dataclasses.replace(kc, scales_kc=moe_nvfp4_scales_by_chunk(kc))
            if kc.qweight_kc is None:
                kc = dataclasses.replace(kc, qweight_kc=moe_nvfp4_codes_by_chunk(kc))
        else:
            if kc.scales_kc is None:
                kc = dataclasses.replace(kc, scales_kc=moe_mxfp4_scales_by_chunk(kc))
            if kc.qweight_kc is None:
                kc = dataclasses.replace(kc, qweight_kc=moe_mxfp4_codes_by_chunk(kc))
        return dataclasses.replace(kc, qweight=None, scales=None)


def moe_align_capacity(T: int, top_k: int, E: int, block_m: int) -> int:
    return lib().moe_align_capacity(T, top_k, E, block_m)


def moe_forward_block_m(T: int, top_k: int, E: int) -> int:
    return lib().moe_forward_block_m(T, top_k, E)


def moe_forward_workspace_bytes(T: int, E: int, top_k: int, hidden: int, inter: int) -> int:
    return lib().moe_forward_workspace_bytes(T, E, top_k, hidden, inter)


def moe_route(logits: torch.Tensor, top_k: int, kind: str = "softmax", expert_bias=None,
              renormalize: bool = True, topk_ids=None, topk_w=None):
    """-> (topk_ids int32 [T,k], topk_w float32 [T,k])."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    if expert_bias is not None:
        _dev(expert_bias, torch.float32, "expert_bias")
    _check(lib().moe_route(_ptr(logits), T, E, top_k, ROUTE[kind], _ptr(expert_bias),
                           int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_w), _stream()),
           "moe_route")
    return topk_ids, topk_w


def moe_align(topk_ids: torch.Tensor, E: int, block_m: int, sorted_ids=None, expert_ids=None,
              num_post_pad=None):
    """-> (sorted_ids int32 [cap], expert_ids int32 [cap/block_m], num_post_pad int32 [1])."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    cap = moe_align_capacity(T, k, E, block_m)
    dev = topk_ids.device
    if sorted_ids is None:
        sorted_ids = torch.empty((cap,), dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty((cap // block_m if block_m else 0,), dtype=torch.int32, device=dev)
    if num_post_pad is None:
        num_post_pad = torch.zeros((1,), dtype=torch.int32, device=dev)
    _check(lib().moe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_ids), _ptr(expert_ids),
                           _ptr(num_post_pad), _stream()), "moe_align")
    return sorted_ids, expert_ids, num_post_pad


def moe_align_large(topk_ids: torch.Tensor, E: int, block_m: int, counts=None):
    """The multi-workgroup sort (same outputs as moe_align) -> (sorted_ids, expert_ids,
    num_post_pad); counts: int32 scratch of moe_align_large_scratch_bytes(E) bytes."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    cap = moe_align_capacity(T, k, E, block_m)
    dev = topk_ids.device
    sorted_ids = torch.empty((cap,), dtype=torch.int32, device=dev)
    expert_ids = torch.empty((cap // block_m if block_m else 0,), dtype=torch.int32, device=dev)
    num_post_pad = torch.zeros((1,), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((max(lib().moe_align_large_scratch_bytes(E) // 4, 1),),
                             dtype=torch.int32, device=dev)
    _check(lib().moe_align_large(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_ids),
                                 _ptr(expert_ids), _ptr(num_post_pad), _ptr(counts), _stream()),
           "moe_align_large")
    return sorted_ids, expert_ids, num_post_pad


def moe_route_align(logits: torch.Tensor, top_k: int, block_m: int, kind: str = "softmax",
                    expert_bias=None, renormalize: bool = True):
    """moe_route then moe_align in one call -> (topk_ids, topk_w, sorted_ids, expert_ids,
    num_post_pad), shaped as those two functions return them."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    cap = moe_align_capacity(T, top_k, E, block_m)
    topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    sorted_ids = torch.empty((cap,), dtype=torch.int32, device=dev)
    expert_ids = torch.empty((cap // block_m if block_m else 0,), dtype=torch.int32, device=dev)
    num_post_pad = torch.zeros((1,), dtype=torch.int32, device=dev)
    if expert_bias is not None:
        _dev(expert_bias, torch.float32, "expert_bias")
    _check(lib().moe_route_align(_ptr(logits), T, E, top_k, ROUTE[kind], _ptr(expert_bias),
                                 int(bool(renormalize)), block_m, _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(sorted_ids), _ptr(expert_ids), _ptr(num_post_pad),
                                 _stream()), "moe_route_align")
    return topk_ids, topk_w, sorted_ids, expert_ids, num_post_pad


def moe_w4a16_gemm1(x: torch.Tensor, top_k: int, w13: QuantWeights, act: str, alpha: float,
                    beta: float, limit: float, sorted_ids, expert_ids, num_post_pad,
                    block_m: int, out=None, topk_w=None, kernel: str = "auto"):
    """x bf16 [size_m, K] -> out bf16 [size_m*top_k, N/2 (gated) or N].

    topk_w (fp32 [size_m*top_k]) given: each input row is scaled by its slot's
    routing weight (the weight applied on the input).  kernel: "auto", "splitk"
    or "wide" for 16/32-row blocks (moe_w4a16_gemm1_ex)."""
    _dev(x, torch.bfloat16, "x")
    if topk_w is not None:
        _dev(topk_w, torch.float32, "topk_w")
    size_m, K = x.shape
    n_out = w13.N // 2 if act == "swigluoai" else w13.N
    if out is None:
        out = torch.zeros((size_m * top_k, n_out), dtype=torch.bfloat16, device=x.device)
    s = w13.struct()
    _check(lib().moe_w4a16_gemm1_ex(_ptr(x), size_m, top_k, K, w13.N, w13.E, ctypes.byref(s),
                                    ACT[act], alpha, beta, limit, _ptr(topk_w),
                                    int(topk_w is not None), _ptr(sorted_ids), _ptr(expert_ids),
                                    _ptr(num_post_pad), block_m, _ptr(out), KERNEL[kernel],
                                    _stream()),
           "moe_w4a16_gemm1_ex")
    return out


def moe_w4a16_gemm2(a: torch.Tensor, w2: QuantWeights, topk_w, mul_topk_weights: bool,
                    sorted_ids, expert_ids, num_post_pad, block_m: int, out=None,
                    top_k: int = 1, kernel: str = "auto"):
    """a bf16 [size_m, K] -> y bf16 [size_m*top_k, N]; row f reads A row f // top_k
    (top_k = 1: one A row per flat slot, the layer's view)."""
    _dev(a, torch.bfloat16, "a")
    size_m, K = a.shape
    if out is None:
        out = torch.zeros((size_m * top_k, w2.N), dtype=torch.bfloat16, device=a.device)
    s = w2.struct()
    _check(lib().moe_w4a16_gemm2_ex(_ptr(a), size_m, top_k, K, w2.N, w2.E, ctypes.byref(s),
                                    _ptr(topk_w), int(bool(mul_topk_weights)), _ptr(sorted_ids),
                                    _ptr(expert_ids), _ptr(num_post_pad), block_m, _ptr(out),
                                    KERNEL[kernel], _stream()), "moe_w4a16_gemm2_ex")
    return out


def moe_gptq_act_order_sort(qweight: torch.Tensor, g_idx: torch.Tensor, group: int):
    """Put act-order GPTQ rows in group order.

    qweight int32 [E, K/8, N], g_idx int32 [E, K] -> (qweight_sorted int32
    [E, K/8, N], k_perm int32 [E, K], status int32 [E]); status[e] != 0 marks
    an expert whose g_idx is not an act-order map."""
    _dev(qweight, torch.int32, "qweight")
    _dev(g_idx, torch.int32, "g_idx")
    E, kq, N = qweight.shape
    K = 8 * kq
    if tuple(g_idx.shape) != (E, K):
        raise ValueError(f"g_idx shape {tuple(g_idx.shape)} != {(E, K)}")
    out = torch.empty_like(qweight)
    k_perm = torch.empty((E, K), dtype=torch.int32, device=qweight.device)
    status = torch.empty((E,), dtype=torch.int32, device=qweight.device)
    _check(lib().moe_gptq_act_order_sort(_ptr(qweight), _ptr(g_idx), E, K, N, group, _ptr(out),
                                         _ptr(k_perm), _ptr(status), _stream()),
           "moe_gptq_act_order_sort")
    return out, k_perm, status


def moe_nvfp4_scales_by_chunk(w: "QuantWeights") -> torch.Tensor:
    """NVFP4 e4m3 scales [E, N, K/16] re-laid by 64-deep K chunk -> uint8 [E, K/64, N, 4]
    (set it as w.scales_kc to let the 64/128-row GEMM kernel stream the scales)."""
    if w.fmt != "nvfp4":
        raise ValueError("scales by chunk are an NVFP4 layout")
    _dev(w.scales, torch.uint8, "scales")
    E = w.scales.shape[0]
    out = torch.empty((E, w.K // 64, w.N, 4), dtype=torch.uint8, device=w.scales.device)
    _check(lib().moe_nvfp4_scales_by_chunk(_ptr(w.scales), E, w.N, w.K, _ptr(out), _stream()),
           "moe_nvfp4_scales_by_chunk")
    return out


def moe_nvfp4_codes_by_chunk(w: "QuantWeights") -> torch.Tensor:
    """NVFP4 codes [E, N, K/2] re-laid by 64-deep K chunk -> uint8 [E, K/64, N, 32]
    (set it as w.qweight_kc, together with w.scales_kc: every kernel then reads it in
    place of w.qweight, which may be dropped, see QuantWeights.chunked_only)."""
    if w.fmt != "nvfp4":
        raise ValueError("codes by chunk are an NVFP4 layout")
    _dev(w.qweight, torch.uint8, "qweight")
    E = w.qweight.shape[0]
    out = torch.empty((E, w.K // 64, w.N, 32), dtype=torch.uint8, device=w.qweight.device)
    _check(lib().moe_nvfp4_codes_by_chunk(_ptr(w.qweight), E, w.N, w.K, _ptr(out), _stream()),
           "moe_nvfp4_codes_by_chunk")
    return out


def moe_mxfp4_codes_by_chunk(w: "QuantWeights") -> torch.Tensor:
    """MXFP4 codes [E, N, K/2] re-laid by 128-deep K chunk -> uint8 [E, ceil(K/128), N, 64],
    zero past K (set it as w.qweight_kc: every kernel then reads it in place of w.qweight)."""
    if w.fmt != "mxfp4":
        raise ValueError("this re-layout is for MXFP4 codes")
    _dev(w.qweight, torch.uint8, "qweight")
    E = w.qweight.shape[0]
    out = torch.empty((E, (w.K + 127) // 128, w.N, 64), dtype=torch.uint8, device=w.qweight.device)
    _check(lib().moe_mxfp4_codes_by_chunk(_ptr(w.qweight), E, w.N, w.K, _ptr(out), _stream()),
           "moe_mxfp4_codes_by_chunk")
    return out


def moe_mxfp4_scales_by_chunk(w: "QuantWeights") -> torch.Tensor:
    """MXFP4 e8m0 scales [E, N, K/32] re-laid by 128-deep K chunk -> uint8
    [E, ceil(K/128), N, 4], zero past K/32 (set it as w.scales_kc: every kernel
    then reads it in place of w.scales)."""
    if w.fmt != "mxfp4":
        raise ValueError("this re-layout is for MXFP4 scales")
    _dev(w.scales, torch.uint8, "scales")
    E = w.scales.shape[0]
    out = torch.empty((E, (w.K + 127) // 128, w.N, 4), dtype=torch.uint8, device=w.scales.device)
    _check(lib().moe_mxfp4_scales_by_chunk(_ptr(w.scales), E, w.N, w.K, _ptr(out), _stream()),
           "moe_mxfp4_scales_by_chunk")
    return out


def moe_permute_slots(src: torch.Tensor, top_k: int, k_perm: torch.Tensor,
                      topk_ids: torch.Tensor, out=None):
    """dst[f] = src[f // top_k][k_perm[topk_ids[f]]] for every flat slot f.

    src bf16 [size_m, K]; topk_ids int32 [size_m*top_k]; out bf16
    [size_m*top_k, K] (may be src itself when top_k is 1)."""
    _dev(src, torch.bfloat16, "src")
    _dev(k_perm, torch.int32, "k_perm")
    _dev(topk_ids, torch.int32, "topk_ids")
    size_m, K = src.shape
    E = k_perm.shape[0]
    if out is None:
        out = torch.zeros((size_m * top_k, K), dtype=torch.bfloat16, device=src.device)
    _check(lib().moe_permute_slots(_ptr(src), size_m, top_k, K, E, _ptr(k_perm), _ptr(topk_ids),
                                   _ptr(out), _stream()), "moe_permute_slots")
    return out


def mxfp8_lda(K: int) -> int:
    """Row stride of MXFP8 codes: K rounded up to 128."""
    return (K + 127) // 128 * 128


def mxfp8_lds(K: int) -> int:
    """Row stride of MXFP8 scales: K/32 rounded up to 16."""
    return (K // 32 + 15) // 16 * 16


def moe_mxfp8_quantize(x: torch.Tensor, codes=True, dequant=False):
    """x bf16 [rows, K] -> (codes uint8 [rows, lda], scales uint8 [rows, lds]) and/or the
    dequantised bf16 [rows, K]; returns (codes, scales, dequant) with None for what was
    not asked for."""
    _dev(x, torch.bfloat16, "x")
    rows, K = x.shape
    c = s = d = None
    if codes:
        c = torch.empty((rows, mxfp8_lda(K)), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, mxfp8_lds(K)), dtype=torch.uint8, device=x.device)
    if dequant:
        d = torch.empty_like(x)
    _check(lib().moe_mxfp8_quantize(_ptr(x), rows, K, _ptr(c), _ptr(s), _ptr(d), _stream()),
           "moe_mxfp8_quantize")
    return c, s, d


def moe_mx_gemm1(codes, scales, top_k: int, K: int, w13: QuantWeights, act: str, alpha: float,
                 beta: float, limit: float, sorted_ids, expert_ids, num_post_pad, block_m: int,
                 out=None):
    """MXFP8 rows (codes [size_m, lda], scales [size_m, lds]) x MXFP4 w13 -> bf16 act."""
    size_m = codes.shape[0]
    n_out = w13.N // 2 if act == "swigluoai" else w13.N
    if out is None:
        out = torch.zeros((size_m * top_k, n_out), dtype=torch.bfloat16, device=codes.device)
    s = w13.struct()
    _check(lib().moe_mx_gemm1(_ptr(codes), _ptr(scales), size_m, top_k, K, w13.N, w13.E,
                              ctypes.byref(s), ACT[act], alpha, beta, limit, _ptr(sorted_ids),
                              _ptr(expert_ids), _ptr(num_post_pad), block_m, _ptr(out), _stream()),
           "moe_mx_gemm1")
    return out


def moe_mx_gemm2(codes, scales, K: int, w2: QuantWeights, topk_w, mul_topk_weights: bool,
                 sorted_ids, expert_ids, num_post_pad, block_m: int, out=None):
    """MXFP8 rows (one per flat slot) x MXFP4 w2 -> bf16 y [size_m, N]."""
    size_m = codes.shape[0]
    if out is None:
        out = torch.zeros((size_m, w2.N), dtype=torch.bfloat16, device=codes.device)
    s = w2.struct()
    _check(lib().moe_mx_gemm2(_ptr(codes), _ptr(scales), size_m, K, w2.N, w2.E, ctypes.byref(s),
                              _ptr(topk_w), int(bool(mul_topk_weights)), _ptr(sorted_ids),
                              _ptr(expert_ids), _ptr(num_post_pad), block_m, _ptr(out), _stream()),
           "moe_mx_gemm2")
    return out


def moe_forward_mxfp8_workspace_bytes(T: int, E: int, top_k: int, hidden: int, inter: int) -> int:
    return lib().moe_forward_mxfp8_workspace_bytes(T, E, top_k, hidden, inter)


def moe_forward_mxfp8(x: torch.Tensor, logits: torch.Tensor, top_k: int, inter: int,
                      w13: QuantWeights, w2: QuantWeights, act: str = "swigluoai",
                      route: str = "softmax", expert_bias=None, renormalize: bool = True,
                      alpha: float = 1.702, beta: float = 1.0, limit: float = 7.0,
                      mul_topk_weights: bool = True, workspace=None, out=None):
    """The layer with MXFP8 activations (MXFP4 weights): x bf16 [T, hidden] -> out bf16."""
    _dev(x, torch.bfloat16, "x")
    _dev(logits, torch.float32, "logits")
    T, hidden = x.shape
    E = logits.shape[1]
    need = moe_forward_mxfp8_workspace_bytes(T, E, top_k, hidden, inter)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=x.device)
    s13, s2 = w13.struct(), w2.struct()
    _check(lib().moe_forward_mxfp8(_ptr(x), _ptr(logits), T, E, top_k, hidden, inter, ROUTE[route],
                                   _ptr(expert_bias), int(bool(renormalize)), ctypes.byref(s13),
                                   ctypes.byref(s2), ACT[act], alpha, beta, limit,
                                   int(bool(mul_topk_weights)), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _ptr(out),
                                   _stream()), "moe_forward_mxfp8")
    return out


def moe_forward(x: torch.Tensor, logits: torch.Tensor, top_k: int, inter: int,
                w13: QuantWeights, w2: QuantWeights, act: str = "swigluoai",
                route: str = "softmax", expert_bias=None, renormalize: bool = True,
                alpha: float = 1.702, beta: float = 1.0, limit: float = 7.0,
                mul_topk_weights: bool = True, workspace=None, out=None,
                weight_on_input: bool = False, kernel: str = "auto"):
    """The whole layer: x bf16 [T, hidden], logits f32 [T, E] -> out bf16 [T, hidden].

    weight_on_input: the routing weight scales GEMM1's input rows instead of
    GEMM2's output rows (top_k must be 1).  kernel: the kernel for 16/32-row
    blocks, "auto", "splitk" or "wide" (moe_forward_ex)."""
    _dev(x, torch.bfloat16, "x")
    _dev(logits, torch.float32, "logits")
    T, hidden = x.shape
    E = logits.shape[1]
    need = moe_forward_workspace_bytes(T, E, top_k, hidden, inter)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=x.device)
    s13, s2 = w13.struct(), w2.struct()
    _check(lib().moe_forward_ex(_ptr(x), _ptr(logits), T, E, top_k, hidden, inter, ROUTE[route],
                                _ptr(expert_bias), int(bool(renormalize)), ctypes.byref(s13),
                                ctypes.byref(s2), ACT[act], alpha, beta, limit,
                                2 if weight_on_input else int(bool(mul_topk_weights)),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _ptr(out), KERNEL[kernel], _stream()),
           "moe_forward_ex")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_FORWARD_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(x: torch.Tensor, logits: torch.Tensor, top_k: int, inter: int,
                        w13: QuantWeights, w2: QuantWeights, out: torch.Tensor,
                        act: str = "swigluoai", route: str = "softmax", expert_bias=None,
                        renormalize: bool = True, alpha: float = 1.702, beta: float = 1.0,
                        limit: float = 7.0, mul_topk_weights: bool = True):
    """moe_forward on the library's fixed per-GPU scratch (no workspace
    argument; the library allocates nothing).  out bf16 [T, hidden] is the
    caller's.  Raises MoeError (status 7) when the call needs more scratch
    than NOALLOC_SCRATCH_BYTES."""
    _dev(x, torch.bfloat16, "x")
    _dev(logits, torch.float32, "logits")
    _dev(out, torch.bfloat16, "out")
    T, hidden = x.shape
    E = logits.shape[1]
    s13, s2 = w13.struct(), w2.struct()
    _check(lib().moe_forward_noalloc(_ptr(x), _ptr(logits), T, E, top_k, hidden, inter,
                                     ROUTE[route], _ptr(expert_bias), int(bool(renormalize)),
                                     ctypes.byref(s13), ctypes.byref(s2), ACT[act], alpha, beta,
                                     limit, int(bool(mul_topk_weights)), _ptr(out), _stream()),
           "moe_forward_noalloc")
    return out
