"""The C-ABI library: it loads, exports every function include/moe_w4a16.h declares,
and rejects invalid arguments on the host before any launch (CPU only: no call
here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import bit_weight_expert_amd as M
from bit_weight_expert_amd._binding import _Wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")

OK, NULL, SHAPE, UNSUP, ALIGN, HIP, WS, TOO_LARGE = range(8)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.library_path()):
        pytest.skip("library not built")
    return M.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert set(names) >= {"moe_route", "moe_align", "moe_w4a16_gemm1", "moe_w4a16_gemm2",
                          "moe_forward", "moe_align_capacity", "moe_forward_workspace_bytes",
                          "moe_status_str", "moe_forward_block_m"}
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"


def test_status_strings(L):
    for s in range(8):
        assert len(L.moe_status_str(s)) > 0


def test_capacity_and_workspace(L):
    assert L.moe_align_capacity(1, 4, 32, 16) == 64          # 4 slots, each may open a block
    assert L.moe_align_capacity(4096, 4, 32, 128) == 16384 + 32 * 128
    assert L.moe_align_capacity(0, 4, 32, 16) == 0
    assert L.moe_forward_workspace_bytes(0, 32, 4, 2880, 2880) == 0
    ws = L.moe_forward_workspace_bytes(64, 32, 4, 2880, 2880)
    assert ws >= 64 * 4 * (2880 + 2880) * 2


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _wq(fmt=0, group=16, qweight=FAKE, scales=FAKE, zeros=None, gs=FAKE, g_idx=None, bias=None,
        k_perm=None, scales_kc=None, qweight_kc=None):
    return _Wq(fmt, group, qweight, scales, zeros, gs, g_idx, bias, k_perm, scales_kc, qweight_kc)


def test_route_rejects(L):
    assert L.moe_route(FAKE, 4, 8, 9, 0, None, 1, FAKE, FAKE, None) == SHAPE      # top_k > E
    assert L.moe_route(FAKE, 4, 2048, 4, 0, None, 1, FAKE, FAKE, None) == SHAPE   # E too large
    assert L.moe_route(FAKE, 4, 64, 17, 0, None, 1, FAKE, FAKE, None) == SHAPE    # top_k > 16
    assert L.moe_route(None, 4, 8, 2, 0, None, 1, FAKE, FAKE, None) == NULL
    assert L.moe_route(FAKE, 4, 8, 2, 1, None, 1, FAKE, FAKE, None) == NULL       # bias needed
    assert L.moe_route(FAKE, 4, 8, 2, 7, None, 1, FAKE, FAKE, None) == UNSUP
    assert L.moe_route(None, 0, 8, 2, 0, None, 1, None, None, None) == OK         # T = 0: no-op


def test_align_rejects(L):
    assert L.moe_align(FAKE, 4, 2, 8, 48, FAKE, FAKE, FAKE, None) == SHAPE       # block_m
    assert L.moe_align(FAKE, 4, 2, 0, 16, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.moe_align(FAKE, 1 << 23, 4, 8, 16, FAKE, FAKE, FAKE, None) == SHAPE  # too many slots
    assert L.moe_align(FAKE, 4, 2, 8, 16, FAKE, None, FAKE, None) == NULL
    assert L.moe_align(None, 0, 2, 8, 16, None, None, None, None) == OK


def _g1(L, w, K=2880, N=5760, act=0, x=FAKE, out=FAKE, block_m=16, tw=None, mul=0):
    return L.moe_w4a16_gemm1(x, 8, 4, K, N, 32, ctypes.byref(w), act, 1.702, 1.0, 7.0,
                             tw, mul, FAKE, FAKE, FAKE, block_m, out, None)


def test_gemm1_rejects(L):
    assert _g1(L, _wq(), K=2880 + 16) == SHAPE           # K % 32
    assert _g1(L, _wq(), N=5760 + 8) == SHAPE            # N % 16
    assert _g1(L, _wq(), N=5760 + 16) == SHAPE           # gated N % 32
    assert _g1(L, _wq(group=32)) == UNSUP                # NVFP4 is group 16
    assert _g1(L, _wq(fmt=1, group=16)) == UNSUP         # MXFP4 is group 32
    assert _g1(L, _wq(fmt=2, group=64, zeros=FAKE), K=2880 + 32) == SHAPE   # K % group
    assert _g1(L, _wq(fmt=2, group=64, zeros=FAKE, g_idx=FAKE), x=None) == NULL  # map accepted
    assert _g1(L, _wq(fmt=2, group=64, zeros=FAKE, k_perm=FAKE)) == UNSUP   # gather first
    assert _g1(L, _wq(k_perm=FAKE)) == UNSUP             # act-order is a GPTQ form
    assert _g1(L, _wq(fmt=2, group=64, zeros=FAKE, scales_kc=FAKE)) == UNSUP   # no GPTQ form
    assert _g1(L, _wq(fmt=1, group=32, gs=None, scales_kc=FAKE), x=None) == NULL  # MXFP4: accepted
    assert _g1(L, _wq(scales_kc=FAKE), K=2880 + 32) == SHAPE       # needs K % 64 == 0
    assert _g1(L, _wq(scales_kc=FAKE + 4)) == ALIGN
    assert _g1(L, _wq(qweight_kc=FAKE)) == UNSUP         # NVFP4 codes by chunk need scales by chunk
    assert _g1(L, _wq(fmt=2, group=64, zeros=FAKE, qweight_kc=FAKE)) == UNSUP   # no GPTQ form
    assert _g1(L, _wq(scales_kc=FAKE, qweight_kc=FAKE), K=2880 + 32) == SHAPE
    assert _g1(L, _wq(scales_kc=FAKE, qweight_kc=FAKE + 4)) == ALIGN
    # chunked-only NVFP4/MXFP4 families: no checkpoint layout, both copies by chunk
    kc = dict(qweight=None, scales=None, scales_kc=FAKE, qweight_kc=FAKE)
    assert _g1(L, _wq(**kc), x=None) == NULL                          # accepted (x checked next)
    assert _g1(L, _wq(fmt=1, group=32, gs=None, **kc), x=None) == NULL  # MXFP4 too
    assert _g1(L, _wq(**kc), K=2880 + 32) == SHAPE                    # NVFP4 by chunk: K % 64
    assert _g1(L, _wq(qweight=None, scales_kc=FAKE, qweight_kc=FAKE)) == NULL  # scales left over
    assert _g1(L, _wq(scales=None, scales_kc=FAKE, qweight_kc=FAKE)) == NULL   # codes left over
    assert _g1(L, _wq(qweight=None, scales=None, scales_kc=FAKE)) == NULL      # no codes at all
    assert _g1(L, _wq(fmt=1, group=32, gs=None, qweight=None, scales=None,
                      qweight_kc=FAKE)) == NULL                       # MXFP4: scales by chunk too
    assert _g1(L, _wq(fmt=2, group=64, zeros=FAKE, **kc)) == NULL     # GPTQ has one layout
    assert _g1(L, _wq(fmt=2, group=64)) == NULL          # zeros missing
    assert _g1(L, _wq(gs=None)) == NULL                  # NVFP4 global scale missing
    assert _g1(L, _wq(fmt=9)) == UNSUP
    assert _g1(L, _wq(), act=5) == UNSUP
    assert _g1(L, _wq(qweight=FAKE + 8)) == ALIGN
    assert _g1(L, _wq(), x=FAKE + 2) == ALIGN
    assert _g1(L, _wq(), x=None) == NULL
    assert _g1(L, _wq(), block_m=8) == SHAPE
    assert _g1(L, _wq(), mul=1) == NULL                  # weight on the input needs the weights


def test_gemm2_rejects(L):
    w = _wq()
    g2 = lambda **kw: L.moe_w4a16_gemm2(kw.get("a", FAKE), 32, kw.get("k", 1), 2880, 2880, 32,
                                        ctypes.byref(kw.get("w", w)),
                                        kw.get("tw", FAKE), kw.get("mul", 1), FAKE, FAKE, FAKE,
                                        kw.get("bm", 16), kw.get("y", FAKE), None)
    assert g2(tw=None) == NULL                           # weights needed when multiplying
    assert g2(bm=256) == SHAPE
    assert g2(y=None) == NULL
    assert g2(w=_wq(scales=None)) == NULL
    assert g2(k=0) == SHAPE                              # top_k >= 1
    assert g2(k=1 << 20) == SHAPE                        # size_m * top_k < 2^24


def test_no_process_wide_state(L):
    """The kernel choice is an argument of the _ex calls, not library state."""
    assert not hasattr(L, "moe_set_decode_policy")


def test_kernel_choice_rejects(L):
    w = _wq()
    g1 = lambda kern: L.moe_w4a16_gemm1_ex(FAKE, 32, 4, 2880, 5760, 32, ctypes.byref(w), 0, 1.702,
                                           1.0, 7.0, None, 0, FAKE, FAKE, FAKE, 16, FAKE, kern, None)
    g2 = lambda kern: L.moe_w4a16_gemm2_ex(FAKE, 32, 1, 2880, 2880, 32, ctypes.byref(w), FAKE, 1,
                                           FAKE, FAKE, FAKE, 16, None, kern, None)
    f = lambda kern: L.moe_forward_ex(FAKE, FAKE, 8, 32, 4, 2880, 2880, 0, None, 1,
                                      ctypes.byref(w), ctypes.byref(w), 0, 1.702, 1.0, 7.0, 1,
                                      FAKE * 16, 0, FAKE, kern, None)
    for bad in (-1, 3, 17):
        assert g1(bad) == UNSUP and g2(bad) == UNSUP and f(bad) == UNSUP
    for good in (0, 1, 2):
        assert g2(good) == NULL                          # accepted, then y = NULL
        assert f(good) == WS                             # accepted, then the workspace size


def test_g_idx_rules(L):
    """GPTQ g_idx is accepted (checked against the identity on the device);
    other formats take none; not together with k_perm; 4-byte alignment."""
    g = dict(fmt=2, group=64, zeros=FAKE)
    g1 = lambda w: L.moe_w4a16_gemm1(FAKE, 32, 4, 2880, 5760, 32, ctypes.byref(w), 0, 1.702, 1.0,
                                     7.0, None, 0, FAKE, FAKE, FAKE, 16, None, None)
    assert g1(_wq(g_idx=FAKE, **g)) == NULL              # accepted, then out = NULL
    assert g1(_wq(g_idx=FAKE + 2, **g)) == ALIGN
    assert g1(_wq(g_idx=FAKE)) == UNSUP                  # NVFP4 has no group map
    assert g1(_wq(fmt=1, group=32, gs=None, g_idx=FAKE)) == UNSUP
    w = _wq(g_idx=FAKE, k_perm=FAKE, **g)
    f = L.moe_forward(FAKE, FAKE, 8, 32, 4, 2880, 2880, 0, None, 1, ctypes.byref(w),
                      ctypes.byref(w), 0, 1.702, 1.0, 7.0, 1, FAKE * 16, 1 << 40, FAKE, None)
    assert f == UNSUP                                    # sorted weights carry no group map


def test_forward_rejects(L):
    w13, w2 = _wq(), _wq()
    f = lambda **kw: L.moe_forward(FAKE, FAKE, kw.get("T", 8), 32, kw.get("k", 4), 2880, 2880,
                                   kw.get("kind", 0), None, 1, ctypes.byref(w13), ctypes.byref(w2),
                                   kw.get("act", 0), 1.702, 1.0, 7.0, kw.get("mul", 1),
                                   kw.get("ws", FAKE * 16), kw.get("wsb", 0), FAKE, None)
    assert f() == WS                                     # workspace too small
    assert f(ws=FAKE + 16, wsb=1 << 40) == ALIGN         # workspace must be 256-byte aligned
    assert f(act=2) == UNSUP                             # forward needs a real activation
    assert f(k=33) == SHAPE
    assert f(kind=1) == NULL                             # sigmoid routing needs the bias
    assert f(T=0) == OK
    assert f(mul=2) == SHAPE                             # weight on the input needs top_k = 1
    assert f(mul=3) == UNSUP
    assert f(mul=2, k=1) == WS                           # accepted with top_k = 1 (then sizes)
    g = dict(fmt=2, group=64, zeros=FAKE)
    w13, w2 = _wq(k_perm=FAKE, **g), _wq(k_perm=FAKE, **g)
    assert f() == WS                                     # act-order families are accepted
    w13 = _wq(k_perm=FAKE + 4, **g)
    assert f(ws=FAKE * 16, wsb=1 << 40) == ALIGN         # k_perm must be 16-byte aligned


def test_act_order_entry_points_reject(L):
    s = lambda **kw: L.moe_gptq_act_order_sort(kw.get("q", FAKE), kw.get("g", FAKE), kw.get("E", 4),
                                               kw.get("K", 2880), 256, kw.get("G", 64),
                                               kw.get("o", FAKE * 2), FAKE, FAKE, None)
    assert s(G=16) == UNSUP
    assert s(K=2880 + 32) == SHAPE                       # K % group
    assert s(K=8192 + 128, G=128) == SHAPE               # K above the staging limit
    assert s(E=0) == SHAPE
    assert s(g=None) == NULL
    assert s(o=FAKE) == UNSUP                            # in place is not allowed
    p = lambda **kw: L.moe_permute_slots(kw.get("src", FAKE), kw.get("m", 8), kw.get("k", 4),
                                         kw.get("K", 2880), 32, kw.get("perm", FAKE), FAKE,
                                         kw.get("dst", FAKE * 2), None)
    assert p(K=2884) == SHAPE
    assert p(dst=FAKE) == UNSUP                          # in place needs top_k = 1
    assert p(perm=FAKE + 4) == ALIGN
    assert p(src=None) == NULL
    assert p(m=0, src=None) == OK


def test_mxfp8_entry_points_reject(L):
    q = lambda **kw: L.moe_mxfp8_quantize(kw.get("x", FAKE), kw.get("rows", 4), kw.get("K", 2880),
                                          kw.get("c", FAKE), kw.get("s", FAKE), kw.get("d", None), None)
    assert q(K=2880 + 16) == SHAPE
    assert q(c=None, s=None, d=None) == NULL
    assert q(x=FAKE + 2) == ALIGN
    assert q(rows=0, x=None) == OK
    mx = dict(fmt=1, group=32)
    g1 = lambda w, bm=128, K=2880, act=0: L.moe_mx_gemm1(FAKE, FAKE, 64, 4, K, 5760, 32, ctypes.byref(w),
                                                         act, 1.702, 1.0, 7.0, FAKE, FAKE, FAKE, bm,
                                                         FAKE, None)
    assert g1(_wq()) == UNSUP                            # NVFP4 weights: not an MX operand
    assert g1(_wq(**mx), bm=32) == UNSUP                 # MX kernel tiles are 64 or 128 rows
    assert g1(_wq(**mx), K=8192) == UNSUP                # scale tiles past the kernel's LDS
    assert g1(_wq(**mx), act=7) == UNSUP
    f = lambda w13, w2, mul=1: L.moe_forward_mxfp8(FAKE, FAKE, 8, 32, 4, 2880, 2880, 0, None, 1,
                                                   ctypes.byref(w13), ctypes.byref(w2), 0, 1.702, 1.0,
                                                   7.0, mul, FAKE * 16, 0, FAKE, None)
    assert f(_wq(), _wq()) == UNSUP                      # MXFP4 weights only
    assert f(_wq(**mx), _wq(**mx), mul=2) == UNSUP       # no routing weight on the input
    assert f(_wq(**mx), _wq(**mx)) == WS
    assert L.moe_forward_mxfp8_workspace_bytes(64, 32, 4, 2880, 2880) > \
        L.moe_forward_workspace_bytes(64, 32, 4, 2880, 2880)


def test_align_large_rejects(L):
    f = lambda **kw: L.moe_align_large(kw.get("ids", FAKE), kw.get("T", 64), 4, kw.get("E", 32),
                                       kw.get("B", 64), FAKE, FAKE, FAKE, kw.get("c", FAKE), None)
    assert f(c=None) == NULL
    assert f(ids=None) == NULL
    assert f(E=0) == SHAPE
    assert f(B=48) == SHAPE
    assert f(T=0, c=None) == 0                           # empty batch: nothing to do
    assert L.moe_align_large_scratch_bytes(32) == 16 * 32 * 4
    assert L.moe_align_large_scratch_bytes(0) == 0


def test_mxfp4_codes_by_chunk_rejects(L):
    f = lambda **kw: L.moe_mxfp4_codes_by_chunk(kw.get("q", FAKE), kw.get("E", 4), 256,
                                                kw.get("K", 2880), kw.get("o", FAKE * 2), None)
    assert f(K=2880 + 16) == SHAPE
    assert f(E=0) == SHAPE
    assert f(q=None) == NULL
    assert f(o=FAKE) == UNSUP
    assert f(o=FAKE * 2 + 4) == ALIGN


def test_codes_by_chunk_rejects(L):
    f = lambda **kw: L.moe_nvfp4_codes_by_chunk(kw.get("q", FAKE), kw.get("E", 4), 256,
                                                kw.get("K", 2880), kw.get("o", FAKE * 2), None)
    assert f(K=2880 + 32) == SHAPE
    assert f(E=0) == SHAPE
    assert f(q=None) == NULL
    assert f(o=FAKE) == UNSUP                            # not in place
    assert f(o=FAKE * 2 + 4) == ALIGN


def test_scales_by_chunk_rejects(L):
    f = lambda **kw: L.moe_nvfp4_scales_by_chunk(kw.get("s", FAKE), kw.get("E", 4), 256,
                                                 kw.get("K", 2880), kw.get("o", FAKE * 2), None)
    assert f(K=2880 + 32) == SHAPE
    assert f(E=0) == SHAPE
    assert f(s=None) == NULL
    assert f(o=FAKE) == UNSUP                            # not in place
    assert f(o=FAKE * 2 + 4) == ALIGN
