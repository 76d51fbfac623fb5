"""Helpers for the GPU tests: upload synthetic layers and compare with the oracle."""
import contextlib

import numpy as np
import torch

import bit_weight_expert_amd as M
from oracle.moe import row_rel_err

TOL = 5e-3  # per-row max relative error (L2 norm of the row) against the float64 oracle


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> float64 numpy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def upload_weights(w) -> "M.QuantWeights":
    return M.QuantWeights.from_arrays(w.fmt, w.group, w.N, w.K, w.qweight, w.scales, w.zeros,
                                      w.global_scale, w.bias)


def upload(L):
    return dict(
        x=dev_bf16(L.x),
        logits=torch.from_numpy(np.ascontiguousarray(L.logits)).cuda(),
        expert_bias=None if L.expert_bias is None else torch.from_numpy(L.expert_bias).cuda(),
        w13=upload_weights(L.w13),
        w2=upload_weights(L.w2),
    )


def gpu_forward(L, D, **kw):
    return M.moe_forward(D["x"], D["logits"], L.top_k, L.I, D["w13"], D["w2"], act=L.act,
                         route=L.route, expert_bias=D["expert_bias"], renormalize=L.renormalize,
                         alpha=L.alpha, beta=L.beta, limit=L.limit,
                         mul_topk_weights=L.mul_topk_weights,
                         weight_on_input=getattr(L, "weight_on_input", False), **kw)


def assert_rows_close(got, ref, rows=None, tol=TOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.isfinite(got).all(), f"{what}: non-finite values in GPU output"
    rel = row_rel_err(got, ref)
    worst = int(np.argmax(rel)) if rel.size else -1
    assert rel.size == 0 or rel.max() <= tol, (
        f"{what}: max per-row rel err {rel.max():.3e} at row {worst} (tol {tol})")
    return float(rel.max()) if rel.size else 0.0


@contextlib.contextmanager
def decode_policy(policy):
    """Run the body with the library's kernel choice for 16/32-row blocks forced."""
    old = M.moe_set_decode_policy(policy)
    try:
        yield
    finally:
        M.moe_set_decode_policy(old)
