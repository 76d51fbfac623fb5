"""Helpers for the GPU tests: upload synthetic layers, poison outputs, compare with the oracle."""
import numpy as np
import torch

import bit_weight_expert_amd as M
from oracle.moe import align, route, row_rel_err

TOL = 5e-3  # per-row max relative error (L2 norm of the row) against the float64 oracle


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> float64 numpy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def poisoned(shape, dtype=torch.bfloat16) -> torch.Tensor:
    """A device tensor whose every byte is 0xFF (bf16 / fp32 NaN, int32 -1): a row
    the kernels skip, or a workspace region they read before writing, shows."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xFF)
    return t


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


def gpu_forward(L, D, kernel="auto", **kw):
    """moe_forward on a workspace and output poisoned with 0xFF bytes."""
    T = D["x"].shape[0]
    E = D["logits"].shape[1]
    ws = poisoned((max(M.moe_forward_workspace_bytes(T, E, L.top_k, L.H, L.I), 1),), torch.uint8)
    out = poisoned((T, L.H))
    return M.moe_forward(D["x"], D["logits"], L.top_k, L.I, D["w13"], D["w2"], act=L.act,
                         route=L.route, expert_bias=D["expert_bias"], renormalize=L.renormalize,
                         alpha=L.alpha, beta=L.beta, limit=L.limit,
                         mul_topk_weights=L.mul_topk_weights,
                         weight_on_input=getattr(L, "weight_on_input", False), workspace=ws,
                         out=out, kernel=kernel, **kw)


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


def assert_untouched(out: torch.Tensor, covered: np.ndarray, what=""):
    """Rows no aligned block covers keep their poison bytes (the kernels leave them)."""
    bits = out.view(torch.int16).cpu().numpy()
    rest = bits[~np.asarray(covered, bool)]
    assert (rest == -1).all(), f"{what}: rows no block covers were written"


def block_covering_tokens(ids: np.ndarray, E: int, block_m: int, extra=(), limit=None):
    """Tokens chosen so that every aligned block of moe_align(ids, E, block_m)
    holds at least one slot of a chosen token: for each block, the token of its
    first real slot (expert ids ascending, so each expert's last, partial block
    is included), plus `extra`.  Returns a sorted list."""
    sorted_ids, expert_ids, npp = align(ids, E, block_m)
    n = ids.size
    k = ids.shape[1]
    toks = set(int(t) for t in extra if t < ids.shape[0])
    for b in range(int(npp) // block_m):
        blk = sorted_ids[b * block_m:(b + 1) * block_m]
        real = blk[blk < n]
        if real.size and not any(int(f) // k in toks for f in real):
            toks.add(int(real[0]) // k)
    out = sorted(toks)
    return out if limit is None else out[:limit]


__all__ = ["TOL", "dev_bf16", "host_bf16", "poisoned", "upload_weights", "upload", "gpu_forward",
           "assert_rows_close", "assert_untouched", "block_covering_tokens", "route"]
