"""Helpers for the GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare with the stated tolerances.

Tolerances (fixed by the method's target, not tuned):
  O    max-abs <= 1e-2 over all elements
  LSE  max-abs <= 1e-3 over finite entries; -inf positions must coincide
  dQ, dK, dV  relative L2 <= 2e-2 per tensor
  rows that see no key: O row and dQ row exactly 0
"""
import sys

import numpy as np
import torch

import oracle
import workloads

O_TOL, LSE_TOL, GRAD_TOL = 1e-2, 1e-3, 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    if isinstance(t, torch.Tensor):
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.float()
        return t.detach().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def gpu_inputs(w, seed=None, device="cuda"):
    q, k, v, do = workloads.make_tensors(w, seed=seed, device=device)
    vec = workloads.mask_tensors(w, device=device)
    return q, k, v, do, vec


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 (8 significant bits) at |x|: the distance from x to the
    nearest bf16 value is at most this."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, np.finfo(np.float64).tiny)))
    return np.exp2(e - 8)


def check_fwd(O, LSE, O_ref, LSE_ref, ctx="", format_slack=False):
    """O max-abs <= O_TOL; with format_slack, per element O_TOL plus half a bf16 ulp of the
    exact value (an output stored in bf16 cannot be nearer to it than that, which is above
    O_TOL once |O| >= 4)."""
    O, LSE = to_np(O), to_np(LSE)
    if format_slack and O.size:
        excess = np.abs(O - O_ref) - bf16_half_ulp(O_ref)
        err = max(float(excess.max()), 0.0)
    else:
        err = np.abs(O - O_ref).max() if O.size else 0.0
    fin = np.isfinite(LSE_ref)
    assert np.array_equal(np.isneginf(LSE), np.isneginf(LSE_ref)), f"{ctx}: -inf LSE rows differ"
    lerr = np.abs(LSE[fin] - LSE_ref[fin]).max() if fin.any() else 0.0
    dead = ~fin
    assert (O[dead] == 0).all(), f"{ctx}: rows that see nothing must give O = 0"
    assert err <= O_TOL, f"{ctx}: O max-abs {err:.3e}"
    assert lerr <= LSE_TOL, f"{ctx}: LSE max-abs {lerr:.3e}"
    return err, lerr


def check_grads(dQ, dK, dV, ref, LSE_ref=None, ctx=""):
    out = []
    for name, x, r in (("dQ", dQ, ref[0]), ("dK", dK, ref[1]), ("dV", dV, ref[2])):
        e = rel_l2(to_np(x), r)
        assert e <= GRAD_TOL, f"{ctx}: {name} rel-L2 {e:.3e}"
        out.append(e)
    if LSE_ref is not None:
        dead = ~np.isfinite(LSE_ref)
        assert (to_np(dQ)[dead] == 0).all(), f"{ctx}: dQ rows that see nothing must be 0"
    return out


def full_parity(w, seed=None, scale=None, bwd=True, key_order=0):
    """HIP fwd (+bwd) vs the full oracle on workload w (small sizes only)."""
    import mask_aware_sparse_amd as fm
    q, k, v, do, vec = gpu_inputs(w, seed)
    O, LSE = fm.attn_fwd(q, k, v, *vec, scale=scale, key_order=key_order)
    if bwd:
        dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec, scale=scale, key_order=key_order)
    torch.cuda.synchronize()
    hq, hk, hv, hdo = (to_np(x) for x in (q, k, v, do))
    if bwd:
        O_ref, LSE_ref, dQr, dKr, dVr = oracle.attention_fwd_bwd(hq, hk, hv, hdo, *w.vectors(),
                                                                 scale=scale)
    else:
        O_ref, LSE_ref = oracle.attention_fwd(hq, hk, hv, *w.vectors(), scale=scale)
    res = {"fwd": check_fwd(O, LSE, O_ref, LSE_ref, ctx=w.name)}
    if bwd:
        res["bwd"] = check_grads(dq, dk, dv, (dQr, dKr, dVr), LSE_ref, ctx=w.name)
    return res
