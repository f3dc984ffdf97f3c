"""Helpers shared by the GPU parity tests (marshalling and comparisons)."""

import sys

import numpy as np
import torch

from block_draft_verification_spec_amd import binding as bd

DEV = 'cuda'

# Tolerances (stated in the test of each op): attention max-abs 2e-3 (fp32
# I/O) / 1e-2 + half a bf16 ulp of |o_ref| (bf16 I/O); committed GDN state
# max|dS| / max|S_ref| <= 1e-4 per (b, h) tile; GDN outputs 2e-3 (fp32) /
# 1e-2 + half a bf16 ulp of |o_ref|.
ATT_TOL = {torch.float32: 2e-3, torch.bfloat16: 1e-2}
GDN_STATE_TOL = 1e-4
# an fp16 state adds one rounding to nearest per stored element (unit
# roundoff 2^-11 relative) on top of the fp32 arithmetic
GDN_STATE_TOL_F16 = 2.0 ** -11 * (1 + GDN_STATE_TOL) + GDN_STATE_TOL
GDN_OUT_TOL = {torch.float32: 2e-3, torch.bfloat16: 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def npi(t):
    return t.detach().cpu().numpy().astype(np.int64)


def bits(t):
    """Raw bit pattern of a tensor as a NumPy integer array."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


def to_dev(d, device=DEV):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def sv_batch(b):
    return bd.make_batch(b.cu_seqlens, b.B, b.max_T, b.total_T)


def err_word():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return np.ldexp(1.0, (e - 8).astype(int))


def check_gdn_state(S_gpu, S_ref, tiles=None, tol=GDN_STATE_TOL):
    """Per (slot, h) tile: max|dS| / max|S_ref| <= tol."""
    S_gpu = np.asarray(S_gpu, dtype=np.float64)
    worst = 0.0
    ns, H = S_ref.shape[:2]
    for s in (range(ns) if tiles is None else tiles):
        for h in range(H):
            ref = S_ref[s, h]
            den = max(np.abs(ref).max(), 1e-30)
            worst = max(worst, np.abs(S_gpu[s, h] - ref).max() / den)
    assert worst <= tol, f'GDN state normwise error {worst:.3e}'
    return worst


def check_gdn_out(o_gpu, o_ref, dtype):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    d = np.abs(o_gpu - o_ref)
    if dtype == torch.bfloat16:
        bound = GDN_OUT_TOL[dtype] + bf16_half_ulp(o_ref)
    else:
        bound = GDN_OUT_TOL[dtype]
    bad = d > bound
    assert not bad.any(), f'GDN output: {bad.sum()} elements out of bound, max err {d.max():.3e}'
    return float(d.max())


def check_attn_out(o_gpu, o_ref, dtype):
    """Max-abs error against the bound of the I/O dtype; a bf16 output also
    carries its own final rounding, half a bf16 ulp of |o_ref| (at |o| >= 4 the
    bf16 neighbours are 2^-5 apart, so no bf16 result is within 1e-2 of
    every real value there)."""
    d = np.abs(np.asarray(o_gpu, dtype=np.float64) - o_ref)
    m = float(d.max()) if d.size else 0.0
    bound = ATT_TOL[dtype]
    if dtype == torch.bfloat16 and d.size:
        bound = ATT_TOL[dtype] + bf16_half_ulp(o_ref)
    bad = d > bound
    assert not np.any(bad), (f'attention: {int(np.sum(bad))} elements out of bound, '
                             f'max abs error {m:.3e}')
    return m
