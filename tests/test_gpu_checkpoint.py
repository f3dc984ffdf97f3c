"""GPU parity of the checkpoint-series commit against the oracle and against
the replay commit (through the C ABI).

The series slot of token c - 1 holds the same fp32 value (rounded once to
the state dtype) that VERIFY_COMMIT stores when it keeps c tokens, so
CommitPrefix must leave exactly the replay commit's state, bit for bit; the
verify outputs equal VERIFY_ONLY's bit for bit.  Against the oracle: state
tolerances as for the GDN tests; conv series are copies of inputs (exact).
Slots no token maps to keep their contents.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import (DEV, GDN_STATE_TOL, GDN_STATE_TOL_F16, bits, check_gdn_out,
                         check_gdn_state, err_word, np64, npi, say, sv_batch)

pytestmark = pytest.mark.gpu


def _gdn_plain(batch, g, mode, commit, slots=None):
    out = torch.full_like(g['v'], float('nan'))
    st = g['state'].clone()
    bd.gdn_verify_commit(sv_batch(batch), mode, st, g['q'], g['k'], g['v'], g['alpha'],
                         g['beta'], commit, out, state_slot=slots)
    return out, st


def _gdn_ckpt(batch, g, window, commit, slots=None):
    sb = sv_batch(batch)
    out = torch.full_like(g['v'], float('nan'))
    H, dv, dk = g['state'].shape[1:]
    ck = torch.full((batch.B, window, H, dv, dk), float('nan'), dtype=g['state'].dtype,
                    device=DEV)
    st = g['state'].clone()
    err = err_word()
    bd.gdn_verify_checkpoint(sb, st, g['q'], g['k'], g['v'], g['alpha'], g['beta'], out, ck,
                             state_slot=slots, err=err)
    torch.cuda.synchronize()
    assert torch.equal(st, g['state'])            # the verify leaves the bank alone
    bd.gdn_commit_prefix(sb, st, ck, commit, state_slot=slots, err=err)
    torch.cuda.synchronize()
    return out, ck, st, int(err.item())


@pytest.mark.parametrize("wi,window,sdt", [(0, 4, torch.float32), (0, 6, torch.float16),
                                           (2, 4, torch.float32), (2, 5, torch.float16)])
def test_gdn_checkpoint_commit(wi, window, sdt):
    w = wl.WORKLOADS[wi]
    if wi == 2:
        w = wl.Workload(**{**w.__dict__, 'B': 16, 'ragged_k': True})
    batch = wl.make_batch(w, 70 + wi, DEV)
    g = wl.make_gdn_layer(w, batch, 71 + wi, DEV, state_dtype=sdt)
    commit = wl.make_commit_len(batch, 72 + wi, device=DEV)
    say('GDN checkpoint', w.name, 'window', window, sdt)
    out, ck, st, err = _gdn_ckpt(batch, g, window, commit)
    assert err == 0
    o_vo, _ = _gdn_plain(batch, g, bd.SV_GDN_VERIFY_ONLY, None)
    assert torch.equal(out, o_vo)
    _, s_vc = _gdn_plain(batch, g, bd.SV_GDN_VERIFY_COMMIT, commit)
    assert torch.equal(st, s_vc)
    # the series against the oracle; untouched slots stay NaN
    o_ref, ser = oracle.gdn_checkpoints(np64(g['state']), None, np64(g['q']), np64(g['k']),
                                        np64(g['v']), np64(g['alpha']), np64(g['beta']),
                                        npi(batch.cu_seqlens), window)
    check_gdn_out(np64(out), o_ref, w.gdn_dtype)
    tol = GDN_STATE_TOL if sdt == torch.float32 else GDN_STATE_TOL_F16
    ckn = np64(ck)
    for b in range(batch.B):
        T = batch.T[b]
        assert np.isnan(ckn[b, :window - T]).all()
        check_gdn_state(ckn[b, window - T:], ser[b, window - T:], tol=tol)
    S_ref = oracle.gdn_commit_prefix(np64(g['state']), None, ser, npi(batch.cu_seqlens),
                                     npi(commit), window)
    check_gdn_state(np64(st), S_ref, tol=tol)


def test_gdn_checkpoint_full_size_with_slots():
    """The hybrid step's GDN layer (B = 64, H = 32, dk = dv = 128), a slot map."""
    w = wl.WORKLOADS[2]
    batch = wl.make_batch(w, 80, DEV)
    ns = batch.B + 5
    g = wl.make_gdn_layer(w, batch, 81, DEV, num_slots=ns)
    slots = wl.make_state_slots(batch, ns, 82, DEV)
    commit = wl.make_commit_len(batch, 83, device=DEV)
    out, ck, st, err = _gdn_ckpt(batch, g, batch.max_T, commit, slots)
    assert err == 0
    o_vo, _ = _gdn_plain(batch, g, bd.SV_GDN_VERIFY_ONLY, None, slots)
    _, s_vc = _gdn_plain(batch, g, bd.SV_GDN_VERIFY_COMMIT, commit, slots)
    assert torch.equal(out, o_vo) and torch.equal(st, s_vc)


def test_gdn_commit_prefix_flags_bad_commit():
    w = wl.WORKLOADS[0]
    batch = wl.make_batch(w, 90, DEV)
    g = wl.make_gdn_layer(w, batch, 91, DEV)
    commit = torch.tensor([1, 9], dtype=torch.int32, device=DEV)
    _, _, st, err = _gdn_ckpt(batch, g, batch.max_T, commit)
    assert err & 8
    assert torch.equal(st[1], g['state'][1])


def _conv_plain(batch, c, mode, commit, silu):
    out = torch.full_like(c['x'], float('nan'))
    st = c['state'].clone()
    bd.short_conv_verify_commit(sv_batch(batch), mode, st, c['x'], c['weight'], c['bias'],
                                commit, out, activation=bd.SV_ACT_SILU if silu else bd.SV_ACT_NONE)
    return out, st


@pytest.mark.parametrize("wi,window,silu", [(0, 4, False), (3, 4, True), (4, 8, True)])
def test_conv_checkpoint_commit(wi, window, silu):
    w = wl.WORKLOADS[wi]
    batch = wl.make_batch(w, 100 + wi, DEV)
    c = wl.make_conv_layer(w, batch, 101 + wi, DEV)
    commit = wl.make_commit_len(batch, 102 + wi, device=DEV)
    sb = sv_batch(batch)
    Km1, C = c['state'].shape[1:]
    ps = torch.full((batch.B, window, Km1, C), float('nan'), dtype=c['state'].dtype, device=DEV)
    out = torch.full_like(c['x'], float('nan'))
    st = c['state'].clone()
    err = err_word()
    act = bd.SV_ACT_SILU if silu else bd.SV_ACT_NONE
    bd.short_conv_verify_checkpoint(sb, st, c['x'], c['weight'], c['bias'], out, ps,
                                    activation=act, err=err)
    torch.cuda.synchronize()
    assert torch.equal(st, c['state'])
    bd.short_conv_commit_prefix(sb, st, ps, commit, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o_vo, _ = _conv_plain(batch, c, bd.SV_GDN_VERIFY_ONLY, None, silu)
    _, s_vc = _conv_plain(batch, c, bd.SV_GDN_VERIFY_COMMIT, commit, silu)
    assert torch.equal(out, o_vo) and torch.equal(st, s_vc)
    y_ref, ser = oracle.conv_checkpoints(np64(c['state']), None, np64(c['x']), np64(c['weight']),
                                         None if c['bias'] is None else np64(c['bias']),
                                         npi(batch.cu_seqlens), window, silu=silu)
    check_gdn_out(np64(out), y_ref, w.gdn_dtype)
    psn = np64(ps)
    for b in range(batch.B):
        T = batch.T[b]
        assert np.array_equal(psn[b, :T], ser[b, :T])
        assert np.isnan(psn[b, T:]).all()
