"""GPU parity at full size, in the launch configuration the benchmark times.

hybrid_step_64l: two consecutive verify steps of the 64-layer hybrid stack
(B = 64, k = 3, contexts U[2048, 8192], 48 GDN + 16 attention layers,
rejection acceptance over V = 151936, deferred schedule: the second step
replays the first step's accepted GDN tokens before verifying its own), then
a flush of the second step's accepted tokens.

stress_ragged_long: one two-phase step (B = 256, k_b ~ U{1..7}, contexts
U[16384, 32768], fragmented pool, one GDN,GDN,GDN,ATT group).

Acceptance, commit lengths and ctx_lens are checked for every sequence.
Layer outputs, the written KV pages and the committed GDN states are checked
on a sample of sequences: every per-sequence result depends on that
sequence's inputs alone, so the oracle runs on the sampled sequence by itself
(its pages gathered into a private pool).  Tolerances as in the per-op tests.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import (DEV, bits, check_attn_out, check_gdn_out, check_gdn_state, err_word,
                         np64, npi, say, sv_batch)

pytestmark = pytest.mark.gpu


def _layers(w, batch, seed):
    layers = []
    for i, kind in enumerate(w.layers):
        if kind == 'attn':
            lay = wl.make_attn_layer(w, batch, seed + 10 * i, DEV)
            lay['out'] = torch.full_like(lay['q'], float('nan'))
        else:
            lay = wl.make_gdn_layer(w, batch, seed + 10 * i, DEV)
            lay['out'] = torch.full_like(lay['v'], float('nan'))
        lay['kind'] = kind
        layers.append(lay)
    return layers


def _step_args(w, batch, layers, acc):
    return bd.StepArgs(
        [1 if l['kind'] == 'attn' else 0 for l in layers],
        bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table,
                       bd.SV_BF16),
        [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'], l['out'])
         for l in layers if l['kind'] == 'attn'],
        bd.gdn_config(w.H, w.dk, w.dv, batch.B, bd.SV_BF16),
        [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'], l['out'])
         for l in layers if l['kind'] == 'gdn'],
        bd.accept_args(bd.SV_ACCEPT_REJECTION, acc['target_logits'], acc['draft_tokens'],
                       acc['draft_logits'], acc['u_accept'], acc['u_final']))


def _seq_pages(batch, b):
    row = npi(batch.block_table[b])
    return row[row >= 0]


def _snapshot(layers, batch, seqs):
    """Host float64 copies of what the oracle needs for the sampled sequences."""
    cu = npi(batch.cu_seqlens)
    snap = []
    for l in layers:
        d = {}
        for b in seqs:
            r = slice(cu[b], cu[b + 1])
            if l['kind'] == 'attn':
                pg = torch.from_numpy(_seq_pages(batch, b)).to(DEV)
                d[b] = dict(K=np64(l['k_cache'][pg]), V=np64(l['v_cache'][pg]),
                            q=np64(l['q'][r]), kn=np64(l['k_new'][r]), vn=np64(l['v_new'][r]))
            else:
                d[b] = dict(S=np64(l['state'][b:b + 1]), q=np64(l['q'][r]), k=np64(l['k'][r]),
                            v=np64(l['v'][r]), alpha=np64(l['alpha'][r]),
                            beta=np64(l['beta'][r]))
        snap.append(d)
    return snap


def _oracle_accept(acc, batch):
    return oracle.rejection_accept(np64(acc['target_logits']), np64(acc['draft_logits']),
                                   npi(acc['draft_tokens']), np64(acc['u_accept']),
                                   np64(acc['u_final']), npi(batch.cu_seqlens), batch.max_T)


def _check_accept(res, ref_acc, ref_out, ctx_before, commit, ctx):
    B = len(ref_acc)
    r = npi(res)
    np.testing.assert_array_equal(r[:B], ref_acc)
    np.testing.assert_array_equal(r[B:].reshape(B, -1), ref_out)
    np.testing.assert_array_equal(npi(commit), ref_acc + 1)
    np.testing.assert_array_equal(npi(ctx), ctx_before + ref_acc + 1)


def _attn_oracle(s, L, T, P):
    """One sequence alone: its pages renumbered 0..n-1 in a private pool."""
    n = s['K'].shape[0]
    sub_t = np.arange(n)[None, :]
    cu = np.array([0, T])
    o = oracle.verify_attention(s['q'], s['kn'], s['vn'], s['K'], s['V'], sub_t,
                                np.array([L]), cu, P)
    K2, V2 = oracle.append_kv(s['K'], s['V'], s['kn'], s['vn'], sub_t, np.array([L]), cu, P)
    return o, K2, V2


def _bits_as(values64, like):
    return bits(torch.from_numpy(values64).to(like.dtype))


def test_hybrid_step_64l_two_deferred_steps():
    w = wl.WORKLOADS[3]
    batch = wl.make_batch(w, 11, DEV, reserve=2 * w.max_T)
    say('full hybrid step: generating 64 layers, B =', batch.B)
    layers = _layers(w, batch, 1100)
    acc = wl.make_accept(w, batch, 1999, 'rejection', DEV)
    torch.cuda.synchronize()
    seqs = sorted({0, 21, 42, batch.B - 1, int(np.argmax(batch.ctx))})
    snap = _snapshot(layers, batch, seqs)
    cu = npi(batch.cu_seqlens)
    ctx0 = npi(batch.ctx_lens)

    args = _step_args(w, batch, layers, acc)
    sb = sv_batch(batch)
    ws = torch.zeros(bd.spec_verify_step_workspace_bytes(sb, args), dtype=torch.uint8,
                     device=DEV)
    ctx = batch.ctx_lens.clone()
    err = err_word()
    results = [torch.full((batch.B * (1 + batch.max_T),), -7, dtype=torch.int32, device=DEV)
               for _ in range(2)]
    commits = [torch.full((batch.B,), -7, dtype=torch.int32, device=DEV) for _ in range(2)]

    say('  step 1 (deferred, nothing pending)')
    bd.spec_verify_step(sb, args, ctx, results[0], commits[0], schedule=bd.SV_SCHEDULE_DEFERRED,
                        workspace=ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ctx1 = ctx.clone()
    out1 = [{b: np64(l['out'][cu[b]:cu[b + 1]]) for b in seqs} for l in layers]
    pages1 = [{b: (bits(l['k_cache'][torch.from_numpy(_seq_pages(batch, b)).to(DEV)]),
                   bits(l['v_cache'][torch.from_numpy(_seq_pages(batch, b)).to(DEV)]))
               for b in seqs} if l['kind'] == 'attn' else None for l in layers]

    say('  step 2 (deferred, replays step 1)')
    pend_arr = (bd.SvGdnLayer * len(args.gdn))(*args.gdn)
    pend = bd.SvStepPending(sb, pend_arr, commits[0].data_ptr())
    for l in layers:
        l['out'].fill_(float('nan'))
    bd.spec_verify_step(sb, args, ctx, results[1], commits[1], schedule=bd.SV_SCHEDULE_DEFERRED,
                        pending=pend, workspace=ws, err=err)
    for l in layers:       # flush the second step's accepted tokens
        if l['kind'] == 'gdn':
            bd.gdn_verify_commit(sb, bd.SV_GDN_COMMIT_ONLY, l['state'], l['q'], l['k'], l['v'],
                                 l['alpha'], l['beta'], commits[1], l['out'])
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    say('  oracle: acceptance over all sequences')
    ref_acc, ref_out = _oracle_accept(acc, batch)
    _check_accept(results[0], ref_acc, ref_out, ctx0, commits[0], ctx1)
    # the same logits and uniforms in step 2: the same decisions
    _check_accept(results[1], ref_acc, ref_out, ctx0 + ref_acc + 1, commits[1], ctx)
    c = ref_acc + 1

    say('  oracle: sampled sequences', seqs)
    worst = {'att': 0.0, 'gdn_o': 0.0, 'gdn_s': 0.0}
    for i, l in enumerate(layers):
        for b in seqs:
            s = snap[i][b]
            T = int(cu[b + 1] - cu[b])
            if l['kind'] == 'attn':
                o1, K1, V1 = _attn_oracle(s, int(ctx0[b]), T, batch.P)
                worst['att'] = max(worst['att'], check_attn_out(out1[i][b], o1, torch.bfloat16))
                assert np.array_equal(pages1[i][b][0], _bits_as(K1, l['k_cache']))
                assert np.array_equal(pages1[i][b][1], _bits_as(V1, l['v_cache']))
                s2 = dict(s, K=K1, V=V1)
                o2, K2, V2 = _attn_oracle(s2, int(ctx0[b] + c[b]), T, batch.P)
                r = slice(cu[b], cu[b + 1])
                worst['att'] = max(worst['att'],
                                   check_attn_out(np64(l['out'][r]), o2, torch.bfloat16))
                pg = torch.from_numpy(_seq_pages(batch, b)).to(DEV)
                assert np.array_equal(bits(l['k_cache'][pg]), _bits_as(K2, l['k_cache']))
                assert np.array_equal(bits(l['v_cache'][pg]), _bits_as(V2, l['v_cache']))
            else:
                args1 = (s['q'], s['k'], s['v'], s['alpha'], s['beta'], np.array([0, T]))
                o1, S1 = oracle.gdn_step(s['S'], None, *args1, np.array([c[b]]),
                                         oracle.GDN_VERIFY_COMMIT)
                o2, S2 = oracle.gdn_step(S1, None, *args1, np.array([c[b]]),
                                         oracle.GDN_VERIFY_COMMIT)
                worst['gdn_o'] = max(worst['gdn_o'],
                                     check_gdn_out(out1[i][b], o1, torch.bfloat16))
                # the flush (commit only) writes no outputs: out holds step 2's
                r = slice(cu[b], cu[b + 1])
                worst['gdn_o'] = max(worst['gdn_o'],
                                     check_gdn_out(np64(l['out'][r]), o2, torch.bfloat16))
                worst['gdn_s'] = max(worst['gdn_s'],
                                     check_gdn_state(np64(l['state'][b:b + 1]), S2))
    say('  worst errors', worst)


def test_stress_ragged_long_two_phase_step():
    w = wl.WORKLOADS[4]
    batch = wl.make_batch(w, 12, DEV)
    say('stress step: B =', batch.B, 'pool pages', batch.num_pages)
    layers = _layers(w, batch, 1200)
    acc = wl.make_accept(w, batch, 1299, 'rejection', DEV)
    torch.cuda.synchronize()
    T_all = np.array(batch.T)
    seqs = sorted({0, batch.B - 1, int(np.argmax(batch.ctx)), int(np.argmin(batch.ctx)),
                   int(np.argmax(T_all)), int(np.argmin(T_all)), 77})
    snap = _snapshot(layers, batch, seqs)
    cu = npi(batch.cu_seqlens)
    ctx0 = npi(batch.ctx_lens)
    args = _step_args(w, batch, layers, acc)
    sb = sv_batch(batch)
    ws = torch.zeros(bd.spec_verify_step_workspace_bytes(sb, args), dtype=torch.uint8,
                     device=DEV)
    ctx = batch.ctx_lens.clone()
    err = err_word()
    result = torch.full((batch.B * (1 + batch.max_T),), -7, dtype=torch.int32, device=DEV)
    commit = torch.full((batch.B,), -7, dtype=torch.int32, device=DEV)
    say('  step (two-phase)')
    bd.spec_verify_step(sb, args, ctx, result, commit, schedule=bd.SV_SCHEDULE_TWO_PHASE,
                        workspace=ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    say('  oracle: acceptance over all sequences')
    ref_acc, ref_out = _oracle_accept(acc, batch)
    _check_accept(result, ref_acc, ref_out, ctx0, commit, ctx)
    c = ref_acc + 1
    say('  oracle: sampled sequences', seqs)
    for i, l in enumerate(layers):
        for b in seqs:
            s = snap[i][b]
            T = int(cu[b + 1] - cu[b])
            r = slice(cu[b], cu[b + 1])
            if l['kind'] == 'attn':
                o, K1, V1 = _attn_oracle(s, int(ctx0[b]), T, batch.P)
                check_attn_out(np64(l['out'][r]), o, torch.bfloat16)
                pg = torch.from_numpy(_seq_pages(batch, b)).to(DEV)
                assert np.array_equal(bits(l['k_cache'][pg]), _bits_as(K1, l['k_cache']))
                assert np.array_equal(bits(l['v_cache'][pg]), _bits_as(V1, l['v_cache']))
            else:
                o, S1 = oracle.gdn_step(s['S'], None, s['q'], s['k'], s['v'], s['alpha'],
                                        s['beta'], np.array([0, T]), np.array([c[b]]),
                                        oracle.GDN_VERIFY_COMMIT)
                check_gdn_out(np64(l['out'][r]), o, torch.bfloat16)
                check_gdn_state(np64(l['state'][b:b + 1]), S1)
