"""GPU parity at full size, in the launch configuration the benchmark times,
for EVERY sequence of EVERY layer.

hybrid_step_64l: two consecutive verify steps of the 64-layer hybrid stack
(B = 64, k = 3, contexts U[2048, 8192], 48 GDN + 16 attention layers,
rejection acceptance over V = 151936, deferred schedule: the second step
replays the first step's accepted GDN tokens before verifying its own), then
a flush of the second step's accepted tokens.

stress_ragged_long: one two-phase step (B = 256, k_b ~ U{1..7}, contexts
U[16384, 32768], fragmented pool, one GDN,GDN,GDN,ATT group).

Checked against the oracle, for all sequences: acceptance, commit lengths
and ctx_lens (bit-exact); every attention output (max-abs <= 1e-2 + half a
bf16 ulp, bf16 I/O); every KV page after each step (bit-exact: each sequence's pages
against the oracle's append, pages no sequence owns unchanged); every GDN
output (1e-2 + half a bf16 ulp) and every committed state tile (normwise
1e-4).  The oracle runs one sequence at a time (a sequence's result depends
on its own inputs only), its pages gathered into a private pool, on a pool
of host threads; its inputs are the generated tensors (never a result of
the library), and step 2 starts from the oracle's own step-1 pages and
states.
"""

import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import (ATT_TOL, DEV, GDN_OUT_TOL, GDN_STATE_TOL, bf16_half_ulp, err_word,
                         np64, npi, say, sv_batch)

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
SEQ_BATCH = 16      # sequences whose pages are on the host at once


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


def _f32(t):
    """Host float32 copy (bf16 widens exactly)."""
    return t.detach().float().cpu().numpy()


def _i32(a):
    return a.view(np.int32)


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


def _seq_pages(table, b):
    row = table[b]
    return row[row >= 0]


def check_attention_layer(batch, q, kn, vn, pool0, steps):
    """Every sequence of one attention layer over consecutive steps.

    pool0:  (K, V) GPU pools before the first step (generated inputs).
    steps:  list of (ctx_before, out_gpu, (K, V) GPU pools after the step);
            step s attends at ctx_before[s] and appends there.
    Returns the largest output error; asserts every page bit for bit.
    """
    cu, table = npi(batch.cu_seqlens), npi(batch.block_table)
    qh, knh, vnh = _f32(q), _f32(kn), _f32(vn)
    outs = [np64(o) for _, o, _ in steps]
    worst = [0.0]
    bad = []

    def one(task):
        b, K, V, got = task
        r = slice(cu[b], cu[b + 1])
        T = int(cu[b + 1] - cu[b])
        sub = np.arange(K.shape[0])[None, :]
        cu1 = np.array([0, T])
        for s, (ctx_s, _, _) in enumerate(steps):
            L = np.array([int(ctx_s[b])])
            o = oracle.verify_attention(qh[r], knh[r], vnh[r], K, V, sub, L, cu1, batch.P)
            e = float(np.abs(outs[s][r] - o).max())
            worst[0] = max(worst[0], e)
            if e > ATT_TOL[torch.bfloat16]:
                bad.append(f'seq {b} step {s}: output error {e:.3e}')
            K, V = oracle.append_kv(K, V, knh[r], vnh[r], sub, L, cu1, batch.P)
            if not (np.array_equal(_i32(K), _i32(got[s][0])) and
                    np.array_equal(_i32(V), _i32(got[s][1]))):
                bad.append(f'seq {b} step {s}: pages differ')

    # one BLAS thread per worker: the workers are the parallelism
    with threadpool_limits(1), cf.ThreadPoolExecutor(THREADS) as ex:
        for b0 in range(0, batch.B, SEQ_BATCH):
            tasks = []
            for b in range(b0, min(batch.B, b0 + SEQ_BATCH)):
                pg = torch.from_numpy(_seq_pages(table, b)).to(DEV)
                got = [(_f32(k[pg]), _f32(v[pg])) for _, _, (k, v) in steps]
                tasks.append((b, _f32(pool0[0][pg]), _f32(pool0[1][pg]), got))
            list(ex.map(one, tasks))
            assert not bad, bad[:8]
    # pages that no sequence owns are never written
    owned = np.zeros(pool0[0].shape[0], dtype=bool)
    owned[table[table >= 0]] = True
    free = torch.from_numpy(np.nonzero(~owned)[0]).to(DEV)
    if free.numel():
        for _, _, (k, v) in steps:
            assert torch.equal(k[free], pool0[0][free]) and torch.equal(v[free], pool0[1][free])
    return worst[0]


def check_gdn_layer(batch, lay, state0, commit, outs, state_final):
    """Every sequence of one GDN layer over len(outs) consecutive steps with
    the same token inputs, each committing `commit` tokens: outs[s] are the
    GPU outputs of step s, state_final the GPU state after the last commit.
    Returns (worst output error, worst state error)."""
    cu = npi(batch.cu_seqlens)
    S0 = np64(state0)
    q, k, v = np64(lay['q']), np64(lay['k']), np64(lay['v'])
    al, be = np64(lay['alpha']), np64(lay['beta'])
    got_o = [np64(o) for o in outs]
    got_S = np64(state_final)
    worst = [0.0, 0.0]
    bad = []

    def one(b):
        r = slice(cu[b], cu[b + 1])
        cu1 = np.array([0, cu[b + 1] - cu[b]])
        S = S0[b:b + 1]
        for s in range(len(outs)):
            o, S = oracle.gdn_step(S, None, q[r], k[r], v[r], al[r], be[r], cu1,
                                   np.array([commit[b]]), oracle.GDN_VERIFY_COMMIT)
            d = np.abs(got_o[s][r] - o)
            worst[0] = max(worst[0], float(d.max()))
            if (d > GDN_OUT_TOL[torch.bfloat16] + bf16_half_ulp(o)).any():
                bad.append(f'seq {b} step {s}: output error {float(d.max()):.3e}')
        for h in range(S.shape[1]):
            e = np.abs(got_S[b, h] - S[0, h]).max() / max(np.abs(S[0, h]).max(), 1e-30)
            worst[1] = max(worst[1], float(e))
            if e > GDN_STATE_TOL:
                bad.append(f'seq {b} head {h}: state error {e:.3e}')

    with threadpool_limits(1), cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(one, range(batch.B)))
    assert not bad, bad[:8]
    return worst


@pytest.fixture(scope='module')
def hybrid_run():
    """Two deferred steps of the 64-layer stack and the flush, on the GPU; the
    generated inputs are kept (GPU clones) for the oracle."""
    w = wl.WORKLOADS[3]
    batch = wl.make_batch(w, 11, DEV, reserve=2 * w.max_T)
    say('full hybrid step: generating 64 layers, B =', batch.B)
    layers = _layers(w, batch, 1100)
    acc = wl.make_accept(w, batch, 1999, 'rejection', DEV)
    init = [{k: l[k].clone() for k in ('k_cache', 'v_cache', 'state') if k in l}
            for l in layers]
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
    ctx1 = ctx.clone()
    out1 = [l['out'].clone() for l in layers]
    pools1 = [(l['k_cache'].clone(), l['v_cache'].clone()) if l['kind'] == 'attn' else None
              for l in layers]
    say('  step 2 (deferred, replays step 1), then the flush')
    pend_arr = (bd.SvGdnLayer * len(args.gdn))(*args.gdn)
    pend = bd.SvStepPending(sb, pend_arr, commits[0].data_ptr())
    for l in layers:
        l['out'].fill_(float('nan'))
    bd.spec_verify_step(sb, args, ctx, results[1], commits[1], schedule=bd.SV_SCHEDULE_DEFERRED,
                        pending=pend, workspace=ws, err=err)
    for l in layers:
        if l['kind'] == 'gdn':
            bd.gdn_verify_commit(sb, bd.SV_GDN_COMMIT_ONLY, l['state'], l['q'], l['k'], l['v'],
                                 l['alpha'], l['beta'], commits[1], l['out'])
    torch.cuda.synchronize()
    return dict(w=w, batch=batch, layers=layers, acc=acc, init=init, results=results,
                commits=commits, ctx1=ctx1, ctx=ctx, out1=out1, pools1=pools1,
                err=int(err.item()))


def test_hybrid_step_acceptance(hybrid_run):
    r = hybrid_run
    assert r['err'] == 0
    batch = r['batch']
    ref_acc, ref_out = _oracle_accept(r['acc'], batch)
    ctx0 = np.array(batch.ctx)
    _check_accept(r['results'][0], ref_acc, ref_out, ctx0, r['commits'][0], r['ctx1'])
    # the same logits and uniforms in step 2: the same decisions
    _check_accept(r['results'][1], ref_acc, ref_out, ctx0 + ref_acc + 1, r['commits'][1],
                  r['ctx'])
    say('  acceptance of all', batch.B, 'sequences, both steps: exact')


def test_hybrid_step_every_attention_layer(hybrid_run):
    r = hybrid_run
    batch = r['batch']
    c = npi(r['commits'][0])
    ctx0 = np.array(batch.ctx)
    worst = 0.0
    for i, l in enumerate(r['layers']):
        if l['kind'] != 'attn':
            continue
        pool0 = (r['init'][i]['k_cache'], r['init'][i]['v_cache'])
        steps = [(ctx0, r['out1'][i], r['pools1'][i]),
                 (ctx0 + c, l['out'], (l['k_cache'], l['v_cache']))]
        e = check_attention_layer(batch, l['q'], l['k_new'], l['v_new'], pool0, steps)
        worst = max(worst, e)
        say(f'  attention layer {i}: 2 steps x {batch.B} sequences, max err {e:.2e}, '
            'pages exact')
    say(f'  worst attention error {worst:.3e}')


def test_hybrid_step_every_gdn_layer(hybrid_run):
    r = hybrid_run
    batch = r['batch']
    c = npi(r['commits'][0])
    worst = [0.0, 0.0]
    for i, l in enumerate(r['layers']):
        if l['kind'] != 'gdn':
            continue
        e = check_gdn_layer(batch, l, r['init'][i]['state'], c, [r['out1'][i], l['out']],
                            l['state'])
        worst = [max(worst[0], e[0]), max(worst[1], e[1])]
        if i % 8 == 0:
            say(f'  GDN layer {i}: out err {e[0]:.2e}, state err {e[1]:.2e}')
    say(f'  worst GDN output error {worst[0]:.3e}, state error {worst[1]:.3e} '
        f'over 48 layers x {batch.B} sequences x 32 heads')


@pytest.fixture(scope='module')
def stress_run():
    w = wl.WORKLOADS[4]
    batch = wl.make_batch(w, 12, DEV)
    say('stress step: B =', batch.B, 'pool pages', batch.num_pages)
    layers = _layers(w, batch, 1200)
    acc = wl.make_accept(w, batch, 1299, 'rejection', DEV)
    init = [{k: l[k].clone() for k in ('k_cache', 'v_cache', 'state') if k in l}
            for l in layers]
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
    return dict(w=w, batch=batch, layers=layers, acc=acc, init=init, result=result,
                commit=commit, ctx=ctx, err=int(err.item()))


def test_stress_step_acceptance(stress_run):
    r = stress_run
    assert r['err'] == 0
    batch = r['batch']
    ref_acc, ref_out = _oracle_accept(r['acc'], batch)
    _check_accept(r['result'], ref_acc, ref_out, np.array(batch.ctx), r['commit'], r['ctx'])


def test_stress_step_every_layer(stress_run):
    r = stress_run
    batch = r['batch']
    c = npi(r['commit'])
    for i, l in enumerate(r['layers']):
        if l['kind'] == 'attn':
            pool0 = (r['init'][i]['k_cache'], r['init'][i]['v_cache'])
            e = check_attention_layer(batch, l['q'], l['k_new'], l['v_new'], pool0,
                                      [(np.array(batch.ctx), l['out'],
                                        (l['k_cache'], l['v_cache']))])
            say(f'  attention layer {i}: {batch.B} sequences, max err {e:.2e}, pages exact')
        else:
            e = check_gdn_layer(batch, l, r['init'][i]['state'], c, [l['out']], l['state'])
            say(f'  GDN layer {i}: out err {e[0]:.2e}, state err {e[1]:.2e}')
