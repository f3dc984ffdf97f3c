"""GPU parity of spec_verify_step (the whole step) against the oracle.

Same tolerances as the per-op tests; acceptance, commit lengths, ctx_lens and
the KV pools are bit-exact.  The deferred schedule must leave exactly the
states of the two-phase schedule (bit for bit) once flushed.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import (DEV, GDN_STATE_TOL, GDN_STATE_TOL_F16, bits, check_attn_out,
                         check_gdn_out, check_gdn_state, err_word, np64, npi, say, sv_batch)

pytestmark = pytest.mark.gpu


def make_step(w, batch, seed, mode, state_dtype=torch.float32):
    layers = []
    for i, kind in enumerate(w.layers):
        if kind == 'attn':
            lay = wl.make_attn_layer(w, batch, seed + 10 * i, DEV)
            lay['out'] = torch.full_like(lay['q'], float('nan'))
        else:
            lay = wl.make_gdn_layer(w, batch, seed + 10 * i, DEV, state_dtype=state_dtype)
            lay['out'] = torch.full_like(lay['v'], float('nan'))
        lay['kind'] = kind
        layers.append(lay)
    acc = wl.make_accept(w, batch, seed + 999, mode, DEV)
    return layers, acc


def run_step(w, batch, layers, acc, mode, schedule=bd.SV_SCHEDULE_TWO_PHASE, pending=None,
             ctx=None, commit_fill=-7):
    dt_a = bd.SV_BF16 if w.attn_dtype == torch.bfloat16 else bd.SV_F32
    dt_g = bd.SV_BF16 if w.gdn_dtype == torch.bfloat16 else bd.SV_F32
    a_layers = [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'],
                              l['out']) for l in layers if l['kind'] == 'attn']
    g_layers = [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'],
                             l['out']) for l in layers if l['kind'] == 'gdn']
    dt_s = next((bd.state_dtype(l['state']) for l in layers if l['kind'] == 'gdn'), bd.SV_F32)
    args = bd.StepArgs([1 if l['kind'] == 'attn' else 0 for l in layers],
                       bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages,
                                      batch.block_table, dt_a),
                       a_layers, bd.gdn_config(w.H, w.dk, w.dv, batch.B, dt_g,
                                               state_dtype=dt_s), g_layers,
                       bd.accept_args(mode, acc['target_logits'], acc['draft_tokens'],
                                      acc.get('draft_logits'), acc.get('u_accept'),
                                      acc.get('u_final')))
    sb = sv_batch(batch)
    ws = torch.zeros(max(1, bd.spec_verify_step_workspace_bytes(sb, args)), dtype=torch.uint8,
                     device=DEV)
    result = torch.full((batch.B * (1 + batch.max_T),), -7, dtype=torch.int32, device=DEV)
    commit = torch.full((batch.B,), commit_fill, dtype=torch.int32, device=DEV)
    ctx = (batch.ctx_lens if ctx is None else ctx).clone()
    err = err_word()
    bd.spec_verify_step(sb, args, ctx, result, commit, schedule=schedule, pending=pending,
                        workspace=ws, err=err)
    torch.cuda.synchronize()
    r = npi(result)
    return dict(acc=r[:batch.B], out=r[batch.B:].reshape(batch.B, batch.max_T),
                commit=commit, ctx=ctx, err=int(err.item()), args=args)


def oracle_step(w, batch, layers, acc, mode, ctx=None):
    lays = []
    for l in layers:
        if l['kind'] == 'attn':
            lays.append({'kind': 'attn', 'q': np64(l['q']), 'k_new': np64(l['k_new']),
                         'v_new': np64(l['v_new']), 'k_cache': np64(l['k_cache']),
                         'v_cache': np64(l['v_cache'])})
        else:
            lays.append({'kind': 'gdn', 'state': np64(l['state']), 'q': np64(l['q']),
                         'k': np64(l['k']), 'v': np64(l['v']), 'alpha': np64(l['alpha']),
                         'beta': np64(l['beta'])})
    ai = {'target_logits': np64(acc['target_logits']), 'draft_tokens': npi(acc['draft_tokens'])}
    if mode == bd.SV_ACCEPT_REJECTION:
        ai.update(draft_logits=np64(acc['draft_logits']), u_accept=np64(acc['u_accept']),
                  u_final=np64(acc['u_final']))
    return oracle.verify_step(lays, npi(batch.cu_seqlens),
                              npi(batch.ctx_lens) if ctx is None else ctx,
                              npi(batch.block_table), batch.P, batch.max_T,
                              'greedy' if mode == bd.SV_ACCEPT_GREEDY else 'rejection', ai)


def compare(w, layers, res, ref, before):
    assert res['err'] == 0
    np.testing.assert_array_equal(res['acc'], ref['accept_len'])
    np.testing.assert_array_equal(res['out'], ref['out_tokens'])
    np.testing.assert_array_equal(npi(res['commit']), ref['commit_len'])
    np.testing.assert_array_equal(npi(res['ctx']), ref['ctx_lens'])
    for i, l in enumerate(layers):
        if l['kind'] == 'attn':
            check_attn_out(np64(l['out']), ref['outputs'][i], w.attn_dtype)
            # pools: compare the bit patterns the oracle's append produced
            assert np.array_equal(bits(l['k_cache']), bits_of(ref['k_cache'][i], before[i][0]))
            assert np.array_equal(bits(l['v_cache']), bits_of(ref['v_cache'][i], before[i][1]))
        else:
            check_gdn_out(np64(l['out']), ref['outputs'][i], w.gdn_dtype)
            check_gdn_state(np64(l['state']), ref['state'][i])


def bits_of(values64, like):
    t = torch.from_numpy(values64).to(like.dtype)
    return bits(t)


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
def test_tiny_fp32_step(mode):
    w = wl.WORKLOADS[0]
    batch = wl.make_batch(w, 0, DEV)
    layers, acc = make_step(w, batch, 1, 'greedy' if mode == 0 else 'rejection')
    ref = oracle_step(w, batch, layers, acc, mode)
    before = [(l.get('k_cache'), l.get('v_cache')) for l in layers]
    for l in layers:
        if l['kind'] == 'attn':
            l['k_cache'] = l['k_cache'].clone()
            l['v_cache'] = l['v_cache'].clone()
        else:
            l['state'] = l['state'].clone()
    say('tiny step mode', mode)
    res = run_step(w, batch, layers, acc, mode)
    compare(w, layers, res, ref, before)


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
def test_hybrid_group_step(mode):
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(1)})
    batch = wl.make_batch(w, 5, DEV)
    layers, acc = make_step(w, batch, 6, 'greedy' if mode == 0 else 'rejection')
    ref = oracle_step(w, batch, layers, acc, mode)
    before = [(l.get('k_cache'), l.get('v_cache')) for l in layers]
    for l in layers:
        if l['kind'] == 'attn':
            l['k_cache'] = l['k_cache'].clone()
            l['v_cache'] = l['v_cache'].clone()
        else:
            l['state'] = l['state'].clone()
    say('hybrid group step mode', mode)
    res = run_step(w, batch, layers, acc, mode)
    compare(w, layers, res, ref, before)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.float16])
def test_deferred_schedule_equals_two_phase(state_dtype):
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(1)})
    batch = wl.make_batch(w, 7, DEV, reserve=8)
    l1, a1 = make_step(w, batch, 8, 'rejection', state_dtype)
    l2, a2 = make_step(w, batch, 9, 'rejection', state_dtype)
    tol = GDN_STATE_TOL if state_dtype == torch.float32 else 2 * GDN_STATE_TOL_F16
    init = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in l.items()}
            for l in l1]

    def fresh(src, states_from, pools_from):
        out = []
        for s, st, pl in zip(src, states_from, pools_from):
            d = dict(s)
            d['out'] = torch.full_like(s['out'], float('nan'))
            if s['kind'] == 'gdn':
                d['state'] = st['state']
            else:
                d['k_cache'], d['v_cache'] = pl['k_cache'], pl['v_cache']
            out.append(d)
        return out

    results = {}
    for sched in (bd.SV_SCHEDULE_TWO_PHASE, bd.SV_SCHEDULE_DEFERRED):
        st = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in l.items()}
              for l in init]
        s1 = fresh(l1, st, st)
        r1 = run_step(w, batch, s1, a1, bd.SV_ACCEPT_REJECTION, schedule=sched)
        s2 = fresh(l2, s1, s1)
        pend = None
        if sched == bd.SV_SCHEDULE_DEFERRED:
            pl = [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'],
                               l['out']) for l in s1 if l['kind'] == 'gdn']
            arr = (bd.SvGdnLayer * len(pl))(*pl)
            pend = bd.SvStepPending(sv_batch(batch), arr, r1['commit'].data_ptr())
        r2 = run_step(w, batch, s2, a2, bd.SV_ACCEPT_REJECTION, schedule=sched, pending=pend,
                      ctx=r1['ctx'])
        assert r1['err'] == 0 and r2['err'] == 0
        if sched == bd.SV_SCHEDULE_DEFERRED:
            for l in s2:     # flush the second step's accepted tokens
                if l['kind'] == 'gdn':
                    bd.gdn_verify_commit(sv_batch(batch), bd.SV_GDN_COMMIT_ONLY, l['state'],
                                         l['q'], l['k'], l['v'], l['alpha'], l['beta'],
                                         r2['commit'], l['out'])
            torch.cuda.synchronize()
        results[sched] = (r1, r2, s2)
    (t1, t2, ts), (d1, d2, ds) = results[0], results[1]
    np.testing.assert_array_equal(t1['out'], d1['out'])
    np.testing.assert_array_equal(t2['out'], d2['out'])
    for a, b in zip(ts, ds):
        assert torch.equal(a['out'], b['out'])
        if a['kind'] == 'gdn':
            assert torch.equal(a['state'], b['state'])
        else:
            assert torch.equal(a['k_cache'], b['k_cache'])
    # and against the oracle: two steps in a row
    ref1 = oracle_step(w, batch, [dict(l, **({'state': i['state']} if l['kind'] == 'gdn' else
                                            {'k_cache': i['k_cache'], 'v_cache': i['v_cache']}))
                                  for l, i in zip(l1, init)], a1, bd.SV_ACCEPT_REJECTION)
    np.testing.assert_array_equal(t1['out'], ref1['out_tokens'])
    for i, l in enumerate(ts):
        if l['kind'] == 'gdn':
            s_mid = ref1['state'][i]
            _, S2 = oracle.gdn_step(s_mid, None, None, np64(l['k']), np64(l['v']),
                                    np64(l['alpha']), np64(l['beta']), npi(batch.cu_seqlens),
                                    npi(t2['commit']), oracle.GDN_COMMIT_ONLY)
            check_gdn_state(np64(l['state']), S2, tol=tol)


def test_step_with_int8_kv_pages():
    """The step's attention layers over INT8 pages (kv_format = SV_KV_INT8):
    acceptance, commit lengths and ctx_lens bit-exact, attention outputs and
    written codes against the INT8 oracle, GDN outputs and committed states
    against the GDN oracle (two-phase schedule)."""
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(1)})
    batch = wl.make_batch(w, 17, DEV)
    layers = []
    for i, kind in enumerate(w.layers):
        if kind == 'attn':
            lay = wl.make_attn_layer_kv8(w, batch, 1700 + 10 * i, DEV)
            lay['out'] = torch.full_like(lay['q'], float('nan'))
        else:
            lay = wl.make_gdn_layer(w, batch, 1700 + 10 * i, DEV)
            lay['out'] = torch.full_like(lay['v'], float('nan'))
        lay['kind'] = kind
        layers.append(lay)
    acc = wl.make_accept(w, batch, 1799, 'rejection', DEV)
    before = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in l.items()}
              for l in layers]
    args = bd.StepArgs(
        [1 if l['kind'] == 'attn' else 0 for l in layers],
        bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table,
                       bd.SV_BF16, kv_format=bd.SV_KV_INT8),
        [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'], l['out'],
                       l['k_scale'], l['v_scale']) for l in layers if l['kind'] == 'attn'],
        bd.gdn_config(w.H, w.dk, w.dv, batch.B, bd.SV_BF16),
        [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'], l['out'])
         for l in layers if l['kind'] == 'gdn'],
        bd.accept_args(bd.SV_ACCEPT_REJECTION, acc['target_logits'], acc['draft_tokens'],
                       acc['draft_logits'], acc['u_accept'], acc['u_final']))
    sb = sv_batch(batch)
    ws = torch.zeros(bd.spec_verify_step_workspace_bytes(sb, args), dtype=torch.uint8, device=DEV)
    result = torch.full((batch.B * (1 + batch.max_T),), -7, dtype=torch.int32, device=DEV)
    commit = torch.full((batch.B,), -7, dtype=torch.int32, device=DEV)
    ctx = batch.ctx_lens.clone()
    err = err_word()
    say('step with INT8 KV pages')
    bd.spec_verify_step(sb, args, ctx, result, commit, workspace=ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    a_ref, o_ref = oracle.rejection_accept(np64(acc['target_logits']), np64(acc['draft_logits']),
                                           npi(acc['draft_tokens']), np64(acc['u_accept']),
                                           np64(acc['u_final']), npi(batch.cu_seqlens),
                                           batch.max_T)
    r = npi(result)
    np.testing.assert_array_equal(r[:batch.B], a_ref)
    np.testing.assert_array_equal(r[batch.B:].reshape(batch.B, -1), o_ref)
    np.testing.assert_array_equal(npi(commit), a_ref + 1)
    np.testing.assert_array_equal(npi(ctx), npi(batch.ctx_lens) + a_ref + 1)
    cu, table, ctx0 = npi(batch.cu_seqlens), npi(batch.block_table), npi(batch.ctx_lens)
    for l, b0 in zip(layers, before):
        if l['kind'] == 'attn':
            ks, vs = b0['k_scale'].cpu().numpy(), b0['v_scale'].cpu().numpy()
            ref = oracle.verify_attention_int8(
                np64(b0['q']), b0['k_new'].float().cpu().numpy(),
                b0['v_new'].float().cpu().numpy(), b0['k_cache'].cpu().numpy(),
                b0['v_cache'].cpu().numpy(), ks, vs, table, ctx0, cu, batch.P)
            check_attn_out(np64(l['out']), ref, torch.bfloat16)
            k_exp, v_exp = oracle.append_kv_int8(
                b0['k_cache'].cpu().numpy(), b0['v_cache'].cpu().numpy(),
                b0['k_new'].float().cpu().numpy(), b0['v_new'].float().cpu().numpy(), ks, vs,
                table, ctx0, cu, batch.P)
            assert np.array_equal(l['k_cache'].cpu().numpy(), k_exp)
            assert np.array_equal(l['v_cache'].cpu().numpy(), v_exp)
        else:
            o, _ = oracle.gdn_step(np64(b0['state']), None, np64(b0['q']), np64(b0['k']),
                                   np64(b0['v']), np64(b0['alpha']), np64(b0['beta']), cu, None,
                                   oracle.GDN_VERIFY_ONLY)
            check_gdn_out(np64(l['out']), o, torch.bfloat16)
            _, S = oracle.gdn_step(np64(b0['state']), None, None, np64(b0['k']), np64(b0['v']),
                                   np64(b0['alpha']), np64(b0['beta']), cu, a_ref + 1,
                                   oracle.GDN_COMMIT_ONLY)
            check_gdn_state(np64(l['state']), S)


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
def test_out_of_vocabulary_draft_skips_the_sequence(mode):
    """A draft id outside the vocabulary flags SV_DERR_TOKEN and skips its
    sequence: accept_len -1, a row of -1, commit length 0 (over a commit
    buffer that held a valid length from an earlier step), ctx_lens kept, so
    the batched two-phase commit and a later deferred flush leave its GDN
    states bit for bit.  Every other sequence matches the oracle."""
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(1)})
    batch = wl.make_batch(w, 25, DEV)
    name = 'greedy' if mode == bd.SV_ACCEPT_GREEDY else 'rejection'
    layers, acc = make_step(w, batch, 26, name)
    bad_b = 3
    cu = npi(batch.cu_seqlens)
    good_drafts = acc['draft_tokens'].clone()
    acc['draft_tokens'][cu[bad_b] - bad_b + 1] = w.V + 5       # its second draft
    ref = oracle_step(w, batch, layers, dict(acc, draft_tokens=good_drafts), mode)
    before = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in l.items()}
              for l in layers]
    say('out-of-vocabulary draft, mode', name)
    res = run_step(w, batch, layers, acc, mode, commit_fill=2)
    assert res['err'] == 16, res['err']                          # SV_DERR_TOKEN
    others = [b for b in range(batch.B) if b != bad_b]
    assert res['acc'][bad_b] == -1 and (res['out'][bad_b] == -1).all()
    assert int(res['commit'][bad_b]) == 0
    assert int(res['ctx'][bad_b]) == batch.ctx[bad_b]
    np.testing.assert_array_equal(res['acc'][others], ref['accept_len'][others])
    np.testing.assert_array_equal(res['out'][others], ref['out_tokens'][others])
    np.testing.assert_array_equal(npi(res['commit'])[others], ref['commit_len'][others])
    np.testing.assert_array_equal(npi(res['ctx'])[others], ref['ctx_lens'][others])
    for i, (l, b0) in enumerate(zip(layers, before)):
        if l['kind'] == 'gdn':
            assert torch.equal(l['state'][bad_b], b0['state'][bad_b])
            S_ref = ref['state'][i]
            check_gdn_state(np64(l['state'][others]), S_ref[others])
            # a deferred flush with this commit buffer keeps it too
            st = l['state'].clone()
            bd.gdn_verify_commit(sv_batch(batch), bd.SV_GDN_COMMIT_ONLY, st, l['q'], l['k'],
                                 l['v'], l['alpha'], l['beta'], res['commit'], l['out'])
            torch.cuda.synchronize()
            assert torch.equal(st[bad_b], b0['state'][bad_b])


def test_refused_step_changes_nothing():
    """A step whose last GDN layer is refused on the host (misaligned q)
    returns the error before any launch: no page, state, length, pending
    replay or output has changed, so a retry after the fix replays the
    pending tokens exactly once."""
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(2)})
    batch = wl.make_batch(w, 27, DEV, reserve=8)
    layers, acc = make_step(w, batch, 28, 'rejection')
    gdn = [l for l in layers if l['kind'] == 'gdn']
    commit_prev = wl.make_commit_len(batch, 29, device=DEV)
    pl = [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'], l['out'])
          for l in gdn]
    arr = (bd.SvGdnLayer * len(pl))(*pl)
    pend = bd.SvStepPending(sv_batch(batch), arr, commit_prev.data_ptr())
    before = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in l.items()}
              for l in layers]
    # the last GDN layer's q, shifted by one bf16 element: not 16-byte aligned
    q_bad = torch.empty(gdn[-1]['q'].numel() + 8, dtype=gdn[-1]['q'].dtype, device=DEV)
    good_q = gdn[-1]['q']
    gdn[-1]['q'] = q_bad[1:1 + good_q.numel()].view(good_q.shape)
    ctx = batch.ctx_lens.clone()
    with pytest.raises(bd.SpecVerifyError) as ei:
        run_step(w, batch, layers, acc, bd.SV_ACCEPT_REJECTION,
                 schedule=bd.SV_SCHEDULE_DEFERRED, pending=pend, ctx=ctx)
    assert 'aligned' in str(ei.value)
    torch.cuda.synchronize()
    for l, b0 in zip(layers, before):
        for key in ('state', 'k_cache', 'v_cache', 'out'):
            if key in l:
                assert torch.equal(l[key], b0[key]) or (
                    key == 'out' and torch.isnan(l[key].float()).all()), key
    assert torch.equal(ctx, batch.ctx_lens)


def _conv_step_args(w, batch, layers, convs, acc, mode, K, act):
    """StepArgs whose GDN layers carry their short convolution."""
    g_layers = []
    gi = 0
    for l in layers:
        if l['kind'] == 'gdn':
            g_layers.append(bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'],
                                         l['beta'], l['out'], conv=convs[gi]))
            gi += 1
    return bd.StepArgs(
        [1 if l['kind'] == 'attn' else 0 for l in layers],
        bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table,
                       bd.SV_BF16),
        [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'], l['out'])
         for l in layers if l['kind'] == 'attn'],
        bd.gdn_config(w.H, w.dk, w.dv, batch.B, bd.SV_BF16, conv_C=w.conv_C, conv_K=K,
                      conv_activation=act), g_layers,
        bd.accept_args(mode, acc['target_logits'], acc['draft_tokens'],
                       acc.get('draft_logits'), acc.get('u_accept'), acc.get('u_final')))


@pytest.mark.parametrize("K,act", [(4, bd.SV_ACT_SILU), (3, bd.SV_ACT_NONE)])
@pytest.mark.parametrize("schedule", [bd.SV_SCHEDULE_TWO_PHASE, bd.SV_SCHEDULE_DEFERRED])
def test_step_with_short_conv(schedule, K, act):
    """Every GDN layer's short convolution inside the step (one launch with
    the GDN verify; two-phase: committed in the batched commit launch;
    deferred: the next step replays its pending inputs).  Two steps, then a
    flush; conv outputs against oracle.conv_step (bf16 tolerance), committed
    conv states bit for bit, GDN states, outputs and acceptance as usual."""
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(1), 'conv_K': K, 'H': 4})
    batch = wl.make_batch(w, 31, DEV, reserve=8)
    mode = bd.SV_ACCEPT_REJECTION
    layers, acc = make_step(w, batch, 32, 'rejection')
    convs = []
    for i in range(sum(1 for l in layers if l['kind'] == 'gdn')):
        c = wl.make_conv_layer(w, batch, 3300 + i, DEV)
        c['out'] = torch.full_like(c['x'], float('nan'))
        convs.append(c)
    init_state = [l['state'].clone() if l['kind'] == 'gdn' else None for l in layers]
    init_conv = [c['state'].clone() for c in convs]
    pools = [(l['k_cache'].clone(), l['v_cache'].clone()) if l['kind'] == 'attn' else None
             for l in layers]
    args = _conv_step_args(w, batch, layers, convs, acc, mode, K, act)
    sb = sv_batch(batch)
    ws = torch.zeros(bd.spec_verify_step_workspace_bytes(sb, args), dtype=torch.uint8,
                     device=DEV)
    ctx = batch.ctx_lens.clone()
    err = err_word()
    results = [torch.full((batch.B * (1 + batch.max_T),), -7, dtype=torch.int32, device=DEV)
               for _ in range(2)]
    commits = [torch.full((batch.B,), -7, dtype=torch.int32, device=DEV) for _ in range(2)]
    say('step with short conv, schedule', schedule, 'K', K)
    bd.spec_verify_step(sb, args, ctx, results[0], commits[0], schedule=schedule,
                        workspace=ws, err=err)
    torch.cuda.synchronize()
    conv_out1 = [c['out'].clone() for c in convs]
    pend = None
    pend_arr = (bd.SvGdnLayer * len(args.gdn))(*args.gdn)
    if schedule == bd.SV_SCHEDULE_DEFERRED:
        pend = bd.SvStepPending(sb, pend_arr, commits[0].data_ptr())
    bd.spec_verify_step(sb, args, ctx, results[1], commits[1], schedule=schedule,
                        pending=pend, workspace=ws, err=err)
    if schedule == bd.SV_SCHEDULE_DEFERRED:     # flush the second step's tokens
        gi = 0
        for l in layers:
            if l['kind'] == 'gdn':
                bd.gdn_verify_commit(sb, bd.SV_GDN_COMMIT_ONLY, l['state'], l['q'], l['k'],
                                     l['v'], l['alpha'], l['beta'], commits[1], l['out'])
                c = convs[gi]
                bd.short_conv_verify_commit(sb, bd.SV_GDN_COMMIT_ONLY, c['state'], c['x'],
                                            c['weight'], c['bias'], commits[1], c['out'],
                                            activation=act)
                gi += 1
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    cu = npi(batch.cu_seqlens)
    a_ref, o_ref = oracle.rejection_accept(np64(acc['target_logits']), np64(acc['draft_logits']),
                                           npi(acc['draft_tokens']), np64(acc['u_accept']),
                                           np64(acc['u_final']), cu, batch.max_T)
    r = npi(results[0])
    np.testing.assert_array_equal(r[:batch.B], a_ref)
    np.testing.assert_array_equal(npi(commits[0]), a_ref + 1)
    np.testing.assert_array_equal(npi(commits[1]), a_ref + 1)
    c1 = a_ref + 1
    silu = act == bd.SV_ACT_SILU
    gi = 0
    for i, l in enumerate(layers):
        if l['kind'] != 'gdn':
            continue
        cv = convs[gi]
        xs, wt, bs = np64(cv['x']), np64(cv['weight']), np64(cv['bias'])
        y1, S1 = oracle.conv_step(np64(init_conv[gi]), None, xs, wt, bs, cu, c1,
                                  oracle.CONV_VERIFY_COMMIT, silu=silu)
        y2, S2 = oracle.conv_step(S1, None, xs, wt, bs, cu, c1, oracle.CONV_VERIFY_COMMIT,
                                  silu=silu)
        check_gdn_out(np64(conv_out1[gi]), y1, torch.bfloat16)
        check_gdn_out(np64(cv['out']), y2, torch.bfloat16)
        assert np.array_equal(bits(cv['state']), bits_of(S2, cv['state']))
        # the GDN state beside it: two commits of c1 tokens
        _, G1 = oracle.gdn_step(np64(init_state[i]), None, None, np64(l['k']), np64(l['v']),
                                np64(l['alpha']), np64(l['beta']), cu, c1,
                                oracle.GDN_COMMIT_ONLY)
        _, G2 = oracle.gdn_step(G1, None, None, np64(l['k']), np64(l['v']), np64(l['alpha']),
                                np64(l['beta']), cu, c1, oracle.GDN_COMMIT_ONLY)
        check_gdn_state(np64(l['state']), G2)
        gi += 1
    for i, l in enumerate(layers):       # the attention layers are untouched by the conv
        if l['kind'] == 'attn':
            ref = oracle.verify_attention(np64(l['q']), np64(l['k_new']), np64(l['v_new']),
                                          *oracle.append_kv(np64(pools[i][0]), np64(pools[i][1]),
                                                            np64(l['k_new']), np64(l['v_new']),
                                                            npi(batch.block_table),
                                                            npi(batch.ctx_lens), cu, batch.P),
                                          npi(batch.block_table), npi(batch.ctx_lens) + c1, cu,
                                          batch.P)
            check_attn_out(np64(l['out']), ref, torch.bfloat16)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.float16])
def test_flush_equals_per_layer_commits_and_two_phase(state_dtype):
    """spec_verify_flush after a deferred step stores, bit for bit, what
    per-layer COMMIT_ONLY calls on the same pending tokens store, and what the
    two-phase step stores, for the GDN states and the short-convolution
    windows (slot map, fp32 or fp16 state bank)."""
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(1), 'H': 4})
    batch = wl.make_batch(w, 41, DEV)
    ns = batch.B + 3
    slots = wl.make_state_slots(batch, ns, 42, DEV)
    layers = []
    for i, kind in enumerate(w.layers):
        if kind == 'attn':
            lay = wl.make_attn_layer(w, batch, 4300 + 10 * i, DEV)
            lay['out'] = torch.full_like(lay['q'], float('nan'))
        else:
            lay = wl.make_gdn_layer(w, batch, 4300 + 10 * i, DEV, num_slots=ns,
                                    state_dtype=state_dtype)
            lay['out'] = torch.full_like(lay['v'], float('nan'))
            c = wl.make_conv_layer(w, batch, 4350 + 10 * i, DEV, num_slots=ns)
            c['out'] = torch.full_like(c['x'], float('nan'))
            lay['conv'] = c
        lay['kind'] = kind
        layers.append(lay)
    acc = wl.make_accept(w, batch, 4399, 'rejection', DEV)
    gdn = [l for l in layers if l['kind'] == 'gdn']
    init = [(l['state'].clone(), l['conv']['state'].clone()) for l in gdn]
    pools = [(l['k_cache'].clone(), l['v_cache'].clone()) for l in layers if l['kind'] == 'attn']
    args = bd.StepArgs(
        [1 if l['kind'] == 'attn' else 0 for l in layers],
        bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table,
                       bd.SV_BF16),
        [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'], l['out'])
         for l in layers if l['kind'] == 'attn'],
        bd.gdn_config(w.H, w.dk, w.dv, ns, bd.SV_BF16, state_slot=slots,
                      state_dtype=bd.state_dtype(gdn[0]['state']), conv_C=w.conv_C,
                      conv_K=w.conv_K, conv_activation=bd.SV_ACT_SILU),
        [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'], l['out'],
                      conv=l['conv']) for l in gdn],
        bd.accept_args(bd.SV_ACCEPT_REJECTION, acc['target_logits'], acc['draft_tokens'],
                       acc['draft_logits'], acc['u_accept'], acc['u_final']))
    sb = sv_batch(batch)
    ws = torch.zeros(bd.spec_verify_step_workspace_bytes(sb, args), dtype=torch.uint8,
                     device=DEV)
    err = err_word()

    def step(schedule):
        for l, (s0, c0) in zip(gdn, init):
            l['state'].copy_(s0)
            l['conv']['state'].copy_(c0)
        ai = 0
        for l in layers:
            if l['kind'] == 'attn':
                l['k_cache'].copy_(pools[ai][0])
                l['v_cache'].copy_(pools[ai][1])
                ai += 1
        result = torch.full((batch.B * (1 + batch.max_T),), -7, dtype=torch.int32, device=DEV)
        commit = torch.full((batch.B,), -7, dtype=torch.int32, device=DEV)
        ctx = batch.ctx_lens.clone()
        bd.spec_verify_step(sb, args, ctx, result, commit, schedule=schedule, workspace=ws,
                            err=err)
        return commit

    say('flush: deferred step, then spec_verify_flush')
    commit = step(bd.SV_SCHEDULE_DEFERRED)
    torch.cuda.synchronize()
    for l, (s0, c0) in zip(gdn, init):   # the deferred step stores nothing
        assert torch.equal(l['state'], s0) and torch.equal(l['conv']['state'], c0)
    bd.spec_verify_flush(args, bd.step_pending(sb, args, commit), err=err)
    torch.cuda.synchronize()
    flushed = [(l['state'].clone(), l['conv']['state'].clone()) for l in gdn]

    say('flush: the same step, then per-layer COMMIT_ONLY calls')
    commit2 = step(bd.SV_SCHEDULE_DEFERRED)
    for l in gdn:
        bd.gdn_verify_commit(sb, bd.SV_GDN_COMMIT_ONLY, l['state'], l['q'], l['k'], l['v'],
                             l['alpha'], l['beta'], commit2, l['out'], state_slot=slots)
        c = l['conv']
        bd.short_conv_verify_commit(sb, bd.SV_GDN_COMMIT_ONLY, c['state'], c['x'], c['weight'],
                                    c['bias'], commit2, c['out'], state_slot=slots,
                                    activation=bd.SV_ACT_SILU)
    torch.cuda.synchronize()
    assert torch.equal(commit, commit2)
    for l, (s1, c1) in zip(gdn, flushed):
        assert torch.equal(l['state'], s1)
        assert torch.equal(l['conv']['state'], c1)

    say('flush: the two-phase step')
    step(bd.SV_SCHEDULE_TWO_PHASE)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for l, (s1, c1) in zip(gdn, flushed):
        assert torch.equal(l['state'], s1)
        assert torch.equal(l['conv']['state'], c1)
    # and against the oracle (one commit of the accepted prefix)
    cu = npi(batch.cu_seqlens)
    for l, (s0, c0), (s1, c1) in zip(gdn, init, flushed):
        _, S = oracle.gdn_step(np64(s0), npi(slots), None, np64(l['k']), np64(l['v']),
                               np64(l['alpha']), np64(l['beta']), cu, npi(commit),
                               oracle.GDN_COMMIT_ONLY)
        check_gdn_state(np64(s1), S, tol=GDN_STATE_TOL if state_dtype == torch.float32
                        else GDN_STATE_TOL_F16)
        _, CS = oracle.conv_step(np64(c0), npi(slots), np64(l['conv']['x']),
                                 np64(l['conv']['weight']), np64(l['conv']['bias']), cu,
                                 npi(commit), oracle.CONV_COMMIT_ONLY)
        assert np.array_equal(bits(c1), bits_of(CS, c1))
