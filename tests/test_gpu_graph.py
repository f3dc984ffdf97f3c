"""spec_verify_step captured into HIP graphs (torch.cuda.CUDAGraph on the
capture stream) and replayed: every replay must equal the eager step bit
for bit (same kernels, same inputs), with eager work and synchronisations
between the replays, and the replayed steps must match the oracle.

The step enqueues kernels only (no memset or copy nodes, nothing
allocated), which is what makes it capturable.  Deferred schedule: one graph
per commit buffer (step i reads the pending commit lengths step i - 1
wrote), replayed alternately, so the recurrent states advance exactly once
per replayed step; the flush of the last step's tokens (spec_verify_flush)
replayed from a graph equals the eager flush.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import DEV, check_gdn_state, err_word, np64, npi, say, sv_batch

pytestmark = pytest.mark.gpu


def _setup(seed, mode):
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(2)})
    batch = wl.make_batch(w, seed, DEV, reserve=8 * w.max_T)
    layers = []
    for i, kind in enumerate(w.layers):
        lay = (wl.make_attn_layer if kind == 'attn' else wl.make_gdn_layer)(
            w, batch, seed + 10 * i, DEV)
        lay['out'] = torch.full_like(lay['q'] if kind == 'attn' else lay['v'], float('nan'))
        lay['kind'] = kind
        layers.append(lay)
    acc = wl.make_accept(w, batch, seed + 999, mode, DEV)
    return w, batch, layers, acc


class Runner:
    """One copy of every buffer the step writes, plus the step's arguments."""

    def __init__(self, w, batch, layers, acc, mode, schedule):
        self.layers = [{k: (v.clone() if isinstance(v, torch.Tensor) else v)
                        for k, v in l.items()} for l in layers]
        self.batch = batch
        self.sb = sv_batch(batch)
        L = self.layers
        amode = bd.SV_ACCEPT_GREEDY if mode == 'greedy' else bd.SV_ACCEPT_REJECTION
        self.gdn = [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'],
                                 l['out']) for l in L if l['kind'] == 'gdn']
        self.args = bd.StepArgs(
            [1 if l['kind'] == 'attn' else 0 for l in L],
            bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table,
                           bd.SV_BF16),
            [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'],
                           l['out']) for l in L if l['kind'] == 'attn'],
            bd.gdn_config(w.H, w.dk, w.dv, batch.B, bd.SV_BF16), self.gdn,
            bd.accept_args(amode, acc['target_logits'], acc['draft_tokens'],
                           acc.get('draft_logits'), acc.get('u_accept'), acc.get('u_final')))
        self.ws = torch.zeros(bd.spec_verify_step_workspace_bytes(self.sb, self.args),
                              dtype=torch.uint8, device=DEV)
        self.result = torch.full((batch.B * (1 + batch.max_T),), -7, dtype=torch.int32,
                                 device=DEV)
        self.commits = [torch.full((batch.B,), -7, dtype=torch.int32, device=DEV)
                        for _ in range(2)]
        self.ctx = batch.ctx_lens.clone()
        self.err = err_word()
        self.schedule = schedule
        arr = (bd.SvGdnLayer * len(self.gdn))(*self.gdn)
        self.pend_arr = arr
        self.pends = [bd.SvStepPending(self.sb, arr, c.data_ptr()) for c in self.commits]

    def step(self, out_j, pend_j):
        bd.spec_verify_step(self.sb, self.args, self.ctx, self.result, self.commits[out_j],
                            schedule=self.schedule,
                            pending=None if pend_j is None else self.pends[pend_j],
                            workspace=self.ws, err=self.err)

    def snapshot(self):
        snap = {'result': self.result.clone(), 'ctx': self.ctx.clone(),
                'commits': [c.clone() for c in self.commits]}
        for i, l in enumerate(self.layers):
            for key in ('out', 'state', 'k_cache', 'v_cache'):
                if key in l:
                    snap[(i, key)] = l[key].clone()
        return snap


def _equal(a, b):
    for k in a:
        if k == 'commits':
            assert all(torch.equal(x, y) for x, y in zip(a[k], b[k])), k
        else:
            assert torch.equal(a[k], b[k]) or (
                a[k].dtype.is_floating_point and
                torch.equal(torch.isnan(a[k]), torch.isnan(b[k])) and
                torch.equal(a[k].nan_to_num(), b[k].nan_to_num())), k


@pytest.mark.parametrize('schedule', [bd.SV_SCHEDULE_DEFERRED, bd.SV_SCHEDULE_TWO_PHASE])
def test_graph_replays_equal_eager_steps(schedule):
    w, batch, layers, acc = _setup(71, 'rejection')
    deferred = schedule == bd.SV_SCHEDULE_DEFERRED
    n_steps = 4
    plan = [(0, None)] + [((i % 2), (i - 1) % 2 if deferred else None)
                          for i in range(1, n_steps)]
    # eager reference: snapshot after every step
    eager = Runner(w, batch, layers, acc, 'rejection', schedule)
    ref = []
    for out_j, pend_j in plan:
        eager.step(out_j, pend_j)
        torch.cuda.synchronize()
        ref.append(eager.snapshot())
    assert int(eager.err.item()) == 0
    # graphs: the first step eager, then one graph per (out, pending) pair
    g = Runner(w, batch, layers, acc, 'rejection', schedule)
    g.step(*plan[0])
    torch.cuda.synchronize()
    _equal(ref[0], g.snapshot())
    graphs = {}
    for pair in set(plan[1:]):
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, capture_error_mode='thread_local'):
            g.step(*pair)
        graphs[pair] = cg
    torch.cuda.synchronize()
    _equal(ref[0], g.snapshot())          # capturing ran nothing
    say('graph replays, schedule', schedule, 'graphs', len(graphs))
    for i in range(1, n_steps):
        junk = torch.randn(1 << 20, device=DEV).sum()     # eager work between replays
        graphs[plan[i]].replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        _equal(ref[i], g.snapshot())
    assert int(g.err.item()) == 0
    if deferred:  # the flush of the last step's tokens, eager and replayed from a graph
        last = plan[-1][0]
        bd.spec_verify_flush(eager.args, bd.step_pending(eager.sb, eager.args,
                                                         eager.commits[last]), err=eager.err)
        torch.cuda.synchronize()
        ref_flush = eager.snapshot()
        pend = bd.step_pending(g.sb, g.args, g.commits[last])
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, capture_error_mode='thread_local'):
            bd.spec_verify_flush(g.args, pend, err=g.err)
        cg.replay()
        torch.cuda.synchronize()
        _equal(ref_flush, g.snapshot())
        assert int(g.err.item()) == 0


def test_graph_replay_matches_the_oracle():
    """Two-phase step captured once and replayed: its acceptance, commit
    lengths, ctx_lens and GDN states against the oracle step."""
    w, batch, layers, acc = _setup(73, 'greedy')
    r = Runner(w, batch, layers, acc, 'greedy', bd.SV_SCHEDULE_TWO_PHASE)
    # warm the launch-shape caches eagerly on a throwaway copy
    Runner(w, batch, layers, acc, 'greedy', bd.SV_SCHEDULE_TWO_PHASE).step(0, None)
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg, capture_error_mode='thread_local'):
        r.step(0, None)
    cg.replay()
    torch.cuda.synchronize()
    assert int(r.err.item()) == 0
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
    ref = oracle.verify_step(lays, npi(batch.cu_seqlens), npi(batch.ctx_lens),
                             npi(batch.block_table), batch.P, batch.max_T, 'greedy',
                             {'target_logits': np64(acc['target_logits']),
                              'draft_tokens': npi(acc['draft_tokens'])})
    res = npi(r.result)
    np.testing.assert_array_equal(res[:batch.B], ref['accept_len'])
    np.testing.assert_array_equal(res[batch.B:].reshape(batch.B, -1), ref['out_tokens'])
    np.testing.assert_array_equal(npi(r.commits[0]), ref['commit_len'])
    np.testing.assert_array_equal(npi(r.ctx), ref['ctx_lens'])
    for i, l in enumerate(r.layers):
        if l['kind'] == 'gdn':
            check_gdn_state(np64(l['state']), ref['state'][i])
