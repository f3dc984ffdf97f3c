"""GPU parity of spec_accept against the oracle (through the C ABI).

Bit-exact: accept_len, output token rows, commit_len and ctx_lens.  Where a
rejection-sampling result differed, the oracle's decision margins would have
to sit inside float64 rounding; none is expected and the test fails.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import DEV, err_word, np64, npi, say, sv_batch

pytestmark = pytest.mark.gpu


def _run(batch, a, mode, ctx=None, bonus=None):
    B, mT = batch.B, batch.max_T
    result = torch.full((B * (1 + mT),), -7, dtype=torch.int32, device=DEV)
    commit = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    ctx = (batch.ctx_lens if ctx is None else ctx).clone()
    ws = torch.empty(bd.spec_accept_workspace_bytes(B, batch.total_T, a['target_logits'].shape[1],
                                                    mode), dtype=torch.uint8, device=DEV)
    err = err_word()
    bd.spec_accept(sv_batch(batch), mode, a['target_logits'], a['draft_tokens'], result,
                   draft_logits=a.get('draft_logits'), u_accept=a.get('u_accept'),
                   u_final=a.get('u_final'), commit_len_out=commit, ctx_lens_inout=ctx,
                   workspace=ws, err=err, bonus_tokens=bonus)
    torch.cuda.synchronize()
    r = npi(result)
    return r[:B], r[B:].reshape(B, mT), npi(commit), npi(ctx), int(err.item())


def _oracle(batch, a, mode, bonus=None):
    cu = npi(batch.cu_seqlens)
    bn = None if bonus is None else npi(bonus)
    if mode == bd.SV_ACCEPT_GREEDY:
        return oracle.greedy_accept(np64(a['target_logits']), npi(a['draft_tokens']), cu,
                                    batch.max_T, bonus_tokens=bn) + (None,)
    dl = a.get('draft_logits')
    return oracle.rejection_accept(np64(a['target_logits']), None if dl is None else np64(dl),
                                   npi(a['draft_tokens']), np64(a['u_accept']),
                                   np64(a['u_final']), cu, batch.max_T, return_margins=True,
                                   bonus_tokens=bn)


def _check(batch, a, mode, bonus=None):
    acc, out, commit, ctx, err = _run(batch, a, mode, bonus=bonus)
    assert err == 0
    acc_r, out_r, margins = _oracle(batch, a, mode, bonus)
    if not (np.array_equal(acc, acc_r) and np.array_equal(out, out_r)):
        bad = np.nonzero((acc != acc_r) | (out != out_r).any(1))[0]
        msg = [f'seq {b}: gpu {acc[b]} {out[b].tolist()} oracle {acc_r[b]} {out_r[b].tolist()}'
               + (f' margins {margins[b]}' if margins else '') for b in bad[:5]]
        raise AssertionError('acceptance mismatch:\n' + '\n'.join(msg))
    np.testing.assert_array_equal(commit, acc_r + 1)
    np.testing.assert_array_equal(ctx, np.array(batch.ctx) + acc_r + 1)
    return acc_r


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
@pytest.mark.parametrize("seed", [0, 100, 101])
def test_tiny_fp32(mode, seed):
    w = wl.WORKLOADS[0]
    batch = wl.make_batch(w, seed, DEV)
    a = wl.make_accept(w, batch, seed + 1, 'greedy' if mode == 0 else 'rejection', DEV)
    say('accept tiny', mode, seed)
    _check(batch, a, mode)


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
def test_hybrid_step_vocab(mode):
    w = wl.WORKLOADS[3]
    batch = wl.make_batch(w, 3, DEV)
    a = wl.make_accept(w, batch, 4, 'greedy' if mode == 0 else 'rejection', DEV)
    say('accept V=151936 B=64 mode', mode)
    acc = _check(batch, a, mode)
    say('  mean accepted', acc.mean())


def test_stress_ragged_rejection():
    w = wl.WORKLOADS[4]
    batch = wl.make_batch(w, 4, DEV)
    a = wl.make_accept(w, batch, 5, 'rejection', DEV)
    say('accept ragged B=256 rejection')
    acc = _check(batch, a, bd.SV_ACCEPT_REJECTION)
    say('  mean accepted', acc.mean())


def test_greedy_bf16_ties_take_lowest_index():
    w = wl.Workload('ties', B=16, k=3, ragged_k=False, ctx=(5, 9), V=151936)
    batch = wl.make_batch(w, 7, DEV)
    a = wl.make_accept(w, batch, 8, 'greedy', DEV)
    t = a['target_logits'].float()
    g = torch.Generator(device='cpu').manual_seed(9)
    for r in range(batch.total_T):
        idx = torch.randint(0, w.V, (3,), generator=g)
        t[r, idx] = 30.0                       # three-way tie for the maximum
    a['target_logits'] = t.to(torch.bfloat16)
    first = [int(torch.nonzero(t[r] == 30.0)[0]) for r in range(batch.total_T)]
    cu = batch.cu_seqlens.tolist()
    d = a['draft_tokens'].clone()
    for b in range(batch.B):
        for i in range(batch.T[b] - 1):
            if (b + i) % 3:
                d[cu[b] - b + i] = first[cu[b] + i]
    a['draft_tokens'] = d
    _check(batch, a, bd.SV_ACCEPT_GREEDY)


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
def test_reject_sampler_layout(mode):
    # lmdeploy pull request 3945 (reject_sampler.py review): 3 sequences,
    # max_spec_len 2 -> rows [[0,1,2],[0,-1,-1],[1,-1,-1]]
    V = 5
    neg = -1.0e4

    def one_hot(idx):
        z = torch.full((len(idx), V), neg)
        z[torch.arange(len(idx)), torch.tensor(idx)] = 0.0
        return z.to(DEV)
    cu = torch.tensor([0, 3, 6, 9], dtype=torch.int32, device=DEV)
    batch = wl.Batch(B=3, max_T=3, T=[3, 3, 3], ctx=[0, 0, 0], cu_seqlens=cu,
                     ctx_lens=torch.zeros(3, dtype=torch.int32, device=DEV),
                     block_table=None, num_pages=0, P=16)
    drafts = [0, 1, 3, 4, 2, 2]
    a = {'target_logits': one_hot([0, 1, 2, 0, 3, 3, 1, 4, 4]),
         'draft_tokens': torch.tensor(drafts, dtype=torch.int32, device=DEV),
         'draft_logits': one_hot(drafts),
         'u_accept': torch.rand(6, device=DEV), 'u_final': torch.rand(3, device=DEV)}
    acc, out, *_ = _run(batch, a, mode)
    assert out.tolist() == [[0, 1, 2], [0, -1, -1], [1, -1, -1]]
    assert acc.tolist() == [2, 0, 0]


def test_rejection_q_equal_p_accepts_everything():
    w = wl.Workload('qp', B=32, k=3, ragged_k=False, ctx=(5, 9), V=32000)
    batch = wl.make_batch(w, 11, DEV)
    a = wl.make_accept(w, batch, 12, 'rejection', DEV)
    cu = batch.cu_seqlens.tolist()
    rows = [cu[b] + i for b in range(batch.B) for i in range(batch.T[b] - 1)]
    a['draft_logits'] = a['target_logits'][torch.tensor(rows, device=DEV)].contiguous()
    acc = _check(batch, a, bd.SV_ACCEPT_REJECTION)
    assert (acc == 3).all()


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
@pytest.mark.parametrize("V", [10007, 8200])
def test_row_layouts(mode, V):
    """V = 10007: bf16 rows are not 16-byte aligned, one element load per
    entry.  V = 8200: aligned rows read with 16-byte loads, and a last chunk
    of 8 entries."""
    w = wl.Workload('layout', B=8, k=3, ragged_k=True, ctx=(5, 9), V=V)
    batch = wl.make_batch(w, 21, DEV)
    a = wl.make_accept(w, batch, 22, 'greedy' if mode == 0 else 'rejection', DEV)
    _check(batch, a, mode)


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
def test_misaligned_logits(mode):
    """Logit rows one element past a 16-byte boundary take the element-load
    path and agree with the oracle."""
    w = wl.Workload('misaligned', B=8, k=3, ragged_k=False, ctx=(5, 9), V=8192)
    batch = wl.make_batch(w, 23, DEV)
    a = wl.make_accept(w, batch, 24, 'greedy' if mode == 0 else 'rejection', DEV)
    for key in ('target_logits', 'draft_logits'):
        t = a.get(key)
        if t is None:   # greedy: no draft logits
            continue
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        view = buf[1:].view(t.shape)
        view.copy_(t)
        assert view.data_ptr() % 16 != 0
        a[key] = view
    _check(batch, a, mode)


def test_bad_draft_token_is_flagged():
    w = wl.WORKLOADS[0]
    batch = wl.make_batch(w, 0, DEV)
    a = wl.make_accept(w, batch, 1, 'rejection', DEV)
    a['draft_tokens'][1] = w.V + 5
    for mode in (bd.SV_ACCEPT_REJECTION, bd.SV_ACCEPT_GREEDY):
        acc, out, commit, ctx, err = _run(batch, a, mode)
        assert err == 16                                     # SV_DERR_TOKEN only
        # sequence 0 skipped: accept_len -1, a row of -1, commit length 0,
        # ctx_lens kept; sequence 1 decided as usual
        assert acc[0] == -1 and (out[0] == -1).all()
        assert commit[0] == 0 and ctx[0] == batch.ctx[0]
        assert acc[1] >= 0 and commit[1] == acc[1] + 1


# ------------------------------------------------ point-mass drafts, supplied bonus
@pytest.mark.parametrize("wi,seed", [(0, 3), (3, 4), (4, 5)])
def test_rejection_point_mass_drafts(wi, seed):
    """No draft logits: each draft is a point mass (accept iff u < p(x),
    residual p without x).  Greedy-style drafts: the planted row maximum
    passes almost surely, the others almost never."""
    w = wl.WORKLOADS[wi]
    batch = wl.make_batch(w, seed, DEV)
    g = wl.make_accept(w, batch, seed + 1, 'greedy', DEV)
    r = wl.make_accept(w, batch, seed + 2, 'rejection', DEV)
    a = {'target_logits': g['target_logits'], 'draft_tokens': g['draft_tokens'],
         'u_accept': r['u_accept'], 'u_final': r['u_final']}
    say('point-mass drafts', w.name)
    acc = _check(batch, a, bd.SV_ACCEPT_REJECTION)
    say('  mean accepted', acc.mean())


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
@pytest.mark.parametrize("wi", [0, 3])
def test_supplied_bonus_tokens(mode, wi):
    w = wl.WORKLOADS[wi]
    batch = wl.make_batch(w, 6, DEV)
    a = wl.make_accept(w, batch, 7, 'greedy' if mode == 0 else 'rejection', DEV)
    bonus = torch.randint(0, w.V, (batch.B,), generator=torch.Generator().manual_seed(8),
                          dtype=torch.int32).to(DEV)
    acc = _check(batch, a, mode, bonus)
    if batch.B >= 32:
        assert (acc == batch.max_T - 1).any()      # some rows take the bonus


def test_bad_bonus_is_flagged_and_skipped():
    w = wl.WORKLOADS[0]
    batch = wl.make_batch(w, 9, DEV)
    a = wl.make_accept(w, batch, 10, 'greedy', DEV)
    # both sequences accept every draft: plant the drafts on the argmax
    g = a['target_logits'].float().argmax(dim=1).to(torch.int32)
    cu = npi(batch.cu_seqlens)
    d = torch.cat([g[cu[b]:cu[b + 1] - 1] for b in range(batch.B)])
    a = dict(a, draft_tokens=d.contiguous())
    bonus = torch.tensor([3, w.V + 5], dtype=torch.int32, device=DEV)
    acc, out, commit, ctx, err = _run(batch, a, bd.SV_ACCEPT_GREEDY, bonus=bonus)
    assert err & 16
    assert acc[0] == batch.max_T - 1 and out[0, batch.max_T - 1] == 3
    assert acc[1] == -1 and (out[1] == -1).all() and commit[1] == 0   # skipped
    assert ctx[1] == batch.ctx[1]
