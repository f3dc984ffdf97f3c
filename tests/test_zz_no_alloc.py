"""spec_accept_noalloc (the library's own device scratch, no workspace)
against spec_accept_args with a caller workspace, on the same inputs: two
calls in a row on one GPU, the second with a smaller batch, in both modes.
Integer results are compared bit for bit (the kernels are the same)."""

import numpy as np
import pytest
import torch

import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import DEV, err_word, npi, say, sv_batch

pytestmark = pytest.mark.gpu


def _both(batch, a, mode):
    B, mT = batch.B, batch.max_T
    outs = []
    for noalloc in (False, True):
        result = torch.full((B * (1 + mT),), -7, dtype=torch.int32, device=DEV)
        commit = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        ctx = batch.ctx_lens.clone()
        err = err_word()
        kw = dict(draft_logits=a.get('draft_logits'), u_accept=a.get('u_accept'),
                  u_final=a.get('u_final'), commit_len_out=commit, ctx_lens_inout=ctx, err=err)
        if noalloc:
            bd.spec_accept_noalloc(sv_batch(batch), mode, a['target_logits'],
                                   a['draft_tokens'], result, **kw)
        else:
            n = bd.spec_accept_workspace_bytes(B, batch.total_T, a['target_logits'].shape[1],
                                               mode)
            ws = torch.full((n,), 0x7f, dtype=torch.uint8, device=DEV)
            bd.spec_accept(sv_batch(batch), mode, a['target_logits'], a['draft_tokens'],
                           result, workspace=ws, **kw)
        torch.cuda.synchronize()
        outs.append((npi(result), npi(commit), npi(ctx), int(err.item())))
    return outs


@pytest.mark.parametrize('mode', [bd.SV_ACCEPT_REJECTION, bd.SV_ACCEPT_GREEDY])
def test_noalloc_matches_workspace_entry_point(mode):
    name = 'rejection' if mode == bd.SV_ACCEPT_REJECTION else 'greedy'
    # first the 256-sequence ragged batch, then a smaller one (64 sequences)
    for wi, seed in ((4, 51), (3, 52)):
        w = wl.WORKLOADS[wi]
        batch = wl.make_batch(w, seed, DEV)
        a = wl.make_accept(w, batch, seed + 1, name, DEV)
        say('noalloc acceptance', name, w.name, 'B', batch.B)
        (r0, c0, x0, e0), (r1, c1, x1, e1) = _both(batch, a, mode)
        assert e0 == 0 and e1 == 0
        np.testing.assert_array_equal(r1, r0)
        np.testing.assert_array_equal(c1, c0)
        np.testing.assert_array_equal(x1, x0)


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    # rejection over V = 151936 needs (2 total_T - B) * 38 chunk records of
    # 16 bytes: 8000 sequences of 8 tokens exceed 8 MiB
    B, T, V = 8000, 8, 151936
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device=DEV)
    b = bd.make_batch(cu, B, T, B * T)
    t = torch.empty((1, V), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros(1, dtype=torch.int32, device=DEV)
    u = torch.zeros(1, dtype=torch.float32, device=DEV)
    res = torch.empty(1, dtype=torch.int32, device=DEV)
    with pytest.raises(bd.SpecVerifyError) as ei:
        bd.spec_accept_noalloc(b, bd.SV_ACCEPT_REJECTION, t, d, res, draft_logits=t,
                               u_accept=u, u_final=u)
    assert ei.value.status == bd.SV_ECAPACITY and 'scratch' in str(ei.value)
