"""A sequence whose block-table range holds a page id outside the pool is
flagged (SV_DERR_PAGE) and skipped by every attention path: its output rows
keep what they held, nothing is appended to its pages, and every other
sequence still matches the oracle (the pools equal the oracle's append of
the other sequences, byte for byte).

The bad id sits in the first page, in a middle page or in the page that holds
the in-flight positions; with long contexts the bad sequence is cut into
pieces over several workgroups, so pieces that never read the bad page must
skip it too.  Tolerances as in the per-path tests (1e-2 bf16 / 2e-3 fp32).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import DEV, bits, check_attn_out, err_word, np64, npi, say, sv_batch

pytestmark = pytest.mark.gpu

BAD = 1   # the sequence that gets the bad id


def _bad_table(batch, where):
    t = batch.block_table.clone()
    L, T = batch.ctx[BAD], batch.T[BAD]
    n = (L + T - 1) // batch.P + 1           # pages the sequence uses
    col = {'first': 0, 'middle': n // 2, 'inflight': (L + T - 1) // batch.P}[where]
    t[BAD, col] = batch.num_pages + 5 if where != 'middle' else -3
    return t


def _others(batch):
    return [b for b in range(batch.B) if b != BAD]


def _sub(batch, rows_of, seqs):
    """Packed rows, table rows, ctx and cu of a subset of the sequences."""
    cu = npi(batch.cu_seqlens)
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in seqs])
    T = [cu[b + 1] - cu[b] for b in seqs]
    return idx, np.concatenate([[0], np.cumsum(T)])


def _ws(w, batch, table, dt):
    n = bd.spec_verify_attention_workspace_bytes(batch.B, batch.total_T, w.Hq, w.Hkv, w.D,
                                                 table.shape[1], batch.P, dt)
    return torch.full((max(n, 1),), 0x7f, dtype=torch.uint8, device=DEV)


def _run(w, batch, lay, table, kind):
    kc, vc = lay['k_cache'].clone(), lay['v_cache'].clone()
    out = torch.full_like(lay['q'], float('nan'))
    err = err_word()
    if kind == 'int8':
        bd.spec_verify_attention_kv8(sv_batch(batch), lay['q'], lay['k_new'], lay['v_new'], kc,
                                     vc, lay['k_scale'], lay['v_scale'], table, batch.ctx_lens,
                                     out, workspace=_ws(w, batch, table, bd.SV_BF16), err=err)
    else:
        dt = bd.SV_BF16 if kind == 'bf16' else bd.SV_F32
        bd.spec_verify_attention(sv_batch(batch), lay['q'], lay['k_new'], lay['v_new'], kc, vc,
                                 table, batch.ctx_lens, out, workspace=_ws(w, batch, table, dt),
                                 err=err)
    torch.cuda.synchronize()
    return out, kc, vc, int(err.item())


def _ref_one(lay, batch, b, kind):
    cu, table, ctx = npi(batch.cu_seqlens), npi(batch.block_table), npi(batch.ctx_lens)
    pages = table[b][table[b] >= 0]
    sub_t = np.arange(len(pages))[None, :]
    rows = slice(cu[b], cu[b + 1])
    pg = torch.from_numpy(pages).to(DEV)
    cu1 = np.array([0, cu[b + 1] - cu[b]])
    if kind == 'int8':
        f32 = lambda t: t.detach().float().cpu().numpy()
        ref = oracle.verify_attention_int8(
            np64(lay['q'][rows]), f32(lay['k_new'][rows]), f32(lay['v_new'][rows]),
            lay['k_cache'][pg].cpu().numpy(), lay['v_cache'][pg].cpu().numpy(),
            f32(lay['k_scale']), f32(lay['v_scale']), sub_t, ctx[b:b + 1], cu1, batch.P)
    else:
        ref = oracle.verify_attention(np64(lay['q'][rows]), np64(lay['k_new'][rows]),
                                      np64(lay['v_new'][rows]), np64(lay['k_cache'][pg]),
                                      np64(lay['v_cache'][pg]), sub_t, ctx[b:b + 1], cu1,
                                      batch.P)
    return ref, rows


CASES = {
    # kind: (dtype, contexts, batch): long bf16 / INT8 contexts split each
    # sequence over several workgroups; the fp32 path takes one wave per row
    'bf16': (torch.bfloat16, (20000, 30000), 5),
    'int8': (torch.bfloat16, (20000, 30000), 5),
    'fp32': (torch.float32, (500, 1500), 4),
}


@pytest.mark.parametrize('where', ['first', 'middle', 'inflight'])
@pytest.mark.parametrize('kind', ['bf16', 'int8', 'fp32'])
def test_bad_page_skips_the_sequence(kind, where):
    dt, ctx, B = CASES[kind]
    w = wl.Workload('bad_page', B=B, k=3, ragged_k=False, ctx=ctx, attn_dtype=dt)
    batch = wl.make_batch(w, 41, DEV)
    lay = (wl.make_attn_layer_kv8 if kind == 'int8' else wl.make_attn_layer)(w, batch, 42, DEV)
    table = _bad_table(batch, where)
    say('bad page', kind, where)
    out, kc, vc, err = _run(w, batch, lay, table, kind)
    assert err == 1, err                                   # SV_DERR_PAGE only
    cu = npi(batch.cu_seqlens)
    assert torch.isnan(out[cu[BAD]:cu[BAD + 1]].float()).all()
    for b in _others(batch):
        ref, rows = _ref_one(lay, batch, b, kind)
        check_attn_out(np64(out[rows]), ref, dt)
    # the pools: the oracle's append of the other sequences only
    seqs = _others(batch)
    idx, cu_s = _sub(batch, None, seqs)
    idx = torch.from_numpy(idx).to(DEV)
    tab = npi(batch.block_table)[seqs]
    ctx_s = npi(batch.ctx_lens)[seqs]
    if kind == 'int8':
        f32 = lambda t: t.detach().float().cpu().numpy()
        k_exp, v_exp = oracle.append_kv_int8(
            lay['k_cache'].cpu().numpy(), lay['v_cache'].cpu().numpy(), f32(lay['k_new'][idx]),
            f32(lay['v_new'][idx]), f32(lay['k_scale']), f32(lay['v_scale']), tab, ctx_s, cu_s,
            batch.P)
        assert np.array_equal(kc.cpu().numpy(), k_exp)
        assert np.array_equal(vc.cpu().numpy(), v_exp)
    else:
        k_exp, v_exp = oracle.append_kv(bits(lay['k_cache']), bits(lay['v_cache']),
                                        bits(lay['k_new'][idx]), bits(lay['v_new'][idx]), tab,
                                        ctx_s, cu_s, batch.P)
        assert np.array_equal(bits(kc), k_exp)
        assert np.array_equal(bits(vc), v_exp)
