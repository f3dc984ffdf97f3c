"""GPU parity of spec_verify_attention against the oracle (through the C ABI).

Tolerance: output max-abs <= 2e-3 at fp32 I/O, <= 1e-2 + half a bf16 ulp of
|o_ref| at bf16 I/O (the output's own rounding).  The KV pools after the
call must equal the oracle's append bit for bit (every slot, written or
not).  Page-permutation invariance is checked bit-exactly.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import (DEV, bits, check_attn_out, err_word, np64, npi, say,
                         sv_batch)

pytestmark = pytest.mark.gpu


def _run(w, batch, lay, table=None, kc=None, vc=None, write_kv=True):
    kc = (lay['k_cache'] if kc is None else kc).clone()
    vc = (lay['v_cache'] if vc is None else vc).clone()
    table = batch.block_table if table is None else table
    out = torch.full_like(lay['q'], float('nan'))
    dt = bd.SV_BF16 if lay['q'].dtype == torch.bfloat16 else bd.SV_F32
    nbytes = bd.spec_verify_attention_workspace_bytes(
        batch.B, batch.total_T, w.Hq, w.Hkv, w.D, table.shape[1], batch.P, dt)
    # garbage scratch: no result may depend on what the workspace held
    ws = torch.full((max(nbytes, 1),), 0x7f, dtype=torch.uint8, device=DEV)
    err = err_word()
    bd.spec_verify_attention(sv_batch(batch), lay['q'], lay['k_new'], lay['v_new'], kc, vc,
                             table, batch.ctx_lens, out, write_kv=write_kv,
                             workspace=ws, err=err)
    torch.cuda.synchronize()
    return out, kc, vc, int(err.item())


def _seq_ref(lay, batch, b):
    """Oracle output of sequence b alone (only its pages gathered)."""
    cu, table, ctx = npi(batch.cu_seqlens), npi(batch.block_table), npi(batch.ctx_lens)
    pages = table[b][table[b] >= 0]
    sub_t = np.full_like(table[b:b + 1], -1)
    sub_t[0, :len(pages)] = np.arange(len(pages))
    rows = slice(cu[b], cu[b + 1])
    return oracle.verify_attention(
        np64(lay['q'][rows]), np64(lay['k_new'][rows]), np64(lay['v_new'][rows]),
        np64(lay['k_cache'][torch.from_numpy(pages).to(DEV)]),
        np64(lay['v_cache'][torch.from_numpy(pages).to(DEV)]), sub_t, ctx[b:b + 1],
        np.array([0, cu[b + 1] - cu[b]]), batch.P), rows


def _check(w, batch, lay, seqs=None):
    out, kc, vc, err = _run(w, batch, lay)
    assert err == 0, err
    cu = npi(batch.cu_seqlens)
    table = npi(batch.block_table)
    ctx = npi(batch.ctx_lens)
    if seqs is None:
        ref = oracle.verify_attention(np64(lay['q']), np64(lay['k_new']), np64(lay['v_new']),
                                      np64(lay['k_cache']), np64(lay['v_cache']), table, ctx,
                                      cu, batch.P)
        e = check_attn_out(np64(out), ref, lay['q'].dtype)
    else:
        e = 0.0
        for b in seqs:    # one sequence at a time: gather only its pages
            ref, rows = _seq_ref(lay, batch, b)
            e = max(e, check_attn_out(np64(out[rows]), ref, lay['q'].dtype))
    # the append, bit for bit over the whole pool
    k_exp, v_exp = oracle.append_kv(bits(lay['k_cache']), bits(lay['v_cache']),
                                    bits(lay['k_new']), bits(lay['v_new']), table, ctx, cu,
                                    batch.P)
    assert np.array_equal(bits(kc), k_exp)
    assert np.array_equal(bits(vc), v_exp)
    return e, out


@pytest.mark.parametrize("ctx", [None, [14, 15], [16, 0], [31, 48]])
def test_tiny_fp32(ctx):
    w = wl.WORKLOADS[0]
    batch = wl.make_batch(w, 0, DEV, ctx_override=ctx)
    lay = wl.make_attn_layer(w, batch, 1, DEV)
    say('attention tiny fp32 ctx', ctx)
    _check(w, batch, lay)


@pytest.mark.parametrize("seed", [1, 103])
def test_full_size_bf16(seed):
    w = wl.WORKLOADS[1]
    batch = wl.make_batch(w, seed, DEV)
    lay = wl.make_attn_layer(w, batch, seed + 1, DEV)
    say('attention full-size bf16 seed', seed)
    e, _ = _check(w, batch, lay)
    say(f'  max abs err {e:.2e}')


@pytest.mark.parametrize("D,P,Hq,Hkv,k,ctx", [
    (64, 16, 8, 2, 7, (0, 300)),       # tiles span 4 pages, 32 query rows
    (128, 32, 16, 2, 7, (60, 700)),    # 64 query rows
    (128, 128, 32, 8, 3, (100, 900)),  # a page spans 2 tiles
    (64, 64, 4, 4, 7, (62, 130)),      # G = 1
])
def test_shapes_and_page_sizes_bf16(D, P, Hq, Hkv, k, ctx):
    w = wl.Workload('shapes', B=7, k=k, ragged_k=True, ctx=ctx, P=P, Hq=Hq, Hkv=Hkv, D=D,
                    pool_factor=1.3)
    batch = wl.make_batch(w, 21, DEV)
    lay = wl.make_attn_layer(w, batch, 22, DEV)
    say('attention shapes', D, P, Hq, Hkv, k, ctx)
    _check(w, batch, lay)


def test_long_context_many_splits():
    w = wl.Workload('long', B=3, k=7, ragged_k=True, ctx=(16384, 32768), pool_factor=1.25)
    batch = wl.make_batch(w, 31, DEV)
    lay = wl.make_attn_layer(w, batch, 32, DEV)
    say('attention long context', batch.ctx)
    _check(w, batch, lay, seqs=range(batch.B))


def test_page_boundary_straddles():
    w = wl.Workload('straddle', B=6, k=3, ragged_k=False, ctx=(0, 1), P=64)
    batch = wl.make_batch(w, 41, DEV, ctx_override=[0, 61, 62, 63, 64, 127])
    lay = wl.make_attn_layer(w, batch, 42, DEV)
    _check(w, batch, lay)


def test_physical_page_permutation_is_bit_exact():
    w = wl.Workload('perm', B=8, k=3, ragged_k=False, ctx=(500, 2000))
    batch = wl.make_batch(w, 51, DEV)
    lay = wl.make_attn_layer(w, batch, 52, DEV)
    out1, kc1, vc1, _ = _run(w, batch, lay)
    perm = torch.randperm(batch.num_pages, generator=torch.Generator().manual_seed(5)).to(DEV)
    kc2 = torch.empty_like(lay['k_cache'])
    vc2 = torch.empty_like(lay['v_cache'])
    kc2[perm] = lay['k_cache']
    vc2[perm] = lay['v_cache']
    t = batch.block_table
    t2 = torch.where(t >= 0, perm[t.clamp(min=0).long()].to(torch.int32), t)
    out2, kc2o, vc2o, _ = _run(w, batch, lay, table=t2, kc=kc2, vc=vc2)
    assert torch.equal(out1, out2)
    assert torch.equal(kc2o[perm], kc1) and torch.equal(vc2o[perm], vc1)


def test_no_write_leaves_pool_untouched():
    w = wl.WORKLOADS[1]
    w = wl.Workload(**{**w.__dict__, 'B': 4})
    batch = wl.make_batch(w, 61, DEV)
    lay = wl.make_attn_layer(w, batch, 62, DEV)
    out, kc, vc, err = _run(w, batch, lay, write_kv=False)
    assert err == 0
    assert torch.equal(kc, lay['k_cache']) and torch.equal(vc, lay['v_cache'])


def test_bad_page_and_capacity_are_flagged():
    w = wl.Workload('bad', B=3, k=3, ragged_k=False, ctx=(100, 200))
    batch = wl.make_batch(w, 71, DEV)
    lay = wl.make_attn_layer(w, batch, 72, DEV)
    t = batch.block_table.clone()
    t[1, 0] = batch.num_pages + 3                   # outside the pool
    _, _, _, err = _run(w, batch, lay, table=t)
    assert err & 1
    c2 = batch.ctx_lens.clone()
    c2[2] = t.shape[1] * batch.P                    # ctx + T overflows the table
    b2 = wl.Batch(**{**batch.__dict__, 'ctx_lens': c2})
    out, _, _, err = _run(w, b2, lay)
    assert err & 2
    rows = slice(int(batch.cu_seqlens[2]), int(batch.cu_seqlens[3]))
    assert torch.isnan(out[rows].float()).all()     # skipped sequence untouched



def test_largest_batch():
    # 2048 sequences (the bf16 path's limit): every thread of the start-up
    # scan owns eight sequences; ragged drafts, short contexts
    w = wl.Workload('b2048', B=2048, k=7, ragged_k=True, ctx=(0, 100))
    batch = wl.make_batch(w, 95, DEV)
    lay = wl.make_attn_layer(w, batch, 96, DEV)
    say('largest batch: B', batch.B, 'total_T', batch.total_T)
    out, kc, vc, err = _run(w, batch, lay)
    assert err == 0
    for b in (0, 1, 255, 256, 511, 1000, 1023, 1024, 1500, 1791, 2000, 2040, 2045, 2046, 2047, 7):
        ref, rows = _seq_ref(lay, batch, b)
        check_attn_out(np64(out[rows]), ref, lay['q'].dtype)
    cu, table, ctx = npi(batch.cu_seqlens), npi(batch.block_table), npi(batch.ctx_lens)
    k_exp, v_exp = oracle.append_kv(bits(lay['k_cache']), bits(lay['v_cache']),
                                    bits(lay['k_new']), bits(lay['v_new']), table, ctx, cu,
                                    batch.P)
    assert np.array_equal(bits(kc), k_exp)
    assert np.array_equal(bits(vc), v_exp)


def test_skipped_sequence_inside_a_workgroup_range():
    # long contexts: each resident workgroup streams tens of tiles, so ranges
    # run across the skipped sequence (no tiles) from one valid one to the next
    w = wl.Workload('skip_mid', B=5, k=3, ragged_k=False, ctx=(20000, 30000))
    batch = wl.make_batch(w, 91, DEV)
    lay = wl.make_attn_layer(w, batch, 92, DEV)
    c2 = batch.ctx_lens.clone()
    c2[2] = batch.block_table.shape[1] * batch.P    # ctx + T overflows the table
    b2 = wl.Batch(**{**batch.__dict__, 'ctx_lens': c2})
    say('skip_mid: B=5, ctx', npi(c2).tolist())
    out, _, _, err = _run(w, b2, lay)
    assert err == 2
    cu = npi(batch.cu_seqlens)
    assert torch.isnan(out[int(cu[2]):int(cu[3])].float()).all()
    for b in (0, 1, 3, 4):
        ref, rows = _seq_ref(lay, batch, b)
        check_attn_out(np64(out[rows]), ref, lay['q'].dtype)


@pytest.mark.parametrize("seed", [5, 15])
def test_fewer_tiles_than_workgroups_on_a_reused_workspace(seed):
    # 2 sequences, 3-5 tiles per segment: far fewer tiles than resident
    # workgroups, so a segment's tiles sit in workgroups with empty ranges
    # between them; the workspace holds garbage, then another call's partials
    w = wl.Workload('few', B=2, k=3, ragged_k=False, ctx=(150, 250))
    batch = wl.make_batch(w, seed, DEV)
    lay = wl.make_attn_layer(w, batch, seed + 1, DEV)
    other = wl.make_attn_layer(w, batch, seed + 2, DEV)
    nbytes = bd.spec_verify_attention_workspace_bytes(
        batch.B, batch.total_T, w.Hq, w.Hkv, w.D, batch.block_table.shape[1], batch.P,
        bd.SV_BF16)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=DEV)   # garbage scratch
    ref = oracle.verify_attention(np64(lay['q']), np64(lay['k_new']), np64(lay['v_new']),
                                  np64(lay['k_cache']), np64(lay['v_cache']),
                                  npi(batch.block_table), npi(batch.ctx_lens),
                                  npi(batch.cu_seqlens), batch.P)
    say('few tiles, reused workspace, seed', seed)
    for src in (None, other):
        if src is not None:   # leave another call's partials in the workspace
            bd.spec_verify_attention(sv_batch(batch), src['q'], src['k_new'], src['v_new'],
                                     src['k_cache'].clone(), src['v_cache'].clone(),
                                     batch.block_table, batch.ctx_lens,
                                     torch.empty_like(src['q']), workspace=ws)
        out = torch.full_like(lay['q'], float('nan'))
        bd.spec_verify_attention(sv_batch(batch), lay['q'], lay['k_new'], lay['v_new'],
                                 lay['k_cache'].clone(), lay['v_cache'].clone(),
                                 batch.block_table, batch.ctx_lens, out, workspace=ws)
        torch.cuda.synchronize()
        check_attn_out(np64(out), ref, lay['q'].dtype)


def test_repeated_calls_on_one_workspace_are_identical():
    w = wl.Workload('reuse', B=6, k=3, ragged_k=False, ctx=(3000, 9000))
    batch = wl.make_batch(w, 81, DEV)
    lay = wl.make_attn_layer(w, batch, 82, DEV)
    nbytes = bd.spec_verify_attention_workspace_bytes(
        batch.B, batch.total_T, w.Hq, w.Hkv, w.D, batch.block_table.shape[1], batch.P,
        bd.SV_BF16)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=DEV)   # garbage scratch
    outs = []
    for _ in range(3):
        out = torch.full_like(lay['q'], float('nan'))
        bd.spec_verify_attention(sv_batch(batch), lay['q'], lay['k_new'], lay['v_new'],
                                 lay['k_cache'].clone(), lay['v_cache'].clone(),
                                 batch.block_table, batch.ctx_lens, out, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    _check(w, batch, lay)
