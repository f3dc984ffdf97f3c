"""GPU parity of spec_verify_attention_kv8 (INT8 pages) against the oracle.

Tolerance: output max-abs <= 1e-2 + half a bf16 ulp of |o_ref| (bf16 I/O, as
for bf16 pages).  The INT8
pools after the call must equal the oracle's append of the in-flight codes
byte for byte (every slot, written or not): the codes are integer decisions
taken in fp32 on both sides.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import DEV, check_attn_out, err_word, np64, npi, say, sv_batch

pytestmark = pytest.mark.gpu


def _ws(w, batch, table):
    n = bd.spec_verify_attention_workspace_bytes(batch.B, batch.total_T, w.Hq, w.Hkv, w.D,
                                                 table.shape[1], batch.P, bd.SV_BF16)
    # garbage scratch: no result may depend on what the workspace held
    return torch.full((max(n, 1),), 0x7f, dtype=torch.uint8, device=DEV)


def _run(w, batch, lay, table=None, ctx=None):
    kc, vc = lay['k_cache'].clone(), lay['v_cache'].clone()
    table = batch.block_table if table is None else table
    ctx = batch.ctx_lens if ctx is None else ctx
    out = torch.full_like(lay['q'], float('nan'))
    err = err_word()
    bd.spec_verify_attention_kv8(sv_batch(batch), lay['q'], lay['k_new'], lay['v_new'], kc, vc,
                                 lay['k_scale'], lay['v_scale'], table, ctx, out,
                                 workspace=_ws(w, batch, table), err=err)
    torch.cuda.synchronize()
    return out, kc, vc, int(err.item())


def _i8(t):
    return t.detach().cpu().numpy()


def _f32(t):
    return t.detach().float().cpu().numpy()


def _check(w, batch, lay, seqs=None):
    out, kc, vc, err = _run(w, batch, lay)
    assert err == 0, err
    cu, table, ctx = npi(batch.cu_seqlens), npi(batch.block_table), npi(batch.ctx_lens)
    ks, vs = _f32(lay['k_scale']), _f32(lay['v_scale'])
    e = 0.0
    for b in (range(batch.B) if seqs is None else seqs):
        pages = table[b][table[b] >= 0]
        sub_t = np.full_like(table[b:b + 1], -1)
        sub_t[0, :len(pages)] = np.arange(len(pages))
        rows = slice(cu[b], cu[b + 1])
        pg = torch.from_numpy(pages).to(DEV)
        ref = oracle.verify_attention_int8(
            np64(lay['q'][rows]), _f32(lay['k_new'][rows]), _f32(lay['v_new'][rows]),
            _i8(lay['k_cache'][pg]), _i8(lay['v_cache'][pg]), ks, vs, sub_t, ctx[b:b + 1],
            np.array([0, cu[b + 1] - cu[b]]), batch.P)
        e = max(e, check_attn_out(np64(out[rows]), ref, torch.bfloat16))
    k_exp, v_exp = oracle.append_kv_int8(_i8(lay['k_cache']), _i8(lay['v_cache']),
                                         _f32(lay['k_new']), _f32(lay['v_new']), ks, vs, table,
                                         ctx, cu, batch.P)
    assert np.array_equal(_i8(kc), k_exp)
    assert np.array_equal(_i8(vc), v_exp)
    return e, out


@pytest.mark.parametrize("D,P,Hq,Hkv,k,ctx", [
    (128, 64, 32, 8, 3, (0, 300)),     # the bench heads; contexts from empty
    (64, 16, 8, 2, 7, (0, 300)),       # tiles span 4 pages, 32 query rows
    (128, 32, 16, 2, 7, (60, 700)),    # 64 query rows
    (128, 128, 32, 8, 3, (100, 900)),  # a page spans 2 tiles
    (64, 64, 4, 4, 7, (62, 130)),      # G = 1
])
def test_shapes_and_page_sizes(D, P, Hq, Hkv, k, ctx):
    w = wl.Workload('kv8', B=7, k=k, ragged_k=True, ctx=ctx, P=P, Hq=Hq, Hkv=Hkv, D=D,
                    pool_factor=1.3)
    batch = wl.make_batch(w, 121, DEV)
    lay = wl.make_attn_layer_kv8(w, batch, 122, DEV)
    say('attention kv8 shapes', D, P, Hq, Hkv, k, ctx)
    e, _ = _check(w, batch, lay)
    say(f'  max abs err {e:.2e}')


def test_full_size_every_sequence():
    """The bench's attention shape (B = 64, k = 3, contexts U[2048, 8192]) in
    the launch configuration it times: every sequence's outputs against the
    oracle (one sequence at a time, its pages gathered), the whole pool byte
    for byte."""
    w = wl.WORKLOADS[3]
    batch = wl.make_batch(w, 131, DEV)
    lay = wl.make_attn_layer_kv8(w, batch, 132, DEV)
    say('attention kv8 full size, every sequence')
    e, _ = _check(w, batch, lay)
    say(f'  max abs err {e:.2e}')


def test_long_context_many_splits():
    w = wl.Workload('long', B=3, k=7, ragged_k=True, ctx=(16384, 32768), pool_factor=1.25)
    batch = wl.make_batch(w, 141, DEV)
    lay = wl.make_attn_layer_kv8(w, batch, 142, DEV)
    _check(w, batch, lay)


def test_saturating_rows_and_page_straddles():
    w = wl.Workload('straddle', B=6, k=3, ragged_k=False, ctx=(0, 1), P=64)
    batch = wl.make_batch(w, 151, DEV, ctx_override=[0, 61, 62, 63, 64, 127])
    lay = wl.make_attn_layer_kv8(w, batch, 152, DEV)
    lay['k_new'] = (lay['k_new'].float() * 8).to(torch.bfloat16)   # many codes clamp at +-127
    _, kc, _, _ = _run(w, batch, lay)
    assert int((kc == 127).sum()) > 0 and int((kc == -128).sum()) == 0
    _check(w, batch, lay)


def test_bad_page_is_flagged():
    w = wl.Workload('bad', B=3, k=3, ragged_k=False, ctx=(100, 200))
    batch = wl.make_batch(w, 161, DEV)
    lay = wl.make_attn_layer_kv8(w, batch, 162, DEV)
    t = batch.block_table.clone()
    t[1, 0] = batch.num_pages + 3
    _, _, _, err = _run(w, batch, lay, table=t)
    assert err & 1


def test_matches_bf16_pages_holding_the_dequantized_values():
    """Pools whose codes dequantize to bf16-exact values (power-of-two scales)
    and in-flight rows on the grid: the INT8 call agrees with the bf16 call on
    the dequantized pools to within the rounding of the MFMA operands."""
    w = wl.Workload('cmp', B=8, k=3, ragged_k=False, ctx=(500, 3000))
    batch = wl.make_batch(w, 171, DEV)
    lay = wl.make_attn_layer_kv8(w, batch, 172, DEV)
    lay['k_scale'] = torch.full_like(lay['k_scale'], 1 / 32)
    lay['v_scale'] = torch.full_like(lay['v_scale'], 1 / 32)
    kq = (lay['k_new'].float() * 32).round().clamp(-127, 127)
    vq = (lay['v_new'].float() * 32).round().clamp(-127, 127)
    lay['k_new'] = (kq / 32).to(torch.bfloat16)
    lay['v_new'] = (vq / 32).to(torch.bfloat16)
    out8, kc8, vc8, err = _run(w, batch, lay)
    assert err == 0
    kcb = (lay['k_cache'].float() / 32).to(torch.bfloat16)
    vcb = (lay['v_cache'].float() / 32).to(torch.bfloat16)
    outb = torch.full_like(lay['q'], float('nan'))
    n = bd.spec_verify_attention_workspace_bytes(batch.B, batch.total_T, w.Hq, w.Hkv, w.D,
                                                 batch.block_table.shape[1], batch.P, bd.SV_BF16)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    bd.spec_verify_attention(sv_batch(batch), lay['q'], lay['k_new'], lay['v_new'], kcb, vcb,
                             batch.block_table, batch.ctx_lens, outb, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal((kc8.float() / 32).to(torch.bfloat16), kcb)
    d = (out8.float() - outb.float()).abs().max().item()
    assert d <= 1e-2, d
