"""The C-ABI library loads and exports every symbol include/*.h declares, and
its host-side validation rejects bad arguments with a status (no GPU work)."""

import ctypes
import glob
import os
import re

import pytest

from block_draft_verification_spec_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, 'include', '*.h')):
        text = open(h).read()
        text = re.sub(r'/\*.*?\*/', '', text, flags=re.S)
        for m in re.finditer(r'SV_API\s+[\w\s\*]+?\b(\w+)\s*\(', text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {'spec_verify_attention', 'gdn_verify_commit', 'spec_accept',
            'spec_verify_step', 'sv_last_error'} <= names
    lib = ctypes.CDLL(bd.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_header_compiles_as_c_and_links():
    """include/spec_verify.h is plain C: a C99 program compiles against it,
    links against the library and gets host-side answers (no GPU work)."""
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which('gcc')
    hip_inc = '/opt/rocm/include'
    if gcc is None or not os.path.isdir(hip_inc):
        pytest.skip('gcc or the HIP headers are not installed')
    lib_dir = os.path.dirname(bd.LIB_PATH)
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, 'c_abi_check')
        r = subprocess.run([gcc, '-std=c99', '-Wall', '-Werror=implicit-function-declaration',
                            '-D__HIP_PLATFORM_AMD__', '-I', hip_inc, '-I',
                            os.path.join(ROOT, 'include'),
                            os.path.join(ROOT, 'tests', 'c_abi_check.c'), '-L', lib_dir,
                            '-lspecverify', '-Wl,-rpath,' + lib_dir, '-o', exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert run.returncode == 0, run.stdout + run.stderr
        assert 'gfx950' in run.stdout


def test_version_and_empty_error():
    assert 'gfx950' in bd.version()


def _batch(B=2, max_T=4, total_T=8, cu=1):
    return bd.SvBatch(B, max_T, total_T, cu)


@pytest.mark.parametrize("B,max_T,total_T,msg", [
    (0, 4, 8, 'B must be'),
    (2, 9, 8, 'max_T'),
    (2, 0, 8, 'max_T'),
    (2, 4, 1, 'inconsistent'),
    (2, 4, 9, 'inconsistent'),
])
def test_batch_validation(B, max_T, total_T, msg):
    L = bd.lib()
    b = _batch(B, max_T, total_T)
    st = L.spec_accept(ctypes.byref(b), 0, 8, None, 1, 10, 8, None, None, 8,
                       None, None, 8, 1 << 20, None, None)
    assert st != bd.SV_OK
    assert msg in L.sv_last_error().decode()


def test_attention_validation():
    L = bd.lib()
    b = _batch()
    args = dict(q=16, k=16, v=16, kc=16, vc=16, bt=16, maxp=4, npages=8, P=64,
                ctx=16, out=16, Hq=32, Hkv=8, D=128, dt=bd.SV_BF16)

    def call(**kw):
        a = {**args, **kw}
        return L.spec_verify_attention(
            ctypes.byref(b), a['q'], a['k'], a['v'], a['kc'], a['vc'], a['bt'],
            a['maxp'], a['npages'], a['P'], a['ctx'], a['out'], a['Hq'],
            a['Hkv'], a['D'], a['dt'], 0.0, 1, 16, 0, None, None)
    assert call(Hq=30) == bd.SV_EINVAL                       # Hq % Hkv
    assert call(D=96) == bd.SV_EDTYPE                        # bf16 head size
    assert call(P=48) == bd.SV_EINVAL                        # page size
    assert call(P=192) == bd.SV_EINVAL                       # not a power of two
    assert call(q=None) == bd.SV_EINVAL
    assert call(dt=7) == bd.SV_EDTYPE
    assert call(Hq=64, Hkv=2) == bd.SV_ECAPACITY             # 32 heads x 4 > 64 rows
    assert call(q=24) == bd.SV_EINVAL                        # misaligned
    b2049 = _batch(B=2049, max_T=4, total_T=2049 * 4)
    assert L.spec_verify_attention(
        ctypes.byref(b2049), 16, 16, 16, 16, 16, 16, 4, 8, 64, 16, 16, 32, 8, 128, bd.SV_BF16,
        0.0, 1, 16, 1 << 30, None, None) == bd.SV_ECAPACITY   # more than 2048 sequences
    assert call() == bd.SV_EWORKSPACE                        # workspace too small
    assert 'workspace' in L.sv_last_error().decode()


def test_attention_kv8_validation():
    L = bd.lib()
    b = _batch()
    args = dict(q=16, kc=16, ks=16, vs=16, P=64, D=128, Hq=32, Hkv=8, ws=16, wsn=1 << 30)

    def call(**kw):
        a = {**args, **kw}
        return L.spec_verify_attention_kv8(
            ctypes.byref(b), a['q'], 16, 16, a['kc'], 16, a['ks'], a['vs'], 16, 4, 8, a['P'],
            16, 16, a['Hq'], a['Hkv'], a['D'], 0.0, a['ws'], a['wsn'], None, None)
    assert call(ks=None) == bd.SV_EINVAL
    assert 'scale' in L.sv_last_error().decode()
    assert call(vs=None) == bd.SV_EINVAL
    assert call(ks=20) == bd.SV_EINVAL                       # misaligned scales
    assert call(kc=24) == bd.SV_EINVAL                       # misaligned pool
    assert call(D=96) == bd.SV_EDTYPE
    assert call(P=48) == bd.SV_EINVAL
    assert call(Hq=30) == bd.SV_EINVAL
    assert call(ws=None) == bd.SV_EWORKSPACE
    assert 'spec_verify_attention_kv8' in L.sv_last_error().decode()


def test_step_rejects_int8_pages_with_fp32_activations():
    L = bd.lib()
    b = _batch()
    kinds = (ctypes.c_uint8 * 1)(1)
    cfg = bd.SvAttnConfig(32, 8, 128, 64, 8, 4, 16, bd.SV_F32, 0.0, bd.SV_KV_INT8)
    lay = (bd.SvAttnLayer * 1)(bd.SvAttnLayer(16, 16, 16, 16, 16, 16, 16, 16))
    acc = bd.SvAcceptArgs(0, bd.SV_BF16, 100, 16, None, 16, None, None)
    st = L.spec_verify_step(ctypes.byref(b), 1, kinds, ctypes.byref(cfg), lay, None, None,
                            ctypes.byref(acc), 16, 16, 16, 0, None, 16, 1 << 30, None, None)
    assert st == bd.SV_EDTYPE and 'INT8' in L.sv_last_error().decode()
    cfg.kv_format = 5
    st = L.spec_verify_step(ctypes.byref(b), 1, kinds, ctypes.byref(cfg), lay, None, None,
                            ctypes.byref(acc), 16, 16, 16, 0, None, 16, 1 << 30, None, None)
    assert st == bd.SV_EINVAL and 'kv_format' in L.sv_last_error().decode()


def test_gdn_validation():
    L = bd.lib()
    b = _batch()

    def call(mode=0, state=16, dk=128, dv=128, q=16, out=16, commit=16, slots=2,
             io=bd.SV_BF16, sdt=bd.SV_F32):
        return L.gdn_verify_commit(ctypes.byref(b), mode, state, sdt, None, slots, q,
                                   16, 16, io, 16, 16, commit, out, 4, dk, dv,
                                   None, None, None)
    assert call(dk=96) == bd.SV_EDTYPE
    assert call(dv=96) == bd.SV_EDTYPE
    assert call(state=None) == bd.SV_EINVAL
    assert call(mode=0, commit=None) == bd.SV_EINVAL         # commit_len required
    assert call(mode=1, q=None) == bd.SV_EINVAL              # q required
    assert call(mode=5) == bd.SV_EINVAL
    assert call(slots=1) == bd.SV_EINVAL                     # identity map needs B slots
    assert call(io=3) == bd.SV_EDTYPE
    assert call(io=bd.SV_F16) == bd.SV_EDTYPE                # fp16 is a state type only
    assert call(sdt=bd.SV_BF16) == bd.SV_EDTYPE
    assert 'state dtype' in L.sv_last_error().decode()
    assert call(state=20) == bd.SV_EINVAL                    # misaligned state
    assert call(q=24) == bd.SV_EINVAL                        # misaligned q
    assert 'aligned' in L.sv_last_error().decode()


def test_short_conv_validation():
    L = bd.lib()
    b = _batch()

    def call(mode=0, state=16, x=16, w=16, K=4, C=64, act=0, commit=16, out=16, slots=2,
             io=bd.SV_BF16):
        return L.short_conv_verify_commit(ctypes.byref(b), mode, state, None, slots, x, w,
                                          None, io, act, commit, out, C, K, None, None, None)
    assert call(K=1) == bd.SV_EINVAL
    assert call(K=9) == bd.SV_EINVAL
    assert call(C=0) == bd.SV_EINVAL
    assert call(act=2) == bd.SV_EINVAL
    assert call(io=2) == bd.SV_EDTYPE
    assert call(state=None) == bd.SV_EINVAL
    assert call(w=None) == bd.SV_EINVAL
    assert call(mode=0, commit=None) == bd.SV_EINVAL         # commit_len required
    assert call(mode=1, out=None) == bd.SV_EINVAL            # out required
    assert call(slots=1) == bd.SV_EINVAL                     # slots < B without a map
    assert call(mode=7) == bd.SV_EINVAL


def test_checkpoint_validation():
    L = bd.lib()
    b = _batch()                                             # max_T = 4

    def gv(window=4, ck=16, sdt=bd.SV_F32, out=16):
        return L.gdn_verify_checkpoint(ctypes.byref(b), 16, sdt, None, 2, 16, 16, 16, bd.SV_BF16,
                                       16, 16, out, ck, window, 4, 128, 128, None, None)
    assert gv(window=3) == bd.SV_EINVAL                      # window < max_T
    assert 'window' in L.sv_last_error().decode()
    assert gv(window=65) == bd.SV_EINVAL
    assert gv(ck=None) == bd.SV_EINVAL
    assert gv(ck=20) == bd.SV_EINVAL                         # misaligned series
    assert gv(out=None) == bd.SV_EINVAL
    assert gv(sdt=bd.SV_BF16) == bd.SV_EDTYPE

    def gc(window=4, commit=16):
        return L.gdn_commit_prefix(ctypes.byref(b), 16, bd.SV_F32, None, 2, 16, window, commit,
                                   4, 128, 128, None, None)
    assert gc(commit=None) == bd.SV_EINVAL
    assert gc(window=2) == bd.SV_EINVAL

    def cv(window=4, ps=16, K=4):
        return L.short_conv_verify_checkpoint(ctypes.byref(b), 16, None, 2, 16, 16, None,
                                              bd.SV_BF16, 0, 16, ps, window, 64, K, None, None)
    assert cv(ps=None) == bd.SV_EINVAL
    assert cv(window=1) == bd.SV_EINVAL
    assert cv(K=9) == bd.SV_EINVAL
    assert L.short_conv_commit_prefix(ctypes.byref(b), 16, None, 2, 16, 4, None, bd.SV_BF16, 64,
                                      4, None, None) == bd.SV_EINVAL


def test_accept_validation():
    L = bd.lib()
    b = _batch()

    def call(mode=1, target=16, draft=16, ua=16, uf=16, dt=None, res=16, ws=16,
             wsn=1 << 30, V=100, dtype=bd.SV_BF16):
        return L.spec_accept(ctypes.byref(b), mode, target, draft, dtype, V,
                             16 if dt is None else dt, ua, uf, res, None, None, ws,
                             wsn, None, None)
    assert call(ua=None) == bd.SV_EINVAL                     # rejection needs u_accept
    assert call(uf=None) == bd.SV_EINVAL
    assert call(mode=0, draft=None, ua=None, uf=None, wsn=4) == bd.SV_EWORKSPACE
    assert call(res=None) == bd.SV_EINVAL
    assert call(V=0) == bd.SV_EINVAL
    assert call(dtype=9) == bd.SV_EDTYPE
    assert call(mode=4) == bd.SV_EINVAL
    # the struct entry point validates the same way
    acc = bd.SvAcceptArgs(1, bd.SV_BF16, 100, 16, None, 16, None, 16, None)
    assert L.spec_accept_args(ctypes.byref(b), ctypes.byref(acc), 16, None, None, 16, 1 << 30,
                              None, None) == bd.SV_EINVAL
    assert L.spec_accept_args(ctypes.byref(b), None, 16, None, None, 16, 1 << 30,
                              None, None) == bd.SV_EINVAL


def test_step_validation():
    L = bd.lib()
    b = _batch()
    kinds = (ctypes.c_uint8 * 2)(0, 2)
    acc = bd.SvAcceptArgs(0, bd.SV_BF16, 100, 16, None, 16, None, None)
    st = L.spec_verify_step(ctypes.byref(b), 2, kinds, None, None, None, None,
                            ctypes.byref(acc), 16, 16, 16, 0, None, 16, 1 << 30,
                            None, None)
    assert st == bd.SV_EINVAL and 'layer_kind' in L.sv_last_error().decode()
    kinds = (ctypes.c_uint8 * 1)(1)
    st = L.spec_verify_step(ctypes.byref(b), 1, kinds, None, None, None, None,
                            ctypes.byref(acc), 16, 16, 16, 0, None, 16, 1 << 30,
                            None, None)
    assert st == bd.SV_EINVAL and 'attention' in L.sv_last_error().decode()


def _hybrid_step(L, last_gdn_q=16, k_scale=16, acc_res=16):
    """A 4-layer step (GDN, GDN, GDN, attention) with fake aligned pointers."""
    b = _batch()
    kinds = (ctypes.c_uint8 * 4)(0, 0, 0, 1)
    acfg = bd.SvAttnConfig(32, 8, 128, 64, 8, 4, 16, bd.SV_BF16, 0.0,
                           bd.SV_KV_INT8 if k_scale != 16 else bd.SV_KV_PLAIN)
    lay = (bd.SvAttnLayer * 1)(bd.SvAttnLayer(16, 16, 16, 16, 16, 16, k_scale, 16))
    gcfg = bd.SvGdnConfig(4, 128, 128, 2, None, bd.SV_BF16, bd.SV_F32)
    g = [bd.SvGdnLayer(16, 16, 16, 16, 16, 16, 16) for _ in range(2)]
    g.append(bd.SvGdnLayer(16, last_gdn_q, 16, 16, 16, 16, 16))
    gl = (bd.SvGdnLayer * 3)(*g)
    acc = bd.SvAcceptArgs(0, bd.SV_BF16, 100, 16, None, 16, None, None)
    return L.spec_verify_step(ctypes.byref(b), 4, kinds, ctypes.byref(acfg), lay,
                              ctypes.byref(gcfg), gl, ctypes.byref(acc), 16, acc_res, 16, 0,
                              None, 16, 1 << 30, None, None)


@pytest.mark.parametrize('bad,layer', [
    (dict(last_gdn_q=24), 'layer 2'),        # misaligned q of the last GDN layer
    (dict(k_scale=None), 'layer 3'),         # INT8 attention layer without scales
    (dict(acc_res=None), 'result'),          # acceptance output missing
])
def test_step_checks_every_layer_before_any_launch(bad, layer):
    """A refused step returns before its first launch: on a host without a GPU
    any launch would fail with SV_EHIP, so a host-side refusal of the last
    layer (or of the acceptance) proves no earlier layer was launched."""
    L = bd.lib()
    st = _hybrid_step(L, **bad)
    assert st in (bd.SV_EINVAL, bd.SV_EDTYPE), L.sv_last_error().decode()
    assert layer in L.sv_last_error().decode()


def _flush(L, n=3, bad_layer=None, bad=None, conv_C=0, pending=True, commit=16):
    """spec_verify_flush over n GDN layers with fake aligned pointers; layer
    bad_layer gets the fields in `bad`."""
    gcfg = bd.SvGdnConfig(4, 128, 128, 2, None, bd.SV_BF16, bd.SV_F32, conv_C, 4, 0)
    layers = []
    for i in range(n):
        f = dict(state=16, q=None, k=16, v=16, alpha=16, beta=16, out=None,
                 conv_state=16, conv_x=16)
        if i == bad_layer:
            f.update(bad)
        layers.append(bd.SvGdnLayer(f['state'], f['q'], f['k'], f['v'], f['alpha'],
                                    f['beta'], f['out'], f['conv_state'], f['conv_x']))
    arr = (bd.SvGdnLayer * max(1, n))(*layers)
    p = bd.SvStepPending(_batch(), arr, commit)
    return L.spec_verify_flush(n, ctypes.byref(gcfg), ctypes.byref(p) if pending else None,
                               None, None)


@pytest.mark.parametrize('kw,msg', [
    (dict(n=-1), 'n_gdn'),
    (dict(pending=False), 'pending is required'),
    (dict(commit=None), 'commit_len'),
    (dict(bad_layer=2, bad=dict(k=24)), 'layer 2'),          # misaligned k, last layer
    (dict(bad_layer=2, bad=dict(alpha=None)), 'layer 2'),
    (dict(bad_layer=1, bad=dict(state=None)), 'layer 1'),
    (dict(bad_layer=2, bad=dict(conv_x=None), conv_C=64), 'layer 2'),
])
def test_flush_validation(kw, msg):
    """Refusals come before the first launch: on a host without a GPU a
    launch would return SV_EHIP, so a refusal of the last layer shows that
    no earlier layer was committed."""
    L = bd.lib()
    st = _flush(L, **kw)
    assert st == bd.SV_EINVAL, L.sv_last_error().decode()
    assert msg in L.sv_last_error().decode()


def test_flush_of_no_layers_is_a_no_op():
    L = bd.lib()
    assert _flush(L, n=0) == bd.SV_OK


def test_device_error_calls_validate():
    L = bd.lib()
    assert L.sv_read_device_error(None, None) == -1
    assert 'null' in L.sv_last_error().decode()
    assert L.sv_clear_device_error(None, None) == bd.SV_EINVAL


def test_aggregate_workspace_covers_every_call():
    L = bd.lib()
    B, T, Hq, Hkv, D, V, mp = 64, 4, 32, 8, 128, 151936, 130
    agg = L.sv_workspace_bytes(B, T, Hq, D, V, mp)
    for dt in (bd.SV_BF16, bd.SV_F32):
        assert agg >= L.spec_verify_attention_workspace_bytes(B, B * T, Hq, Hkv, D, mp, 64, dt)
    for mode in (bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION):
        assert agg >= L.spec_accept_workspace_bytes(B, B * T, V, mode)
    assert L.sv_workspace_bytes(B, 9, Hq, D, V, mp) == 0          # max_T beyond the limit
    assert L.sv_workspace_bytes(0, T, Hq, D, V, mp) == 0


def test_workspace_sizes_are_consistent():
    L = bd.lib()
    a = L.spec_verify_attention_workspace_bytes(64, 256, 32, 8, 128, 130, 64, bd.SV_BF16)
    assert a > 256 * 32 * 128 * 4
    assert L.spec_verify_attention_workspace_bytes(64, 256, 32, 8, 128, 130, 64, bd.SV_F32) == 0
    g = L.spec_accept_workspace_bytes(64, 256, 151936, bd.SV_ACCEPT_GREEDY)
    r = L.spec_accept_workspace_bytes(64, 256, 151936, bd.SV_ACCEPT_REJECTION)
    assert 0 < g < r


def test_step_layers_are_checked_against_their_configuration():
    """The binding refuses step layers whose pools or states do not have the
    configured element type or shape (the library sees only pointers, so an
    INT8 pool under a bf16 configuration would be read out of bounds)."""
    import types

    import torch
    B, H, dk, dv, Hq, Hkv, D, P, pages = 2, 2, 64, 64, 4, 2, 64, 16, 6

    def attn(cache_dtype, act=torch.bfloat16, shape=(pages, Hkv, P, D), scales=False):
        t = dict(q=torch.zeros(8, Hq, D, dtype=act), k_new=torch.zeros(8, Hkv, D, dtype=act),
                 v_new=torch.zeros(8, Hkv, D, dtype=act), out=torch.zeros(8, Hq, D, dtype=act),
                 k_cache=torch.zeros(shape, dtype=cache_dtype),
                 v_cache=torch.zeros(shape, dtype=cache_dtype),
                 k_scale=torch.ones(Hkv, D) if scales else None,
                 v_scale=torch.ones(Hkv, D) if scales else None)
        return types.SimpleNamespace(tensors=t)

    def gdn(state_dtype=torch.float32, io=torch.bfloat16, slots=B):
        t = dict(state=torch.zeros(slots, H, dv, dk, dtype=state_dtype),
                 q=torch.zeros(8, H, dk, dtype=io), k=torch.zeros(8, H, dk, dtype=io),
                 v=torch.zeros(8, H, dv, dtype=io), out=torch.zeros(8, H, dv, dtype=io),
                 alpha=torch.ones(8, H), beta=torch.ones(8, H),
                 conv_state=None, conv_x=None, conv_out=None)
        return types.SimpleNamespace(tensors=t)

    cfg = bd.SvAttnConfig(Hq, Hkv, D, P, pages, 4, None, bd.SV_BF16, 0.0, bd.SV_KV_PLAIN)
    cfg8 = bd.SvAttnConfig(Hq, Hkv, D, P, pages, 4, None, bd.SV_BF16, 0.0, bd.SV_KV_INT8)
    gcfg = bd.SvGdnConfig(H, dk, dv, B, None, bd.SV_BF16, bd.SV_F32)
    gcfg16 = bd.SvGdnConfig(H, dk, dv, B, None, bd.SV_BF16, bd.SV_F16)
    bd._check_step_layers(cfg, [attn(torch.bfloat16)], gcfg, [gdn()])        # consistent
    bd._check_step_layers(cfg8, [attn(torch.int8, scales=True)], gcfg16,
                          [gdn(torch.float16)])
    for args, msg in [
        ((cfg, [attn(torch.int8)], gcfg, []), 'k_cache must be torch.bfloat16'),
        ((cfg8, [attn(torch.bfloat16, scales=True)], gcfg, []), 'k_cache must be torch.int8'),
        ((cfg8, [attn(torch.int8)], gcfg, []), 'k_scale'),
        ((cfg, [attn(torch.bfloat16, shape=(pages, Hkv, 2 * P, D))], gcfg, []), 'page_size'),
        ((cfg, [attn(torch.bfloat16, act=torch.float32)], gcfg, []), 'q must be'),
        ((cfg, [], gcfg, [gdn(torch.float16)]), 'state must be torch.float32'),
        ((cfg, [], gcfg16, [gdn()]), 'state must be torch.float16'),
        ((cfg, [], gcfg, [gdn(io=torch.float32)]), 'q must be torch.bfloat16'),
        ((cfg, [], gcfg, [gdn(slots=1)]), 'state must be'),
    ]:
        with pytest.raises(ValueError, match=msg):
            bd._check_step_layers(*args)


def test_binding_refuses_cpu_tensors():
    import torch
    b = _batch()
    with pytest.raises((ValueError, RuntimeError)):
        bd.spec_accept(b, 0, torch.zeros(8, 100, dtype=torch.bfloat16),
                       torch.zeros(6, dtype=torch.int32),
                       torch.zeros(10, dtype=torch.int32))
