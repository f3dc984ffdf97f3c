"""Thin ctypes binding of ``libspecverify.so`` (see ``include/spec_verify.h``).

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the computation runs in the HIP
kernels.  There is no fallback: if the library is missing, or a call is made
with tensors that are not on the GPU, the call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, 'libspecverify.so')

SV_OK, SV_EINVAL, SV_EDTYPE, SV_ECAPACITY, SV_EWORKSPACE, SV_EHIP = range(6)
SV_F32, SV_BF16, SV_F16 = 0, 1, 2
SV_GDN_VERIFY_COMMIT, SV_GDN_VERIFY_ONLY, SV_GDN_COMMIT_ONLY = 0, 1, 2
SV_ACCEPT_GREEDY, SV_ACCEPT_REJECTION = 0, 1
SV_SCHEDULE_TWO_PHASE, SV_SCHEDULE_DEFERRED = 0, 1
SV_KV_PLAIN, SV_KV_INT8 = 0, 1
SV_ACT_NONE, SV_ACT_SILU = 0, 1
SV_DERR = {1: 'PAGE', 2: 'CAPACITY', 4: 'SEQLEN', 8: 'COMMIT', 16: 'TOKEN',
           32: 'SLOT'}

_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class SvBatch(ctypes.Structure):
    _fields_ = [('B', _c_i32), ('max_T', _c_i32), ('total_T', _c_i32),
                ('cu_seqlens', _vp)]


class SvGdnPending(ctypes.Structure):
    _fields_ = [('batch', SvBatch), ('k', _vp), ('v', _vp), ('alpha', _vp),
                ('beta', _vp), ('commit_len', _vp)]


class SvConvPending(ctypes.Structure):
    _fields_ = [('batch', SvBatch), ('x', _vp), ('commit_len', _vp)]


class SvAttnLayer(ctypes.Structure):
    _fields_ = [('q', _vp), ('k_new', _vp), ('v_new', _vp), ('k_cache', _vp),
                ('v_cache', _vp), ('out', _vp), ('k_scale', _vp), ('v_scale', _vp)]


class SvGdnLayer(ctypes.Structure):
    _fields_ = [('state', _vp), ('q', _vp), ('k', _vp), ('v', _vp),
                ('alpha', _vp), ('beta', _vp), ('out', _vp),
                ('conv_state', _vp), ('conv_x', _vp), ('conv_out', _vp),
                ('conv_weight', _vp), ('conv_bias', _vp)]


class SvAttnConfig(ctypes.Structure):
    _fields_ = [('Hq', _c_i32), ('Hkv', _c_i32), ('D', _c_i32),
                ('page_size', _c_i32), ('num_pages', _c_i32),
                ('max_pages_per_seq', _c_i32), ('block_table', _vp),
                ('dtype', ctypes.c_int), ('scale', ctypes.c_float),
                ('kv_format', ctypes.c_int)]


class SvGdnConfig(ctypes.Structure):
    _fields_ = [('H', _c_i32), ('dk', _c_i32), ('dv', _c_i32),
                ('num_slots', _c_i32), ('state_slot', _vp),
                ('io_dtype', ctypes.c_int), ('state_dtype', ctypes.c_int),
                ('conv_C', _c_i32), ('conv_K', _c_i32), ('conv_activation', _c_i32)]


class SvAcceptArgs(ctypes.Structure):
    _fields_ = [('mode', ctypes.c_int), ('logit_dtype', ctypes.c_int),
                ('V', _c_i32), ('target_logits', _vp), ('draft_logits', _vp),
                ('draft_tokens', _vp), ('u_accept', _vp), ('u_final', _vp),
                ('bonus_tokens', _vp)]


class SvStepPending(ctypes.Structure):
    _fields_ = [('batch', SvBatch), ('layers', ctypes.POINTER(SvGdnLayer)),
                ('commit_len', _vp)]


_SIGS = {
    'sv_last_error': ([], ctypes.c_char_p),
    'sv_workspace_bytes': ([_c_i32] * 6, _sz),
    'sv_read_device_error': ([_vp, _vp], _c_i32),
    'sv_clear_device_error': ([_vp, _vp], ctypes.c_int),
    'sv_version': ([], ctypes.c_char_p),
    'spec_verify_attention_workspace_bytes': (
        [_c_i32] * 7 + [ctypes.c_int], _sz),
    'spec_verify_attention': (
        [ctypes.POINTER(SvBatch), _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32,
         _c_i32, _vp, _vp, _c_i32, _c_i32, _c_i32, ctypes.c_int,
         ctypes.c_float, _c_i32, _vp, _sz, _vp, _vp], ctypes.c_int),
    'spec_verify_attention_kv8': (
        [ctypes.POINTER(SvBatch), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32,
         _c_i32, _vp, _vp, _c_i32, _c_i32, _c_i32, ctypes.c_float, _vp, _sz, _vp, _vp],
        ctypes.c_int),
    'gdn_verify_commit': (
        [ctypes.POINTER(SvBatch), ctypes.c_int, _vp, ctypes.c_int, _vp, _c_i32, _vp,
         _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
         ctypes.POINTER(SvGdnPending), _vp, _vp], ctypes.c_int),
    'short_conv_verify_commit': (
        [ctypes.POINTER(SvBatch), ctypes.c_int, _vp, _vp, _c_i32, _vp, _vp, _vp,
         ctypes.c_int, _c_i32, _vp, _vp, _c_i32, _c_i32, ctypes.POINTER(SvConvPending),
         _vp, _vp], ctypes.c_int),
    'gdn_verify_checkpoint': (
        [ctypes.POINTER(SvBatch), _vp, ctypes.c_int, _vp, _c_i32, _vp, _vp, _vp, ctypes.c_int,
         _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp], ctypes.c_int),
    'gdn_commit_prefix': (
        [ctypes.POINTER(SvBatch), _vp, ctypes.c_int, _vp, _c_i32, _vp, _c_i32, _vp, _c_i32,
         _c_i32, _c_i32, _vp, _vp], ctypes.c_int),
    'short_conv_verify_checkpoint': (
        [ctypes.POINTER(SvBatch), _vp, _vp, _c_i32, _vp, _vp, _vp, ctypes.c_int, _c_i32, _vp,
         _vp, _c_i32, _c_i32, _c_i32, _vp, _vp], ctypes.c_int),
    'short_conv_commit_prefix': (
        [ctypes.POINTER(SvBatch), _vp, _vp, _c_i32, _vp, _c_i32, _vp, ctypes.c_int, _c_i32,
         _c_i32, _vp, _vp], ctypes.c_int),
    'spec_accept_workspace_bytes': ([_c_i32, _c_i32, _c_i32, ctypes.c_int], _sz),
    'spec_accept_args': (
        [ctypes.POINTER(SvBatch), ctypes.POINTER(SvAcceptArgs), _vp, _vp, _vp, _vp, _sz, _vp,
         _vp], ctypes.c_int),
    'spec_accept_noalloc': (
        [ctypes.POINTER(SvBatch), ctypes.POINTER(SvAcceptArgs), _vp, _vp, _vp, _vp, _vp],
        ctypes.c_int),
    'spec_accept': (
        [ctypes.POINTER(SvBatch), ctypes.c_int, _vp, _vp, ctypes.c_int, _c_i32,
         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp], ctypes.c_int),
    'spec_verify_step_workspace_bytes': (
        [ctypes.POINTER(SvBatch), ctypes.POINTER(SvAttnConfig),
         ctypes.POINTER(SvAcceptArgs)], _sz),
    'spec_verify_step': (
        [ctypes.POINTER(SvBatch), _c_i32, ctypes.POINTER(ctypes.c_uint8),
         ctypes.POINTER(SvAttnConfig), ctypes.POINTER(SvAttnLayer),
         ctypes.POINTER(SvGdnConfig), ctypes.POINTER(SvGdnLayer),
         ctypes.POINTER(SvAcceptArgs), _vp, _vp, _vp, ctypes.c_int,
         ctypes.POINTER(SvStepPending), _vp, _sz, _vp, _vp], ctypes.c_int),
    'spec_verify_flush': (
        [_c_i32, ctypes.POINTER(SvGdnConfig), ctypes.POINTER(SvStepPending), _vp, _vp],
        ctypes.c_int),
}

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status, text):
        super().__init__(f'status {status}: {text}')
        self.status = status


def lib():
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f'{LIB_PATH} is missing: build it with '
                '`python -m block_draft_verification_spec_amd.build`')
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status):
    if status != SV_OK:
        raise SpecVerifyError(status, lib().sv_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError('expected a torch tensor')
    if not t.is_cuda:
        raise ValueError('tensor must live on the GPU')
    if not t.is_contiguous():
        raise ValueError('tensor must be contiguous')
    return t.data_ptr()


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise ValueError(f'unsupported dtype {t.dtype}')


def _require(dtype, **tensors):
    """Every named tensor (None skipped) has `dtype`: the library sees only
    pointers, so a page pool or state of another element size would be read
    out of bounds."""
    for name, t in tensors.items():
        if t is not None and t.dtype != dtype:
            raise ValueError(f'{name} must be {dtype}, not {t.dtype}')


def _pool_shape(k_cache, v_cache, Hkv, D):
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or \
            k_cache.shape[1] != Hkv or k_cache.shape[3] != D:
        raise ValueError(f'page pools must both be [num_pages, {Hkv}, page_size, {D}], '
                         f'not {tuple(k_cache.shape)} and {tuple(v_cache.shape)}')


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _i32(t, name):
    if t is not None and t.dtype != torch.int32:
        raise ValueError(f'{name} must be int32')
    return _ptr(t)


def make_batch(cu_seqlens, B, max_T, total_T):
    """sv_batch from a device int32 ``cu_seqlens`` and host sizes."""
    return SvBatch(int(B), int(max_T), int(total_T), _i32(cu_seqlens, 'cu_seqlens'))


def version():
    return lib().sv_version().decode()


def sv_workspace_bytes(B, max_T, Hq, D, V, max_pages_per_seq):
    """One workspace size for every call of such a batch (``sv_workspace_bytes``)."""
    return lib().sv_workspace_bytes(B, max_T, Hq, D, V, max_pages_per_seq)


def read_device_error(err, stream=None):
    """The device error word after the stream's work (``sv_read_device_error``)."""
    v = lib().sv_read_device_error(_i32(err, 'err'), _stream(stream))
    if v < 0:
        raise SpecVerifyError(SV_EHIP, lib().sv_last_error().decode())
    return v


def clear_device_error(err, stream=None):
    """Enqueue the zeroing of the device error word (``sv_clear_device_error``)."""
    _check(lib().sv_clear_device_error(_i32(err, 'err'), _stream(stream)))


def spec_verify_attention_workspace_bytes(B, total_T, Hq, Hkv, D,
                                          max_pages_per_seq, page_size, dtype):
    return lib().spec_verify_attention_workspace_bytes(
        B, total_T, Hq, Hkv, D, max_pages_per_seq, page_size, dtype)


def spec_verify_attention(batch, q, k_new, v_new, k_cache, v_cache,
                          block_table, ctx_lens, out, scale=0.0, write_kv=True,
                          workspace=None, err=None, stream=None):
    """Paged verification attention (``spec_verify_attention``).

    Shapes: q/out [total_T, Hq, D]; k_new/v_new [total_T, Hkv, D];
    caches [num_pages, Hkv, P, D]; block_table int32 [B, max_pages];
    ctx_lens int32 [B].
    """
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_new.shape[1]
    _require(q.dtype, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, out=out)
    _pool_shape(k_cache, v_cache, Hkv, D)
    num_pages, P = k_cache.shape[0], k_cache.shape[2]
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().spec_verify_attention(
        ctypes.byref(batch), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), _i32(block_table, 'block_table'), block_table.shape[1],
        num_pages, P, _i32(ctx_lens, 'ctx_lens'), _ptr(out), Hq, Hkv, D,
        _dtype(q), float(scale), int(bool(write_kv)), _ptr(workspace), ws_n,
        _i32(err, 'err'), _stream(stream)))


def spec_verify_attention_kv8(batch, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                              block_table, ctx_lens, out, scale=0.0, workspace=None, err=None,
                              stream=None):
    """Verification attention over INT8 pages (``spec_verify_attention_kv8``).

    q/k_new/v_new/out bf16 as for ``spec_verify_attention``; caches int8
    [num_pages, Hkv, P, D]; k_scale / v_scale fp32 [Hkv, D].
    """
    if k_cache.dtype != torch.int8 or v_cache.dtype != torch.int8:
        raise ValueError('INT8 pages must be torch.int8')
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32:
        raise ValueError('scales must be float32')
    _require(torch.bfloat16, q=q, k_new=k_new, v_new=v_new, out=out)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_new.shape[1]
    _pool_shape(k_cache, v_cache, Hkv, D)
    num_pages, P = k_cache.shape[0], k_cache.shape[2]
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().spec_verify_attention_kv8(
        ctypes.byref(batch), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _i32(block_table, 'block_table'), block_table.shape[1],
        num_pages, P, _i32(ctx_lens, 'ctx_lens'), _ptr(out), Hq, Hkv, D, float(scale),
        _ptr(workspace), ws_n, _i32(err, 'err'), _stream(stream)))


def gdn_verify_commit(batch, mode, state, q, k, v, alpha, beta, commit_len,
                      out, state_slot=None, pending=None, err=None,
                      stream=None):
    """GDN verify / commit (``gdn_verify_commit``).

    state fp32 or fp16 [num_slots, H, dv, dk]; q/k [total_T, H, dk]; v/out
    [total_T, H, dv]; alpha/beta fp32 [total_T, H]; commit_len int32 [B].
    ``pending``: an ``SvGdnPending`` or None.
    """
    num_slots, H, dv, dk = state.shape
    _require(k.dtype, q=q, v=v, out=out)
    _require(torch.float32, alpha=alpha, beta=beta)
    _check(lib().gdn_verify_commit(
        ctypes.byref(batch), int(mode), _ptr(state), state_dtype(state),
        _i32(state_slot, 'state_slot'),
        num_slots, _ptr(q), _ptr(k), _ptr(v), _dtype(k), _ptr(alpha), _ptr(beta),
        _i32(commit_len, 'commit_len'), _ptr(out), H, dk, dv,
        ctypes.byref(pending) if pending is not None else None,
        _i32(err, 'err'), _stream(stream)))


def make_gdn_pending(batch, k, v, alpha, beta, commit_len):
    return SvGdnPending(batch, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                        _i32(commit_len, 'commit_len'))


def short_conv_verify_commit(batch, mode, state, x, weight, bias, commit_len, out,
                             state_slot=None, activation=SV_ACT_NONE, pending=None, err=None,
                             stream=None):
    """Short causal convolution verify / commit (``short_conv_verify_commit``).

    state [num_slots, K-1, C] and x / out [total_T, C] in one I/O dtype;
    weight fp32 [C, K]; bias fp32 [C] or None; commit_len int32 [B].
    ``pending``: an ``SvConvPending`` or None.
    """
    num_slots, Km1, C = state.shape
    if weight.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise ValueError('weight and bias must be float32')
    _check(lib().short_conv_verify_commit(
        ctypes.byref(batch), int(mode), _ptr(state), _i32(state_slot, 'state_slot'),
        num_slots, _ptr(x), _ptr(weight), _ptr(bias), _dtype(x), int(activation),
        _i32(commit_len, 'commit_len'), _ptr(out), C, Km1 + 1,
        ctypes.byref(pending) if pending is not None else None,
        _i32(err, 'err'), _stream(stream)))


def make_conv_pending(batch, x, commit_len):
    return SvConvPending(batch, _ptr(x), _i32(commit_len, 'commit_len'))


def gdn_verify_checkpoint(batch, state, q, k, v, alpha, beta, out, checkpoints,
                          state_slot=None, err=None, stream=None):
    """Verify writing the checkpoint series (``gdn_verify_checkpoint``).

    checkpoints [B, window, H, dv, dk] in the state's dtype; the state bank is
    read only.
    """
    num_slots, H, dv, dk = state.shape
    if checkpoints.dtype != state.dtype:
        raise ValueError('checkpoints must have the state dtype')
    _check(lib().gdn_verify_checkpoint(
        ctypes.byref(batch), _ptr(state), state_dtype(state), _i32(state_slot, 'state_slot'),
        num_slots, _ptr(q), _ptr(k), _ptr(v), _dtype(k), _ptr(alpha), _ptr(beta), _ptr(out),
        _ptr(checkpoints), checkpoints.shape[1], H, dk, dv, _i32(err, 'err'), _stream(stream)))


def gdn_commit_prefix(batch, state, checkpoints, commit_len, state_slot=None, err=None,
                      stream=None):
    """CommitPrefix over a GatedDeltaNet checkpoint series (``gdn_commit_prefix``)."""
    num_slots, H, dv, dk = state.shape
    if checkpoints.dtype != state.dtype:
        raise ValueError('checkpoints must have the state dtype')
    _check(lib().gdn_commit_prefix(
        ctypes.byref(batch), _ptr(state), state_dtype(state), _i32(state_slot, 'state_slot'),
        num_slots, _ptr(checkpoints), checkpoints.shape[1], _i32(commit_len, 'commit_len'), H,
        dk, dv, _i32(err, 'err'), _stream(stream)))


def short_conv_verify_checkpoint(batch, state, x, weight, bias, out, prefix_states,
                                 state_slot=None, activation=SV_ACT_NONE, err=None,
                                 stream=None):
    """Short-conv verify writing the prefix-state series
    (``short_conv_verify_checkpoint``); prefix_states [B, window, K-1, C]."""
    num_slots, Km1, C = state.shape
    _check(lib().short_conv_verify_checkpoint(
        ctypes.byref(batch), _ptr(state), _i32(state_slot, 'state_slot'), num_slots, _ptr(x),
        _ptr(weight), _ptr(bias), _dtype(x), int(activation), _ptr(out), _ptr(prefix_states),
        prefix_states.shape[1], C, Km1 + 1, _i32(err, 'err'), _stream(stream)))


def short_conv_commit_prefix(batch, state, prefix_states, commit_len, state_slot=None,
                             err=None, stream=None):
    """CommitPrefix over the conv's prefix-state series (``short_conv_commit_prefix``)."""
    num_slots, Km1, C = state.shape
    _check(lib().short_conv_commit_prefix(
        ctypes.byref(batch), _ptr(state), _i32(state_slot, 'state_slot'), num_slots,
        _ptr(prefix_states), prefix_states.shape[1], _i32(commit_len, 'commit_len'),
        _dtype(state), C, Km1 + 1, _i32(err, 'err'), _stream(stream)))


def spec_accept_workspace_bytes(B, total_T, V, mode):
    return lib().spec_accept_workspace_bytes(B, total_T, V, mode)


def spec_accept(batch, mode, target_logits, draft_tokens, result,
                draft_logits=None, u_accept=None, u_final=None,
                commit_len_out=None, ctx_lens_inout=None, workspace=None,
                err=None, stream=None, bonus_tokens=None):
    """Acceptance.  ``result`` int32 [B * (1 + max_T)].  Rejection without
    ``draft_logits`` treats each draft as a point mass; ``bonus_tokens``
    (int32 [B]) goes through ``spec_accept_args``."""
    V = target_logits.shape[1]
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if bonus_tokens is not None:
        acc = accept_args(mode, target_logits, draft_tokens, draft_logits, u_accept, u_final,
                          bonus_tokens)
        _check(lib().spec_accept_args(
            ctypes.byref(batch), ctypes.byref(acc), _i32(result, 'result'),
            _i32(commit_len_out, 'commit_len_out'), _i32(ctx_lens_inout, 'ctx_lens'),
            _ptr(workspace), ws_n, _i32(err, 'err'), _stream(stream)))
        return
    _check(lib().spec_accept(
        ctypes.byref(batch), int(mode), _ptr(target_logits), _ptr(draft_logits),
        _dtype(target_logits), V, _i32(draft_tokens, 'draft_tokens'),
        _ptr(u_accept), _ptr(u_final), _i32(result, 'result'),
        _i32(commit_len_out, 'commit_len_out'), _i32(ctx_lens_inout, 'ctx_lens'),
        _ptr(workspace), ws_n, _i32(err, 'err'), _stream(stream)))


def spec_accept_noalloc(batch, mode, target_logits, draft_tokens, result, draft_logits=None,
                        u_accept=None, u_final=None, commit_len_out=None, ctx_lens_inout=None,
                        err=None, stream=None, bonus_tokens=None):
    """Acceptance with the library's own scratch (``spec_accept_noalloc``): no
    workspace argument, nothing allocated."""
    acc = accept_args(mode, target_logits, draft_tokens, draft_logits, u_accept, u_final,
                      bonus_tokens)
    _check(lib().spec_accept_noalloc(
        ctypes.byref(batch), ctypes.byref(acc), _i32(result, 'result'),
        _i32(commit_len_out, 'commit_len_out'), _i32(ctx_lens_inout, 'ctx_lens'),
        _i32(err, 'err'), _stream(stream)))


_TORCH_DTYPE = {SV_F32: torch.float32, SV_BF16: torch.bfloat16, SV_F16: torch.float16}


def _check_step_layers(attn_cfg, attn_layers, gdn_cfg, gdn_layers):
    """The step's layers against its configurations (layers made by attn_layer
    and gdn_layer carry their tensors): page pools of the configured format
    and shape, activations and states of the configured dtypes."""
    for i, lay in enumerate(attn_layers):
        t = getattr(lay, 'tensors', None)
        if t is None or attn_cfg is None:
            continue
        int8 = attn_cfg.kv_format == SV_KV_INT8
        act = torch.bfloat16 if int8 else _TORCH_DTYPE.get(attn_cfg.dtype)
        try:
            _require(act, q=t['q'], k_new=t['k_new'], v_new=t['v_new'], out=t['out'])
            _require(torch.int8 if int8 else act, k_cache=t['k_cache'], v_cache=t['v_cache'])
            _pool_shape(t['k_cache'], t['v_cache'], attn_cfg.Hkv, attn_cfg.D)
            if t['k_cache'].shape[0] != attn_cfg.num_pages or \
                    t['k_cache'].shape[2] != attn_cfg.page_size:
                raise ValueError('page pools do not match num_pages / page_size')
            if int8:
                if t['k_scale'] is None or t['v_scale'] is None:
                    raise ValueError('INT8 pages need k_scale and v_scale')
                _require(torch.float32, k_scale=t['k_scale'], v_scale=t['v_scale'])
        except ValueError as e:
            raise ValueError(f'attention layer {i}: {e}') from None
    for i, lay in enumerate(gdn_layers):
        t = getattr(lay, 'tensors', None)
        if t is None or gdn_cfg is None:
            continue
        io = _TORCH_DTYPE.get(gdn_cfg.io_dtype)
        try:
            _require(_TORCH_DTYPE.get(gdn_cfg.state_dtype), state=t['state'])
            _require(io, q=t['q'], k=t['k'], v=t['v'], out=t['out'], conv_state=t['conv_state'],
                     conv_x=t['conv_x'], conv_out=t['conv_out'])
            _require(torch.float32, alpha=t['alpha'], beta=t['beta'])
            if tuple(t['state'].shape[1:]) != (gdn_cfg.H, gdn_cfg.dv, gdn_cfg.dk) or \
                    t['state'].shape[0] < gdn_cfg.num_slots:
                raise ValueError(f'state must be [{gdn_cfg.num_slots}, {gdn_cfg.H}, '
                                 f'{gdn_cfg.dv}, {gdn_cfg.dk}], not {tuple(t["state"].shape)}')
        except ValueError as e:
            raise ValueError(f'GDN layer {i}: {e}') from None


class StepArgs:
    """Host-side structures of one ``spec_verify_step`` call.

    Keeps the ctypes arrays alive for as long as the object lives (the call
    reads them only while it enqueues, so they can be reused step to step).
    """

    def __init__(self, layer_kind, attn_cfg, attn_layers, gdn_cfg, gdn_layers,
                 accept_args):
        _check_step_layers(attn_cfg, attn_layers, gdn_cfg, gdn_layers)
        self.layer_kind = (ctypes.c_uint8 * len(layer_kind))(*layer_kind)
        self.n_layers = len(layer_kind)
        self.attn_cfg = attn_cfg
        self.attn = (SvAttnLayer * max(1, len(attn_layers)))(*attn_layers)
        self.gdn_cfg = gdn_cfg
        self.gdn = (SvGdnLayer * max(1, len(gdn_layers)))(*gdn_layers)
        self.acc = accept_args


def attn_config(Hq, Hkv, D, page_size, num_pages, block_table, dtype, scale=0.0,
                kv_format=SV_KV_PLAIN):
    return SvAttnConfig(Hq, Hkv, D, page_size, num_pages, block_table.shape[1],
                        _i32(block_table, 'block_table'), dtype, float(scale), kv_format)


def state_dtype(state):
    """The ``sv_dtype`` of a recurrent-state tensor (fp32 or fp16)."""
    if state.dtype == torch.float32:
        return SV_F32
    if state.dtype == torch.float16:
        return SV_F16
    raise ValueError(f'state must be float32 or float16, not {state.dtype}')


def gdn_config(H, dk, dv, num_slots, io_dtype, state_slot=None, state_dtype=SV_F32,
               conv_C=0, conv_K=0, conv_activation=SV_ACT_NONE):
    """GDN layer shapes of the step; conv_C > 0 runs every GDN layer's short
    convolution (width conv_K) in the step too."""
    return SvGdnConfig(H, dk, dv, num_slots, _i32(state_slot, 'state_slot'), io_dtype,
                       state_dtype, int(conv_C), int(conv_K), int(conv_activation))


def attn_layer(q, k_new, v_new, k_cache, v_cache, out, k_scale=None, v_scale=None):
    """One attention layer of the step (its tensors' dtypes and pool shapes are
    checked against the step's attention configuration in StepArgs)."""
    lay = SvAttnLayer(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                      _ptr(v_cache), _ptr(out), _ptr(k_scale), _ptr(v_scale))
    lay.tensors = dict(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                       out=out, k_scale=k_scale, v_scale=v_scale)
    return lay


def gdn_layer(state, q, k, v, alpha, beta, out, conv=None):
    """One GDN layer of the step; conv: None, or a dict with the layer's short
    convolution tensors 'state', 'x', 'out', 'weight', 'bias' (bias may be
    None)."""
    c = conv or {}
    if c and (c['weight'].dtype != torch.float32 or
              (c.get('bias') is not None and c['bias'].dtype != torch.float32)):
        raise ValueError('conv weight and bias must be float32')
    lay = SvGdnLayer(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                     _ptr(beta), _ptr(out), _ptr(c.get('state')), _ptr(c.get('x')),
                     _ptr(c.get('out')), _ptr(c.get('weight')), _ptr(c.get('bias')))
    lay.tensors = dict(state=state, q=q, k=k, v=v, alpha=alpha, beta=beta, out=out,
                       conv_state=c.get('state'), conv_x=c.get('x'), conv_out=c.get('out'))
    return lay


def accept_args(mode, target_logits, draft_tokens, draft_logits=None,
                u_accept=None, u_final=None, bonus_tokens=None):
    return SvAcceptArgs(int(mode), _dtype(target_logits), target_logits.shape[1],
                        _ptr(target_logits), _ptr(draft_logits),
                        _i32(draft_tokens, 'draft_tokens'), _ptr(u_accept),
                        _ptr(u_final), _i32(bonus_tokens, 'bonus_tokens'))


def spec_verify_step_workspace_bytes(batch, step_args):
    a = step_args
    has_attn = any(k == 1 for k in a.layer_kind)
    return lib().spec_verify_step_workspace_bytes(
        ctypes.byref(batch), ctypes.byref(a.attn_cfg) if has_attn else None,
        ctypes.byref(a.acc))


def spec_verify_step(batch, step_args, ctx_lens, result, commit_len,
                     schedule=SV_SCHEDULE_TWO_PHASE, pending=None,
                     workspace=None, err=None, stream=None):
    """The whole step (``spec_verify_step``).  ``pending``: SvStepPending."""
    a = step_args
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().spec_verify_step(
        ctypes.byref(batch), a.n_layers, a.layer_kind,
        ctypes.byref(a.attn_cfg) if a.attn_cfg is not None else None, a.attn,
        ctypes.byref(a.gdn_cfg) if a.gdn_cfg is not None else None, a.gdn,
        ctypes.byref(a.acc), _i32(ctx_lens, 'ctx_lens'), _i32(result, 'result'),
        _i32(commit_len, 'commit_len'), int(schedule),
        ctypes.byref(pending) if pending is not None else None,
        _ptr(workspace), ws_n, _i32(err, 'err'), _stream(stream)))


def step_pending(batch, step_args, commit_len):
    """The deferred schedule's pending tokens (``sv_step_pending``): the GDN
    layers of a step that ran with ``step_args`` on ``batch``, and the commit
    lengths it returned.  The structure keeps ``step_args`` alive."""
    p = SvStepPending(batch, step_args.gdn, _i32(commit_len, 'commit_len'))
    p.keep = step_args
    return p


def spec_verify_flush(step_args, pending, err=None, stream=None):
    """Commit the pending tokens of every GDN layer (``spec_verify_flush``):
    ``step_args`` gives the GDN configuration and layer count."""
    a = step_args
    n_gdn = sum(1 for k in a.layer_kind if k == 0)
    _check(lib().spec_verify_flush(
        n_gdn, ctypes.byref(a.gdn_cfg) if a.gdn_cfg is not None else None,
        ctypes.byref(pending), _i32(err, 'err'), _stream(stream)))
