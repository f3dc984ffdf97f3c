"""Oracle for one whole block speculative-verification step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Order of the step (lmdeploy PR 5019, feature list: the executor splits the
target pass from the speculative round, whose recurrent-state commit runs
after acceptance; onnxruntime-genai PR 2457: direct commit of the accepted
prefix out of the wide verify, with the verify-row argmax read back once):

1. every layer in model order runs its verify pass on the ``T_b`` in-flight
   tokens: attention layers write the in-flight K/V through into their pages
   and attend; GDN layers produce outputs from the untouched state, and so
   does the short convolution of a GDN layer that has one (a separate
   operator with its own rolling state: onnxruntime-genai PR 2457, commit
   message on the ``VarlenCausalConvWithState`` and ``GatedDeltaNet`` state
   series);
2. acceptance turns the supplied logits into ``accept_len`` and the output
   token rows;
3. ``commit_len = accept_len + 1`` (verify token 0 is the previous round's
   committed token, so a sequence keeps ``a_b + 1`` tokens), every GDN layer
   (and its convolution) stores the state after its first ``commit_len``
   tokens, and
   ``ctx_lens += commit_len`` (the KV commit is a length update only: slots
   past the new length are simply stale).
"""

import numpy as np

from .accept import greedy_accept, rejection_accept
from .attention import append_kv, verify_attention
from .gdn import GDN_COMMIT_ONLY, GDN_VERIFY_ONLY, gdn_step
from .short_conv import CONV_COMMIT_ONLY, CONV_VERIFY_ONLY, conv_step


def verify_step(layers, cu_seqlens, ctx_lens, block_table, page_size, max_T,
                accept_mode, accept_inputs, state_slot=None):
    """Run the step.

    layers        list of dicts in model order, each either
                  ``{'kind': 'attn', 'q', 'k_new', 'v_new', 'k_cache',
                  'v_cache'[, 'scale']}`` or ``{'kind': 'gdn', 'state', 'q',
                  'k', 'v', 'alpha', 'beta'[, 'conv']}``, ``conv`` being the
                  layer's short convolution ``{'state', 'x', 'weight',
                  'bias', 'silu'}``; every attention layer shares
                  ``block_table`` / ``ctx_lens`` and every GDN layer (and
                  convolution) shares ``state_slot``.
    accept_mode   'greedy' or 'rejection'
    accept_inputs dict with ``target_logits``, ``draft_tokens`` and, for
                  rejection, ``draft_logits``, ``u_accept``, ``u_final``.

    Returns a dict: ``outputs`` (per layer, float64), ``k_cache`` /
    ``v_cache`` / ``state`` (per layer, after the step; ``None`` where the
    layer has no such buffer), ``conv_outputs`` / ``conv_state`` (per layer,
    ``None`` without a convolution), ``accept_len``, ``out_tokens``,
    ``commit_len`` and ``ctx_lens`` (after the step).
    """
    outputs, kcs, vcs, states = [], [], [], []
    conv_outs, conv_states = [], []
    for lay in layers:
        if lay['kind'] == 'attn':
            outputs.append(verify_attention(
                lay['q'], lay['k_new'], lay['v_new'], lay['k_cache'],
                lay['v_cache'], block_table, ctx_lens, cu_seqlens, page_size,
                lay.get('scale')))
            kc, vc = append_kv(lay['k_cache'], lay['v_cache'], lay['k_new'],
                               lay['v_new'], block_table, ctx_lens,
                               cu_seqlens, page_size)
            kcs.append(kc)
            vcs.append(vc)
            states.append(None)
            conv_outs.append(None)
            conv_states.append(None)
        elif lay['kind'] == 'gdn':
            o, _ = gdn_step(lay['state'], state_slot, lay['q'], lay['k'],
                            lay['v'], lay['alpha'], lay['beta'], cu_seqlens,
                            None, GDN_VERIFY_ONLY)
            outputs.append(o)
            kcs.append(None)
            vcs.append(None)
            states.append(None)
            cv = lay.get('conv')
            if cv is not None:
                y, _ = conv_step(cv['state'], state_slot, cv['x'], cv['weight'],
                                 cv.get('bias'), cu_seqlens, None, CONV_VERIFY_ONLY,
                                 silu=cv.get('silu', False))
                conv_outs.append(y)
            else:
                conv_outs.append(None)
            conv_states.append(None)
        else:
            raise ValueError(f"unknown layer kind {lay['kind']!r}")

    ai = accept_inputs
    if accept_mode == 'greedy':
        accept_len, out_tokens = greedy_accept(
            ai['target_logits'], ai['draft_tokens'], cu_seqlens, max_T)
    elif accept_mode == 'rejection':
        accept_len, out_tokens = rejection_accept(
            ai['target_logits'], ai['draft_logits'], ai['draft_tokens'],
            ai['u_accept'], ai['u_final'], cu_seqlens, max_T)
    else:
        raise ValueError(f"unknown accept mode {accept_mode!r}")

    commit_len = (accept_len + 1).astype(np.int32)
    for idx, lay in enumerate(layers):
        if lay['kind'] == 'gdn':
            _, S = gdn_step(lay['state'], state_slot, None, lay['k'],
                            lay['v'], lay['alpha'], lay['beta'], cu_seqlens,
                            commit_len, GDN_COMMIT_ONLY)
            states[idx] = S
            cv = lay.get('conv')
            if cv is not None:
                _, CS = conv_step(cv['state'], state_slot, cv['x'], cv['weight'],
                                  cv.get('bias'), cu_seqlens, commit_len,
                                  CONV_COMMIT_ONLY)
                conv_states[idx] = CS
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    if ctx.shape != commit_len.shape:
        raise ValueError(f'ctx_lens has {ctx.shape[0]} entries for {commit_len.shape[0]} sequences')
    new_ctx = (ctx + commit_len).astype(np.int32)
    return {
        'outputs': outputs, 'k_cache': kcs, 'v_cache': vcs, 'state': states,
        'conv_outputs': conv_outs, 'conv_state': conv_states,
        'accept_len': accept_len, 'out_tokens': out_tokens,
        'commit_len': commit_len, 'ctx_lens': new_ctx,
    }
