"""Oracle for the paged verification attention and its KV append.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition written out here (lmdeploy PR 5019, feature list: block speculative
verification with paged verification attention over a fixed draft chain):
sequence ``b`` holds ``L_b`` tokens in a paged KV cache and brings ``T_b``
in-flight tokens (the last committed token followed by the drafts).  Verify
token ``j`` attends, per query head ``h``, to every cached position and to the
in-flight positions ``0..j`` (a chain, so the mask is plain causal), with the
GQA key/value head ``g = h * Hkv // Hq``:

    o[b, h, j] = sum_p softmax_p(scale * q[b, h, j] . K[b, g, p]) V[b, g, p]

Pool layout (the pages do not fix one): ``cache[num_pages, Hkv, P, D]``;
logical position ``p`` of sequence ``b`` lives in physical page
``block_table[b, p // P]`` at slot ``p % P``.  Reading a sequence back as a
dense array is the gather that ``flatten_kv_cache.py`` performs in lmdeploy
PR 3945 (review comments on that file).  The in-flight keys and values are
written through into the pages at positions ``L_b .. L_b + T_b - 1``; that
append is idempotent, unlike the recurrent state (onnxruntime-genai PR 2457,
commit message on the graph-capture recurrent-state fix-up).
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gather_context(cache, block_table_row, length, page_size):
    """Dense ``[length, Hkv, D]`` copy of positions ``0..length-1``.

    Position ``p`` is read from page ``block_table_row[p // page_size]``,
    slot ``p % page_size`` of ``cache[num_pages, Hkv, P, D]``.
    """
    pos = np.arange(int(length))
    pages = np.asarray(block_table_row, dtype=np.int64)[pos // page_size]
    slots = pos % page_size
    # Two index arrays separated by a slice: the indexed axis comes first.
    return np.array(cache[pages, :, slots, :])


def append_kv(k_cache, v_cache, k_new, v_new, block_table, ctx_lens,
              cu_seqlens, page_size):
    """Return copies of the pools with the in-flight K/V written through.

    In-flight token ``j`` of sequence ``b`` goes to logical position
    ``ctx_lens[b] + j``.  Every other slot keeps its value.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        for j in range(int(cu[b + 1] - cu[b])):
            pos = int(ctx_lens[b]) + j
            page = int(block_table[b][pos // page_size])
            slot = pos % page_size
            kc[page, :, slot, :] = k_new[cu[b] + j]
            vc[page, :, slot, :] = v_new[cu[b] + j]
    return kc, vc


def verify_attention(q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens,
                     cu_seqlens, page_size, scale=None):
    """Verification attention, float64.  Returns ``o[total_T, Hq, D]``.

    ``q[total_T, Hq, D]`` and ``k_new/v_new[total_T, Hkv, D]`` are packed
    varlen rows (sequence ``b`` owns rows ``cu_seqlens[b]:cu_seqlens[b+1]``);
    the caches hold ``ctx_lens[b]`` tokens per sequence before this step.
    ``scale`` defaults to ``1/sqrt(D)``.
    """
    q = _f64(q)
    k_new = _f64(k_new)
    v_new = _f64(v_new)
    total_T, Hq, D = q.shape
    Hkv = k_new.shape[1]
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(D)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros((total_T, Hq, D), dtype=np.float64)
    G = Hq // Hkv
    for b in range(len(cu) - 1):
        L = int(ctx_lens[b])
        T = int(cu[b + 1] - cu[b])
        Kc = _f64(gather_context(k_cache, block_table[b], L, page_size))
        Vc = _f64(gather_context(v_cache, block_table[b], L, page_size))
        K_all = np.concatenate([Kc, k_new[cu[b]:cu[b] + T]], axis=0)
        V_all = np.concatenate([Vc, v_new[cu[b]:cu[b] + T]], axis=0)
        # Query row r of KV head g is (head h = g*G + r % G, token j = r // G);
        # it sees positions 0 .. L + j (cached, then in-flight 0..j).
        j_of_row = np.repeat(np.arange(T), G)
        visible = np.arange(L + T)[None, :] <= (L + j_of_row)[:, None]
        for g in range(Hkv):
            Kg = np.ascontiguousarray(K_all[:, g, :])       # [L+T, D]
            Vg = np.ascontiguousarray(V_all[:, g, :])
            Qg = q[cu[b]:cu[b] + T, g * G:(g + 1) * G, :].reshape(T * G, D)
            s = np.where(visible, (Qg @ Kg.T) * scale, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))  # exp(-inf) = 0
            o = (w @ Vg) / w.sum(axis=1, keepdims=True)
            out[cu[b]:cu[b] + T, g * G:(g + 1) * G, :] = o.reshape(T, G, D)
    return out
