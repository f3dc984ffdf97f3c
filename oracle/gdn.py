"""Oracle for the gated delta-net (GDN) recurrent-state verify and commit.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Recurrence (gated delta rule, Yang, Kautz & Hatamizadeh, ICLR 2025), per
sequence ``b`` and head ``h``, with ``S`` the ``dv x dk`` state stored V-major
in float32 (onnxruntime-genai PR 2457, commit message on the GatedDeltaNet
cherry-pick defects: the operator needs a V-major fp32 state) and gates
``alpha_t, beta_t`` supplied already in float32 (the packed varlen operator of
the same message takes pre-cast gates):

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t                     (output read after the update)

Commit (lmdeploy PR 5019, "Two fixes" item 2: the recurrent state is written
back after the speculative round has accepted tokens; onnxruntime-genai
PR 2457: ``CommitPrefix`` keeps the state of the accepted prefix, with no
snapshot and no replay forward): with ``c_b`` the number of leading verify
tokens whose effect is kept (``0 <= c_b <= T_b``), the stored state becomes
``S_{c_b}``; ``c_b = 0`` leaves it as it was.  That is exactly the state a run
over only the first ``c_b`` tokens would leave ("undo equals never applied").

Modes:
    GDN_VERIFY_COMMIT  outputs for all T_b tokens, state stored at c_b
    GDN_VERIFY_ONLY    outputs for all T_b tokens, state untouched
    GDN_COMMIT_ONLY    no outputs; the first c_b tokens are applied and stored
"""

import numpy as np

GDN_VERIFY_COMMIT = 0
GDN_VERIFY_ONLY = 1
GDN_COMMIT_ONLY = 2


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def gdn_step(state, state_slot, q, k, v, alpha, beta, cu_seqlens, commit_len,
             mode):
    """Run one verify / commit pass.

    state       [num_slots, H, dv, dk]   recurrent states (not modified)
    state_slot  [B] int or None          slot of sequence b (None: slot b)
    q, k        [total_T, H, dk]
    v           [total_T, H, dv]
    alpha, beta [total_T, H]
    commit_len  [B] int in 0..T_b        (ignored for GDN_VERIFY_ONLY)

    Returns ``(o, new_state)``: ``o[total_T, H, dv]`` float64 (``None`` for
    GDN_COMMIT_ONLY) and a float64 copy of the whole state bank after the
    commit.
    """
    S_bank = _f64(state).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    H, dv = S_bank.shape[1], S_bank.shape[2]
    total_T = int(cu[-1])
    o = None if mode == GDN_COMMIT_ONLY else np.zeros((total_T, H, dv))
    for b in range(B):
        slot = b if state_slot is None else int(state_slot[b])
        T = int(cu[b + 1] - cu[b])
        c = None if mode == GDN_VERIFY_ONLY else int(commit_len[b])
        n_run = c if mode == GDN_COMMIT_ONLY else T
        # The H heads of sequence b are independent recurrences; they are
        # advanced together, S[h] being head h's [dv, dk] state.
        S = S_bank[slot].copy()
        S_commit = S.copy()                          # c == 0 keeps S_0
        for t in range(n_run):
            x = cu[b] + t
            a_t = alpha[x][:, None, None]            # [H, 1, 1]
            b_t = beta[x][:, None, None]
            k_t, v_t = k[x], v[x]                    # [H, dk], [H, dv]
            Sk = np.matmul(S, k_t[:, :, None])       # S_{t-1} k_t, [H, dv, 1]
            S = a_t * (S - b_t * (Sk * k_t[:, None, :])) \
                + b_t * (v_t[:, :, None] * k_t[:, None, :])
            if o is not None:
                o[x] = np.matmul(S, q[x][:, :, None])[:, :, 0]
            if c is not None and t == c - 1:
                S_commit = S.copy()
        if mode != GDN_VERIFY_ONLY:
            S_bank[slot] = S_commit
    return o, S_bank
