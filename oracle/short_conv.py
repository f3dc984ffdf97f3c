"""Oracle for the causal short-convolution state verify and commit.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The linear-attention layers of the hybrid models on the pages run a short
causal convolution in front of the recurrence, with its own rolling state;
the packed varlen operator publishes that state after every token for
rollback, and the conv's state slot j is the state after local token j
(onnxruntime-genai pull request 2457, commit message on emitting the
``VarlenCausalConvWithState.prefix_states`` and ``GatedDeltaNet.checkpoints``
series).  The pages print no formula; the reading written out here is the
plain depthwise causal convolution of width ``K`` over each sequence's token
stream, per channel ``c``:

    z = [state_0 .. state_{K-2}, x_0 .. x_{T-1}]        (oldest first)
    y_t[c] = act( sum_{i<K} w[c, i] * z_{t+i}[c] + bias[c] )

so tap ``K-1`` multiplies the newest input ``x_t``.  ``act`` is the identity
or SiLU (``u * sigmoid(u)``).  The state holds the last ``K-1`` inputs.

Commit, as for the recurrent state ("undo equals never applied"): with
``c_b`` leading verify tokens kept, the stored state becomes the last ``K-1``
rows of ``[state, x_0 .. x_{c_b - 1}]`` -- exactly what a run over only those
tokens leaves; ``c_b = 0`` keeps the state.

Modes (same numbering as the GDN oracle):
    CONV_VERIFY_COMMIT  outputs for all T_b tokens, state committed at c_b
    CONV_VERIFY_ONLY    outputs for all T_b tokens, state untouched
    CONV_COMMIT_ONLY    no outputs; state committed at c_b
"""

import numpy as np

CONV_VERIFY_COMMIT = 0
CONV_VERIFY_ONLY = 1
CONV_COMMIT_ONLY = 2


def _silu(u):
    return u / (1.0 + np.exp(-u))


def conv_step(state, state_slot, x, weight, bias, cu_seqlens, commit_len, mode,
              silu=False):
    """One verify / commit pass, float64.

    state      [num_slots, K-1, C]   rolling inputs, oldest first (not modified)
    state_slot [B] int or None       slot of sequence b (None: slot b)
    x          [total_T, C]          packed varlen inputs
    weight     [C, K]                taps; weight[:, K-1] multiplies x_t
    bias       [C] or None
    commit_len [B] int in 0..T_b     (ignored for CONV_VERIFY_ONLY)

    Returns ``(y, new_state)``: ``y[total_T, C]`` (``None`` for
    CONV_COMMIT_ONLY) and a float64 copy of the whole state bank after the
    commit.
    """
    S = np.array(state, dtype=np.float64, copy=True)
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    bias = None if bias is None else np.asarray(bias, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    K = w.shape[1]
    y = None if mode == CONV_COMMIT_ONLY else np.zeros_like(x)
    for b in range(B):
        slot = b if state_slot is None else int(state_slot[b])
        rows = slice(cu[b], cu[b + 1])
        T = int(cu[b + 1] - cu[b])
        z = np.concatenate([S[slot], x[rows]], axis=0)  # [K-1+T, C]
        if y is not None:
            for t in range(T):
                u = np.zeros(x.shape[1])
                for i in range(K):
                    u += w[:, i] * z[t + i]
                if bias is not None:
                    u += bias
                y[cu[b] + t] = _silu(u) if silu else u
        if mode != CONV_VERIFY_ONLY:
            c = int(commit_len[b])
            S[slot] = z[c:c + K - 1]
    return y, S
