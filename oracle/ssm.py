"""Mamba-2 state recurrence and its checkpoint + replay verification, float64.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: "Nemotron 3.5 Super and Lightning" (serving section: where the
throughput comes from): a Mamba layer keeps a fixed-size state per head; each
token updates it as  new state = decay * old state + outer product of the
token's key and value,  and the token's output is its query times the state.
Shapes from "Nemotron 3 Super" section 3.1 (state dimension 128, 8 groups, 128
heads of dimension 64): per head h the state S is [P, N] (P = head dim, N =
state dim), key k and query q are N-vectors shared by the heads of one group
(group of head h = h // (H // G)), value v is a P-vector per head and the decay
a a scalar per head.  Readings (the page leaves them open): the output of a
token is taken after its own update, y_t = S_t q_t; the state is stored in
bf16 ("16-bit Mamba state", "Nemotron 3 Ultra" limitations) and computed in
higher precision.

This module is the plain definition: the recurrence, run token by token.  The
replay form the GPU path computes (checkpoint times the decay products plus a
decayed sum over the buffered records) is the same quantity; the tests pin the
recurrence itself and check the GPU against it.
"""
from __future__ import annotations

import numpy as np


def head_group(H: int, G: int) -> np.ndarray:
    """Group index of each head (heads of one group share key and query)."""
    return np.arange(H) // (H // G)


def recurrence(S0, k, v, a, q=None):
    """Run the recurrence over L tokens for every head.

    S0: [H, P, N] initial state; k: [L, G, N]; v: [L, H, P]; a: [L, H];
    q: [L, G, N] or None.  Returns (states [L, H, P, N], outputs [L, H, P] or
    None): states[t] is the state after token t, outputs[t] = states[t] q_t.
    """
    S0 = np.asarray(S0, dtype=np.float64)
    k, v, a = (np.asarray(z, dtype=np.float64) for z in (k, v, a))
    L = k.shape[0]
    H = S0.shape[0]
    grp = head_group(H, k.shape[1])
    S = S0.copy()
    states = np.empty((L,) + S0.shape)
    outs = None if q is None else np.empty((L, H, S0.shape[1]))
    for t in range(L):
        kt = k[t][grp]                                     # [H, N]
        S = a[t][:, None, None] * S + v[t][:, :, None] * kt[:, None, :]
        states[t] = S
        if q is not None:
            qt = np.asarray(q[t], dtype=np.float64)[grp]   # [H, N]
            outs[t] = np.einsum("hpn,hn->hp", S, qt)
    return states, outs


def verify_outputs(ckpt, buf_k, buf_v, buf_a, n_buf, draft_q, draft_k, draft_v, draft_a):
    """Outputs of the T draft tokens of one request: the state is the checkpoint
    advanced by the n_buf buffered records, then by the drafts one at a time.
    Returns [T, H, P]."""
    k = np.concatenate([buf_k[:n_buf], draft_k])
    v = np.concatenate([buf_v[:n_buf], draft_v])
    a = np.concatenate([buf_a[:n_buf], draft_a])
    T = draft_q.shape[0]
    q = np.concatenate([np.zeros((n_buf,) + draft_q.shape[1:]), draft_q])
    _, outs = recurrence(ckpt, k, v, a, q)
    return outs[n_buf:n_buf + T]


def flush_state(ckpt, buf_k, buf_v, buf_a, n_buf):
    """The state after the checkpoint and the first n_buf buffered records
    (the checkpoint itself when n_buf is 0).  Returns [H, P, N] float64."""
    if n_buf == 0:
        return np.asarray(ckpt, dtype=np.float64).copy()
    states, _ = recurrence(ckpt, buf_k[:n_buf], buf_v[:n_buf], buf_a[:n_buf])
    return states[-1]
