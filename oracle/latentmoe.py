"""LatentMoE layer forward in float64, written out from its definition.

Source: "Nemotron 3 Super: Open, Efficient Mixture-of-Experts Hybrid
Mamba-Transformer Model for Agentic Reasoning", section 3.2 (LatentMoE):
a token x in R^d is projected by a learned W_down in R^{l x d} into the latent
space, routed to experts that compute in latent width, and the result is
projected back by a learned W_up in R^{d x l}; the gating network and the shared
expert stay at the full width d.

Per token t (readings of what the page leaves open are marked *):
  1. logits   l = W_r x + b                       (gating at width d; b optional*)
  2. select   S = first K experts ordered by (-l_e, e)   (lowest index wins ties*)
  3. gates    g_k = exp(l_{S_k} - max) / sum_j exp(l_{S_j} - max)   (softmax over the K*)
  4. latent   z = W_down x
  5. experts  o_k = W2_{S_k} relu(W1_{S_k} z)^2          (squared ReLU*, two matrices*)
  6. combine  y_lat = sum_k g_k o_k, in k order
  7. output   y = W_up y_lat + S2 relu(S1 x)^2           (shared expert, ungated*)

All inputs are the stored bytes (bf16 bit patterns, float32, block-scaled FP4
codes for the experts and optionally the shared expert, per-tensor FP8 codes
optionally for W_down and W_up), decoded to float64 by ``formats``; every
operation is float64.
Experts are evaluated one expert at a time over the tokens routed to it, which
is the same per-token sum; nothing is fused or blocked.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, fp4_dequant, fp8_dequant


def router_logits(x_bits, router_w, router_bias=None):
    """Step 1: float64 logits [T, N] = x W_r^T (+ b)."""
    x = bf16_to_f64(x_bits)
    l = x @ np.asarray(router_w, dtype=np.float64).T
    if router_bias is not None:
        l = l + np.asarray(router_bias, dtype=np.float64)[None, :]
    return l


def select_topk(logits, k):
    """Step 2: per row, the K experts first in the order (-logit, index).

    Returns int64 [T, K] in that order (largest logit first, ties to the lower
    index)."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    T, n = logits.shape
    out = np.empty((T, k), dtype=np.int64)
    idx = np.arange(n)
    for t in range(T):
        order = np.lexsort((idx, -logits[t]))  # primary key -logit, then index
        out[t] = order[:k]
    return out


def softmax_selected(logits, idx):
    """Step 3: softmax over each row's K selected logits (in the order of idx)."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    sel = np.take_along_axis(logits, idx, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def topk_gap(logits, k):
    """Distance between the K-th and (K+1)-th largest logit of each row
    (inf when K equals the number of experts)."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    if k >= logits.shape[1]:
        return np.full(logits.shape[0], np.inf)
    s = -np.sort(-logits, axis=1)
    return s[:, k - 1] - s[:, k]


def expert_ffn(z, w1, w2):
    """Step 5 for one expert: W2 relu(W1 z)^2 for each row of z [rows, l]."""
    u = z @ w1.T
    h = np.maximum(u, 0.0) ** 2
    return h @ w2.T


def shared_expert(x, s1, s2):
    """Full-width shared expert: S2 relu(S1 x)^2 for each row of x [rows, d]."""
    h = np.maximum(x @ s1.T, 0.0) ** 2
    return h @ s2.T


def expert_weights(W, e):
    """Float64 (W1_e [m, l], W2_e [l, m]) of expert e from the stored bytes."""
    if "expert_w1_scale" in W:
        w1 = fp4_dequant(W["expert_w1"][e], W["expert_w1_scale"][e], W["expert_w1_tscale"][e])
        w2 = fp4_dequant(W["expert_w2"][e], W["expert_w2_scale"][e], W["expert_w2_tscale"][e])
    else:
        w1 = bf16_to_f64(W["expert_w1"][e])
        w2 = bf16_to_f64(W["expert_w2"][e])
    return w1, w2


def shared_weights(W):
    """Float64 (S1 [m_s, d], S2 [d, m_s]) of the shared expert from the stored bytes."""
    if W.get("shared_w1_scale") is not None:
        s1 = fp4_dequant(W["shared_w1"], W["shared_w1_scale"], np.ravel(W["shared_w1_tscale"])[0])
        s2 = fp4_dequant(W["shared_w2"], W["shared_w2_scale"], np.ravel(W["shared_w2_tscale"])[0])
    else:
        s1 = bf16_to_f64(W["shared_w1"])
        s2 = bf16_to_f64(W["shared_w2"])
    return s1, s2


def projection_weights(W):
    """Float64 (W_down [l, d], W_up [d, l]) from the stored bytes."""
    if W.get("w_down_tscale") is not None:
        return (fp8_dequant(W["w_down"], np.ravel(W["w_down_tscale"])[0]),
                fp8_dequant(W["w_up"], np.ravel(W["w_up_tscale"])[0]))
    return bf16_to_f64(W["w_down"]), bf16_to_f64(W["w_up"])


def forward(x_bits, W, top_k, tokens=None, intermediates=False):
    """LatentMoE forward for the rows ``tokens`` of x (all rows if None).

    Returns a dict with y [Ts, d], idx [Ts, K], gates [Ts, K], logits [Ts, N];
    with ``intermediates`` also z [Ts, l], y_lat [Ts, l], y_shared [Ts, d].
    """
    x_bits = np.asarray(x_bits)
    if tokens is not None:
        x_bits = x_bits[np.asarray(tokens)]
    Ts = x_bits.shape[0]
    x = bf16_to_f64(x_bits)

    logits = router_logits(x_bits, W["router_w"], W.get("router_bias"))   # step 1
    idx = select_topk(logits, top_k)                                      # step 2
    gates = softmax_selected(logits, idx)                                 # step 3

    w_down, w_up = projection_weights(W)
    z = x @ w_down.T                                                      # step 4
    latent = z.shape[1]

    out = np.zeros((Ts, top_k, latent))                                   # step 5
    for e in np.unique(idx):
        t_sel, k_sel = np.nonzero(idx == e)
        w1, w2 = expert_weights(W, int(e))
        out[t_sel, k_sel] = expert_ffn(z[t_sel], w1, w2)

    y_lat = np.zeros((Ts, latent))                                        # step 6
    for k in range(top_k):
        y_lat += gates[:, k:k + 1] * out[:, k]

    y_shared = shared_expert(x, *shared_weights(W))
    y = y_lat @ w_up.T + y_shared                                         # step 7

    res = dict(y=y, idx=idx, gates=gates, logits=logits)
    if intermediates:
        res.update(z=z, y_lat=y_lat, y_shared=y_shared)
    return res
