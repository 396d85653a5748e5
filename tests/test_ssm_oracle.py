"""Pins for the Mamba-2 state recurrence oracle (oracle/ssm.py): a hand-worked
example, special cases with closed forms, the group sharing of keys and queries,
and the replay form that "Nemotron 3.5 Super and Lightning" (serving section)
states to be equal to the recurrence, written out here with explicit loops."""
import numpy as np

from oracle import ssm


def test_hand_example_two_tokens():
    # H = G = 1, P = N = 2; S1 = 0.5 S0 + v1 k1^T, y1 = S1 q1; S2 = 0.25 S1 + v2 k2^T
    S0 = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    k = np.array([[[1.0, 0.0]], [[0.0, 2.0]]])
    v = np.array([[[0.0, 1.0]], [[1.0, 1.0]]])
    a = np.array([[0.5], [0.25]])
    q = np.array([[[1.0, 1.0]], [[2.0, -1.0]]])
    states, y = ssm.recurrence(S0, k, v, a, q)
    np.testing.assert_array_equal(states[0][0], [[0.5, 0.0], [1.0, 0.5]])
    np.testing.assert_array_equal(states[1][0], [[0.125, 2.0], [0.25, 2.125]])
    np.testing.assert_array_equal(y[0][0], [0.5, 1.5])
    np.testing.assert_array_equal(y[1][0], [-1.75, -1.625])


def _rand(rng, L, H, G, P, N):
    S0 = rng.standard_normal((H, P, N))
    k = rng.standard_normal((L, G, N))
    v = rng.standard_normal((L, H, P))
    a = rng.uniform(0.2, 1.0, (L, H))
    q = rng.standard_normal((L, G, N))
    return S0, k, v, a, q


def test_unit_decay_from_zero_is_linear_attention():
    rng = np.random.default_rng(1)
    L, H, G, P, N = 6, 4, 2, 3, 5
    _, k, v, _, q = _rand(rng, L, H, G, P, N)
    _, y = ssm.recurrence(np.zeros((H, P, N)), k, v, np.ones((L, H)), q)
    for t in range(L):
        for h in range(H):
            g = h // (H // G)
            ref = sum(v[j, h] * float(np.dot(k[j, g], q[t, g])) for j in range(t + 1))
            np.testing.assert_allclose(y[t, h], ref, rtol=1e-12, atol=1e-12)


def test_zero_decay_keeps_only_the_last_token():
    rng = np.random.default_rng(2)
    L, H, G, P, N = 4, 2, 1, 3, 4
    S0, k, v, _, q = _rand(rng, L, H, G, P, N)
    states, y = ssm.recurrence(S0, k, v, np.zeros((L, H)), q)
    for t in range(L):
        for h in range(H):
            np.testing.assert_array_equal(states[t, h], np.outer(v[t, h], k[t, 0]))
            np.testing.assert_allclose(y[t, h], v[t, h] * np.dot(k[t, 0], q[t, 0]), rtol=1e-13)


def test_keys_and_queries_are_shared_within_a_group():
    rng = np.random.default_rng(3)
    L, H, G, P, N = 3, 4, 2, 2, 3
    S0, k, v, a, q = _rand(rng, L, H, G, P, N)
    _, y = ssm.recurrence(S0, k, v, a, q)
    k2, q2 = k.copy(), q.copy()
    k2[:, 1] += 1.0
    q2[:, 1] -= 0.5
    _, y2 = ssm.recurrence(S0, k2, v, a, q2)
    np.testing.assert_array_equal(y[:, :2], y2[:, :2])   # heads 0, 1: group 0
    assert np.all(np.abs(y[:, 2:] - y2[:, 2:]) > 0)       # heads 2, 3: group 1
    assert list(ssm.head_group(128, 8)[[0, 15, 16, 127]]) == [0, 0, 1, 7]


def test_replay_form_equals_the_recurrence():
    """The page's replay: the output at step p is the query times the checkpoint,
    scaled by the product of the decays since the checkpoint, plus, for every
    buffered record j <= p, the value v_j weighted by the dot product of the query
    with k_j and by the product of the decays after record j."""
    rng = np.random.default_rng(4)
    L, H, G, P, N = 9, 4, 2, 3, 5
    S0, k, v, a, q = _rand(rng, L, H, G, P, N)
    _, y = ssm.recurrence(S0, k, v, a, q)
    for p in range(L):
        for h in range(H):
            g = h // (H // G)
            dec_all = 1.0
            for i in range(p + 1):
                dec_all *= a[i, h]
            ref = dec_all * (S0[h] @ q[p, g])
            for j in range(p + 1):
                w = 1.0
                for i in range(j + 1, p + 1):
                    w *= a[i, h]
                ref = ref + w * float(np.dot(q[p, g], k[j, g])) * v[j, h]
            np.testing.assert_allclose(y[p, h], ref, rtol=1e-11, atol=1e-12)


def test_verify_outputs_and_flush():
    rng = np.random.default_rng(5)
    CAP, T, H, G, P, N = 16, 4, 4, 2, 3, 5
    S0, bk, bv, ba, _ = _rand(rng, CAP, H, G, P, N)
    _, dk, dv, da, dq = _rand(rng, T, H, G, P, N)
    for n in (0, 5, CAP - T):
        y = ssm.verify_outputs(S0, bk, bv, ba, n, dq, dk, dv, da)
        S = ssm.flush_state(S0, bk, bv, ba, n)
        # the drafts' outputs continue from the flushed state
        _, y2 = ssm.recurrence(S, dk, dv, da, dq)
        np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(ssm.flush_state(S0, bk, bv, ba, 0), S0)
