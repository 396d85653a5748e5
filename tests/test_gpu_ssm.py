"""GPU parity of the Mamba-2 checkpoint + replay verification (include/ssm_replay.h)
against the fp64 recurrence of oracle/ssm.py, on the same seeded bytes.

Bars: appended records bit-exact; outputs within 1e-4 * rms of the oracle (fp32
arithmetic on exact bf16 inputs); flushed and written states within one bf16
step of the oracle's state plus 1e-5 * rms (the GPU rounds its fp32 value)."""
import numpy as np
import pytest

import oracle
from oracle.formats import bf16_to_f64
from sparse_moe_layer_logits_amd import binding, synth

from gpu_common import log

pytestmark = pytest.mark.gpu

Y_TOL = 1e-4


def shape_of(wl):
    return binding.ssm_shape(wl.H, wl.G, wl.P, wl.N, wl.cap)


def upload(d):
    return {k: binding.to_device(v) for k, v in d.items()}


def stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def host(t, dtype=None):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def ref_outputs(d, r, n_buf):
    f = bf16_to_f64
    return oracle.ssm.verify_outputs(
        f(d["ckpt"][r]), f(d["buf_k"][r]), f(d["buf_v"][r]), d["buf_a"][r].astype(np.float64), n_buf,
        f(d["draft_q"][r]), f(d["draft_k"][r]), f(d["draft_v"][r]), d["draft_a"][r].astype(np.float64))


def check_close(got, ref, what):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    log("%s: max|gpu-oracle| = %.3e, rms = %.3e, ratio %.2e" % (what, err, rms, err / rms))
    assert err <= Y_TOL * rms, (what, err, rms)


def check_state_bf16(got_bits, ref, what):
    """GPU state (bf16 bits) against the oracle's fp64 state: within one bf16 step
    of the value, plus the fp32 accumulation error of its O(rms) terms (elements that
    cancel to near zero carry that absolute error before rounding)."""
    got = bf16_to_f64(got_bits)
    step = np.abs(ref) * 2.0 ** -7 + 1e-5 * np.sqrt(np.mean(ref ** 2))
    bad = np.abs(got - ref) > step
    log("%s: %d of %d elements beyond one bf16 step" % (what, int(bad.sum()), bad.size))
    assert not bad.any(), what


def run_verify(wl, d, dev, y):
    binding.ssm_replay_verify(shape_of(wl), wl.R, wl.T, dev["ckpt"].data_ptr(), dev["buf_k"].data_ptr(),
                              dev["buf_v"].data_ptr(), dev["buf_a"].data_ptr(), dev["buf_len"].data_ptr(),
                              dev["draft_q"].data_ptr(), dev["draft_k"].data_ptr(),
                              dev["draft_v"].data_ptr(), dev["draft_a"].data_ptr(), y.data_ptr(), stream())


@pytest.mark.parametrize("seed,P,N", [(0, 64, 128), (1, 64, 128), (2, 128, 64), (3, 64, 64),
                                      (4, 128, 128)])
def test_replay_verify_matches_recurrence_and_appends(seed, P, N):
    import torch
    wl = synth.SSM_WORKLOADS["ssm_tiny"].replace(P=P, N=N)
    d = synth.make_ssm(wl, seed)
    d["buf_len"][0] = 0                      # empty buffer
    d["buf_len"][1] = wl.cap - wl.T          # exactly full after the append
    d["buf_len"][2] = wl.cap - wl.T + 1      # no room: NaN outputs, buffer untouched
    dev = upload(d)
    y = torch.empty((wl.R, wl.T, wl.H, wl.P), dtype=torch.float32, device="cuda")
    run_verify(wl, d, dev, y)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().astype(np.float64)
    for r in range(wl.R):
        n = int(d["buf_len"][r])
        bk, bv, ba = host(dev["buf_k"])[r], host(dev["buf_v"])[r], host(dev["buf_a"])[r]
        if n + wl.T > wl.cap:
            assert np.all(np.isnan(yg[r]))
            assert np.array_equal(bk, d["buf_k"][r]) and np.array_equal(bv, d["buf_v"][r])
            assert np.array_equal(ba, d["buf_a"][r])
            continue
        check_close(yg[r], ref_outputs(d, r, n), "seed %d request %d (n_buf %d)" % (seed, r, n))
        # the appended records, bit for bit, and the rest of the buffer unchanged
        ek, ev, ea = d["buf_k"][r].copy(), d["buf_v"][r].copy(), d["buf_a"][r].copy()
        ek[n:n + wl.T], ev[n:n + wl.T], ea[n:n + wl.T] = d["draft_k"][r], d["draft_v"][r], d["draft_a"][r]
        assert np.array_equal(bk, ek) and np.array_equal(bv, ev) and np.array_equal(ba, ea)
    assert np.array_equal(host(dev["buf_len"]), d["buf_len"])   # verify leaves the counters


def test_commit_flush_and_continue():
    """append -> commit -> flush -> verify again: the whole cycle against the
    recurrence over the accepted tokens only."""
    import torch
    wl = synth.SSM_WORKLOADS["ssm_tiny"]
    d = synth.make_ssm(wl, 3)
    d["buf_len"][:] = [1, 0, 2]
    dev = upload(d)
    st = stream()
    y = torch.empty((wl.R, wl.T, wl.H, wl.P), dtype=torch.float32, device="cuda")
    run_verify(wl, d, dev, y)
    accepted = np.array([wl.T, 0, 2], np.int32)
    acc_dev = binding.to_device(accepted)
    binding.ssm_replay_commit(wl.R, acc_dev.data_ptr(), dev["buf_len"].data_ptr(), st)
    torch.cuda.synchronize()
    lens = d["buf_len"] + accepted
    assert np.array_equal(host(dev["buf_len"]), lens)
    # oracle: checkpoint advanced by the kept records (old buffer, then the accepted drafts)
    f = bf16_to_f64
    ref_state = []
    for r in range(wl.R):
        n0 = int(d["buf_len"][r])
        k = np.concatenate([f(d["buf_k"][r][:n0]), f(d["draft_k"][r][:accepted[r]])])
        v = np.concatenate([f(d["buf_v"][r][:n0]), f(d["draft_v"][r][:accepted[r]])])
        a = np.concatenate([d["buf_a"][r][:n0], d["draft_a"][r][:accepted[r]]]).astype(np.float64)
        ref_state.append(oracle.ssm.flush_state(f(d["ckpt"][r]), k, v, a, len(k)))
    binding.ssm_replay_flush(shape_of(wl), wl.R, dev["ckpt"].data_ptr(), dev["buf_k"].data_ptr(),
                             dev["buf_v"].data_ptr(), dev["buf_a"].data_ptr(), dev["buf_len"].data_ptr(), st)
    torch.cuda.synchronize()
    assert np.all(host(dev["buf_len"]) == 0)
    ck = host(dev["ckpt"])
    for r in range(wl.R):
        if lens[r] == 0:
            assert np.array_equal(ck[r], d["ckpt"][r])      # empty buffer: checkpoint kept
        else:
            check_state_bf16(ck[r], ref_state[r], "flushed state, request %d" % r)
    # next step: new drafts verified against the flushed checkpoint
    d2 = synth.make_ssm(wl, 4)
    for key in ("draft_q", "draft_k", "draft_v", "draft_a"):
        dev[key].copy_(binding.to_device(d2[key]))
    run_verify(wl, d2, dev, y)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().astype(np.float64)
    for r in range(wl.R):
        S = bf16_to_f64(ck[r])
        _, ref = oracle.ssm.recurrence(S, f(d2["draft_k"][r]), f(d2["draft_v"][r]),
                                       d2["draft_a"][r].astype(np.float64), f(d2["draft_q"][r]))
        check_close(yg[r], ref, "after flush, request %d" % r)


@pytest.mark.parametrize("P,N", [(64, 128), (128, 64)])
def test_state_writing_scheme_matches_recurrence(P, N):
    import torch
    wl = synth.SSM_WORKLOADS["ssm_tiny"].replace(P=P, N=N)
    d = synth.make_ssm(wl, 5)
    dev = upload(d)
    states = torch.empty((wl.R, wl.T, wl.H, wl.P, wl.N), dtype=torch.int16, device="cuda")
    y = torch.empty((wl.R, wl.T, wl.H, wl.P), dtype=torch.float32, device="cuda")
    binding.ssm_states_verify(shape_of(wl), wl.R, wl.T, dev["ckpt"].data_ptr(), dev["draft_q"].data_ptr(),
                              dev["draft_k"].data_ptr(), dev["draft_v"].data_ptr(), dev["draft_a"].data_ptr(),
                              states.data_ptr(), y.data_ptr(), stream())
    torch.cuda.synchronize()
    sg, yg = host(states), y.cpu().numpy().astype(np.float64)
    f = bf16_to_f64
    for r in range(wl.R):
        ref_s, ref_y = oracle.ssm.recurrence(f(d["ckpt"][r]), f(d["draft_k"][r]), f(d["draft_v"][r]),
                                             d["draft_a"][r].astype(np.float64), f(d["draft_q"][r]))
        check_close(yg[r], ref_y, "state-writing outputs, request %d" % r)
        check_state_bf16(sg[r], ref_s, "written states, request %d" % r)


def test_super_mamba_verify_sampled():
    """Super's Mamba shapes (128 heads of 64, state 128, 8 groups), 64 requests x 8
    tokens: every request's appended records, outputs of a spread sample of
    requests; the two schemes agree on every request."""
    import torch
    wl = synth.SSM_WORKLOADS["super_mamba_verify"]
    d = synth.make_ssm(wl, 0)
    dev = upload(d)
    y = torch.empty((wl.R, wl.T, wl.H, wl.P), dtype=torch.float32, device="cuda")
    run_verify(wl, d, dev, y)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().astype(np.float64)
    bk = host(dev["buf_k"])
    for r in range(wl.R):
        n = int(d["buf_len"][r])
        assert np.array_equal(bk[r][n:n + wl.T], d["draft_k"][r])
    for r in (0, 21, 42, 63):
        check_close(yg[r], ref_outputs(d, r, int(d["buf_len"][r])), "super request %d" % r)
    # the state-writing scheme from the state the buffer represents gives the same outputs
    f = bf16_to_f64
    cur = np.stack([oracle.ssm.flush_state(f(d["ckpt"][r]), f(d["buf_k"][r]), f(d["buf_v"][r]),
                                           d["buf_a"][r].astype(np.float64), int(d["buf_len"][r]))
                    for r in (0, 63)])
    cur_bits = synth.f32_to_bf16_bits(cur.astype(np.float32))
    st_dev = binding.to_device(np.ascontiguousarray(cur_bits))
    sub = {k: binding.to_device(np.ascontiguousarray(d[k][[0, 63]]))
           for k in ("draft_q", "draft_k", "draft_v", "draft_a")}
    states = torch.empty((2, wl.T, wl.H, wl.P, wl.N), dtype=torch.int16, device="cuda")
    y2 = torch.empty((2, wl.T, wl.H, wl.P), dtype=torch.float32, device="cuda")
    binding.ssm_states_verify(shape_of(wl), 2, wl.T, st_dev.data_ptr(), sub["draft_q"].data_ptr(),
                              sub["draft_k"].data_ptr(), sub["draft_v"].data_ptr(), sub["draft_a"].data_ptr(),
                              states.data_ptr(), y2.data_ptr(), stream())
    torch.cuda.synchronize()
    y2g = y2.cpu().numpy().astype(np.float64)
    for i, r in enumerate((0, 63)):
        # the state-writing path starts from the bf16-rounded current state, replay from the
        # checkpoint: they agree to the rounding of that state (~2^-9 relative)
        rms = np.sqrt(np.mean(yg[r] ** 2))
        assert np.max(np.abs(y2g[i] - yg[r])) <= 2e-2 * rms
