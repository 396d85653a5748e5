"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Bar: top-K indices bit-exact as per-token sets; gates within 1e-6;
max |y_gpu - y_oracle| <= 1e-2 * rms(y_oracle) (3e-2 with FP4 experts, the
oracle decoding the same FP4 bytes); bucketing exact.
"""
import numpy as np
import pytest

import oracle
from sparse_moe_layer_logits_amd import binding, synth

from gpu_common import (check_bucketing, check_topk, check_y, full_check, full_size_check, log,
                        oracle_y_chunked, run_layer, tolerance)

pytestmark = pytest.mark.gpu


def small_wl(**kw):
    base = dict(name="small", T=8, d=256, latent=64, n_experts=16, top_k=4, expert_hidden=128,
                shared_hidden=256)
    base.update(kw)
    return synth.Workload(**base)


def gen(wl, seed=0):
    x, W = synth.make(wl, seed, threads=8)
    # keep the top-K boundary away from ties (redraw offending rows)
    if wl.top_k < wl.n_experts:
        red = {}
        for _ in range(50):
            gap = oracle.topk_gap(oracle.router_logits(x, W["router_w"], W["router_bias"]), wl.top_k)
            bad = np.nonzero(gap < 1e-4)[0]
            if len(bad) == 0:
                break
            for t in bad:
                red[int(t)] = red.get(int(t), 0) + 1
                x[t] = synth.x_row(seed, int(t), red[int(t)], wl.d)
    return x, W


def test_fp4_decoder_exhaustive():
    import torch
    codes = np.arange(16, dtype=np.uint8)
    scales = np.array([s for s in range(256) if s not in (0x7F, 0xFF)], dtype=np.uint8)
    # one block per (scale, code pair): block b holds codes c, c+1 ... cycling all 16
    blocks = []
    sc = []
    for s in scales:
        row = np.array([(codes[(2 * j) % 16]) | (codes[(2 * j + 1) % 16] << 4) for j in range(8)], np.uint8)
        blocks.append(row)
        sc.append(s)
    packed = np.stack(blocks)
    sc = np.array(sc, np.uint8)
    out = torch.empty((len(sc), 16), dtype=torch.int16, device="cuda")
    cd, sd = binding.to_device(packed), binding.to_device(sc)
    binding.latentmoe_fp4_decode(cd.data_ptr(), sd.data_ptr(), len(sc), out.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    ref = oracle.fp4_dequant(packed, sc[:, None], np.float32(1.0))
    ref_bits = synth.f32_to_bf16_bits(ref.astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f64(ref_bits), ref)   # products are bf16-exact
    assert np.array_equal(got, ref_bits)


def test_fp8_decoder_exhaustive():
    import torch
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    # 16 groups of 16 bytes: every finite code, each at several byte positions
    codes = np.concatenate([finite, finite[:2]])
    codes = np.stack([np.roll(codes, 5 * i) for i in range(4)]).reshape(-1, 16)
    out = torch.empty(codes.shape, dtype=torch.int16, device="cuda")
    cd = binding.to_device(codes)
    binding.latentmoe_fp8_decode(cd.data_ptr(), codes.shape[0], out.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    ref = oracle.fp8_dequant(codes, np.float32(1.0))
    ref_bits = synth.f32_to_bf16_bits(ref.astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f64(ref_bits), ref)   # E4M3 values are bf16-exact
    assert np.array_equal(got, ref_bits)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny(seed):
    wl = synth.WORKLOADS["tiny"]
    x, W = gen(wl, seed)
    log("tiny seed", seed)
    full_check(wl, x, W)


def test_ragged_stream_path():
    # T not a multiple of 16, several 128-wide column blocks, few rows per expert
    wl = small_wl(T=37, d=512, latent=128, n_experts=64, top_k=6, expert_hidden=192, shared_hidden=320)
    x, W = gen(wl, 3)
    log("ragged stream path", wl)
    full_check(wl, x, W)


def test_tiled_path():
    # more than 64 tokens (LDS-tiled dense GEMMs) and > 48 rows per expert (tiled expert GEMMs)
    wl = small_wl(T=300, d=256, latent=128, n_experts=32, top_k=8, expert_hidden=192, shared_hidden=320)
    x, W = gen(wl, 4)
    log("tiled path", wl)
    full_check(wl, x, W)


def test_mid_rows_stream_path():
    # 24 < rows per expert <= 48: 64-row streaming tiles, some experts span two tiles
    wl = small_wl(T=240, d=256, latent=64, n_experts=32, top_k=4, expert_hidden=128, shared_hidden=256)
    x, W = gen(wl, 5)
    log("64-row stream tiles", wl)
    full_check(wl, x, W)


def test_rows32_stream_path():
    # 12 < rows per expert <= 24: 32-row streaming tiles, bf16 and FP4 experts
    wl = small_wl(T=160, d=256, latent=128, n_experts=32, top_k=4, expert_hidden=192, shared_hidden=256)
    x, W = gen(wl, 13)
    log("32-row stream tiles", wl)
    full_check(wl, x, W)
    wl4 = small_wl(T=160, d=256, latent=128, n_experts=32, top_k=4, expert_hidden=192,
                   shared_hidden=256, experts="fp4")
    x4, W4 = gen(wl4, 14)
    full_check(wl4, x4, W4, tol=3e-2)


def test_fp4_mid_kernel_small():
    # FP4 experts, 24 < rows per expert <= 48: the LDS-staged FP4 kernel; up-proj
    # N = 512 runs two 8-wave blocks of 256 rows, down-proj N = 128 one 4-wave
    # block; K = 128 is a single stage
    wl = small_wl(T=240, d=256, latent=128, n_experts=32, top_k=4, expert_hidden=512,
                  shared_hidden=256, experts="fp4")
    x, W = gen(wl, 15)
    log("FP4 mid kernel", wl)
    full_check(wl, x, W, tol=3e-2)


def test_fp4_mid_kernel_waves_past_n():
    # down-proj N = latent = 192 in 4-wave blocks of 128 rows: the second block has
    # two waves past N (they stage activations and skip their products); K = 512
    wl = small_wl(T=240, d=256, latent=192, n_experts=32, top_k=4, expert_hidden=512,
                  shared_hidden=256, experts="fp4")
    x, W = gen(wl, 17)
    log("FP4 kernel, waves past N", wl)
    full_check(wl, x, W, tol=3e-2)


def test_fp4_mid_kernel_partial_last_block():
    # up-proj N = m = 1088 in 8-wave blocks of 256 rows (N >= 1024 takes 8 waves): the
    # fifth block has two active waves and six past N
    wl = small_wl(T=240, d=256, latent=128, n_experts=32, top_k=4, expert_hidden=1088,
                  shared_hidden=256, experts="fp4")
    x, W = gen(wl, 18)
    log("FP4 kernel, partial last block", wl)
    full_check(wl, x, W, tol=3e-2)


def test_fp4_mid_kernel_chunks():
    # the FP4 kernel over many k stages: expert up K = 896 (seven stages of 128, not a
    # multiple of its three register sets), N = 1536 in 8-wave blocks; expert down
    # K = 1536 (twelve stages), N = 896 in 7-wave blocks; 30 rows per expert
    wl = small_wl(T=240, d=256, latent=896, n_experts=32, top_k=4, expert_hidden=1536,
                  shared_hidden=256, experts="fp4")
    x, W = gen(wl, 16)
    log("FP4 kernel, several chunks", wl)
    full_check(wl, x, W, tol=3e-2)


def test_k_equals_n():
    wl = small_wl(T=9, n_experts=16, top_k=16)
    x, W = gen(wl, 6)
    full_check(wl, x, W)


def test_zero_router_tie_break():
    wl = synth.WORKLOADS["tiny"]
    x, W = gen(wl, 0)
    W["router_w"] = np.zeros_like(W["router_w"])
    out, ref, _ = full_check(wl, x, W)
    assert (out["idx"] == np.arange(wl.top_k)[None, :]).all()      # order too: all logits tie
    assert np.all(np.abs(out["gates"] - 1.0 / wl.top_k) <= 1e-7)


def test_split_rows_large_tiles_zipf():
    # > 48 rows per expert with a skewed router: the large-tile path with rows
    # split by gate (hi + lo rows first), ragged tiles of both classes
    wl = small_wl(T=400, d=256, latent=128, n_experts=32, top_k=5, expert_hidden=192,
                  shared_hidden=256, router="zipf")
    x, W = gen(wl, 16)
    log("split rows, large tiles, zipf", wl)
    full_check(wl, x, W)


@pytest.mark.parametrize("T,N,K,path", [
    (40, 1024, 64, "stream"),     # N = 1024 (the 16-slot top-K kernel), K = 64, 2.5 rows per expert
    (1500, 1024, 40, "tiles"),    # N = 1024 with ~59 rows per expert: large tiles, two row classes
    (40, 2048, 64, "stream"),     # 32 slots per lane, two experts per bucketing thread
    (40, 4096, 64, "stream"),     # N = 4096: 64 slots per lane, four experts per bucketing thread
    (3200, 4096, 64, "tiles"),    # N = 4096 at 50 rows per expert: chunked bucketing, large tiles
    (50, 16, 1, "stream"),        # K = 1: each token's gate is 1
    (2100, 16, 1, "tiles"),       # K = 1 at ~131 rows per expert: every row paired (hi + lo)
    (300, 128, 64, "tiles"),      # K = 64 at 150 rows per expert: flat gates, most rows paired
])
def test_extreme_expert_counts(T, N, K, path):
    """The widest expert count and top-K the boundary accepts (N = 4096, K = 64), the
    top-K kernel's slot counts and K = 1, on the streaming and the large-tile expert
    paths."""
    wl = small_wl(T=T, d=256, latent=64, n_experts=N, top_k=K, expert_hidden=128, shared_hidden=256)
    avg = T * K / N
    assert (avg > 48) == (path == "tiles")
    x, W = gen(wl, 31 + K)
    log("extreme expert counts", wl)
    out, ref, _ = full_check(wl, x, W)
    if K == 1:
        assert np.all(out["gates"] == 1.0)


def test_zipf_bias_router():
    wl = small_wl(T=40, n_experts=32, top_k=5, router="zipf")
    x, W = gen(wl, 7)
    full_check(wl, x, W)


def test_fp4_experts_small():
    wl = small_wl(T=24, d=256, latent=128, n_experts=16, top_k=4, expert_hidden=192,
                  shared_hidden=256, experts="fp4")
    x, W = gen(wl, 8)
    full_check(wl, x, W, tol=3e-2)


@pytest.mark.parametrize("experts,shared,proj", [("bf16", "fp4", "bf16"), ("bf16", "bf16", "fp8"),
                                                 ("fp4", "fp4", "fp8")])
def test_precision_mix_stream_path(experts, shared, proj):
    # <= 64 tokens: the FP4 shared expert and FP8 projections are streamed and decoded
    # in registers; d = 512 splits the K = d GEMMs in two (partials, then the reduce
    # applies the tensor scale)
    wl = small_wl(T=40, d=512, latent=128, n_experts=32, top_k=4, expert_hidden=192,
                  shared_hidden=320, experts=experts, shared=shared, proj=proj)
    x, W = gen(wl, 17)
    log("precision mix, stream path", wl)
    full_check(wl, x, W, tol=tolerance(wl))


def test_precision_mix_tiled_path():
    # > 64 tokens: dense GEMMs on the LDS-tiled kernel read the bf16 values expanded
    # at init, the tensor scales still applied in the epilogues; then a 40-token call
    # on the same handle streams the stored bytes
    wl = small_wl(T=300, d=256, latent=128, n_experts=32, top_k=8, expert_hidden=192,
                  shared_hidden=320, shared="fp4", proj="fp8")
    x, W = gen(wl, 18)
    log("precision mix, tiled path", wl)
    full_check(wl, x, W, tol=tolerance(wl))
    wl40 = wl.replace(T=40)
    full_check(wl40, x[:40], W, tol=tolerance(wl), max_tokens=300)


@pytest.mark.parametrize("n_experts", [32, 256])
def test_chunked_bucketing(n_experts):
    # 1100 tokens x 8 rows: more rows than one workgroup places and 69 mask blocks, so
    # the prefix runs in 5 chunks of 16 blocks (the last one partial); 32 experts put
    # ~275 rows on each (large tiles, two row classes), 256 experts ~34 (64-row streaming
    # tiles, one class).  Every token's output and the whole permutation are checked.
    wl = small_wl(T=1100, d=256, latent=64, n_experts=n_experts, top_k=8, expert_hidden=128,
                  shared_hidden=256)
    x, W = gen(wl, 21)
    log("chunked bucketing", wl)
    full_check(wl, x, W)


def test_workspace_allocation_failure(monkeypatch):
    """LATENTMOE_FAIL_ALLOC=1 makes init's workspace allocation fail: init returns
    OUT_OF_MEMORY and hands out no handle; without it the same weights initialise
    and the layer runs."""
    import torch
    wl = synth.WORKLOADS["tiny"]
    x, W = gen(wl, 0)
    Wd = binding.upload_weights(W)
    monkeypatch.setenv("LATENTMOE_FAIL_ALLOC", "1")
    with pytest.raises(binding.LatentMoEError) as e:
        binding.LatentMoE(wl, Wd, max_tokens=wl.T)
    assert e.value.status == binding.LATENTMOE_ERR_OUT_OF_MEMORY
    monkeypatch.delenv("LATENTMOE_FAIL_ALLOC")
    layer = binding.LatentMoE(wl, Wd, max_tokens=wl.T)
    y, idx, g = layer.forward(binding.to_device(x))
    torch.cuda.synchronize()
    ref = oracle.forward(x, W, wl.top_k)
    assert np.max(np.abs(y.cpu().numpy() - ref["y"])) <= 1e-2 * np.sqrt(np.mean(ref["y"] ** 2))
    layer.close()


def test_edge_token_counts_and_reuse():
    import torch
    wl = small_wl(T=33, d=256, latent=64, n_experts=16, top_k=4)
    x, W = gen(wl, 9)
    ref = oracle.forward(x, W, wl.top_k)
    Wd = binding.upload_weights(W)
    layer = binding.LatentMoE(wl, Wd, max_tokens=33)
    xd = binding.to_device(x)
    stream = torch.cuda.current_stream().cuda_stream
    # T = 0 is a no-op; T > max_tokens is rejected before any work
    y0 = torch.full((1, wl.d), 7.0, device="cuda")
    binding.latentmoe_forward(layer.h, xd.data_ptr(), 0, y0.data_ptr(), 0, 0, stream)
    with pytest.raises(binding.LatentMoEError) as e:
        binding.latentmoe_forward(layer.h, xd.data_ptr(), 34, y0.data_ptr(), 0, 0, stream)
    assert e.value.status == binding.LATENTMOE_ERR_INVALID_ARG
    # full, then smaller T (first row, odd count), then full again
    for T in (33, 1, 17, 33):
        y, idx, g = layer.forward(xd[:T])
        torch.cuda.synchronize()
        rms = np.sqrt(np.mean(ref["y"][:T] ** 2))
        assert np.max(np.abs(y.cpu().numpy() - ref["y"][:T])) <= 1e-2 * rms
        assert [sorted(r) for r in idx.cpu().numpy().tolist()] == [sorted(r) for r in ref["idx"][:T].tolist()]
    assert float(y0[0, 0]) == 7.0
    layer.close()


# ---- full sizes: every token's top-K, bucketing and output against the oracle ----

def test_super_decode_full():
    full_size_check("super_decode", 1e-2)


def test_super_fp4_full():
    full_size_check("super_fp4", 3e-2)


def test_super_recipe_full():
    # FP4 experts and shared expert, FP8 W_down / W_up, 1024 tokens
    full_size_check("super_recipe", tolerance(synth.WORKLOADS["super_recipe"]))


def test_super_recipe_decode():
    # the same weights at a 64-token decode step: every dense GEMM streams its stored format
    full_size_check("super_recipe", tolerance(synth.WORKLOADS["super_recipe"]), T=64)


def test_super_prefill_full():
    full_size_check("super_prefill", 1e-2)


def test_ultra_full():
    full_size_check("ultra", 1e-2)


def test_graph_replay_matches_eager_and_oracle():
    """latentmoe_forward_graph: replays see new buffer contents, equal the eager
    forward bit for bit, and a new T re-captures."""
    import torch
    wl = small_wl(T=40, d=256, latent=128, n_experts=32, top_k=4, expert_hidden=128, shared_hidden=256)
    xa, W = gen(wl, 11)
    xb, _ = gen(wl, 12)
    Wd = binding.upload_weights(W)
    layer = binding.LatentMoE(wl, Wd, max_tokens=wl.T)
    xd = binding.to_device(xa)
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.T, wl.top_k), dtype=torch.int32, device="cuda")
    g = torch.empty((wl.T, wl.top_k), dtype=torch.float32, device="cuda")
    for rep, xs in enumerate([xa, xb, xa, xb, xa]):
        xd.copy_(binding.to_device(xs))
        layer.forward(xd, y, idx, g, graph=True)
        torch.cuda.synchronize()
        yg, ig, gg = y.clone(), idx.clone(), g.clone()
        ye, ie, ge = layer.forward(xd)                 # eager, fresh outputs
        torch.cuda.synchronize()
        assert torch.equal(yg, ye) and torch.equal(ig, ie) and torch.equal(gg, ge), rep
        ref = oracle.forward(xs, W, wl.top_k)
        rms = np.sqrt(np.mean(ref["y"] ** 2))
        assert np.max(np.abs(yg.cpu().numpy() - ref["y"])) <= 1e-2 * rms
    # a smaller T (new arguments) re-captures; then the original again
    for T in (17, 40):
        y2, i2, g2 = layer.forward(xd[:T], graph=True)
        torch.cuda.synchronize()
        ref = oracle.forward(xa[:T], W, wl.top_k)
        assert np.max(np.abs(y2.cpu().numpy() - ref["y"])) <= 1e-2 * np.sqrt(np.mean(ref["y"] ** 2))
    layer.close()


@pytest.mark.parametrize("T,experts,shared,proj", [
    (37, "bf16", "bf16", "bf16"),   # decode-sized path: one stream, stacked GEMMs
    (600, "bf16", "bf16", "bf16"),  # large-tile path: > 64 tokens, > 48 rows per expert, two row classes
    (40, "fp4", "fp4", "fp8"),      # the released precision mix on the streaming kernels
    (300, "fp4", "fp4", "fp8"),     # the mix above 64 tokens: LDS-staged FP4 expert kernel
])
def test_widths_multiple_of_16(T, experts, shared, proj):
    """d, l, m, m_s multiples of 16 (the FP4 block) but not of 64: the layer runs on
    zero-padded weight copies at the widths rounded up to 64 and crops y; z, y_lat
    and the bucketing come back at the caller's widths and match the oracle run at
    the caller's widths.  Graph replay (the padding and cropping copies captured
    with the forward) equals the eager forward bit for bit."""
    import torch
    wl = small_wl(T=T, d=208, latent=80, n_experts=32, top_k=4, expert_hidden=112, shared_hidden=144,
                  experts=experts, shared=shared, proj=proj)
    x, W = gen(wl, 21)
    log("padded widths", wl)
    full_check(wl, x, W, tol=tolerance(wl))
    Wd = binding.upload_weights(W)
    layer = binding.LatentMoE(wl, Wd, max_tokens=wl.T)
    xd = binding.to_device(x)
    ye, ie, ge = layer.forward(xd)
    yg, ig, gg = layer.forward(xd, graph=True)
    torch.cuda.synchronize()
    assert torch.equal(yg, ye) and torch.equal(ig, ie) and torch.equal(gg, ge)
    layer.close()


def test_graph_replay_large_tiles():
    """The large-tile path with two row classes in a graph (the hi class's expert
    down runs on a side stream beside the other class's expert up): every replay
    equals the eager forward bit for bit, and the oracle within the bar."""
    import torch
    wl = small_wl(T=1100, d=256, latent=64, n_experts=32, top_k=8, expert_hidden=128, shared_hidden=256)
    x, W = gen(wl, 23)
    Wd = binding.upload_weights(W)
    layer = binding.LatentMoE(wl, Wd, max_tokens=wl.T)
    xd = binding.to_device(x)
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.T, wl.top_k), dtype=torch.int32, device="cuda")
    g = torch.empty((wl.T, wl.top_k), dtype=torch.float32, device="cuda")
    for rep in range(3):
        y.fill_(float("nan"))
        layer.forward(xd, y, idx, g, graph=True)
        torch.cuda.synchronize()
        ye, ie, ge = layer.forward(xd)
        torch.cuda.synchronize()
        assert torch.equal(y, ye) and torch.equal(idx, ie) and torch.equal(g, ge), rep
    ref = oracle.forward(x, W, wl.top_k)
    rms = np.sqrt(np.mean(ref["y"] ** 2))
    err = np.max(np.abs(y.cpu().numpy() - ref["y"]))
    log("large-tile graph replay: max|gpu-oracle| / rms = %.2e" % (err / rms))
    assert err <= 1e-2 * rms
    layer.close()


def test_stage_timing_keeps_outputs():
    """Stage-timed forwards (latentmoe_profile_begin) run every stage in program
    order on the caller's stream, where untimed ones fork side streams (W_down, the
    shared expert, and on the large-tile path the hi class's expert down beside the
    other class's expert up): both give the same outputs bit for bit, and every
    stage reports a time."""
    import torch
    wl = small_wl(T=1100, d=256, latent=64, n_experts=32, top_k=8, expert_hidden=128, shared_hidden=256)
    x, W = gen(wl, 24)
    Wd = binding.upload_weights(W)
    layer = binding.LatentMoE(wl, Wd, max_tokens=wl.T)
    xd = binding.to_device(x)
    y0, i0, g0 = layer.forward(xd)
    torch.cuda.synchronize()
    layer.profile_begin(2)
    for _ in range(2):
        y1, i1, g1 = layer.forward(xd)
    stages, calls = layer.profile_end()
    torch.cuda.synchronize()
    assert calls == 2
    assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(g0, g1)
    log("stage ms over 2 calls: %s" % {k: round(v, 4) for k, v in stages.items()})
    assert all(v > 0 for v in stages.values()), stages
    layer.close()


def test_super_verify_sweep():
    """Speculative-verify decode batches at Super shapes, T = users x 8 from 8 to
    512 (prefixes of one 512-token batch; the 16-, 32- and 64-row expert tiles):
    every token's top-K, exact bucketing and output, eager and graph."""
    import torch
    wl = synth.WORKLOADS["super_verify"]
    x, W = synth.make(wl, 0, redraws=synth.load_redraws("super_verify", 0))
    logits = oracle.router_logits(x, W["router_w"], W["router_bias"])
    assert np.all(oracle.topk_gap(logits, wl.top_k) >= 1e-4)
    ref_idx = oracle.select_topk(logits, wl.top_k)
    ref_g = oracle.softmax_selected(logits, ref_idx)
    Ts = (8, 16, 24, 40, 64, 128, 256, 512)
    # a token's output does not depend on the batch it is in: one oracle pass over
    # the 512-token batch serves every prefix
    ref_y = oracle_y_chunked(x, W, wl.top_k, label="verify sweep")
    Wd = binding.upload_weights(W)
    layer = binding.LatentMoE(wl, Wd, max_tokens=wl.T)
    xd = binding.to_device(x)
    K, L = wl.top_k, wl.latent
    for T in Ts:
        for graph in (False, True):
            y, idx, g = layer.forward(xd[:T], graph=graph)
            counts = layer.intermediate("counts", (wl.n_experts,), torch.int32)
            offsets = layer.intermediate("offsets", (wl.n_experts + 1,), torch.int32)
            row_src = layer.intermediate("row_src", (T * K,), torch.int32)
            inv = layer.intermediate("inv", (T * K,), torch.int32)
            torch.cuda.synchronize()
            idx_h = idx.cpu().numpy()
            check_topk(idx_h, g.cpu().numpy(), ref_idx[:T], ref_g[:T])
            check_bucketing(dict(counts=counts.cpu().numpy(), offsets=offsets.cpu().numpy(),
                                 row_src=row_src.cpu().numpy(), inv=inv.cpu().numpy()),
                            idx_h, wl.n_experts, K)
            check_y(y.cpu().numpy().astype(np.float64), ref_y[:T], 1e-2)
            log("verify sweep: T=%d graph=%s ok" % (T, graph))
    layer.close()
