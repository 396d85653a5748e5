"""Seeded synthetic inputs for the LatentMoE layer forward.

This module only *draws and encodes* numbers: it holds none of the layer's
arithmetic (no logits, no top-K, no projections).  Both the HIP path and the
fp64 oracle consume the bytes it produces; each of them decodes those bytes
with its own code.

Shapes follow the LatentMoE description and the Super shape table in
"Nemotron 3 Super: Open, Efficient Mixture-of-Experts Hybrid Mamba-Transformer
Model for Agentic Reasoning" (section 3.1 table, section 3.2), and the Ultra
expert counts in "Nemotron 3 Ultra" (method section).

Recipe (one independent PCG64 stream per tensor, and per expert / per token row):

* bf16 tensors: float32 standard normal draws times ``1/sqrt(fan_in)`` (in
  float32), rounded to bf16 with round-to-nearest-even.  Activations ``x`` use
  std 1.
* router weight: float32 normal draws times ``1/sqrt(d)``, kept in float32.
* Zipf router bias (prefill workload): a seeded permutation gives each expert a
  rank r in 1..N; the bias is ``r**-1.1`` standardised to mean 0 and
  population std 1, stored as float32.
* FP4 expert weights: bf16 masters drawn as above, then encoded as E2M1 codes
  with one E4M3 scale per 16 consecutive input-dim elements and one float32
  scale per expert matrix (``encode_fp4``).
* token rows can be redrawn one at a time: row ``t`` at attempt ``a`` comes from
  its own stream, so a caller may replace rows without touching the others.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                # tokens
    d: int                # model width
    latent: int           # latent width (ell)
    n_experts: int        # N
    top_k: int            # K
    expert_hidden: int    # m
    shared_hidden: int    # m_s
    router: str = "normal"   # "normal" | "zipf" (adds a Zipf(1.1) per-expert bias)
    experts: str = "bf16"    # "bf16" | "fp4"
    shared: str = "bf16"     # "bf16" | "fp4" (the shared expert's two matrices)
    proj: str = "bf16"       # "bf16" | "fp8" (W_down and W_up, per-tensor scale)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny correctness case
    "tiny": Workload("tiny", T=8, d=256, latent=64, n_experts=16, top_k=4,
                     expert_hidden=128, shared_hidden=256),
    # Super layer shapes (Nemotron 3 Super, section 3.1 table), decode step
    "super_decode": Workload("super_decode", T=64, d=4096, latent=1024, n_experts=512,
                             top_k=22, expert_hidden=2688, shared_hidden=5376),
    # Super shapes, 8K-token prefill chunk with a skewed (Zipf) router
    "super_prefill": Workload("super_prefill", T=8192, d=4096, latent=1024, n_experts=512,
                              top_k=22, expert_hidden=2688, shared_hidden=5376,
                              router="zipf"),
    # Ultra expert shapes (Nemotron 3 Ultra, method section); d and ell chosen here
    "ultra": Workload("ultra", T=256, d=8192, latent=2048, n_experts=512, top_k=22,
                      expert_hidden=5120, shared_hidden=10240),
    # Super decode shapes at the speculative-verify batch sizes: T = users x 8
    # (a draft of 7 plus the verified token); smaller T are prefixes of this batch
    "super_verify": Workload("super_verify", T=512, d=4096, latent=1024, n_experts=512,
                             top_k=22, expert_hidden=2688, shared_hidden=5376),
    # Super shapes with block-scaled FP4 expert weights
    "super_fp4": Workload("super_fp4", T=1024, d=4096, latent=1024, n_experts=512,
                          top_k=22, expert_hidden=2688, shared_hidden=5376,
                          experts="fp4"),
    # Super shapes in the released precision mix: FP4 experts and shared expert,
    # FP8 W_down / W_up (x and router as in super_fp4)
    "super_recipe": Workload("super_recipe", T=1024, d=4096, latent=1024, n_experts=512,
                             top_k=22, expert_hidden=2688, shared_hidden=5376,
                             experts="fp4", shared="fp4", proj="fp8"),
}

@dataclasses.dataclass(frozen=True)
class SsmWorkload:
    """Mamba-2 speculative-verify step: R requests, each verifying T tokens (the
    drafts plus the verified token) against a checkpoint and a record buffer."""
    name: str
    R: int            # requests
    T: int            # tokens verified per request
    H: int            # heads
    G: int            # groups (heads of a group share key and query)
    P: int            # head dimension
    N: int            # state dimension
    cap: int = 16     # buffer capacity: records between checkpoints

    def replace(self, **kw) -> "SsmWorkload":
        return dataclasses.replace(self, **kw)


SSM_WORKLOADS = {
    "ssm_tiny": SsmWorkload("ssm_tiny", R=3, T=4, H=8, G=2, P=64, N=128, cap=8),
    # Super's Mamba shapes ("Nemotron 3 Super", section 3.1 table), 64 users each
    # verifying 7 drafts + 1 token, 16-record buffer
    "super_mamba_verify": SsmWorkload("super_mamba_verify", R=64, T=8, H=128, G=8, P=64,
                                      N=128, cap=16),
}


# stream identifiers (one PCG64 stream per tensor / expert / row)
TID_X = 1
TID_ROUTER_W = 2
TID_ROUTER_BIAS = 3
TID_W_DOWN = 4
TID_W_UP = 5
TID_EXPERT_W1 = 6
TID_EXPERT_W2 = 7
TID_SHARED_W1 = 8
TID_SHARED_W2 = 9

TID_SSM_STATE = 20
TID_SSM_K = 21
TID_SSM_V = 22
TID_SSM_Q = 23
TID_SSM_DT = 24
TID_SSM_A = 25
TID_SSM_LEN = 26

FP4_BLOCK = 16


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# encodings (bit-level, RNE)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even. Finite inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_positive_table() -> np.ndarray:
    """float32 value of each E4M3FN code 0..126 (positive, finite)."""
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return vals


_E4M3_POS = _e4m3_positive_table()
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _rne_encode(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Nearest code of a sorted positive table; ties go to the even code.
    Values above the last entry saturate to it."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(table, mag, side="left")          # table[hi-1] < mag <= table[hi]
    hi = np.clip(hi, 1, len(table) - 1)
    lo = hi - 1
    dlo = mag - table[lo]
    dhi = table[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag >= table[-1], len(table) - 1, code)
    code = np.where(mag <= 0.0, 0, code)
    return code.astype(np.uint8)


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Non-negative float -> E4M3FN code (RNE, saturating at 448)."""
    return _rne_encode(v, _E4M3_POS)


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """float -> 4-bit E2M1 code (sign in bit 3), RNE, clamped to +-6; zero -> 0x0."""
    v = np.asarray(v, dtype=np.float64)
    code = _rne_encode(np.abs(v), _E2M1_POS)
    sign = ((v < 0) & (code != 0)).astype(np.uint8) << 3
    return (code | sign).astype(np.uint8)


def encode_fp4(w_bf16: np.ndarray):
    """Encode one expert matrix [rows, cols] (bf16 bits) in the block-scaled FP4 format.

    Blocks are 16 consecutive elements along ``cols`` (the input dimension).
    Returns (packed codes [rows, cols//2] u8, block scales [rows, cols//16] u8 (E4M3FN),
    tensor scale (float32)).  Element 2j sits in the low nibble of byte j.
    """
    w = bf16_bits_to_f32(w_bf16)
    rows, cols = w.shape
    assert cols % FP4_BLOCK == 0
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    ts = np.float32(amax / np.float32(6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    if ts == 0:  # amax tiny enough to underflow
        ts = np.float32(1.0)
    blk = w.reshape(rows, cols // FP4_BLOCK, FP4_BLOCK)
    bmax = np.max(np.abs(blk), axis=2)
    sb_code = encode_e4m3((bmax / (np.float32(6.0) * ts)).astype(np.float32))
    sb = _E4M3_POS[sb_code].astype(np.float32)
    denom = (sb * ts).astype(np.float32)
    safe = np.where(denom > 0, denom, np.float32(1.0)).astype(np.float32)
    q = (blk / safe[:, :, None]).astype(np.float32)
    codes = encode_e2m1(q)
    codes = np.where((denom > 0)[:, :, None], codes, 0).astype(np.uint8)
    codes = codes.reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb_code, ts


def encode_fp8(w_bf16: np.ndarray):
    """Encode one matrix [rows, cols] (bf16 bits) as E4M3FN codes with one float32
    tensor scale: scale = amax / 448, code = RNE(w / scale) with the sign in bit 7.
    Returns (codes [rows, cols] u8, tensor scale (float32))."""
    w = bf16_bits_to_f32(w_bf16)
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    ts = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    if ts == 0:
        ts = np.float32(1.0)
    q = (w / ts).astype(np.float32)
    mag = encode_e4m3(np.abs(q))
    sign = ((q < 0) & (mag != 0)).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8), ts


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------


def _normal_bf16(seed: int, key: tuple, shape, std: float) -> np.ndarray:
    a = _rng(seed, *key).standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return f32_to_bf16_bits(a)


def x_row(seed: int, t: int, attempt: int, d: int) -> np.ndarray:
    """Token row t (bf16 bits), drawn from its own stream (seed, x, t, attempt)."""
    return _normal_bf16(seed, (TID_X, t, attempt), (d,), 1.0)


def make_x(wl: Workload, seed: int = 0, redraws: dict | None = None) -> np.ndarray:
    redraws = redraws or {}
    x = np.empty((wl.T, wl.d), dtype=np.uint16)
    for t in range(wl.T):
        x[t] = x_row(seed, t, int(redraws.get(t, 0)), wl.d)
    return x


def zipf_bias(n: int, seed: int) -> np.ndarray:
    perm = _rng(seed, TID_ROUTER_BIAS).permutation(n)
    rank = perm.astype(np.float64) + 1.0
    b = rank ** -1.1
    b = (b - b.mean()) / b.std()
    return b.astype(np.float32)


def make_router(wl: Workload, seed: int = 0) -> dict:
    """Router weight [N, d] float32 and optional bias [N] float32."""
    n, d = wl.n_experts, wl.d
    w = (_rng(seed, TID_ROUTER_W).standard_normal((n, d), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
    return {"router_w": w, "router_bias": zipf_bias(n, seed) if wl.router == "zipf" else None}


def load_redraws(name: str, seed: int, path: str | None = None) -> dict:
    """Row redraw table {row: attempt} for a workload and seed (empty if none stored)."""
    import json
    path = path or REDRAW_TABLE
    if not os.path.exists(path):
        return {}
    tab = json.load(open(path))
    return {int(r): int(a) for r, a in tab.get(name, {}).get(str(seed), {}).items()}


REDRAW_TABLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tests", "golden", "gap_redraws.json")


def make_weights(wl: Workload, seed: int = 0, threads: int | None = None) -> dict:
    """All layer weights as stored bytes (numpy, host)."""
    threads = threads or _threads()
    d, l, n, m, ms = wl.d, wl.latent, wl.n_experts, wl.expert_hidden, wl.shared_hidden
    W = make_router(wl, seed)
    W["w_down"] = _normal_bf16(seed, (TID_W_DOWN,), (l, d), 1.0 / np.sqrt(d))
    W["w_up"] = _normal_bf16(seed, (TID_W_UP,), (d, l), 1.0 / np.sqrt(l))
    W["shared_w1"] = _normal_bf16(seed, (TID_SHARED_W1,), (ms, d), 1.0 / np.sqrt(d))
    W["shared_w2"] = _normal_bf16(seed, (TID_SHARED_W2,), (d, ms), 1.0 / np.sqrt(ms))
    if wl.proj == "fp8":   # quantised from the same bf16 masters
        for k in ("w_down", "w_up"):
            W[k], ts = encode_fp8(W[k])
            W[k + "_tscale"] = np.array([ts], np.float32)
    elif wl.proj != "bf16":
        raise ValueError(wl.proj)
    if wl.shared == "fp4":
        for k in ("shared_w1", "shared_w2"):
            W[k], W[k + "_scale"], ts = encode_fp4(W[k])
            W[k + "_tscale"] = np.array([ts], np.float32)
    elif wl.shared != "bf16":
        raise ValueError(wl.shared)

    if wl.experts == "bf16":
        w1 = np.empty((n, m, l), dtype=np.uint16)
        w2 = np.empty((n, l, m), dtype=np.uint16)

        def one(e):
            w1[e] = _normal_bf16(seed, (TID_EXPERT_W1, e), (m, l), 1.0 / np.sqrt(l))
            w2[e] = _normal_bf16(seed, (TID_EXPERT_W2, e), (l, m), 1.0 / np.sqrt(m))

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n)))
        W["expert_w1"], W["expert_w2"] = w1, w2
    elif wl.experts == "fp4":
        c1 = np.empty((n, m, l // 2), dtype=np.uint8)
        s1 = np.empty((n, m, l // FP4_BLOCK), dtype=np.uint8)
        t1 = np.empty((n,), dtype=np.float32)
        c2 = np.empty((n, l, m // 2), dtype=np.uint8)
        s2 = np.empty((n, l, m // FP4_BLOCK), dtype=np.uint8)
        t2 = np.empty((n,), dtype=np.float32)

        def one(e):
            m1 = _normal_bf16(seed, (TID_EXPERT_W1, e), (m, l), 1.0 / np.sqrt(l))
            c1[e], s1[e], t1[e] = encode_fp4(m1)
            m2 = _normal_bf16(seed, (TID_EXPERT_W2, e), (l, m), 1.0 / np.sqrt(m))
            c2[e], s2[e], t2[e] = encode_fp4(m2)

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n)))
        W.update(expert_w1=c1, expert_w1_scale=s1, expert_w1_tscale=t1,
                 expert_w2=c2, expert_w2_scale=s2, expert_w2_tscale=t2)
    else:
        raise ValueError(wl.experts)
    return W


def make(wl: Workload | str, seed: int = 0, redraws: dict | None = None,
         threads: int | None = None):
    """(x bf16 bits [T,d], weights dict) for a workload."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    return make_x(wl, seed, redraws), make_weights(wl, seed, threads)


# --------------------------------------------------------------------------
# Mamba-2 verify inputs
# --------------------------------------------------------------------------


def make_ssm(wl: SsmWorkload, seed: int = 0) -> dict:
    """Checkpoint, record buffer (with n_buf records per request) and the T tokens
    to verify.  bf16 tensors as bit patterns, decays and lengths as fp32 / int32.

    checkpoint ~ N(0, 1); keys and queries ~ N(0, 1/N); values ~ N(0, 1); decays
    a = exp(-dt * A) with A ~ U[1, 16] per head and dt log-uniform on [1e-3, 1e-1]
    per token and head (the usual Mamba-2 ranges); n_buf ~ U{0 .. cap - T}.
    """
    R, T, H, G, P, N, C = wl.R, wl.T, wl.H, wl.G, wl.P, wl.N, wl.cap
    out = {"ckpt": _normal_bf16(seed, (TID_SSM_STATE,), (R, H, P, N), 1.0)}
    A = _rng(seed, TID_SSM_A).uniform(1.0, 16.0, H)

    def decays(key, L):
        u = _rng(seed, TID_SSM_DT, key).uniform(np.log(1e-3), np.log(1e-1), (R, L, H))
        return np.exp(-np.exp(u) * A).astype(np.float32)

    out["buf_k"] = _normal_bf16(seed, (TID_SSM_K, 0), (R, C, G, N), 1.0 / np.sqrt(N))
    out["buf_v"] = _normal_bf16(seed, (TID_SSM_V, 0), (R, C, H, P), 1.0)
    out["buf_a"] = decays(0, C)
    out["draft_q"] = _normal_bf16(seed, (TID_SSM_Q, 1), (R, T, G, N), 1.0 / np.sqrt(N))
    out["draft_k"] = _normal_bf16(seed, (TID_SSM_K, 1), (R, T, G, N), 1.0 / np.sqrt(N))
    out["draft_v"] = _normal_bf16(seed, (TID_SSM_V, 1), (R, T, H, P), 1.0)
    out["draft_a"] = decays(1, T)
    out["buf_len"] = _rng(seed, TID_SSM_LEN).integers(0, C - T + 1, R).astype(np.int32)
    return out
