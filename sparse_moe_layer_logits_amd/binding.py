"""ctypes binding of liblatentmoe.so (argument marshalling only).

The names mirror the C ABI in include/latentmoe.h.  PyTorch supplies device
memory and the stream; every step of the layer runs in the HIP library.  If
the library has not been built, loading fails with an error: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "liblatentmoe.so")

LATENTMOE_OK = 0
LATENTMOE_ERR_INVALID_ARG = -1
LATENTMOE_ERR_UNSUPPORTED = -2
LATENTMOE_ERR_OUT_OF_MEMORY = -3
LATENTMOE_ERR_HIP = -4
LATENTMOE_ERR_SCRATCH = -5
LATENTMOE_STATIC_SCRATCH_BYTES = 64 << 20

LATENTMOE_FORMAT_BF16 = 0
LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16 = 1
LATENTMOE_FORMAT_FP8_E4M3 = 2
LATENTMOE_EXPERTS_BF16 = LATENTMOE_FORMAT_BF16
LATENTMOE_EXPERTS_FP4_E2M1_E4M3_B16 = LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16

INTER = dict(z=0, y_lat=1, counts=2, offsets=3, row_src=4, inv=5, h=6, hs_hi=7, hs_lo=8, y_lat_lo=9, z_lo=10, h_lo=11,
             paired=12)
STAGES = ["router", "topk", "bucket", "down_proj", "expert_up", "expert_down", "combine",
          "shared_up", "shared_down", "up_proj"]

EXPORTED = [
    "latentmoe_init", "latentmoe_forward", "latentmoe_forward_graph", "latentmoe_destroy",
    "latentmoe_status_string",
    "latentmoe_workspace_bytes", "latentmoe_debug_copy", "latentmoe_profile_begin",
    "latentmoe_profile_end", "latentmoe_fp4_decode", "latentmoe_fp8_decode", "latentmoe_forward_static",
]
# include/ssm_replay.h: Mamba-2 checkpoint + replay verification
SSM_EXPORTED = ["ssm_check_shape", "ssm_replay_verify", "ssm_replay_commit", "ssm_replay_flush",
                "ssm_states_verify"]
SSM_OK = 0
SSM_ERR_INVALID_ARG = -1
SSM_ERR_UNSUPPORTED = -2
SSM_ERR_HIP = -4


class latentmoe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d", "latent", "n_experts", "top_k", "expert_hidden", "shared_hidden", "max_tokens",
        "expert_format", "shared_format", "proj_format")]


class latentmoe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_bias", "w_down", "w_up", "expert_w1", "expert_w2",
        "expert_w1_scale", "expert_w2_scale", "expert_w1_tscale", "expert_w2_tscale",
        "shared_w1", "shared_w2", "shared_w1_scale", "shared_w2_scale", "shared_w1_tscale",
        "shared_w2_tscale", "w_down_tscale", "w_up_tscale")]


class ssm_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("heads", "groups", "head_dim", "state_dim", "capacity")]


class LatentMoEError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("liblatentmoe.so is not built (%s); run "
                           "`python -m sparse_moe_layer_logits_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.latentmoe_init.argtypes = [ctypes.POINTER(latentmoe_config), ctypes.POINTER(latentmoe_weights),
                                   vp, ctypes.POINTER(vp)]
    lib.latentmoe_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.latentmoe_forward_graph.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.latentmoe_destroy.argtypes = [vp]
    lib.latentmoe_status_string.argtypes = [ctypes.c_int]
    lib.latentmoe_status_string.restype = ctypes.c_char_p
    lib.latentmoe_workspace_bytes.argtypes = [ctypes.POINTER(latentmoe_config), ctypes.POINTER(sz)]
    lib.latentmoe_debug_copy.argtypes = [vp, ctypes.c_int, vp, sz, vp]
    lib.latentmoe_profile_begin.argtypes = [vp, ctypes.c_int, ctypes.c_uint32]
    lib.latentmoe_profile_end.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_int)]
    lib.latentmoe_fp4_decode.argtypes = [vp, vp, ctypes.c_int64, vp, vp]
    lib.latentmoe_fp8_decode.argtypes = [vp, ctypes.c_int64, vp, vp]
    lib.latentmoe_forward_static.argtypes = [ctypes.POINTER(latentmoe_config), ctypes.POINTER(latentmoe_weights),
                                             vp, i32, vp, vp, vp, vp]
    sp = ctypes.POINTER(ssm_shape)
    lib.ssm_check_shape.argtypes = [sp]
    lib.ssm_replay_verify.argtypes = [sp, i32, i32] + [vp] * 11  # 10 pointers + stream
    lib.ssm_replay_commit.argtypes = [i32, vp, vp, vp]
    lib.ssm_replay_flush.argtypes = [sp, i32] + [vp] * 6  # 5 pointers + stream
    lib.ssm_states_verify.argtypes = [sp, i32, i32] + [vp] * 8  # 7 pointers + stream
    for name in EXPORTED + SSM_EXPORTED:
        if name != "latentmoe_status_string":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().latentmoe_status_string(int(status)).decode()


def _check(fn, st):
    if st != LATENTMOE_OK:
        raise LatentMoEError(fn, st)


# ---- thin wrappers with the C names ----

def latentmoe_workspace_bytes(cfg: latentmoe_config) -> int:
    n = ctypes.c_size_t(0)
    _check("latentmoe_workspace_bytes", load().latentmoe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def latentmoe_init(cfg: latentmoe_config, w: latentmoe_weights, stream: int) -> int:
    h = ctypes.c_void_p(0)
    _check("latentmoe_init", load().latentmoe_init(ctypes.byref(cfg), ctypes.byref(w),
                                                   ctypes.c_void_p(stream), ctypes.byref(h)))
    return h.value


def latentmoe_forward(h: int, x_ptr: int, T: int, y_ptr: int, idx_ptr: int, gate_ptr: int,
                      stream: int) -> None:
    _check("latentmoe_forward", load().latentmoe_forward(
        ctypes.c_void_p(h), ctypes.c_void_p(x_ptr), int(T), ctypes.c_void_p(y_ptr),
        ctypes.c_void_p(idx_ptr or None), ctypes.c_void_p(gate_ptr or None), ctypes.c_void_p(stream)))


def latentmoe_forward_graph(h: int, x_ptr: int, T: int, y_ptr: int, idx_ptr: int, gate_ptr: int,
                            stream: int) -> None:
    _check("latentmoe_forward_graph", load().latentmoe_forward_graph(
        ctypes.c_void_p(h), ctypes.c_void_p(x_ptr), int(T), ctypes.c_void_p(y_ptr),
        ctypes.c_void_p(idx_ptr or None), ctypes.c_void_p(gate_ptr or None), ctypes.c_void_p(stream)))


def latentmoe_forward_static(cfg: latentmoe_config, w: latentmoe_weights, x_ptr: int, T: int, y_ptr: int,
                             idx_ptr: int, gate_ptr: int, stream: int) -> None:
    _check("latentmoe_forward_static", load().latentmoe_forward_static(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.c_void_p(x_ptr), int(T), ctypes.c_void_p(y_ptr),
        ctypes.c_void_p(idx_ptr or None), ctypes.c_void_p(gate_ptr or None), ctypes.c_void_p(stream)))


def latentmoe_destroy(h: int) -> None:
    _check("latentmoe_destroy", load().latentmoe_destroy(ctypes.c_void_p(h)))


def latentmoe_debug_copy(h: int, which: int, dst_ptr: int, nbytes: int, stream: int) -> None:
    _check("latentmoe_debug_copy", load().latentmoe_debug_copy(
        ctypes.c_void_p(h), int(which), ctypes.c_void_p(dst_ptr), nbytes, ctypes.c_void_p(stream)))


def latentmoe_profile_begin(h: int, max_calls: int, stage_mask: int = (1 << 10) - 1) -> None:
    _check("latentmoe_profile_begin", load().latentmoe_profile_begin(ctypes.c_void_p(h), int(max_calls),
                                                                     int(stage_mask)))


def latentmoe_profile_end(h: int) -> tuple[list, int]:
    ms = (ctypes.c_float * len(STAGES))()
    calls = ctypes.c_int(0)
    _check("latentmoe_profile_end", load().latentmoe_profile_end(
        ctypes.c_void_p(h), ms, len(STAGES), ctypes.byref(calls)))
    return list(ms), calls.value


def latentmoe_fp4_decode(codes_ptr: int, scales_ptr: int, n_blocks: int, out_ptr: int, stream: int) -> None:
    _check("latentmoe_fp4_decode", load().latentmoe_fp4_decode(
        ctypes.c_void_p(codes_ptr), ctypes.c_void_p(scales_ptr), int(n_blocks),
        ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream)))


def latentmoe_fp8_decode(codes_ptr: int, n_groups: int, out_ptr: int, stream: int) -> None:
    _check("latentmoe_fp8_decode", load().latentmoe_fp8_decode(
        ctypes.c_void_p(codes_ptr), int(n_groups), ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream)))


class SsmError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed with status %d" % (fn, status))
        self.status = status


def _ssm_check(fn, st):
    if st != SSM_OK:
        raise SsmError(fn, st)


def _vp(x):
    return ctypes.c_void_p(int(x))


def ssm_check_shape(shape: ssm_shape) -> int:
    return load().ssm_check_shape(ctypes.byref(shape))


def ssm_replay_verify(shape, R, T, ckpt, buf_k, buf_v, buf_a, buf_len, q, k, v, a, y, stream):
    """Device pointers (ints); see include/ssm_replay.h."""
    _ssm_check("ssm_replay_verify", load().ssm_replay_verify(
        ctypes.byref(shape), int(R), int(T), *[_vp(x) for x in (ckpt, buf_k, buf_v, buf_a, buf_len,
                                                                q, k, v, a, y, stream)]))


def ssm_replay_commit(R, accepted, buf_len, stream):
    _ssm_check("ssm_replay_commit", load().ssm_replay_commit(
        int(R), _vp(accepted), _vp(buf_len), _vp(stream)))


def ssm_replay_flush(shape, R, ckpt, buf_k, buf_v, buf_a, buf_len, stream):
    _ssm_check("ssm_replay_flush", load().ssm_replay_flush(
        ctypes.byref(shape), int(R), *[_vp(x) for x in (ckpt, buf_k, buf_v, buf_a, buf_len, stream)]))


def ssm_states_verify(shape, R, T, state, q, k, v, a, states_out, y, stream):
    _ssm_check("ssm_states_verify", load().ssm_states_verify(
        ctypes.byref(shape), int(R), int(T), *[_vp(x) for x in (state, q, k, v, a, states_out, y,
                                                                stream)]))


# ---- torch-facing convenience layer ----

def _torch():
    import torch
    return torch


def to_device(a: np.ndarray | None, device="cuda"):
    """numpy (bf16 bits as uint16, fp32, uint8) -> torch device tensor of the same bytes."""
    if a is None:
        return None
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def upload_weights(W: dict, device="cuda") -> dict:
    return {k: to_device(v, device) for k, v in W.items()}


def _ptr(t):
    return 0 if t is None else t.data_ptr()


class LatentMoE:
    """A layer handle over device weights (a dict of torch tensors as produced
    by ``upload_weights``).  The tensors are kept referenced for the handle's
    lifetime, as the C ABI borrows them."""

    def __init__(self, dims, Wd: dict, max_tokens: int, stream=None):
        torch = _torch()
        self.dims = dims
        self.Wd = Wd
        def has(k):
            return Wd.get(k) is not None

        # the stored formats follow from which scale tensors are present
        self.cfg = latentmoe_config(
            dims.d, dims.latent, dims.n_experts, dims.top_k, dims.expert_hidden,
            dims.shared_hidden, int(max_tokens),
            LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16 if has("expert_w1_scale") else LATENTMOE_FORMAT_BF16,
            LATENTMOE_FORMAT_FP4_E2M1_E4M3_B16 if has("shared_w1_scale") else LATENTMOE_FORMAT_BF16,
            LATENTMOE_FORMAT_FP8_E4M3 if has("w_down_tscale") else LATENTMOE_FORMAT_BF16)
        w = latentmoe_weights()
        for name, _ in latentmoe_weights._fields_:
            setattr(w, name, _ptr(Wd.get(name)) or None)
        self.w = w
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.h = latentmoe_init(self.cfg, w, self.stream.cuda_stream)
        self.device = next(v for v in Wd.values() if v is not None).device

    def forward(self, x, y=None, idx=None, gates=None, graph=False):
        """x: [T, d] int16 (bf16 bits) device tensor.  Returns (y fp32, idx int32, gates fp32).
        graph=True replays a captured HIP graph (latentmoe_forward_graph)."""
        torch = _torch()
        T = x.shape[0]
        K = self.dims.top_k
        if y is None:
            y = torch.empty((T, self.dims.d), dtype=torch.float32, device=self.device)
        if idx is None:
            idx = torch.empty((T, K), dtype=torch.int32, device=self.device)
        if gates is None:
            gates = torch.empty((T, K), dtype=torch.float32, device=self.device)
        fn = latentmoe_forward_graph if graph else latentmoe_forward
        fn(self.h, x.data_ptr(), T, y.data_ptr(), _ptr(idx), _ptr(gates), self.stream.cuda_stream)
        return y, idx, gates

    def intermediate(self, which: str, shape, dtype):
        torch = _torch()
        out = torch.empty(shape, dtype=dtype, device=self.device)
        latentmoe_debug_copy(self.h, INTER[which], out.data_ptr(), out.numel() * out.element_size(),
                             self.stream.cuda_stream)
        return out

    def profile_begin(self, max_calls: int, stages=None):
        mask = (1 << len(STAGES)) - 1 if stages is None else sum(1 << STAGES.index(s) for s in stages)
        latentmoe_profile_begin(self.h, max_calls, mask)

    def profile_end(self):
        ms, calls = latentmoe_profile_end(self.h)
        return dict(zip(STAGES, ms)), calls

    def close(self):
        if self.h:
            latentmoe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
