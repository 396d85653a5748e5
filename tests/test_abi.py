"""The C-ABI library: it builds, loads without a GPU, and exports every
function that include/latentmoe.h and include/ssm_replay.h declare.  No compute
calls are made."""
import ctypes
import os
import re

import pytest

from sparse_moe_layer_logits_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "latentmoe.h")
SSM_HEADER = os.path.join(ROOT, "include", "ssm_replay.h")


def declared_functions(header=HEADER, prefix="latentmoe_"):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(%s[a-z0-9_]+)\s*\(" % prefix, text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("latentmoe_init", "latentmoe_forward", "latentmoe_destroy"):
        assert must in names
    assert set(names) == set(binding.EXPORTED)
    assert set(declared_functions(SSM_HEADER, "ssm_")) == set(binding.SSM_EXPORTED)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("liblatentmoe.so not built; run python -m sparse_moe_layer_logits_amd.build")
    return ctypes.CDLL(binding.LIB_PATH)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions() + declared_functions(SSM_HEADER, "ssm_"):
        assert hasattr(lib, name), name


def test_ssm_shape_checks_on_the_host(lib):
    ok = binding.ssm_shape(128, 8, 64, 128, 16)
    assert binding.ssm_check_shape(ok) == binding.SSM_OK
    for bad, st in ((binding.ssm_shape(128, 7, 64, 128, 16), binding.SSM_ERR_UNSUPPORTED),   # G does not divide H
                    (binding.ssm_shape(128, 8, 48, 128, 16), binding.SSM_ERR_UNSUPPORTED),   # head dim
                    (binding.ssm_shape(128, 8, 64, 96, 16), binding.SSM_ERR_UNSUPPORTED),    # state dim
                    (binding.ssm_shape(128, 8, 64, 128, 64), binding.SSM_ERR_UNSUPPORTED),   # capacity
                    (binding.ssm_shape(0, 8, 64, 128, 16), binding.SSM_ERR_INVALID_ARG)):
        assert binding.ssm_check_shape(bad) == st
    # argument checks happen before any device work
    with pytest.raises(binding.SsmError) as e:
        binding.ssm_replay_verify(ok, 1, 17, *([0] * 11))     # T above the capacity
    assert e.value.status == binding.SSM_ERR_INVALID_ARG
    with pytest.raises(binding.SsmError) as e:
        binding.ssm_replay_verify(ok, 1, 8, *([0] * 11))      # null pointers
    assert e.value.status == binding.SSM_ERR_INVALID_ARG
    with pytest.raises(binding.SsmError) as e:
        binding.ssm_replay_flush(ok, -1, *([0] * 6))
    assert e.value.status == binding.SSM_ERR_INVALID_ARG


def test_status_strings_and_host_side_validation(lib):
    # host-only entry points: no device work happens in these calls
    assert binding.status_string(0) == "ok"
    assert binding.status_string(-1) == "invalid argument"
    assert binding.status_string(12345) == "unknown status"
    cfg = binding.latentmoe_config(256, 64, 16, 4, 128, 256, 8, 0)
    n = binding.latentmoe_workspace_bytes(cfg)
    assert n > 0
    assert binding.latentmoe_workspace_bytes(binding.latentmoe_config(256, 64, 4096, 64, 128, 256, 8, 0)) > n
    bad = [binding.latentmoe_config(250, 64, 16, 4, 128, 256, 8, 0),   # d not a multiple of 16
           binding.latentmoe_config(256, 72, 16, 4, 128, 256, 8, 0),   # l not a multiple of 16
           binding.latentmoe_config(256, 64, 16, 17, 128, 256, 8, 0),  # K > N
           binding.latentmoe_config(256, 64, 20, 4, 128, 256, 8, 0),   # N not a multiple of 16
           binding.latentmoe_config(256, 64, 4112, 4, 128, 256, 8, 0),  # N above 4096
           binding.latentmoe_config(256, 64, 16, 4, 128, 256, 8, 7)]   # unknown format
    for c in bad:
        with pytest.raises(binding.LatentMoEError) as e:
            binding.latentmoe_workspace_bytes(c)
        assert e.value.status == binding.LATENTMOE_ERR_UNSUPPORTED
    with pytest.raises(binding.LatentMoEError) as e:
        binding.latentmoe_workspace_bytes(binding.latentmoe_config(256, 64, 16, 4, 128, 256, 0, 0))
    assert e.value.status == binding.LATENTMOE_ERR_INVALID_ARG
    # init rejects null weight pointers before touching the device
    w = binding.latentmoe_weights()
    with pytest.raises(binding.LatentMoEError) as e:
        binding.latentmoe_init(cfg, w, 0)
    assert e.value.status == binding.LATENTMOE_ERR_INVALID_ARG
    # forward / destroy on a null handle
    assert lib.latentmoe_forward(None, None, 1, None, None, None, None) == binding.LATENTMOE_ERR_INVALID_ARG
    assert lib.latentmoe_destroy(None) == 0


def test_widths_multiple_of_16_run_padded(lib):
    """Widths that are multiples of 16 but not of 64 are accepted: the layer runs
    at the widths rounded up to 64, on zero-padded copies of the weights plus a
    padded x and y buffer, so its workspace is that of the rounded widths and
    more.  The entry point that allocates nothing has no room for the copies and
    rejects such widths before any device work."""
    odd = binding.latentmoe_config(208, 80, 16, 4, 112, 144, 8, 0)
    rounded = binding.latentmoe_config(256, 128, 16, 4, 128, 192, 8, 0)
    assert binding.latentmoe_workspace_bytes(odd) > binding.latentmoe_workspace_bytes(rounded)
    fp4 = binding.latentmoe_config(208, 80, 16, 4, 112, 144, 8, 1)
    assert binding.latentmoe_workspace_bytes(fp4) > 0
    w = binding.latentmoe_weights()
    for name in ("router_w", "w_down", "w_up", "expert_w1", "expert_w2", "shared_w1", "shared_w2"):
        setattr(w, name, 4096)   # non-null; never dereferenced: the shape check comes first
    with pytest.raises(binding.LatentMoEError) as e:
        binding.latentmoe_forward_static(odd, w, 4096, 1, 4096, 0, 0, 0)
    assert e.value.status == binding.LATENTMOE_ERR_UNSUPPORTED


def test_32bit_activation_offsets_bound():
    """Configs whose activation matrices reach 2^31 elements are rejected (the
    large-tile kernels address rows with 32-bit offsets): at the Super shapes
    h = [T K, m] is the widest, 36314 tokens are accepted and 36315 are not."""
    ok = binding.latentmoe_config(4096, 1024, 512, 22, 2688, 5376, 36314, 0)
    assert binding.latentmoe_workspace_bytes(ok) > 0
    for cfg in (binding.latentmoe_config(4096, 1024, 512, 22, 2688, 5376, 36315, 0),
                binding.latentmoe_config(8192, 2048, 512, 22, 5120, 10240, 19066, 0),
                binding.latentmoe_config(1 << 16, 64, 16, 1, 64, 64, 1 << 15, 0)):
        with pytest.raises(binding.LatentMoEError) as e:
            binding.latentmoe_workspace_bytes(cfg)
        assert e.value.status == binding.LATENTMOE_ERR_UNSUPPORTED


def test_workspace_grows_with_max_tokens():
    a = binding.latentmoe_workspace_bytes(binding.latentmoe_config(4096, 1024, 512, 22, 2688, 5376, 64, 0))
    b = binding.latentmoe_workspace_bytes(binding.latentmoe_config(4096, 1024, 512, 22, 2688, 5376, 8192, 0))
    assert b > a
    assert b < 4 << 30   # the prefill workspace stays a few GB
