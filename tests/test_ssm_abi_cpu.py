"""CPU checks of the sampled-softmax C ABI (include/ssm.h): every declared
entry point is exported, the config mirror matches, and bad arguments are
rejected on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")


@pytest.fixture(scope="module")
def S():
    from sparse_hashed_gram_amd import ssm
    return ssm


def _declared():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(S):
    names = _declared()
    assert len(names) == 9
    L = ctypes.CDLL(S._LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in ssm.h but not exported"


def test_config_layout_and_version(S):
    assert ctypes.sizeof(S.SsmConfig) == 24 and S.SsmConfig.max_tokens.offset == 16
    assert S.lib().ssm_abi_version() == 2
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert S.status_string(s) not in ("", "unknown status")


@pytest.mark.parametrize("field,value", [("vocab", 0), ("dim", 512), ("candidates", 0),
                                         ("candidates", 50305), ("reserved", 1), ("max_tokens", 0),
                                         ("max_tokens", (1 << 24) + 1)])
def test_config_rejects(S, field, value):
    c = S.config(50304, 10240, 49152)
    setattr(c, field, value)
    n = ctypes.c_uint64()
    assert S.lib().ssm_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == -3


def test_workspace_bytes_scale(S):
    small = S.workspace_bytes(S.config(50304, 1024, 1024))
    big = S.workspace_bytes(S.config(50304, 10240, 49152))
    # the forward's fp16 exp(z - M) and dz in bf16 dominate: 4 T C bytes
    assert 4 * 49152 * 10240 < big < 4 * 49152 * 10240 * 1.15
    assert small < big
    assert S.workspace_bytes(S.config(50304, 10240, 49153)) > big   # T padded to 128


def test_host_rejections_enqueue_nothing(S):
    L = S.lib()
    c = S.config(1000, 100, 256)
    cp = ctypes.byref(c)
    ws = 1 << 20      # a fake, 256-byte aligned device address: never dereferenced on these paths
    p = 1 << 12
    assert L.ssm_candidates(cp, None, p, 10, p, p, p, None) == -1
    assert L.ssm_candidates(cp, ws, p, 10, None, p, p, None) == -1
    assert L.ssm_candidates(cp, ws + 8, p, 10, p, p, p, None) == -2
    assert L.ssm_candidates(cp, ws, p, 257, p, p, p, None) == -4
    assert L.ssm_candidates(cp, ws, p, -1, p, p, p, None) == -4
    assert L.ssm_candidates(cp, ws, p, 0, p, p, p, None) == 0          # T = 0: nothing to do
    assert L.ssm_loss_fwd(cp, ws, p + 2, p, p, p, 10, p, p, None) == -2  # X misaligned
    assert L.ssm_loss_fwd(cp, ws, p, p, p, p, 10, None, p, None) == -1
    assert L.ssm_loss_fwd(cp, ws, p, p, p, p, 300, p, p, None) == -4
    assert L.ssm_loss_bwd(cp, ws, p, p, p, p, p, p, 10, p + 4, p, None) == -2  # dX misaligned
    assert L.ssm_loss_bwd(cp, ws, p, p, p, p, None, p, 10, p, p, None) == -1
    assert L.ssm_profile_events(7, None, None) == -5
    assert L.ssm_profile_events(0, None, None) == 0
