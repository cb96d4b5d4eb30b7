"""Python binding of the sampled-softmax loss (ctypes).  Argument marshalling
only: every function forwards to the C ABI in ``include/ssm.h`` of the same
name, inside the in-tree libngram.so; PyTorch supplies device memory and the
current HIP stream.  Importing this module raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libngram.so")

DIM = 768

FLAG_BAD_TARGET = 0x1
FLAG_OVERFLOW = 0x2
FLAG_BAD_PERM = 0x4
FLAG_BAD_CAND = 0x8
FLAG_BAD_SLOT = 0x10
FLAG_NO_LOGITS = 0x20

PROF_CAND = 0
PROF_FWD = 1
PROF_LSE = 2
PROF_TRANS = 3
PROF_DZ = 4
PROF_DX = 5
PROF_DW = 6
PROF_GROUPS = 7


class SsmConfig(ctypes.Structure):
    _fields_ = [
        ("vocab", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("candidates", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64),
    ]


def config(vocab: int, candidates: int, max_tokens: int) -> SsmConfig:
    c = SsmConfig()
    c.vocab = int(vocab)
    c.dim = DIM
    c.candidates = int(candidates)
    c.reserved = 0
    c.max_tokens = int(max_tokens)
    return c


class SsmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libngram is not built ({_LIB_PATH} missing): run "
                               "`python -m sparse_hashed_gram_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        cp = ctypes.POINTER(SsmConfig)
        sig = {
            "ssm_abi_version": ([], ctypes.c_int),
            "ssm_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "ssm_workspace_bytes": ([cp, vp], ctypes.c_int),
            "ssm_workspace_init": ([cp, vp, ctypes.c_uint64, vp], ctypes.c_int),
            "ssm_candidates": ([cp, vp, vp, i64, vp, vp, vp, vp], ctypes.c_int),
            "ssm_loss_fwd": ([cp, vp, vp, vp, vp, vp, i64, vp, vp, vp], ctypes.c_int),
            "ssm_loss_bwd": ([cp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp], ctypes.c_int),
            "ssm_device_status": ([cp, vp, vp, ctypes.c_int, vp], ctypes.c_int),
            "ssm_profile_events": ([ctypes.c_int, vp, vp], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


lib()   # fail at import time if the HIP library is missing: there is no fallback


def status_string(status: int) -> str:
    return lib().ssm_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise SsmError(fn, status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def workspace_bytes(cfg: SsmConfig) -> int:
    n = ctypes.c_uint64()
    _check("ssm_workspace_bytes", lib().ssm_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return int(n.value)


class Workspace:
    """Device workspace (a uint8 tensor, 256-byte aligned)."""

    def __init__(self, cfg: SsmConfig, device="cuda"):
        self.cfg = cfg
        self.nbytes = workspace_bytes(cfg)
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self._buf.data_ptr()) % 256
        self.tensor = self._buf[off:off + self.nbytes]
        _check("ssm_workspace_init", lib().ssm_workspace_init(
            ctypes.byref(cfg), self.ptr, self.nbytes, _stream()))

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr()


def candidates(cfg: SsmConfig, ws: Workspace, targets: torch.Tensor, perm: torch.Tensor,
               cand: torch.Tensor | None = None, slot: torch.Tensor | None = None):
    """(cand int32 [C], slot int32 [T]) of one batch."""
    T = targets.numel()
    cand = cand if cand is not None else torch.empty(cfg.candidates, dtype=torch.int32, device=targets.device)
    slot = slot if slot is not None else torch.empty(T, dtype=torch.int32, device=targets.device)
    _check("ssm_candidates", lib().ssm_candidates(
        ctypes.byref(cfg), ws.ptr, _dev(targets, "targets", torch.int32), T,
        _dev(perm, "perm", torch.int32, (cfg.vocab,)), _dev(cand, "cand", torch.int32, (cfg.candidates,)),
        _dev(slot, "slot", torch.int32, (T,)), _stream()))
    return cand, slot


def loss_fwd(cfg: SsmConfig, ws: Workspace, X: torch.Tensor, W: torch.Tensor, cand: torch.Tensor,
             slot: torch.Tensor, loss: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """(loss fp32 [T], lse fp32 [T])."""
    T = X.shape[0]
    loss = loss if loss is not None else torch.empty(T, dtype=torch.float32, device=X.device)
    lse = lse if lse is not None else torch.empty(T, dtype=torch.float32, device=X.device)
    _check("ssm_loss_fwd", lib().ssm_loss_fwd(
        ctypes.byref(cfg), ws.ptr, _dev(X, "X", torch.bfloat16, (T, DIM)),
        _dev(W, "W", torch.bfloat16, (cfg.vocab, DIM)), _dev(cand, "cand", torch.int32, (cfg.candidates,)),
        _dev(slot, "slot", torch.int32, (T,)), T, _dev(loss, "loss", torch.float32, (T,)),
        _dev(lse, "lse", torch.float32, (T,)), _stream()))
    return loss, lse


def loss_bwd(cfg: SsmConfig, ws: Workspace, X: torch.Tensor, W: torch.Tensor, cand: torch.Tensor,
             slot: torch.Tensor, lse: torch.Tensor, dloss: torch.Tensor, dW: torch.Tensor,
             dX: torch.Tensor | None = None):
    """dX (fp32 [T, 768], returned) and dW[cand] += ... in place (fp32 [V, 768]).

    Reads the logits the last loss_fwd on this workspace stored: call it after
    that forward with the same X, W, cand, slot (else FLAG_NO_LOGITS and zero
    gradients where the library can tell)."""
    T = X.shape[0]
    dX = dX if dX is not None else torch.empty((T, DIM), dtype=torch.float32, device=X.device)
    _check("ssm_loss_bwd", lib().ssm_loss_bwd(
        ctypes.byref(cfg), ws.ptr, _dev(X, "X", torch.bfloat16, (T, DIM)),
        _dev(W, "W", torch.bfloat16, (cfg.vocab, DIM)), _dev(cand, "cand", torch.int32, (cfg.candidates,)),
        _dev(slot, "slot", torch.int32, (T,)), _dev(lse, "lse", torch.float32, (T,)),
        _dev(dloss, "dloss", torch.float32, (T,)), T, _dev(dX, "dX", torch.float32, (T, DIM)),
        _dev(dW, "dW", torch.float32, (cfg.vocab, DIM)), _stream()))
    return dX


def device_status(cfg: SsmConfig, ws: Workspace, clear: bool = False) -> int:
    f = ctypes.c_uint32()
    _check("ssm_device_status", lib().ssm_device_status(
        ctypes.byref(cfg), ws.ptr, ctypes.byref(f), int(clear), _stream()))
    return int(f.value)


def profile_events(group: int, start, stop):
    """Attach raw hipEvent_t handles (ints) to a kernel group; None detaches."""
    _check("ssm_profile_events", lib().ssm_profile_events(group, start, stop))
