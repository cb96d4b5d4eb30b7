"""Python binding of libngram (ctypes).  Argument marshalling only.

Every function here forwards to the C ABI in ``include/ngram.h`` of the same
name; PyTorch only supplies device memory and the current HIP stream.  There
is no fallback: if the HIP library has not been built, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libngram.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
MODE_SPREAD = 0
MODE_BURST = 1
MODE_BURST_REF = 2
OPT_PRESORT = 0x1
OPT_OUT_F32 = 0x2
OPT_DIRECT = 0x4
OPT_NEST_ALWAYS = 0x8
_MODES = {"spread": MODE_SPREAD, "burst": MODE_BURST, "burst_ref": MODE_BURST_REF}

FLAG_BAD_TOKEN = 0x1
FLAG_WINDOW_FULL = 0x2
FLAG_STASH_FULL = 0x4
FLAG_STEP_ORDER = 0x8
FLAG_BAD_PARAMS = 0x10
FLAG_WINDOW_UNREADY = 0x20
FLAG_KEYS_MISMATCH = 0x40

PROF_FWD = 0
PROF_SORT = 1
PROF_REDUCE = 2
PROF_STEP = 3
PROF_STASH = 4
PROF_GROUPS = 5

DIM = 768


class NgramConfig(ctypes.Structure):
    _fields_ = [
        ("vocab", ctypes.c_int32),
        ("eos_id", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rows", ctypes.c_int64 * 2),
        ("seed", ctypes.c_uint64 * 2),
        ("max_tokens", ctypes.c_int64),
        ("accum_steps", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("window_rows", ctypes.c_int64),
        ("dy_dtype", ctypes.c_int32),
        ("options", ctypes.c_int32),
    ]

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == DTYPE_F32 else torch.bfloat16

    @property
    def out_torch_dtype(self):
        return torch.float32 if (self.dtype == DTYPE_F32 or self.options & OPT_OUT_F32) else torch.bfloat16

    @property
    def dy_torch_dtype(self):
        return torch.float32 if self.dy_dtype == DTYPE_F32 else torch.bfloat16

    @property
    def window_capacity(self) -> int:
        if self.window_rows > 0:
            return int(self.window_rows)
        return int(min(max(self.rows[0], self.rows[1]), self.accum_steps * self.max_tokens))


def config(vocab: int, eos_id: int, rows, dtype: str = "bf16", seeds=(1, 2),
           max_tokens: int = 1 << 16, accum_steps: int = 4, mode: str = "spread",
           window_rows: int = 0, dy_dtype: str = "f32", presort: bool = False,
           out_f32: bool = False, direct: bool = False, nest_always: bool = False) -> NgramConfig:
    """direct: one table indexed by the token id (value embeddings); rows
    is then (rows of that table, 1) and W_t / state_t may be None.
    nest_always: fused reductions of any size complete trigram rows of
    several positions in the bigram pass (NGRAM_OPT_NEST_ALWAYS)."""
    c = NgramConfig()
    c.vocab = vocab
    c.eos_id = eos_id
    c.dim = DIM
    c.dtype = DTYPE_F32 if dtype == "f32" else DTYPE_BF16
    c.rows[0], c.rows[1] = int(rows[0]), int(rows[1])
    c.seed[0], c.seed[1] = int(seeds[0]), int(seeds[1])
    c.max_tokens = int(max_tokens)
    c.accum_steps = int(accum_steps)
    c.mode = _MODES[mode]
    c.window_rows = int(window_rows)
    c.dy_dtype = DTYPE_F32 if dy_dtype == "f32" else DTYPE_BF16
    c.options = ((OPT_PRESORT if presort else 0) | (OPT_OUT_F32 if out_f32 else 0) | (OPT_DIRECT if direct else 0)
                 | (OPT_NEST_ALWAYS if nest_always else 0))
    return c


class NgramError(RuntimeError):
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
        vp, i32, i64, u64p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        cp = ctypes.POINTER(NgramConfig)
        sig = {
            "ngram_abi_version": ([], ctypes.c_int),
            "ngram_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "ngram_config_check": ([cp], ctypes.c_int),
            "ngram_workspace_bytes": ([cp, u64p], ctypes.c_int),
            "ngram_workspace_init": ([cp, vp, ctypes.c_uint64, vp], ctypes.c_int),
            "ngram_hash": ([cp, vp, i64, vp, vp, vp], ctypes.c_int),
            "ngram_embed_fwd": ([cp, vp, vp, vp, i64, vp, vp, vp], ctypes.c_int),
            "ngram_embed_bwd_accum": ([cp, vp, vp, vp, i64, vp], ctypes.c_int),
            "ngram_window_reduce": ([cp, vp, vp], ctypes.c_int),
            "ngram_window_keys": ([cp, vp, vp, i64, vp], ctypes.c_int),
            "ngram_window_sort": ([cp, vp, vp], ctypes.c_int),
            "ngram_sparse_step": ([cp, vp, vp, vp, vp, vp, i32, ctypes.c_float,
                                   ctypes.c_float, ctypes.c_float, vp], ctypes.c_int),
            "ngram_embed_bwd_step": ([cp, vp, vp, vp, i64, vp, vp, vp, vp, i32, ctypes.c_float,
                                      ctypes.c_float, ctypes.c_float, vp], ctypes.c_int),
            "ngram_sparse_step_dev": ([cp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "ngram_embed_bwd_step_dev": ([cp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "ngram_window_export": ([cp, vp, ctypes.c_int, vp, vp, i64, vp, vp], ctypes.c_int),
            "ngram_touched_rows": ([cp, vp, ctypes.c_int, vp, i64, vp, vp], ctypes.c_int),
            "ngram_window_step_noalloc": ([cp, vp, vp, i64, i32, vp, vp, vp, vp, i32, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_float, vp, vp], ctypes.c_int),
            "ngram_device_status": ([cp, vp, vp, ctypes.c_int, vp], ctypes.c_int),
            "ngram_profile_events": ([ctypes.c_int, vp, vp], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


lib()   # fail at import time if the HIP library is missing: there is no fallback


def status_string(status: int) -> str:
    return lib().ngram_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise NgramError(fn, status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor | None, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def config_check(cfg: NgramConfig) -> int:
    return lib().ngram_config_check(ctypes.byref(cfg))


def workspace_bytes(cfg: NgramConfig) -> int:
    n = ctypes.c_uint64()
    _check("ngram_workspace_bytes", lib().ngram_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return int(n.value)


class Workspace:
    """Device workspace of one table pair (a uint8 tensor, 256-byte aligned)."""

    def __init__(self, cfg: NgramConfig, device="cuda"):
        self.cfg = cfg
        self.nbytes = workspace_bytes(cfg)
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self._buf.data_ptr()) % 256
        self.tensor = self._buf[off:off + self.nbytes]
        self.reset()

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr()

    def reset(self):
        _check("ngram_workspace_init",
               lib().ngram_workspace_init(ctypes.byref(self.cfg), self.ptr, self.nbytes, _stream()))


def _ws(ws: Workspace | None):
    return None if ws is None else ws.ptr


def hash(cfg: NgramConfig, tokens: torch.Tensor, ws: Workspace | None = None) -> torch.Tensor:
    """Packed indices int32 [2, T] (bit pattern row | neg << 31)."""
    T = tokens.numel()
    idx = torch.empty((2, T), dtype=torch.int32, device=tokens.device)
    _check("ngram_hash", lib().ngram_hash(ctypes.byref(cfg), _dev(tokens, "tokens", torch.int32), T,
                                          idx.data_ptr(), _ws(ws), _stream()))
    return idx


def _check_tables(cfg: NgramConfig, W_b, W_t):
    for c, W in ((0, W_b), (1, W_t)):
        if W is None and c == 1 and cfg.options & OPT_DIRECT:
            continue
        if tuple(W.shape) != (cfg.rows[c], DIM):
            raise ValueError(f"table {c} must be [{cfg.rows[c]}, {DIM}], got {tuple(W.shape)}")


def new_state(rows: int, device="cuda") -> torch.Tensor:
    """Optimizer state of a table: float32 [rows, 2], one 8-byte record
    (v, t_last) per row (ngram_row_state); column 1 holds int32 bits."""
    return torch.zeros((rows, 2), dtype=torch.float32, device=device)


def state_v(st: torch.Tensor) -> torch.Tensor:
    """The second moments v (a strided float32 view)."""
    return st[:, 0]


def state_t_last(st: torch.Tensor) -> torch.Tensor:
    """The last-update steps t_last (a strided int32 view)."""
    return st.view(torch.int32)[:, 1]


def _check_state(cfg: NgramConfig, st_b, st_t):
    for c, x in ((0, st_b), (1, st_t)):
        if x is None and c == 1 and cfg.options & OPT_DIRECT:
            continue
        if tuple(x.shape) != (cfg.rows[c], 2) or x.dtype != torch.float32:
            raise ValueError(f"optimizer state of channel {c} must be float32 [{cfg.rows[c]}, 2]")


def embed_fwd(cfg: NgramConfig, W_b: torch.Tensor, W_t: torch.Tensor, tokens: torch.Tensor,
              out: torch.Tensor | None = None, ws: Workspace | None = None) -> torch.Tensor:
    T = tokens.numel()
    _check_tables(cfg, W_b, W_t)
    if out is None:
        out = torch.empty((T, DIM), dtype=cfg.out_torch_dtype, device=tokens.device)
    if tuple(out.shape) != (T, DIM):
        raise ValueError(f"out must be [{T}, {DIM}]")
    _check("ngram_embed_fwd", lib().ngram_embed_fwd(
        ctypes.byref(cfg), _dev(W_b, "W_b", cfg.torch_dtype), _dev(W_t, "W_t", cfg.torch_dtype),
        _dev(tokens, "tokens", torch.int32), T, _dev(out, "out", cfg.out_torch_dtype), _ws(ws), _stream()))
    return out


def embed_bwd_accum(cfg: NgramConfig, ws: Workspace, tokens: torch.Tensor, dY: torch.Tensor):
    """In burst_ref mode dY must stay alive and unchanged until the window's step."""
    T = tokens.numel()
    if dY.shape != (T, DIM):
        raise ValueError(f"dY must be [{T}, {DIM}], got {tuple(dY.shape)}")
    _check("ngram_embed_bwd_accum", lib().ngram_embed_bwd_accum(
        ctypes.byref(cfg), ws.ptr, _dev(tokens, "tokens", torch.int32), _dev(dY, "dY", cfg.dy_torch_dtype),
        T, _stream()))


def window_keys(cfg: NgramConfig, ws: Workspace, tokens: torch.Tensor):
    """Burst modes: keep the sort keys of the window's next micro-step now."""
    _check("ngram_window_keys", lib().ngram_window_keys(
        ctypes.byref(cfg), ws.ptr, _dev(tokens, "tokens", torch.int32), tokens.numel(), _stream()))


def window_sort(cfg: NgramConfig, ws: Workspace):
    """Burst modes: sort the window's kept keys (on the current stream)."""
    _check("ngram_window_sort", lib().ngram_window_sort(ctypes.byref(cfg), ws.ptr, _stream()))


def window_reduce(cfg: NgramConfig, ws: Workspace):
    _check("ngram_window_reduce", lib().ngram_window_reduce(ctypes.byref(cfg), ws.ptr, _stream()))


def sparse_step(cfg: NgramConfig, ws: Workspace, W_b, W_t, state_b, state_t, t: int,
                lr: float, beta2: float, eps: float):
    """state_b / state_t: float32 [rows, 2] from new_state()."""
    dt = cfg.torch_dtype
    _check_tables(cfg, W_b, W_t)
    _check_state(cfg, state_b, state_t)
    _check("ngram_sparse_step", lib().ngram_sparse_step(
        ctypes.byref(cfg), ws.ptr, _dev(W_b, "W_b", dt), _dev(W_t, "W_t", dt),
        _dev(state_b, "state_b", torch.float32), _dev(state_t, "state_t", torch.float32),
        int(t), float(lr), float(beta2), float(eps), _stream()))


def embed_bwd_step(cfg: NgramConfig, ws: Workspace, tokens: torch.Tensor, dY: torch.Tensor,
                   W_b, W_t, state_b, state_t, t: int, lr: float, beta2: float, eps: float):
    """The window's last micro-step fused with its sparse step."""
    T = tokens.numel()
    if dY.shape != (T, DIM):
        raise ValueError(f"dY must be [{T}, {DIM}], got {tuple(dY.shape)}")
    dt = cfg.torch_dtype
    _check_tables(cfg, W_b, W_t)
    _check_state(cfg, state_b, state_t)
    _check("ngram_embed_bwd_step", lib().ngram_embed_bwd_step(
        ctypes.byref(cfg), ws.ptr, _dev(tokens, "tokens", torch.int32), _dev(dY, "dY", cfg.dy_torch_dtype), T,
        _dev(W_b, "W_b", dt), _dev(W_t, "W_t", dt), _dev(state_b, "state_b", torch.float32),
        _dev(state_t, "state_t", torch.float32), int(t), float(lr), float(beta2), float(eps), _stream()))


def step_params(t: int, lr: float, beta2: float, eps: float, out: torch.Tensor | None = None,
                device="cuda") -> torch.Tensor:
    """Step parameters for the _dev entry points: a 16-byte device tensor
    (int32 t, then float32 lr, beta2, eps), written in place if `out` is
    given (an ordinary copy on the current stream)."""
    host = torch.tensor([float(lr), float(beta2), float(eps)], dtype=torch.float32)
    rec = torch.empty(4, dtype=torch.int32)
    rec[0] = int(t)
    rec[1:] = host.view(torch.int32)
    if out is None:
        out = torch.empty(4, dtype=torch.int32, device=device)
    out.copy_(rec)
    return out


def _check_params(p: torch.Tensor):
    if p.numel() != 4 or p.element_size() != 4 or p.data_ptr() % 16:
        raise ValueError("step parameters must be a 16-byte aligned 4 x 32-bit device tensor")


def sparse_step_dev(cfg: NgramConfig, ws: Workspace, W_b, W_t, state_b, state_t, params: torch.Tensor):
    """sparse_step with (t, lr, beta2, eps) read from `params` (step_params)
    when the kernels run."""
    dt = cfg.torch_dtype
    _check_tables(cfg, W_b, W_t)
    _check_state(cfg, state_b, state_t)
    _check_params(params)
    _check("ngram_sparse_step_dev", lib().ngram_sparse_step_dev(
        ctypes.byref(cfg), ws.ptr, _dev(W_b, "W_b", dt), _dev(W_t, "W_t", dt),
        _dev(state_b, "state_b", torch.float32), _dev(state_t, "state_t", torch.float32),
        _dev(params, "params"), _stream()))


def embed_bwd_step_dev(cfg: NgramConfig, ws: Workspace, tokens: torch.Tensor, dY: torch.Tensor,
                       W_b, W_t, state_b, state_t, params: torch.Tensor):
    """embed_bwd_step with the step parameters in device memory."""
    T = tokens.numel()
    if dY.shape != (T, DIM):
        raise ValueError(f"dY must be [{T}, {DIM}], got {tuple(dY.shape)}")
    dt = cfg.torch_dtype
    _check_tables(cfg, W_b, W_t)
    _check_state(cfg, state_b, state_t)
    _check_params(params)
    _check("ngram_embed_bwd_step_dev", lib().ngram_embed_bwd_step_dev(
        ctypes.byref(cfg), ws.ptr, _dev(tokens, "tokens", torch.int32), _dev(dY, "dY", cfg.dy_torch_dtype), T,
        _dev(W_b, "W_b", dt), _dev(W_t, "W_t", dt), _dev(state_b, "state_b", torch.float32),
        _dev(state_t, "state_t", torch.float32), _dev(params, "params"), _stream()))


def touched_rows(cfg: NgramConfig, ws: Workspace, channel: int, rows: torch.Tensor | None = None,
                 count: torch.Tensor | None = None):
    """The window's distinct rows of one channel, ascending, as (rows int32
    [capacity], count int64 [1]) device tensors: no synchronisation (the first
    count.item() entries are the rows).  capacity defaults to the window's
    row capacity."""
    dev = ws.tensor.device
    if rows is None:
        rows = torch.empty(cfg.window_capacity, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=dev)
    _check("ngram_touched_rows", lib().ngram_touched_rows(
        ctypes.byref(cfg), ws.ptr, int(channel), _dev(rows, "rows", torch.int32), rows.numel(),
        _dev(count, "count", torch.int64), _stream()))
    return rows, count


def window_step_noalloc(cfg: NgramConfig, tokens: torch.Tensor, dY: torch.Tensor, T: int, n_micro: int,
                        W_b, W_t, state_b, state_t, t: int, lr: float, beta2: float, eps: float,
                        flags: torch.Tensor | None = None):
    """One whole window (tokens int32 [n_micro * T], dY [n_micro * T, 768])
    reduced and stepped with no workspace (the library's fixed device array
    serves as one).  flags: an optional int32 device word the call ORs its
    device flags into."""
    if tokens.numel() != n_micro * T or tuple(dY.shape) != (n_micro * T, DIM):
        raise ValueError("tokens must hold n_micro * T ids and dY [n_micro * T, 768] rows")
    dt = cfg.torch_dtype
    _check_tables(cfg, W_b, W_t)
    _check_state(cfg, state_b, state_t)
    if flags is not None and (flags.numel() != 1 or flags.element_size() != 4):
        raise ValueError("flags must be one 32-bit device word")
    _check("ngram_window_step_noalloc", lib().ngram_window_step_noalloc(
        ctypes.byref(cfg), _dev(tokens, "tokens", torch.int32), _dev(dY, "dY", cfg.dy_torch_dtype), int(T),
        int(n_micro), _dev(W_b, "W_b", dt), _dev(W_t, "W_t", dt), _dev(state_b, "state_b", torch.float32),
        _dev(state_t, "state_t", torch.float32), int(t), float(lr), float(beta2), float(eps),
        _dev(flags, "flags"), _stream()))


def window_export(cfg: NgramConfig, ws: Workspace, channel: int, with_grad: bool = True):
    """(rows int64 [n], G float32 [n, 768] or None) of the current window.
    Synchronises the stream to read n."""
    cap = cfg.window_capacity
    dev = ws.tensor.device
    rows = torch.empty(cap, dtype=torch.int32, device=dev)
    G = torch.empty((cap, DIM), dtype=torch.float32, device=dev) if with_grad else None
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    _check("ngram_window_export", lib().ngram_window_export(
        ctypes.byref(cfg), ws.ptr, int(channel), rows.data_ptr(),
        None if G is None else G.data_ptr(), cap, cnt.data_ptr(), _stream()))
    n = int(cnt.item())
    n = min(n, cap)
    r = rows[:n].to(torch.int64) & 0xFFFFFFFF
    return r, (G[:n] if G is not None else None)


def device_status(cfg: NgramConfig, ws: Workspace, clear: bool = False) -> int:
    f = ctypes.c_uint32()
    _check("ngram_device_status", lib().ngram_device_status(
        ctypes.byref(cfg), ws.ptr, ctypes.byref(f), int(bool(clear)), _stream()))
    return int(f.value)


def profile_events(group: int, start, stop):
    """Record two HIP events (raw hipEvent_t handles, or None) around the
    kernels of `group` in this thread's later calls."""
    _check("ngram_profile_events", lib().ngram_profile_events(int(group), start, stop))
