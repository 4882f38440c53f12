"""Python binding of libdeltalog, the DeltaLog recurrent-state decode step for
linear attention (GDN, KDA, RWKV6) on MI355X.

Argument marshalling only: every call goes to the C ABI declared in
``include/deltalog.h`` (same function names), whose HIP kernels do all of the
arithmetic.  torch tensors are accepted wherever the C ABI takes a device
pointer; torch supplies device memory and the current stream.  There is no
fallback: if ``libdeltalog.so`` has not been built, importing this package
raises.

    from recurrent_state_update_amd import DeltaLogState
    st = DeltaLogState("gdn", B, H, 128, 128, M=8, dtype=torch.bfloat16, base=S0)
    o = st.step(q, k, v, beta, log_decay)      # o_t = S_t q_t, [B,H,d_v] fp32
    st.merge()                                  # st.base now holds S_t
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdeltalog.so")

OPS = {"gdn": 0, "kda": 1, "rwkv6": 2}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "DL_OK", 1: "DL_E_INVALID", 2: "DL_E_SHAPE", 3: "DL_E_ALIGN", 4: "DL_E_HIP",
          5: "DL_E_STATE", 6: "DL_E_SCRATCH"}
EXPORTS = ("dl_workspace_bytes", "dl_state_create", "dl_decode_step", "dl_replay_prep",
           "dl_append_decode", "dl_merge", "dl_state_reset", "dl_log_len", "dl_set_log_len",
           "dl_state_destroy", "dl_eager_step", "dl_status_string", "dl_suggest_merge_interval",
           "dl_state_enable_slots", "dl_slot_admit", "dl_slot_merge", "dl_slot_log_len",
           "dl_slot_release", "dl_decode_step_staged_noalloc", "dl_choose_merge_interval")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python recurrent_state_update_amd/_build.py` "
                      "(or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)
_i, _p, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t


_SIG = {
    "dl_workspace_bytes": ([_i] * 7, _sz),
    "dl_state_create": ([_i] * 7 + [_p, _p, _p, ctypes.POINTER(_p)], _i),
    "dl_decode_step": ([_p] * 8, _i),
    "dl_replay_prep": ([_p] * 5, _i),
    "dl_append_decode": ([_p] * 7, _i),
    "dl_merge": ([_p, _p], _i),
    "dl_state_reset": ([_p], _i),
    "dl_log_len": ([_p], _i),
    "dl_set_log_len": ([_p, _i], _i),
    "dl_state_destroy": ([_p], _i),
    "dl_eager_step": ([_i] * 6 + [_p] * 9, _i),
    "dl_status_string": ([_i], ctypes.c_char_p),
    "dl_suggest_merge_interval": ([_i] * 6, _i),
    "dl_state_enable_slots": ([_p, _p], _i),
    "dl_slot_admit": ([_p, _i, _p], _i),
    "dl_slot_merge": ([_p, _i, _p], _i),
    "dl_slot_log_len": ([_p, _i], _i),
    "dl_slot_release": ([_p, _i, _p], _i),
    "dl_decode_step_staged_noalloc": ([_p] * 8, _i),
    "dl_choose_merge_interval": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), _i], _i),
}
for _name, (_args, _res) in _SIG.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class DeltaLogError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({_lib.dl_status_string(status).decode()})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DeltaLogError(status, where)


def _ptr(x):
    """Device pointer of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------- raw C ABI --
# Same names and argument order as include/deltalog.h; tensors or ints for
# pointers; return the status code (int) like the C functions.

def dl_workspace_bytes(B, H, d_k, d_v, M, op, in_dtype) -> int:
    return int(_lib.dl_workspace_bytes(B, H, d_k, d_v, M, op, in_dtype))


def dl_state_create(B, H, d_k, d_v, M, op, in_dtype, base, workspace, u):
    """Returns (status, handle)."""
    h = _p()
    st = _lib.dl_state_create(B, H, d_k, d_v, M, op, in_dtype, _ptr(base), _ptr(workspace),
                              _ptr(u), ctypes.byref(h))
    return st, h.value


def dl_decode_step(s, q, k, v, beta, log_decay, o, stream=None):
    return _lib.dl_decode_step(s, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_decay),
                               _ptr(o), _stream(stream))


def dl_decode_step_staged_noalloc(s, q, k, v, beta, log_decay, o, stream=None):
    return _lib.dl_decode_step_staged_noalloc(s, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                              _ptr(log_decay), _ptr(o), _stream(stream))


def dl_replay_prep(s, q, k, log_decay, stream=None):
    return _lib.dl_replay_prep(s, _ptr(q), _ptr(k), _ptr(log_decay), _stream(stream))


def dl_append_decode(s, q, k, v, beta, o, stream=None):
    return _lib.dl_append_decode(s, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(o),
                                 _stream(stream))


def dl_merge(s, stream=None):
    return _lib.dl_merge(s, _stream(stream))


def dl_state_reset(s):
    return _lib.dl_state_reset(s)


def dl_log_len(s) -> int:
    return _lib.dl_log_len(s)


def dl_set_log_len(s, n):
    return _lib.dl_set_log_len(s, n)


def dl_state_destroy(s):
    return _lib.dl_state_destroy(s)


def dl_eager_step(op, B, H, d_k, d_v, in_dtype, S, q, k, v, beta, log_decay, u, o, stream=None):
    return _lib.dl_eager_step(op, B, H, d_k, d_v, in_dtype, _ptr(S), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(beta), _ptr(log_decay), _ptr(u), _ptr(o), _stream(stream))


def dl_suggest_merge_interval(B, H, d_k, d_v, op, in_dtype) -> int:
    return int(_lib.dl_suggest_merge_interval(B, H, d_k, d_v, op, in_dtype))


def dl_choose_merge_interval(append_us, merge_us, max_M=None) -> int:
    """append_us[n], merge_us[n]: measured launch times (us) at log length n;
    max_M defaults to their length."""
    max_M = len(merge_us) if max_M is None else max_M
    A = (ctypes.c_double * max(len(append_us), 1))(*append_us)
    Mg = (ctypes.c_double * max(len(merge_us), 1))(*merge_us)
    if len(append_us) < max_M - 1 or len(merge_us) < max_M:
        raise ValueError("want max_M - 1 append times and max_M merge times")
    return int(_lib.dl_choose_merge_interval(A, Mg, max_M))


def dl_state_enable_slots(s, stream=None):
    return _lib.dl_state_enable_slots(s, _stream(stream))


def dl_slot_admit(s, slot, stream=None):
    return _lib.dl_slot_admit(s, slot, _stream(stream))


def dl_slot_merge(s, slot, stream=None):
    return _lib.dl_slot_merge(s, slot, _stream(stream))


def dl_slot_log_len(s, slot) -> int:
    return _lib.dl_slot_log_len(s, slot)


def dl_slot_release(s, slot, stream=None):
    return _lib.dl_slot_release(s, slot, _stream(stream))


def dl_status_string(st) -> str:
    return _lib.dl_status_string(st).decode()


# ------------------------------------------------------------ torch helpers --

def _op_id(op) -> int:
    if op not in OPS:
        raise ValueError(f"unknown operator {op!r}: want one of {sorted(OPS)}")
    return OPS[op]


def _dtype_id(dtype) -> int:
    if dtype not in DTYPES:
        raise ValueError(f"unsupported input dtype {dtype}: want torch.bfloat16 or torch.float32")
    return DTYPES[dtype]


def _want(t, name, dtype, shape, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: want contiguous {dtype} {tuple(shape)} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the state on {device}")


class DeltaLogState:
    """One DeltaLog state (base + log) for B slots x H heads, over device
    memory allocated with torch.  ``base`` is the S-bar tensor [B,H,d_k,d_v]
    fp32; it holds the logical state whenever ``log_len == 0``."""

    def __init__(self, op: str, B: int, H: int, d_k: int, d_v: int, M: int,
                 dtype=torch.bfloat16, base: torch.Tensor | None = None,
                 u: torch.Tensor | None = None, device="cuda"):
        self.op, self.B, self.H, self.d_k, self.d_v, self.M = op, B, H, d_k, d_v, M
        self.dtype = dtype
        opi, dti = _op_id(op), _dtype_id(dtype)
        nbytes = dl_workspace_bytes(B, H, d_k, d_v, M, opi, dti)
        if nbytes == 0:
            raise ValueError(f"unsupported DeltaLog shape {op} B={B} H={H} d_k={d_k} d_v={d_v} M={M}")
        if base is None:
            base = torch.zeros(B, H, d_k, d_v, dtype=torch.float32, device=device)
        _want(base, "base", torch.float32, (B, H, d_k, d_v))
        self.base = base
        # 256-byte aligned workspace (torch's caching allocator aligns to 512)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=base.device)
        if op == "rwkv6":
            _want(u, "u", torch.float32, (H, d_k), base.device)
        self.u = u
        st, h = dl_state_create(B, H, d_k, d_v, M, opi, dti, base, self.workspace, u)
        _check(st, "dl_state_create")
        self._h = h
        self._per_slot = False

    # validation of per-step tensors
    def _inputs(self, q, k, v, beta, log_decay, o):
        B, H, dk, dv = self.B, self.H, self.d_k, self.d_v
        dev = self.base.device
        _want(q, "q", self.dtype, (B, H, dk), dev)
        _want(k, "k", self.dtype, (B, H, dk), dev)
        _want(v, "v", self.dtype, (B, H, dv), dev)
        if self.op != "rwkv6":
            _want(beta, "beta", torch.float32, (B, H), dev)
        if log_decay is not None:
            _want(log_decay, "log_decay", torch.float32, (B, H) if self.op == "gdn" else (B, H, dk), dev)
        if o is None:
            # on a per-slot handle the workgroups of released slots store
            # nothing, so their rows of o keep what the buffer held: zeros
            o = (torch.zeros if self._per_slot else torch.empty)(B, H, dv, dtype=torch.float32, device=dev)
        _want(o, "o", torch.float32, (B, H, dv), dev)
        return o

    def _log_decay(self, log_decay):
        _want(log_decay, "log_decay", torch.float32,
              (self.B, self.H) if self.op == "gdn" else (self.B, self.H, self.d_k), self.base.device)

    def step(self, q, k, v, beta, log_decay, o=None, stream=None):
        """One decode step; returns o_t [B,H,d_v] fp32.  On a handle with
        per-slot logs, the rows of released slots are left as ``o`` held them
        (zeros when ``o`` is not given)."""
        o = self._inputs(q, k, v, beta, log_decay, o)
        self._log_decay(log_decay)
        _check(dl_decode_step(self._h, q, k, v, beta, log_decay, o, stream), "dl_decode_step")
        return o

    def replay_prep(self, q, k, log_decay, stream=None):
        """Stage 1 of the two-stage step (append_decode is stage 2)."""
        dev = self.base.device
        _want(q, "q", self.dtype, (self.B, self.H, self.d_k), dev)
        _want(k, "k", self.dtype, (self.B, self.H, self.d_k), dev)
        self._log_decay(log_decay)
        _check(dl_replay_prep(self._h, q, k, log_decay, stream), "dl_replay_prep")

    def append_decode(self, q, k, v, beta, o=None, stream=None):
        o = self._inputs(q, k, v, beta, None, o)
        _check(dl_append_decode(self._h, q, k, v, beta, o, stream), "dl_append_decode")
        return o

    def merge(self, stream=None):
        _check(dl_merge(self._h, stream), "dl_merge")

    def reset(self):
        _check(dl_state_reset(self._h), "dl_state_reset")

    @property
    def log_len(self) -> int:
        return dl_log_len(self._h)

    # per-slot logs (continuous batching)
    def enable_slots(self, stream=None):
        _check(dl_state_enable_slots(self._h, stream), "dl_state_enable_slots")
        self._per_slot = True

    def admit(self, slot: int, stream=None):
        """Start a new request in ``slot``: write its initial state into
        ``base[slot]`` first (on the same stream), then admit; the slot's
        pending log is dropped."""
        _check(dl_slot_admit(self._h, slot, stream), "dl_slot_admit")

    def merge_slot(self, slot: int, stream=None):
        _check(dl_slot_merge(self._h, slot, stream), "dl_slot_merge")

    def release(self, slot: int, stream=None):
        """The request in ``slot`` finished: later steps and merges skip the
        slot (no traffic) until it is admitted again.  Merge it first to keep
        its state."""
        _check(dl_slot_release(self._h, slot, stream), "dl_slot_release")

    def slot_log_len(self, slot: int) -> int:
        return dl_slot_log_len(self._h, slot)

    def set_log_len(self, n: int):
        _check(dl_set_log_len(self._h, n), "dl_set_log_len")

    def close(self):
        if getattr(self, "_h", None):
            dl_state_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def eager_step(op: str, S, q, k, v, beta, log_decay, u=None, o=None, stream=None):
    """The eager baseline: one step that reads and rewrites S [B,H,d_k,d_v]."""
    B, H, dk, dv = S.shape
    dtype = q.dtype
    opi, dti = _op_id(op), _dtype_id(dtype)
    dev = S.device
    _want(S, "S", torch.float32, (B, H, dk, dv))
    _want(q, "q", dtype, (B, H, dk), dev)
    _want(k, "k", dtype, (B, H, dk), dev)
    _want(v, "v", dtype, (B, H, dv), dev)
    if op != "rwkv6":
        _want(beta, "beta", torch.float32, (B, H), dev)
    else:
        _want(u, "u", torch.float32, (H, dk), dev)
    _want(log_decay, "log_decay", torch.float32, (B, H) if op == "gdn" else (B, H, dk), dev)
    if o is None:
        o = torch.empty(B, H, dv, dtype=torch.float32, device=dev)
    _want(o, "o", torch.float32, (B, H, dv), dev)
    _check(dl_eager_step(opi, B, H, dk, dv, dti, S, q, k, v, beta, log_decay, u, o,
                         stream), "dl_eager_step")
    return o
