"""Thin Python binding of libsparse_ffn.so (the C ABI in include/sparse_ffn.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
PyTorch supplies device memory (tensors) and the stream (the current HIP stream).  If the
shared library is missing this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SFFN_LIB names another build of the same sources (the host-sanitizer test uses it)
LIB_PATH = os.environ.get("SFFN_LIB") or os.path.join(_HERE, "libsparse_ffn.so")

SFFN_OK = 0
SFFN_ERR_INVALID_ARGUMENT = 1
SFFN_ERR_UNSUPPORTED = 2
SFFN_ERR_BACKUP_OVERFLOW = 3
SFFN_ERR_DEVICE = 4
SFFN_F32 = 0
SFFN_BF16 = 1

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class SffnError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {status_string(status)}: {message}")
        self.status = status


class ConfigC(ctypes.Structure):
    _fields_ = [("d_model", _I32), ("d_ff", _I32), ("tile", _I32), ("ell_width", _I32),
                ("max_tokens", _I32), ("backup_capacity", _I32), ("dtype", ctypes.c_int)]


class BuffersC(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("counts", "vals", "cols", "bk_tile", "bk_tok", "bk_vals",
                                  "bk_tile_ptr", "bk_n", "status", "workspace")]


BUFFER_FIELDS = [n for n, _ in BuffersC._fields_]


class SizesC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in BUFFER_FIELDS]


class StatsC(ctypes.Structure):
    _fields_ = [("nnz", ctypes.c_int64), ("slots_used", ctypes.c_int64),
                ("overflow_tile_rows", ctypes.c_int64), ("backup_nonzeros", ctypes.c_int64),
                ("backup_needed", ctypes.c_int64), ("max_count", _I32),
                ("backup_overflowed", _I32), ("density", ctypes.c_double),
                ("ell_fill", ctypes.c_double), ("bytes_main", ctypes.c_int64),
                ("bytes_backup", ctypes.c_int64), ("bytes_dense_equiv", ctypes.c_int64)]


# Down-projection policies (mirror the header's SFFN_DOWN_* values).
DOWN_AUTO, DOWN_GATHER, DOWN_MFMA, DOWN_TILES, DOWN_UNION, DOWN_SPARSE = 0, 1, 2, 3, 4, 5
DOWN_GATHER_DENSITY_DEFAULT = 0.0005
DOWN_MFMA_DENSITY_DEFAULT = 0.005
DOWN_TILES_MIN_T = 4096
DOWN_MFMA_MIN_T = 64
# Largest d_ff / tile a configuration may have (the header's SFFN_MAX_TILES).
MAX_TILES = 4096

# Exported entry points and their prototypes (restype is always the status enum unless set).
_PROTOS = {
    "sffn_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sffn_last_error": ([], ctypes.c_char_p),
    "twell_buffer_sizes": ([ctypes.POINTER(ConfigC), _I32, ctypes.POINTER(SizesC)], ctypes.c_int),
    "twell_buffer_bytes": ([ctypes.POINTER(ConfigC), _I32, ctypes.POINTER(ctypes.c_size_t)],
                           ctypes.c_int),
    "sparse_ffn_create": ([ctypes.POINTER(ConfigC), _P, _P, _P, ctypes.POINTER(_P)], ctypes.c_int),
    "sparse_ffn_destroy": ([_P], ctypes.c_int),
    "twell_pack": ([ctypes.POINTER(ConfigC), _P, _I32, ctypes.POINTER(BuffersC), _P], ctypes.c_int),
    "sparse_ffn_forward": ([_P, _P, _I32, _P, ctypes.POINTER(BuffersC), _P], ctypes.c_int),
    "sparse_ffn_down": ([_P, ctypes.POINTER(BuffersC), _I32, _P, _P], ctypes.c_int),
    "sparse_ffn_set_down_policy": ([_P, _I32, ctypes.c_float, ctypes.c_float], ctypes.c_int),
    "sparse_ffn_backward": ([_P, _P, _P, _I32, ctypes.POINTER(BuffersC), _P, _P, _P, _P, _P, _P,
                             _P], ctypes.c_int),
    "twell_stats": ([ctypes.POINTER(ConfigC), ctypes.POINTER(BuffersC), _I32,
                     ctypes.POINTER(StatsC), _P], ctypes.c_int),
    "sparse_ffn_check": ([ctypes.POINTER(BuffersC), _P], ctypes.c_int),
    "sparse_ffn_forward_noalloc": ([_P, _P, _I32, _P, ctypes.POINTER(BuffersC), _P], ctypes.c_int),
    "sparse_ffn_forward_dump": ([_P, _P, _I32, _P, ctypes.POINTER(BuffersC), _P, _P], ctypes.c_int),
    "sffn_profile_enable": ([_I32], ctypes.c_int),
    "sffn_profile_only": ([ctypes.c_char_p], ctypes.c_int),
    "sffn_profile_reset": ([], ctypes.c_int),
    "sffn_profile_read": ([ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                           ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
    "sffn_probe_gather_fma": ([_P, _I32, _I32, _P, _P, _I32, _I32, _P, _P], ctypes.c_int),
    "twell_count_histogram": ([ctypes.POINTER(ConfigC), ctypes.POINTER(BuffersC), _I32,
                               ctypes.POINTER(ctypes.c_int64), _P], ctypes.c_int),
    "twell_choose_ell_width": ([ctypes.POINTER(ConfigC), ctypes.POINTER(ctypes.c_int64),
                                ctypes.POINTER(ctypes.c_int32), _I32,
                                ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)],
                               ctypes.c_int),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m activation_sparse_transformer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _PROTOS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def exported_names():
    return list(_PROTOS)


def status_string(s: int) -> str:
    return lib().sffn_status_string(int(s)).decode()


def last_error() -> str:
    return lib().sffn_last_error().decode()


def _check(status: int, where: str):
    if status != SFFN_OK:
        raise SffnError(status, where, last_error())


@dataclass(frozen=True)
class Config:
    d_model: int
    d_ff: int
    tile: int
    ell_width: int
    max_tokens: int
    backup_capacity: int
    dtype: str = "bf16"   # "bf16" or "f32"

    @property
    def n_tiles(self) -> int:
        return self.d_ff // self.tile

    def c(self) -> ConfigC:
        return ConfigC(self.d_model, self.d_ff, self.tile, self.ell_width, self.max_tokens,
                       self.backup_capacity, SFFN_BF16 if self.dtype == "bf16" else SFFN_F32)

    @property
    def esz(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def buffer_sizes(cfg: Config, T: int) -> dict:
    out = SizesC()
    c = cfg.c()
    _check(lib().twell_buffer_sizes(ctypes.byref(c), int(T), ctypes.byref(out)), "twell_buffer_sizes")
    return {n: int(getattr(out, n)) for n in BUFFER_FIELDS}


def buffer_bytes(cfg: Config, T: int) -> list:
    """twell_buffer_bytes: the same sizes as buffer_sizes, as a list in field order."""
    out = (ctypes.c_size_t * len(BUFFER_FIELDS))()
    c = cfg.c()
    _check(lib().twell_buffer_bytes(ctypes.byref(c), int(T), out), "twell_buffer_bytes")
    return [int(v) for v in out]


def _stream_ptr(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(int(s.cuda_stream))


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(int(t.data_ptr()))


class TwellBuffers:
    """Device buffers (torch uint8 tensors) of one packed activation.  They are sized for
    `capacity` tokens and serve any call with fewer; `T` is the token count of the
    activation they hold (set by the call that packs into them)."""

    def __init__(self, cfg: Config, T: int, device="cuda"):
        import torch
        self.cfg = cfg
        self.T = int(T)
        self.capacity = self.T
        self.sizes = buffer_sizes(cfg, self.T)
        self.t = {n: torch.empty(max(sz, 1), dtype=torch.uint8, device=device)
                  for n, sz in self.sizes.items()}
        self._c = BuffersC(*[int(self.t[n].data_ptr()) for n in BUFFER_FIELDS])

    def c(self) -> BuffersC:
        return self._c

    def _hold(self, cfg: Config, T: int):
        """Checks that these buffers can take a call of T tokens of layer cfg; records T."""
        if self.cfg != cfg:
            raise ValueError("TwELL buffers were sized for another layer configuration")
        if not 1 <= T <= self.capacity:
            raise ValueError(f"TwELL buffers hold at most {self.capacity} tokens, not {T}")
        self.T = int(T)

    # ---- host copies (for tests and statistics; synchronous)
    def _np(self, name, dtype):
        return self.t[name][: self.sizes[name]].cpu().numpy().view(dtype)

    def to_host(self) -> dict:
        cfg, T = self.cfg, self.T
        nt, W, K = cfg.n_tiles, cfg.ell_width, cfg.tile
        counts = self._np("counts", np.uint16)[: nt * T].reshape(nt, T)
        vdt = np.uint16 if cfg.dtype == "bf16" else np.float32
        vals = self._np("vals", vdt)[: nt * T * W].reshape(nt, T, W)
        cols = self._np("cols", np.uint8)[: nt * T * W].reshape(nt, T, W)
        bk_n = int(self._np("bk_n", np.int32)[0])
        status = int(self._np("status", np.int32)[0])
        r = min(bk_n, cfg.backup_capacity)
        cap = max(cfg.backup_capacity, 1)
        bk_tile = self._np("bk_tile", np.int32)[:r].copy()
        bk_tok = self._np("bk_tok", np.int32)[:r].copy()
        bk_vals = self._np("bk_vals", vdt).reshape(cap, K)[:r].copy()
        ptr = self._np("bk_tile_ptr", np.int32)[: nt + 1].copy()
        return {"counts": counts, "vals": vals, "cols": cols, "bk_tile": bk_tile,
                "bk_tok": bk_tok, "bk_vals": bk_vals, "bk_n": bk_n, "status": status,
                "bk_tile_ptr": ptr}


def twell_pack(cfg: Config, h, out: Optional[TwellBuffers] = None, stream=None) -> TwellBuffers:
    """Pack a dense fp32 device tensor h [T, d_ff] into TwELL (runs the pack kernels)."""
    import torch
    assert h.dtype == torch.float32 and h.is_contiguous() and h.is_cuda
    T = h.shape[0]
    buf = out if out is not None else TwellBuffers(cfg, T, device=h.device)
    buf._hold(cfg, T)
    c = cfg.c()
    _check(lib().twell_pack(ctypes.byref(c), _ptr(h), int(T), ctypes.byref(buf.c()),
                            _stream_ptr(stream)), "twell_pack")
    return buf


def twell_stats(cfg: Config, buf: TwellBuffers, stream=None, raise_on_overflow=True) -> dict:
    out = StatsC()
    c = cfg.c()
    st = lib().twell_stats(ctypes.byref(c), ctypes.byref(buf.c()), int(buf.T), ctypes.byref(out),
                           _stream_ptr(stream))
    if st != SFFN_OK and (raise_on_overflow or st != SFFN_ERR_BACKUP_OVERFLOW):
        _check(st, "twell_stats")
    d = {n: getattr(out, n) for n, _ in StatsC._fields_}
    d["status"] = st
    return d


def count_histogram(cfg: Config, buf: TwellBuffers, stream=None) -> np.ndarray:
    """hist[c] = tile-rows of `buf` holding c nonzeros, c = 0 .. tile (computed on the device)."""
    out = (ctypes.c_int64 * (cfg.tile + 1))()
    c = cfg.c()
    _check(lib().twell_count_histogram(ctypes.byref(c), ctypes.byref(buf.c()), int(buf.T), out,
                                       _stream_ptr(stream)), "twell_count_histogram")
    return np.array(out[:], dtype=np.int64)


def choose_ell_width(cfg: Config, hist, candidates=None):
    """(W, bytes): the ELL width with the fewest stored bytes for a count histogram (host)."""
    h = np.ascontiguousarray(hist, dtype=np.int64)
    if h.size != cfg.tile + 1:
        raise ValueError(f"histogram needs tile + 1 = {cfg.tile + 1} bins")
    c = cfg.c()
    w = ctypes.c_int32()
    nb = ctypes.c_int64()
    if candidates is None:
        cand, n = None, 0
    else:
        arr = np.ascontiguousarray(candidates, dtype=np.int32)
        cand, n = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(arr.size)
    _check(lib().twell_choose_ell_width(ctypes.byref(c), h.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                        cand, n, ctypes.byref(w), ctypes.byref(nb)),
           "twell_choose_ell_width")
    return int(w.value), int(nb.value)


def check(buf: TwellBuffers, stream=None) -> int:
    """Synchronise and return the device status (SFFN_OK or SFFN_ERR_BACKUP_OVERFLOW)."""
    st = lib().sparse_ffn_check(ctypes.byref(buf.c()), _stream_ptr(stream))
    if st not in (SFFN_OK, SFFN_ERR_BACKUP_OVERFLOW):
        _check(st, "sparse_ffn_check")
    return st


class SparseFFN:
    """Handle of one layer.  W_up, W_down [d_ff, d_model] and b_up [d_ff] are device tensors
    in the layer dtype; they are borrowed (kept referenced here), not copied."""

    def __init__(self, cfg: Config, W_up, b_up, W_down):
        import torch
        want = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        for name, t, shape in (("W_up", W_up, (cfg.d_ff, cfg.d_model)), ("b_up", b_up, (cfg.d_ff,)),
                               ("W_down", W_down, (cfg.d_ff, cfg.d_model))):
            if t.dtype != want or not t.is_contiguous() or not t.is_cuda or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be a contiguous {want} device tensor of shape {shape}")
        self.cfg = cfg
        self._keep = (W_up, b_up, W_down)
        h = ctypes.c_void_p()
        c = cfg.c()
        _check(lib().sparse_ffn_create(ctypes.byref(c), _ptr(W_up), _ptr(b_up), _ptr(W_down),
                                       ctypes.byref(h)), "sparse_ffn_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.sparse_ffn_destroy(h)
            self._h = None

    def _check_x(self, x):
        import torch
        want = torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32
        if x.dtype != want or not x.is_contiguous() or not x.is_cuda or x.dim() != 2 \
                or x.shape[1] != self.cfg.d_model:
            raise ValueError(f"x must be a contiguous {want} device tensor [T, {self.cfg.d_model}]")

    def forward(self, x, act: Optional[TwellBuffers] = None, y=None, stream=None):
        """y = ReLU(x W_up^T + b) W_down; returns (y, act) where act is the packed TwELL."""
        import torch
        self._check_x(x)
        T = x.shape[0]
        act = act if act is not None else TwellBuffers(self.cfg, T, device=x.device)
        act._hold(self.cfg, T)
        y = y if y is not None else torch.empty_like(x)
        _check(lib().sparse_ffn_forward(self._h, _ptr(x), int(T), _ptr(y), ctypes.byref(act.c()),
                                        _stream_ptr(stream)), "sparse_ffn_forward")
        return y, act

    def forward_noalloc(self, x, act: TwellBuffers, y, stream=None, workspace=False):
        """sparse_ffn_forward_noalloc: the forward with its workspace in the library's fixed
        device scratch.  act (TwELL and backup outputs) and y are the caller's; act's own
        workspace is passed as NULL unless `workspace` is set (it is ignored either way)."""
        self._check_x(x)
        T = x.shape[0]
        act._hold(self.cfg, T)
        if tuple(y.shape) != tuple(x.shape) or y.dtype != x.dtype or not y.is_contiguous():
            raise ValueError("y must be a contiguous tensor shaped and typed like x")
        c = act.c()
        b = BuffersC(*[getattr(c, n) for n in BUFFER_FIELDS])
        if not workspace:
            b.workspace = None
        _check(lib().sparse_ffn_forward_noalloc(self._h, _ptr(x), int(T), _ptr(y), ctypes.byref(b),
                                                _stream_ptr(stream)), "sparse_ffn_forward_noalloc")
        return y, act

    def forward_dump(self, x, stream=None):
        """Forward that also returns the fp32 pre-activation z [T, d_ff] of the up kernel."""
        import torch
        self._check_x(x)
        T = x.shape[0]
        act = TwellBuffers(self.cfg, T, device=x.device)
        y = torch.empty_like(x)
        z = torch.empty((T, self.cfg.d_ff), dtype=torch.float32, device=x.device)
        _check(lib().sparse_ffn_forward_dump(self._h, _ptr(x), int(T), _ptr(y),
                                             ctypes.byref(act.c()), _ptr(z), _stream_ptr(stream)),
               "sparse_ffn_forward_dump")
        return y, act, z

    def set_down_policy(self, policy: str = "auto",
                        gather_density: float = DOWN_GATHER_DENSITY_DEFAULT,
                        mfma_density: float = DOWN_MFMA_DENSITY_DEFAULT):
        """Choice of the down-projection kernel: "auto" (by the layer's stored density,
        decided on the device: the per-token gather up to `gather_density`, the LDS-tile
        vector kernel up to `mfma_density`, the matrix cores above), or always "gather",
        "tiles", "mfma", "union" (matrix cores over each 64-token block's column union) or
        "sparse" (the 2:4 structured-sparse matrix-core instruction)."""
        code = {"auto": DOWN_AUTO, "gather": DOWN_GATHER, "mfma": DOWN_MFMA,
                "tiles": DOWN_TILES, "union": DOWN_UNION, "sparse": DOWN_SPARSE}.get(policy)
        if code is None:
            raise ValueError(f"unknown down policy {policy!r}")
        _check(lib().sparse_ffn_set_down_policy(self._h, code, float(gather_density),
                                                float(mfma_density)),
               "sparse_ffn_set_down_policy")

    def backward(self, x, dy, act: TwellBuffers, with_db: bool = True, out=None, stream=None):
        """Gradients of sparse_ffn_forward(x) -> act for dL/dy = dy.  Returns
        (dx, dW_up, dW_down, db_up or None, dh_vals, dh_bk_vals); dh is in act's TwELL
        structure (dh_vals [n_t, T, W], dh_bk_vals [backup_capacity, tile], layer dtype).
        `out` may pass that tuple back in to be overwritten instead of allocated."""
        import torch
        self._check_x(x)
        self._check_x(dy)
        T = x.shape[0]
        if dy.shape[0] != T or act.T != T:
            raise ValueError("x, dy and act must have the same number of tokens")
        cfg = self.cfg
        if out is not None:
            dx, dW_up, dW_down, db, dh_vals, dh_bk = out
        else:
            dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
            dev = x.device
            dh_vals = torch.empty((cfg.n_tiles, T, cfg.ell_width), dtype=dt, device=dev)
            dh_bk = torch.empty((max(cfg.backup_capacity, 1), cfg.tile), dtype=dt, device=dev)
            dx = torch.empty_like(x)
            dW_up = torch.empty((cfg.d_ff, cfg.d_model), dtype=torch.float32, device=dev)
            dW_down = torch.empty_like(dW_up)
            db = torch.empty(cfg.d_ff, dtype=torch.float32, device=dev) if with_db else None
        _check(lib().sparse_ffn_backward(self._h, _ptr(x), _ptr(dy), int(T), ctypes.byref(act.c()),
                                         _ptr(dh_vals), _ptr(dh_bk), _ptr(dx), _ptr(dW_up),
                                         _ptr(dW_down), _ptr(db) if db is not None else None,
                                         _stream_ptr(stream)), "sparse_ffn_backward")
        return dx, dW_up, dW_down, db, dh_vals, dh_bk

    def down(self, act: TwellBuffers, y=None, stream=None):
        """Down-projection only, from an existing TwELL."""
        import torch
        T = act.T
        dt = torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32
        y = y if y is not None else torch.empty((T, self.cfg.d_model), dtype=dt,
                                                device=act.t["vals"].device)
        _check(lib().sparse_ffn_down(self._h, ctypes.byref(act.c()), int(T), _ptr(y),
                                     _stream_ptr(stream)), "sparse_ffn_down")
        return y


def profile_enable(on: bool = True):
    _check(lib().sffn_profile_enable(1 if on else 0), "sffn_profile_enable")


def profile_only(names=None):
    """Time only the named kernels while profiling is enabled (None: all of them)."""
    arg = ",".join(names).encode() if names else None
    _check(lib().sffn_profile_only(arg), "sffn_profile_only")


def profile_reset():
    _check(lib().sffn_profile_reset(), "sffn_profile_reset")


def probe_gather_fma(W, rows, vals, y=None, stream=None):
    """y[t] = sum_j vals[t, j] W[rows[t, j]] (the library's measurement probe of a vector
    down-projection's gather-multiply-add).  W [F, d] bf16, rows [T, n] int32, vals [T, n]
    bf16, y [T, d] bf16; device tensors.  Returns y."""
    import torch
    F, d = W.shape
    T, n = rows.shape
    if y is None:
        y = torch.empty((T, d), dtype=torch.bfloat16, device=W.device)
    for t_, name in ((W, "W"), (rows, "rows"), (vals, "vals"), (y, "y")):
        if not t_.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if rows.dtype != torch.int32 or vals.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("W and vals bf16, rows int32")
    _check(lib().sffn_probe_gather_fma(_ptr(W), int(F), int(d), _ptr(rows), _ptr(vals), int(T),
                                       int(n), _ptr(y), _stream_ptr(stream)),
           "sffn_probe_gather_fma")
    return y


def profile_read(kernel: str):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().sffn_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)),
           "sffn_profile_read")
    return ms.value, n.value
