"""Thin ctypes binding of ``libh2o.so`` (the C ABI declared in include/h2o.h).

The functions below carry the C names and only marshal arguments: torch
tensors become device pointers (after their shape, dtype, device and layout
are checked on the host, since the C ABI takes bare pointers), a stream
becomes its ``hipStream_t`` handle, and a non-OK status raises ``H2OError``
with the library's message. Every step of the path runs in the HIP kernels;
there is no fallback of any kind: if the library is not built, loading fails.

``H2OCache`` bundles one layer's cache tensors (allocated with torch, which
provides device memory and streams) with its descriptor.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; H2O_LIBRARY may name another build of the same sources
# (e.g. one with the host code sanitised), which is checked the same way.
LIB_PATH = os.environ.get("H2O_LIBRARY") or os.path.join(PKG, "libh2o.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "h2o.h")

H2O_OK, H2O_EINVAL, H2O_ESTATE, H2O_EWORKSPACE, H2O_EDEVICE = 0, 1, 2, 3, 4
H2O_F32, H2O_BF16, H2O_F16 = 0, 1, 2
H2O_POLICY_ACCUMULATED, H2O_POLICY_AVERAGED, H2O_POLICY_POSITION = 0, 1, 2
H2O_QUANT_NONE, H2O_QUANT_U8, H2O_QUANT_U4, H2O_QUANT_U2 = 0, 1, 2, 3
QUANT_CODE = {"u8": H2O_QUANT_U8, "u4": H2O_QUANT_U4, "u2": H2O_QUANT_U2}
QUANT_BITS = {"u8": 8, "u4": 4, "u2": 2}
POLICY_CODE = {"accumulated": H2O_POLICY_ACCUMULATED, "averaged": H2O_POLICY_AVERAGED,
               "position": H2O_POLICY_POSITION}
DTYPE_CODE = {torch.float32: H2O_F32, torch.bfloat16: H2O_BF16, torch.float16: H2O_F16}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}
STATUS_NAME = {0: "H2O_OK", 1: "H2O_EINVAL", 2: "H2O_ESTATE", 3: "H2O_EWORKSPACE", 4: "H2O_EDEVICE"}


def _header_int(name: str) -> int:
    with open(HEADER) as f:
        m = re.search(rf"#define\s+{name}\s+(\d+)", f.read())
    return int(m.group(1))


H2O_MAX_SLOTS = _header_int("H2O_MAX_SLOTS")
H2O_SPLIT_SCRATCH_BYTES = 16 << 20  # checked against include/h2o.h by the CPU tests
H2O_MAX_PROMPT = _header_int("H2O_MAX_PROMPT")


class H2OError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAME.get(status, status)}: {message}")
        self.status = status


class h2o_cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k_heavy", ctypes.c_int32), ("k_recent", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("policy", ctypes.c_int32), ("scale", ctypes.c_float),
        ("K", ctypes.c_void_p), ("V", ctypes.c_void_p),
        ("score", ctypes.c_void_p), ("pos", ctypes.c_void_p),
        ("n_used", ctypes.c_int32), ("t_next", ctypes.c_int32),
        ("steps", ctypes.c_int64), ("magic", ctypes.c_uint32), ("quant", ctypes.c_int32),
        ("k_qparam", ctypes.c_void_p), ("v_qparam", ctypes.c_void_p),
    ]


class h2o_state(ctypes.Structure):
    _fields_ = [
        ("n_used", ctypes.c_int32), ("t_next", ctypes.c_int32), ("k", ctypes.c_int32),
        ("k_heavy", ctypes.c_int32), ("k_recent", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("steps", ctypes.c_int64),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGNATURES = {
    "h2o_cache_init": (_I, [ctypes.POINTER(h2o_cache), _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                            _P, _P, _P, _P, _P]),
    "h2o_cache_init_quant": (_I, [ctypes.POINTER(h2o_cache), _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                                  _P, _P, _P, _P, _P, _P, _P]),
    "h2o_prefill_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "h2o_prefill_select": (_I, [ctypes.POINTER(h2o_cache), _P, _P, _P, _I, _P, ctypes.c_size_t, _P, _P]),
    "h2o_prefill_attention": (_I, [ctypes.POINTER(h2o_cache), _P, _P, _P, _I, _P, ctypes.c_size_t, _P, _P, _P,
                                   _P]),
    "h2o_prefill_select_lse": (_I, [ctypes.POINTER(h2o_cache), _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P,
                                    _P]),
    "h2o_decode_step": (_I, [ctypes.POINTER(h2o_cache), _P, _P, _P, _P, _P, _P]),
    "h2o_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "h2o_decode_step_split": (_I, [ctypes.POINTER(h2o_cache), _P, _P, _P, _P, _P, _I, _P, ctypes.c_size_t, _P]),
    "h2o_decode_step_split_noalloc": (_I, [ctypes.POINTER(h2o_cache), _P, _P, _P, _P, _P, _I, _P]),
    "h2o_cache_state": (_I, [ctypes.POINTER(h2o_cache), ctypes.POINTER(h2o_state), _P, _P, _P]),
    "h2o_cache_restore": (_I, [ctypes.POINTER(h2o_cache), _I, ctypes.c_int64]),
    "h2o_fullcache_decode": (_I, [_I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P, _P, _P]),
    "h2o_last_error": (ctypes.c_char_p, []),
    "h2o_build_digest": (ctypes.c_char_p, []),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built HIP library. Raises if it has not been built, or if the
    in-tree library was built from sources other than the ones beside it."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m kv_cache_eviction_decode_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    if os.path.abspath(path) == os.path.abspath(LIB_PATH):
        from .build import source_digest
        have, want = lib.h2o_build_digest().decode(), source_digest()
        if have != want:
            raise ImportError(f"{path} was built from sources {have}, the sources beside it are {want}: "
                              "rebuild with `python -m kv_cache_eviction_decode_amd.build`")
    _lib = lib
    return lib


def _check(status: int):
    if status != H2O_OK:
        raise H2OError(status, load_library().h2o_last_error().decode())


def _stream_handle(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _same_device(a: torch.device, b: torch.device) -> bool:
    return a.type == b.type and (b.index is None or a.index == b.index)


def _expect(t: torch.Tensor, name: str, shape, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and not _same_device(t.device, torch.device(device)):
        raise ValueError(f"{name} is on {t.device}, cache is on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ----------------------------------------------------------------------------- C names
def h2o_last_error() -> str:
    return load_library().h2o_last_error().decode()


def h2o_build_digest() -> str:
    return load_library().h2o_build_digest().decode()


def h2o_prefill_workspace_bytes(batch: int, heads: int, n: int) -> int:
    return int(load_library().h2o_prefill_workspace_bytes(batch, heads, n))


def h2o_cache_init(desc: h2o_cache, batch, heads, head_dim, k_heavy, k_recent, policy, scale,
                   K: torch.Tensor, V: torch.Tensor, score: torch.Tensor, pos: torch.Tensor, stream=None):
    k = k_heavy + k_recent
    dev = K.device
    dt = K.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    _expect(K, "K", (batch, heads, k, head_dim), dt)
    _expect(V, "V", (batch, heads, k, head_dim), dt, dev)
    _expect(score, "score", (batch, heads, k), torch.float32, dev)
    _expect(pos, "pos", (batch, heads, k), torch.int32, dev)
    code = POLICY_CODE.get(policy, policy) if isinstance(policy, str) else int(policy)
    _check(load_library().h2o_cache_init(ctypes.byref(desc), batch, heads, head_dim, k_heavy, k_recent,
                                         code, DTYPE_CODE[dt], float(scale), _ptr(K), _ptr(V),
                                         _ptr(score), _ptr(pos), _stream_handle(stream)))


def h2o_cache_init_quant(desc: h2o_cache, batch, heads, head_dim, k_heavy, k_recent, policy, dtype, scale,
                         quant: str, Kq: torch.Tensor, Vq: torch.Tensor, k_qparam: torch.Tensor,
                         v_qparam: torch.Tensor, score: torch.Tensor, pos: torch.Tensor, stream=None):
    """quant: "u8", "u4" or "u2"; Kq and Vq hold head_dim * bits / 8 bytes per row."""
    k = k_heavy + k_recent
    if dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dtype}")
    if quant not in QUANT_CODE:
        raise ValueError(f"unknown quantisation {quant!r}")
    dev = Kq.device
    rb = head_dim * QUANT_BITS[quant] // 8
    _expect(Kq, "Kq", (batch, heads, k, rb), torch.uint8)
    _expect(Vq, "Vq", (batch, heads, k, rb), torch.uint8, dev)
    _expect(k_qparam, "k_qparam", (batch, heads, 2, head_dim), torch.float32, dev)
    _expect(v_qparam, "v_qparam", (batch, heads, k, 2), torch.float32, dev)
    _expect(score, "score", (batch, heads, k), torch.float32, dev)
    _expect(pos, "pos", (batch, heads, k), torch.int32, dev)
    code = POLICY_CODE.get(policy, policy) if isinstance(policy, str) else int(policy)
    _check(load_library().h2o_cache_init_quant(ctypes.byref(desc), batch, heads, head_dim, k_heavy, k_recent,
                                               code, DTYPE_CODE[dtype], float(scale), QUANT_CODE[quant],
                                               _ptr(Kq), _ptr(Vq), _ptr(k_qparam), _ptr(v_qparam), _ptr(score),
                                               _ptr(pos), _stream_handle(stream)))


def _desc_dtype(desc):
    return CODE_DTYPE[desc.dtype]


def h2o_prefill_select(desc: h2o_cache, Q, K, V, workspace: torch.Tensor | None,
                       colsum_out: torch.Tensor | None = None, stream=None, device=None):
    B, H, d = desc.batch, desc.heads, desc.head_dim
    n = Q.shape[2]
    dt = _desc_dtype(desc)
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _expect(t, name, (B, H, n, d), dt, device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _expect(workspace, "workspace", (workspace.numel(),), torch.uint8, device)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    if colsum_out is not None:
        _expect(colsum_out, "colsum_out", (B, H, n), torch.float32, device)
    _check(load_library().h2o_prefill_select(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), n, ws_ptr,
                                             ws_bytes, _ptr(colsum_out), _stream_handle(stream)))


def _prompt_args(desc, Q, K, V, workspace, colsum_out, device):
    B, H, d = desc.batch, desc.heads, desc.head_dim
    n = Q.shape[2]
    dt = _desc_dtype(desc)
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _expect(t, name, (B, H, n, d), dt, device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _expect(workspace, "workspace", (workspace.numel(),), torch.uint8, device)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    if colsum_out is not None:
        _expect(colsum_out, "colsum_out", (B, H, n), torch.float32, device)
    return n, ws_ptr, ws_bytes


def h2o_prefill_attention(desc: h2o_cache, Q, K, V, workspace, out, lse_out=None, colsum_out=None, stream=None,
                          device=None):
    n, ws_ptr, ws_bytes = _prompt_args(desc, Q, K, V, workspace, colsum_out, device)
    shape = (desc.batch, desc.heads, n)
    _expect(out, "out", shape + (desc.head_dim,), torch.float32, device)
    if lse_out is not None:
        _expect(lse_out, "lse_out", shape, torch.float32, device)
    _check(load_library().h2o_prefill_attention(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), n, ws_ptr,
                                                ws_bytes, _ptr(out), _ptr(lse_out), _ptr(colsum_out),
                                                _stream_handle(stream)))


def h2o_prefill_select_lse(desc: h2o_cache, Q, K, V, lse, workspace, colsum_out=None, stream=None, device=None):
    n, ws_ptr, ws_bytes = _prompt_args(desc, Q, K, V, workspace, colsum_out, device)
    _expect(lse, "lse", (desc.batch, desc.heads, n), torch.float32, device)
    _check(load_library().h2o_prefill_select_lse(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), n, _ptr(lse),
                                                 ws_ptr, ws_bytes, _ptr(colsum_out), _stream_handle(stream)))


def h2o_decode_step(desc: h2o_cache, q, k_new, v_new, out, evicted, stream=None, device=None):
    B, H, d = desc.batch, desc.heads, desc.head_dim
    dt = _desc_dtype(desc)
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _expect(t, name, (B, H, d), dt, device)
    _expect(out, "out", (B, H, d), torch.float32, device)
    _expect(evicted, "evicted", (B, H), torch.int32, device)
    _check(load_library().h2o_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new),
                                          _ptr(out), _ptr(evicted), _stream_handle(stream)))


def h2o_decode_workspace_bytes(batch: int, heads: int, head_dim: int, k: int) -> int:
    return int(load_library().h2o_decode_workspace_bytes(batch, heads, head_dim, k))


def h2o_decode_step_split(desc: h2o_cache, q, k_new, v_new, out, evicted, workspace: torch.Tensor,
                          chunk_rows: int = 0, stream=None, device=None):
    B, H, d = desc.batch, desc.heads, desc.head_dim
    dt = _desc_dtype(desc)
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _expect(t, name, (B, H, d), dt, device)
    _expect(out, "out", (B, H, d), torch.float32, device)
    _expect(evicted, "evicted", (B, H), torch.int32, device)
    _expect(workspace, "workspace", (workspace.numel(),), torch.uint8, device)
    _check(load_library().h2o_decode_step_split(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new),
                                                _ptr(out), _ptr(evicted), int(chunk_rows), _ptr(workspace),
                                                workspace.numel(), _stream_handle(stream)))


def h2o_decode_step_split_noalloc(desc: h2o_cache, q, k_new, v_new, out, evicted, chunk_rows: int = 0,
                                  stream=None, device=None):
    """h2o_decode_step_split on the library's own workspace (allocates nothing)."""
    B, H, d = desc.batch, desc.heads, desc.head_dim
    dt = _desc_dtype(desc)
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _expect(t, name, (B, H, d), dt, device)
    _expect(out, "out", (B, H, d), torch.float32, device)
    _expect(evicted, "evicted", (B, H), torch.int32, device)
    _check(load_library().h2o_decode_step_split_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new),
                                                        _ptr(out), _ptr(evicted), int(chunk_rows),
                                                        _stream_handle(stream)))


def h2o_cache_state(desc: h2o_cache, pos_host=None, score_host=None, stream=None) -> h2o_state:
    st = h2o_state()
    k = desc.k_heavy + desc.k_recent
    shape = (desc.batch, desc.heads, k)
    for name, t, dt in (("pos_host", pos_host, torch.int32), ("score_host", score_host, torch.float32)):
        if t is not None:
            if tuple(t.shape) != shape or t.dtype != dt or t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous host {dt} tensor of shape {shape}")
    _check(load_library().h2o_cache_state(ctypes.byref(desc), ctypes.byref(st), _ptr(pos_host),
                                          _ptr(score_host), _stream_handle(stream)))
    return st


def h2o_cache_restore(desc: h2o_cache, t_next: int, steps: int = 0):
    _check(load_library().h2o_cache_restore(ctypes.byref(desc), int(t_next), int(steps)))


def h2o_fullcache_decode(q, Kc, Vc, out, scale, stream=None):
    B, H, L, d = Kc.shape
    dt = Kc.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    _expect(q, "q", (B, H, d), dt)
    _expect(Kc, "Kc", (B, H, L, d), dt, q.device)
    _expect(Vc, "Vc", (B, H, L, d), dt, q.device)
    _expect(out, "out", (B, H, d), torch.float32, q.device)
    _check(load_library().h2o_fullcache_decode(B, H, d, DTYPE_CODE[dt], float(scale), L, _ptr(q),
                                               _ptr(Kc), _ptr(Vc), _ptr(out), _stream_handle(stream)))


# ----------------------------------------------------------------------------- convenience
class H2OCache:
    """One layer's H2O cache: torch-allocated device tensors plus the C descriptor.

    quant=None stores rows in `dtype`; quant="u8", "u4" or "u2" stores 8-, 4- or
    2-bit codes (K and V are then uint8 [batch, heads, k, head_dim * bits / 8],
    with the grids in k_qparam and v_qparam) and `dtype` is that of the
    queries, keys and values handed in.
    """

    def __init__(self, batch, heads, head_dim, k_heavy, k_recent, dtype=torch.bfloat16,
                 scale=None, device="cuda", stream=None, policy="accumulated", quant=None):
        k = k_heavy + k_recent
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        if quant is not None and quant not in QUANT_CODE:
            raise ValueError(f"unknown quantisation {quant!r}")
        self.quant = quant
        self.dtype = dtype
        store = torch.uint8 if quant else dtype
        row = head_dim * QUANT_BITS[quant] // 8 if quant else head_dim
        self.K = torch.zeros(batch, heads, k, row, dtype=store, device=self.device)
        self.V = torch.zeros_like(self.K)
        self.score = torch.zeros(batch, heads, k, dtype=torch.float32, device=self.device)
        self.pos = torch.full((batch, heads, k), -1, dtype=torch.int32, device=self.device)
        self.scale = float(head_dim ** -0.5 if scale is None else scale)
        self.desc = h2o_cache()
        self._workspace = None
        self._split_ws = None
        if quant:
            self.k_qparam = torch.zeros(batch, heads, 2, head_dim, dtype=torch.float32, device=self.device)
            self.v_qparam = torch.zeros(batch, heads, k, 2, dtype=torch.float32, device=self.device)
            h2o_cache_init_quant(self.desc, batch, heads, head_dim, k_heavy, k_recent, policy, dtype, self.scale,
                                 quant, self.K, self.V, self.k_qparam, self.v_qparam, self.score, self.pos, stream)
        else:
            h2o_cache_init(self.desc, batch, heads, head_dim, k_heavy, k_recent, policy, self.scale,
                           self.K, self.V, self.score, self.pos, stream)

    @property
    def batch(self):
        return self.desc.batch

    @property
    def heads(self):
        return self.desc.heads

    @property
    def k(self):
        return self.desc.k_heavy + self.desc.k_recent

    @property
    def n_used(self):
        return self.desc.n_used

    @property
    def t_next(self):
        return self.desc.t_next

    def workspace(self, n: int) -> torch.Tensor:
        need = h2o_prefill_workspace_bytes(self.batch, self.heads, n)
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._workspace

    def prefill_select(self, Q, K, V, colsum_out=None, stream=None):
        n = Q.shape[2]
        ws = self.workspace(n) if n > 0 else None
        h2o_prefill_select(self.desc, Q, K, V, ws, colsum_out, stream, self.device)

    def prefill_attention(self, Q, K, V, out=None, lse_out=None, colsum_out=None, stream=None):
        """Prefill that also returns the prompt's attention output [B, H, n, d] (fp32)."""
        n = Q.shape[2]
        if out is None:
            out = torch.empty(self.batch, self.heads, n, self.desc.head_dim, dtype=torch.float32,
                              device=self.device)
        ws = self.workspace(n) if n > 0 else None
        h2o_prefill_attention(self.desc, Q, K, V, ws, out, lse_out, colsum_out, stream, self.device)
        return out

    def prefill_select_lse(self, Q, K, V, lse, colsum_out=None, stream=None):
        """Prefill scoring with the prompt rows' log normalisers given (natural log)."""
        n = Q.shape[2]
        ws = self.workspace(n) if n > 0 else None
        h2o_prefill_select_lse(self.desc, Q, K, V, lse, ws, colsum_out, stream, self.device)

    def decode_step(self, q, k_new, v_new, out=None, evicted=None, stream=None):
        if out is None:
            out = torch.empty(self.batch, self.heads, self.desc.head_dim, dtype=torch.float32, device=self.device)
        if evicted is None:
            evicted = torch.empty(self.batch, self.heads, dtype=torch.int32, device=self.device)
        h2o_decode_step(self.desc, q, k_new, v_new, out, evicted, stream, self.device)
        return out, evicted

    def split_workspace(self) -> torch.Tensor:
        """Workspace of the split decode step (logits and per-chunk partials)."""
        if self._split_ws is None:
            need = h2o_decode_workspace_bytes(self.batch, self.heads, self.desc.head_dim, self.k)
            self._split_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._split_ws

    def decode_step_split(self, q, k_new, v_new, out=None, evicted=None, chunk_rows=0, stream=None):
        if out is None:
            out = torch.empty(self.batch, self.heads, self.desc.head_dim, dtype=torch.float32, device=self.device)
        if evicted is None:
            evicted = torch.empty(self.batch, self.heads, dtype=torch.int32, device=self.device)
        h2o_decode_step_split(self.desc, q, k_new, v_new, out, evicted, self.split_workspace(), chunk_rows,
                              stream, self.device)
        return out, evicted

    def decode_step_split_noalloc(self, q, k_new, v_new, out, evicted, chunk_rows=0, stream=None):
        """Split decode step on the library's own workspace; out and evicted must be given."""
        h2o_decode_step_split_noalloc(self.desc, q, k_new, v_new, out, evicted, chunk_rows, stream, self.device)
        return out, evicted

    def state(self, copy=False, stream=None):
        if not copy:
            return h2o_cache_state(self.desc, stream=stream)
        pos = torch.empty(self.batch, self.heads, self.k, dtype=torch.int32)
        score = torch.empty(self.batch, self.heads, self.k, dtype=torch.float32)
        st = h2o_cache_state(self.desc, pos, score, stream)
        return st, pos, score

    def restore(self, t_next: int, steps: int = 0):
        h2o_cache_restore(self.desc, t_next, steps)
