"""ctypes binding of libkvq.so: the C ABI of include/kvq.h, one Python function
per entry point, over torch tensors (device pointers and the current stream).
Argument marshalling only -- every step runs in the HIP library."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
BLOCK_ROWS = 32
CODECS = {"q8_0": 0, "q4_0": 1, "q4_g64": 2, "f16": 3}   # f16: the control codec (no scales)
GROUP = {"q8_0": 32, "q4_0": 32, "q4_g64": 64}
ROLE_K, ROLE_V = 0, 1

STATUS = {0: "KVQ_OK", 1: "KVQ_EINVAL", 2: "KVQ_EUNSUPPORTED", 3: "KVQ_ERANGE",
          4: "KVQ_EWORKSPACE", 5: "KVQ_EHIP", 6: "KVQ_EOVERFLOW", 7: "KVQ_EWAIT"}
KVQ_EOVERFLOW, KVQ_EWAIT = 6, 7


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class _Plane(ctypes.Structure):
    _fields_ = [("codec", ctypes.c_int32), ("role", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("k", _Plane), ("v", _Plane)]


class _PagedLayer(ctypes.Structure):
    _fields_ = [("pool", _Layer), ("block_table", ctypes.c_void_p), ("n_seqs", ctypes.c_int32),
                ("max_pages", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    """libkvq.so beside this file, or the file KVQ_LIBRARY names (another
    build of the same library, e.g. one with host sanitizers)."""
    return os.environ.get("KVQ_LIBRARY") or os.path.join(HERE, "libkvq.so")


def load_library():
    """Loads libkvq.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with block_quantized_kv_amd/build.py "
                          "(there is no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    PL, LY, PG = ctypes.POINTER(_Plane), ctypes.POINTER(_Layer), ctypes.POINTER(_PagedLayer)
    sig = {
        "kvq_row_code_bytes": (sz, [i32, i32]),
        "kvq_plane_bytes": (i32, [i32, i32, i32, i32, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "kvq_append": (i32, [LY, P, P, P, P, i32, P, P]),
        "kvq_decode_workspace_bytes": (sz, [LY, i32, i32, i64]),
        "kvq_attend_decode": (i32, [LY, P, P, i32, i32, i64, f32, P, P, sz, P, P]),
        "kvq_decode_mq_workspace_bytes": (sz, [LY, i32, i32, i32, i64]),
        "kvq_attend_decode_mq": (i32, [LY, P, P, i32, i32, i32, i64, f32, P, P, sz, P, P]),
        "kvq_append_attend_decode": (i32, [LY, P, P, P, P, i32, i32, i64, f32, P, P, sz, P, P]),
        "kvq_append_attend_decode_mq": (i32, [LY, P, P, P, P, i32, i32, i32, i64, f32, P, P, sz, P, P]),
        "kvq_append_attend_decode_noalloc": (i32, [LY, P, P, P, P, i32, i32, i64, f32, P, P, P]),
        "kvq_noalloc_scratch_bytes": (sz, []),
        "kvq_prefill_workspace_bytes": (sz, [LY, i32, i32]),
        "kvq_attend_prefill": (i32, [LY, P, i32, i64, i32, i32, f32, P, P, sz, P, P]),
        "kvq_dequant": (i32, [PL, i32, i64, i64, P, P]),
        "kvq_paged_append": (i32, [PG, P, P, P, P, i32, P, P]),
        "kvq_paged_decode_workspace_bytes": (sz, [PG, i32, i32, i32, i64]),
        "kvq_paged_attend_decode_mq": (i32, [PG, P, P, i32, i32, i32, i64, f32, P, P, sz, P, P]),
        "kvq_paged_append_attend_decode_mq": (i32, [PG, P, P, P, P, i32, i32, i32, i64, f32, P, P, sz, P, P]),
        "kvq_paged_attend_prefill": (i32, [PG, P, i32, i64, i32, i32, f32, P, P, sz, P, P]),
        "kvq_debug_append_wait": (i32, [i32, i32]),
        "kvq_status_str": (ctypes.c_char_p, [i32]),
        "kvq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def kvq_debug_append_wait(polls: int, hold_flag: bool = False) -> None:
    """The fused append's wait bound (polls) and, for tests only, a switch
    that keeps the appending wave from signalling."""
    _check(load_library().kvq_debug_append_wait(polls, 1 if hold_flag else 0))


def kvq_status_str(status: int) -> str:
    return load_library().kvq_status_str(status).decode()


def kvq_last_error() -> str:
    return load_library().kvq_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise KvqError(status, kvq_last_error())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _status(dev_status):
    """The optional device status word (int32 [1]) of an attention call."""
    if dev_status is not None:
        _need(dev_status, "dev_status", torch.int32, (1,))
    return _ptr(dev_status)


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def kvq_row_code_bytes(codec: str, head_dim: int) -> int:
    return int(load_library().kvq_row_code_bytes(CODECS[codec], head_dim))


def kvq_plane_bytes(codec: str, head_dim: int, n_kv_heads: int, n_seqs: int, capacity: int):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().kvq_plane_bytes(CODECS[codec], head_dim, n_kv_heads, n_seqs, capacity,
                                          ctypes.byref(c), ctypes.byref(s)))
    return c.value, s.value


class Plane:
    """One K or V cache plane (device memory owned by torch tensors)."""

    def __init__(self, codec: str, role: int, head_dim: int, n_kv_heads: int, n_seqs: int,
                 capacity: int, device="cuda", zero: bool = True):
        cb, sb = kvq_plane_bytes(codec, head_dim, n_kv_heads, n_seqs, capacity)
        alloc = torch.zeros if zero else torch.empty
        self.codes = alloc(cb, dtype=torch.uint8, device=device)
        self.scales = alloc(sb // 2, dtype=torch.int16, device=device)
        self.codec, self.role, self.head_dim = codec, role, head_dim
        self.n_kv_heads, self.n_seqs, self.capacity = n_kv_heads, n_seqs, capacity

    def struct(self) -> _Plane:
        return _Plane(CODECS[self.codec], self.role, self.head_dim, self.n_kv_heads, self.n_seqs,
                      0, self.capacity, self.codes.data_ptr(), self.scales.data_ptr())

    def clone(self) -> "Plane":
        p = object.__new__(Plane)
        p.__dict__.update(self.__dict__)
        p.codes, p.scales = self.codes.clone(), self.scales.clone()
        return p

    @property
    def nbytes(self) -> int:
        return self.codes.numel() + 2 * self.scales.numel()


class Layer:
    """The K and V planes of one layer (codecs may differ)."""

    def __init__(self, k: Plane, v: Plane):
        assert k.role == ROLE_K and v.role == ROLE_V
        self.k, self.v = k, v

    @classmethod
    def create(cls, k_codec: str, v_codec: str, head_dim: int, n_kv_heads: int, n_seqs: int,
               capacity: int, device="cuda", zero: bool = True) -> "Layer":
        return cls(Plane(k_codec, ROLE_K, head_dim, n_kv_heads, n_seqs, capacity, device, zero),
                   Plane(v_codec, ROLE_V, head_dim, n_kv_heads, n_seqs, capacity, device, zero))

    def struct(self) -> _Layer:
        return _Layer(self.k.struct(), self.v.struct())

    def clone(self) -> "Layer":
        return Layer(self.k.clone(), self.v.clone())

    @property
    def nbytes(self) -> int:
        return self.k.nbytes + self.v.nbytes


def _need(t, name, dtype, shape):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous device {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _one_device(owner, **named):
    """Every tensor (and stream) of a call must sit on the cache's device: a
    pointer into another GPU's memory would reach the kernels unchecked."""
    dev = owner.device
    for name, t in named.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}; the cache is on {dev}")


def kvq_append(layer: Layer, k_new, v_new, seq_idx, pos, dev_status=None, stream=None) -> None:
    """k_new/v_new fp32 [n_tokens][n_kv_heads][head_dim] (either may be None),
    seq_idx int32 [n_tokens], pos int64 [n_tokens] -- all device tensors."""
    _one_device(layer.k.codes, v_planes=layer.v.codes, k_new=k_new, v_new=v_new, seq_idx=seq_idx, pos=pos,
                dev_status=dev_status, stream=stream)
    n = int(seq_idx.numel())
    _need(seq_idx, "seq_idx", torch.int32, (n,))
    _need(pos, "pos", torch.int64, (n,))
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t is not None:
            _need(t, name, torch.float32, (n, layer.k.n_kv_heads, layer.k.head_dim))
    if dev_status is not None:
        _need(dev_status, "dev_status", torch.int32, (1,))
    L = layer.struct()
    _check(load_library().kvq_append(ctypes.byref(L), _ptr(k_new), _ptr(v_new), _ptr(seq_idx),
                                     _ptr(pos), n, _ptr(dev_status), _stream(stream)))


def kvq_decode_workspace_bytes(layer: Layer, n_q_heads: int, n_seqs: int, max_len: int) -> int:
    L = layer.struct()
    return int(load_library().kvq_decode_workspace_bytes(ctypes.byref(L), n_q_heads, n_seqs, max_len))


def decode_workspace(layer: Layer, n_q_heads: int, n_seqs: int, max_len: int):
    """A decode workspace (scratch for the split partials)."""
    nbytes = max(kvq_decode_workspace_bytes(layer, n_q_heads, n_seqs, max_len), 256)
    return torch.zeros(nbytes, dtype=torch.uint8, device=layer.k.codes.device)


def kvq_attend_decode(layer: Layer, q, seq_len, max_len: int, softmax_scale: float, out=None,
                      workspace=None, dev_status=None, stream=None):
    """q fp32 [n_seqs][n_q_heads][head_dim]; seq_len int64 [n_seqs] (device)."""
    _one_device(layer.k.codes, v_planes=layer.v.codes, q=q, seq_len=seq_len, out=out, workspace=workspace,
                dev_status=dev_status, stream=stream)
    n_seqs, hq, d = q.shape
    _need(q, "q", torch.float32, (n_seqs, hq, layer.k.head_dim))
    _need(seq_len, "seq_len", torch.int64, (n_seqs,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, (n_seqs, hq, layer.k.head_dim))
    if workspace is None:
        workspace = decode_workspace(layer, hq, n_seqs, max_len)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    L = layer.struct()
    _check(load_library().kvq_attend_decode(ctypes.byref(L), _ptr(q), _ptr(seq_len), n_seqs, hq,
                                            max_len, softmax_scale, _ptr(out), _ptr(workspace),
                                            workspace.numel(), _status(dev_status), _stream(stream)))
    return out


def kvq_decode_mq_workspace_bytes(layer: Layer, n_q_heads: int, n_seqs: int, q_len: int, max_len: int) -> int:
    L = layer.struct()
    return int(load_library().kvq_decode_mq_workspace_bytes(ctypes.byref(L), n_q_heads, n_seqs, q_len, max_len))


def decode_mq_workspace(layer: Layer, n_q_heads: int, n_seqs: int, q_len: int, max_len: int):
    """A multi-query decode workspace (scratch for the split partials)."""
    nbytes = max(kvq_decode_mq_workspace_bytes(layer, n_q_heads, n_seqs, q_len, max_len), 256)
    return torch.zeros(nbytes, dtype=torch.uint8, device=layer.k.codes.device)


def kvq_attend_decode_mq(layer: Layer, q, seq_len, max_len: int, softmax_scale: float, out=None,
                         workspace=None, dev_status=None, stream=None):
    """q fp32 [n_seqs][q_len][n_q_heads][head_dim]; query i of sequence b sits at
    row seq_len[b] - q_len + i (already appended) and attends rows up to it."""
    _one_device(layer.k.codes, v_planes=layer.v.codes, q=q, seq_len=seq_len, out=out, workspace=workspace,
                dev_status=dev_status, stream=stream)
    n_seqs, q_len, hq, d = q.shape
    _need(q, "q", torch.float32, (n_seqs, q_len, hq, layer.k.head_dim))
    _need(seq_len, "seq_len", torch.int64, (n_seqs,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, (n_seqs, q_len, hq, layer.k.head_dim))
    if workspace is None:
        workspace = decode_mq_workspace(layer, hq, n_seqs, q_len, max_len)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    L = layer.struct()
    _check(load_library().kvq_attend_decode_mq(ctypes.byref(L), _ptr(q), _ptr(seq_len), n_seqs, q_len, hq,
                                               max_len, softmax_scale, _ptr(out), _ptr(workspace),
                                               workspace.numel(), _status(dev_status), _stream(stream)))
    return out


def kvq_append_attend_decode(layer: Layer, k_new, v_new, q, seq_len, max_len: int, softmax_scale: float,
                             out=None, workspace=None, dev_status=None, stream=None):
    """k_new, v_new fp32 [n_seqs][n_kv_heads][head_dim] become row seq_len[b] - 1
    of sequence b; then q fp32 [n_seqs][n_q_heads][head_dim] attends as
    kvq_attend_decode (one launch does both)."""
    _one_device(layer.k.codes, v_planes=layer.v.codes, k_new=k_new, v_new=v_new, q=q, seq_len=seq_len, out=out,
                workspace=workspace, dev_status=dev_status, stream=stream)
    n_seqs, hq, d = q.shape
    H = layer.k.n_kv_heads
    _need(q, "q", torch.float32, (n_seqs, hq, layer.k.head_dim))
    _need(k_new, "k_new", torch.float32, (n_seqs, H, layer.k.head_dim))
    _need(v_new, "v_new", torch.float32, (n_seqs, H, layer.k.head_dim))
    _need(seq_len, "seq_len", torch.int64, (n_seqs,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, (n_seqs, hq, layer.k.head_dim))
    if workspace is None:
        workspace = decode_workspace(layer, hq, n_seqs, max_len)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    L = layer.struct()
    _check(load_library().kvq_append_attend_decode(ctypes.byref(L), _ptr(k_new), _ptr(v_new), _ptr(q),
                                                   _ptr(seq_len), n_seqs, hq, max_len, softmax_scale,
                                                   _ptr(out), _ptr(workspace), workspace.numel(),
                                                   _status(dev_status), _stream(stream)))
    return out


def kvq_noalloc_scratch_bytes() -> int:
    return int(load_library().kvq_noalloc_scratch_bytes())


def kvq_append_attend_decode_noalloc(layer: Layer, k_new, v_new, q, seq_len, max_len: int, softmax_scale: float,
                                     out, dev_status=None, stream=None):
    """kvq_append_attend_decode without a workspace: the library's own device
    scratch holds the split partials (the call allocates nothing; `out` must
    be given)."""
    _one_device(layer.k.codes, v_planes=layer.v.codes, k_new=k_new, v_new=v_new, q=q, seq_len=seq_len, out=out,
                dev_status=dev_status, stream=stream)
    n_seqs, hq, d = q.shape
    H = layer.k.n_kv_heads
    _need(q, "q", torch.float32, (n_seqs, hq, layer.k.head_dim))
    _need(k_new, "k_new", torch.float32, (n_seqs, H, layer.k.head_dim))
    _need(v_new, "v_new", torch.float32, (n_seqs, H, layer.k.head_dim))
    _need(seq_len, "seq_len", torch.int64, (n_seqs,))
    _need(out, "out", torch.float32, (n_seqs, hq, layer.k.head_dim))
    L = layer.struct()
    _check(load_library().kvq_append_attend_decode_noalloc(ctypes.byref(L), _ptr(k_new), _ptr(v_new), _ptr(q),
                                                           _ptr(seq_len), n_seqs, hq, max_len, softmax_scale,
                                                           _ptr(out), _status(dev_status), _stream(stream)))
    return out


def kvq_append_attend_decode_mq(layer: Layer, k_new, v_new, q, seq_len, max_len: int, softmax_scale: float,
                                out=None, workspace=None, dev_status=None, stream=None):
    """k_new, v_new fp32 [n_seqs][q_len][n_kv_heads][head_dim] become rows
    seq_len[b] - q_len + i; then q fp32 [n_seqs][q_len][n_q_heads][head_dim]
    attends as kvq_attend_decode_mq (the first launch appends)."""
    _one_device(layer.k.codes, v_planes=layer.v.codes, k_new=k_new, v_new=v_new, q=q, seq_len=seq_len, out=out,
                workspace=workspace, dev_status=dev_status, stream=stream)
    n_seqs, q_len, hq, d = q.shape
    H = layer.k.n_kv_heads
    _need(q, "q", torch.float32, (n_seqs, q_len, hq, layer.k.head_dim))
    _need(k_new, "k_new", torch.float32, (n_seqs, q_len, H, layer.k.head_dim))
    _need(v_new, "v_new", torch.float32, (n_seqs, q_len, H, layer.k.head_dim))
    _need(seq_len, "seq_len", torch.int64, (n_seqs,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, (n_seqs, q_len, hq, layer.k.head_dim))
    if workspace is None:
        workspace = decode_mq_workspace(layer, hq, n_seqs, q_len, max_len)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    L = layer.struct()
    _check(load_library().kvq_append_attend_decode_mq(ctypes.byref(L), _ptr(k_new), _ptr(v_new), _ptr(q),
                                                      _ptr(seq_len), n_seqs, q_len, hq, max_len,
                                                      softmax_scale, _ptr(out), _ptr(workspace),
                                                      workspace.numel(), _status(dev_status), _stream(stream)))
    return out


def kvq_prefill_workspace_bytes(layer: Layer, n_q_heads: int, n_tokens: int) -> int:
    L = layer.struct()
    return int(load_library().kvq_prefill_workspace_bytes(ctypes.byref(L), n_q_heads, n_tokens))


def kvq_attend_prefill(layer: Layer, q_bf16, seq: int, pos0: int, softmax_scale: float, out=None,
                       workspace=None, dev_status=None, stream=None):
    """q_bf16 bfloat16 [n_tokens][n_q_heads][head_dim] (device); rows of the chunk
    must already be appended at positions pos0..pos0+n_tokens-1."""
    _one_device(layer.k.codes, v_planes=layer.v.codes, q_bf16=q_bf16, out=out, workspace=workspace,
                dev_status=dev_status, stream=stream)
    T, hq, d = q_bf16.shape
    _need(q_bf16, "q_bf16", torch.bfloat16, (T, hq, layer.k.head_dim))
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32, device=q_bf16.device)
    _need(out, "out", torch.float32, (T, hq, layer.k.head_dim))
    ws_bytes = kvq_prefill_workspace_bytes(layer, hq, T)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q_bf16.device)
    L = layer.struct()
    _check(load_library().kvq_attend_prefill(ctypes.byref(L), _ptr(q_bf16), seq, pos0, T, hq,
                                             softmax_scale, _ptr(out), _ptr(workspace),
                                             0 if workspace is None else workspace.numel(),
                                             _status(dev_status), _stream(stream)))
    return out


def kvq_dequant(plane: Plane, seq: int, row0: int, n_rows: int, out=None, stream=None):
    """-> fp32 [n_kv_heads][n_rows][head_dim] of x_hat = code * scale."""
    _one_device(plane.codes, out=out, stream=stream)
    if out is None:
        out = torch.empty((plane.n_kv_heads, n_rows, plane.head_dim), dtype=torch.float32,
                          device=plane.codes.device)
    _need(out, "out", torch.float32, (plane.n_kv_heads, n_rows, plane.head_dim))
    P = plane.struct()
    _check(load_library().kvq_dequant(ctypes.byref(P), seq, row0, n_rows, _ptr(out), _stream(stream)))
    return out


class PagedLayer:
    """A page pool (a Layer whose "sequences" are pages and whose capacity is
    the rows per page) plus a block table int32 [n_seqs][max_pages] (device):
    entry [b][i] is the page holding rows [i * page_rows, (i + 1) * page_rows)
    of sequence b."""

    def __init__(self, pool: Layer, block_table):
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_cuda \
                or not block_table.is_contiguous():
            raise ValueError("block_table: expected a contiguous device int32 [n_seqs][max_pages] tensor")
        self.pool, self.block_table = pool, block_table
        self.n_seqs, self.max_pages = block_table.shape
        self.page_rows = pool.k.capacity

    def struct(self) -> _PagedLayer:
        return _PagedLayer(self.pool.struct(), self.block_table.data_ptr(), self.n_seqs, self.max_pages)


def kvq_paged_append(pl: PagedLayer, k_new, v_new, seq_idx, pos, dev_status=None, stream=None) -> None:
    """kvq_append through the block table (pos is the row within the sequence)."""
    _one_device(pl.pool.k.codes, v_planes=pl.pool.v.codes, block_table=pl.block_table, k_new=k_new, v_new=v_new,
                seq_idx=seq_idx, pos=pos, dev_status=dev_status, stream=stream)
    n = int(seq_idx.numel())
    _need(seq_idx, "seq_idx", torch.int32, (n,))
    _need(pos, "pos", torch.int64, (n,))
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t is not None:
            _need(t, name, torch.float32, (n, pl.pool.k.n_kv_heads, pl.pool.k.head_dim))
    if dev_status is not None:
        _need(dev_status, "dev_status", torch.int32, (1,))
    P = pl.struct()
    _check(load_library().kvq_paged_append(ctypes.byref(P), _ptr(k_new), _ptr(v_new), _ptr(seq_idx), _ptr(pos), n,
                                           _ptr(dev_status), _stream(stream)))


def kvq_paged_decode_workspace_bytes(pl: PagedLayer, n_q_heads: int, n_seqs: int, q_len: int, max_len: int) -> int:
    P = pl.struct()
    return int(load_library().kvq_paged_decode_workspace_bytes(ctypes.byref(P), n_q_heads, n_seqs, q_len, max_len))


def paged_decode_workspace(pl: PagedLayer, n_q_heads: int, n_seqs: int, q_len: int, max_len: int):
    nbytes = max(kvq_paged_decode_workspace_bytes(pl, n_q_heads, n_seqs, q_len, max_len), 256)
    return torch.zeros(nbytes, dtype=torch.uint8, device=pl.pool.k.codes.device)


def _paged_decode(pl: PagedLayer, k_new, v_new, q, seq_len, max_len, softmax_scale, out, workspace, dev_status,
                  stream):
    _one_device(pl.pool.k.codes, v_planes=pl.pool.v.codes, block_table=pl.block_table, k_new=k_new, v_new=v_new,
                q=q, seq_len=seq_len, out=out, workspace=workspace, dev_status=dev_status, stream=stream)
    n_seqs, q_len, hq, d = q.shape
    H, D = pl.pool.k.n_kv_heads, pl.pool.k.head_dim
    _need(q, "q", torch.float32, (n_seqs, q_len, hq, D))
    _need(seq_len, "seq_len", torch.int64, (n_seqs,))
    if k_new is not None:
        _need(k_new, "k_new", torch.float32, (n_seqs, q_len, H, D))
        _need(v_new, "v_new", torch.float32, (n_seqs, q_len, H, D))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, (n_seqs, q_len, hq, D))
    if workspace is None:
        workspace = paged_decode_workspace(pl, hq, n_seqs, q_len, max_len)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    P = pl.struct()
    lib = load_library()
    if k_new is None:
        st = lib.kvq_paged_attend_decode_mq(ctypes.byref(P), _ptr(q), _ptr(seq_len), n_seqs, q_len, hq, max_len,
                                            softmax_scale, _ptr(out), _ptr(workspace), workspace.numel(),
                                            _status(dev_status), _stream(stream))
    else:
        st = lib.kvq_paged_append_attend_decode_mq(ctypes.byref(P), _ptr(k_new), _ptr(v_new), _ptr(q),
                                                   _ptr(seq_len), n_seqs, q_len, hq, max_len, softmax_scale,
                                                   _ptr(out), _ptr(workspace), workspace.numel(),
                                                   _status(dev_status), _stream(stream))
    _check(st)
    return out


def kvq_paged_attend_decode_mq(pl: PagedLayer, q, seq_len, max_len: int, softmax_scale: float, out=None,
                               workspace=None, dev_status=None, stream=None):
    """q fp32 [n_seqs][q_len][n_q_heads][head_dim]: kvq_attend_decode_mq over paged planes."""
    return _paged_decode(pl, None, None, q, seq_len, max_len, softmax_scale, out, workspace, dev_status, stream)


def kvq_paged_append_attend_decode_mq(pl: PagedLayer, k_new, v_new, q, seq_len, max_len: int,
                                      softmax_scale: float, out=None, workspace=None, dev_status=None, stream=None):
    """kvq_append_attend_decode_mq over paged planes (k_new, v_new fp32
    [n_seqs][q_len][n_kv_heads][head_dim])."""
    return _paged_decode(pl, k_new, v_new, q, seq_len, max_len, softmax_scale, out, workspace, dev_status, stream)


def kvq_paged_attend_prefill(pl: PagedLayer, q_bf16, seq: int, pos0: int, softmax_scale: float, out=None,
                             dev_status=None, stream=None):
    """kvq_attend_prefill over paged planes: q_bf16 bfloat16 [n_tokens][n_q_heads][head_dim];
    the chunk's rows must already be appended (through the table) at pos0..pos0+n_tokens-1."""
    _one_device(pl.pool.k.codes, v_planes=pl.pool.v.codes, block_table=pl.block_table, q_bf16=q_bf16, out=out,
                dev_status=dev_status, stream=stream)
    T, hq, d = q_bf16.shape
    _need(q_bf16, "q_bf16", torch.bfloat16, (T, hq, pl.pool.k.head_dim))
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32, device=q_bf16.device)
    _need(out, "out", torch.float32, (T, hq, pl.pool.k.head_dim))
    P = pl.struct()
    _check(load_library().kvq_paged_attend_prefill(ctypes.byref(P), _ptr(q_bf16), seq, pos0, T, hq, softmax_scale,
                                                   _ptr(out), None, 0, _status(dev_status), _stream(stream)))
    return out
