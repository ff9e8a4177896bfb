"""Python binding of libpa.so: argument marshalling only.

Every function here turns torch tensors into ``pa_tensor`` descriptors
(device pointer, dtype, shape, strides) and calls the C ABI declared in
``include/pa.h``; all arithmetic happens in the library's HIP kernels.  torch
is used for device memory and the current stream, nothing else.  If the
library is missing or a tensor is not on the GPU the call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY may point at another build of the same library (A/B timing).
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_PKG, "libpa.so")

PA_F32, PA_F16, PA_BF16, PA_I32 = 0, 1, 2, 3
_DTYPES = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
           torch.int32: PA_I32}

PA_OK = 0
STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_DTYPE", -3: "PA_ERR_SHAPE",
          -4: "PA_ERR_STRIDE", -5: "PA_ERR_UNSUPPORTED", -6: "PA_ERR_ALLOC",
          -7: "PA_ERR_LAUNCH", -8: "PA_ERR_ARG"}


class PaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class PaDecodePlanInfo(ctypes.Structure):
    _fields_ = [("workers", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("grid", ctypes.c_int64 * 3), ("workspace_bytes", ctypes.c_int64)]


class PAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


_lib = None

EXPORTS = ("pa_decode", "pa_decode_noalloc", "pa_decode_shared_prefix", "pa_prefill", "pa_write_kv", "pa_copy_blocks", "pa_status_string",
           "pa_last_error", "pa_decode_plan", "pa_workspace_release", "pa_profiler_enable",
           "pa_profiler_reset", "pa_profiler_read", "pa_profiler_samples",
           "pa_clock_probe", "pa_bm_create", "pa_bm_destroy",
           "pa_bm_num_free", "pa_bm_refcount", "pa_bm_add", "pa_bm_fork", "pa_bm_append",
           "pa_bm_take_copies", "pa_bm_free", "pa_bm_block_table")


def lib():
    """Load libpa.so (built in-tree by ``paged_kv_cache_decode_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m paged_kv_cache_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(PaTensor)
    L.pa_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, ctypes.c_void_p]
    L.pa_decode_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, P, ctypes.c_void_p]
    L.pa_decode_lse.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_void_p]
    L.pa_merge_states.argtypes = [P, P, P, P, ctypes.c_void_p]
    L.pa_decode_shared_prefix.argtypes = [P, P, P, P, P, ctypes.c_int32, ctypes.c_float, P,
                                          ctypes.c_void_p]
    L.pa_prefill.argtypes = [P, P, P, P, P, P, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                             P, ctypes.c_void_p]
    L.pa_write_kv.argtypes = [P, P, P, P, P, ctypes.c_void_p]
    L.pa_decode_plan.argtypes = [P, P, P, P, P, P, ctypes.POINTER(PaDecodePlanInfo)]
    L.pa_workspace_release.argtypes = [ctypes.c_void_p]
    L.pa_copy_blocks.argtypes = [P, P, P, P, ctypes.c_void_p]
    L.pa_profiler_samples.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_float),
                                      ctypes.c_int64]
    L.pa_profiler_samples.restype = ctypes.c_int64
    L.pa_clock_probe.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.pa_clock_probe.restype = ctypes.c_int
    V, I32P, I64P = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    L.pa_bm_create.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.pa_bm_create.restype = V
    L.pa_bm_destroy.argtypes = [V]
    L.pa_bm_destroy.restype = None
    L.pa_bm_num_free.argtypes = [V]
    L.pa_bm_refcount.argtypes = [V, ctypes.c_int32]
    L.pa_bm_add.argtypes = [V, ctypes.c_int64]
    L.pa_bm_fork.argtypes = [V, ctypes.c_int64, ctypes.c_int64]
    L.pa_bm_append.argtypes = [V, ctypes.c_int64, ctypes.c_int32, I32P]
    L.pa_bm_take_copies.argtypes = [V, I32P, I32P, ctypes.c_int32]
    L.pa_bm_free.argtypes = [V, ctypes.c_int64]
    L.pa_bm_block_table.argtypes = [V, I64P, ctypes.c_int32, ctypes.c_int32, I32P, I32P]
    for f in ("pa_decode", "pa_decode_noalloc", "pa_decode_lse", "pa_merge_states", "pa_decode_shared_prefix",
              "pa_prefill", "pa_write_kv",
              "pa_copy_blocks", "pa_decode_plan",
              "pa_workspace_release", "pa_profiler_enable", "pa_profiler_read", "pa_bm_num_free",
              "pa_bm_refcount", "pa_bm_add", "pa_bm_fork", "pa_bm_append", "pa_bm_take_copies",
              "pa_bm_free", "pa_bm_block_table"):
        getattr(L, f).restype = ctypes.c_int
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_profiler_enable.argtypes = [ctypes.c_int]
    L.pa_profiler_reset.argtypes = []
    L.pa_profiler_reset.restype = None
    L.pa_profiler_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int64)]
    _lib = L
    return L


def describe(t: torch.Tensor) -> PaTensor:
    """pa_tensor descriptor of a GPU tensor (no copy)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors passed to libpa must live on the GPU")
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d = PaTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _check(status: int):
    if status != PA_OK:
        raise PAError(status, lib().pa_last_error().decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def decode(q, k_pool, v_pool, block_table, context_lens, scale, out=None, out_dtype=None,
           stream=None):
    """Paged decode attention; returns ``out [S, H, d]`` (see ``pa_decode``)."""
    L = lib()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens)]
    o = describe(out)
    _check(L.pa_decode(*[ctypes.byref(a) for a in args], ctypes.c_float(scale),
                       ctypes.byref(o), _stream(stream)))
    return out


def decode_noalloc(q, k_pool, v_pool, block_table, context_lens, scale, out=None,
                   out_dtype=None, stream=None):
    """pa_decode on the library's fixed per-GPU workspace (no allocation in
    the call); see ``pa_decode_noalloc``."""
    L = lib()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens)]
    o = describe(out)
    _check(L.pa_decode_noalloc(*[ctypes.byref(a) for a in args], ctypes.c_float(scale),
                               ctypes.byref(o), _stream(stream)))
    return out


def decode_lse(q, k_pool, v_pool, block_table, context_lens, scale, out=None, lse=None,
               out_dtype=None, stream=None):
    """Paged decode that also returns each (sequence, head)'s natural-log
    log-sum-exp: ``(out [S, H, d], lse [S, H] f32)`` (see ``pa_decode_lse``)."""
    L = lib()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens)]
    o, ls = describe(out), describe(lse)
    _check(L.pa_decode_lse(*[ctypes.byref(a) for a in args], ctypes.c_float(scale),
                           ctypes.byref(o), ctypes.byref(ls), _stream(stream)))
    return out, lse


def merge_states(part_out, part_lse, out=None, lse=None, out_dtype=torch.float32,
                 want_lse=True, stream=None):
    """Join partial attention states ``part_out [P, S, H, d]`` (f32) with
    their log-sum-exps ``part_lse [P, S, H]``; returns ``(out, lse)`` (lse
    None unless wanted) -- see ``pa_merge_states``."""
    L = lib()
    if out is None:
        out = torch.empty(part_out.shape[1:], dtype=out_dtype, device=part_out.device)
    if lse is None and want_lse:
        lse = torch.empty(part_out.shape[1:3], dtype=torch.float32, device=part_out.device)
    a, b, o = describe(part_out), describe(part_lse), describe(out)
    ls = describe(lse) if lse is not None else None
    _check(L.pa_merge_states(ctypes.byref(a), ctypes.byref(b), ctypes.byref(o),
                             ctypes.byref(ls) if ls is not None else None, _stream(stream)))
    return out, lse


def decode_shared_prefix(q, k_pool, v_pool, block_table, context_lens, prefix_len, scale,
                         out=None, out_dtype=None, stream=None):
    """pa_decode for sequences sharing their first ``prefix_len`` tokens (in
    the same physical blocks); see ``pa_decode_shared_prefix``."""
    L = lib()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens)]
    o = describe(out)
    _check(L.pa_decode_shared_prefix(*[ctypes.byref(a) for a in args], int(prefix_len),
                                     ctypes.c_float(scale), ctypes.byref(o), _stream(stream)))
    return out


def decode_plan(q, k_pool, v_pool, block_table, context_lens, out):
    """What pa_decode would launch (workers, grid, workspace)."""
    L = lib()
    info = PaDecodePlanInfo()
    args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens, out)]
    _check(L.pa_decode_plan(*[ctypes.byref(a) for a in args], ctypes.byref(info)))
    return dict(workers=info.workers, waves_per_group=info.waves_per_group,
                block_threads=info.block_threads, grid=tuple(info.grid),
                workspace_bytes=info.workspace_bytes)


def prefill(q, k_pool, v_pool, block_table, context_lens, query_start_loc, max_query_len,
            scale, causal=True, out=None, out_dtype=None, stream=None):
    """Paged prefill attention; returns ``out [T, H, d]`` (see ``pa_prefill``)."""
    L = lib()
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens, query_start_loc)]
    o = describe(out)
    _check(L.pa_prefill(*[ctypes.byref(a) for a in args], ctypes.c_int32(int(max_query_len)),
                        ctypes.c_float(scale), ctypes.c_int32(1 if causal else 0),
                        ctypes.byref(o), _stream(stream)))
    return out


def write_kv(k_new, v_new, slot_mapping, k_pool, v_pool, stream=None):
    """Write new tokens' K/V rows into their pool slots, in place."""
    L = lib()
    args = [describe(x) for x in (k_new, v_new, slot_mapping, k_pool, v_pool)]
    _check(L.pa_write_kv(*[ctypes.byref(a) for a in args], _stream(stream)))


def copy_blocks(k_pool, v_pool, src, dst, stream=None):
    """Copy whole blocks src[i] -> dst[i] in both pools (device int32 ids)."""
    L = lib()
    args = [describe(x) for x in (k_pool, v_pool, src, dst)]
    _check(L.pa_copy_blocks(*[ctypes.byref(a) for a in args], _stream(stream)))


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class BlockManager:
    """The library's host block manager (``pa_bm_*``): block tables, on-demand
    blocks, forks that share blocks, copy-on-write pairs."""

    def __init__(self, num_blocks: int, block_size: int):
        self._L = lib()
        self._h = self._L.pa_bm_create(num_blocks, block_size)
        if not self._h:
            raise PAError(-8, self._L.pa_last_error().decode())
        self.block_size = block_size

    def close(self):
        if self._h:
            self._L.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _call(self, st):
        if st < 0:
            raise PAError(st, self._L.pa_last_error().decode())
        return st

    @property
    def num_free(self) -> int:
        return self._call(self._L.pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return self._call(self._L.pa_bm_refcount(self._h, block))

    def add(self, seq_id: int):
        self._call(self._L.pa_bm_add(self._h, seq_id))

    def fork(self, parent: int, child: int):
        self._call(self._L.pa_bm_fork(self._h, parent, child))

    def append(self, seq_id: int, n: int) -> np.ndarray:
        """Slots (block * B + position) of n new tokens, int32 [n]."""
        out = np.empty(max(n, 1), dtype=np.int32)
        self._call(self._L.pa_bm_append(self._h, seq_id, n, _i32p(out)))
        return out[:n]

    def take_copies(self, max_pairs: int = 1 << 16):
        """Queued copy-on-write pairs as (src, dst) int32 arrays."""
        src = np.empty(max_pairs, dtype=np.int32)
        dst = np.empty(max_pairs, dtype=np.int32)
        k = self._call(self._L.pa_bm_take_copies(self._h, _i32p(src), _i32p(dst), max_pairs))
        return src[:k].copy(), dst[:k].copy()

    def free(self, seq_id: int):
        self._call(self._L.pa_bm_free(self._h, seq_id))

    def block_table(self, seq_ids, max_blocks: int):
        """(table int32 [S, max_blocks] with -1 padding, lens int32 [S])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        S = len(ids)
        table = np.empty((max(S, 1), max(max_blocks, 1)), dtype=np.int32)
        lens = np.empty(max(S, 1), dtype=np.int32)
        self._call(self._L.pa_bm_block_table(
            self._h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), S, max_blocks,
            _i32p(table), _i32p(lens)))
        return table[:S, :max_blocks].copy(), lens[:S].copy()


def workspace_release(stream=None):
    """Free the decode workspace the library keeps for `stream`."""
    _check(lib().pa_workspace_release(_stream(stream)))


def clock_probe(out, ticks: int = 20000, stream=None):
    """Launch pa_clock_probe writing into ``out`` (int64 [2] on the GPU);
    shader MHz = 100 * out[0] / out[1] once the stream has run it."""
    if out.dtype != torch.int64 or out.numel() < 2 or not out.is_cuda:
        raise ValueError("out must be a GPU int64 tensor of 2 elements")
    _check(lib().pa_clock_probe(int(ticks), ctypes.c_void_p(out.data_ptr()), _stream(stream)))


def profiler_enable(on: bool = True):
    lib().pa_profiler_enable(1 if on else 0)


def profiler_reset():
    lib().pa_profiler_reset()


def profiler_read(kernel: str):
    """(total milliseconds, launches) recorded for a kernel name."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().pa_profiler_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def profiler_samples(kernel: str):
    """Per-launch durations (ms, launch order) recorded for a kernel name."""
    _, n = profiler_read(kernel)
    if n == 0:
        return []
    buf = (ctypes.c_float * n)()
    got = lib().pa_profiler_samples(kernel.encode(), buf, n)
    if got < 0:
        _check(int(got))
    return list(buf[:got])


class PreparedDecode:
    """A pa_decode call (or, with ``prefix_len``, a pa_decode_shared_prefix
    call) with its descriptors built once (for tight loops)."""

    def __init__(self, q, k_pool, v_pool, block_table, context_lens, scale, out,
                 prefix_len=None):
        self._keep = (q, k_pool, v_pool, block_table, context_lens, out)
        self._args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens)]
        self._out = describe(out)
        self._refs = [ctypes.byref(x) for x in self._args]
        self._scale = ctypes.c_float(scale)
        self._prefix = prefix_len
        self._L = lib()

    def __call__(self, stream=None):
        if self._prefix is None:
            _check(self._L.pa_decode(*self._refs, self._scale, ctypes.byref(self._out),
                                     _stream(stream)))
        else:
            _check(self._L.pa_decode_shared_prefix(*self._refs, int(self._prefix), self._scale,
                                                   ctypes.byref(self._out), _stream(stream)))
        return self._keep[-1]


class PreparedPrefill:
    """A pa_prefill call with its descriptors built once."""

    def __init__(self, q, k_pool, v_pool, block_table, context_lens, query_start_loc,
                 max_query_len, scale, causal, out):
        self._keep = (q, k_pool, v_pool, block_table, context_lens, query_start_loc, out)
        self._args = [describe(x) for x in (q, k_pool, v_pool, block_table, context_lens,
                                            query_start_loc)]
        self._out = describe(out)
        self._refs = [ctypes.byref(x) for x in self._args]
        self._maxq = ctypes.c_int32(int(max_query_len))
        self._scale = ctypes.c_float(scale)
        self._causal = ctypes.c_int32(1 if causal else 0)
        self._L = lib()

    def __call__(self, stream=None):
        _check(self._L.pa_prefill(*self._refs, self._maxq, self._scale, self._causal,
                                  ctypes.byref(self._out), _stream(stream)))
        return self._keep[-1]


_TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def upload(a, dtype: str | None = None) -> torch.Tensor:
    """Copy a storage-format numpy array (uint16 bit patterns for 16-bit
    formats) to a GPU tensor of the matching torch dtype."""
    import numpy as np
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(_TORCH_DT[dtype]).cuda()
    return torch.from_numpy(a).cuda()


def upload_pool(a: np.ndarray, dtype: str | None = None, head_major: bool = False):
    """A [NB, B, Hkv, d] pool on the device.  With head_major the memory is a
    contiguous [NB, Hkv, B, d] buffer (a KV head's B rows of a block
    adjacent) and the tensor is its [NB, B, Hkv, d] view; the library reads
    either layout."""
    if not head_major:
        return upload(a, dtype)
    return upload(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), dtype).permute(0, 2, 1, 3)


def upload_case(case, head_major: bool = False) -> dict:
    """Device copies of a workloads.PagedCase's arrays (pools in the
    token-major layout, or head-major within blocks)."""
    d = dict(q=upload(case.q, case.dtype),
             k_pool=upload_pool(case.k_pool, case.dtype, head_major),
             v_pool=upload_pool(case.v_pool, case.dtype, head_major),
             block_table=upload(case.block_table), context_lens=upload(case.context_lens))
    if case.query_start_loc is not None:
        d["query_start_loc"] = upload(case.query_start_loc)
    return d
