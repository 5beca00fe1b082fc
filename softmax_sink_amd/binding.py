"""ctypes binding of libsinkattn.so (include/sink_attn.h).

Argument marshalling only: every step of the computation runs in the
library's HIP kernels; torch provides device memory and the stream. The
functions ``sink_attn_metadata``, ``sink_attn_fwd``, ``sink_attn_bwd``,
``sink_attn_metadata_paged``, ``sink_attn_fwd_paged``,
``sink_attn_metadata_padded``, ``sink_attn_fwd_padded``,
``sink_attn_bwd_padded``, ``sink_attn_merge`` and ``sink_attn_arm_timing``
mirror the C entry points one to one. ``Plan``, ``PagedPlan``,
``PaddedPlan``, ``forward``, ``forward_paged``, ``forward_padded``,
``backward``, ``backward_padded``, ``SinkAttnFunction``,
``learnable_sink_attn_varlen`` and ``learnable_sink_attn_padded`` are
conveniences that allocate outputs and workspace with torch and call them.

If the library has not been built the first call raises: there is no other
path.
"""
import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsinkattn.so")

OK, E_INVALID, E_UNSUPPORTED, E_META_MISMATCH, E_BUFFER_TOO_SMALL, E_HIP = range(6)
FP32, BF16, FP16 = 0, 1, 2
TND, BSND, BNSD = 0, 1, 2
LAYOUTS = {"TND": TND, "BSND": BSND, "BNSD": BNSD}


def dtype_code(dtype):
    """sink_attn_dtype of a name ("fp32", "bf16", "fp16") or torch dtype."""
    import torch
    codes = {"fp32": FP32, "bf16": BF16, "fp16": FP16, torch.float32: FP32,
             torch.bfloat16: BF16, torch.float16: FP16}
    if dtype not in codes:
        raise SinkAttnError(E_UNSUPPORTED, f"dtype {dtype}")
    return codes[dtype]


class SinkAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_heads_q", "num_heads_k", "head_dim",
        "total_q", "total_k", "max_seqlen_q", "max_seqlen_k",
        "causal", "win_left", "win_right", "dtype",
        "layout_q", "layout_out", "seq_q", "seq_k")]


def _problem(*fields):
    """Problem from Python ints, each checked to fit its int32 field (ctypes
    would silently keep only the low 32 bits, e.g. turn a window of
    2**32 + 5 into 5)."""
    vals = [int(x) for x in fields]
    for (name, _), x in zip(Problem._fields_, vals):
        if not -2 ** 31 <= x < 2 ** 31:
            raise ValueError(f"{name} = {x} does not fit an int32 field")
    return Problem(*vals)


PA_BBND, PA_BNBD = 0, 1
CACHE_LAYOUTS = {"BBND": PA_BBND, "BNBD": PA_BNBD}


class PagedKV(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("block_size", "max_blocks_per_seq", "num_blocks",
                                              "layout")]


_lib = None


def lib():
    """The loaded library (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m softmax_sink_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        vp = ctypes.c_void_p
        L.sink_attn_metadata.argtypes = [ctypes.POINTER(Problem), i32p, i32p, i32p,
                                         ctypes.c_int64, i64p, i64p, i64p]
        L.sink_attn_metadata.restype = ctypes.c_int
        L.sink_attn_fwd.argtypes = [ctypes.POINTER(Problem), i32p, vp, vp, vp, vp, vp, vp,
                                    vp, ctypes.c_float, vp, vp, vp, ctypes.c_int64, vp]
        L.sink_attn_fwd.restype = ctypes.c_int
        L.sink_attn_bwd.argtypes = [ctypes.POINTER(Problem), i32p, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
                                    ctypes.c_int64, vp]
        L.sink_attn_bwd.restype = ctypes.c_int
        L.sink_attn_bwd_noalloc.argtypes = L.sink_attn_bwd.argtypes[:17] + [vp]
        L.sink_attn_bwd_noalloc.restype = ctypes.c_int
        L.sink_attn_metadata_paged.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PagedKV),
                                               i32p, i32p, i32p, i32p, ctypes.c_int64, i64p,
                                               i64p]
        L.sink_attn_metadata_paged.restype = ctypes.c_int
        L.sink_attn_fwd_paged.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PagedKV), i32p,
                                          vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                          vp, vp, ctypes.c_int64, vp]
        L.sink_attn_fwd_paged.restype = ctypes.c_int
        L.sink_attn_metadata_padded.argtypes = [ctypes.POINTER(Problem), i32p, i32p, i32p,
                                                ctypes.c_int64, i64p, i64p, i64p]
        L.sink_attn_metadata_padded.restype = ctypes.c_int
        L.sink_attn_fwd_padded.argtypes = L.sink_attn_fwd.argtypes
        L.sink_attn_fwd_padded.restype = ctypes.c_int
        L.sink_attn_bwd_padded.argtypes = L.sink_attn_bwd.argtypes
        L.sink_attn_bwd_padded.restype = ctypes.c_int
        L.sink_attn_merge.argtypes = [ctypes.c_int32] * 6 + [vp, vp, vp, vp, vp, vp]
        L.sink_attn_merge.restype = ctypes.c_int
        L.sink_attn_upload_table.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.sink_attn_upload_table.restype = ctypes.c_int
        L.sink_attn_arm_timing.argtypes = [vp, vp]
        L.sink_attn_arm_timing.restype = ctypes.c_int
        L.sink_attn_status_string.argtypes = [ctypes.c_int]
        L.sink_attn_status_string.restype = ctypes.c_char_p
        L.sink_attn_abi_version.argtypes = []
        L.sink_attn_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(s):
    return lib().sink_attn_status_string(int(s)).decode()


def abi_version():
    return lib().sink_attn_abi_version()


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if a is not None else None


def _ptr(t):
    """Device pointer of a tensor (or an int address), None -> NULL. A host
    tensor or a strided view is refused here: the kernels address device
    memory densely from the base pointer."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor is not on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor is not contiguous")
    return t.data_ptr()


def _torch_dtype(code):
    import torch
    return {FP32: torch.float32, BF16: torch.bfloat16, FP16: torch.float16}[int(code)]


def _expect(t, name, shape, dtype):
    """A tensor handed to the kernels must be on the GPU, contiguous, and of
    the shape and dtype its plan implies: a shorter buffer would be read or
    written past its end."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got "
                         f"{tuple(t.shape)} {t.dtype}")


def _expect_sinks(sinks, hq):
    import torch
    if sinks is not None:
        _expect(sinks, "sinks", (hq,), torch.float32)


def _expect_packed(plan, q=None, k=None, v=None, dout=None, out=None, lse=None):
    """Shapes of the packed (TND) tensors of a Plan or PagedPlan."""
    import torch
    p = plan.problem
    dt = _torch_dtype(p.dtype)
    qs, ks = (p.total_q, p.num_heads_q, p.head_dim), (p.total_k, p.num_heads_k, p.head_dim)
    for t, name, shape in ((q, "q", qs), (dout, "dout", qs), (out, "out", qs), (k, "k", ks),
                           (v, "v", ks)):
        if t is not None:
            _expect(t, name, shape, dt)
    if lse is not None:
        _expect(lse, "lse", (p.num_heads_q, p.total_q), torch.float32)


def _expect_padded(plan, q=None, k=None, v=None, dout=None, out=None, lse=None):
    """Shapes of the batch-padded tensors of a PaddedPlan."""
    import torch
    p = plan.problem
    dt = _torch_dtype(p.dtype)
    if plan.layout == "BNSD":
        qs, ks = (p.batch, p.num_heads_q, p.seq_q, p.head_dim), (p.batch, p.num_heads_k, p.seq_k, p.head_dim)
    else:
        qs, ks = (p.batch, p.seq_q, p.num_heads_q, p.head_dim), (p.batch, p.seq_k, p.num_heads_k, p.head_dim)
    os_ = plan.out_shape()
    for t, name, shape in ((q, "q", qs), (k, "k", ks), (v, "v", ks), (dout, "dout", os_),
                           (out, "out", os_)):
        if t is not None:
            _expect(t, name, shape, dt)
    if lse is not None:
        _expect(lse, "lse", (p.batch, p.num_heads_q, p.seq_q), torch.float32)


def make_problem(cu_q, cu_k, num_heads_q, num_heads_k, head_dim, causal,
                 win_left=-1, win_right=-1, dtype=BF16):
    """Problem struct from host cu_seqlens (numpy int32)."""
    cu_q = np.asarray(cu_q, dtype=np.int32)
    cu_k = np.asarray(cu_k, dtype=np.int32)
    lq, lk = np.diff(cu_q), np.diff(cu_k)
    return _problem(len(cu_q) - 1, num_heads_q, num_heads_k, head_dim,
                    int(cu_q[-1]), int(cu_k[-1]),
                    int(lq.max()) if len(lq) else 0, int(lk.max()) if len(lk) else 0,
                    int(bool(causal)), win_left, win_right, dtype)


def _metadata(name, call, words, out):
    """The two-call protocol of the metadata entry points. call(meta_ptr,
    capacity) runs the C function; words receives the table size. With `out`
    (a C-contiguous int32 array, e.g. a view of pinned host memory) the table
    is written straight into it in one call and the filled prefix returned."""
    if out is not None:
        if out.dtype != np.int32 or not out.flags.c_contiguous:
            raise ValueError("out must be a C-contiguous int32 array")
        st = call(_i32p(out), len(out))
        if st == E_BUFFER_TOO_SMALL:
            raise SinkAttnError(st, f"{name}: out holds {len(out)} words, "
                                    f"the table needs {words.value}")
        if st != OK:
            raise SinkAttnError(st, name)
        return out[:words.value]
    st = call(None, 0)
    if st != OK:
        raise SinkAttnError(st, name)
    meta = np.zeros(words.value, dtype=np.int32)
    st = call(_i32p(meta), words.value)
    if st != OK:
        raise SinkAttnError(st, name)
    return meta


def sink_attn_metadata(problem, cu_seqlens_q_host, cu_seqlens_k_host, out=None):
    """-> (meta int32 array, fwd_workspace_bytes, bwd_workspace_bytes); with
    `out`, the table is written into it (see _metadata)."""
    L = lib()
    cq = np.ascontiguousarray(cu_seqlens_q_host, dtype=np.int32)
    ck = np.ascontiguousarray(cu_seqlens_k_host, dtype=np.int32)
    words, fws, bws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    meta = _metadata("sink_attn_metadata", lambda m, cap: L.sink_attn_metadata(
        ctypes.byref(problem), _i32p(cq), _i32p(ck), m, cap, ctypes.byref(words),
        ctypes.byref(fws), ctypes.byref(bws)), words, out)
    return meta, fws.value, bws.value


def make_problem_padded(batch, seq_q, seq_k, seqused_q, seqused_kv, num_heads_q,
                        num_heads_k, head_dim, causal, win_left=-1, win_right=-1,
                        dtype=BF16, layout="BSND", layout_out=None):
    """Problem struct for a batch-padded layout ("BSND" or "BNSD"; out
    defaults to q's layout). seqused_q / seqused_kv: host int32 [batch] or
    None (all rows in use)."""
    lq = np.full(batch, seq_q) if seqused_q is None else np.asarray(seqused_q)
    lk = np.full(batch, seq_k) if seqused_kv is None else np.asarray(seqused_kv)
    lay = LAYOUTS[layout]
    lay_out = lay if layout_out is None else LAYOUTS[layout_out]
    return _problem(int(batch), num_heads_q, num_heads_k, head_dim,
                    int(batch) * int(seq_q), int(batch) * int(seq_k),
                    int(lq.max()) if len(lq) else 0, int(lk.max()) if len(lk) else 0,
                    int(bool(causal)), win_left, win_right, dtype,
                    lay, lay_out, int(seq_q), int(seq_k))


def sink_attn_metadata_padded(problem, seqused_q_host, seqused_kv_host, out=None):
    """-> (meta int32 array, fwd_workspace_bytes, bwd_workspace_bytes)."""
    L = lib()
    uq = None if seqused_q_host is None else np.ascontiguousarray(seqused_q_host, np.int32)
    uk = None if seqused_kv_host is None else np.ascontiguousarray(seqused_kv_host, np.int32)
    words, fws, bws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    meta = _metadata("sink_attn_metadata_padded", lambda m, cap: L.sink_attn_metadata_padded(
        ctypes.byref(problem), _i32p(uq), _i32p(uk), m, cap, ctypes.byref(words),
        ctypes.byref(fws), ctypes.byref(bws)), words, out)
    return meta, fws.value, bws.value


def make_problem_paged(cu_q, seqused_kv, num_heads_q, num_heads_k, head_dim, causal,
                       win_left=-1, win_right=-1, dtype=BF16):
    """Problem struct for a paged forward: key lengths from seqused_kv."""
    used = np.asarray(seqused_kv, dtype=np.int64)
    return make_problem(cu_q, np.concatenate([[0], np.cumsum(used)]), num_heads_q,
                        num_heads_k, head_dim, causal, win_left, win_right, dtype)


def sink_attn_metadata_paged(problem, kv, cu_seqlens_q_host, seqused_kv_host,
                             block_table_host, out=None):
    """-> (meta int32 array, fwd_workspace_bytes)."""
    L = lib()
    cq = np.ascontiguousarray(cu_seqlens_q_host, dtype=np.int32)
    su = np.ascontiguousarray(seqused_kv_host, dtype=np.int32)
    bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
    words, fws = ctypes.c_int64(), ctypes.c_int64()
    meta = _metadata("sink_attn_metadata_paged", lambda m, cap: L.sink_attn_metadata_paged(
        ctypes.byref(problem), ctypes.byref(kv), _i32p(cq), _i32p(su), _i32p(bt), m, cap,
        ctypes.byref(words), ctypes.byref(fws)), words, out)
    return meta, fws.value


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def sink_attn_fwd(problem, meta_host, meta_dev, q, k, v, cu_q, cu_k, sinks, scale,
                  out, lse, workspace=None, workspace_bytes=0, stream=None,
                  check=True):
    st = lib().sink_attn_fwd(ctypes.byref(problem), _i32p(meta_host), _ptr(meta_dev),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(cu_k),
                             _ptr(sinks), float(scale), _ptr(out), _ptr(lse),
                             _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and st != OK:
        raise SinkAttnError(st, "sink_attn_fwd")
    return st


def sink_attn_fwd_paged(problem, kv, meta_host, meta_dev, q, k_cache, v_cache, block_table,
                        cu_q, seqused_kv, sinks, scale, out, lse, workspace=None,
                        workspace_bytes=0, stream=None, check=True):
    st = lib().sink_attn_fwd_paged(ctypes.byref(problem), ctypes.byref(kv), _i32p(meta_host),
                                   _ptr(meta_dev), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_table), _ptr(cu_q), _ptr(seqused_kv),
                                   _ptr(sinks), float(scale), _ptr(out), _ptr(lse),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and st != OK:
        raise SinkAttnError(st, "sink_attn_fwd_paged")
    return st


def sink_attn_fwd_padded(problem, meta_host, meta_dev, q, k, v, seqused_q, seqused_kv,
                         sinks, scale, out, lse, workspace=None, workspace_bytes=0,
                         stream=None, check=True):
    st = lib().sink_attn_fwd_padded(ctypes.byref(problem), _i32p(meta_host), _ptr(meta_dev),
                                    _ptr(q), _ptr(k), _ptr(v), _ptr(seqused_q),
                                    _ptr(seqused_kv), _ptr(sinks), float(scale), _ptr(out),
                                    _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                    _stream(stream))
    if check and st != OK:
        raise SinkAttnError(st, "sink_attn_fwd_padded")
    return st


def sink_attn_bwd_padded(problem, meta_host, meta_dev, dout, q, k, v, out, lse, seqused_q,
                         seqused_kv, sinks, scale, dq, dk, dv, dsink, workspace=None,
                         workspace_bytes=0, stream=None, check=True):
    st = lib().sink_attn_bwd_padded(ctypes.byref(problem), _i32p(meta_host), _ptr(meta_dev),
                                    _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                    _ptr(lse), _ptr(seqused_q), _ptr(seqused_kv),
                                    _ptr(sinks), float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(dsink), _ptr(workspace), int(workspace_bytes),
                                    _stream(stream))
    if check and st != OK:
        raise SinkAttnError(st, "sink_attn_bwd_padded")
    return st


def sink_attn_merge(num_parts, total_q, num_heads_q, head_dim, part_dtype, out_dtype,
                    partial_out, partial_lse, sinks, out, lse, stream=None, check=True):
    st = lib().sink_attn_merge(int(num_parts), int(total_q), int(num_heads_q), int(head_dim),
                               int(part_dtype), int(out_dtype), _ptr(partial_out),
                               _ptr(partial_lse), _ptr(sinks), _ptr(out), _ptr(lse),
                               _stream(stream))
    if check and st != OK:
        raise SinkAttnError(st, "sink_attn_merge")
    return st


def merge(partial_out, partial_lse, sinks, out_dtype=None):
    """Merge sink-free partials: partial_out [P, Tq, Hq, D], partial_lse
    [P, Hq, Tq] fp32 -> out [Tq, Hq, D] (out_dtype, default the partials'),
    lse [Hq, Tq] (sink inclusive)."""
    import torch
    P, Tq, Hq, D = partial_out.shape
    _expect(partial_lse.contiguous(), "partial_lse", (P, Hq, Tq), torch.float32)
    _expect_sinks(sinks, Hq)
    out_dtype = out_dtype or partial_out.dtype
    out = torch.empty(Tq, Hq, D, dtype=out_dtype, device=partial_out.device)
    lse = torch.empty(Hq, Tq, dtype=torch.float32, device=partial_out.device)
    sink_attn_merge(P, Tq, Hq, D, dtype_code(partial_out.dtype), dtype_code(out_dtype),
                    partial_out.contiguous(), partial_lse.contiguous(), sinks, out, lse)
    return out, lse


def sink_attn_bwd(problem, meta_host, meta_dev, dout, q, k, v, out, lse, cu_q, cu_k,
                  sinks, scale, dq, dk, dv, dsink, workspace=None, workspace_bytes=0,
                  stream=None, check=True):
    st = lib().sink_attn_bwd(ctypes.byref(problem), _i32p(meta_host), _ptr(meta_dev),
                             _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                             _ptr(cu_q), _ptr(cu_k), _ptr(sinks), float(scale),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), _ptr(workspace),
                             int(workspace_bytes), _stream(stream))
    if check and st != OK:
        raise SinkAttnError(st, "sink_attn_bwd")
    return st


def sink_attn_bwd_noalloc(problem, meta_host, meta_dev, dout, q, k, v, out, lse, cu_q, cu_k,
                          sinks, scale, dq, dk, dv, dsink, stream=None, check=True):
    """sink_attn_bwd without a workspace: the library's static device
    scratch array (SINK_ATTN_NOALLOC_SCRATCH_BYTES per GPU) holds it."""
    st = lib().sink_attn_bwd_noalloc(ctypes.byref(problem), _i32p(meta_host), _ptr(meta_dev),
                                     _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                     _ptr(lse), _ptr(cu_q), _ptr(cu_k), _ptr(sinks),
                                     float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink),
                                     _stream(stream))
    if check and st != OK:
        raise SinkAttnError(st, "sink_attn_bwd_noalloc")
    return st


NOALLOC_SCRATCH_BYTES = 64 << 20


META_FWD_WORDS = 47     # header word: length of the table prefix the forward reads


def forward_table_words(meta):
    """Words at the start of a metadata table that the forward calls read
    (a forward-only caller may copy just these to the device)."""
    return int(meta[META_FWD_WORDS])


def sink_attn_upload_table(host, dev, words=None, stream=None):
    """Copy an int32 table from a pinned host tensor to a device tensor with
    a kernel on the stream (see include/sink_attn.h)."""
    import torch
    if host.device.type != "cpu" or not host.is_pinned() or host.dtype != torch.int32:
        raise ValueError("host must be a pinned int32 CPU tensor")
    if not host.is_contiguous():
        raise ValueError("host must be contiguous")
    n = host.numel() if words is None else int(words)
    _expect(dev, "dev", tuple(dev.shape), torch.int32)
    if n > min(host.numel(), dev.numel()):
        raise ValueError(f"{n} words do not fit host ({host.numel()}) or dev ({dev.numel()})")
    st = lib().sink_attn_upload_table(host.data_ptr(), _ptr(dev), n, _stream(stream))
    if st != OK:
        raise SinkAttnError(st, "sink_attn_upload_table")


def sink_attn_arm_timing(start, stop):
    """start/stop: torch.cuda.Event (recorded by the next fwd/bwd call
    around its main kernel) or None to disarm."""
    def h(e):
        if e is None:
            return None
        e.record()       # torch creates the event on first record; the
        return e.cuda_event  # library records it again around its kernel
    st = lib().sink_attn_arm_timing(h(start), h(stop))
    if st != OK:
        raise SinkAttnError(st, "sink_attn_arm_timing")


def _upload(arr, device):
    """Host array -> device tensor without stalling the host: the bytes are
    staged in pinned memory and copied on the current stream (a plain copy
    from pageable memory would first wait for all the work queued on it).
    torch's pinned-memory cache keeps the staging block until the copy ran."""
    import torch
    host = torch.from_numpy(np.ascontiguousarray(arr))
    if torch.device(device).type != "cuda":
        return host.to(device)
    return host.pin_memory().to(device, non_blocking=True)


# ---------------------------------------------------------------------------
# Conveniences over the C entry points (allocation with torch only).
# ---------------------------------------------------------------------------
class Plan:
    """Metadata for one packed batch: build once, use for fwd and bwd."""

    def __init__(self, cu_seqlens_q, cu_seqlens_k, num_heads_q, num_heads_k,
                 head_dim, causal, window=(-1, -1), dtype="bf16", device="cuda"):
        import torch
        self.cu_q_host = np.asarray(cu_seqlens_q, dtype=np.int32)
        self.cu_k_host = np.asarray(cu_seqlens_k, dtype=np.int32)
        self.dtype_code = dtype_code(dtype)
        self.problem = make_problem(self.cu_q_host, self.cu_k_host, num_heads_q,
                                    num_heads_k, head_dim, causal, window[0],
                                    window[1], self.dtype_code)
        self.meta, self.fwd_ws_bytes, self.bwd_ws_bytes = sink_attn_metadata(
            self.problem, self.cu_q_host, self.cu_k_host)
        self.device = device
        self.meta_dev = _upload(self.meta, device)
        self.cu_q = _upload(self.cu_q_host, device)
        self.cu_k = _upload(self.cu_k_host, device)

    @property
    def mode(self):
        return int(self.meta[14])


class PagedPlan:
    """Metadata for a paged forward over one batch (host block table and
    key lengths); the device copies are made here."""

    def __init__(self, cu_seqlens_q, seqused_kv, block_table, block_size, num_blocks,
                 num_heads_q, num_heads_k, head_dim, causal, window=(-1, -1),
                 device="cuda", dtype="bf16", cache_layout="BBND"):
        import torch
        self.cu_q_host = np.asarray(cu_seqlens_q, dtype=np.int32)
        self.seqused_host = np.asarray(seqused_kv, dtype=np.int32)
        self.block_table_host = np.ascontiguousarray(block_table, dtype=np.int32)
        self.kv = PagedKV(int(block_size), int(self.block_table_host.shape[1]), int(num_blocks),
                          CACHE_LAYOUTS[cache_layout])
        self.problem = make_problem_paged(self.cu_q_host, self.seqused_host, num_heads_q,
                                          num_heads_k, head_dim, causal, window[0],
                                          window[1], dtype_code(dtype))
        self.meta, self.fwd_ws_bytes = sink_attn_metadata_paged(
            self.problem, self.kv, self.cu_q_host, self.seqused_host, self.block_table_host)
        self.meta_dev = _upload(self.meta, device)
        self.cu_q = _upload(self.cu_q_host, device)
        self.seqused = _upload(self.seqused_host, device)
        self.block_table = _upload(self.block_table_host, device)


class PaddedPlan:
    """Metadata for one batch in a padded layout ("BSND" or "BNSD"):
    seq_q / seq_k rows per sequence, of which seqused_q / seqused_kv (host
    int32 [batch], or None for all) are in use."""

    def __init__(self, batch, seq_q, seq_k, seqused_q, seqused_kv, num_heads_q,
                 num_heads_k, head_dim, causal, window=(-1, -1), dtype="bf16",
                 layout="BSND", layout_out=None, device="cuda"):
        import torch
        self.layout = layout
        self.layout_out = layout_out or layout
        self.used_q_host = None if seqused_q is None else np.asarray(seqused_q, np.int32)
        self.used_k_host = None if seqused_kv is None else np.asarray(seqused_kv, np.int32)
        self.problem = make_problem_padded(batch, seq_q, seq_k, self.used_q_host,
                                           self.used_k_host, num_heads_q, num_heads_k,
                                           head_dim, causal, window[0], window[1],
                                           dtype_code(dtype), layout, layout_out)
        self.meta, self.fwd_ws_bytes, self.bwd_ws_bytes = sink_attn_metadata_padded(
            self.problem, self.used_q_host, self.used_k_host)
        self.meta_dev = _upload(self.meta, device)
        self.used_q = (None if self.used_q_host is None
                       else _upload(self.used_q_host, device))
        self.used_k = (None if self.used_k_host is None
                       else _upload(self.used_k_host, device))

    def out_shape(self):
        p = self.problem
        if self.layout_out == "BNSD":
            return (p.batch, p.num_heads_q, p.seq_q, p.head_dim)
        return (p.batch, p.seq_q, p.num_heads_q, p.head_dim)


def _workspace(nbytes, device):
    import torch
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def forward(plan, q, k, v, sinks, scale):
    """-> out (q's dtype, THD), lse [Hq, Tq] fp32."""
    import torch
    _expect_packed(plan, q=q, k=k, v=v)
    _expect_sinks(sinks, plan.problem.num_heads_q)
    out = torch.empty_like(q)
    lse = torch.empty(plan.problem.num_heads_q, plan.problem.total_q,
                      dtype=torch.float32, device=q.device)
    ws = _workspace(plan.fwd_ws_bytes, q.device)
    sink_attn_fwd(plan.problem, plan.meta, plan.meta_dev, q, k, v, plan.cu_q, plan.cu_k,
                  sinks, scale, out, lse, ws, plan.fwd_ws_bytes)
    return out, lse


def forward_paged(plan, q, k_cache, v_cache, sinks, scale):
    """Paged forward -> out, lse (k_cache, v_cache: [num_blocks, block_size,
    Hk, D], or [num_blocks, Hk, block_size, D] for a BNBD plan)."""
    import torch
    p, kv = plan.problem, plan.kv
    _expect_packed(plan, q=q)
    cache = ((kv.num_blocks, p.num_heads_k, kv.block_size, p.head_dim) if kv.layout == PA_BNBD
             else (kv.num_blocks, kv.block_size, p.num_heads_k, p.head_dim))
    _expect(k_cache, "k_cache", cache, _torch_dtype(p.dtype))
    _expect(v_cache, "v_cache", cache, _torch_dtype(p.dtype))
    _expect_sinks(sinks, p.num_heads_q)
    out = torch.empty_like(q)
    lse = torch.empty(plan.problem.num_heads_q, plan.problem.total_q,
                      dtype=torch.float32, device=q.device)
    ws = _workspace(plan.fwd_ws_bytes, q.device)
    sink_attn_fwd_paged(plan.problem, plan.kv, plan.meta, plan.meta_dev, q, k_cache, v_cache,
                        plan.block_table, plan.cu_q, plan.seqused, sinks, scale, out, lse,
                        ws, plan.fwd_ws_bytes)
    return out, lse


def forward_padded(plan, q, k, v, sinks, scale, out=None, lse=None):
    """Padded-layout forward -> out (plan.layout_out), lse [B, Hq, S_q] fp32.
    Rows past the used lengths keep what `out` / `lse` held (fresh, they are
    uninitialised)."""
    import torch
    p = plan.problem
    _expect_padded(plan, q=q, k=k, v=v, out=out, lse=lse)
    _expect_sinks(sinks, p.num_heads_q)
    if out is None:
        out = torch.empty(plan.out_shape(), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(p.batch, p.num_heads_q, p.seq_q, dtype=torch.float32,
                          device=q.device)
    ws = _workspace(plan.fwd_ws_bytes, q.device)
    sink_attn_fwd_padded(p, plan.meta, plan.meta_dev, q, k, v, plan.used_q, plan.used_k,
                         sinks, scale, out, lse, ws, plan.fwd_ws_bytes)
    return out, lse


def backward_padded(plan, dout, q, k, v, out, lse, sinks, scale, dq=None, dk=None, dv=None):
    """Padded-layout backward -> dq, dk, dv, dsink (rows past the used
    lengths keep what dq / dk / dv held)."""
    import torch
    _expect_padded(plan, q=q, k=k, v=v, dout=dout, out=out, lse=lse)
    _expect_sinks(sinks, plan.problem.num_heads_q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _expect_padded(plan, q=dq, k=dk, v=dv)
    dsink = (torch.empty(plan.problem.num_heads_q, dtype=torch.float32, device=q.device)
             if sinks is not None else None)
    ws = _workspace(plan.bwd_ws_bytes, q.device)
    sink_attn_bwd_padded(plan.problem, plan.meta, plan.meta_dev, dout, q, k, v, out, lse,
                         plan.used_q, plan.used_k, sinks, scale, dq, dk, dv, dsink, ws,
                         plan.bwd_ws_bytes)
    return dq, dk, dv, dsink


def backward(plan, dout, q, k, v, out, lse, sinks, scale):
    """-> dq, dk, dv, dsink (dsink None without sinks)."""
    import torch
    _expect_packed(plan, q=q, k=k, v=v, dout=dout, out=out, lse=lse)
    _expect_sinks(sinks, plan.problem.num_heads_q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsink = (torch.empty(plan.problem.num_heads_q, dtype=torch.float32, device=q.device)
             if sinks is not None else None)
    ws = _workspace(plan.bwd_ws_bytes, q.device)
    sink_attn_bwd(plan.problem, plan.meta, plan.meta_dev, dout, q, k, v, out, lse,
                  plan.cu_q, plan.cu_k, sinks, scale, dq, dk, dv, dsink, ws,
                  plan.bwd_ws_bytes)
    return dq, dk, dv, dsink


def _host_i32(x):
    """cu_seqlens as a host int32 array (a tensor on the GPU is copied back)."""
    if hasattr(x, "cpu"):
        x = x.cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.int32)


def _autograd_function():
    import torch

    class SinkAttnFunction(torch.autograd.Function):
        """Autograd wrapper with the argument order of the "slime" wrapper
        (q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
        softmax_offset, softmax_scale, causal, window_size)."""

        @staticmethod
        def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, softmax_offset, softmax_scale, causal, window_size):
            plan = Plan(_host_i32(cu_seqlens_q), _host_i32(cu_seqlens_k),
                        q.shape[1], k.shape[1], q.shape[2], causal, window_size,
                        q.dtype, q.device)
            if plan.problem.max_seqlen_q != max_seqlen_q or plan.problem.max_seqlen_k != max_seqlen_k:
                raise SinkAttnError(E_INVALID, "max_seqlen does not match cu_seqlens")
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            sinks = softmax_offset.float().contiguous() if softmax_offset is not None else None
            out, lse = forward(plan, q, k, v, sinks, softmax_scale)
            ctx.save_for_backward(q, k, v, out, lse, sinks)
            ctx.plan, ctx.scale = plan, softmax_scale
            ctx.has_sink = softmax_offset is not None
            ctx.offset_dtype = softmax_offset.dtype if softmax_offset is not None else None
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse, sinks = ctx.saved_tensors
            dq, dk, dv, dsink = backward(ctx.plan, dout.contiguous(), q, k, v, out, lse,
                                         sinks if ctx.has_sink else None, ctx.scale)
            if dsink is not None:
                dsink = dsink.to(ctx.offset_dtype)
            return dq, dk, dv, None, None, None, None, dsink, None, None, None

    return SinkAttnFunction


_SAF = None


def learnable_sink_attn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                               max_seqlen_k, softmax_offset, softmax_scale=None,
                               causal=False, window_size=(-1, -1)):
    """Packed (THD) attention with a learnable per-head sink logit; default
    scale 1/sqrt(head_dim) as in the "slime" wrapper. The tile schedule is
    built on the host from cu_seqlens: pass them as host (CPU) tensors or
    arrays, as a data loader has them, to spare a device-to-host copy (which
    waits for the queued work) on every call."""
    global _SAF
    if _SAF is None:
        _SAF = _autograd_function()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    return _SAF.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                      softmax_offset, softmax_scale, causal, tuple(window_size))


def _padded_autograd_function():
    import torch

    class SinkAttnPaddedFunction(torch.autograd.Function):
        """Autograd wrapper over the batch-padded (BSND / BNSD) calls. Rows
        past the used lengths come out as zeros in out, dq, dk and dv."""

        @staticmethod
        def forward(ctx, q, k, v, softmax_offset, softmax_scale, causal, window_size, layout,
                    layout_out, seqused_q, seqused_kv):
            bsnd = layout == "BSND"
            batch, seq_q = q.shape[0], q.shape[1] if bsnd else q.shape[2]
            seq_k = k.shape[1] if bsnd else k.shape[2]
            hq, hk = (q.shape[2], k.shape[2]) if bsnd else (q.shape[1], k.shape[1])
            host = lambda t: None if t is None else t.detach().to("cpu", torch.int32).numpy()
            plan = PaddedPlan(batch, seq_q, seq_k, host(seqused_q), host(seqused_kv), hq, hk,
                              q.shape[3], causal, window_size, q.dtype, layout, layout_out,
                              q.device)
            padded = seqused_q is not None or seqused_kv is not None
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            sinks = softmax_offset.float().contiguous() if softmax_offset is not None else None
            out = (torch.zeros if padded else torch.empty)(plan.out_shape(), dtype=q.dtype,
                                                           device=q.device)
            lse = torch.zeros(batch, hq, seq_q, dtype=torch.float32, device=q.device)
            forward_padded(plan, q, k, v, sinks, softmax_scale, out, lse)
            ctx.save_for_backward(q, k, v, out, lse, sinks)
            ctx.plan, ctx.scale, ctx.padded = plan, softmax_scale, padded
            ctx.has_sink = softmax_offset is not None
            ctx.offset_dtype = softmax_offset.dtype if softmax_offset is not None else None
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse, sinks = ctx.saved_tensors
            alloc = torch.zeros_like if ctx.padded else torch.empty_like
            dq, dk, dv, dsink = backward_padded(ctx.plan, dout.contiguous(), q, k, v, out, lse,
                                                sinks if ctx.has_sink else None, ctx.scale,
                                                alloc(q), alloc(k), alloc(v))
            if dsink is not None:
                dsink = dsink.to(ctx.offset_dtype)
            return dq, dk, dv, dsink, None, None, None, None, None, None, None

    return SinkAttnPaddedFunction


_SAPF = None


def learnable_sink_attn_padded(q, k, v, softmax_offset, softmax_scale=None, causal=False,
                               window_size=(-1, -1), layout="BSND", layout_out=None,
                               seqused_q=None, seqused_kv=None):
    """Batch-padded sink attention with autograd: q [B, S_q, Hq, D] and k, v
    [B, S_k, Hk, D] for "BSND", [B, H, S, D] for "BNSD" (out may be BSND for
    BNSD q); seqused_q / seqused_kv: int32 [B] rows in use (None: all)."""
    global _SAPF
    if _SAPF is None:
        _SAPF = _padded_autograd_function()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    return _SAPF.apply(q, k, v, softmax_offset, softmax_scale, causal, tuple(window_size),
                       layout, layout_out, seqused_q, seqused_kv)


def softmax_n_attn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                          max_seqlen_k, n, softmax_scale=None, causal=False,
                          window_size=(-1, -1)):
    """softmax_n attention ("Flash-Attention-Softmax-N" README): the sink logit
    is ln n for every head (n = 0: no sink)."""
    import torch
    if n < 0:
        raise ValueError("softmax_n needs n >= 0")
    sinks = None if n == 0 else torch.full((q.shape[1],), math.log(n),
                                          dtype=torch.float32, device=q.device)
    return learnable_sink_attn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                      max_seqlen_k, sinks, softmax_scale, causal,
                                      window_size)
