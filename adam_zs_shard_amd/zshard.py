"""Thin ctypes binding of libzshard (include/zshard.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libzshard.so.  There is no CPU fallback; if the library is not
built, every call raises.  Tensors are used for their device addresses;
plain integers are accepted as addresses too.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzshard.so")

ZS_OK, ZS_ERR_NULL, ZS_ERR_ARG, ZS_ERR_DTYPE, ZS_ERR_RANGE, ZS_ERR_ALIAS, ZS_ERR_CAPACITY, \
    ZS_ERR_HIP, ZS_ERR_UNSUPPORTED, ZS_ERR_RESOURCE = range(10)
ZS_F16, ZS_BF16 = 1, 2
ZS_ADAM_STANDARD, ZS_ADAM_PAGE1_LITERAL, ZS_SGD, ZS_SGD_MOMENTUM = 0, 1, 2, 3
ZS_STATE_M, ZS_STATE_V = 1, 2
ZS_MAX_P = 1024
ZS_KERNARG_P = 256
ZS_STATIC_SCRATCH_BYTES = 8192
ZS_MAX_TABLE_STEPS = 1 << 24

FORMS = {"standard": ZS_ADAM_STANDARD, "page1_literal": ZS_ADAM_PAGE1_LITERAL, "sgd": ZS_SGD,
         "sgd_momentum": ZS_SGD_MOMENTUM}
# bytes per element of one step at p ranks, by form (gradients, state read and
# written, the 16-bit working copy)
BYTES_PER_ELEM = {ZS_ADAM_STANDARD: 26, ZS_ADAM_PAGE1_LITERAL: 26, ZS_SGD: 10,
                  ZS_SGD_MOMENTUM: 18}
DTYPE_NAMES = {"f16": ZS_F16, "bf16": ZS_BF16}


class ZsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = lib().zs_status_string(status).decode()
        extra = f" (hipError {lib().zs_last_hip_error()})" if status == ZS_ERR_HIP else ""
        super().__init__(f"{where}: {name}{extra}")


class zs_adam_hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("step", C.c_int64), ("form", C.c_int32),
                ("reserved", C.c_int32)]


class zs_shard_args(C.Structure):
    _fields_ = [("n", C.c_int64), ("p", C.c_int32), ("k", C.c_int32),
                ("grads", C.POINTER(C.c_void_p)), ("grad_dtype", C.c_int32),
                ("param_dtype", C.c_int32), ("grad_base", C.c_int64),
                ("w", C.c_void_p), ("m", C.c_void_p), ("v", C.c_void_p),
                ("param", C.c_void_p), ("param_base", C.c_int64),
                ("hp", C.POINTER(zs_adam_hparams)), ("stream", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t)]


class zs_piece(C.Structure):
    _fields_ = [("tensor", C.c_int32), ("reserved", C.c_int32), ("tensor_off", C.c_int64),
                ("shard_off", C.c_int64), ("len", C.c_int64)]


class zs_piece_ptrs(C.Structure):
    _fields_ = [("w", C.c_void_p), ("m", C.c_void_p), ("v", C.c_void_p),
                ("param", C.c_void_p), ("grads", C.POINTER(C.c_void_p))]


class zs_mt_table(C.Structure):
    _fields_ = [("workspace", C.c_void_p), ("nchunks", C.c_int64), ("chunk_elems", C.c_int64),
                ("npieces", C.c_int32), ("p", C.c_int32), ("grad_dtype", C.c_int32),
                ("param_dtype", C.c_int32), ("state", C.c_int32), ("reserved", C.c_int32)]


class zs_offload_args(C.Structure):
    _fields_ = [("n", C.c_int64), ("p", C.c_int32), ("k", C.c_int32),
                ("grads", C.POINTER(C.c_void_p)), ("grad_dtype", C.c_int32),
                ("param_dtype", C.c_int32), ("grad_base", C.c_int64), ("param", C.c_void_p),
                ("param_base", C.c_int64), ("g16_dev", C.c_void_p), ("partial", C.c_void_p),
                ("g16_host", C.c_void_p * 2), ("w", C.c_void_p), ("m", C.c_void_p),
                ("v", C.c_void_p), ("param_host", C.c_void_p), ("bucket_elems", C.c_int64),
                ("threads", C.c_int32), ("reserved", C.c_int32), ("compute_stream", C.c_void_p),
                ("d2h_stream", C.c_void_p), ("h2d_stream", C.c_void_p)]


ZS_OFFLOAD_PLAIN, ZS_OFFLOAD_RECEIVE, ZS_OFFLOAD_DELAYED = 0, 1, 2


class zs_step_table(C.Structure):
    _fields_ = [("dev", C.c_void_p), ("first_step", C.c_int64), ("nsteps", C.c_int32),
                ("p", C.c_int32), ("form", C.c_int32), ("reserved", C.c_int32)]


EXPORTS = [
    "zs_status_string", "zs_version", "zs_last_hip_error", "zs_plan_shards",
    "zs_shard_workspace_bytes", "zs_fused_shard_step", "zs_fused_shard_step_static",
    "zs_reduce_scatter_mean_local",
    "zs_reduce_scatter_mean_local16", "zs_adam_step", "zs_plan_chunks", "zs_mt_chunk_elems",
    "zs_plan_buckets", "zs_mt_workspace_bytes", "zs_mt_upload", "zs_fused_shard_step_multi",
    "zs_step_table_bytes", "zs_step_table_init", "zs_step_table_advance", "zs_step_table_status",
    "zs_fused_shard_step_multi_dev", "zs_cpu_adam_step", "zs_offload_step",
]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        i32, i64, vp = C.c_int32, C.c_int64, C.c_void_p
        L.zs_status_string.argtypes = [i32]
        L.zs_status_string.restype = C.c_char_p
        L.zs_version.argtypes = []
        L.zs_version.restype = i32
        L.zs_last_hip_error.argtypes = []
        L.zs_last_hip_error.restype = i32
        L.zs_plan_shards.argtypes = [i64, i32, C.POINTER(i64), C.POINTER(i64), C.POINTER(i64)]
        L.zs_plan_shards.restype = i32
        L.zs_shard_workspace_bytes.argtypes = [i32]
        L.zs_shard_workspace_bytes.restype = C.c_size_t
        L.zs_fused_shard_step.argtypes = [C.POINTER(zs_shard_args)]
        L.zs_fused_shard_step.restype = i32
        L.zs_fused_shard_step_static.argtypes = [C.POINTER(zs_shard_args)]
        L.zs_fused_shard_step_static.restype = i32
        L.zs_reduce_scatter_mean_local.argtypes = [C.POINTER(vp), i32, i64, i64, i32, i32, vp, vp]
        L.zs_reduce_scatter_mean_local.restype = i32
        L.zs_reduce_scatter_mean_local16.argtypes = [C.POINTER(vp), i32, i64, i64, i32, i32, vp,
                                                     i32, vp, vp]
        L.zs_reduce_scatter_mean_local16.restype = i32
        L.zs_adam_step.argtypes = [vp, vp, vp, vp, vp, i32, i64, C.POINTER(zs_adam_hparams), vp]
        L.zs_adam_step.restype = i32
        L.zs_plan_chunks.argtypes = [C.POINTER(i64), i32, i32, i32, i64, C.POINTER(zs_piece), i32,
                                     C.POINTER(i32), C.POINTER(i64)]
        L.zs_plan_chunks.restype = i32
        L.zs_mt_chunk_elems.argtypes = [i64, i32, i32]
        L.zs_mt_chunk_elems.restype = i64
        L.zs_plan_buckets.argtypes = [C.POINTER(zs_piece), i32, i64, C.POINTER(i32), C.POINTER(i32)]
        L.zs_plan_buckets.restype = i32
        L.zs_mt_workspace_bytes.argtypes = [i32, i64, i32]
        L.zs_mt_workspace_bytes.restype = C.c_size_t
        L.zs_mt_upload.argtypes = [C.POINTER(zs_piece), C.POINTER(zs_piece_ptrs), i32, i32, i32,
                                   i32, i64, vp, C.c_size_t, vp, C.POINTER(zs_mt_table)]
        L.zs_mt_upload.restype = i32
        L.zs_fused_shard_step_multi.argtypes = [C.POINTER(zs_mt_table),
                                                C.POINTER(zs_adam_hparams), vp]
        L.zs_fused_shard_step_multi.restype = i32
        L.zs_step_table_bytes.argtypes = [i32]
        L.zs_step_table_bytes.restype = C.c_size_t
        L.zs_step_table_init.argtypes = [C.POINTER(zs_adam_hparams), i32, i32, vp, C.c_size_t, vp,
                                         C.POINTER(zs_step_table)]
        L.zs_step_table_init.restype = i32
        L.zs_step_table_advance.argtypes = [C.POINTER(zs_step_table), vp]
        L.zs_step_table_advance.restype = i32
        L.zs_step_table_status.argtypes = [C.POINTER(zs_step_table), C.POINTER(i64),
                                           C.POINTER(i32), vp]
        L.zs_step_table_status.restype = i32
        L.zs_fused_shard_step_multi_dev.argtypes = [C.POINTER(zs_mt_table),
                                                    C.POINTER(zs_step_table), vp]
        L.zs_fused_shard_step_multi_dev.restype = i32
        L.zs_cpu_adam_step.argtypes = [vp, i32, vp, vp, vp, vp, i32, i64,
                                       C.POINTER(zs_adam_hparams), i32]
        L.zs_cpu_adam_step.restype = i32
        L.zs_offload_step.argtypes = [C.POINTER(zs_offload_args), C.POINTER(zs_adam_hparams),
                                      i32, i32]
        L.zs_offload_step.restype = i32
        _lib = L
    return _lib


# ----------------------------------------------------------------- marshalling

def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _dtype_of(x, given) -> int:
    if given is not None:
        return DTYPE_NAMES[given] if isinstance(given, str) else int(given)
    import torch

    if x.dtype == torch.float16:
        return ZS_F16
    if x.dtype == torch.bfloat16:
        return ZS_BF16
    raise ValueError(f"16-bit tensor expected, got {x.dtype}")


def _stream(stream):
    if stream is None:
        import torch

        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr_array(xs):
    arr = (C.c_void_p * len(xs))(*[_addr(x) for x in xs])
    return C.cast(arr, C.POINTER(C.c_void_p)), arr


def _check(st: int, where: str):
    if st != ZS_OK:
        raise ZsError(st, where)


def hparams(lr, beta1, beta2, eps, step, form="standard") -> zs_adam_hparams:
    f = FORMS[form] if isinstance(form, str) else int(form)
    return zs_adam_hparams(float(lr), float(beta1), float(beta2), float(eps), int(step), f, 0)


# ----------------------------------------------------------------- entry points

def zs_version() -> int:
    return lib().zs_version()


def zs_status_string(status: int) -> str:
    return lib().zs_status_string(status).decode()


def zs_last_hip_error() -> int:
    return lib().zs_last_hip_error()


def zs_plan_shards(n: int, p: int):
    """(M, starts, ends) for all p ranks."""
    m = C.c_int64()
    s = (C.c_int64 * max(p, 1))()
    e = (C.c_int64 * max(p, 1))()
    _check(lib().zs_plan_shards(n, p, C.byref(m), s, e), "zs_plan_shards")
    return m.value, list(s)[:p], list(e)[:p]


def zs_shard_workspace_bytes(p: int) -> int:
    return lib().zs_shard_workspace_bytes(p)


def zs_fused_shard_step(n, p, k, grads, w, m, v, param, hp: zs_adam_hparams, *,
                        grad_base=0, param_base=0, grad_dtype=None, param_dtype=None,
                        stream=None, workspace=None, workspace_bytes=None, static=False,
                        check=True) -> int:
    """workspace: device memory for the rank pointer table (needed when p >
    ZS_KERNARG_P); workspace_bytes defaults to the tensor's size in bytes.
    static=True calls zs_fused_shard_step_static (no workspace: the library's
    static device scratch)."""
    gptr, keep = _ptr_array(grads)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    a = zs_shard_args(
        n=n, p=p, k=k, grads=gptr if grads is not None else None,
        grad_dtype=_dtype_of(grads[0], grad_dtype) if grads else (grad_dtype or ZS_F16),
        param_dtype=_dtype_of(param, param_dtype) if param is not None else (param_dtype or 0),
        grad_base=grad_base, w=_addr(w), m=_addr(m), v=_addr(v), param=_addr(param),
        param_base=param_base, hp=C.pointer(hp), stream=_stream(stream),
        workspace=_addr(workspace), workspace_bytes=workspace_bytes)
    fn = lib().zs_fused_shard_step_static if static else lib().zs_fused_shard_step
    st = fn(C.byref(a))
    del keep
    if check:
        _check(st, "zs_fused_shard_step_static" if static else "zs_fused_shard_step")
    return st


def zs_reduce_scatter_mean_local(grads, n, p, k, g_out, *, grad_base=0, grad_dtype=None,
                                 stream=None, check=True) -> int:
    gptr, keep = _ptr_array(grads)
    st = lib().zs_reduce_scatter_mean_local(gptr, _dtype_of(grads[0], grad_dtype), grad_base,
                                            n, p, k, _addr(g_out), _stream(stream))
    del keep
    if check:
        _check(st, "zs_reduce_scatter_mean_local")
    return st


def zs_reduce_scatter_mean_local16(grads, n, p, k, g_out, out_dtype=None, *, grad_base=0,
                                   grad_dtype=None, partial=None, stream=None,
                                   check=True) -> int:
    """The rank mean rounded to 16 bits into g_out (out_dtype defaults to
    g_out's dtype); partial: fp32 device array of the shard length, needed
    when p > ZS_KERNARG_P."""
    gptr, keep = _ptr_array(grads)
    st = lib().zs_reduce_scatter_mean_local16(gptr, _dtype_of(grads[0], grad_dtype), grad_base,
                                              n, p, k, _addr(g_out),
                                              _dtype_of(g_out, out_dtype), _addr(partial),
                                              _stream(stream))
    del keep
    if check:
        _check(st, "zs_reduce_scatter_mean_local16")
    return st


def zs_adam_step(g, w, m, v, param, length: int, hp: zs_adam_hparams, *, param_dtype=None,
                 stream=None, check=True) -> int:
    pdt = _dtype_of(param, param_dtype) if param is not None else 0
    st = lib().zs_adam_step(_addr(g), _addr(w), _addr(m), _addr(v), _addr(param), pdt, length,
                            C.byref(hp), _stream(stream))
    if check:
        _check(st, "zs_adam_step")
    return st


def zs_plan_chunks(numel, p: int, k: int, chunk_elems: int):
    """([(tensor, tensor_off, shard_off, len), ...], nchunks)."""
    nm = (C.c_int64 * max(len(numel), 1))(*numel)
    npieces = C.c_int32()
    nchunks = C.c_int64()
    st = lib().zs_plan_chunks(nm, len(numel), p, k, chunk_elems, None, 0, C.byref(npieces),
                              C.byref(nchunks))
    if st not in (ZS_OK, ZS_ERR_CAPACITY):
        _check(st, "zs_plan_chunks")
    cap = npieces.value
    arr = (zs_piece * max(cap, 1))()
    _check(lib().zs_plan_chunks(nm, len(numel), p, k, chunk_elems, arr, cap, C.byref(npieces),
                                C.byref(nchunks)), "zs_plan_chunks")
    return [(x.tensor, x.tensor_off, x.shard_off, x.len) for x in arr[:npieces.value]], \
        nchunks.value


def zs_mt_chunk_elems(shard_len: int, npieces: int, cu_count: int = 0) -> int:
    return lib().zs_mt_chunk_elems(shard_len, npieces, cu_count)


def zs_plan_buckets(pieces, bucket_elems: int):
    """Bucket index of each piece (runs of consecutive pieces of at least
    bucket_elems elements) and the bucket count."""
    n = len(pieces)
    pa = (zs_piece * max(n, 1))(*[zs_piece(t, 0, to, so, ln) for (t, to, so, ln) in pieces])
    out = (C.c_int32 * max(n, 1))()
    nb = C.c_int32()
    _check(lib().zs_plan_buckets(pa, n, bucket_elems, out, C.byref(nb)), "zs_plan_buckets")
    return list(out)[:n], nb.value


def zs_mt_workspace_bytes(npieces: int, nchunks: int, p: int) -> int:
    return lib().zs_mt_workspace_bytes(npieces, nchunks, p)


def zs_mt_upload(pieces, ptrs, p: int, grad_dtype, param_dtype, chunk_elems: int, workspace,
                 ws_bytes: int, *, stream=None) -> zs_mt_table:
    """pieces: [(tensor, tensor_off, shard_off, len)]; ptrs: [dict(w, m, v, param, grads)]
    with device addresses (or tensors) at each piece's first element."""
    n = len(pieces)
    pa = (zs_piece * max(n, 1))(*[zs_piece(t, 0, to, so, ln) for (t, to, so, ln) in pieces])
    keep = []
    qa = (zs_piece_ptrs * max(n, 1))()
    for i, q in enumerate(ptrs):
        gp, g_keep = _ptr_array(q["grads"])
        keep.append(g_keep)
        qa[i] = zs_piece_ptrs(_addr(q["w"]), _addr(q["m"]), _addr(q["v"]), _addr(q["param"]), gp)
    gdt = DTYPE_NAMES[grad_dtype] if isinstance(grad_dtype, str) else int(grad_dtype)
    pdt = DTYPE_NAMES[param_dtype] if isinstance(param_dtype, str) else int(param_dtype)
    table = zs_mt_table()
    st = lib().zs_mt_upload(pa, qa, n, p, gdt, pdt, chunk_elems, _addr(workspace), ws_bytes,
                            _stream(stream), C.byref(table))
    del keep
    _check(st, "zs_mt_upload")
    return table


def zs_fused_shard_step_multi(table: zs_mt_table, hp: zs_adam_hparams, *, stream=None,
                              check=True) -> int:
    st = lib().zs_fused_shard_step_multi(C.byref(table), C.byref(hp), _stream(stream))
    if check:
        _check(st, "zs_fused_shard_step_multi")
    return st


def zs_step_table_bytes(nsteps: int) -> int:
    return lib().zs_step_table_bytes(nsteps)


def zs_step_table_init(hp: zs_adam_hparams, p: int, nsteps: int, dev, nbytes: int, *,
                       stream=None) -> zs_step_table:
    t = zs_step_table()
    _check(lib().zs_step_table_init(C.byref(hp), p, nsteps, _addr(dev), nbytes, _stream(stream),
                                    C.byref(t)), "zs_step_table_init")
    return t


def zs_step_table_advance(table: zs_step_table, *, stream=None, check=True) -> int:
    st = lib().zs_step_table_advance(C.byref(table), _stream(stream))
    if check:
        _check(st, "zs_step_table_advance")
    return st


def zs_step_table_status(table: zs_step_table, *, stream=None):
    """(cursor, exhausted) read back from the device."""
    cur = C.c_int64()
    ex = C.c_int32()
    _check(lib().zs_step_table_status(C.byref(table), C.byref(cur), C.byref(ex), _stream(stream)),
           "zs_step_table_status")
    return cur.value, ex.value


def zs_fused_shard_step_multi_dev(table: zs_mt_table, steps: zs_step_table, *, stream=None,
                                  check=True) -> int:
    st = lib().zs_fused_shard_step_multi_dev(C.byref(table), C.byref(steps), _stream(stream))
    if check:
        _check(st, "zs_fused_shard_step_multi_dev")
    return st


def _host_addr(x) -> int | None:
    """Address of a host numpy array or CPU tensor (or an int / None)."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    if x.is_cuda:
        raise ValueError("zs_cpu_adam_step takes host memory")
    return x.data_ptr()


def zs_cpu_adam_step(g, grad_dtype, w, m, v, param, param_dtype, length: int,
                     hp: zs_adam_hparams, *, threads: int = 0, check=True) -> int:
    """The update of one shard on the host CPU (optimizer offload); every
    buffer is host memory (numpy arrays or CPU tensors).  grad_dtype /
    param_dtype: "f16", "bf16" or the zs_dtype value."""
    gdt = DTYPE_NAMES[grad_dtype] if isinstance(grad_dtype, str) else int(grad_dtype)
    pdt = 0 if param is None else (DTYPE_NAMES[param_dtype] if isinstance(param_dtype, str)
                                   else int(param_dtype))
    st = lib().zs_cpu_adam_step(_host_addr(g), gdt, _host_addr(w), _host_addr(m), _host_addr(v),
                                _host_addr(param), pdt, length, C.byref(hp), threads)
    if check:
        _check(st, "zs_cpu_adam_step")
    return st


def zs_offload_step(n, p, k, grads, param, g16_dev, g16_host, w, m, v, param_host,
                    hp: zs_adam_hparams, mode: int, slot: int, *, grad_base=0, param_base=0,
                    grad_dtype=None, param_dtype=None, partial=None, bucket_elems=0, threads=0,
                    compute_stream=None, d2h_stream=None, h2d_stream=None, check=True) -> int:
    """One offloaded step (see zshard.h): device tensors grads, param,
    g16_dev, partial; pinned host tensors (or numpy arrays) g16_host (two),
    w, m, v, param_host; streams default to the current stream."""
    gptr, keep = _ptr_array(grads)
    a = zs_offload_args(
        n=n, p=p, k=k, grads=gptr, grad_dtype=_dtype_of(grads[0], grad_dtype),
        param_dtype=_dtype_of(param, param_dtype), grad_base=grad_base, param=_addr(param),
        param_base=param_base, g16_dev=_addr(g16_dev), partial=_addr(partial),
        g16_host=(C.c_void_p * 2)(_host_addr(g16_host[0]), _host_addr(g16_host[1])),
        w=_host_addr(w), m=_host_addr(m), v=_host_addr(v), param_host=_host_addr(param_host),
        bucket_elems=bucket_elems, threads=threads, reserved=0,
        compute_stream=_stream(compute_stream), d2h_stream=_stream(d2h_stream),
        h2d_stream=_stream(h2d_stream))
    st = lib().zs_offload_step(C.byref(a), C.byref(hp), mode, slot)
    del keep
    if check:
        _check(st, "zs_offload_step")
    return st
