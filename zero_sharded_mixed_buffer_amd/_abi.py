"""ctypes binding of libzs.so (include/zs.h), one Python function per C entry point.

Argument marshalling only: every computation runs in the HIP library.  Pointer
arguments accept an int (a device or host address), None (NULL) or anything
with .data_ptr() (a torch tensor); a tensor in the wrong memory (a host tensor
where the library wants device memory, or the reverse) is refused before the
call, since it would be dereferenced on the wrong side.  `stream` accepts a
torch stream, an int handle or None (the current torch stream of the current
device).  A non-zero
status raises ZsError carrying zs_last_error().  If the library is not built
the first call raises ImportError; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_double, c_int32, c_int64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzs.so")

ZS_BF16, ZS_FP16, ZS_FP32 = 0, 1, 2
STATUS = {0: "ZS_OK", -1: "ZS_EINVAL", -2: "ZS_EHIP", -3: "ZS_ENOMEM", -4: "ZS_EUNSUPPORTED"}


class ZsError(RuntimeError):
    """A non-OK status from the library; `status` holds the zs_status code."""

    def __init__(self, what, status, message):
        super().__init__(f"{what} failed with {STATUS.get(status, status)}: {message}")
        self.status = status


class ZsInvalidArgument(ZsError, ValueError):
    """ZS_EINVAL: an argument was rejected before anything ran (also a ValueError, the
    convention for bad input in Python)."""


class AdamwHParams(ctypes.Structure):
    _fields_ = [("lr", c_double), ("beta1", c_double), ("beta2", c_double), ("eps", c_double),
                ("weight_decay", c_double), ("max_norm", c_double)]


class StateHost(ctypes.Structure):
    _fields_ = [("loss_scale", c_double), ("scale_floor", c_double), ("dynamic", c_int32),
                ("growth_interval", c_int32), ("growth_tracker", c_int64), ("step_t", c_int64),
                ("skipped_total", c_int64), ("overflow", c_int32), ("reserved", c_int32),
                ("local_sumsq", c_double), ("sumsq", c_double), ("grad_norm", c_double),
                ("clip_coef", c_double)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


_lib = None

_SIGS = {
    "zs_plan": [c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p, c_void_p, c_void_p, c_void_p],
    "zs_plan_segments": [c_void_p, c_int32, c_int32, c_int32, c_int64, c_int32, c_void_p, c_void_p, c_void_p,
                         c_int64, c_void_p],
    "zs_layout_create": [c_void_p, c_int32, c_int32, c_int32, c_int64, POINTER(c_void_p)],
    "zs_layout_info": [c_void_p, c_void_p, c_void_p, c_void_p],
    "zs_state_create": [c_void_p, POINTER(StateHost), POINTER(c_void_p)],
    "zs_state_read": [c_void_p, POINTER(StateHost), c_void_p],
    "zs_state_write": [c_void_p, POINTER(StateHost), c_void_p],
    "zs_pack": [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p],
    "zs_pack_accumulate": [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p],
    "zs_plan_buckets": [c_void_p, c_int32, c_int64, c_void_p, c_void_p],
    "zs_layout_set_no_decay": [c_void_p, c_void_p, c_int32, c_void_p],
    "zs_bucket_range": [c_void_p, c_int32, c_int32, c_void_p, c_void_p],
    "zs_pack_bucket": [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p],
    "zs_unscale_check": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p],
    "zs_grad_norm": [c_void_p, c_void_p, c_int32, c_void_p, POINTER(AdamwHParams), c_void_p, c_void_p, c_void_p],
    "zs_adamw_step": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, POINTER(AdamwHParams), c_void_p,
                      c_void_p, c_void_p, c_int32, c_void_p],
    "zs_unpack": [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_void_p],
    "zs_scaler_update": [c_void_p, c_void_p],
    "zs_step": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, POINTER(AdamwHParams), c_void_p, c_void_p,
                c_void_p, c_void_p, c_int32, c_void_p],
    "zs_step_flat": [c_void_p, c_void_p, c_int32, c_void_p, POINTER(AdamwHParams), c_void_p, c_void_p, c_void_p,
                     c_void_p, c_int32, c_void_p],
    "zs_step_flat_noalloc": [c_void_p, c_int32, c_int64, c_void_p, POINTER(AdamwHParams), c_void_p, c_void_p,
                             c_void_p, c_void_p, c_int32, c_void_p],
    "zs_host_adamw_step": [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int64, POINTER(AdamwHParams),
                           POINTER(StateHost), c_void_p, c_int32, c_int32],
    "zs_probe_mix": [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p],
    "zs_probe_copy": [c_void_p, c_void_p, c_int64, c_void_p],
    "zs_probe_read": [c_void_p, c_int64, c_void_p, c_void_p],
    "zs_probe_write": [c_void_p, c_int64, c_void_p],
    "zs_offload_adamw_step": [c_void_p, c_void_p, c_int32, c_void_p, POINTER(AdamwHParams), c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int32, c_int32, c_void_p],
}


def lib():
    """Load libzs.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m zero_sharded_mixed_buffer_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = c_int32
        L.zs_layout_destroy.argtypes = [c_void_p]
        L.zs_layout_destroy.restype = None
        L.zs_state_destroy.argtypes = [c_void_p]
        L.zs_state_destroy.restype = None
        L.zs_last_error.argtypes = []
        L.zs_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status, what):
    if status != 0:
        cls = ZsInvalidArgument if status == -1 else ZsError  # ZS_EINVAL
        raise cls(what, status, lib().zs_last_error().decode(errors="replace"))


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, ctypes.Array):
        return ctypes.addressof(x)
    return int(x)


def _dptr(x, what, where):
    """A device-memory argument: a host tensor here would be dereferenced by a kernel and
    fault the GPU, so it is refused before the call (raw integers pass unchecked)."""
    if x is not None and hasattr(x, "data_ptr") and not x.is_cuda:
        raise ZsInvalidArgument(where, -1, f"{what} must be device memory, got a host tensor")
    return _ptr(x)


def _hptr(x, what, where):
    """A host-memory argument: a device tensor here would be dereferenced by the host."""
    if x is not None and hasattr(x, "data_ptr") and x.is_cuda:
        raise ZsInvalidArgument(where, -1, f"{what} must be host memory, got a device tensor")
    return _ptr(x)


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _i64_array(values):
    return (c_int64 * len(values))(*[int(v) for v in values])


def dtype_code(dtype):
    """ZS_* code of a torch dtype (bfloat16, float16, float32) or of an int code."""
    if isinstance(dtype, int):
        return dtype
    import torch
    return {torch.bfloat16: ZS_BF16, torch.float16: ZS_FP16, torch.float32: ZS_FP32}[dtype]


# ------------------------------------------------------------------------------ planning

def zs_plan(numels, dp_world, dp_rank, align_elems=1):
    """Returns (offsets, flat_numel, shard_begin, shard_numel)."""
    n = len(numels)
    arr = _i64_array(numels)
    offs = (c_int64 * max(n, 1))()
    fn, sb, sn = c_int64(), c_int64(), c_int64()
    _check(lib().zs_plan(ctypes.addressof(arr) if n else None, n, dp_world, dp_rank, align_elems,
                         ctypes.addressof(offs), byref(fn), byref(sb), byref(sn)), "zs_plan")
    return list(offs)[:n], fn.value, sb.value, sn.value


def zs_plan_segments(numels, dp_world, dp_rank, align_elems=1, whole_flat=False):
    """Returns (seg_begin, seg_tensor, seg_local) lists of the kernels' segment map."""
    n = len(numels)
    arr = _i64_array(numels)
    count = c_int64()
    _check(lib().zs_plan_segments(ctypes.addressof(arr), n, dp_world, dp_rank, align_elems, int(bool(whole_flat)),
                                  None, None, None, 0, byref(count)), "zs_plan_segments")
    k = count.value
    b, t, loc = (c_int64 * max(k, 1))(), (c_int32 * max(k, 1))(), (c_int64 * max(k, 1))()
    _check(lib().zs_plan_segments(ctypes.addressof(arr), n, dp_world, dp_rank, align_elems, int(bool(whole_flat)),
                                  ctypes.addressof(b), ctypes.addressof(t), ctypes.addressof(loc), k, byref(count)),
           "zs_plan_segments")
    return list(b)[:k], list(t)[:k], list(loc)[:k]


# ------------------------------------------------------------------------------ handles

def zs_layout_create(numels, dp_world, dp_rank, align_elems=1):
    arr = _i64_array(numels)
    out = c_void_p()
    _check(lib().zs_layout_create(ctypes.addressof(arr) if len(numels) else None, len(numels), dp_world, dp_rank,
                                  align_elems, byref(out)), "zs_layout_create")
    return out.value


def zs_layout_destroy(layout):
    lib().zs_layout_destroy(layout)


def zs_plan_buckets(numels, bucket_numel):
    """Returns the [tensor_begin, tensor_end) pairs of the buckets, in closing order."""
    n = len(numels)
    arr = _i64_array(numels)
    bounds = (c_int32 * max(2 * n, 1))()
    nb = c_int32()
    _check(lib().zs_plan_buckets(ctypes.addressof(arr) if n else None, n, bucket_numel, ctypes.addressof(bounds),
                                 byref(nb)), "zs_plan_buckets")
    return [(bounds[2 * i], bounds[2 * i + 1]) for i in range(nb.value)]


def zs_bucket_range(layout, tensor_begin, tensor_end):
    """Returns the flat range (begin, end) of the bucket of tensors [tensor_begin, tensor_end)."""
    b, e = c_int64(), c_int64()
    _check(lib().zs_bucket_range(layout, tensor_begin, tensor_end, byref(b), byref(e)), "zs_bucket_range")
    return b.value, e.value


def zs_layout_set_no_decay(layout, no_decay, stream=None):
    """Per-tensor no-decay flags (a sequence of bools, one per tensor), or None to clear; the
    table is uploaded on `stream` and applies to the steps enqueued after it there."""
    if no_decay is None:
        _check(lib().zs_layout_set_no_decay(layout, None, 0, _stream(stream)), "zs_layout_set_no_decay")
        return
    flags = (ctypes.c_uint8 * max(len(no_decay), 1))(*[1 if f else 0 for f in no_decay])
    _check(lib().zs_layout_set_no_decay(layout, ctypes.addressof(flags), len(no_decay), _stream(stream)),
           "zs_layout_set_no_decay")


def zs_layout_info(layout):
    """Returns (flat_numel, shard_begin, shard_numel)."""
    a, b, c = c_int64(), c_int64(), c_int64()
    _check(lib().zs_layout_info(layout, byref(a), byref(b), byref(c)), "zs_layout_info")
    return a.value, b.value, c.value


def state_host(loss_scale=1.0, scale_floor=1.0, dynamic=False, growth_interval=1000, growth_tracker=0, step_t=0,
               skipped_total=0, clip_coef=1.0):
    s = StateHost()
    s.loss_scale, s.scale_floor, s.dynamic = loss_scale, scale_floor, int(bool(dynamic))
    s.growth_interval, s.growth_tracker, s.step_t, s.skipped_total = growth_interval, growth_tracker, step_t, skipped_total
    s.clip_coef = clip_coef
    return s


def zs_state_create(layout, init: StateHost):
    out = c_void_p()
    _check(lib().zs_state_create(layout, byref(init), byref(out)), "zs_state_create")
    return out.value


def zs_state_destroy(state):
    lib().zs_state_destroy(state)


def zs_state_read(state, stream=None) -> StateHost:
    out = StateHost()
    _check(lib().zs_state_read(state, byref(out), _stream(stream)), "zs_state_read")
    return out


def zs_state_write(state, value: StateHost, stream=None):
    _check(lib().zs_state_write(state, byref(value), _stream(stream)), "zs_state_write")


def hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0):
    return AdamwHParams(lr, beta1, beta2, eps, weight_decay, max_norm)


# ------------------------------------------------------------------------------ step calls

def zs_pack(layout, src_ptrs, src_dtype, dst, dst_dtype, whole_flat=True, fuse_check=None, stream=None):
    W = "zs_pack"
    _check(lib().zs_pack(layout, _dptr(src_ptrs, "src_ptrs", W), dtype_code(src_dtype), _dptr(dst, "dst", W),
                         dtype_code(dst_dtype), int(bool(whole_flat)), fuse_check, _stream(stream)), W)


def zs_pack_accumulate(layout, src_ptrs, src_dtype, acc, acc_dtype, whole_flat=True, fuse_check=None, stream=None):
    W = "zs_pack_accumulate"
    _check(lib().zs_pack_accumulate(layout, _dptr(src_ptrs, "src_ptrs", W), dtype_code(src_dtype),
                                    _dptr(acc, "acc", W), dtype_code(acc_dtype), int(bool(whole_flat)), fuse_check,
                                    _stream(stream)), W)


def zs_pack_bucket(layout, src_ptrs, src_dtype, flat, flat_dtype, tensor_begin, tensor_end, accumulate=False,
                   stream=None):
    W = "zs_pack_bucket"
    _check(lib().zs_pack_bucket(layout, _dptr(src_ptrs, "src_ptrs", W), dtype_code(src_dtype), _dptr(flat, "flat", W),
                                dtype_code(flat_dtype), tensor_begin, tensor_end, int(bool(accumulate)),
                                _stream(stream)), W)


def zs_unscale_check(layout, shard, grad_dtype, state, ext_overflow=None, local_sumsq_out=None, stream=None):
    W = "zs_unscale_check"
    _check(lib().zs_unscale_check(layout, _dptr(shard, "shard", W), dtype_code(grad_dtype), state,
                                  _dptr(ext_overflow, "ext_overflow", W),
                                  _dptr(local_sumsq_out, "local_sumsq_out", W), _stream(stream)), W)


def zs_grad_norm(layout, shard, grad_dtype, state, hp: AdamwHParams, rank_sumsq=None, local_sumsq_out=None,
                 stream=None):
    W = "zs_grad_norm"
    _check(lib().zs_grad_norm(layout, _dptr(shard, "shard", W), dtype_code(grad_dtype), state, byref(hp),
                              _dptr(rank_sumsq, "rank_sumsq", W), _dptr(local_sumsq_out, "local_sumsq_out", W),
                              _stream(stream)), W)


def zs_adamw_step(layout, shard, grad_dtype, master, m, v, hp: AdamwHParams, state, param_ptrs=None,
                  flat_param_out=None, param_dtype=ZS_BF16, stream=None):
    W = "zs_adamw_step"
    _check(lib().zs_adamw_step(layout, _dptr(shard, "shard", W), dtype_code(grad_dtype), _dptr(master, "master", W),
                               _dptr(m, "m", W), _dptr(v, "v", W), byref(hp), state,
                               _dptr(param_ptrs, "param_ptrs", W), _dptr(flat_param_out, "flat_param_out", W),
                               dtype_code(param_dtype), _stream(stream)), W)


def zs_unpack(layout, src, src_dtype, whole_flat, dst_ptrs, dst_dtype, honour_skip=None, stream=None):
    W = "zs_unpack"
    _check(lib().zs_unpack(layout, _dptr(src, "src", W), dtype_code(src_dtype), int(bool(whole_flat)),
                           _dptr(dst_ptrs, "dst_ptrs", W), dtype_code(dst_dtype), honour_skip, _stream(stream)), W)


def zs_scaler_update(state, stream=None):
    _check(lib().zs_scaler_update(state, _stream(stream)), "zs_scaler_update")


def zs_step(layout, grad_ptrs, grad_dtype, flat, state, hp: AdamwHParams, master, m, v, param_ptrs,
            param_dtype=ZS_BF16, stream=None):
    """The whole single-rank step: pack, check, norm, AdamW with scatter, scaler commit."""
    W = "zs_step"
    _check(lib().zs_step(layout, _dptr(grad_ptrs, "grad_ptrs", W), dtype_code(grad_dtype), _dptr(flat, "flat", W),
                         state, byref(hp), _dptr(master, "master", W), _dptr(m, "m", W), _dptr(v, "v", W),
                         _dptr(param_ptrs, "param_ptrs", W), dtype_code(param_dtype), _stream(stream)), W)


def zs_step_flat(layout, flat, grad_dtype, state, hp: AdamwHParams, master, m, v, flat_param_out,
                 param_dtype=ZS_BF16, stream=None):
    """The single-rank step over contiguous gradient and parameter buffers: check, norm,
    AdamW writing the parameter buffer, scaler commit."""
    W = "zs_step_flat"
    _check(lib().zs_step_flat(layout, _dptr(flat, "flat", W), dtype_code(grad_dtype), state, byref(hp),
                              _dptr(master, "master", W), _dptr(m, "m", W), _dptr(v, "v", W),
                              _dptr(flat_param_out, "flat_param_out", W), dtype_code(param_dtype),
                              _stream(stream)), W)


def zs_step_flat_noalloc(flat, grad_dtype, n, state, hp: AdamwHParams, master, m, v, flat_param_out,
                         param_dtype=ZS_BF16, stream=None):
    """zs_step_flat with no layout, no zs_state and no allocation: `state` is device memory
    holding a zs_state_host (e.g. a uint8 tensor of ctypes.sizeof(StateHost) bytes), and the
    library's fixed per-GPU scratch replaces the state's workspace."""
    W = "zs_step_flat_noalloc"
    _check(lib().zs_step_flat_noalloc(_dptr(flat, "flat", W), dtype_code(grad_dtype), int(n),
                                      _dptr(state, "state", W), byref(hp), _dptr(master, "master", W),
                                      _dptr(m, "m", W), _dptr(v, "v", W), _dptr(flat_param_out, "flat_param_out", W),
                                      dtype_code(param_dtype), _stream(stream)), W)


def zs_last_error():
    return lib().zs_last_error().decode(errors="replace")


# ------------------------------------------------------------------------------ offloaded step

def zs_host_adamw_step(grad, grad_dtype, master, m, v, count, hp: AdamwHParams, scalars: StateHost,
                       param_out=None, param_dtype=None, n_threads=0):
    """Host AdamW over `count` elements of host arrays (see zs.h)."""
    pdt = dtype_code(param_dtype) if param_dtype is not None else ZS_BF16
    W = "zs_host_adamw_step"
    _check(lib().zs_host_adamw_step(_hptr(grad, "grad", W), dtype_code(grad_dtype), _hptr(master, "master", W),
                                    _hptr(m, "m", W), _hptr(v, "v", W), int(count), byref(hp), byref(scalars),
                                    _hptr(param_out, "param_out", W), pdt, int(n_threads)),
           "zs_host_adamw_step")


def zs_offload_adamw_step(layout, shard, grad_dtype, state, hp: AdamwHParams, master, m, v, grad_stage, param_stage,
                          chunk_numel, flat_param_out, param_dtype, n_threads=0, stream=None):
    """Offloaded update of the rank's shard: chunks down, host update, parameters up (see zs.h)."""
    W = "zs_offload_adamw_step"
    _check(lib().zs_offload_adamw_step(layout, _dptr(shard, "shard", W), dtype_code(grad_dtype), state, byref(hp),
                                       _hptr(master, "master", W), _hptr(m, "m", W), _hptr(v, "v", W),
                                       _hptr(grad_stage, "grad_stage", W), _hptr(param_stage, "param_stage", W),
                                       int(chunk_numel), _dptr(flat_param_out, "flat_param_out", W),
                                       dtype_code(param_dtype), int(n_threads), _stream(stream)),
           "zs_offload_adamw_step")


# ---------------------------------------------------------------------------- bandwidth yardsticks
# (include/zs_probe.h: the update's access patterns without its arithmetic; they overwrite the
# buffers they are given)

def zs_probe_mix(g, p, m, v, out, n, stream=None):
    w = "zs_probe_mix"
    _check(lib().zs_probe_mix(_dptr(g, "g", w), _dptr(p, "p", w), _dptr(m, "m", w), _dptr(v, "v", w),
                              _dptr(out, "out", w), int(n), _stream(stream)), w)


def zs_probe_copy(src, dst, nbytes, stream=None):
    w = "zs_probe_copy"
    _check(lib().zs_probe_copy(_dptr(src, "src", w), _dptr(dst, "dst", w), int(nbytes), _stream(stream)), w)


def zs_probe_read(src, nbytes, sink, stream=None):
    w = "zs_probe_read"
    _check(lib().zs_probe_read(_dptr(src, "src", w), int(nbytes), _dptr(sink, "sink", w), _stream(stream)), w)


def zs_probe_write(dst, nbytes, stream=None):
    w = "zs_probe_write"
    _check(lib().zs_probe_write(_dptr(dst, "dst", w), int(nbytes), _stream(stream)), w)
