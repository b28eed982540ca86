"""Thin ctypes binding of libcbs (include/cbs.h), same entry-point names.

Argument marshalling only: every step of the fused conv path runs in the HIP
kernels of libcbs.so.  Device buffers may be given as torch tensors (their
``data_ptr()`` is passed) or as raw integer addresses; streams as
``torch.cuda.Stream`` objects, raw handles or None (the current torch stream).
Host arrays (weights, BN parameters) are numpy arrays.

A tensor handed to a run call is checked before the call: it must live on a
GPU and its storage must hold, from the tensor's first byte, at least the
bytes the layer reads or writes there (cbs_layer_info's in_bytes, out_bytes,
res_bytes); the kernels take their buffer ranges from the layer, not from
the allocation, so a host pointer or a short buffer would otherwise become an
out-of-range device access.  Raw integer addresses are passed unchecked.

torch is imported before libcbs.so is loaded so that both share the one HIP
runtime (libamdhip64.so.7) that torch loads.  If libcbs.so is missing this
module raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime first)

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libcbs.so")

CBS_OK = 0
CBS_EINVAL = -1
CBS_EUNSUPPORTED = -2
CBS_ENOMEM = -3
CBS_EDEVICE = -4
CBS_ELAUNCH = -5
CBS_F32 = 0
CBS_I8 = 1
CBS_U8 = 2
CBS_ACT_SILU = 0
CBS_ACT_NONE = 1
CBS_TUNE_FORCE = 1

_STATUS_NAMES = {0: "CBS_OK", -1: "CBS_EINVAL", -2: "CBS_EUNSUPPORTED", -3: "CBS_ENOMEM",
                 -4: "CBS_EDEVICE", -5: "CBS_ELAUNCH"}


class CbsError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, _STATUS_NAMES.get(status, status), message))


class cbs_conv_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("c_in", ctypes.c_int32), ("h", ctypes.c_int32),
                ("w", ctypes.c_int32), ("c_out", ctypes.c_int32), ("k", ctypes.c_int32),
                ("stride", ctypes.c_int32), ("pad", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_row_pitch", ctypes.c_int32), ("in_scale", ctypes.c_float),
                ("bn_eps", ctypes.c_float), ("act", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("out_scale", ctypes.c_float), ("in_c_stride", ctypes.c_int32), ("in_c_offset", ctypes.c_int32),
                ("out_c_stride", ctypes.c_int32), ("out_c_offset", ctypes.c_int32),
                ("res_c_stride", ctypes.c_int32), ("res_c_offset", ctypes.c_int32), ("res_scale", ctypes.c_float),
                ("in_zero_point", ctypes.c_int32), ("out_zero_point", ctypes.c_int32),
                ("res_zero_point", ctypes.c_int32), ("in2_channels", ctypes.c_int32), ("in2_c_stride", ctypes.c_int32)]


class cbs_layer_info_t(ctypes.Structure):
    _fields_ = [("c_in_pad", ctypes.c_int32), ("c_out_pad", ctypes.c_int32), ("oh", ctypes.c_int32),
                ("ow", ctypes.c_int32), ("out_row_pitch", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("in_bytes", ctypes.c_int64), ("out_bytes", ctypes.c_int64), ("flops", ctypes.c_int64),
                ("alg_bytes", ctypes.c_int64), ("config", ctypes.c_int32), ("splitk", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("threads", ctypes.c_int32), ("config_name", ctypes.c_char * 48),
                ("res_bytes", ctypes.c_int64), ("in2_bytes", ctypes.c_int64)]


class cbs_graph_group_info_t(ctypes.Structure):
    _fields_ = [("group_id", ctypes.c_int32), ("members", ctypes.c_int32), ("kept", ctypes.c_int32),
                ("config", ctypes.c_int32), ("us_grouped", ctypes.c_float), ("us_separate", ctypes.c_float)]


class cbs_step(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_void_p), ("in_", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("residual", ctypes.c_void_p), ("in2", ctypes.c_void_p)]


# Every symbol the header declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGNATURES = {
    "cbs_create_layer": (_I, [ctypes.POINTER(cbs_conv_desc), _P, _P, _P, _P, _P, ctypes.POINTER(_P)]),
    "cbs_create_layer_folded": (_I, [ctypes.POINTER(cbs_conv_desc), _P, _P, _P, ctypes.POINTER(_P)]),
    "cbs_destroy_layer": (None, [_P]),
    "cbs_run_layer": (_I, [_P, _P, _P, _P]),
    "cbs_run_layer_res": (_I, [_P, _P, _P, _P, _P]),
    "cbs_run_layer_in2": (_I, [_P, _P, _P, _P, _P, _P]),
    "cbs_run_layer_noalloc": (_I, [_P, _P, _P, _I, _P]),
    "cbs_run_steps": (_I, [ctypes.POINTER(cbs_step), _I, _P]),
    "cbs_graph_create_steps": (_I, [ctypes.POINTER(cbs_step), _I, _P, ctypes.POINTER(_P)]),
    "cbs_run_layer_list": (_I, [ctypes.POINTER(_P), _I, ctypes.POINTER(_P), ctypes.POINTER(_P), _P]),
    "cbs_graph_create": (_I, [ctypes.POINTER(_P), _I, ctypes.POINTER(_P), ctypes.POINTER(_P), _P,
                              ctypes.POINTER(_P)]),
    "cbs_graph_create_grouped": (_I, [ctypes.POINTER(_P), _I, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                      ctypes.POINTER(_I), _P, ctypes.POINTER(_P)]),
    "cbs_graph_info": (_I, [_P, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "cbs_graph_group_info": (_I, [_P, _I, ctypes.POINTER(cbs_graph_group_info_t)]),
    "cbs_graph_launch": (_I, [_P, _P]),
    "cbs_graph_destroy": (None, [_P]),
    "cbs_group_create": (_I, [ctypes.POINTER(_P), _I, _I, ctypes.POINTER(_P)]),
    "cbs_group_run": (_I, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), _P]),
    "cbs_group_config": (_I, [_P]),
    "cbs_group_destroy": (None, [_P]),
    "cbs_layer_info": (_I, [_P, ctypes.POINTER(cbs_layer_info_t)]),
    "cbs_layer_set_config": (_I, [_P, _I, _I]),
    "cbs_num_configs": (_I, []),
    "cbs_layer_autotune": (_I, [_P, _P, _P, _P, _I, _I, _P, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "cbs_autotune_clear_cache": (None, []),
    "cbs_config_name": (ctypes.c_char_p, [_I]),
    "cbs_last_error": (ctypes.c_char_p, []),
    "cbs_pack_nhwc_f32": (_I, [_P, _P, _I, _I, _I, _I, _I, _P]),
    "cbs_quantize_nhwc_i8": (_I, [_P, _P, ctypes.c_float, _I, _I, _I, _I, _I, _P]),
    "cbs_quantize_nhwc_u8": (_I, [_P, _P, ctypes.c_float, _I, _I, _I, _I, _I, _I, _P]),
    "cbs_run_layer_raw_acc": (_I, [_P, _P, _P, _P]),
    "cbs_get_qweights": (_I, [_P, _P, _P]),
    "cbs_get_folded": (_I, [_P, _P, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libcbs.so not built at %s (run __graft_entry__.build())" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int, where: str) -> None:
    if status != CBS_OK:
        msg = lib.cbs_last_error()
        raise CbsError(status, where, msg.decode() if msg else "")


def _dev_ptr(buf, need: int = 0, what: str = "buffer") -> int:
    """Device address of a tensor (or a raw address, unchecked).  A tensor must be
    on a GPU and its storage must hold at least `need` bytes from its first byte."""
    if buf is None:
        return 0
    if isinstance(buf, int):
        return buf
    if not buf.is_cuda:
        raise ValueError("%s is not on a GPU (device %s)" % (what, buf.device))
    ptr = int(buf.data_ptr())
    if need > 0:
        st = buf.untyped_storage()
        avail = int(st.data_ptr()) + int(st.nbytes()) - ptr
        if avail < need:
            raise ValueError("%s holds %d bytes from its start; the layer needs %d" % (what, avail, need))
    return ptr


def _in_ptr(layer, buf, what="input"):
    return _dev_ptr(buf, layer.in_bytes, what)


def _out_ptr(layer, buf, what="output"):
    return _dev_ptr(buf, layer.out_bytes, what)


def _res_ptr(layer, buf, what="residual"):
    return _dev_ptr(buf, layer.res_bytes, what)


def _in2_ptr(layer, buf, what="second input"):
    return _dev_ptr(buf, layer.in2_bytes, what)


def _stream(stream) -> int:
    if stream is None:
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _host(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class Layer:
    """Handle of a created layer (a cbs_layer*), destroyed on garbage collection.
    The byte counts are the buffer sizes a run reads or writes (cbs_layer_info)."""
    handle: int
    desc: cbs_conv_desc
    in_bytes: int = 0
    out_bytes: int = 0
    res_bytes: int = 0
    in2_bytes: int = 0
    acc_bytes: int = 0  # int32 accumulators of cbs_run_layer_raw_acc

    def __post_init__(self):
        info = cbs_layer_info_t()
        _check(lib.cbs_layer_info(self.handle, ctypes.byref(info)), "cbs_layer_info")
        self.in_bytes, self.out_bytes, self.res_bytes = int(info.in_bytes), int(info.out_bytes), int(info.res_bytes)
        self.in2_bytes = int(info.in2_bytes)
        self.acc_bytes = self.desc.n * info.oh * info.out_row_pitch * info.c_out_pad * 4

    def __del__(self):
        if getattr(self, "handle", 0) and lib is not None:
            lib.cbs_destroy_layer(self.handle)
            self.handle = 0


def make_desc(n, c_in, h, w, c_out, k, stride, pad, dtype=CBS_F32, out_row_pitch=0, in_scale=0.0,
              bn_eps=1e-3, act=CBS_ACT_SILU, out_dtype=CBS_F32, out_scale=0.0, in_c_stride=0, in_c_offset=0,
              out_c_stride=0, out_c_offset=0, res_c_stride=0, res_c_offset=0, res_scale=0.0, in_zero_point=0,
              out_zero_point=0, res_zero_point=0, in2_channels=0, in2_c_stride=0) -> cbs_conv_desc:
    return cbs_conv_desc(n, c_in, h, w, c_out, k, stride, pad, dtype, out_row_pitch, float(in_scale),
                         float(bn_eps), act, out_dtype, float(out_scale), in_c_stride, in_c_offset,
                         out_c_stride, out_c_offset, res_c_stride, res_c_offset, float(res_scale),
                         int(in_zero_point), int(out_zero_point), int(res_zero_point), int(in2_channels),
                         int(in2_c_stride))


def cbs_create_layer(desc: cbs_conv_desc, w_oihw, gamma, beta, mean, var) -> Layer:
    ws = [_host(a, np.float32) for a in (w_oihw, gamma, beta, mean, var)]
    h = _P()
    _check(lib.cbs_create_layer(ctypes.byref(desc), *[p for _, p in ws], ctypes.byref(h)), "cbs_create_layer")
    return Layer(h.value, desc)


def cbs_create_layer_folded(desc: cbs_conv_desc, w_oihw, scale, bias) -> Layer:
    ws = [_host(a, np.float32) for a in (w_oihw, scale, bias)]
    h = _P()
    _check(lib.cbs_create_layer_folded(ctypes.byref(desc), *[p for _, p in ws], ctypes.byref(h)),
           "cbs_create_layer_folded")
    return Layer(h.value, desc)


def cbs_destroy_layer(layer: Layer) -> None:
    if layer.handle:
        lib.cbs_destroy_layer(layer.handle)
        layer.handle = 0


def cbs_run_layer(layer: Layer, inp, out, stream=None) -> None:
    _check(lib.cbs_run_layer(layer.handle, _in_ptr(layer, inp), _out_ptr(layer, out), _stream(stream)),
           "cbs_run_layer")


CBS_NOALLOC_PARTIAL_BYTES = 8 << 20
CBS_NOALLOC_TICKETS = 16384


def cbs_run_layer_noalloc(layer: Layer, inp, out, splitk: int = 0, stream=None) -> None:
    _check(lib.cbs_run_layer_noalloc(layer.handle, _in_ptr(layer, inp), _out_ptr(layer, out), int(splitk),
                                     _stream(stream)), "cbs_run_layer_noalloc")


def cbs_run_layer_res(layer: Layer, inp, out, residual, stream=None) -> None:
    _check(lib.cbs_run_layer_res(layer.handle, _in_ptr(layer, inp), _out_ptr(layer, out), _res_ptr(layer, residual),
                                 _stream(stream)), "cbs_run_layer_res")


def cbs_run_layer_in2(layer: Layer, inp, in2, out, residual=None, stream=None) -> None:
    _check(lib.cbs_run_layer_in2(layer.handle, _in_ptr(layer, inp), _in2_ptr(layer, in2), _out_ptr(layer, out),
                                 _res_ptr(layer, residual), _stream(stream)), "cbs_run_layer_in2")


def _step_array(steps):
    """steps: (layer, in, out), (layer, in, out, residual) or (layer, in, out, residual,
    second input) tuples (residual None when the layer has none)."""
    arr = (cbs_step * max(1, len(steps)))()
    for i, st in enumerate(steps):
        layer, inp, out = st[:3]
        res = st[3] if len(st) > 3 else None
        in2 = st[4] if len(st) > 4 else None
        w = "step %d " % i
        arr[i] = cbs_step(layer.handle, _in_ptr(layer, inp, w + "input"), _out_ptr(layer, out, w + "output"),
                          _res_ptr(layer, res, w + "residual"), _in2_ptr(layer, in2, w + "second input"))
    return arr


def cbs_run_steps(steps, stream=None) -> None:
    _check(lib.cbs_run_steps(_step_array(steps), len(steps), _stream(stream)), "cbs_run_steps")


class StepList:
    """A step list marshalled once (see LayerList), so that run() costs one C call."""

    def __init__(self, steps):
        self.n = len(steps)
        self._arr = _step_array(steps)
        self._keep = list(steps)

    def run(self, stream=None) -> None:
        _check(lib.cbs_run_steps(self._arr, self.n, _stream(stream)), "cbs_run_steps")


def cbs_graph_create_steps(steps, stream=None) -> "Graph":
    h = _P()
    _check(lib.cbs_graph_create_steps(_step_array(steps), len(steps), _stream(stream), ctypes.byref(h)),
           "cbs_graph_create_steps")
    return Graph(h.value, list(steps))


def _ptr_array(items):
    arr = (_P * max(1, len(items)))()
    for i, it in enumerate(items):
        arr[i] = it
    return arr


def _list_arrays(layers, ins, outs):
    if not (len(layers) == len(ins) == len(outs)):
        raise ValueError("layers, ins and outs differ in length")
    return (_ptr_array([l.handle for l in layers]),
            _ptr_array([_in_ptr(l, b, "input %d" % i) for i, (l, b) in enumerate(zip(layers, ins))]),
            _ptr_array([_out_ptr(l, b, "output %d" % i) for i, (l, b) in enumerate(zip(layers, outs))]))


def cbs_run_layer_list(layers, ins, outs, stream=None) -> None:
    la, ia, oa = _list_arrays(layers, ins, outs)
    _check(lib.cbs_run_layer_list(la, len(layers), ia, oa, _stream(stream)), "cbs_run_layer_list")


class LayerList:
    """A layer list marshalled once (pointer arrays built and checked here), so
    that run() costs one C call: used where the host time of building the
    arguments must stay out of a timed region."""

    def __init__(self, layers, ins, outs):
        self.n = len(layers)
        self._arrays = _list_arrays(layers, ins, outs)
        self._keep = (list(layers), list(ins), list(outs))

    def run(self, stream=None) -> None:
        la, ia, oa = self._arrays
        _check(lib.cbs_run_layer_list(la, self.n, ia, oa, _stream(stream)), "cbs_run_layer_list")


class Graph:
    """A captured layer list (cbs_graph*), destroyed on garbage collection."""

    def __init__(self, handle: int, keep):
        self.handle = handle
        self._keep = keep  # layers and buffers must outlive the graph

    def __del__(self):
        if getattr(self, "handle", 0) and lib is not None:
            lib.cbs_graph_destroy(self.handle)
            self.handle = 0


def cbs_graph_create(layers, ins, outs, stream=None) -> Graph:
    h = _P()
    la, ia, oa = _list_arrays(layers, ins, outs)
    _check(lib.cbs_graph_create(la, len(layers), ia, oa, _stream(stream), ctypes.byref(h)), "cbs_graph_create")
    return Graph(h.value, (list(layers), list(ins), list(outs)))


def cbs_graph_create_grouped(layers, ins, outs, group_of, stream=None) -> Graph:
    """group_of: one int per layer, its candidate group (>= 0) or -1 (alone)."""
    h = _P()
    la, ia, oa = _list_arrays(layers, ins, outs)
    if len(group_of) != len(layers):
        raise ValueError("group_of has %d entries for %d layers" % (len(group_of), len(layers)))
    ga = (_I * max(1, len(group_of)))(*[int(g) for g in group_of])
    _check(lib.cbs_graph_create_grouped(la, len(layers), ia, oa, ga, _stream(stream), ctypes.byref(h)),
           "cbs_graph_create_grouped")
    return Graph(h.value, (list(layers), list(ins), list(outs)))


def cbs_graph_info(graph: Graph):
    """-> (kernel launches per replay, candidate groups)."""
    a, b = _I(), _I()
    _check(lib.cbs_graph_info(graph.handle, ctypes.byref(a), ctypes.byref(b)), "cbs_graph_info")
    return a.value, b.value


def cbs_graph_group_info(graph: Graph, i: int) -> dict:
    info = cbs_graph_group_info_t()
    _check(lib.cbs_graph_group_info(graph.handle, int(i), ctypes.byref(info)), "cbs_graph_group_info")
    return {name: getattr(info, name) for name, _ in cbs_graph_group_info_t._fields_}


def cbs_graph_launch(graph: Graph, stream=None) -> None:
    _check(lib.cbs_graph_launch(graph.handle, _stream(stream)), "cbs_graph_launch")


def cbs_graph_destroy(graph: Graph) -> None:
    if graph.handle:
        lib.cbs_graph_destroy(graph.handle)
        graph.handle = 0


CBS_GROUP_MAX = 4


class Group:
    """Independent layers run by one launch (a cbs_group*), destroyed on garbage collection."""

    def __init__(self, handle: int, layers):
        self.handle = handle
        self._layers = layers  # the layers must outlive the group

    def __del__(self):
        if getattr(self, "handle", 0) and lib is not None:
            lib.cbs_group_destroy(self.handle)
            self.handle = 0


def cbs_group_create(layers, config: int = -1) -> Group:
    h = _P()
    _check(lib.cbs_group_create(_ptr_array([l.handle for l in layers]), len(layers), config, ctypes.byref(h)),
           "cbs_group_create")
    return Group(h.value, list(layers))


def cbs_group_run(group: Group, ins, outs, stream=None) -> None:
    _, ia, oa = _list_arrays(group._layers, ins, outs)
    _check(lib.cbs_group_run(group.handle, ia, oa, _stream(stream)), "cbs_group_run")


def cbs_group_config(group: Group) -> int:
    return lib.cbs_group_config(group.handle)


def cbs_layer_info(layer: Layer) -> dict:
    info = cbs_layer_info_t()
    _check(lib.cbs_layer_info(layer.handle, ctypes.byref(info)), "cbs_layer_info")
    d = {name: getattr(info, name) for name, _ in cbs_layer_info_t._fields_}
    d["config_name"] = info.config_name.decode()
    return d


def cbs_layer_set_config(layer: Layer, config: int, splitk: int = 0) -> None:
    _check(lib.cbs_layer_set_config(layer.handle, int(config), int(splitk)), "cbs_layer_set_config")


def cbs_layer_autotune(layer: Layer, inp, out, residual=None, iters=0, flags=0, stream=None):
    """Time every configuration on these buffers and keep the fastest; returns (config, splitk)."""
    c, k = _I(), _I()
    _check(lib.cbs_layer_autotune(layer.handle, _in_ptr(layer, inp), _out_ptr(layer, out),
                                  _res_ptr(layer, residual), int(iters), int(flags), _stream(stream),
                                  ctypes.byref(c), ctypes.byref(k)),
           "cbs_layer_autotune")
    return c.value, k.value


def cbs_autotune_clear_cache() -> None:
    lib.cbs_autotune_clear_cache()


def cbs_num_configs() -> int:
    return int(lib.cbs_num_configs())


def cbs_config_name(config: int):
    r = lib.cbs_config_name(int(config))
    return r.decode() if r else None


def cbs_last_error() -> str:
    r = lib.cbs_last_error()
    return r.decode() if r else ""


def cbs_pack_nhwc_f32(nchw, nhwc, n, c, h, w, c_pad, stream=None) -> None:
    _check(lib.cbs_pack_nhwc_f32(_dev_ptr(nchw, 4 * n * c * h * w, "NCHW input"),
                                 _dev_ptr(nhwc, 4 * n * h * w * c_pad, "NHWC output"), n, c, h, w, c_pad,
                                 _stream(stream)),
           "cbs_pack_nhwc_f32")


def cbs_quantize_nhwc_i8(nchw, nhwc, s_x, n, c, h, w, c_pad, stream=None) -> None:
    _check(lib.cbs_quantize_nhwc_i8(_dev_ptr(nchw, 4 * n * c * h * w, "NCHW input"),
                                    _dev_ptr(nhwc, n * h * w * c_pad, "NHWC output"), float(s_x), n, c, h, w, c_pad,
                                    _stream(stream)), "cbs_quantize_nhwc_i8")


def cbs_quantize_nhwc_u8(nchw, nhwc, s_x, z, n, c, h, w, c_pad, stream=None) -> None:
    _check(lib.cbs_quantize_nhwc_u8(_dev_ptr(nchw, 4 * n * c * h * w, "NCHW input"),
                                    _dev_ptr(nhwc, n * h * w * c_pad, "NHWC output"), float(s_x), int(z), n, c, h, w,
                                    c_pad,
                                    _stream(stream)), "cbs_quantize_nhwc_u8")


def cbs_run_layer_raw_acc(layer: Layer, inp, acc, stream=None) -> None:
    _check(lib.cbs_run_layer_raw_acc(layer.handle, _in_ptr(layer, inp), _dev_ptr(acc, layer.acc_bytes, "accumulators"),
                                     _stream(stream)), "cbs_run_layer_raw_acc")


def cbs_get_qweights(layer: Layer):
    d = layer.desc
    q = np.empty((d.c_out, d.c_in, d.k, d.k), np.int8)
    s = np.empty((d.c_out,), np.float64)
    _check(lib.cbs_get_qweights(layer.handle, q.ctypes.data_as(_P), s.ctypes.data_as(_P)), "cbs_get_qweights")
    return q, s


def cbs_get_folded(layer: Layer):
    d = layer.desc
    w = np.empty((d.c_out, d.c_in, d.k, d.k), np.float32) if d.dtype == CBS_F32 else None
    b = np.empty((d.c_out,), np.float32)
    _check(lib.cbs_get_folded(layer.handle, w.ctypes.data_as(_P) if w is not None else None,
                              b.ctypes.data_as(_P)), "cbs_get_folded")
    return w, b
