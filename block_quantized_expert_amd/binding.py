"""Thin ctypes binding over libmoe.so (declared in include/moe.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are passed as device pointers (``data_ptr()``) together with
the current HIP stream of torch.  There is no fallback: if the library is
missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_ACT_F32, MOE_ACT_BF16 = 0, 1
MOE_W_MXFP4, MOE_W_FP8E4M3_B128 = 0, 1
MOE_DEVERR_EXPERT_ID, MOE_DEVERR_TOKEN_ID, MOE_DEVERR_SYNC = 1, 2, 4
MOE_FORWARD_SYNC_BYTES = 8192
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/*.h declare
EXPORTED = ["moe_route", "moe_route_hash", "moe_route_group", "moe_group_workspace_bytes",
            "moe_group", "moe_ffn_workspace_bytes", "moe_ffn_forward", "moe_ffn_gate_up",
            "moe_ffn_down", "moe_ffn_forward_timed", "moe_forward_workspace_bytes",
            "moe_forward_single_kernel", "moe_forward_workspace_init", "moe_forward",
            "moe_forward_timed", "moe_forward_noalloc", "moe_status_string",
            "moe_stream_read", "moe_mfma_rate", "moe_mfma_rate_out_floats", "moe_route_ex", "moe_route_group_ex", "moe_ffn_forward_ex",
            "moe_forward_ex", "moe_packed_experts_bytes", "moe_pack_experts"]

WEIGHT_TYPES = {"mxfp4": MOE_W_MXFP4, "fp8_e4m3_b128": MOE_W_FP8E4M3_B128}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s" % (where, status_string(status)))
        self.status = status


class MoeProj(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class MoeOpts(ctypes.Structure):
    _fields_ = [("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("sel_bias", ctypes.c_void_p), ("keep_max", ctypes.c_int32),
                ("min_w", ctypes.c_float), ("lazy_tau", ctypes.c_float)]


def make_opts(n_group=0, topk_group=0, sel_bias=None, keep_max=0, min_w=0.0, lazy_tau=0.0):
    """A moe_opts; ``sel_bias`` is a device fp32 tensor [n_experts] or None
    (the struct keeps a reference to it, so its memory stays valid while the
    struct lives)."""
    o = MoeOpts()
    o.n_group, o.topk_group, o.keep_max = n_group, topk_group, keep_max
    o.sel_bias = None if sel_bias is None else sel_bias.data_ptr()
    o.min_w, o.lazy_tau = min_w, lazy_tau
    o._sel_bias_tensor = sel_bias
    return o


def _opts_ref(opts):
    return None if opts is None else ctypes.byref(opts)


class MoeLayer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("gate", MoeProj), ("up", MoeProj), ("down", MoeProj),
                ("has_shared", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("shared_gate", MoeProj), ("shared_up", MoeProj), ("shared_down", MoeProj),
                ("packed_experts", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmoe.so is not built (%s); run "
                               "python -m block_quantized_expert_amd.build" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.moe_route.argtypes = [P, I, I, I, F, P, P, P]
        L.moe_route_hash.argtypes = [P, I, P, P, I, I, I, P, P, P, P]
        L.moe_group_workspace_bytes.argtypes = [I, I, I]
        L.moe_group_workspace_bytes.restype = S
        L.moe_group.argtypes = [P, I, I, I, P, P, P, P, P, P, S, P]
        L.moe_route_group.argtypes = [P, I, I, I, F, P, P, P, P, P, P, P, P]
        L.moe_ffn_forward_timed.argtypes = [ctypes.POINTER(MoeLayer), P, I, I, P, P, P, P, P,
                                            P, P, S, P, P, P, P, P]
        L.moe_ffn_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayer), I]
        L.moe_ffn_workspace_bytes.restype = S
        ffn_args = [ctypes.POINTER(MoeLayer), P, I, I, P, P, P, P, P, P, P, S, P]
        for name in ("moe_ffn_forward", "moe_ffn_gate_up", "moe_ffn_down"):
            getattr(L, name).argtypes = ffn_args
        for name in ("moe_route", "moe_route_hash", "moe_route_group", "moe_group",
                     "moe_ffn_forward", "moe_ffn_gate_up", "moe_ffn_down",
                     "moe_ffn_forward_timed"):
            getattr(L, name).restype = ctypes.c_int
        L.moe_forward_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayer), I]
        L.moe_forward_workspace_bytes.restype = S
        L.moe_forward_workspace_init.argtypes = [P, S, P]
        L.moe_forward_single_kernel.argtypes = [ctypes.POINTER(MoeLayer), I, I]
        L.moe_forward_single_kernel.restype = ctypes.c_int
        fwd = [ctypes.POINTER(MoeLayer), P, F, P, I, I, P, P, P, P, P, P, P, P, S, P, P]
        L.moe_forward.argtypes = fwd
        L.moe_forward_timed.argtypes = fwd + [P, P]
        L.moe_forward_noalloc.argtypes = fwd[:13] + [P, P]
        for name in ("moe_forward_workspace_init", "moe_forward", "moe_forward_timed",
                     "moe_forward_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        O = ctypes.POINTER(MoeOpts)
        L.moe_route_ex.argtypes = [P, I, I, I, F, O, P, P, P]
        L.moe_route_group_ex.argtypes = [P, I, I, I, F, O, P, P, P, P, P, P, P, P]
        L.moe_ffn_forward_ex.argtypes = [ctypes.POINTER(MoeLayer), P, I, I, P, P, P, P, P, P, O,
                                         P, S, P, P, P, P, P]
        L.moe_forward_ex.argtypes = [ctypes.POINTER(MoeLayer), P, F, O, P, I, I, P, P, P, P, P,
                                     P, P, P, S, P, P, P, P]
        for name in ("moe_route_ex", "moe_route_group_ex", "moe_ffn_forward_ex",
                     "moe_forward_ex"):
            getattr(L, name).restype = ctypes.c_int
        L.moe_stream_read.argtypes = [P, S, P, P]
        L.moe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
        L.moe_mfma_rate.restype = ctypes.c_int
        L.moe_mfma_rate_out_floats.argtypes = []
        L.moe_mfma_rate_out_floats.restype = S
        L.moe_packed_experts_bytes.argtypes = [ctypes.POINTER(MoeLayer)]
        L.moe_packed_experts_bytes.restype = S
        L.moe_pack_experts.argtypes = [ctypes.POINTER(MoeLayer), P, S, P]
        L.moe_stream_read.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


class HipEvent:
    """A timing hipEvent_t made with the HIP runtime the process has already
    loaded (the one torch and libmoe.so share).  Events recorded by the
    library from kernel dispatches are read with ``elapsed_ms``."""

    _rt = None

    @classmethod
    def runtime(cls):
        if cls._rt is None:
            rt = ctypes.CDLL("libamdhip64.so.7")
            rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
            rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            cls._rt = rt
        return cls._rt

    def __init__(self):
        self.handle = ctypes.c_void_p()
        if self.runtime().hipEventCreate(ctypes.byref(self.handle)) != 0:
            raise RuntimeError("hipEventCreate failed")

    def __del__(self):
        if self._rt is not None and self.handle:
            self._rt.hipEventDestroy(self.handle)

    def elapsed_ms(self, stop: "HipEvent") -> float:
        ms = ctypes.c_float()
        rt = self.runtime()
        rt.hipEventSynchronize(stop.handle)
        if rt.hipEventElapsedTime(ctypes.byref(ms), self.handle, stop.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------------------
# Layer description
# ----------------------------------------------------------------------------


class Layer:
    """A moe_layer over device tensors; keeps the tensors alive.

    ``weights`` is the dict made by ``inputs.make_layer`` (stacked routed
    tensors [E][rows][...], optional ``shared``)."""

    def __init__(self, weights: dict, top_k: int):
        self.weights = weights
        L = MoeLayer()
        L.hidden = weights["hidden"]
        L.inter = weights["inter"]
        L.n_experts = weights["n_experts"]
        L.top_k = top_k
        for name in ("gate", "up", "down"):
            setattr(L, name, self._proj(weights[name]))
        shared = weights.get("shared")
        L.has_shared = 1 if shared is not None else 0
        if shared is not None:
            L.shared_inter = shared["inter"]
            L.shared_gate = self._proj(shared["gate"])
            L.shared_up = self._proj(shared["up"])
            L.shared_down = self._proj(shared["down"])
        self.c = L

    @staticmethod
    def _proj(p: dict) -> MoeProj:
        return MoeProj(WEIGHT_TYPES[p["type"]], p["codes"].data_ptr(), p["scales"].data_ptr())

    @property
    def hidden(self):
        return self.c.hidden

    @property
    def top_k(self):
        return self.c.top_k

    def workspace_bytes(self, n_tokens: int) -> int:
        return lib().moe_ffn_workspace_bytes(ctypes.byref(self.c), n_tokens)

    def packed_bytes(self) -> int:
        return lib().moe_packed_experts_bytes(ctypes.byref(self.c))

    def pack(self, stream=None) -> bool:
        """Writes the packed copy of the MXFP4 matrices (moe_pack_experts) into
        a new device buffer and points the layer at it; False when the layer
        cannot be packed.  ``unpack()`` drops it again."""
        n = self.packed_bytes()
        if n == 0:
            return False
        dev = self.weights["gate"]["codes"].device
        buf = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        off = (-buf.data_ptr()) % 256
        view = buf[off:off + n]
        st = lib().moe_pack_experts(ctypes.byref(self.c), ctypes.c_void_p(view.data_ptr()),
                                    ctypes.c_size_t(n), _stream(stream))
        _check(st, "moe_pack_experts")
        self._packed = buf
        self.c.packed_experts = view.data_ptr()
        return True

    def unpack(self):
        self.c.packed_experts = None
        self._packed = None

    def forward_workspace_bytes(self, n_tokens: int) -> int:
        return lib().moe_forward_workspace_bytes(ctypes.byref(self.c), n_tokens)


# ----------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ----------------------------------------------------------------------------


def moe_route(logits, top_k, routed_scale=1.5, ids=None, w=None, stream=None):
    n, e = logits.shape
    dev = logits.device
    ids = torch.empty((n, top_k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((n, top_k), dtype=torch.float32, device=dev) if w is None else w
    _check(lib().moe_route(_ptr(logits), n, e, top_k, routed_scale, _ptr(ids), _ptr(w),
                           _stream(stream)), "moe_route")
    return ids, w


def moe_route_hash(token_ids, tid2eid, tid2w, n_experts, ids=None, w=None, dev_error=None,
                   stream=None):
    n = token_ids.shape[0]
    vocab, top_k = tid2eid.shape
    dev = token_ids.device
    ids = torch.empty((n, top_k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((n, top_k), dtype=torch.float32, device=dev) if w is None else w
    _check(lib().moe_route_hash(_ptr(token_ids), n, _ptr(tid2eid), _ptr(tid2w), vocab, n_experts,
                                top_k, _ptr(ids), _ptr(w), _ptr(dev_error), _stream(stream)),
           "moe_route_hash")
    return ids, w


def moe_route_ex(logits, top_k, opts, routed_scale=1.5, stream=None):
    n, e = logits.shape
    dev = logits.device
    ids = torch.empty((n, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((n, top_k), dtype=torch.float32, device=dev)
    _check(lib().moe_route_ex(_ptr(logits), n, e, top_k, routed_scale, _opts_ref(opts), _ptr(ids),
                              _ptr(w), _stream(stream)), "moe_route_ex")
    return ids, w


def moe_route_group_ex(logits, top_k, opts, routed_scale=1.5, dev_error=None, stream=None):
    """Route with options and group.  Returns (ids, w, (counts, offsets, perm, inv_perm))."""
    n, e = logits.shape
    dev = logits.device
    ids = torch.empty((n, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((n, top_k), dtype=torch.float32, device=dev)
    g = (torch.empty(e, dtype=torch.int32, device=dev),
         torch.empty(e + 1, dtype=torch.int32, device=dev),
         torch.empty(n * top_k, dtype=torch.int32, device=dev),
         torch.empty(n * top_k, dtype=torch.int32, device=dev))
    _check(lib().moe_route_group_ex(_ptr(logits), n, e, top_k, routed_scale, _opts_ref(opts),
                                    _ptr(ids), _ptr(w), *[_ptr(t) for t in g], _ptr(dev_error),
                                    _stream(stream)), "moe_route_group_ex")
    return ids, w, g


def moe_group(ids, n_experts, out=None, dev_error=None, stream=None):
    """Returns (counts, offsets, perm, inv_perm)."""
    n, k = ids.shape
    dev = ids.device
    if out is None:
        out = (torch.empty(n_experts, dtype=torch.int32, device=dev),
               torch.empty(n_experts + 1, dtype=torch.int32, device=dev),
               torch.empty(n * k, dtype=torch.int32, device=dev),
               torch.empty(n * k, dtype=torch.int32, device=dev))
    counts, offsets, perm, inv_perm = out
    _check(lib().moe_group(_ptr(ids), n, k, n_experts, _ptr(counts), _ptr(offsets), _ptr(perm),
                           _ptr(inv_perm), _ptr(dev_error), None, 0, _stream(stream)),
           "moe_group")
    return counts, offsets, perm, inv_perm


def moe_route_group(logits, top_k, routed_scale=1.5, dev_error=None, stream=None):
    """Fused route + group.  Returns (ids, w, (counts, offsets, perm, inv_perm))."""
    n, e = logits.shape
    dev = logits.device
    ids = torch.empty((n, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((n, top_k), dtype=torch.float32, device=dev)
    g = (torch.empty(e, dtype=torch.int32, device=dev),
         torch.empty(e + 1, dtype=torch.int32, device=dev),
         torch.empty(n * top_k, dtype=torch.int32, device=dev),
         torch.empty(n * top_k, dtype=torch.int32, device=dev))
    _check(lib().moe_route_group(_ptr(logits), n, e, top_k, routed_scale, _ptr(ids), _ptr(w),
                                 *[_ptr(t) for t in g], _ptr(dev_error), _stream(stream)),
           "moe_route_group")
    return ids, w, g


def _ffn_call(name, layer: Layer, x, w, grouping, y, workspace, stream):
    n = x.shape[0]
    x_type = MOE_ACT_BF16 if x.dtype == torch.bfloat16 else MOE_ACT_F32
    if y is None:
        y = torch.empty((n, layer.hidden), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(layer.workspace_bytes(n), 1), dtype=torch.uint8,
                                device=x.device)
    counts, offsets, perm, inv_perm = grouping
    fn = getattr(lib(), name)
    _check(fn(ctypes.byref(layer.c), _ptr(x), x_type, n, _ptr(w), _ptr(counts), _ptr(offsets),
              _ptr(perm), _ptr(inv_perm), _ptr(y), _ptr(workspace), workspace.numel(),
              _stream(stream)), name)
    return y


def moe_ffn_forward(layer: Layer, x, w, grouping, y=None, workspace=None, stream=None):
    return _ffn_call("moe_ffn_forward", layer, x, w, grouping, y, workspace, stream)


def moe_ffn_gate_up(layer: Layer, x, w, grouping, y=None, workspace=None, stream=None):
    return _ffn_call("moe_ffn_gate_up", layer, x, w, grouping, y, workspace, stream)


def moe_ffn_down(layer: Layer, x, w, grouping, y=None, workspace=None, stream=None):
    return _ffn_call("moe_ffn_down", layer, x, w, grouping, y, workspace, stream)


def moe_ffn_forward_timed(layer: Layer, x, w, grouping, events, y=None, workspace=None,
                          stream=None):
    """``events``: four HipEvent (or None) for gate/up start, gate/up stop,
    down start, down stop."""
    n = x.shape[0]
    x_type = MOE_ACT_BF16 if x.dtype == torch.bfloat16 else MOE_ACT_F32
    if y is None:
        y = torch.empty((n, layer.hidden), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(layer.workspace_bytes(n), 1), dtype=torch.uint8,
                                device=x.device)
    counts, offsets, perm, inv_perm = grouping
    evs = [None if e is None else e.handle for e in events]
    _check(lib().moe_ffn_forward_timed(ctypes.byref(layer.c), _ptr(x), x_type, n, _ptr(w),
                                       _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv_perm),
                                       _ptr(y), _ptr(workspace), workspace.numel(),
                                       _stream(stream), *evs), "moe_ffn_forward_timed")
    return y


def moe_ffn_forward_ex(layer: Layer, x, w, grouping, opts, y=None, workspace=None, events=None,
                       stream=None):
    n = x.shape[0]
    x_type = MOE_ACT_BF16 if x.dtype == torch.bfloat16 else MOE_ACT_F32
    if y is None:
        y = torch.empty((n, layer.hidden), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(layer.workspace_bytes(n), 1), dtype=torch.uint8,
                                device=x.device)
    counts, offsets, perm, inv_perm = grouping
    evs = [None] * 4 if events is None else [None if e is None else e.handle for e in events]
    _check(lib().moe_ffn_forward_ex(ctypes.byref(layer.c), _ptr(x), x_type, n, _ptr(w),
                                    _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv_perm),
                                    _ptr(y), _opts_ref(opts), _ptr(workspace), workspace.numel(),
                                    _stream(stream), *evs), "moe_ffn_forward_ex")
    return y


def forward(layer: Layer, x, routing: dict, routed_scale=1.5, stream=None):
    """Route, group and run the FFN (all on the device).  Returns
    (y, ids, w, grouping)."""
    if routing["kind"] == "learned":
        ids, w, grouping = moe_route_group(routing["logits"], layer.top_k, routed_scale,
                                           stream=stream)
    else:
        ids, w = moe_route_hash(routing["token_ids"], routing["tid2eid"], routing["tid2w"],
                                layer.c.n_experts, stream=stream)
        grouping = moe_group(ids, layer.c.n_experts, stream=stream)
    y = moe_ffn_forward(layer, x, w, grouping, stream=stream)
    return y, ids, w, grouping


class ForwardBuffers:
    """Outputs and workspace of moe_forward for a batch of n tokens; the
    workspace's synchronisation words are zeroed once here."""

    def __init__(self, layer: Layer, n_tokens: int, device, stream=None, workspace=True):
        n, k, e = n_tokens, layer.top_k, layer.c.n_experts
        self.n = n
        self.ids = torch.empty((n, k), dtype=torch.int32, device=device)
        self.w = torch.empty((n, k), dtype=torch.float32, device=device)
        self.grouping = (torch.empty(e, dtype=torch.int32, device=device),
                         torch.empty(e + 1, dtype=torch.int32, device=device),
                         torch.empty(max(n * k, 1), dtype=torch.int32, device=device),
                         torch.empty(max(n * k, 1), dtype=torch.int32, device=device))
        self.y = torch.empty((n, layer.hidden), dtype=torch.float32, device=device)
        self.dev_error = torch.zeros(1, dtype=torch.int32, device=device)
        self.workspace = None
        if workspace:
            nbytes = max(layer.forward_workspace_bytes(n), MOE_FORWARD_SYNC_BYTES)
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
            _check(lib().moe_forward_workspace_init(_ptr(self.workspace), nbytes,
                                                    _stream(stream)),
                   "moe_forward_workspace_init")

    def args(self):
        counts, offsets, perm, inv_perm = self.grouping
        return [_ptr(self.ids), _ptr(self.w), _ptr(counts), _ptr(offsets), _ptr(perm),
                _ptr(inv_perm), _ptr(self.y), _ptr(self.workspace),
                0 if self.workspace is None else self.workspace.numel(), _ptr(self.dev_error)]


def moe_forward(layer: Layer, logits, x, routed_scale=1.5, buffers: ForwardBuffers = None,
                stream=None, events=None):
    """The whole layer from router logits (learned routing) in one call.
    Returns the ForwardBuffers holding y, ids, w, grouping and dev_error.
    ``events``: (start, stop) HipEvents or None."""
    n = x.shape[0]
    if buffers is None:
        buffers = ForwardBuffers(layer, n, x.device, stream)
    x_type = MOE_ACT_BF16 if x.dtype == torch.bfloat16 else MOE_ACT_F32
    common = [ctypes.byref(layer.c), _ptr(logits), routed_scale, _ptr(x), x_type, n]
    if events is None:
        _check(lib().moe_forward(*common, *buffers.args(), _stream(stream)), "moe_forward")
    else:
        evs = [None if e is None else e.handle for e in events]
        _check(lib().moe_forward_timed(*common, *buffers.args(), _stream(stream), *evs),
               "moe_forward_timed")
    return buffers


def moe_forward_noalloc(layer: Layer, logits, x, routed_scale=1.5, buffers: ForwardBuffers = None,
                        stream=None):
    """moe_forward on the library's own scratch array (no workspace).  Only
    the output tensors of ``buffers`` are used.  Returns the buffers."""
    n = x.shape[0]
    if buffers is None:
        buffers = ForwardBuffers(layer, n, x.device, stream, workspace=False)
    x_type = MOE_ACT_BF16 if x.dtype == torch.bfloat16 else MOE_ACT_F32
    a = buffers.args()
    _check(lib().moe_forward_noalloc(ctypes.byref(layer.c), _ptr(logits), routed_scale, _ptr(x),
                                     x_type, n, *a[:7], a[9], _stream(stream)),
           "moe_forward_noalloc")
    return buffers


def moe_forward_ex(layer: Layer, logits, x, opts, routed_scale=1.5,
                   buffers: ForwardBuffers = None, stream=None, events=None):
    """moe_forward with a moe_opts.  Returns the ForwardBuffers."""
    n = x.shape[0]
    if buffers is None:
        buffers = ForwardBuffers(layer, n, x.device, stream)
    x_type = MOE_ACT_BF16 if x.dtype == torch.bfloat16 else MOE_ACT_F32
    evs = [None, None] if events is None else [None if e is None else e.handle for e in events]
    _check(lib().moe_forward_ex(ctypes.byref(layer.c), _ptr(logits), routed_scale,
                                _opts_ref(opts), _ptr(x), x_type, n, *buffers.args(),
                                _stream(stream), *evs), "moe_forward_ex")
    return buffers
