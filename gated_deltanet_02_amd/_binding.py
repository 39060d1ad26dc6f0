"""ctypes binding of libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: torch tensors become ``gdn_tensor`` descriptors
and the current HIP stream is passed through.  Every step of the prefill runs
in the library's gfx950 kernels; there is no fallback.  The library is found
at $GDN_LIB or next to this file (built by ``gated_deltanet_02_amd.build``);
if it is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

GDN_OK = 0
# The C ABI these structures and prototypes describe (GDN_ABI_VERSION of
# include/gdn.h); a library built from other sources is refused at load.
ABI_VERSION = 9
STATUS_NAMES = {0: "GDN_OK", -1: "GDN_ERR_NULL_ARG", -2: "GDN_ERR_DTYPE",
                -3: "GDN_ERR_SHAPE", -4: "GDN_ERR_LAYOUT",
                -5: "GDN_ERR_UNSUPPORTED", -6: "GDN_ERR_WORKSPACE",
                -7: "GDN_ERR_HIP", -8: "GDN_ERR_INPUT"}
STAGE_TABLE, STAGE_WY, STAGE_SCAN, STAGE_ALL = 1, 2, 4, 7
SCAN_AUTO, SCAN_ONE_PASS, SCAN_TWO_LEVEL = 0, 1, 2
FLAG_BETA_LOGITS, FLAG_DECAY_PROJ, FLAG_OUTPUT_GATE, FLAG_QKV_SILU, FLAG_QKV_CONV = 1, 2, 4, 8, 16
EXPORTED = ("gdn_abi_version", "gdn_default_options", "gdn_prefill",
            "gdn_prefill_ex", "gdn_prefill_noalloc", "gdn_workspace_size", "gdn_get_workspace_layout",
            "gdn_decode", "gdn_output_gate", "gdn_check_cu_seqlens", "gdn_graph_cache_create", "gdn_graph_cache_destroy",
            "gdn_graph_cache_clear", "gdn_graph_cache_stats", "gdn_prefill_graph",
            "gdn_status_string", "gdn_last_error")

_DTYPES = {torch.bfloat16: 1, torch.float32: 2, torch.int32: 3, torch.int64: 4}


class GdnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 4),
                ("stride", ctypes.c_int64 * 4)]


class GdnOptions(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("stages", ctypes.c_uint32),
                ("scan_split", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("decay_a_log", ctypes.c_void_p), ("decay_bias", ctypes.c_void_p),
                ("gate_z", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("segment_chunks", ctypes.c_int32),
                ("conv_weight", ctypes.c_void_p), ("conv_width", ctypes.c_int32),
                ("conv_state_in", ctypes.c_void_p), ("conv_state_out", ctypes.c_void_p)]


class GdnWorkspaceLayout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("max_chunks", ctypes.c_int64)] + [
        (n, ctypes.c_size_t) for n in ("chunk_table", "chunk_offsets", "seq_starts",
                                       "decay", "w", "qp", "ut", "oloc")] + [
        ("split_chunks", ctypes.c_int32)] + [
        (n, ctypes.c_size_t) for n in ("split_y", "split_hmid", "split_hmid_t", "split_psi",
                                       "split_phi")] + [
        ("segment_chunks", ctypes.c_int32), ("segment_state", ctypes.c_size_t),
        ("k_act", ctypes.c_size_t)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    env = os.environ.get("GDN_LIB")
    if env:
        return env
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"libgdn.so not found at {path}; build it with "
                "`python -m gated_deltanet_02_amd.build`")
        L = ctypes.CDLL(path)
        P = ctypes.POINTER
        T = P(GdnTensor)
        L.gdn_abi_version.restype = ctypes.c_int
        built = L.gdn_abi_version()
        if built != ABI_VERSION:
            raise RuntimeError(
                f"{path} implements ABI {built}, this binding ABI {ABI_VERSION}; rebuild it with "
                "`python -m gated_deltanet_02_amd.build`")
        L.gdn_default_options.argtypes = [P(GdnOptions)]
        L.gdn_default_options.restype = None
        L.gdn_prefill.argtypes = [T] * 9 + [ctypes.c_void_p]
        L.gdn_prefill.restype = ctypes.c_int
        L.gdn_prefill_ex.argtypes = [T] * 9 + [P(GdnOptions), ctypes.c_void_p,
                                               ctypes.c_size_t, ctypes.c_void_p]
        L.gdn_prefill_ex.restype = ctypes.c_int
        L.gdn_prefill_noalloc.argtypes = [T] * 9 + [P(GdnOptions), ctypes.c_void_p]
        L.gdn_prefill_noalloc.restype = ctypes.c_int
        L.gdn_workspace_size.argtypes = [T, T, T, T, P(GdnOptions), P(ctypes.c_size_t)]
        L.gdn_workspace_size.restype = ctypes.c_int
        L.gdn_get_workspace_layout.argtypes = [T, T, T, T, P(GdnOptions), P(GdnWorkspaceLayout)]
        L.gdn_get_workspace_layout.restype = ctypes.c_int
        L.gdn_decode.argtypes = [T] * 7 + [P(GdnOptions), ctypes.c_void_p]
        L.gdn_decode.restype = ctypes.c_int
        L.gdn_output_gate.argtypes = [T, T, ctypes.c_void_p, ctypes.c_float, T, ctypes.c_void_p]
        L.gdn_output_gate.restype = ctypes.c_int
        L.gdn_check_cu_seqlens.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        L.gdn_check_cu_seqlens.restype = ctypes.c_int
        L.gdn_graph_cache_create.argtypes = [ctypes.c_int, P(ctypes.c_void_p)]
        L.gdn_graph_cache_create.restype = ctypes.c_int
        L.gdn_graph_cache_destroy.argtypes = [ctypes.c_void_p]
        L.gdn_graph_cache_destroy.restype = None
        L.gdn_graph_cache_clear.argtypes = [ctypes.c_void_p]
        L.gdn_graph_cache_clear.restype = None
        L.gdn_graph_cache_stats.argtypes = [ctypes.c_void_p, P(ctypes.c_int), P(ctypes.c_int64),
                                            P(ctypes.c_int64), P(ctypes.c_int64), P(ctypes.c_int64)]
        L.gdn_graph_cache_stats.restype = ctypes.c_int
        L.gdn_prefill_graph.argtypes = [ctypes.c_void_p] + [T] * 9 + [
            P(GdnOptions), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gdn_prefill_graph.restype = ctypes.c_int
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def describe(t: Optional[torch.Tensor]):
    """A gdn_tensor descriptor for a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d = GdnTensor()
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = _DTYPES.get(t.dtype, 0)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _dev_ptr(t: Optional[torch.Tensor], name: str, dtype=torch.float32):
    if t is None:
        return None
    if t.device.type != "cuda" or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor")
    return t.data_ptr()


def options(chunk: int = 0, scale: float = 1.0, l2_eps: float = 1e-6,
            stages: int = STAGE_ALL, scan_split: int = 0, beta_logits: bool = False,
            decay_proj: bool = False, decay_a_log: Optional[torch.Tensor] = None,
            decay_bias: Optional[torch.Tensor] = None,
            gate_z: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
            norm_eps: float = 1e-6, segment_chunks: int = 0,
            qkv_silu: bool = False, conv_weight: Optional[torch.Tensor] = None,
            conv_state_in: Optional[torch.Tensor] = None,
            conv_state_out: Optional[torch.Tensor] = None) -> GdnOptions:
    """scan_split: SCAN_AUTO (0), SCAN_ONE_PASS (1) or SCAN_TWO_LEVEL (2);
    segment_chunks: 0 automatic, -1 never, n > 0 segments of n chunks;
    qkv_silu: q, k, v hold pre-activation values and the kernels take silu;
    conv_weight: the short convolution's taps, a contiguous f32 GPU tensor
    [2 Hk dk + Hv dv, W] (sets the convolution flag, W = its second size),
    with the history rows conv_state_in and the new history conv_state_out,
    contiguous [N, W - 1, 2 Hk dk + Hv dv] GPU tensors of the input dtype
    (None: zeros / not written; they may be one tensor);
    beta_logits: beta holds raw projections b and the kernels use sigmoid(b);
    decay_proj: g holds the decay gate's raw projection a, with per value head
    f32 tensors decay_a_log and decay_bias (None: zeros);
    gate_z: the output gate's projection, laid out exactly as ``out`` (sets
    the output-gate flag), with the f32 [dv] norm_weight (None: ones).  The
    options hold raw device pointers: the tensors are kept referenced by the
    returned object and must stay alive while calls using it may run."""
    o = GdnOptions()
    o.chunk, o.scale, o.l2_eps, o.stages, o.scan_split = chunk, scale, l2_eps, stages, scan_split
    o.flags = ((FLAG_BETA_LOGITS if beta_logits else 0) | (FLAG_DECAY_PROJ if decay_proj else 0)
               | (FLAG_QKV_SILU if qkv_silu else 0))
    o.decay_a_log = _dev_ptr(decay_a_log, "decay_a_log")
    o.decay_bias = _dev_ptr(decay_bias, "decay_bias")
    o.norm_weight = _dev_ptr(norm_weight, "norm_weight")
    o.norm_eps = norm_eps
    o.segment_chunks = segment_chunks
    o.conv_width = 4
    if conv_weight is not None:
        if conv_weight.dim() != 2:
            raise ValueError("conv_weight must be [channels, width]")
        o.conv_weight = _dev_ptr(conv_weight, "conv_weight")
        o.conv_width = conv_weight.shape[1]
        o.flags |= FLAG_QKV_CONV
        for name, t in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
            if t is not None:
                setattr(o, name, _dev_ptr(t, name, t.dtype))
    if gate_z is not None:
        if gate_z.device.type != "cuda":
            raise ValueError("gate_z must be a GPU tensor")
        o.gate_z = gate_z.data_ptr()
        o.flags |= FLAG_OUTPUT_GATE
    o._keep = (decay_a_log, decay_bias, gate_z, norm_weight, conv_weight, conv_state_in,
               conv_state_out)
    return o


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, lib().gdn_last_error().decode())


def _stream_handle(stream, ref: torch.Tensor) -> int:
    if stream is None:
        return torch.cuda.current_stream(ref.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(stream, device) -> torch.cuda.Stream:
    if isinstance(stream, torch.cuda.Stream):
        return stream
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.ExternalStream(handle, device=device)


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(status).decode()


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


def gdn_default_options() -> GdnOptions:
    o = GdnOptions()
    lib().gdn_default_options(ctypes.byref(o))
    return o


def _descs(q, k, v, g, beta, cu_seqlens, init_state, out, final_state):
    ts = (q, k, v, g, beta, cu_seqlens, init_state, out, final_state)
    for name, t in zip(("q", "k", "v", "g", "beta", "cu_seqlens", "init_state",
                        "out", "final_state"), ts):
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    return [describe(x) for x in ts]


def gdn_prefill(q, k, v, g, beta, cu_seqlens=None, init_state=None, out=None,
                final_state=None, stream=None):
    """Whole prefill with default options; the library allocates its
    workspace stream-ordered.  ``out`` is allocated like ``v`` if None;
    ``final_state`` is written only when given.  Returns (out, final_state)."""
    if out is None:
        out = torch.empty_like(v)
    ds = _descs(q, k, v, g, beta, cu_seqlens, init_state, out, final_state)
    _check(lib().gdn_prefill(*[_ref(d) for d in ds], _stream_handle(stream, v)))
    return out, final_state


def gdn_workspace_size(q, k, v, cu_seqlens=None, opts: Optional[GdnOptions] = None) -> int:
    n = ctypes.c_size_t(0)
    ds = [describe(x) for x in (q, k, v, cu_seqlens)]
    _check(lib().gdn_workspace_size(*[_ref(d) for d in ds],
                                    ctypes.byref(opts) if opts else None, ctypes.byref(n)))
    return n.value


def gdn_get_workspace_layout(q, k, v, cu_seqlens=None,
                             opts: Optional[GdnOptions] = None) -> GdnWorkspaceLayout:
    lay = GdnWorkspaceLayout()
    ds = [describe(x) for x in (q, k, v, cu_seqlens)]
    _check(lib().gdn_get_workspace_layout(*[_ref(d) for d in ds],
                                          ctypes.byref(opts) if opts else None,
                                          ctypes.byref(lay)))
    return lay


def alloc_workspace(q, k, v, cu_seqlens=None, opts=None) -> torch.Tensor:
    """A device byte tensor large enough for gdn_prefill_ex (torch's caching
    allocator returns 256-byte aligned blocks)."""
    n = gdn_workspace_size(q, k, v, cu_seqlens, opts)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def gdn_prefill_ex(q, k, v, g, beta, cu_seqlens=None, init_state=None,
                   out=None, final_state=None, opts: Optional[GdnOptions] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Prefill with options and a caller-owned workspace (allocated here with
    torch if None).  Returns (out, final_state)."""
    if out is None:
        out = torch.empty_like(v)
    own_ws = workspace is None
    if own_ws:
        workspace = alloc_workspace(q, k, v, cu_seqlens, opts)
    if workspace.device.type != "cuda":
        raise ValueError("workspace must be a GPU tensor")
    ds = _descs(q, k, v, g, beta, cu_seqlens, init_state, out, final_state)
    handle = _stream_handle(stream, v)
    _check(lib().gdn_prefill_ex(*[_ref(d) for d in ds],
                                ctypes.byref(opts) if opts else None,
                                workspace.data_ptr(), workspace.numel(), handle))
    if own_ws and stream is not None:
        # the temporary workspace came from the current stream's pool while
        # the kernels run on ``stream``: keep the block from being handed out
        # again before that stream has finished with it
        workspace.record_stream(_torch_stream(stream, v.device))
    return out, final_state


NOALLOC_SCRATCH_BYTES = 96 << 20


def gdn_prefill_noalloc(q, k, v, g, beta, cu_seqlens=None, init_state=None,
                        out=None, final_state=None, opts: Optional[GdnOptions] = None,
                        stream=None):
    """gdn_prefill_ex on the library's static device scratch: no allocation
    by the library (``out`` must be given).  Calls that overlap on one GPU
    share the scratch and must be serialised.  Returns (out, final_state)."""
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    ds = _descs(q, k, v, g, beta, cu_seqlens, init_state, out, final_state)
    _check(lib().gdn_prefill_noalloc(*[_ref(d) for d in ds],
                                     ctypes.byref(opts) if opts else None,
                                     _stream_handle(stream, v)))
    return out, final_state


def gdn_output_gate(x, z, weight=None, eps: float = 1e-6, out=None, stream=None):
    """out = x / sqrt(mean(x^2) + eps) * weight * silu(z) over the last axis
    (x, z, out [R, dv] or [T, H, dv], one dtype; out may be x).  Returns out."""
    if out is None:
        out = torch.empty_like(x)
    for name, t in (("x", x), ("z", z), ("out", out)):
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    w = _dev_ptr(weight, "weight")
    ds = [describe(t) for t in (x, z, out)]
    _check(lib().gdn_output_gate(_ref(ds[0]), _ref(ds[1]), w, ctypes.c_float(eps), _ref(ds[2]),
                                 _stream_handle(stream, x)))
    return out


def gdn_check_cu_seqlens(cu, t_total: int) -> None:
    """Checks a host copy of cu_seqlens (int32, N + 1 entries) against the
    prefill's preconditions; raises GdnError (GDN_ERR_INPUT) naming the
    first bad entry."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(cu.cpu() if hasattr(cu, "cpu") else cu, dtype=np.int32))
    if a.ndim != 1:
        raise ValueError("cu_seqlens must be 1-D")
    _check(lib().gdn_check_cu_seqlens(a.ctypes.data if a.size else None, a.size - 1, int(t_total)))


def gdn_decode(q, k, v, g, beta, state, out=None, opts: Optional[GdnOptions] = None,
               stream=None):
    """One recurrent step per sequence on ``state`` (updated in place).
    q, k [N, Hk, dk]; v [N, Hv, dv]; g, beta [N, Hv]; state [N, Hv, dk, dv]
    f32.  Returns out [N, Hv, dv]."""
    if out is None:
        out = torch.empty_like(v)
    ts = (q, k, v, g, beta, state, out)
    for name, t in zip(("q", "k", "v", "g", "beta", "state", "out"), ts):
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    ds = [describe(x) for x in ts]
    _check(lib().gdn_decode(*[_ref(d) for d in ds], ctypes.byref(opts) if opts else None,
                            _stream_handle(stream, v)))
    return out


class GraphCache:
    """A gdn_graph_cache: captured replays of gdn_prefill_ex, found by its
    shapes and options and then by its buffers (new buffers of a stored
    shape update a stored graph in place; see include/gdn.h).  ``prefill``
    takes the arguments of gdn_prefill_ex; the workspace is required.
    ``stats`` counts hits, misses (new graphs), updates and fallbacks."""

    def __init__(self, capacity: int = 64):
        self._h = ctypes.c_void_p()
        self._lib = lib()
        _check(self._lib.gdn_graph_cache_create(capacity, ctypes.byref(self._h)))

    def prefill(self, q, k, v, g, beta, cu_seqlens=None, init_state=None, out=None,
                final_state=None, opts: Optional[GdnOptions] = None,
                workspace: Optional[torch.Tensor] = None, stream=None):
        if out is None:
            raise ValueError("out is required (it is part of the captured launches)")
        if workspace is None or workspace.device.type != "cuda":
            raise ValueError("a GPU workspace is required")
        ds = _descs(q, k, v, g, beta, cu_seqlens, init_state, out, final_state)
        _check(self._lib.gdn_prefill_graph(self._h, *[_ref(d) for d in ds],
                                           ctypes.byref(opts) if opts else None,
                                           workspace.data_ptr(), workspace.numel(),
                                           _stream_handle(stream, v)))
        return out, final_state

    def stats(self) -> dict:
        n, h, m, u, f = (ctypes.c_int(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(),
                         ctypes.c_int64())
        _check(self._lib.gdn_graph_cache_stats(self._h, ctypes.byref(n), ctypes.byref(h),
                                               ctypes.byref(m), ctypes.byref(u), ctypes.byref(f)))
        return {"entries": n.value, "hits": h.value, "misses": m.value, "updates": u.value,
                "fallbacks": f.value}

    def clear(self):
        self._lib.gdn_graph_cache_clear(self._h)

    def close(self):
        if self._h:
            self._lib.gdn_graph_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PreparedPrefill:
    """gdn_prefill_ex with its descriptors built once, for tight loops
    (benchmarks, repeated calls on fixed buffers).  Calling it enqueues the
    selected stages on the given stream (default: current) and raises on a
    non-zero status.  The tensors must stay alive as long as this object."""

    def __init__(self, q, k, v, g, beta, cu_seqlens=None, init_state=None,
                 out=None, final_state=None, opts: Optional[GdnOptions] = None,
                 workspace: Optional[torch.Tensor] = None):
        if out is None:
            out = torch.empty_like(v)
        if workspace is None:
            workspace = alloc_workspace(q, k, v, cu_seqlens, opts)
        self.tensors = (q, k, v, g, beta, cu_seqlens, init_state, out, final_state, workspace)
        self.out, self.final_state, self.workspace = out, final_state, workspace
        self._d = _descs(q, k, v, g, beta, cu_seqlens, init_state, out, final_state)
        self._refs = [_ref(d) for d in self._d]
        self._opts = opts if opts is not None else gdn_default_options()
        self._fn = lib().gdn_prefill_ex
        self._ws = (workspace.data_ptr(), workspace.numel())
        self._dev = v.device

    def with_stages(self, stages: int) -> "PreparedPrefill":
        o = GdnOptions.from_buffer_copy(self._opts)
        o.stages = stages
        p = object.__new__(PreparedPrefill)
        p.__dict__.update(self.__dict__)
        p._opts = o
        return p

    def __call__(self, stream=None):
        s = torch.cuda.current_stream(self._dev).cuda_stream if stream is None else stream
        rc = self._fn(*self._refs, ctypes.byref(self._opts), self._ws[0], self._ws[1], s)
        if rc != GDN_OK:
            _check(rc)
