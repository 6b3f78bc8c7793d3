"""ctypes binding of libgdn (include/gdn.h).

Argument marshalling only: shape/dtype/device checks, output allocation with
torch, and passing data pointers plus torch's current HIP stream to the C
ABI. Every step of the computation runs in the library's HIP kernels; there
is no fallback. If libgdn.so is missing the first call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libgdn.so")

GDN_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "GDN_SUCCESS", 1: "GDN_ERROR_INVALID_VALUE", 2: "GDN_ERROR_NOT_SUPPORTED",
          3: "GDN_ERROR_WORKSPACE", 4: "GDN_ERROR_HIP"}

# Names the library must export (every function declared in include/gdn.h).
EXPORTS = ("gdn_chunk_fwd", "gdn_chunk_fwd_stages", "gdn_chunk_fwd_workspace_bytes",
           "gdn_chunk_bwd", "gdn_chunk_bwd_stages", "gdn_chunk_bwd_workspace_bytes",
           "gdn_decode_step", "gdn_decode_multi", "gdn_status_string", "gdn_last_error_message",
           "gdn_chunk_fwd_workspace_layout", "gdn_chunk_fwd_noalloc")

# GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h
NOALLOC_SCRATCH_BYTES = 128 << 20


class GdnDims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int64), ("total_tokens", ctypes.c_int64),
                ("h_qk", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class GdnWorkspaceLayout(ctypes.Structure):
    _fields_ = [("chunk_table", ctypes.c_size_t), ("seq_chunk_offset", ctypes.c_size_t),
                ("gate_prefix", ctypes.c_size_t), ("beta_chunk", ctypes.c_size_t),
                ("tinv", ctypes.c_size_t), ("w", ctypes.c_size_t), ("key_t", ctypes.c_size_t),
                ("q_frag", ctypes.c_size_t), ("pmask", ctypes.c_size_t),
                ("dtab", ctypes.c_size_t), ("total", ctypes.c_size_t),
                ("max_chunks", ctypes.c_int64)]


class GdnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path=None):
    """Load libgdn.so (once) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is not built: run `python -m linear_attention_recurrence_delta_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dims_p = ctypes.POINTER(GdnDims)
    lib.gdn_chunk_fwd.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd.restype = i32
    lib.gdn_chunk_fwd_stages.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                         i32, i32]
    lib.gdn_chunk_fwd_stages.restype = i32
    lib.gdn_chunk_fwd_noalloc.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_noalloc.restype = i32
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [dims_p]
    lib.gdn_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_workspace_layout.argtypes = [dims_p, ctypes.POINTER(GdnWorkspaceLayout)]
    lib.gdn_chunk_fwd_workspace_layout.restype = i32
    bwd = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_bwd.argtypes = bwd
    lib.gdn_chunk_bwd.restype = i32
    lib.gdn_chunk_bwd_stages.argtypes = bwd + [i32, i32]
    lib.gdn_chunk_bwd_stages.restype = i32
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [dims_p]
    lib.gdn_chunk_bwd_workspace_bytes.restype = sz
    lib.gdn_decode_step.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_decode_step.restype = i32
    lib.gdn_decode_multi.argtypes = [dims_p, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_decode_multi.restype = i32
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error_message.argtypes = []
    lib.gdn_last_error_message.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status):
    if status != 0:
        msg = load_library().gdn_last_error_message().decode()
        raise GdnError(status, msg)


GDN_FLAG_PREPARE_INPUTS = 1
GDN_FLAG_NO_DELTA_RULE = 2


def _flags(prepare_inputs, delta_rule):
    return (GDN_FLAG_PREPARE_INPUTS if prepare_inputs else 0) | (0 if delta_rule else GDN_FLAG_NO_DELTA_RULE)


def make_dims(num_seqs, total_tokens, h_qk, h_v, dk, dv, chunk, dtype, flags=0):
    code = GDN_DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return GdnDims(int(num_seqs), int(total_tokens), int(h_qk), int(h_v), int(dk), int(dv),
                   int(chunk), code, int(flags))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gdn_chunk_fwd_workspace_bytes(dims):
    n = load_library().gdn_chunk_fwd_workspace_bytes(ctypes.byref(dims))
    if n == 0:
        # the size query has no status; the layout query reports the reason
        gdn_chunk_fwd_workspace_layout(dims)
        raise GdnError(1, load_library().gdn_last_error_message().decode())
    return n


def gdn_chunk_fwd_workspace_layout(dims):
    lay = GdnWorkspaceLayout()
    _check(load_library().gdn_chunk_fwd_workspace_layout(ctypes.byref(dims), ctypes.byref(lay)))
    return lay


def gdn_chunk_fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, chunk=64,
                  output_final_state=True, workspace=None, o=None, final_state=None,
                  stages=None, prepare_inputs=False, delta_rule=True):
    """Prefill through gdn_chunk_fwd. Shapes: q, k [T,Hqk,d]; v [T,Hv,d];
    log_alpha, beta [T,Hv] fp32; init_state [N,Hv,d,d] fp32 or None;
    cu_seqlens int32 [N+1] or None. Returns (o, final_state or None).
    `workspace` (uint8 CUDA tensor) may be passed to reuse scratch memory.
    `stages=(first, last)` calls gdn_chunk_fwd_stages instead (diagnostic).
    `prepare_inputs=True` sets GDN_FLAG_PREPARE_INPUTS: q, k raw and
    log_alpha, beta holding the gate logits. `delta_rule=False` sets
    GDN_FLAG_NO_DELTA_RULE: the gate-only update S = a S + b k v^T."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_fwd needs CUDA (HIP) tensors")
    T, h_qk, d = q.shape
    h_v = v.shape[1]
    n = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    _need(q, "q", dev, shape=(T, h_qk, d))
    _need(k, "k", dev, q.dtype, (T, h_qk, d))
    _need(v, "v", dev, q.dtype, (T, h_v, v.shape[2]))
    _need(log_alpha, "log_alpha", dev, torch.float32, (T, h_v))
    _need(beta, "beta", dev, torch.float32, (T, h_v))
    if init_state is not None:
        _need(init_state, "init_state", dev, torch.float32, (n, h_v, d, v.shape[2]))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dev, torch.int32, (n + 1,))
    if q.dtype not in GDN_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dims = make_dims(n, T, h_qk, h_v, d, v.shape[2], chunk, q.dtype, _flags(prepare_inputs, delta_rule))
    nbytes = gdn_chunk_fwd_workspace_bytes(dims)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", dev, torch.uint8)
    if o is None:
        o = torch.empty_like(v)
    _need(o, "o", dev, v.dtype, tuple(v.shape))
    if output_final_state and final_state is None:
        final_state = torch.empty((n, h_v, d, v.shape[2]), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", dev, torch.float32, (n, h_v, d, v.shape[2]))
    args = (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
            _ptr(init_state), _ptr(cu_seqlens), _ptr(o), _ptr(final_state), _ptr(workspace),
            workspace.numel(), _stream(dev))
    if stages is None:
        _check(lib.gdn_chunk_fwd(*args))
    else:
        _check(lib.gdn_chunk_fwd_stages(*args, int(stages[0]), int(stages[1])))
    return o, final_state


def gdn_chunk_fwd_noalloc(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, chunk=64,
                          output_final_state=True, o=None, final_state=None, prepare_inputs=False,
                          delta_rule=True):
    """Prefill through gdn_chunk_fwd_noalloc: gdn_chunk_fwd with the
    library's own device scratch array as its workspace (no workspace
    argument; the library allocates nothing). Same arguments and results as
    gdn_chunk_fwd otherwise; `o` and `final_state` are allocated here by
    torch when not given."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_fwd_noalloc needs CUDA (HIP) tensors")
    T, h_qk, d = q.shape
    h_v = v.shape[1]
    n = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    _need(q, "q", dev, shape=(T, h_qk, d))
    _need(k, "k", dev, q.dtype, (T, h_qk, d))
    _need(v, "v", dev, q.dtype, (T, h_v, v.shape[2]))
    _need(log_alpha, "log_alpha", dev, torch.float32, (T, h_v))
    _need(beta, "beta", dev, torch.float32, (T, h_v))
    if init_state is not None:
        _need(init_state, "init_state", dev, torch.float32, (n, h_v, d, v.shape[2]))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dev, torch.int32, (n + 1,))
    if q.dtype not in GDN_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dims = make_dims(n, T, h_qk, h_v, d, v.shape[2], chunk, q.dtype, _flags(prepare_inputs, delta_rule))
    if o is None:
        o = torch.empty_like(v)
    _need(o, "o", dev, v.dtype, tuple(v.shape))
    if output_final_state and final_state is None:
        final_state = torch.empty((n, h_v, d, v.shape[2]), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", dev, torch.float32, (n, h_v, d, v.shape[2]))
    _check(lib.gdn_chunk_fwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                     _ptr(init_state), _ptr(cu_seqlens), _ptr(o), _ptr(final_state), _stream(dev)))
    return o, final_state


def gdn_chunk_bwd_workspace_bytes(dims):
    n = load_library().gdn_chunk_bwd_workspace_bytes(ctypes.byref(dims))
    if n == 0:
        raise GdnError(2 if dims.flags else 1, load_library().gdn_last_error_message().decode())
    return n


def gdn_chunk_bwd(q, k, v, log_alpha, beta, d_o, init_state=None, cu_seqlens=None, d_final_state=None,
                  chunk=64, workspace=None, grads=None, stages=None):
    """Backward pass through gdn_chunk_bwd: gradients of a scalar loss given
    d_o = dL/do [T,Hv,d] (dtype of v) and d_final_state = dL/d(final state)
    [N,Hv,d,d] fp32 or None. Other arguments as for gdn_chunk_fwd. Returns a
    dict dq, dk [T,Hqk,d]; dv [T,Hv,d] (input dtype); dlog_alpha, dbeta
    [T,Hv] fp32; d_init_state [N,Hv,d,d] fp32. `grads` (a dict of the same
    tensors) may be passed to reuse outputs; `stages=(first, last)` calls
    gdn_chunk_bwd_stages (diagnostic)."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_bwd needs CUDA (HIP) tensors")
    T, h_qk, d = q.shape
    h_v, dv = v.shape[1], v.shape[2]
    n = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    _need(q, "q", dev, shape=(T, h_qk, d))
    _need(k, "k", dev, q.dtype, (T, h_qk, d))
    _need(v, "v", dev, q.dtype, (T, h_v, dv))
    _need(log_alpha, "log_alpha", dev, torch.float32, (T, h_v))
    _need(beta, "beta", dev, torch.float32, (T, h_v))
    _need(d_o, "d_o", dev, q.dtype, (T, h_v, dv))
    if init_state is not None:
        _need(init_state, "init_state", dev, torch.float32, (n, h_v, d, dv))
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", dev, torch.float32, (n, h_v, d, dv))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dev, torch.int32, (n + 1,))
    if q.dtype not in GDN_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dims = make_dims(n, T, h_qk, h_v, d, dv, chunk, q.dtype)
    nbytes = gdn_chunk_bwd_workspace_bytes(dims)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", dev, torch.uint8)
    if grads is None:
        grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                     dlog_alpha=torch.empty_like(log_alpha), dbeta=torch.empty_like(beta),
                     d_init_state=torch.empty((n, h_v, d, dv), dtype=torch.float32, device=dev))
    for name, ref in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", log_alpha), ("dbeta", beta)):
        _need(grads[name], name, dev, ref.dtype, tuple(ref.shape))
    if grads.get("d_init_state") is not None:
        _need(grads["d_init_state"], "d_init_state", dev, torch.float32, (n, h_v, d, dv))
    args = (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state),
            _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state), _ptr(grads["dq"]), _ptr(grads["dk"]),
            _ptr(grads["dv"]), _ptr(grads["dlog_alpha"]), _ptr(grads["dbeta"]), _ptr(grads.get("d_init_state")),
            _ptr(workspace), workspace.numel(), _stream(dev))
    if stages is None:
        _check(lib.gdn_chunk_bwd(*args))
    else:
        _check(lib.gdn_chunk_bwd_stages(*args, int(stages[0]), int(stages[1])))
    return grads


def gdn_decode_step(q, k, v, log_alpha, beta, state, o=None, prepare_inputs=False, delta_rule=True):
    """One decode step through gdn_decode_step. q, k [N,Hqk,d]; v [N,Hv,d];
    log_alpha, beta [N,Hv] fp32; state [N,Hv,d,d] fp32 (updated in place).
    Returns o [N,Hv,d]. `prepare_inputs`, `delta_rule` as for gdn_chunk_fwd."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_decode_step needs CUDA (HIP) tensors")
    n, h_qk, d = q.shape
    h_v = v.shape[1]
    _need(q, "q", dev)
    _need(k, "k", dev, q.dtype, (n, h_qk, d))
    _need(v, "v", dev, q.dtype, (n, h_v, v.shape[2]))
    _need(log_alpha, "log_alpha", dev, torch.float32, (n, h_v))
    _need(beta, "beta", dev, torch.float32, (n, h_v))
    _need(state, "state", dev, torch.float32, (n, h_v, d, v.shape[2]))
    if q.dtype not in GDN_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if o is None:
        o = torch.empty_like(v)
    _need(o, "o", dev, v.dtype, tuple(v.shape))
    dims = make_dims(n, n, h_qk, h_v, d, v.shape[2], 0, q.dtype, _flags(prepare_inputs, delta_rule))
    _check(lib.gdn_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                               _ptr(beta), _ptr(state), _ptr(o), _stream(dev)))
    return o


def gdn_decode_multi(q, k, v, log_alpha, beta, state, o=None, snapshots=None, prepare_inputs=False,
                     delta_rule=True):
    """K drafted tokens per sequence through gdn_decode_multi. q, k [K,N,Hqk,d];
    v [K,N,Hv,d]; log_alpha, beta [K,N,Hv] fp32; state [N,Hv,d,d] fp32.
    With `snapshots` ([K,N,Hv,d,d] fp32) the state after each token goes there
    and `state` is only read; without, `state` ends as the state after all K
    tokens. Returns o [K,N,Hv,d]. `prepare_inputs`, `delta_rule` as for
    gdn_chunk_fwd."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_decode_multi needs CUDA (HIP) tensors")
    kt, n, h_qk, d = q.shape
    h_v, dv = v.shape[2], v.shape[3]
    _need(q, "q", dev)
    _need(k, "k", dev, q.dtype, (kt, n, h_qk, d))
    _need(v, "v", dev, q.dtype, (kt, n, h_v, dv))
    _need(log_alpha, "log_alpha", dev, torch.float32, (kt, n, h_v))
    _need(beta, "beta", dev, torch.float32, (kt, n, h_v))
    _need(state, "state", dev, torch.float32, (n, h_v, d, dv))
    if q.dtype not in GDN_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if o is None:
        o = torch.empty_like(v)
    _need(o, "o", dev, v.dtype, tuple(v.shape))
    if snapshots is not None:
        _need(snapshots, "snapshots", dev, torch.float32, (kt, n, h_v, d, dv))
    dims = make_dims(n, n, h_qk, h_v, d, dv, 0, q.dtype, _flags(prepare_inputs, delta_rule))
    _check(lib.gdn_decode_multi(ctypes.byref(dims), int(kt), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                _ptr(beta), _ptr(state), _ptr(o),
                                _ptr(snapshots) if snapshots is not None else None, _stream(dev)))
    return o
