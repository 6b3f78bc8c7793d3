"""ctypes wrapper of the fp64 C oracle (gdn_ref.c): the form-1 recurrence
for every (sequence, V head), one thread per pair.

TEST INFRASTRUCTURE ONLY (see the package docstring). Same arguments,
readings and results as gdn_oracle.recurrent_form1; it exists so that
full-size workloads can be checked against the recurrence in seconds.
build() compiles gdn_ref.c with gcc next to this file; load() builds it when
no library is there yet.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdn_ref.c")
LIBRARY = os.path.join(HERE, "libgdn_ref.so")

_lib = None


def build(verbose=False):
    """Compile gdn_ref.c into libgdn_ref.so (always); returns its path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the oracle")
    tmp = LIBRARY + ".tmp"
    cmd = [cc, "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-o", tmp, SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        lib = ctypes.CDLL(LIBRARY)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.gdn_ref_form1.argtypes = [i64, i64, p, i64, i64, i64, i64, p, p, p, p, p, p, p, p, ctypes.c_int]
        lib.gdn_ref_form1.restype = ctypes.c_int
        lib.gdn_ref_max_threads.argtypes = []
        lib.gdn_ref_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads():
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def recurrent_form1(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, threads=None):
    """Form-1 recurrence with readout o_t = S_t^T q_t (post-update state).

    q, k [T, Hqk, dk]; v [T, Hv, dv]; log_alpha, beta [T, Hv]: any real
    arrays whose values are float32 numbers (bfloat16 and float32 inputs
    are; they are passed as float32, exactly). init_state [N, Hv, dk, dv]
    or None; cu_seqlens [N + 1] or None. Returns float64
    (o [T, Hv, dv], final_state [N, Hv, dk, dv]).
    """
    lib = load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    la, b = _f32(log_alpha), _f32(beta)
    T, h_qk, dk = q.shape
    h_v, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or la.shape != (T, h_v) or b.shape != (T, h_v):
        raise ValueError("inconsistent shapes")
    cu = None if cu_seqlens is None else np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = 1 if cu is None else len(cu) - 1
    init = None
    if init_state is not None:
        init = np.ascontiguousarray(np.asarray(init_state, dtype=np.float64).reshape(n, h_v, dk, dv))
    o = np.empty((T, h_v, dv))
    final = np.empty((n, h_v, dk, dv))
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    rc = lib.gdn_ref_form1(T, n, ptr(cu), h_qk, h_v, dk, dv, ptr(q), ptr(k), ptr(v), ptr(la), ptr(b),
                           ptr(init), ptr(o), ptr(final), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("gdn_ref_form1 rejected its arguments")
    return o, final


def decode_steps(state0, q, k, v, log_alpha, beta, threads=None):
    """Successive single-token steps for a batch: inputs stacked by step,
    q, k [K, N, Hqk, dk]; v [K, N, Hv, dv]; log_alpha, beta [K, N, Hv];
    state0 [N, Hv, dk, dv]. Each sequence's K tokens are its own sequence
    of the recurrence. Returns (o [K, N, Hv, dv], state after step K)."""
    K, N = np.shape(q)[:2]
    per_seq = lambda x: np.swapaxes(np.asarray(x), 0, 1).reshape((N * K,) + np.shape(x)[2:])  # noqa: E731
    cu = np.arange(0, N * K + 1, K)
    o, final = recurrent_form1(per_seq(q), per_seq(k), per_seq(v), per_seq(log_alpha), per_seq(beta),
                               state0, cu, threads)
    return np.swapaxes(o.reshape((N, K) + o.shape[1:]), 0, 1), final
