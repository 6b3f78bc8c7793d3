"""C ABI host-side checks that need no GPU: the library loads, exports every
function include/gdn.h declares, and rejects bad arguments with the
documented status before enqueuing anything. Every call here fails
validation, so none of them reaches a kernel launch on any machine."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_recurrence_delta_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

INVALID, NOT_SUPPORTED, WORKSPACE = 1, 2, 3
FAKE = 0x10000  # a 256-aligned non-null address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIBRARY_PATH):
        pytest.skip("libgdn.so not built")
    return B.load_library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(gdn_\w+)\(", text, re.M)))


def test_header_declares_expected_functions():
    assert header_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIBRARY_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(gdn_\w+)$", out, re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def dims(**kw):
    base = dict(num_seqs=1, total_tokens=128, h_qk=16, h_v=48, dk=128, dv=128, chunk=64,
                dtype=1, flags=0)
    base.update(kw)
    return B.GdnDims(*[base[f] for f, _ in B.GdnDims._fields_])


def ws_bytes(lib, d):
    return lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(d))


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=0), INVALID),
    (dict(total_tokens=-1), INVALID),
    (dict(h_qk=0), INVALID),
    (dict(h_v=47), INVALID),                # not a multiple of h_qk
    (dict(dk=0), INVALID),
    (dict(dtype=7), INVALID),
    (dict(chunk=0), INVALID),
    (dict(dk=64, dv=64), NOT_SUPPORTED),
    (dict(dk=128, dv=64), NOT_SUPPORTED),
    (dict(chunk=32), NOT_SUPPORTED),
    (dict(flags=4), INVALID),                # unknown flag
    (dict(flags=-1), INVALID),
])
def test_dims_validation(lib, kw, status):
    d = dims(**kw)
    assert ws_bytes(lib, d) == 0
    lay = B.GdnWorkspaceLayout()
    assert lib.gdn_chunk_fwd_workspace_layout(ctypes.byref(d), ctypes.byref(lay)) == status
    assert lib.gdn_last_error_message().decode() != ""


def test_workspace_size_formula(lib):
    # regions: chunk table, sequence offsets, gate prefixes, per-chunk b,
    # Tinv diag(b) and W fragments (per V head), K^T and Q fragments (per
    # QK head), masked q.k fragments and row factors (per V head); each
    # padded to 256 bytes. Fragments of a C x C tile take C*C elements, of a
    # D x C tile D*C elements (C = 64 is a whole number of 32-steps).
    d = dims(num_seqs=3, total_tokens=1000)
    nc = 1000 // 64 + 3
    def up(x):
        return (x + 255) // 256 * 256
    want = (up(nc * 16) + up(4 * 4) + 2 * up(nc * 48 * 64 * 4) + up(nc * 48 * 64 * 64 * 2)
            + up(nc * 48 * 64 * 128 * 2) + up(nc * 16 * 128 * 64 * 2) + up(nc * 16 * 64 * 128 * 2) + up(nc * 48 * 64 * 64 * 2) + up(nc * 48 * (2 * 64 + 4) * 4))
    assert ws_bytes(lib, d) == want
    lay = B.GdnWorkspaceLayout()
    assert lib.gdn_chunk_fwd_workspace_layout(ctypes.byref(d), ctypes.byref(lay)) == 0
    assert lay.total == want and lay.max_chunks == nc
    offs = [lay.chunk_table, lay.seq_chunk_offset, lay.gate_prefix, lay.beta_chunk, lay.tinv,
            lay.w, lay.key_t, lay.q_frag, lay.pmask, lay.dtab]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)


def call_fwd(lib, d, q=FAKE, k=FAKE, v=FAKE, la=FAKE, b=FAKE, init=None, cu=None, o=FAKE * 2,
             fin=None, ws=FAKE * 4, wsb=None):
    if wsb is None:
        wsb = ws_bytes(lib, d) if ws_bytes(lib, d) else 1 << 40
    vp = ctypes.c_void_p
    return lib.gdn_chunk_fwd(ctypes.byref(d), vp(q), vp(k), vp(v), vp(la), vp(b), vp(init),
                             vp(cu), vp(o), vp(fin), vp(ws), wsb, None)


def test_fwd_rejects_bad_pointers(lib):
    d = dims()
    assert call_fwd(lib, d, q=None) == INVALID
    assert "q is NULL" in lib.gdn_last_error_message().decode()
    assert call_fwd(lib, d, v=FAKE + 8) == INVALID               # 16-byte alignment
    assert call_fwd(lib, d, la=FAKE + 2) == INVALID              # 4-byte alignment
    assert call_fwd(lib, d, o=FAKE) == INVALID                   # o aliases q
    assert call_fwd(lib, d, init=FAKE + 4) == INVALID
    assert call_fwd(lib, d, fin=FAKE + 4) == INVALID
    assert call_fwd(lib, dims(num_seqs=2), cu=None) == INVALID   # N > 1 needs cu_seqlens
    assert call_fwd(lib, dims(num_seqs=2), cu=FAKE + 2) == INVALID


def test_fwd_rejects_bad_workspace(lib):
    d = dims()
    need = ws_bytes(lib, d)
    assert call_fwd(lib, d, ws=None) == WORKSPACE
    assert call_fwd(lib, d, ws=FAKE * 4 + 16) == WORKSPACE       # 256-byte alignment
    assert call_fwd(lib, d, wsb=need - 1) == WORKSPACE
    assert "needed" in lib.gdn_last_error_message().decode()


def test_fwd_rejects_unsupported(lib):
    assert call_fwd(lib, dims(dk=64, dv=64)) == NOT_SUPPORTED
    assert call_fwd(lib, dims(chunk=128)) == NOT_SUPPORTED
    assert ws_bytes(lib, dims(dtype=0)) > 0                       # fp32 at head dim 128, chunk 64
    assert ws_bytes(lib, dims(dtype=0, chunk=16)) > 0
    assert ws_bytes(lib, dims(dtype=0, dk=16, dv=16)) > 0


def test_stage_range_validation(lib):
    d = dims()
    vp = ctypes.c_void_p
    for first, last in ((0, 2), (1, 3), (2, 1)):
        st = lib.gdn_chunk_fwd_stages(ctypes.byref(d), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                      vp(FAKE), None, None, vp(FAKE * 2), None, vp(FAKE * 4),
                                      ws_bytes(lib, d), None, first, last)
        assert st == INVALID


def test_decode_validation(lib):
    vp = ctypes.c_void_p
    def call(d, q=FAKE, k=FAKE, v=FAKE, la=FAKE, b=FAKE, s=FAKE * 8, o=FAKE * 2):
        return lib.gdn_decode_step(ctypes.byref(d), vp(q), vp(k), vp(v), vp(la), vp(b), vp(s),
                                   vp(o), None)
    d = dims(num_seqs=4, total_tokens=4)
    assert call(dims(num_seqs=4, total_tokens=5)) == INVALID
    assert call(d, s=None) == INVALID
    assert call(d, s=FAKE * 8 + 4) == INVALID
    assert call(d, o=FAKE * 8) == INVALID                        # o aliases state
    assert call(dims(num_seqs=4, total_tokens=4, dk=32, dv=32)) == NOT_SUPPORTED


def test_decode_multi_validation(lib):
    vp = ctypes.c_void_p
    def call(d, kt=3, q=FAKE, k=FAKE, v=FAKE, la=FAKE, b=FAKE, s=FAKE * 8, o=FAKE * 2, snap=None):
        return lib.gdn_decode_multi(ctypes.byref(d), kt, vp(q), vp(k), vp(v), vp(la), vp(b), vp(s),
                                    vp(o), vp(snap), None)
    d = dims(num_seqs=4, total_tokens=4)
    assert call(d, kt=0) == INVALID
    assert "num_tokens" in lib.gdn_last_error_message().decode()
    assert call(d, kt=-2) == INVALID
    assert call(dims(num_seqs=4, total_tokens=5)) == INVALID
    assert call(d, v=None) == INVALID
    assert call(d, s=FAKE * 8 + 4) == INVALID
    assert call(d, o=FAKE * 8) == INVALID                        # o aliases state
    assert call(d, snap=FAKE * 8) == INVALID                     # snapshots alias state
    assert call(d, snap=FAKE * 16, o=FAKE * 16) == INVALID       # o aliases snapshots
    assert call(d, snap=FAKE * 16 + 8) == INVALID                # misaligned snapshots
    assert call(dims(num_seqs=4, total_tokens=4, dk=32, dv=32)) == NOT_SUPPORTED
    assert call(dims(num_seqs=1 << 20, total_tokens=1 << 20), kt=1 << 12) == NOT_SUPPORTED


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_flags_are_accepted_and_keep_the_workspace(lib, flags):
    assert B.GDN_FLAG_PREPARE_INPUTS == 1 and B.GDN_FLAG_NO_DELTA_RULE == 2
    d = dims(flags=flags)
    assert ws_bytes(lib, d) == ws_bytes(lib, dims())
    assert ctypes.sizeof(B.GdnDims) == 48


def test_header_flag_values_match_the_binding():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    assert re.search(r"GDN_FLAG_PREPARE_INPUTS = 1\b", text)
    assert re.search(r"GDN_FLAG_NO_DELTA_RULE = 2\b", text)


def test_status_strings(lib):
    for code, name in B.STATUS.items():
        assert lib.gdn_status_string(code).decode() == name


# --- backward pass ---------------------------------------------------------

def bwd_bytes(lib, d):
    return lib.gdn_chunk_bwd_workspace_bytes(ctypes.byref(d))


def call_bwd(lib, d, q=FAKE, k=FAKE, v=FAKE, la=FAKE, b=FAKE, init=None, cu=None, do=FAKE * 3,
             dfin=None, dq=FAKE * 5, dk=FAKE * 6, dv=FAKE * 7, dla=FAKE * 9, db=FAKE * 10, dinit=None,
             ws=FAKE * 12, wsb=None, stages=None):
    if wsb is None:
        wsb = bwd_bytes(lib, d) if bwd_bytes(lib, d) else 1 << 40
    vp = ctypes.c_void_p
    args = [ctypes.byref(d), vp(q), vp(k), vp(v), vp(la), vp(b), vp(init), vp(cu), vp(do), vp(dfin), vp(dq),
            vp(dk), vp(dv), vp(dla), vp(db), vp(dinit), vp(ws), wsb, None]
    if stages is None:
        return lib.gdn_chunk_bwd(*args)
    return lib.gdn_chunk_bwd_stages(*args, *stages)


def test_bwd_workspace_size_formula(lib):
    # the forward workspace, then K, Q^T, query-indexed q.k fragments (per QK
    # head), P^T, W^T fragments, Tinv^T, the chunk-start states, U, dS_end
    # and dU (per V head), each padded to 256 bytes
    d = dims(num_seqs=3, total_tokens=1000)
    nc = 1000 // 64 + 3
    def up(x):
        return (x + 255) // 256 * 256
    want = (ws_bytes(lib, d) + up(nc * 16 * 64 * 128 * 2) + up(nc * 16 * 128 * 64 * 2) + up(nc * 16 * 64 * 64 * 2)
            + up(nc * 48 * 64 * 64 * 2) + up(nc * 48 * 128 * 64 * 2) + up(nc * 48 * 64 * 64 * 2)
            + up(nc * 48 * 128 * 128 * 2) + up(nc * 48 * 64 * 128 * 2) + up(nc * 48 * 128 * 128 * 2)
            + up(nc * 48 * 64 * 128 * 2))
    assert bwd_bytes(lib, d) == want


def test_bwd_rejects_flags_and_bad_arguments(lib):
    d = dims()
    for flags in (1, 2, 3):
        assert bwd_bytes(lib, dims(flags=flags)) == 0
        assert call_bwd(lib, dims(flags=flags), wsb=1 << 40) == NOT_SUPPORTED
    assert call_bwd(lib, d, do=None) == INVALID
    assert "d_o is NULL" in lib.gdn_last_error_message().decode()
    assert call_bwd(lib, d, dla=FAKE * 9 + 2) == INVALID          # 4-byte alignment
    assert call_bwd(lib, d, dq=FAKE) == INVALID                   # dq aliases q
    assert call_bwd(lib, d, dv=FAKE * 5) == INVALID               # dv aliases dq
    assert call_bwd(lib, d, db=FAKE * 3) == INVALID               # dbeta aliases d_o
    assert call_bwd(lib, d, init=FAKE * 14, dinit=FAKE * 14) == INVALID
    assert call_bwd(lib, d, dfin=FAKE * 14 + 4) == INVALID
    assert call_bwd(lib, dims(num_seqs=2), cu=None) == INVALID
    assert call_bwd(lib, d, ws=None) == WORKSPACE
    assert call_bwd(lib, d, wsb=bwd_bytes(lib, d) - 1) == WORKSPACE
    assert call_bwd(lib, dims(dtype=0)) == NOT_SUPPORTED          # fp32 at head dim 128 needs chunk 16
    assert bwd_bytes(lib, dims(dtype=0)) == 0
    assert bwd_bytes(lib, dims(dtype=0, chunk=16)) > 0
    for st in ((0, 5), (1, 6), (4, 3)):
        assert call_bwd(lib, d, stages=st) == INVALID


# --- the host code under AddressSanitizer and UndefinedBehaviorSanitizer ----

def test_abi_host_code_under_sanitizers(tmp_path):
    """gdn_api.cpp built with g++ -fsanitize=address,undefined against host
    stand-ins of the HIP calls and launchers (tests/host_asan), driven through
    every entry point: validation, workspace carving, the launch arguments,
    GDN_DEBUG's cu_seqlens check and GDN_DEBUG_SYNC. No GPU involved."""
    import shutil
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    here = os.path.join(ROOT, "tests", "host_asan")
    csrc = os.path.join(ROOT, "linear_attention_recurrence_delta_amd", "csrc")
    exe = str(tmp_path / "abi_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", csrc, "-I", here, "-I", "/opt/rocm/include", os.path.join(csrc, "gdn_api.cpp"),
           os.path.join(here, "hip_stub.cpp"), os.path.join(here, "abi_driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode and "asan" in build.stderr.lower() and "cannot find" in build.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr[-3000:]
    # (verify_asan_link_order=0: a library that the environment preloads may
    # come before the sanitizer runtime; it is left in place)
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("GDN_DEBUG", None)
    env.pop("GDN_DEBUG_SYNC", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-3000:]
    assert "checks ok" in run.stdout
