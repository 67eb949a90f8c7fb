"""The C-ABI library: it loads, exports every symbol include/kda.h declares,
and validates arguments on the host before touching the device (no GPU needed)."""

import ctypes
import os
import re
import subprocess

import pytest

from kda_chunked_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def header_symbols():
    import glob
    text = "".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    return sorted(set(re.findall(r"^\S.*?\b(kda_[a-z_]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert header_symbols() == sorted(B.EXPORTS)


def test_library_exports_every_header_symbol():
    lib = B.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(kda_[a-z_]+)$", out, flags=re.M))
    for sym in header_symbols():
        assert sym in exported, sym
        assert getattr(lib, sym) is not None
    assert lib.kda_abi_version() == 1


def test_library_is_built_for_gfx950_only(tmp_path):
    fatbin = tmp_path / "fatbin.bin"
    # objcopy with one file argument rewrites that file: always name the output
    r = subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", B.LIB_PATH,
                        str(fatbin)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("objcopy cannot extract the device code section here")
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          f"--input={fatbin}"], capture_output=True, text=True, check=True)
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets and all("gfx950" in t for t in targets)


def _p(**kw):
    base = dict(T=1000, H=4, num_seqs=2, gate="g", l2norm=False)
    base.update(kw)
    return B.problem(**base)


def test_sizes():
    p = _p()
    nc = 1000 // 64 + 2
    s = B.saved_bytes(p)
    assert s >= nc * 4 * 128 * 128 * 4 + 3 * nc * 4 * 64 * 64 * 4
    assert B.workspace_bytes(p, True, True) > B.workspace_bytes(p, True, False)
    assert B.workspace_bytes(p, False) > 0
    # a saving forward keeps its per-chunk set in `saved`, not in the workspace
    assert B.workspace_bytes(p, False, True) >= B.workspace_bytes(p, False, False) + s
    wide = _p(T=1000, H=64)          # enough chains: one per document, no segment buffers
    assert B.workspace_bytes(wide, False, False) < 4096
    # few chains (2 documents x 4 heads): 64-chunk documents are cut into
    # segments of 16 chunks, whose summaries need two 128 x 128 fp32 buffers
    seg = _p(T=8192, H=4)
    ns = (8192 // 64 + 2) // 16 + 2
    assert B.workspace_bytes(seg, False, False) >= 2 * ns * 4 * 128 * 128 * 4
    # documents averaging fewer than two segments are not cut
    assert B.workspace_bytes(_p(T=3548, H=4), False, False) < 4096
    # invalid problems size to zero
    assert B.saved_bytes(_p(H=0)) == 0
    assert B.workspace_bytes(_p(dk=64), False) == 0


def _fwd_status(p, **ptrs):
    lib = B.lib()
    args = dict(q=16, k=16, v=16, beta=16, g=16, A_log=None, dt_bias=None, cu=16, o=16,
                saved=None, ws=16, ws_bytes=1 << 40)
    args.update(ptrs)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    rc = lib.kda_fwd(ctypes.byref(p), vp(args["q"]), vp(args["k"]), vp(args["v"]),
                     vp(args["beta"]), vp(args["g"]), vp(args["A_log"]), vp(args["dt_bias"]),
                     vp(args["cu"]), vp(args["o"]), vp(args["saved"]), vp(args["ws"]),
                     args["ws_bytes"], None)
    return rc, lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=0), 1, "head"),
    (dict(num_seqs=0), 1, "document"),
    (dict(T=-1), 1, "negative"),
    (dict(dk=64), 2, "128"),
    (dict(dv=256), 2, "128"),
    (dict(H=65536), 2, "65535"),
    (dict(H=65535, num_seqs=1 << 14), 2, "2^29"),
    (dict(T=1 << 30, H=1024), 2, "2^31"),
])
def test_invalid_problem_rejected_before_launch(kw, status, msg):
    rc, err = _fwd_status(_p(**kw))
    assert rc == status and msg in err


def test_null_and_misaligned_pointers_rejected():
    rc, err = _fwd_status(_p(), q=None)
    assert rc == 1 and "q is NULL" in err
    rc, err = _fwd_status(_p(), k=18)
    assert rc == 1 and "aligned" in err
    rc, err = _fwd_status(_p(gate="raw"))
    assert rc == 1 and "A_log" in err


def test_small_workspace_rejected():
    rc, err = _fwd_status(_p(), ws_bytes=100)
    assert rc == 3 and "workspace" in err


def test_zero_tokens_is_a_no_op():
    rc, _ = _fwd_status(_p(T=0), q=None, k=None, v=None)
    assert rc == 0


def test_saving_forward_needs_no_private_set():
    p = _p()
    small = B.workspace_bytes(p, False, False)
    rc, err = _fwd_status(p, saved=16, ws_bytes=small)
    assert rc == 0 or "workspace" not in err
    rc, err = _fwd_status(p, saved=None, ws_bytes=small)
    assert rc == 3 and "workspace" in err


def _bwd_status(p, **ptrs):
    lib = B.lib()
    args = dict(dA_log=16, ddt_bias=16)
    args.update(ptrs)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    rc = lib.kda_bwd(ctypes.byref(p), *([None] * 10), None, None, None, None, None,
                     vp(args["dA_log"]), vp(args["ddt_bias"]), None, 0, None)
    return rc, lib.kda_last_error().decode()


def test_zero_tokens_raw_backward_validates_parameter_gradients():
    """With T == 0 the raw form's dA_log and ddt_bias are zero sums that the
    library writes; their pointers are checked on the host first (the write
    itself needs a GPU and is covered by the GPU tests)."""
    rc, err = _bwd_status(_p(T=0, gate="raw"), dA_log=None)
    assert rc == 1 and "dA_log" in err
    rc, err = _bwd_status(_p(T=0, gate="raw"), ddt_bias=18)
    assert rc == 1 and "ddt_bias" in err
    rc, _ = _bwd_status(_p(T=0, gate="g"), dA_log=None, ddt_bias=None)
    assert rc == 0


def test_status_strings():
    lib = B.lib()
    lib.kda_status_string.restype = ctypes.c_char_p
    assert lib.kda_status_string(0) == b"ok"
    assert lib.kda_status_string(3) == b"workspace too small"


def test_bwd_binding_signature_and_validation():
    """kda_bwd through the Python binding: an invalid problem is rejected on
    the host (so no tensor memory is touched and no GPU is needed)."""
    import torch
    p = B.problem(100, 0, 1)
    t = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(B.KdaError) as e:
        B.kda_bwd(p, t, t, t, t, t, None, None, t, t, None, t, t, t, t, t, None, None, t)
    assert e.value.status == 1 and "head" in str(e.value)
    with pytest.raises(B.KdaError) as e:
        B.kda_fwd(p, t, t, t, t, t, None, None, t, t, None, t)
    assert e.value.status == 1


def test_host_tensors_refused_for_a_valid_problem():
    import torch
    p = B.problem(100, 2, 1)
    t = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        B.kda_fwd(p, t, t, t, t, t, None, None, t, t, None, t)


def _noalloc_status(p, saved=None):
    lib = B.lib()
    vp = lambda x: ctypes.c_void_p(x) if x else None
    rc = lib.kda_fwd_noalloc(ctypes.byref(p), *([vp(16)] * 8), vp(16), vp(saved), None)
    return rc, lib.kda_last_error().decode()


def test_noalloc_forward_rejects_calls_beyond_its_scratch():
    """The no-alloc forward checks its fixed scratch size on the host before it
    looks up the device array or launches anything."""
    big = _p(T=16384, H=4, num_seqs=3)
    assert B.workspace_bytes(big, False, True) > B.NOALLOC_SCRATCH_BYTES
    rc, err = _noalloc_status(big, saved=None)
    assert rc == 3 and "scratch" in err
    rc, err = _noalloc_status(_p(H=0))
    assert rc == 1 and "head" in err
    # with a saved set the workspace is the chunk table and, for few chains,
    # the segment summaries (at most about 112 chain matrices): below the scratch
    assert B.workspace_bytes(big, False, False) < 16 << 20 < B.NOALLOC_SCRATCH_BYTES


# ---------------------------------------------------------------- GQA attention

def _attn(**kw):
    a = dict(Tq=1000, Tk=1500, num_seqs=3, Hq=24, Hkv=4, D=256, scale=None)
    a.update(kw)
    return B.attn_problem(**a)


def _attn_bwd_status(p, form=0, ws_bytes=1 << 30, dst_rows=0, **ptrs):
    base = dict(q=256, k=512, v=768, cu_q=1024, cu_k=1280, o=1536, lse=1792, dO=2048, dq=2304,
                dk=2560, dv=2816, row_map=3072, ws=4096)
    base.update(ptrs)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = B.lib().kda_attn_bwd(ctypes.byref(p), *(vp(base[n]) for n in (
        "q", "k", "v", "cu_q", "cu_k", "o", "lse", "dO", "dq", "dk", "dv")), form,
        vp(base["row_map"]), dst_rows, vp(base["ws"]), ws_bytes, None)
    return rc, B.lib().kda_last_error().decode()


def test_attn_workspace_sizes():
    p = _attn()
    fwd, bwd = B.attn_workspace_bytes(p, 0), B.attn_workspace_bytes(p, 1)
    add = B.attn_workspace_bytes(p, 2, 700)
    assert 0 < fwd < bwd < add
    # the row-map form keeps two fp32 windows [Tk, Hkv, 256] and two key arrays
    assert add - bwd >= 2 * 4 * 1500 * 4 * 256 + 2 * 8 * 1500
    assert B.attn_workspace_bytes(p, 3) == 0
    assert B.attn_workspace_bytes(_attn(Hq=6, Hkv=4), 0) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Hq=6, Hkv=4), 1, "multiple"),
    (dict(Hkv=0), 1, "at least one head"),
    (dict(D=128), 2, "256"),
    (dict(num_seqs=0), 1, "num_seqs"),
    (dict(Tq=-1), 1, "Tq"),
    (dict(scale=float("nan")), 1, "scale"),
])
def test_attn_invalid_problem_rejected(kw, status, msg):
    rc, err = _attn_bwd_status(_attn(**kw))
    assert rc == status and msg in err


def test_attn_argument_checks():
    p = _attn()
    rc, err = _attn_bwd_status(p, form=3)
    assert rc == 1 and "dkv_form" in err
    rc, err = _attn_bwd_status(p, dq=None)
    assert rc == 1 and "dq is NULL" in err
    rc, err = _attn_bwd_status(p, form=2, dst_rows=10, row_map=None)
    assert rc == 1 and "dkv_row_map" in err
    rc, err = _attn_bwd_status(p, form=2, dst_rows=-1)
    assert rc == 1 and "dkv_dst_rows" in err
    rc, err = _attn_bwd_status(p, k=520)
    assert rc == 1 and "aligned" in err
    rc, err = _attn_bwd_status(p, ws_bytes=B.attn_workspace_bytes(p, 1) - 1)
    assert rc == 3
    rc, err = _attn_bwd_status(p, form=2, dst_rows=10, ws_bytes=B.attn_workspace_bytes(p, 1))
    assert rc == 3
    # nothing to do: no launch, no pointer needed
    rc, _ = _attn_bwd_status(_attn(Tq=0, Tk=0), q=None, k=None, v=None, ws=None)
    assert rc == 0


def test_attn_fwd_binding_signature():
    p = _attn(D=64)
    vp = ctypes.c_void_p
    rc = B.lib().kda_attn_fwd(ctypes.byref(p), *(vp(256 * i) for i in range(1, 9)), 1 << 20, None)
    assert rc == 2 and "256" in B.lib().kda_last_error().decode()
    with pytest.raises(ValueError):     # host tensors for a valid problem
        import torch
        t = torch.zeros(16, dtype=torch.uint8)
        B.attn_fwd(_attn(), t, t, t, t, t, t, None, t)


def test_state_entry_points_validate_on_the_host():
    """The boundary-state calls of a sequence split over ranks reject bad
    arguments before anything is enqueued (no GPU needed for these paths)."""
    lib = B.lib()
    vp = lambda x: ctypes.c_void_p(x) if x else None
    err = lambda: lib.kda_last_error().decode()
    # kda_state_apply: head count, transpose flag, pointers
    assert lib.kda_state_apply(0, vp(16), 0, None, vp(16), vp(16), None) == 1 and "H" in err()
    assert lib.kda_state_apply(65536, vp(16), 0, None, vp(16), vp(16), None) == 1
    assert lib.kda_state_apply(2, vp(16), 2, None, vp(16), vp(16), None) == 1
    assert "transpose" in err()
    assert lib.kda_state_apply(2, None, 0, None, vp(16), vp(16), None) == 1 and "M is NULL" in err()
    assert lib.kda_state_apply(2, vp(16), 1, vp(24), vp(16), vp(16), None) == 1
    assert "B is not 16-byte aligned" in err()
    # kda_state_summary / kda_state_grad_summary: problem, outputs, workspace
    assert B.state_summary_workspace_bytes(_p(H=0)) == 0
    assert B.state_summary_workspace_bytes(_p()) > 0
    ptrs = [vp(16)] * 8
    summ = lambda p, *a: lib.kda_state_summary(ctypes.byref(p), *a)
    assert summ(_p(H=0), *ptrs, vp(16), vp(16), None, vp(16), 1 << 40, None) == 1
    assert summ(_p(), *ptrs, vp(20), None, None, vp(16), 1 << 40, None) == 1
    assert "M is not 16-byte aligned" in err()
    assert summ(_p(), *ptrs, vp(16), vp(16), None, vp(16), 100, None) == 3 and "workspace" in err()
    assert summ(_p(), *ptrs, vp(16), vp(16), vp(40), vp(16), 100, None) == 1 and "saved" in err()
    rc = summ(_p(), *([vp(16)] * 7), None, vp(16), vp(16), None, vp(16), 1 << 40, None)
    assert rc == 1 and "cu_seqlens is NULL" in err()
    rc = lib.kda_state_grad_summary(ctypes.byref(_p()), *ptrs, vp(16), None, None, vp(16),
                                    1 << 40, None)
    assert rc == 1 and "dB is NULL" in err()
    rc = lib.kda_state_grad_summary(ctypes.byref(_p()), *ptrs, None, None, vp(16), vp(16),
                                    1 << 40, None)
    assert rc == 1 and "dO is NULL" in err()
    rc = lib.kda_state_grad_summary(ctypes.byref(_p()), *ptrs, vp(16), vp(24), vp(16), vp(16),
                                    1 << 40, None)
    assert rc == 1 and "saved" in err()
    rc = lib.kda_state_grad_summary(ctypes.byref(_p()), *ptrs, vp(16), None, vp(16), vp(16), 64,
                                    None)
    assert rc == 3 and "workspace" in err()
    # kda_fwd_state / kda_bwd_state: the boundary states' alignment
    fs = lambda *a: lib.kda_fwd_state(ctypes.byref(_p()), *ptrs, *a)
    assert fs(vp(40), vp(16), vp(16), vp(16), 0, vp(16), 1 << 40, None) == 1 and "s_init" in err()
    assert fs(None, vp(16), vp(20), vp(16), 0, vp(16), 1 << 40, None) == 1 and "s_final" in err()
    assert fs(None, vp(16), None, vp(16), 4, vp(16), 1 << 40, None) == 1 and "flags" in err()
    assert fs(None, vp(16), None, None, 1, vp(16), 1 << 40, None) == 1 and "saved" in err()
    bw = [vp(16)] * 8
    rc = lib.kda_bwd_state(ctypes.byref(_p()), *bw, None, vp(16), vp(36), None, *([vp(16)] * 7),
                           None, vp(16), 1 << 40, None)
    assert rc == 1 and "ds_final" in err()
    rc = lib.kda_bwd_state(ctypes.byref(_p()), *bw, None, vp(16), None, None, *([vp(16)] * 7),
                           vp(52), vp(16), 1 << 40, None)
    assert rc == 1 and "ds_init" in err()
