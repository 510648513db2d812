"""The C ABI loads and validates on the host (no GPU, no compute calls).

Every function declared in include/qsa.h must be exported by libqsa.so, and
every validation rule must return its documented status before any HIP call.
"""
import ctypes
import math
import os
import re

import pytest

import quantized_softmax_approximation_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(qsa.lib_path()), reason="libqsa.so not built")

GOOD = dict(B=1, H=4, Hkv=2, N=100, d=64, causal=1, variant=qsa.POT, k_levels=8, window=0.0, dtype=qsa.DT_BF16)


def v(**kw):
    a = dict(GOOD)
    a.update(kw)
    return qsa.attn_validate(a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["causal"], a["variant"], a["k_levels"],
                             a["window"], a["dtype"])


def test_every_declared_symbol_is_exported():
    src = open(HEADER).read()
    names = re.findall(r"^\s*(?:int|const char\*)\s+(qsa_\w+)\s*\(", src, flags=re.M)
    assert set(names) == {"qsa_attn_fwd", "qsa_attn_fwd_ex", "qsa_attn_bwd", "qsa_attn_validate",
                          "qsa_status_string", "qsa_last_error", "qsa_version"}
    L = ctypes.CDLL(qsa.lib_path(), mode=os.RTLD_NOW | os.RTLD_LOCAL)  # every symbol resolves at load
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert qsa.version() == 1
    assert qsa.status_string(0) == "QSA_OK"
    assert [qsa.status_string(i) for i in range(1, 6)] == [
        "QSA_ERR_NULL_PTR", "QSA_ERR_SHAPE", "QSA_ERR_PARAM", "QSA_ERR_UNSUPPORTED", "QSA_ERR_HIP"]
    assert qsa.status_string(99) == "QSA_ERR_UNKNOWN"


def test_header_constants_match_binding():
    src = open(HEADER).read()
    for name, val in [("QSA_EXACT", qsa.EXACT), ("QSA_KINT", qsa.KINT), ("QSA_POT", qsa.POT),
                      ("QSA_EXACT_ANCHORED", qsa.EXACT_ANCHORED), ("QSA_TRUNC", qsa.TRUNC),
                      ("QSA_UNIFORM", qsa.UNIFORM), ("QSA_POT_RUNNING", qsa.POT_RUNNING), ("QSA_DT_F32", qsa.DT_F32),
                      ("QSA_DT_BF16", qsa.DT_BF16), ("QSA_DT_FP8_E4M3", qsa.DT_FP8_E4M3),
                      ("QSA_GRAD_STE_POST", qsa.GRADS["ste_post"]), ("QSA_GRAD_EXACT", qsa.GRADS["exact"]),
                      ("QSA_GRAD_EXACT_DETACHED", qsa.GRADS["exact_detached"]),
                      ("QSA_GRAD_STE_PRE", qsa.GRADS["ste_pre"]),
                      ("QSA_GRAD_STE_PRE_DETACHED", qsa.GRADS["ste_pre_detached"])]:
        m = re.search(rf"\b{name}\s*=\s*(\d+)", src)
        assert m and int(m.group(1)) == val, name
    for name, val in [("QSA_F_INTERP", qsa.F_INTERP), ("QSA_F_WINDOW", qsa.F_WINDOW), ("QSA_F_FLUSH", qsa.F_FLUSH)]:
        m = re.search(rf"\b{name}\s*=\s*1\s*<<\s*(\d+)", src)
        assert m and (1 << int(m.group(1))) == val, name


def test_valid_arguments():
    assert v() == qsa.OK
    assert qsa.last_error() == ""
    for var, kl, w in [(qsa.EXACT, 0, 0.0), (qsa.EXACT_ANCHORED, 0, 0.0), (qsa.KINT, 4, 0.0),
                       (qsa.KINT | qsa.F_INTERP, 16, 0.0), (qsa.KINT | qsa.F_WINDOW, 16, 8.0),
                       (qsa.KINT | qsa.F_WINDOW | qsa.F_FLUSH | qsa.F_INTERP, 64, 8.0),
                       (qsa.POT | qsa.F_FLUSH, 64, 0.0), (qsa.POT, 1, 0.0), (qsa.TRUNC, 0, 2.0),
                       (qsa.UNIFORM, 0, 0.5), (qsa.POT_RUNNING, 2, 0.0), (qsa.POT_RUNNING | qsa.F_FLUSH, 64, 0.0)]:
        assert v(variant=var, k_levels=kl, window=w) == qsa.OK, (var, kl, w)
    assert v(d=128, N=1, H=64, Hkv=8) == qsa.OK
    assert v(dtype=qsa.DT_F32) == qsa.OK


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), qsa.ERR_SHAPE), (dict(H=0), qsa.ERR_SHAPE), (dict(Hkv=0), qsa.ERR_SHAPE), (dict(N=0), qsa.ERR_SHAPE),
    (dict(H=6, Hkv=4), qsa.ERR_SHAPE), (dict(N=(1 << 20) + 1), qsa.ERR_SHAPE), (dict(d=0), qsa.ERR_SHAPE),
    (dict(d=96), qsa.ERR_UNSUPPORTED), (dict(d=256), qsa.ERR_UNSUPPORTED),
    (dict(B=1024, H=64, N=65536, d=128), qsa.ERR_SHAPE),
    (dict(dtype=3), qsa.ERR_PARAM), (dict(dtype=-1), qsa.ERR_PARAM),
    (dict(variant=7), qsa.ERR_PARAM), (dict(variant=qsa.POT | (1 << 8)), qsa.ERR_PARAM),
    (dict(variant=qsa.POT_RUNNING, k_levels=1), qsa.ERR_PARAM),
    (dict(variant=qsa.POT_RUNNING, k_levels=65), qsa.ERR_PARAM),
    (dict(variant=qsa.POT_RUNNING, k_levels=17, dtype=qsa.DT_FP8_E4M3), qsa.ERR_PARAM),
    (dict(variant=qsa.POT_RUNNING | qsa.F_INTERP, k_levels=8), qsa.ERR_PARAM),
    (dict(variant=qsa.TRUNC, window=0.0), qsa.ERR_PARAM), (dict(variant=qsa.UNIFORM, window=-2.0), qsa.ERR_PARAM),
    (dict(variant=qsa.TRUNC, window=math.inf), qsa.ERR_PARAM), (dict(variant=qsa.UNIFORM, window=math.nan), qsa.ERR_PARAM),
    (dict(variant=qsa.TRUNC | qsa.F_FLUSH, window=2.0), qsa.ERR_PARAM),
    (dict(variant=qsa.UNIFORM | qsa.F_WINDOW, window=2.0), qsa.ERR_PARAM),
    (dict(variant=qsa.POT | qsa.F_INTERP), qsa.ERR_PARAM), (dict(variant=qsa.POT | qsa.F_WINDOW, window=8.0), qsa.ERR_PARAM),
    (dict(variant=qsa.EXACT | qsa.F_FLUSH), qsa.ERR_PARAM),
    (dict(variant=qsa.EXACT_ANCHORED | qsa.F_FLUSH), qsa.ERR_PARAM),
    (dict(variant=qsa.KINT, k_levels=0), qsa.ERR_PARAM), (dict(variant=qsa.KINT, k_levels=65), qsa.ERR_PARAM),
    (dict(variant=qsa.POT, k_levels=0), qsa.ERR_PARAM), (dict(variant=qsa.POT, k_levels=65), qsa.ERR_PARAM),
    (dict(variant=qsa.POT, k_levels=17, dtype=qsa.DT_FP8_E4M3), qsa.ERR_PARAM),
    (dict(variant=qsa.KINT | qsa.F_WINDOW, k_levels=4, window=0.0), qsa.ERR_PARAM),
    (dict(variant=qsa.KINT | qsa.F_WINDOW, k_levels=4, window=-1.0), qsa.ERR_PARAM),
    (dict(variant=qsa.KINT | qsa.F_WINDOW, k_levels=4, window=math.inf), qsa.ERR_PARAM),
    (dict(variant=qsa.KINT | qsa.F_WINDOW, k_levels=4, window=math.nan), qsa.ERR_PARAM),
])
def test_invalid_arguments(kw, status):
    assert v(**kw) == status
    assert qsa.last_error() != ""


def _fwd(Q=1, K=1, V=1, O=1, **kw):
    a = dict(GOOD)
    a.update(kw)
    L = qsa.lib()
    return L.qsa_attn_fwd(Q, K, V, O, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["causal"], a["variant"],
                          a["k_levels"], a["window"], a["dtype"], None)


def test_null_pointers_rejected_before_any_hip_call():
    for args in [dict(Q=None), dict(K=None), dict(V=None), dict(O=None)]:
        assert _fwd(**args) == qsa.ERR_NULL_PTR
    # validation runs first: a bad shape wins over a NULL pointer
    assert _fwd(Q=None, B=0) == qsa.ERR_SHAPE


def _fwd_ex(opts, **kw):
    a = dict(GOOD)
    a.update(kw)
    L = qsa.lib()
    return L.qsa_attn_fwd_ex(1, 1, 1, 1, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["causal"], a["variant"],
                             a["k_levels"], a["window"], a["dtype"], ctypes.byref(opts), None)


@pytest.mark.parametrize("fields,kw,status", [
    (dict(scale=-1.0), {}, qsa.ERR_PARAM), (dict(scale=math.inf), {}, qsa.ERR_PARAM),
    (dict(scale=math.nan), {}, qsa.ERR_PARAM),
    (dict(q_descale=2.0), {}, qsa.ERR_PARAM),                         # descale on bf16
    (dict(v_descale=-1.0), dict(dtype=qsa.DT_FP8_E4M3), qsa.ERR_PARAM),
    (dict(k_descale=math.inf), dict(dtype=qsa.DT_FP8_E4M3), qsa.ERR_PARAM),
    (dict(row_lo=8), dict(variant=qsa.EXACT), qsa.ERR_PARAM),
    (dict(row_lo=8), dict(variant=qsa.POT_RUNNING), qsa.ERR_PARAM),
    (dict(grid_idx=8, idx_row0=0, idx_rows=0), {}, qsa.ERR_SHAPE),
    (dict(grid_idx=8, idx_row0=-1, idx_rows=4), {}, qsa.ERR_SHAPE),
    (dict(grid_idx=8, idx_row0=98, idx_rows=4), {}, qsa.ERR_SHAPE),
    (dict(grid_idx=8, idx_row0=0, idx_rows=65536), dict(N=65536, H=64, Hkv=8, B=1), qsa.ERR_SHAPE),
])
def test_invalid_options(fields, kw, status):
    o = qsa._Opts()
    for k_, val in fields.items():
        setattr(o, k_, val)
    assert _fwd_ex(o, **kw) == status
    assert qsa.last_error() != ""


def test_binding_rejects_bad_tensors_on_host():
    import torch
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        qsa.attn_fwd_ex(q, q, q)                      # CPU tensors
    with pytest.raises(ValueError):
        qsa.attn_fwd_ex(q, q[:, :, :4], q)            # shape mismatch
    with pytest.raises(ValueError):
        qsa.attn_fwd_ex(q, q.double(), q)             # dtype mismatch


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_ex"])
def test_binding_refuses_short_kv_before_launch(fn):
    # the kernels size their K and V reads from q's N and d: a k or v with fewer keys, another
    # head dimension or a missing axis must be refused by the shape check (it runs before the
    # device check, so host tensors reach it without a GPU)
    import torch
    f = getattr(qsa, fn)
    q = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16)
    good = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    for bad_k, bad_v in ((q[:, :2, :32], good), (good, q[:, :2, :32]), (good[..., :32], good),
                         (good[0], good), (torch.zeros(2, 2, 64, 64, dtype=torch.bfloat16), good)):
        with pytest.raises(ValueError, match="k and v must be|must be 4-D"):
            f(q, bad_k.contiguous(), bad_v.contiguous(), kind="pot", levels=8)


def _bwd(ptrs=(1, 1, 1, 1, 1, 1, 1), grad=0, scale=0.0, **kw):
    a = dict(GOOD)
    a.update(kw)
    return qsa.lib().qsa_attn_bwd(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["causal"], a["variant"],
                                  a["k_levels"], a["window"], a["dtype"], grad, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), qsa.ERR_SHAPE), (dict(H=3), qsa.ERR_SHAPE), (dict(d=96), qsa.ERR_UNSUPPORTED),
    (dict(dtype=qsa.DT_FP8_E4M3), qsa.ERR_UNSUPPORTED), (dict(grad=-1), qsa.ERR_PARAM),
    (dict(grad=5), qsa.ERR_PARAM), (dict(scale=-1.0), qsa.ERR_PARAM), (dict(scale=math.nan), qsa.ERR_PARAM),
    (dict(variant=qsa.KINT, k_levels=0), qsa.ERR_PARAM), (dict(variant=qsa.TRUNC, window=0.0), qsa.ERR_PARAM),
    (dict(variant=qsa.POT_RUNNING), qsa.ERR_UNSUPPORTED),
])
def test_backward_validation_before_any_hip_call(kw, status):
    assert _bwd(**kw) == status
    assert qsa.last_error() != ""


def test_backward_null_pointers_rejected():
    for i in range(7):
        ptrs = [1] * 7
        ptrs[i] = None
        assert _bwd(ptrs=tuple(ptrs)) == qsa.ERR_NULL_PTR
    assert _bwd(ptrs=(None,) * 7, B=0) == qsa.ERR_SHAPE      # validation first


def test_backward_binding_rejects_bad_tensors_on_host():
    import torch
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        qsa.attn_bwd(q, q, q, q)                      # CPU tensors
    with pytest.raises(ValueError):
        qsa.attn_bwd(q, q, q, q, grad="nope")         # unknown mode


def test_host_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The host layer (qsa_api.cpp) built by g++ with ASan + UBSan against stub launchers
    (tests/host/abi_host_check.cpp) and driven through every validation branch, the argument
    marshalling and the error reporting; any sanitizer report aborts the run."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "abi_host_check")
    csrc = os.path.join(ROOT, "quantized_softmax_approximation_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + csrc, os.path.join(csrc, "qsa_api.cpp"), os.path.join(ROOT, "tests", "host", "abi_host_check.cpp"),
           "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("host checks passed"), (r.stdout + r.stderr)[-4000:]
