"""The C ABI layer's device and HIP failure paths, on the CPU, and the ABI
tests under AddressSanitizer and UndefinedBehaviorSanitizer.

The ABI layer (csrc/api.cpp with the host-side planner csrc/plan.cpp) is
built with g++ into a host-only library, linked with tests/abi_host/
hip_stub.cpp in place of the HIP runtime and the kernel launches.  The stub
reports a chosen current device (device 1 is not gfx950) and returns chosen
errors from hipGetDevice, a launch and the scratch lookup, so the layer's
EA_EDEVICE and EA_EHIP paths run without a GPU.  On a GPU that is not
gfx950 the pages' library fails with "RuntimeError: CUDA error" ("Flash
Attention | Hermes Skill", Common issues); this library returns EA_EDEVICE.

The sanitizer test rebuilds the same host library with
-fsanitize=address,undefined (no recovery) and runs tests/test_abi.py and the
failure-path tests below against it in a child process.
"""
import ctypes
import os
import subprocess
import sys

import pytest

from exact_attention_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_04_amd", "csrc")
STUB = os.path.join(ROOT, "tests", "abi_host", "hip_stub.cpp")

HIP_ERROR_NO_DEVICE = 100
HIP_ERROR_INVALID_DEVICE_FUNCTION = 98
HIP_ERROR_INVALID_SYMBOL = 13

pytestmark = pytest.mark.skipif(subprocess.run(["which", "g++"], capture_output=True).returncode != 0,
                                reason="g++ not available")


def build_host_library(out_dir, sanitize=False):
    """g++ build of api.cpp + plan.cpp + the HIP stub into out_dir."""
    out = os.path.join(out_dir, "libea_attn_host_san.so" if sanitize else "libea_attn_host.so")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    if sanitize:
        flags += ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    else:
        flags += ["-Wl,--no-undefined"]
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"), STUB]
    res = subprocess.run(["g++"] + flags + srcs + ["-o", out], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out


@pytest.fixture(scope="module")
def host():
    path = os.environ.get("EA_ABI_TEST_LIB")
    if path is None:
        import tempfile
        path = build_host_library(tempfile.mkdtemp(prefix="ea_abi_host_"))
    h = _lib.bind(ctypes.CDLL(path))
    h.ea_stub_set.argtypes = [ctypes.c_int] * 4
    h.ea_stub_launches.restype = ctypes.c_int
    h.ea_stub_symbol_lookups.restype = ctypes.c_int
    yield h
    h.ea_stub_set(0, 0, 0, 0)


def _args():
    from test_abi import make
    return make()


def _split_args():
    # causal fp8 B1 H2 N1000: the plan splits the keys (its workspace is 2 chunks)
    from test_abi import make
    return make(B=1, N=1000, H=2, D=128, causal=1, dtype=_lib.EA_FP8_E4M3)


def _bwd_args():
    from test_abi import make_bwd
    return make_bwd()


def test_device_must_be_gfx950(host):
    fwd = lambda a: host.ea_attn_fwd(ctypes.byref(a), None)
    noalloc = lambda a: host.ea_attn_fwd_noalloc(ctypes.byref(a), None)
    bwd = lambda a: host.ea_attn_bwd(ctypes.byref(a), None)
    for dev, want in ((1, _lib.EA_EDEVICE), (2, _lib.EA_EDEVICE), (4, _lib.EA_EDEVICE),
                      (0, _lib.EA_OK), (3, _lib.EA_OK)):
        host.ea_stub_set(dev, 0, 0, 0)
        before = host.ea_stub_launches()
        assert fwd(_args()) == want, dev
        assert noalloc(_args()) == want, dev
        assert bwd(_bwd_args()) == want, dev
        launched = host.ea_stub_launches() - before
        assert launched == (3 if want == _lib.EA_OK else 0), (dev, launched)
    assert "gfx950" in host.ea_status_string(_lib.EA_EDEVICE).decode()


def test_hip_errors_are_reported(host):
    # hipGetDevice failing
    host.ea_stub_set(0, HIP_ERROR_NO_DEVICE, 0, 0)
    for call, a in ((host.ea_attn_fwd, _args()), (host.ea_attn_fwd_noalloc, _args()), (host.ea_attn_bwd, _bwd_args())):
        assert call(ctypes.byref(a), None) == _lib.EA_EHIP
        assert host.ea_last_hip_error() == HIP_ERROR_NO_DEVICE
    # a launch failing
    host.ea_stub_set(0, 0, HIP_ERROR_INVALID_DEVICE_FUNCTION, 0)
    for call, a in ((host.ea_attn_fwd, _args()), (host.ea_attn_fwd_noalloc, _args()), (host.ea_attn_bwd, _bwd_args())):
        assert call(ctypes.byref(a), None) == _lib.EA_EHIP
        assert host.ea_last_hip_error() == HIP_ERROR_INVALID_DEVICE_FUNCTION
    # the static scratch lookup failing (only a split launch looks it up)
    host.ea_stub_set(0, 0, 0, HIP_ERROR_INVALID_SYMBOL)
    n = host.ea_stub_symbol_lookups()
    assert host.ea_attn_fwd_noalloc(ctypes.byref(_args()), None) == _lib.EA_OK      # no split: no lookup
    assert host.ea_stub_symbol_lookups() == n
    assert host.ea_attn_fwd_noalloc(ctypes.byref(_split_args()), None) == _lib.EA_EHIP
    assert host.ea_last_hip_error() == HIP_ERROR_INVALID_SYMBOL
    # the forward with a caller workspace does not touch the static scratch
    host.ea_stub_set(0, 0, 0, 0)
    assert host.ea_attn_fwd(ctypes.byref(_split_args()), None) == _lib.EA_OK
    assert host.ea_attn_fwd_noalloc(ctypes.byref(_split_args()), None) == _lib.EA_OK
    assert host.ea_stub_symbol_lookups() > n


def test_last_hip_error_is_per_thread(host):
    import threading
    host.ea_stub_set(0, HIP_ERROR_NO_DEVICE, 0, 0)
    assert host.ea_attn_fwd(ctypes.byref(_args()), None) == _lib.EA_EHIP
    seen = []
    t = threading.Thread(target=lambda: seen.append(host.ea_last_hip_error()))
    t.start()
    t.join()
    assert seen == [0] and host.ea_last_hip_error() == HIP_ERROR_NO_DEVICE
    host.ea_stub_set(0, 0, 0, 0)


def test_python_binding_maps_the_failures():
    # the binding's status mapping: argument errors raise ValueError, device
    # and HIP failures RuntimeError (with the hipError_t for EA_EHIP)
    for code in (_lib.EA_EINVAL, _lib.EA_EUNSUPPORTED, _lib.EA_ESCRATCH):
        with pytest.raises(ValueError):
            _lib.check(code)
    for code in (_lib.EA_EDEVICE, _lib.EA_EHIP):
        with pytest.raises(RuntimeError) as ei:
            _lib.check(code)
        assert not isinstance(ei.value, ValueError)


@pytest.mark.skipif(bool(os.environ.get("EA_ABI_TEST_LIB")), reason="already inside the sanitizer run")
def test_abi_tests_under_address_and_undefined_behavior_sanitizers(tmp_path):
    san = build_host_library(str(tmp_path), sanitize=True)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.exists(asan), asan
    env = dict(os.environ)
    env.update({
        "EA_ABI_TEST_LIB": san,
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
