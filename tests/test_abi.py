"""CPU checks of the C-ABI library: it builds for gfx950, loads, exports every
function include/llar.h declares, and its host-side argument checks work
without a GPU (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llar.h")


@pytest.fixture(scope="module")
def L():
    import message_allreduce_amd as m
    if not os.path.exists(m.library_path):
        from message_allreduce_amd import _build
        _build.build()
    return m.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(llar_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_three_core_calls():
    names = declared_functions()
    for core in ("llar_create", "llar_allreduce", "llar_destroy"):
        assert core in names


def test_library_exports_every_declared_symbol(L):
    import message_allreduce_amd as m
    out = subprocess.run(["nm", "-D", "--defined-only", m.library_path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (llar_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    # the binding lists exactly the header's functions
    assert sorted(m.EXPORTED_SYMBOLS) == declared_functions()


def test_library_is_built_for_gfx950(L):
    import message_allreduce_amd as m
    blob = open(m.library_path, "rb").read()
    # the embedded device code object carries its offload target id
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings(L):
    import message_allreduce_amd as m
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = m.llar_status_string(code)
        assert s.startswith(m.STATUS[code])


def test_null_handle_is_rejected_without_touching_the_gpu(L):
    import message_allreduce_amd as m
    assert L.llar_allreduce(None, None, None, 16, 0, 0, None) == -1
    assert L.llar_destroy(None) == 0
    assert L.llar_send_recv(None, None, None, 16, 0, 1, None) == -1
    assert L.llar_set_option(None, b"timing", 2) == -1  # NULL: the process defaults; 2 is out of range
    assert L.llar_get_device_status(None, None) == -1
    assert L.llar_staging_bytes(None, 1) == 0
    v = ctypes.c_double(0)
    assert L.llar_floor_measure(99, 0, ctypes.byref(v)) == -1
    assert L.llar_floor_measure(-1, 0, ctypes.byref(v)) == -1


def test_create_rejects_bad_arguments(L):
    import message_allreduce_amd as m
    assert not L.llar_create(0, 0, 1024) and L.llar_last_error() == -1
    assert not L.llar_create(2, 7, 1024) and L.llar_last_error() == -1
    assert not L.llar_create(2, 0, 0) and L.llar_last_error() == -1
    assert not L.llar_create(9, 0, 1024) and L.llar_last_error() == -2


def test_package_has_no_cpu_fallback():
    # the product package must not import the oracle or compute on the host
    pkg = os.path.join(ROOT, "message_allreduce_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "oracle/" not in src, f


def test_device_header_is_self_contained_and_demo_exports():
    """include/llar_wire.h compiles on its own for gfx950, and the demo
    library written against it exports its launchers."""
    import shutil
    import subprocess
    import tempfile
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.hip")
        with open(src, "w") as f:
            f.write('#include "llar_wire.h"\n'
                    '__global__ void k(uint8_t* s, uint32_t e) {\n'
                    '  llar_wire::Wire w = llar_wire::make_wire(s, 4096);\n'
                    '  llar_wire::ll_put<llar_wire::kDevice>(w, 0, llar_wire::u32x2{1u, 2u}, e);\n'
                    '  llar_wire::sentinel_put<2, llar_wire::kXcd>(w, 16, llar_wire::u32x4{0u, 0u, 0u, 0u});\n'
                    '}\n')
        res = subprocess.run([hipcc, "--offload-arch=gfx950", "--cuda-device-only", "-fsyntax-only", "-std=c++17",
                              "-I", os.path.join(root, "include"), src], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
    lib = os.path.join(root, "tests", "device_api", "libwire_demo.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location("wire_demo_build", os.path.join(root, "tests", "device_api", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    L = ctypes.CDLL(lib)
    for name in ("demo_scaled_allreduce_ll", "demo_sentinel_chain", "demo_ll128_reduce"):
        assert hasattr(L, name)



def test_bench_refuses_more_than_one_gpu():
    """bench.py emulates the ranks on one GPU: --gpus N > 1 exits with a
    message before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout


_ENV_PROBE = r'''
import ctypes, json, sys
L = ctypes.CDLL(sys.argv[1])
L.llar_get_option.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.POINTER(ctypes.c_longlong)]
L.llar_set_option.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_longlong]
out = {}
for key in sys.argv[2:]:
    v = ctypes.c_longlong(-99)
    st = L.llar_get_option(None, key.encode(), ctypes.byref(v))
    out[key] = v.value if st == 0 else ("error", st)
print(json.dumps(out))
'''


def _read_defaults(env, keys):
    import json
    import sys
    import message_allreduce_amd as m
    full = dict(os.environ)
    for k in list(full):
        if k.startswith("LLAR_"):
            del full[k]
    full.update(env)
    r = subprocess.run([sys.executable, "-c", _ENV_PROBE, m.library_path, *keys], capture_output=True, text=True,
                       env=full, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout), r.stderr


def test_environment_knobs_set_the_process_defaults(L, tmp_path):
    """Each knob lands in the option table that communicators start from,
    readable through llar_get_option with a NULL handle (no device needed)."""
    keys = ["spin_timeout_us", "auto_protocol", "ll128_acc", "log", "keep_staging", "auto_threshold_sentinel",
            "chunk_bytes", "threads"]
    base, _ = _read_defaults({}, keys)
    assert base == {"spin_timeout_us": 200000, "auto_protocol": 0, "ll128_acc": 0, "log": 0, "keep_staging": 0,
                    "auto_threshold_sentinel": 65536, "chunk_bytes": 0, "threads": 0}
    tune = tmp_path / "tune.txt"
    tune.write_text("# thresholds measured elsewhere\nauto_threshold_sentinel 4096\nchunk_bytes=131072\n\nthreads 256\n")
    got, err = _read_defaults({"LLAR_SPIN_TIMEOUT_US": "1234", "LLAR_PROTOCOL": "sentinel_pipelined",
                               "LLAR_ACCUM": "16", "LLAR_LOG": "1", "LLAR_DEBUG_KEEP_STAGING": "1",
                               "LLAR_TUNE": str(tune)}, keys)
    assert got == {"spin_timeout_us": 1234, "auto_protocol": 5, "ll128_acc": 1, "log": 1, "keep_staging": 1,
                   "auto_threshold_sentinel": 4096, "chunk_bytes": 131072, "threads": 256}, (got, err)
    assert err == ""
    for env, name in (({"LLAR_PROTOCOL": "ll"}, 1), ({"LLAR_PROTOCOL": "3"}, 3), ({"LLAR_ACCUM": "fp32"}, 0)):
        got, _ = _read_defaults(env, ["auto_protocol", "ll128_acc"])
        assert name in got.values()


def test_environment_knobs_with_bad_values_are_reported_and_ignored(L, tmp_path):
    tune = tmp_path / "tune.txt"
    tune.write_text("threads 300\nno_such_key 1\nchunk_bytes abc\nslices 16\n")
    got, err = _read_defaults({"LLAR_SPIN_TIMEOUT_US": "0", "LLAR_PROTOCOL": "fastest", "LLAR_ACCUM": "8",
                               "LLAR_LOG": "yes", "LLAR_TUNE": str(tune)},
                              ["spin_timeout_us", "auto_protocol", "ll128_acc", "log", "threads", "chunk_bytes",
                               "slices"])
    assert got == {"spin_timeout_us": 200000, "auto_protocol": 0, "ll128_acc": 0, "log": 0, "threads": 0,
                   "chunk_bytes": 0, "slices": 16}
    for word in ("LLAR_SPIN_TIMEOUT_US=0", "LLAR_PROTOCOL=fastest", "LLAR_ACCUM=8", "LLAR_LOG=yes",
                 "LLAR_TUNE=300", "LLAR_TUNE=abc"):
        assert "ignoring " + word in err, (word, err)
    got, err = _read_defaults({"LLAR_TUNE": str(tmp_path / "missing.txt")}, ["threads"])
    assert got == {"threads": 0} and "cannot open" in err


def test_null_handle_options_are_the_process_defaults(L):
    v = ctypes.c_longlong(0)
    assert L.llar_set_option(None, b"threads", 300) == -1
    assert L.llar_set_option(None, b"no_such_key", 1) == -1
    assert L.llar_get_option(None, b"local_placement_ok", ctypes.byref(v)) == -1
    assert L.llar_get_option(None, b"auto_threshold_pipelined", ctypes.byref(v)) == 0 and v.value == 3 << 19
    assert L.llar_set_option(None, b"auto_threshold_pipelined", 2 << 20) == 0
    assert L.llar_get_option(None, b"auto_threshold_pipelined", ctypes.byref(v)) == 0 and v.value == 2 << 20
    assert L.llar_set_option(None, b"auto_threshold_pipelined", 3 << 19) == 0  # the default again
