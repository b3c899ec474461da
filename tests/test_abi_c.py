"""The library used from plain C through include/tpshard.h (tests/c/abi_smoke.c,
compiled here with gcc against libtpshard.so and the HIP runtime): the
host-only calls without a GPU (the Pop Quiz of [SB6] §6.1 through
tp_shard_shape, a workspace query, an argument refused before any launch),
and on the GPU the column-parallel output and the row-parallel fp32 partial
on hipMalloc'd buffers against exact products computed in the C program
(integer inputs)."""
import json
import os
import shutil
import subprocess

import pytest

import tensor_sharded_matmul_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_smoke.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(not os.path.exists(T.lib_path()) or shutil.which("gcc") is None
                                or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")),
                                reason="needs libtpshard.so, gcc and the HIP headers")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("abi_c") / "abi_smoke")
    libdir = os.path.dirname(T.lib_path())
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", f"-I{ROOT}/include", f"-I{ROCM}/include",
           "-D__HIP_PLATFORM_AMD__", SRC, f"-L{libdir}", "-ltpshard", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{ROCM}/lib", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=120)
    return r.returncode, r.stdout


def test_host_calls_from_c(exe):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "shard_quiz.json")))
    axes = [a for a, _ in g["mesh"]]
    masks = [sum(1 << axes.index(a) for a in dims) for dims in g["spec"]]
    rc, out = _run(exe, "host", len(g["shape"]), *g["shape"], g["elem_bytes"], len(axes),
                   *[s for _, s in g["mesh"]], *masks)
    lines = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert rc == 0, out
    assert int(lines["version"]) == T.tp_version()
    shape, rest = lines["shape"].split(" bytes ")
    assert [int(x) for x in shape.split()] == g["local_shape"]
    b, t = rest.split(" total ")
    assert int(b) == g["local_bytes"] and int(t) == g["total_bytes"]
    assert int(lines["workspace"]) == T.workspace_size("tp_col_linear", 16, 8192, 1280, 0)
    assert lines["refused"].startswith("3 ") and "multiple of 64" in lines["refused"]
    # one mesh axis splitting two dims is refused
    bad = [sum(1 << axes.index(a) for a in dims) for dims in g["illegal_same_axis_spec"]]
    rc, out = _run(exe, "host", len(g["shape"]), *g["shape"], g["elem_bytes"], len(axes),
                   *[s for _, s in g["mesh"]], *bad)
    assert "status 1 " in out


@pytest.mark.gpu
@pytest.mark.parametrize("N,k,n", [(16, 8192, 1280), (16, 1024, 8192), (37, 256, 192), (300, 1024, 512)])
def test_products_from_c(exe, N, k, n):
    print(f"abi_smoke gpu {N} {k} {n}", flush=True)
    rc, out = _run(exe, "gpu", N, k, n)
    print(out, flush=True)
    assert rc == 0 and out.startswith("ok"), out
