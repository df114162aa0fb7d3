"""bench.py on the CPU: the one-GPU refusal and the hash tying profiles to the built kernels."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True,
                           text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, (r.returncode, r.stderr[-500:])
        msg = json.loads(r.stdout.strip().splitlines()[-1])
        assert "one GPU" in msg["error"]


def _tiny_library(tmp_path, name, kernel_body, host_comment=""):
    """Two translation units, each with a kernel, the second's body given."""
    first = tmp_path / f"{name}_1.hip"
    first.write_text("#include <hip/hip_runtime.h>\n"
                     "__global__ void k1(float* x) { x[threadIdx.x] += 1.0f; }\n")
    second = tmp_path / f"{name}_2.hip"
    second.write_text("#include <hip/hip_runtime.h>\n"
                      f"// {host_comment}\n"
                      f"__global__ void k2(float* x) {{ {kernel_body} }}\n"
                      'extern "C" int host_entry(int v) { return v + 1; }\n')
    so = str(tmp_path / f"lib{name}.so")
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", str(first), str(second), "-o",
                           so], stderr=subprocess.DEVNULL)
    return so


def test_kernel_code_hash_follows_the_device_code(tmp_path):
    """The hash that ties a profile to the kernels is taken over the built
    device code (.text, .rodata, .note of every amdgcn code object, one bundle
    per translation unit): two builds of the same sources agree although the
    bundles' bytes differ, a comment or host-code edit leaves it alone, and a
    change to a kernel in any translation unit moves it."""
    import shutil

    if shutil.which("hipcc") is None:
        import pytest

        pytest.skip("hipcc is not installed")
    sys.path.insert(0, ROOT)
    import bench

    body = "x[threadIdx.x] *= 2.0f;"
    a = bench.kernel_code_hash(_tiny_library(tmp_path, "a", body))
    b = bench.kernel_code_hash(_tiny_library(tmp_path, "b", body, host_comment="another comment"))
    c = bench.kernel_code_hash(_tiny_library(tmp_path, "c", "x[threadIdx.x] *= 3.0f;"))
    assert a == b and a != c and len(a) == 64
