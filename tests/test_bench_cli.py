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


def test_phase_stamps_pool():
    """The phase summary of --phase-stamps on a hand-made stamp set: durations
    are the gaps between a workgroup's consecutive stamps (100 MHz clock),
    named by the later stamp's code; unwritten events and workgroups drop out."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench

    st = np.zeros((4, 16, 2), dtype=np.uint64)
    # workgroup 0: start at 1000, merged (+200 = 2 us), tested (+50), bonus draw (+300)
    st[0, :4] = [[1000, 0], [1200, 1], [1250, 2], [1550, 3]]
    # workgroup 2: start at 1100, merged (+400 = 4 us), tested (+50), residual pass (+500)
    st[2, :4] = [[1100, 0], [1500, 1], [1550, 2], [2050, 4]]
    r = bench.pool_stamps([st], 1)
    ph = r["phases_us_count_p50_p90"]
    assert r["workgroups"] == 2 and r["calls"] == 1
    assert ph[bench.phase_name(1)][0] == 2 and ph[bench.phase_name(1)][1] == 3.0  # median of 2 and 4 us
    assert ph[bench.phase_name(2)] == [2, 0.5, 0.5]
    assert ph[bench.phase_name(3)][:2] == [1, 3.0] and ph[bench.phase_name(4)][:2] == [1, 5.0]
    assert r["workgroup_span_us_p50_p90_max"][2] == 9.5  # workgroup 2: 1100 -> 2050
    assert r["first_start_to_last_stamp_us_p50"] == 10.5  # 1000 -> 2050
    assert "note" in bench.pool_stamps([np.zeros((4, 16, 2), dtype=np.uint64)], 1)
    assert bench.phase_name(102).endswith("after 2 rejections") and bench.phase_name(201).startswith("level: all 1")
