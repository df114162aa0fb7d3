"""bench.py on the CPU: the one-GPU refusal and the hash tying profiles to the kernel sources."""
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


def test_source_hash_ignores_comments_only():
    """The hash that ties a profile to the kernel sources follows the code:
    comments (line and block) and blank lines drop out, literals stay whole."""
    sys.path.insert(0, ROOT)
    import bench

    code = 'int f(int x) {\n  return x + 1;  // one\n}\nconst char* s = "a // b /* c */";\nchar q = \'"\';\n'
    commented = '/* header\n   block */\nint f(int x) {  // f\n\n  return x + 1;  // another note\n}\n' \
                'const char* s = "a // b /* c */";\nchar q = \'"\';  /* q */\n'
    assert bench.strip_c_comments(code) == bench.strip_c_comments(commented)
    assert "a // b /* c */" in bench.strip_c_comments(code)
    assert bench.strip_c_comments(code) != bench.strip_c_comments(code.replace("x + 1", "x + 2"))
