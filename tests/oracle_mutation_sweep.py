"""Automatic single-site mutants of the oracle, against its pins (CPU only).

Where the named mutants in test_oracle_mutations.py plant chosen mistakes,
this sweep plants every mechanical one it can find in oracle.c, one at a time:
a flipped comparison (< <=, > >=, == !=), a swapped logical operator, an
off-by-one constant (+ 1, - 1), 0.0 replaced by 1.0, += by -=, ++ by --, and
each assignment statement deleted.  Each mutant is compiled into a temporary
directory and run through mutant_runner.py; the real oracle is never touched.
The report counts mutants that fail a pin (caught), crash or time out, do not
compile, or pass every pin (survived, listed with their line).  A survivor is
a gap in the pins unless it is equivalent to the original (for example an
allocation guard `n > 0 ? n : 1` turned into `n >= 0`) or only reads out of
bounds.

With --sanitize each mutant is built with gcc -fsanitize=address,undefined
and run with the AddressSanitizer runtime preloaded, so a mutant that reads
or writes out of bounds fails even where the values it reads would pass.

Usage: python tests/oracle_mutation_sweep.py [--jobs 8] [--timeout 120] [--sanitize]
Not collected by pytest: a full sweep takes several minutes on 8 cores.
"""
import argparse
import collections
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402

OPERATORS = [
    (r"(?<![<>=!])<(?![<=])", "<="),
    (r"<=", "<"),
    (r"(?<![<>=-])>(?![>=])", ">="),
    (r">=", ">"),
    (r"==", "!="),
    (r"!=", "=="),
    (r"&&", "||"),
    (r"\|\|", "&&"),
    (r"\+ 1\b", "+ 0"),
    (r"- 1\b", "- 0"),
    (r"\b0\.0\b", "1.0"),
    (r"\+=", "-="),
    (r"\+\+", "--"),
]


def mutants(lines):
    """(line index, operator, mutated line) for every site outside comments
    and preprocessor lines; operator 'del' deletes an assignment statement."""
    out = []
    for i, line in enumerate(lines):
        s = line.strip()
        if s.startswith(("/*", "*", "//", "#")):
            continue
        code = line.split("/*")[0].split("//")[0]
        for pat, rep in OPERATORS:
            for m in re.finditer(pat, code):
                if pat.startswith("(?<![<>=-])>") and "->" in code[max(0, m.start() - 1):m.end() + 1]:
                    continue
                out.append((i, pat, line[:m.start()] + rep + line[m.end():]))
        if s.endswith(";") and "=" in s and not s.startswith(("for", "return")):
            out.append((i, "del", ""))
    return out


def run_one(lines, site, timeout, asan_rt=None):
    i, _, new = site
    mutated = list(lines)
    mutated[i] = new
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        so = os.path.join(d, "libmutant.so")
        with open(src, "w") as f:
            f.write("\n".join(mutated))
        # the oracle's own build line (gcc -O2 -std=c99, IEEE semantics), quiet
        san = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"] if asan_rt else ["-O2"]
        cc = subprocess.run(["gcc", *san, "-std=c99", "-fPIC", "-shared", "-w", "-o", so, src, "-lm"],
                            capture_output=True)
        if cc.returncode:
            return "nocompile"
        env = dict(os.environ)
        if asan_rt:
            env.update(LD_PRELOAD=asan_rt, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1")
        try:
            r = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), so], capture_output=True,
                               text=True, timeout=timeout, env=env)
        except subprocess.TimeoutExpired:
            return "timeout"
        if "Sanitizer" in r.stderr:
            return "sanitizer"
    if r.returncode == 0:
        return "survived"
    return "caught" if "caught" in r.stdout else f"crash({r.returncode})"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--timeout", type=int, default=120)
    ap.add_argument("--sanitize", action="store_true")
    args = ap.parse_args()
    asan_rt = None
    if args.sanitize:
        asan_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    with open(oracle.SRC) as f:
        lines = f.read().split("\n")
    sites = mutants(lines)
    print(f"{len(sites)} mutants of {os.path.basename(oracle.SRC)}", flush=True)
    with ThreadPoolExecutor(args.jobs) as ex:
        results = list(ex.map(lambda s: run_one(lines, s, args.timeout, asan_rt), sites))
    print(dict(collections.Counter(results)))
    for (i, pat, new), res in zip(sites, results):
        if res == "survived":
            print(f"survived: line {i + 1} [{pat}] {lines[i].strip()[:80]}  ->  {new.strip()[:80]}")


if __name__ == "__main__":
    main()
