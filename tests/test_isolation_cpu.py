"""The oracle and the HIP path share no code.

The package (kernels, headers, binding, input generators) neither imports
nor includes anything under oracle/, and the oracle imports nothing from the
package: only tests, smoke() and bench.py's CPU baseline call the oracle.
"""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _files(top, exts):
    for d, _, names in os.walk(os.path.join(ROOT, top)):
        if "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def test_package_does_not_use_the_oracle():
    pat = re.compile(r"^\s*(from\s+oracle\b|import\s+oracle\b|#\s*include\s+[\"<][^\">]*oracle)",
                     re.M)
    for top in ("atomic_expert_routing_amd", "include"):
        for f in _files(top, (".py", ".hip", ".h", ".cpp")):
            assert not pat.search(open(f, encoding="utf-8").read()), f


def test_oracle_does_not_use_the_package():
    pat = re.compile(r"^\s*(from|import)\s+atomic_expert_routing_amd\b", re.M)
    for f in _files("oracle", (".py",)):
        assert not pat.search(open(f, encoding="utf-8").read()), f


def test_bench_calls_the_oracle_only_in_its_cpu_baseline():
    src = open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read()
    # every oracle import sits inside cpu_baseline()
    funcs = re.split(r"^def ", src, flags=re.M)
    users = [f.split("(")[0] for f in funcs[1:] if re.search(r"\boracle\b.*import|import .*oracle|from oracle", f)]
    assert users == ["cpu_baseline"], users
