"""The oracle and the HIP path share no code and do not import each other;
the product package never reaches the oracle (CPU only)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _py_files(d):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith((".py", ".hip", ".h", ".cpp", ".c")):
                yield os.path.join(dp, f)


def test_package_never_imports_oracle():
    for f in _py_files("group_dft_structured_amd"):
        text = open(f).read()
        assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
        assert "oracle" not in re.findall(r"include\s+\"([^\"]+)\"", text), f


def test_oracle_never_imports_package():
    for f in _py_files("oracle"):
        text = open(f).read()
        assert "group_dft_structured_amd" not in text, f
        assert "eqlinear.h" not in text, f
