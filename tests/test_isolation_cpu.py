"""The product path stands apart from the oracle: importing the package (and
the input generators it shares with the tests) loads nothing under oracle/,
no product source names it, and a missing library fails loudly instead of
falling back to anything else."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "differential_softmax_attention_diffattn_amd")


def test_importing_the_package_loads_no_oracle_module():
    code = ("import sys; sys.path.insert(0, %r); "
            "import differential_softmax_attention_diffattn_amd as da; "
            "from differential_softmax_attention_diffattn_amd import inputs; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "print(bad); sys.exit(1 if bad else 0)") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_no_product_source_names_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "diffattn_oracle" not in text, f


def test_a_missing_library_fails_loudly(tmp_path):
    code = ("import sys; sys.path.insert(0, %r); "
            "from differential_softmax_attention_diffattn_amd import _lib; "
            "_lib.load(%r)") % (ROOT, str(tmp_path / "absent.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "is missing" in r.stderr
