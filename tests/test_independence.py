"""The oracle and the HIP path share no code and neither imports the other; the
product path never reaches the oracle.  CPU only (reads sources)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources(folder, exts):
    for dp, _, fns in os.walk(os.path.join(ROOT, folder)):
        for fn in fns:
            if fn.endswith(exts):
                yield os.path.join(dp, fn)


def test_oracle_imports_nothing_from_the_library():
    for p in _sources("oracle", (".py",)):
        src = open(p).read()
        assert not re.search(r"^\s*(from|import)\s+(gemm_decode_amd|ctypes|torch)\b", src, re.M), p


def test_library_never_reaches_the_oracle():
    for p in _sources("gemm_decode_amd", (".py", ".hip", ".cpp", ".h", ".hpp")):
        src = open(p).read()
        assert not re.search(r"^\s*(from|import)\s+oracle\b", src, re.M), p
        assert "oracle/" not in src and "oracle." not in src, p


def test_synth_holds_no_method_arithmetic():
    src = open(os.path.join(ROOT, "synth", "__init__.py")).read()
    code = "\n".join(l for l in src.splitlines() if not l.lstrip().startswith(("#", '"', "*")))
    for word in ("rint(", "clip(", "127", "dequant(", " @ ", "import oracle", "gemm_decode_amd"):
        assert word not in code, word
