"""Static checks of the repository layout: the product path and the oracle
share no code and do not import each other."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "prompt_conditioned_keypoint_amd")

ORACLE_REFS = re.compile(r"(^\s*(import|from)\s+oracle\b)|libgko|gko\.c|\bgko_\w+\(",
                         re.M)
PRODUCT_REFS = re.compile(r"(^\s*(import|from)\s+prompt_conditioned_keypoint_amd\b)|"
                          r"libgkdhead|gkdhead\.h|\bgkd_\w+\(", re.M)


def _sources(top, exts):
    for dirpath, _, files in os.walk(top):
        for f in files:
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def test_product_path_never_references_the_oracle():
    for path in _sources(PKG, (".py", ".hip", ".hpp", ".h", ".cpp", ".c")):
        assert not ORACLE_REFS.search(open(path).read()), path


def test_oracle_never_references_the_product_path():
    for path in _sources(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        assert not PRODUCT_REFS.search(open(path).read()), path


def test_generators_hold_no_head_arithmetic():
    """The shared input generator imports neither side."""
    for path in _sources(os.path.join(ROOT, "gkdsynth"), (".py",)):
        text = open(path).read()
        assert not ORACLE_REFS.search(text), path
        assert not PRODUCT_REFS.search(text), path
        for word in ("interpolate(", "argmax(", "np.exp(", "math.exp(", "einsum(",
                     "tensordot("):
            assert word not in text, (path, word)
