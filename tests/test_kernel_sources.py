"""CPU checks on the HIP sources themselves.

No inline assembly in the kernels: the compiler keeps a VALU instruction
that reads an MFMA's result the required number of wait states behind the
MFMA (gfx950 has no interlock for it), but it does not look inside inline
asm, and an asm max over score registers once read them early (results
within tolerance, not reproducible bit for bit).  Builtins keep the
compiler's hazard checks."""
import os
import re

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "paged_kv_cache_346_amd", "csrc")


def _sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            path = os.path.join(CSRC, name)
            with open(path) as f:
                yield name, f.read()


def _code(text):
    """The text with // and /* */ comments removed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return re.sub(r"//[^\n]*", " ", text)


def test_no_inline_assembly():
    found = [name for name, text in _sources()
             if re.search(r"\b(asm|__asm__)\s*(volatile\s*)?\(", _code(text))]
    assert found == [], f"inline asm in {found}"


def test_packed_fp32_ops_stay_off():
    """Every HIP compile turns the packed-fp32 feature off (no v_pk_*_f32)."""
    with open(os.path.join(ROOT, "paged_kv_cache_346_amd", "build.py")) as f:
        build = f.read()
    assert '"-packed-fp32-ops"' in build
    for name, text in _sources():
        assert not re.search(r"v_pk_(add|mul|fma)_f32", _code(text)), name
