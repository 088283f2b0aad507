"""Source-level guards (CPU): code shapes the kernels rely on for correctness.

* Every 16-byte buffer store passes a zero soffset, all of its offset in the
  per-lane voffset.  With a register soffset the compiler was seen dropping
  the wait state that protects a 16-byte store's data registers from the next
  vector-ALU write, which corrupted a few lanes of the output now and then.
* All HIP code is built without packed-fp32 instructions, and no source
  writes one by hand.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hybrid_sliding_window_swa_amd", "csrc")


def _sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h", ".c")):
            with open(os.path.join(CSRC, name)) as f:
                yield name, f.read()


def _calls(text, fn):
    """Argument lists (top-level comma split) of every call of fn in text."""
    out = []
    for m in re.finditer(r"\b" + re.escape(fn) + r"\s*(<[^>]*>)?\s*\(", text):
        i, depth, args, cur = m.end(), 1, [], ""
        while depth:
            ch = text[i]
            if ch in "([{":
                depth += 1
            elif ch in ")]}":
                depth -= 1
            if depth == 0 or (ch == "," and depth == 1):
                args.append(cur.strip())
                cur = ""
            else:
                cur += ch
            i += 1
        out.append((text.count("\n", 0, m.start()) + 1, args))
    return out


def test_buffer_stores_pass_zero_soffset():
    seen = 0
    for name, text in _sources():
        for line, args in _calls(text, "buf_store16"):
            if args and args[0].startswith("u32x4 v"):
                continue  # the definition
            seen += 1
            assert args[-1] == "0", f"{name}:{line}: buf_store16 with soffset {args[-1]!r}"
        for line, args in _calls(text, "__builtin_amdgcn_raw_buffer_store_b128"):
            # only the wrapper may call the builtin, and it forwards soff
            assert name == "common.hpp" and args[3] == "(int)soff", f"{name}:{line}: direct buffer store"
    assert seen >= 2


def test_no_packed_fp32():
    import importlib.util
    spec = importlib.util.spec_from_file_location("swa_build", os.path.join(ROOT, "hybrid_sliding_window_swa_amd",
                                                                             "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    flags = " ".join(build.HIP_FLAGS)
    assert "-target-feature -Xclang -packed-fp32-ops" in flags
    for name, text in _sources():
        assert not re.search(r"v_pk_(add|mul|fma)_f32", text), name


if __name__ == "__main__":
    pytest.main([__file__, "-q"])
