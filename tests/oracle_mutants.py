"""Planted mistakes in the oracle, for checking that its pins catch them (CPU only).

build(tmp_dir, function, old, new) copies oracle/gs_oracle.c, replaces the text `old` by `new` inside the definition
of `function` (it must occur there exactly once), compiles the copy with the oracle's own flags and returns the
library's path; `oracle.variant(path)` then runs the oracle's wrappers against it. The oracle's source itself is never
changed."""
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "gs_oracle.c")


def function_span(text, function):
    """[start, end) of the definition of `function` (return type at the start of a line, up to its closing brace
    at the start of a line)."""
    m = re.search(r"^[A-Za-z_][^\n;]*\b" + re.escape(function) + r"\(", text, re.M)
    if m is None:
        raise KeyError(function)
    end = text.index("\n}\n", m.start()) + 3
    return m.start(), end


def mutate(text, function, old, new):
    a, b = function_span(text, function)
    body = text[a:b]
    if body.count(old) != 1:
        raise ValueError(f"{old!r} occurs {body.count(old)} times in {function}")
    return text[:a] + body.replace(old, new) + text[b:]


def build(tmp_dir, function, old, new, name=None):
    src = mutate(open(SOURCE).read(), function, old, new)
    name = name or re.sub(r"\W+", "_", f"{function}_{abs(hash((old, new)))}")
    c_path = os.path.join(str(tmp_dir), name + ".c")
    so_path = os.path.join(str(tmp_dir), name + ".so")
    with open(c_path, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
                           "-Wno-unknown-pragmas", c_path, "-o", so_path, "-lm"])
    return so_path
