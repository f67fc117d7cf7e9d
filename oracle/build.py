"""Compile the fp64 oracle into ``oracle/liboracle.so`` with gcc and OpenMP.

TEST INFRASTRUCTURE: the library this builds is loaded only by the tests, the
smoke check and the benchmark's CPU-baseline leg.

``build_variant`` compiles a copy of the source with textual substitutions; the
oracle's own tests use it to plant mistakes and check that its pins catch them.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "paged_attn_oracle.c")
APPEND_SRC = os.path.join(HERE, "kv_append_oracle.c")
PREFILL_SRC = os.path.join(HERE, "prefill_attn_oracle.c")
SOURCES = [SRC, APPEND_SRC, PREFILL_SRC]
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def _compile(srcs: list[str], out: str, include_dir: str) -> None:
    cmd = ["gcc", *CFLAGS, f"-I{include_dir}", "-o", out + ".tmp", *srcs, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)


def build(out: str = LIB) -> str:
    """Compile the oracle; returns the path of the shared library."""
    _compile(SOURCES, out, HERE)
    return out


def build_variant(substitutions: list[tuple[str, str]], out_dir: str | None = None,
                  source: str = SRC) -> str:
    """Compile a copy of the oracle with each ``(old, new)`` text replaced once
    in ``source`` (one of ``SOURCES``); the other sources are built unchanged.

    Raises ``ValueError`` if some ``old`` text is not found exactly once.
    """
    with open(source) as f:
        text = f.read()
    for old, new in substitutions:
        if text.count(old) != 1:
            raise ValueError(f"substitution target not unique: {old!r}")
        text = text.replace(old, new)
    d = out_dir or tempfile.mkdtemp(prefix="oracle_variant_")
    src = os.path.join(d, "variant.c")
    with open(src, "w") as f:
        f.write(text)
    out = os.path.join(d, "libvariant.so")
    _compile([src if s == source else s for s in SOURCES], out, HERE)
    return out


if __name__ == "__main__":
    print(build())
