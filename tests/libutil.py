"""Locate (and if needed build) libspechead.so for the tests."""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "drafter_lm_head_slimspec_amd")
LIB = os.path.join(PKG, "libspechead.so")
HEADER = os.path.join(ROOT, "include", "spechead.h")


def sources_newer_than_lib():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    srcs = glob.glob(os.path.join(PKG, "csrc", "*")) + [HEADER]
    return any(os.path.getmtime(s) > t for s in srcs)


def ensure_built():
    if sources_newer_than_lib():
        from drafter_lm_head_slimspec_amd import build
        build.build()
    return LIB


def header_functions():
    """Names of the functions declared in include/spechead.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))
