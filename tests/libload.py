"""Load the built library for the host-side tests (building it first when no
library is there), without importing the package before the build."""
from __future__ import annotations

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def build_module():
    spec = importlib.util.spec_from_file_location(
        "kv_cache_streaming_amd_build", os.path.join(ROOT, "kv_cache_streaming_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def kv_module():
    b = build_module()
    if not os.path.exists(b.LIB):
        b.build()
    import kv_cache_streaming_amd as kv
    return kv
