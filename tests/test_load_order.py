"""The binding loads libpkv.so on torch's HIP runtime: loading the library
before anything else has imported torch still leaves exactly one
libamdhip64 mapped in the process (torch's), so the library and torch share
one runtime, its devices and its streams."""

import subprocess
import sys
import textwrap
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


def test_library_binds_to_torchs_runtime():
    if not (ROOT / "paged_kv_cache_map_amd" / "libpkv.so").exists():
        pytest.skip("libpkv.so is not built")
    code = textwrap.dedent("""
        import sys
        sys.path.insert(0, %r)
        import paged_kv_cache_map_amd as pkv
        pkv.library()
        import torch, os
        maps = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l]
        paths = sorted(set(os.path.realpath(p) for p in maps))
        torch_lib = os.path.realpath(os.path.join(os.path.dirname(torch.__file__), "lib"))
        print(len(paths), all(p.startswith(torch_lib) for p in paths))
    """ % str(ROOT))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["1", "True"], out.stdout
