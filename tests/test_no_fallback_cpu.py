"""The product path has no CPU fallback: without the built HIP library the
binding raises instead of computing anything, and neither the binding nor
the kernels' sources import or link the oracle."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_raises_without_library():
    code = (
        "import w8a8_post_quantization_amd as sq\n"
        "sq.LIB_PATH = '/nonexistent/libsq.so'\n"
        "sq._lib = None\n"
        "try:\n"
        "    sq.lib()\n"
        "except ImportError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('no error')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "no CPU fallback" in r.stdout


def test_product_sources_do_not_use_the_oracle():
    pkg = os.path.join(ROOT, "w8a8_post_quantization_amd")
    srcs = [os.path.join(dp, f) for dp, _, fs in os.walk(pkg) for f in fs
            if f.endswith((".py", ".hip", ".cpp", ".h"))]
    srcs.append(os.path.join(ROOT, "include", "sq.h"))
    for path in srcs:
        text = open(path, encoding="utf-8").read()
        assert not re.search(r"\bimport\s+oracle\b|\bfrom\s+oracle\b|sq_oracle|orc_", text), path
