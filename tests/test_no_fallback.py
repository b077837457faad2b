"""The binding has no fallback: without the built HIP library it refuses to import."""
import subprocess
import sys
import textwrap
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def test_binding_refuses_to_import_without_the_library():
    code = textwrap.dedent("""
        import os
        real = os.path.exists
        os.path.exists = lambda p: False if str(p).endswith("libawq.so") else real(p)
        try:
            import weight_only_int4_act_amd.awq
        except ImportError as e:
            assert "no fallback" in str(e), e
            print("refused")
        else:
            raise SystemExit("imported without libawq.so")
    """)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "refused" in r.stdout
