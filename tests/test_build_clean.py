"""The library builds from a clean checkout: the tracked files alone, with no libnvfp4.so present,
through both documented routes (the package's build module, then the graft entry point, which
also compiles the C oracle and loads the library), and the result exports every function the C
header declares.  CPU only (hipcc cross-compiles for gfx950)."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "nvfp4.h")).read(), flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


@pytest.mark.skipif(shutil.which("git") is None or not os.path.isdir(os.path.join(ROOT, ".git")),
                    reason="needs the git checkout")
def test_clean_checkout_builds(tmp_path):
    files = subprocess.run(["git", "ls-files", "-z"], cwd=ROOT, capture_output=True, check=True).stdout
    dst = tmp_path / "tree"
    for rel in filter(None, files.decode().split("\0")):
        src = os.path.join(ROOT, rel)
        if not os.path.isfile(src):  # deleted in the working tree
            continue
        os.makedirs(os.path.dirname(dst / rel), exist_ok=True)
        shutil.copy2(src, dst / rel)
    lib = dst / "bit_gemm_nvfp4_amd" / "libnvfp4.so"
    assert not lib.exists()
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "bit_gemm_nvfp4_amd.build"], cwd=dst, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    assert lib.exists()
    os.remove(lib)
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__; __graft_entry__.build()"], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    out = subprocess.run(["nm", "-D", "--defined-only", str(lib)], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    missing = _declared() - exported
    assert not missing, missing
