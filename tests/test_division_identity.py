"""Runs tests/division_identity.c: exhaustive host-side proof of the two
division shortcuts in the activation quantizer (see the C file's header)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the check")
def test_division_identities_exhaustive(tmp_path):
    exe = str(tmp_path / "division_identity")
    subprocess.run(["gcc", "-O2", "-mfma", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "division_identity.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert "quotient identity: 0 mismatches" in out.stdout
    assert "scale identity: 0 mismatches" in out.stdout
