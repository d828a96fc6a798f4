"""The checked build (device-side invariant tests) on the GPU.

tests/checked_cases.py runs its cases in a child process on
libfwpkm_checked.so and here on the product library.  On every well-formed
case no check may fire, and the two builds must agree: selected slots
exactly, values to float32 rounding (the checks add no arithmetic, though the
compiler may schedule the kernels' floating point differently).  On the case
with NaN queries in dot mode the checked build must report the non-finite
weights as FWPKM_ERR_DEVICE_CHECK, where the product build cannot tell.
"""

import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from sparse_weight_memory_amd import _lib

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import checked_cases  # noqa: E402


@pytest.mark.gpu
def test_checked_build_agrees_and_reports(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    if not os.path.exists(_lib.CHECKED_LIB_PATH):
        pytest.skip("checked build missing: python -m sparse_weight_memory_amd.build --checked")
    out = str(tmp_path / "checked.npz")
    env = dict(os.environ, FWPKM_LIB_PATH=_lib.CHECKED_LIB_PATH)
    print("[checked] child process on the checked build", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "checked_cases.py"), out], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    got = np.load(out)
    status = json.load(open(out + ".json"))
    assert status["checked_build"] == 1
    assert _lib.load().fwpkm_checked_build() == 0
    for name in checked_cases.CASES:
        print(f"[checked] {name} on the product build", flush=True)
        ref, code, msg = checked_cases.run(name)
        assert code == 0, f"{name}: product build failed: {msg}"
        st = status[name]
        if name == "nan_dot":
            assert st["code"] == _lib.ERR_DEVICE_CHECK, st
            assert "selection weight" in st["message"], st
            continue
        assert st["code"] == 0, f"{name}: {st['message']}"
        for key, want in ref.items():
            have = got[f"{name}/{key}"]
            if key.startswith("slots"):
                np.testing.assert_array_equal(have, want, err_msg=f"{name}/{key}")
            else:
                np.testing.assert_allclose(have, want, rtol=1e-5, atol=1e-6, err_msg=f"{name}/{key}")
