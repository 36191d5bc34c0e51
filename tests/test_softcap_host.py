"""CPU test of the kernels' logit softcap (Muse Glimmer page, Details >
Softcap: z = T tanh(m a / T)) against float64 tanh.

``tests/host/softcap_host.cpp`` compiles the softcap helpers of
``device_common.hpp`` (CapSeries with its folded series coefficients, the
range switch, the exponential form, the unfolded series for |m / T| > 2^12)
for the host and applies them to raw accumulator values exactly as the fused
forward epilogue and the materialised-logits epilogue do.  Bound: relative
error at most 4e-7 against T tanh(m a / T) evaluated in float64 on the same
float32 inputs, over |m a / T| from 1e-8 to 20 (both signs, the series range
|m a / T| < 1/4 and the exponential form beyond it, the switch itself), for
T from 1e-6 to 1e4 and m in [-1, 1]; exact zero at a = 0; every value finite.
On the GPU the exponential form uses the hardware exp2 and reciprocal; the
GPU softcap test checks those kernels' logits against the same bound.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BOUND = 4e-7


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    hipcc = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("softcap") / "softcap_host")
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-ffp-contract=off",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "linear_cross_entropy_gemm_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "softcap_host.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe


def capped(exe, m, T, a):
    a = np.asarray(a, dtype=np.float32)
    inp = struct.pack("ff", m, T) + struct.pack("q", a.size) + a.tobytes()
    out = subprocess.run([exe], input=inp, capture_output=True, check=True)
    return np.frombuffer(out.stdout, dtype=np.float32).astype(np.float64)


def reference(m, T, a):
    m64, T64 = float(np.float32(m)), float(np.float32(T))
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    return T64 * np.tanh(m64 * a64 / T64) if T > 0 else m64 * a64


def grid(m, T):
    """Raw accumulator values a with |m a / T| spanning both branches and the
    switch at 1/4 (with its neighbouring float32 values)."""
    s = abs(np.float32(m) / np.float32(T))
    x = np.concatenate([np.linspace(0.0, 20.0, 20001), np.logspace(-8, 1.5, 2000), [0.25]])
    a = (x / s).astype(np.float32)
    edge = np.float32(0.25 / s)
    near = [np.nextafter(edge, np.float32(0)), edge, np.nextafter(edge, np.float32(1e30))]
    a = np.concatenate([a, np.array(near, dtype=np.float32)])
    return np.concatenate([a, -a])


@pytest.mark.parametrize("T", [1e-6, 1.5e-5, 1e-3, 0.5, 1.0, 2.0, 30.0, 1e4])
@pytest.mark.parametrize("m", [-1.0, -0.37, 0.5, 1.0])
def test_softcap_matches_float64_tanh(harness, m, T):
    a = grid(m, T)
    z = capped(harness, m, T, a)
    ref = reference(m, T, a)
    assert np.all(np.isfinite(z))
    nz = ref != 0.0
    rel = np.abs(z[nz] - ref[nz]) / np.abs(ref[nz])
    assert rel.max() <= BOUND, (m, T, float(rel.max()))
    assert np.all(z[~nz] == 0.0)
    # odd, and never above the cap
    assert np.all(z[: a.size // 2] == -z[a.size // 2:])
    assert np.all(np.abs(z) <= np.float32(T))


def test_no_cap_is_the_multiplied_logit(harness):
    a = np.linspace(-50.0, 50.0, 1001, dtype=np.float32)
    z = capped(harness, 0.5, 0.0, a)
    assert np.array_equal(z, (a * np.float32(0.5)).astype(np.float64))


def test_series_and_exponential_form_agree_at_the_switch(harness):
    """At |m a / T| = 1/4 the two forms meet: consecutive float32 inputs across
    the switch give outputs within the bound of each other (no jump)."""
    for m, T in [(0.5, 30.0), (1.0, 1.0), (-0.37, 2.0), (1.0, 1e-5)]:
        s = abs(np.float32(m) / np.float32(T))
        edge = np.float32(0.25 / s)
        a = [edge]
        for _ in range(8):
            a.insert(0, np.nextafter(a[0], np.float32(0)))
            a.append(np.nextafter(a[-1], np.float32(1e30)))
        a = np.array(a, dtype=np.float32)
        z = capped(harness, m, T, a)
        ref = reference(m, T, a)
        assert np.max(np.abs(z - ref) / np.abs(ref)) <= BOUND
        assert np.all(np.diff(z) * np.sign(m) >= -BOUND * np.abs(z[:-1]))
