"""Parity bars of the GPU tests against the fp64 oracle, shared by every GPU test file.

Max-abs error: fp32 1e-5; fp16/bf16 2e-2; fp8 KV (E5M2 or E4M3) 5e-2 against the
oracle fed the same dequantized values.  At long contexts the outputs are small
(about sqrt(e / n) for n visible keys with N(0,1) data), so the absolute bar alone
is loose there: every comparison also bounds rms(err) / rms(ref) (1e-2 for 16-bit
inputs, 2e-2 for fp8 KV, 1e-5 for fp32) and compares lse, natural log, to an
absolute max(bar, 1e-4) with the same -inf pattern (a row with no visible key).
"""

import sys

import numpy as np

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2, "e5m2": 5e-2, "e4m3": 5e-2}
RMS_BAR = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2, "e5m2": 2e-2, "e4m3": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare(name, kind, got, ref, got_lse=None, ref_lse=None):
    """Asserts the bars of `kind` on outputs (and lse when given); returns (max-abs, rms ratio)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    rel = mx / max(float(np.abs(ref).max()), 1e-30) if err.size else 0.0
    rms = float(np.sqrt((err ** 2).mean()) / max(np.sqrt((ref ** 2).mean()), 1e-30)) if err.size else 0.0
    say(f"  {name}: max|err|={mx:.3e} max|err|/max|ref|={rel:.3e} rms ratio={rms:.3e} (bar {TOL[kind]})")
    assert mx <= TOL[kind], f"{name}: max-abs error {mx} > {TOL[kind]}"
    assert rms <= RMS_BAR[kind], f"{name}: rms ratio {rms} > {RMS_BAR[kind]}"
    if got_lse is not None:
        gl = np.asarray(got_lse, np.float64)
        rl = np.asarray(ref_lse, np.float64)
        assert gl.shape == rl.shape, (gl.shape, rl.shape)
        assert (np.isfinite(gl) == np.isfinite(rl)).all(), f"{name}: lse -inf pattern differs"
        fin = np.isfinite(rl)
        if fin.any():
            lerr = float(np.abs(gl[fin] - rl[fin]).max())
            say(f"  {name}: lse max|err|={lerr:.3e}")
            assert lerr <= max(TOL[kind], 1e-4), f"{name}: lse error {lerr}"
    return mx, rms
