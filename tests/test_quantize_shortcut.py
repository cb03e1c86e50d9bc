"""CPU check of the argument behind the GPU quantiser's division shortcut.

The kernels compute q = rne(fl32(x / s)) as rne(fl32(x * rc)) with rc the
hardware reciprocal of s (relative error <= 2^-23), and fall back to the IEEE
division whenever fl32(x * rc) lies within 2^-13 of a half-integer. This test
emulates rc as any float32 within one ulp of fl32(1/s) and checks, over random
scales and dense sweeps around every half-integer boundary, that whenever the
shortcut is taken it agrees with numpy's IEEE float32 division.
"""

import numpy as np

F32 = np.float32


def _shortcut_mismatches(amax, rng):
    s = F32(amax / F32(127))
    r0 = F32(1) / s
    total = taken = bad = 0
    k = np.arange(-128, 128, dtype=np.float64) + 0.5
    center = (k * np.float64(s)).astype(np.float32)
    sweeps = [center]
    up = dn = center
    for _ in range(24):
        up = np.nextafter(up, F32(np.inf))
        dn = np.nextafter(dn, F32(-np.inf))
        sweeps += [up, dn]
    sweeps.append((rng.uniform(-1, 1, 4000) * amax).astype(np.float32))
    x = np.concatenate(sweeps)
    x = x[np.abs(x) <= amax]
    exact = np.rint(x / s)
    for rc in (np.nextafter(r0, F32(-np.inf)), r0, np.nextafter(r0, F32(np.inf))):
        y = (x * F32(rc)).astype(np.float32)
        ry = np.rint(y)
        fast = np.abs(np.abs(y - ry) - F32(0.5)) > F32(2.0 ** -13)
        total += x.size
        taken += int(fast.sum())
        bad += int((exact[fast] != ry[fast]).sum())
    return total, taken, bad


def test_reciprocal_shortcut_is_exact_when_taken():
    rng = np.random.default_rng(0)
    total = taken = bad = 0
    for amax in np.exp(rng.uniform(np.log(1e-28), np.log(1e30), 60)).astype(np.float32):
        t, f, b = _shortcut_mismatches(F32(amax), rng)
        total, taken, bad = total + t, taken + f, bad + b
    assert bad == 0
    assert taken > 0.25 * total       # most inputs are near-tie sweeps here; random ones take it
