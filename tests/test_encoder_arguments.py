"""CPU checks of two arguments that the HIP key encoders rest on, by brute force against the
exact arithmetic of the definitions (no GPU; the encoders themselves are checked against the
oracle by the GPU parity tests).

* Midpoint screen (MSE-searched append): when fl(|y| rcp(g) + tiny) has its 17 significand
  bits below the top 7 at least 16 units away from 0 and from 2^17, the converter quotient
  fl(|y| rcp(fl(sigma g))) lies on the same side of every E2M1 midpoint t as the exact
  |y| / (sigma g), for every E4M3 scale sigma and for reciprocals within one ulp of exact.
* Candidate entries of the whole-wavefront search (fused decode step): the run codes
  first + v, v < 17, that pass the interval test, plus the absmax code when it lies outside
  the run, are exactly the oracle's candidate set of the block.
"""
import numpy as np

from oracle import nvfp4_oracle as O

MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
SIGMAS = np.array([float(O.e4m3_decode(c)) for c in range(1, 127)])
TINY = np.float64(np.frombuffer(np.uint32(0x00804000).tobytes(), dtype=np.float32)[0])
SCREEN_ULPS = 16


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def fma_tiny_f32(a32: np.ndarray, b32: np.float32) -> np.ndarray:
    """fl32(a * b + TINY) for fp32 a, b >= 0: a * b is exact in fp64, and the tiny positive
    addend only breaks a tie of the fp32 rounding upwards."""
    r = a32.astype(np.float64) * np.float64(b32) + TINY           # exact unless r ~ TINY
    w = r.astype(np.float32)
    lo = np.where(w.astype(np.float64) > r, np.nextafter(w, np.float32(0)), w)
    hi = np.nextafter(lo, np.float32(np.inf))
    d_lo, d_hi = r - lo.astype(np.float64), hi.astype(np.float64) - r
    return np.where(d_hi <= d_lo, hi, lo)


def screen_passes(y32: np.ndarray, rg32: np.float32) -> np.ndarray:
    b = fma_tiny_f32(np.abs(y32), rg32).view(np.uint32).astype(np.uint64)
    x = ((b << np.uint64(15)) + np.uint64(SCREEN_ULPS << 15)) & np.uint64(0xFFFFFFFF)
    return x >= np.uint64((2 * SCREEN_ULPS) << 15)


def reciprocals(x32: np.float32) -> list:
    """The correctly rounded fp32 reciprocal and its two neighbours (a 1-ulp reciprocal)."""
    r = np.float32(np.float64(1.0) / np.float64(x32))
    return [r, np.nextafter(r, np.float32(0)), np.nextafter(r, np.float32(np.inf))]


def near_midpoint_values(g: np.float32, rng, n: int) -> np.ndarray:
    """fp32 values at sigma t g (1 + k 2^-24) for random scales, midpoints and |k| <= 64."""
    sig = rng.choice(SIGMAS, n)
    t = rng.choice(MIDPOINTS, n)
    k = rng.integers(-64, 65, n)
    return f32(sig * t * np.float64(g) * (1.0 + k * 2.0 ** -24))


def test_midpoint_screen_keeps_every_decision():
    rng = np.random.default_rng(5)
    for g in (np.float32(0.0021), np.float32(3.7e-5), np.float32(2.0 ** -7)):
        y = np.concatenate([near_midpoint_values(g, rng, 6000),
                            f32(np.exp(rng.uniform(-12, 9, 3000)) * np.float64(g)),
                            np.zeros(4, dtype=np.float32)])
        for rg in reciprocals(g):
            ok = screen_passes(y, rg)
            assert np.all(ok[-4:])                               # zeros pass
            ay = np.abs(y[ok]).astype(np.float64)
            checked = 0
            for sigma in SIGMAS:
                u = np.float32(np.float64(sigma) * np.float64(g))
                if u < np.float32(2.0 ** -125):                # the encoder brackets these
                    continue
                for R in reciprocals(u):
                    z = (ay * np.float64(R)).astype(np.float32).astype(np.float64)
                    for t in MIDPOINTS:
                        exact_above = ay - t * sigma * np.float64(g)      # exact in fp64
                        assert np.all(exact_above != 0.0)
                        assert np.all((z > t) == (exact_above > 0.0)) and np.all(z != t)
                        checked += ay.size
            assert checked > 0
        # the screen lets most generic values through, and flags those on a midpoint
        if g != np.float32(2.0 ** -7):
            assert np.mean(screen_passes(y[6000:-4], reciprocals(g)[0])) > 0.99
        on_mid = f32(rng.choice(SIGMAS, 500) * rng.choice(MIDPOINTS, 500) * np.float64(g))
        assert not np.any(screen_passes(on_mid[on_mid > 0], reciprocals(g)[0]))


def first_code(S0: int, A: float, g: float) -> int:
    """The run's first code as the encoders form it: from S0 - 2 (at least 1), stepping up
    at most three times past codes whose scale is below A/7."""
    c = S0 - 2 if S0 >= 3 else 1
    for _ in range(3):
        if c < 126 and A - 7.0 * float(O.e4m3_decode(c)) * g > 0.0:
            c += 1
    return c


def in_run(c: int, A: float, g: float) -> bool:
    if c < 1 or c > 126:
        return False
    s = float(O.e4m3_decode(c))
    return not (A - 7.0 * s * g > 0.0) and not (A - 1.75 * s * g < 0.0)


def test_wavefront_search_entries_cover_the_candidates():
    rng = np.random.default_rng(6)
    # a generic tensor scale, and one with 5 significant bits so that 7 g sigma is exact
    for g in (np.float64(np.float32(0.0021)), np.float64(1.3125 * 2.0 ** -7)):
        A = f32(np.exp(rng.uniform(-16, 10, 3000)) * g).astype(np.float64)
        corners = np.concatenate([7.0 * SIGMAS * g, 1.75 * SIGMAS * g, [0.0]])   # run ends
        A = np.concatenate([A, corners[f32(corners).astype(np.float64) == corners]])
        S0 = O.absmax_scale_codes(A, g)
        cand = O.mse_candidates(A, g, S0)
        normal = (A >= 6.0 * g * 2.0 ** -6) & (A < 6.0 * g * 400.0)   # absmax scale normal, unsaturated
        third_round = n17 = 0
        for i in range(A.size):
            a, s0 = float(A[i]), int(S0[i])
            want = {int(c) for c in cand[i] if c >= 0}
            first = first_code(s0, a, float(g))
            entries = [first + v for v in range(17) if in_run(first + v, a, float(g))]
            if not in_run(s0, a, float(g)):
                entries.append(s0)
            assert set(entries) == want, (a, s0)
            assert len(entries) == len(set(entries))
            if i < 3000 and normal[i]:
                third_round += int(in_run(first + 16, a, float(g)) or not in_run(s0, a, float(g)))
            if i >= 3000 and 8 <= first <= 110 and a == 7.0 * float(O.e4m3_decode(first)) * float(g):
                assert in_run(first + 16, a, float(g))         # normal scales: a run of 17 codes
                n17 += 1
        # absmaxes whose absmax-to-6 scale is a normal E4M3 value below saturation skip the
        # third round (in this sample, always)
        assert np.count_nonzero(normal[:3000]) > 1000 and third_round == 0
        assert n17 > 0 or g == np.float64(np.float32(0.0021))
