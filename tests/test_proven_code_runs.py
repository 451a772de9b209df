"""CPU check of the full-grid search's proven-code runs: in a chunk of 512 consecutive binary16
patterns (the E <= 8 layout: 64 lanes x 8 scales), a weight w' with |w'| <= fl32(fl32(s0 / 2)
(1 - 2^-20)) has code 0 at every scale of the chunk, and a weight with w' >= fl32(fl32((qmax - 1/4)
s1) (1 + 2^-20)) (or w' <= the same with qmin + 1/4) has the range end as its code there, s0 and s1
the chunk's smallest and largest scale.  The thresholds are formed in binary32 as the kernel forms
them; the codes are the screen's: round half to even of the binary32 product of w' and a
reciprocal within one rounding of 1/s (both neighbours of the correctly rounded reciprocal are
tried), then the clip.  Weights are placed at the thresholds and a few binary32 spacings around
them, pre-scaled as the kernel pre-scales (max |w'| in [1, 2))."""
import numpy as np
import pytest

CHUNK = 512
f32 = np.float32


def _grid():
    b = np.arange(1, 0x7C00, dtype=np.uint16)
    return b.view(np.float16).astype(np.float32)


def _codes(w, s, qmin, qmax):
    """Screen codes of weights w at scales s (outer product), for the three reciprocals within one
    binary32 rounding of 1/s."""
    r = (f32(1.0) / s).astype(np.float32)
    out = []
    for rr in (r, np.nextafter(r, f32(0)), np.nextafter(r, f32(np.inf))):
        x = (w[:, None] * rr[None, :]).astype(np.float32)
        out.append(np.clip(np.rint(x), qmin, qmax))
    return out


@pytest.mark.parametrize("qmin,qmax", [(-8, 7), (-4, 3), (0, 15), (-128, 127)])
def test_proven_code_runs_hold_at_every_scale_of_their_chunk(qmin, qmax):
    grid = _grid()
    rng = np.random.default_rng(99 + qmax)
    # pre-scaling by a power of two puts max |w'| in [1, 2): scales run over the grid times 2^k
    for k in (0, 5, 12, 20):
        g = (grid * f32(2.0 ** k)).astype(np.float32)
        chunks = rng.choice(np.arange(0, g.size // CHUNK), size=12, replace=False)
        for c in chunks:
            s = g[c * CHUNK:(c + 1) * CHUNK]
            s0, s1 = s[0], s[-1]
            tz = f32(f32(f32(0.5) * s0) * f32(1.0 - 2.0 ** -20))
            near = np.concatenate([np.nextafter(np.full(4, tz), f32(0)), [tz]]).astype(np.float32)
            wz = np.concatenate([near, -near, (rng.uniform(0, 1, 64) * tz).astype(np.float32)])
            wz = wz[(np.abs(wz) <= tz) & (np.abs(wz) < 2.0)]
            for q in _codes(wz, s, qmin, qmax):
                assert np.all(q == 0), (k, c)
            if qmax > 0:
                tf = f32(f32(f32(qmax - 0.25) * s1) * f32(1.0 + 2.0 ** -20))
                wf = np.array([tf, np.nextafter(tf, f32(np.inf)), f32(tf * f32(1.5))], np.float32)
                for q in _codes(wf, s, qmin, qmax):
                    assert np.all(q == qmax), (k, c)
            if qmin < 0:
                ta = f32(f32(f32(qmin + 0.25) * s1) * f32(1.0 + 2.0 ** -20))
                wa = np.array([ta, np.nextafter(ta, f32(-np.inf)), f32(ta * f32(1.5))], np.float32)
                for q in _codes(wa, s, qmin, qmax):
                    assert np.all(q == qmin), (k, c)
            # the thresholds are tight enough to matter: just above the code-0 bound, some scale
            # of the chunk rounds a weight of twice the bound away from 0
            w2 = np.array([f32(2.0) * tz], np.float32)
            assert np.any(_codes(w2, s, qmin, qmax)[0] != 0) or qmax == 0
