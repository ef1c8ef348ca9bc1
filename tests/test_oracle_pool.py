"""The pooled oracle (BF ranges in worker processes) against one serial oracle call."""
import numpy as np

from oracle import ssb_oracle as O
from oracle.pool import OraclePool
from synth import WORKLOADS, cached_counts


def test_pool_equals_serial_small():
    w = WORKLOADS["small"]
    counts = cached_counts(w)
    g = O.OGeom.from_any(w.geometry)
    dc = O.dc_value(counts)
    params = (-31.0, 7.5, 1.3)
    with OraclePool(lambda a, b: counts[a:b], shape=counts.shape, workers=3, chunk_bf=100) as pool:
        s1, s2 = pool.moments(g, params, dc)
        r1, r2 = O.bf_moments(g, counts, params, dc)
        assert abs(s2 - r2) <= 1e-13 * r2 and np.max(np.abs(s1 - r1)) <= 1e-12
        assert abs(pool.loss(g, params, dc) - O.loss(g, counts, params, dc)) <= 1e-13
        p1, s1r = pool.moments(g, params, dc, 37, 131)
        q1, q2 = O.bf_moments(g, counts[37:131], params, dc, list(range(37, 131)))
        assert abs(s1r - q2) <= 1e-13 * q2 and np.max(np.abs(p1 - q1)) <= 1e-12
        ph, psi = pool.object_wave(g, params, dc)
        rph, rpsi = O.object_wave(g, counts, params, dc)
        assert np.max(np.abs(psi - rpsi)) <= 1e-12 * np.abs(rpsi).max()
        assert np.max(np.abs(np.angle(np.exp(1j * (ph - rph))))) < 1e-10
        f1, f2 = pool.moments(g, params, dc, full_plane=True)
        g1, g2 = O.bf_moments_full_plane(g, counts, params, dc)
        assert abs(f2 - g2) <= 1e-13 * g2 and np.max(np.abs(f1 - g1)) <= 1e-12
