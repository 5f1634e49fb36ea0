"""The sampled-accept comparisons skip a request only when the oracle marks
it exempt.  The band the ratio test states (|u - min(1, p/q)| < 1e-6) is
the only reason a request of the committed seeds may be skipped: these
checks fail a test whose seed puts a residual mass below 1e-6 or a terminal
draw within 2e-8 of a CDF edge, so that no request is skipped silently for
those reasons."""
import numpy as np

Z_BAND = 1e-6
DRAW_BAND = 2e-8


def other_exemptions(o):
    """Requests the oracle output `o` would exempt for a reason other than
    the ratio-test band."""
    return np.nonzero((np.asarray(o["z_min"]) < Z_BAND) |
                      (np.asarray(o["draw_margin"]) < DRAW_BAND))[0]


def assert_only_ratio_band(o, label=""):
    other = other_exemptions(o)
    assert other.size == 0, (f"{label}: requests exempt outside the ratio-test band: "
                             f"{other.tolist()[:16]} (z_min {np.asarray(o['z_min'])[other][:4]}, "
                             f"draw_margin {np.asarray(o['draw_margin'])[other][:4]})")
