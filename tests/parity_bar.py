"""The parity bar the GPU tests apply, shared with its CPU negative controls.

rel-L2 = ||got - ref|| / ||ref|| <= 3e-3 over the compared rows, and
|got_i - ref_i| <= 2e-2 * max(1, |ref_i|) per element, where ref is the
oracle's unrounded fp64 result and got the bf16 output widened to fp64; got
must also be finite.
"""
import numpy as np

REL_L2 = 3e-3
ELEM = 2e-2


def as_f64(x):
    """A torch tensor (any device, any float dtype) or an array, as fp64 numpy."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    return x.float().cpu().double().numpy()


def parity_stats(got, ref, seqs=None):
    """(rel-L2, worst |err| / element bound, all finite) of got against ref."""
    g = as_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    if seqs is not None:
        g, r = g[seqs], r[seqs]
    finite = bool(np.isfinite(g).all())
    err = g - r
    nrm = np.linalg.norm(r)
    rel = np.linalg.norm(err) / nrm if nrm > 0 else np.linalg.norm(err)
    bound = ELEM * np.maximum(1.0, np.abs(r))
    worst = float((np.abs(err) / bound).max()) if err.size else 0.0
    return float(rel), worst, finite


def check_parity(got, ref, seqs=None, what=""):
    rel, worst, finite = parity_stats(got, ref, seqs)
    assert finite, "%s: non-finite output" % what
    print("%s: rel-L2 %.3e, worst |err|/bound %.3f" % (what, rel, worst))
    assert rel <= REL_L2, "%s: rel-L2 %.3e > %.1e" % (what, rel, REL_L2)
    assert worst <= 1.0, "%s: element error %.3f x bound" % (what, worst)
    return rel
