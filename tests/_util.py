"""Small comparison helpers shared by the tests (no method arithmetic)."""
import numpy as np


def rel_err(x, ref):
    """Normwise relative error max|x - ref| / max|ref| (elementwise relative
    error is meaningless where ref is close to zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    return num / den if den > 0 else num
