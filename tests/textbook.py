"""Independent textbook formulas used to pin the oracle (no matrix products).

Coordinate-wise Adam without bias correction, as the pipeline-staleness page
writes the update (section 2.1) and the three-layer-decoupling page writes the
second-moment recurrence (section 2.1). The rotated step must reduce to this
when both bases are identities and never refreshed.
"""

import numpy as np


def f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def bf16_via_torch(x):
    """bfloat16 rounding computed by torch's own float32 -> bfloat16 cast.

    Only exact for inputs that are already binary32 values (single rounding).
    """
    import torch
    t = torch.from_numpy(np.asarray(x, np.float32).copy())
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def adam_coordinatewise(w, m, v, g, beta1, beta2, eps, lr, m_round):
    """One Adam step, element by element, in float64 with binary32 hyper-params."""
    b1, b2, e, a = (float(np.float32(x)) for x in (beta1, beta2, eps, lr))
    w = np.array(w, np.float64, copy=True)
    m = np.array(m, np.float64, copy=True)
    v = np.array(v, np.float64, copy=True)
    g = np.asarray(g, np.float64)
    it = np.nditer([w, m, v, g], flags=["multi_index"], op_flags=[["readwrite"]] * 3 + [["readonly"]])
    for wi, mi, vi, gi in it:
        mi[...] = m_round(b1 * mi + (1.0 - b1) * gi)
        vi[...] = f32(b2 * vi + (1.0 - b2) * gi * gi)
        wi[...] = f32(wi - a * (mi / (np.sqrt(vi) + e)))
    return w, m, v
