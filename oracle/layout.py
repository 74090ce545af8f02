"""V pool shape: the sub-tile view the oracle indexes.

Test infrastructure only (see the package docstring).

The V pool holds, per (block, kv head), the block's bs tokens in sub-tiles of
vs = min(bs, 16) tokens, each channel-major: [P][Hkv][bs/vs][d][vs]. For bs <= 16
there is one sub-tile and the pool may equally be given as [P][Hkv][d][bs].
"""

import numpy as np


def v_view5(pool, bs):
    """The V pool as a [P][Hkv][bs/vs][d][vs] view (no copy)."""
    pool = np.asarray(pool)
    vs = min(bs, 16)
    if pool.ndim == 5:
        if pool.shape[2] * pool.shape[4] != bs or pool.shape[4] != vs:
            raise ValueError(f"V pool shape {pool.shape} does not match bs={bs}")
        return pool
    if pool.ndim == 4 and bs <= 16 and pool.shape[3] == bs:
        P, Hkv, d, _ = pool.shape
        return pool.reshape(P, Hkv, 1, d, bs)
    raise ValueError(f"V pool shape {pool.shape} does not match bs={bs}")
