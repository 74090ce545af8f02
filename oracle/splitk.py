"""Split-K decode attention: partial softmax sums per partition, then an exact merge.

Test infrastructure only (see the package docstring).

The pages do not split a sequence. Long sequences are cut into partitions of a
fixed number of tokens so that many workgroups can share one sequence; each
partition keeps its own maximum m_p, its sum of exponentials l_p and its
unnormalised output o_p, and the merge rescales them to a common maximum:

    M = max_p m_p,  out = sum_p e^(m_p - M) o_p  /  sum_p e^(m_p - M) l_p

which equals the single-pass softmax exactly in real arithmetic. This module
computes that in float64 so a test can hold it against
``attention.contiguous_decode_attn``.
"""

import numpy as np


def partition_then_merge(q_i, K, V, sigma, part):
    """[Hq][d]: attention over contiguous float64 K/V via partitions of ``part`` tokens."""
    Hq, d = q_i.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    qg = q_i.reshape(Hkv, G, d)
    ms, ls, os_ = [], [], []
    for start in range(0, L, part):
        Kp = K[start:start + part].transpose(1, 0, 2)
        Vp = V[start:start + part].transpose(1, 0, 2)
        s = sigma * (qg @ Kp.transpose(0, 2, 1))         # [Hkv][G][Lp]
        m = s.max(axis=-1, keepdims=True)
        p = np.exp(s - m)
        ms.append(m)
        ls.append(p.sum(axis=-1, keepdims=True))
        os_.append(p @ Vp)
    M = np.max(np.stack(ms), axis=0)
    num = sum(np.exp(m - M) * o for m, o in zip(ms, os_))
    den = sum(np.exp(m - M) * l for m, l in zip(ms, ls))
    return (num / den).reshape(Hq, d)
