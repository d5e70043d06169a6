"""Error bounds for the GPU checks of the token-gated attention backward.

Test code, not part of the oracle: the oracle returns gradients only.  This
module describes how large the GPU's rounding error in the score, gain and
temperature gradients may be, so the tests can hold each element to a bar.

Those three gradients are sums of dS_ij = p_ij (dp_ij - D_i) terms, and they
cancel (every softmax row of dS sums to zero), so a bar relative to the result
does not fit them element by element.  On the GPU, D_i = dout_i . out_i is
formed from the forward's rounded output, off by at most ~2^-8 relative per
element, so |dD_i| <= 2^-8 A_i with A_i = sum_f |dout_if out_if|, and every
dS_ij carries an error of at most 2^-8 p_ij A_i plus its own rounding.  The
summation bound then gives |error| <= 2^-8 * the sum of the terms' magnitudes
with dS_ij replaced by

    mag_ij = p_ij (|dp_ij - D_i| + A_i).

``term_magnitude_sums`` computes those sums in float64 with numpy; it is
pinned in tests/test_oracle_pins.py against a plain loop over every (head,
row, key) triple on tiny inputs.
"""

import math

import numpy as np


def term_magnitude_sums(q, k, v, key_score, gain, tau, dout, row_block: int = 256):
    """Per key j: |g_h| sum_{h,i} mag_ij (score gradient); per head h:
    sum_ij mag_ij |s_j| (gain gradient) and sum_ij mag_ij |q_i.k_j| / (sqrt(d)
    tau_h^2) (temperature gradient).  Shapes as the oracle's backward; returns
    dict(dscore, dgain, dtau) of float64 arrays."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    m, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    dout = np.asarray(dout, dtype=np.float64).reshape(m, hq, d)
    s = np.asarray(key_score, dtype=np.float64).reshape(m)
    gain = np.asarray(gain, dtype=np.float64).reshape(hq)
    tau = np.asarray(tau, dtype=np.float64).reshape(hq)
    sc_score = np.zeros(m)
    sc_gain = np.zeros(hq)
    sc_tau = np.zeros(hq)
    for h in range(hq):
        g = h // group
        kh = k[:, g, :].astype(np.float64)
        vh = v[:, g, :].astype(np.float64)
        scale = 1.0 / (math.sqrt(d) * tau[h])
        for b0 in range(0, m, row_block):
            rb = np.arange(b0, min(b0 + row_block, m))
            kend = int(rb[-1]) + 1
            qk = q[rb, h, :].astype(np.float64) @ kh[:kend].T
            logits = qk * scale + gain[h] * s[None, :kend]
            logits = np.where(np.arange(kend)[None, :] <= rb[:, None], logits, -np.inf)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dob = dout[rb, h, :]
            dp = dob @ vh[:kend].T
            dsum = (p * dp).sum(axis=1, keepdims=True)
            a = np.abs(dob * (p @ vh[:kend])).sum(axis=1, keepdims=True)
            mag = p * (np.abs(dp - dsum) + a)
            sc_score[:kend] += abs(gain[h]) * mag.sum(axis=0)
            sc_gain[h] += (mag * np.abs(s[None, :kend])).sum()
            sc_tau[h] += (mag * np.abs(qk)).sum() / (math.sqrt(d) * tau[h] ** 2)
    return dict(dscore=sc_score, dgain=sc_gain, dtau=sc_tau)
