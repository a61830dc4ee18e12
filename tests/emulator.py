"""Error emulator of the fused attention kernel (test infrastructure).

Not the oracle: the oracle (oracle/attention.py) is the plain definition in
fp64.  This module follows the blockwise online-softmax recurrence of
"ops-transformer：Transformer算子融合与推理加速实战" §3.2 (keys processed tile
by tile with a running row maximum and sum, the output rescaled when the
maximum rises) in the precisions the kernel uses (§2.4: 16-bit storage and
products, fp32 statistics and accumulation, one rounding to the storage type
at the end), so that its distance to the oracle predicts the GPU's:

* scores in fp32 from the 16-bit inputs, scaled by scale·log2(e) inside the
  exponent argument (one fused multiply-add), exponentials in base 2;
* key tiles of 64 keys (32 for fp32), masked entries -inf;
* the running maximum of a row is raised only when some row of its group of
  32 rows (one wavefront) sees a tile maximum more than 2^8 above its own
  (otherwise the stale maximum is kept and the output is not rescaled);
* P rounded to the input type (fp32 kept as is) before the P·V product, the
  row sum taken over those rounded values, LSE over the unrounded ones;
* O divided by the row sum in fp32, then rounded to the storage type.

It does not model the order of the fp32 sums inside one product, the
hardware exponential's last-bit error, or the split of a causal block's keys
between two groups (a different association of the same sums): effects of
the size of the ones modelled.  With ``exact=True`` every step is fp64 with
no rounding, and the result must equal the oracle to rounding: that pins the
recurrence itself (tests/test_emulator.py).
"""

import numpy as np

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453
RESCALE_LOG2 = 8.0


def round_bf16(x):
    """float32 array -> nearest bfloat16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def round_to(x, dtype):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    return np.asarray(x, dtype=np.float32)


def emulate_head(qh, kh, vh, scale, dtype, causal=False, key_len=None, exact=False, rows=None):
    """One (batch, query head): qh (S, D), kh and vh (S, D) of the kv head, as
    float arrays holding the values the kernel reads.  Returns (O, LSE) as
    float64: O (R, D) rounded to ``dtype`` (R = len(rows), default all S
    rows), LSE (R,).  Unless ``exact``, ``rows`` must be whole, aligned
    groups of 32 rows (the rescale decision is taken per group)."""
    S, D = qh.shape
    key_len = S if key_len is None else int(min(max(key_len, 0), S))
    rows = np.arange(S) if rows is None else np.asarray(rows)
    if not exact:
        # the rescale decision is taken per group of 32 rows (one wavefront)
        assert len(rows) % 32 == 0 and rows[0] % 32 == 0
        assert np.all(rows.reshape(-1, 32) == rows.reshape(-1, 32)[:, :1] + np.arange(32))
    ft = np.float64 if exact else np.float32
    bn = 32 if dtype == "fp32" else 64
    q = qh[rows].astype(ft)
    k = kh.astype(ft)
    v = vh.astype(ft)
    R = len(rows)
    sl2 = ft(scale) * ft(LOG2E)
    m_run = np.full(R, -np.inf, ft)
    l_run = np.zeros(R, ft)
    l_lse = np.zeros(R, ft)
    o = np.zeros((R, D), ft)
    for t0 in range(0, S, bn):
        t1 = min(t0 + bn, S)
        s = q @ k[t0:t1].T                                    # (R, n) scores
        j = np.arange(t0, t1)[None, :]
        ok = j < key_len
        if causal:
            ok = ok & (j <= rows[:, None])
        s = np.where(ok, s, -np.inf).astype(ft)
        mxs = s.max(axis=1) * sl2
        if exact:
            need = mxs > m_run
        else:
            grp = (mxs > m_run + ft(RESCALE_LOG2)).reshape(-1, 32).any(axis=1)
            need = np.repeat(grp, 32)
        m_new = np.where(need, np.maximum(m_run, mxs), m_run)
        with np.errstate(invalid="ignore"):
            alpha = np.where(need & (m_new != -np.inf), np.exp2(m_run - m_new), 1.0).astype(ft)
        l_run *= alpha
        l_lse *= alpha
        o *= alpha[:, None]
        m_run = m_new
        m_use = np.where(m_run == -np.inf, 0.0, m_run).astype(ft)
        with np.errstate(invalid="ignore", over="ignore"):
            arg = s * sl2 - m_use[:, None] if exact else (s.astype(np.float64) * sl2 - m_use[:, None]).astype(ft)
            p = np.exp2(arg).astype(ft)
        p = np.where(ok, p, 0.0).astype(ft)
        pr = p if exact else round_to(p, dtype)
        l_run += pr.sum(axis=1, dtype=ft)
        l_lse += p.sum(axis=1, dtype=ft)
        o += pr @ v[t0:t1]
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(l_run[:, None] > 0, o / l_run[:, None], 0.0)
        lse = np.where(l_lse > 0, (m_run + np.log2(l_lse)) * LN2, -np.inf)
    out = out if exact else round_to(out.astype(np.float32), dtype)
    return np.asarray(out, np.float64), np.asarray(lse, np.float64)
