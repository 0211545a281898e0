"""Gradients of block-sparse and offset attention in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The forward is masked softmax attention (``oracle.attention``,
``oracle.offsets``); every page trains models through it, and its gradient is
the gradient of o_t = sum_s p_ts v_s with p_ts = exp(s_ts - lse_t) over the
allowed keys (s_ts = scale <q_t, k_s>).  With dO the upstream gradient:

    D_t    = <dO_t, o_t>
    dv_s   = sum_t p_ts dO_t
    dp_ts  = <dO_t, v_s>
    ds_ts  = p_ts (dp_ts - D_t)
    dq_t   = scale * sum_s ds_ts k_s
    dk_s   = scale * sum_t ds_ts q_t

summed over the allowed (t, s) pairs; masked pairs contribute nothing, and a
query with no allowed key contributes nothing.  Grouped-query heads add their
contributions into the shared K/V head.

* ``dense_masked_attention_bwd`` -- the N x N form over the expanded token
  mask (compression paper Sec. 3.4; BigBird Sec. 3 sketch).
* ``csr_attention_bwd`` -- the CSR-gather form, one query block at a time over
  its listed key blocks.
* ``offset_attention_bwd`` -- the offset pattern ("Depth-Staggered Fibonacci
  Spacing", Sec. 2), one distance at a time.
"""

import numpy as np

from . import attention as oa


def _grads(qh, kh, vh, doh, allowed, scale, mags=False):
    """dq, dk, dv of one head over a boolean [Nq, Nk] mask (rows without keys
    give zero).  With ``mags`` also the term magnitudes of each entry, the same
    sums with every factor replaced by its absolute value and D_t by
    sum_x |dO_tx| |o_tx| added to |dp - D| (what a relative perturbation of the
    weights p, of the products and of D can move the entry by)."""
    s = scale * (qh @ kh.T)
    s = np.where(allowed, s, -np.inf)
    p, _ = oa._softmax_rows(s)
    o = p @ vh
    D = np.sum(doh * o, axis=1)
    dv = p.T @ doh
    dp = doh @ vh.T
    ds = p * (dp - D[:, None])
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    if not mags:
        return dq, dk, dv
    Dabs = np.sum(np.abs(doh) * np.abs(o), axis=1)
    dsm = p * (np.abs(dp - D[:, None]) + Dabs[:, None])
    return (dq, dk, dv), (abs(scale) * (dsm @ np.abs(kh)), abs(scale) * (dsm.T @ np.abs(qh)), p.T @ np.abs(doh))


def dense_masked_attention_bwd(q, k, v, do, block_masks, block, causal, scale,
                               mask_batch_stride=0, mask_head_stride=0):
    """(dq, dk, dv) float64 for a [G, N_b, N_b] boolean block mask."""
    B, H, N, d = q.shape
    rep = H // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    cache = {}
    for b in range(B):
        for h in range(H):
            g = b * mask_batch_stride + h * mask_head_stride
            if g not in cache:
                cache[g] = oa.expand_block_mask(block_masks[g], block, causal)
            kh = h // rep
            a, c, e = _grads(q[b, h], k[b, kh], v[b, kh], do[b, h], cache[g], scale)
            dq[b, h] = a
            dk[b, kh] += c
            dv[b, kh] += e
    return dq, dk, dv


def csr_attention_bwd(q, k, v, do, row_ptr, col_idx, block, causal, scale,
                      mask_batch_stride=0, mask_head_stride=0, heads=None, mags=False):
    """(dq, dk, dv) float64, one query block at a time over its key blocks.

    ``heads`` optionally restricts the work to (b, h) pairs (their
    contributions only).  ``mags``: also return the term magnitudes (see
    ``_grads``) as a second triple."""
    B, H, N, d = q.shape
    rep = H // k.shape[1]
    nb = N // block
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        g = b * mask_batch_stride + h * mask_head_stride
        kh = h // rep
        for qb in range(nb):
            r = g * nb + qb
            cols = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)
            if cols.size == 0:
                continue
            qi = np.arange(qb * block, (qb + 1) * block)
            keys = (cols[:, None] * block + np.arange(block)[None, :]).reshape(-1)
            allowed = np.ones((block, keys.size), dtype=bool)
            if causal:
                allowed = keys[None, :] <= qi[:, None]
            r = _grads(q[b, h, qi], k[b, kh, keys], v[b, kh, keys], do[b, h, qi], allowed, scale, mags)
            (a, c, e), m = (r, None) if not mags else r
            dq[b, h, qi] = a
            np.add.at(dk[b, kh], keys, c)
            np.add.at(dv[b, kh], keys, e)
            if mags:
                mq[b, h, qi] = m[0]
                np.add.at(mk[b, kh], keys, m[1])
                np.add.at(mv[b, kh], keys, m[2])
    return ((dq, dk, dv), (mq, mk, mv)) if mags else (dq, dk, dv)


def offset_attention_bwd(q, k, v, do, offsets, scale, mags=False):
    """(dq, dk, dv) float64 for keys {t - delta : delta in offsets, t - delta >= 0}
    (``mags``: also the term magnitudes, as for csr_attention_bwd)."""
    B, H, N, d = q.shape
    rep = H // k.shape[1]
    offs = list(offsets)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    t = np.arange(N)
    for b in range(B):
        for h in range(H):
            kh = h // rep
            s = np.full((N, len(offs)), -np.inf)
            for n, delta in enumerate(offs):
                src = t - delta
                ok = src >= 0
                s[ok, n] = scale * np.einsum("ij,ij->i", q[b, h, t[ok]], k[b, kh, src[ok]])
            p, _ = oa._softmax_rows(s)
            o = np.zeros((N, d))
            for n, delta in enumerate(offs):
                src = t - delta
                ok = src >= 0
                o[ok] += p[ok, n][:, None] * v[b, kh, src[ok]]
            D = np.sum(do[b, h] * o, axis=1)
            Dabs = np.sum(np.abs(do[b, h]) * np.abs(o), axis=1)
            for n, delta in enumerate(offs):
                src = t - delta
                ok = src >= 0
                tt, ss = t[ok], src[ok]
                dp = np.einsum("ij,ij->i", do[b, h, tt], v[b, kh, ss])
                ds = p[ok, n] * (dp - D[ok])
                dq[b, h, tt] += scale * ds[:, None] * k[b, kh, ss]
                np.add.at(dk[b, kh], ss, scale * ds[:, None] * q[b, h, tt])
                np.add.at(dv[b, kh], ss, p[ok, n][:, None] * do[b, h, tt])
                if mags:
                    dsm = p[ok, n] * (np.abs(dp - D[ok]) + Dabs[ok])
                    mq[b, h, tt] += abs(scale) * dsm[:, None] * np.abs(k[b, kh, ss])
                    np.add.at(mk[b, kh], ss, abs(scale) * dsm[:, None] * np.abs(q[b, h, tt]))
                    np.add.at(mv[b, kh], ss, p[ok, n][:, None] * np.abs(do[b, h, tt]))
    return ((dq, dk, dv), (mq, mk, mv)) if mags else (dq, dk, dv)
