"""Block-sparse attention forward in fp64, written two independent ways.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The sparse method changes only which (query, key) terms exist; the result is
ordinary masked softmax attention over the allowed keys:

    s_ts  = scale * <q_t, k_s>           for s in K(t)
    o_t   = sum_s exp(s_ts - m) v_s / sum_s exp(s_ts - m),   m = max_s s_ts
    lse_t = m + ln sum_s exp(s_ts - m)

with K(t) = union over listed key blocks kb of row floor(t/b) of the tokens of
kb, AND s <= t when causal.  An empty K(t) gives o_t = 0 and lse_t = -inf.

* ``csr_attention`` gathers the listed key blocks per query block (the
  "block-sparse" gather of BigBird Sec. 3, closing paragraph).
* ``dense_masked_attention`` expands the block mask to N x N tokens
  (compression paper Sec. 3.4 "Block-to-token expansion"; Algorithm 1 step 4),
  ANDs the causal triangle, fills masked logits with -inf and takes a full
  softmax (BigBird Sec. 3 reference sketch).

Both take float64 arrays q [B, H, N, d] and k, v [B, H_kv, N, d]; head h reads
K/V head h // (H / H_kv).  The mask group of (b, h) is b*mbs + h*mhs.
"""

import numpy as np


def _softmax_rows(s):
    """Row softmax and log-sum-exp of a float64 matrix with -inf for masked terms."""
    m = np.max(s, axis=1, initial=-np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    e[:, :] = np.where(np.isfinite(s), e, 0.0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    ok = l > 0
    p[ok] = e[ok] / l[ok][:, None]
    lse = np.full(s.shape[0], -np.inf)
    lse[ok] = m_safe[ok] + np.log(l[ok])
    return p, lse


def csr_attention(q, k, v, row_ptr, col_idx, block, causal, scale,
                  mask_batch_stride=0, mask_head_stride=0, heads=None):
    """CSR-gather form.  Returns (o [B,H,N,d], lse [B,H,N]) in float64.

    ``heads`` optionally restricts the work to a list of (b, h) pairs (other
    outputs stay zero / -inf).
    """
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    nb = N // block
    rep = H // Hkv
    o = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        g = b * mask_batch_stride + h * mask_head_stride
        kh = h // rep
        for qb in range(nb):
            r = g * nb + qb
            cols = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)
            qi = np.arange(qb * block, (qb + 1) * block)
            if cols.size == 0:
                continue
            keys = (cols[:, None] * block + np.arange(block)[None, :]).reshape(-1)
            s = scale * (q[b, h, qi] @ k[b, kh, keys].T)
            if causal:
                s = np.where(keys[None, :] <= qi[:, None], s, -np.inf)
            p, l = _softmax_rows(s)
            o[b, h, qi] = p @ v[b, kh, keys]
            lse[b, h, qi] = l
    return o, lse


def expand_block_mask(block_mask_g, block, causal):
    """N x N token mask M'[t, s] = M[t // b, s // b], AND s <= t when causal.

    Compression paper Sec. 3.4 ("indexing entry (i,j) from M[floor(i/b),
    floor(j/b)]") and Algorithm 1 step 4 (AND NOT triu(1, 1)).
    """
    nb = block_mask_g.shape[0]
    tok = np.repeat(np.repeat(block_mask_g, block, axis=0), block, axis=1)
    if causal:
        n = nb * block
        tok = tok & ~np.triu(np.ones((n, n), dtype=bool), 1)
    return tok


def dense_masked_attention(q, k, v, block_masks, block, causal, scale,
                           mask_batch_stride=0, mask_head_stride=0):
    """Dense-masked form over a [G, N_b, N_b] boolean block mask.

    Full N x N logits, masked_fill(-inf) outside the expanded mask, softmax,
    then P @ V (BigBird Sec. 3 sketch).  Returns (o, lse) in float64.
    """
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    rep = H // Hkv
    o = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    cache = {}
    for b in range(B):
        for h in range(H):
            g = b * mask_batch_stride + h * mask_head_stride
            if g not in cache:
                cache[g] = expand_block_mask(block_masks[g], block, causal)
            allowed = cache[g]
            kh = h // rep
            s = scale * (q[b, h] @ k[b, kh].T)
            s = np.where(allowed, s, -np.inf)
            p, l = _softmax_rows(s)
            o[b, h] = p @ v[b, kh]
            lse[b, h] = l
    return o, lse


def csr_attention_rows(q, k, v, row_ptr, col_idx, block, causal, scale, samples,
                       mask_batch_stride=0, mask_head_stride=0):
    """CSR-gather form for single query tokens.

    ``samples`` is a list of (b, h, t).  Returns (o [len, d], lse [len]).
    """
    H = q.shape[1]
    Hkv = k.shape[1]
    rep = H // Hkv
    nb = q.shape[2] // block
    d = q.shape[3]
    o = np.zeros((len(samples), d))
    lse = np.full(len(samples), -np.inf)
    for n, (b, h, t) in enumerate(samples):
        g = b * mask_batch_stride + h * mask_head_stride
        r = g * nb + t // block
        cols = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)
        if cols.size == 0:
            continue
        keys = (cols[:, None] * block + np.arange(block)[None, :]).reshape(-1)
        if causal:
            keys = keys[keys <= t]
        if keys.size == 0:
            continue
        kh = h // rep
        s = scale * (k[b, kh, keys] @ q[b, h, t])
        p, l = _softmax_rows(s[None, :])
        o[n] = p[0] @ v[b, kh, keys]
        lse[n] = l[0]
    return o, lse
