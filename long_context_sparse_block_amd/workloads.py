"""Seeded synthetic workloads: shapes, mask parameters and Q/K/V generators.

This module holds no attention or mask arithmetic.  It only names the
workloads (their sizes and mask parameters) and draws their inputs, so that the
HIP library and the CPU oracle can be fed the very same values.  It imports
nothing else from this package.

Inputs: Q, K, V iid N(0, 1), drawn as float32 from ``torch.Generator`` seeded
per workload (q, then k, then v), then rounded to the compute dtype with
round-to-nearest-even.  Byte streams for gzip-derived literal flags come from
``synthetic_bytes`` (seeded numpy generator; it stands in for book text).
"""

import numpy as np
import torch

BF16 = "bf16"
F32 = "f32"

# Block-sparse workloads.  Mask parameters are in blocks.
#   groups: "shared"       one mask for every (batch, head)
#           "per-sequence" one mask per batch entry, shared by its heads
BLOCK_WORKLOADS = {
    "tiny-fp32": dict(
        B=1, H=1, N=512, d=64, block=64, dtype=F32, causal=True,
        win_before=1, win_after=0, win_clamp=False, global_blocks=[0],
        num_random=1, literal_mode="none", literal_p=0.0, mask_seed=1,
        groups="shared", qkv_seed=1001),
    "compression-guided": dict(
        B=4, H=8, N=8192, d=64, block=64, dtype=BF16, causal=True,
        win_before=3, win_after=0, win_clamp=False, global_blocks=[],
        num_random=0, literal_mode="pair", literal_p=0.25, mask_seed=2,
        groups="per-sequence", qkv_seed=1002),
    "bigbird": dict(
        B=2, H=12, N=4096, d=64, block=64, dtype=BF16, causal=False,
        win_before=1, win_after=1, win_clamp=True, global_blocks=[0, 63],
        num_random=3, literal_mode="none", literal_p=0.0, mask_seed=3,
        groups="shared", qkv_seed=1003),
    # Sec. 4.1 of the compression paper: 8192-byte sequences, 128-byte
    # blocks, literal flags from per-block gzip sizes, +-1-block local window,
    # no globals (the "Gzip-Guided" mask); 12 heads of d = 64.
    "gzip-guided": dict(
        B=4, H=12, N=8192, d=64, block=128, dtype=BF16, causal=True,
        win_before=1, win_after=0, win_clamp=False, global_blocks=[],
        num_random=0, literal_mode="pair", literal_p=0.0, mask_seed=7,
        groups="per-sequence", qkv_seed=1007, literal_source="gzip", text_seed=7),
    # the same with the paper's head groups (Sec. 3.3): heads 0-5 local,
    # 6-8 long-range, 9-11 hybrid; one mask group per (sequence, head)
    "gzip-head-groups": dict(
        B=4, H=12, N=8192, d=64, block=128, dtype=BF16, causal=True,
        win_before=1, win_after=0, win_clamp=False, global_blocks=[],
        num_random=0, literal_mode="pair", literal_p=0.0, mask_seed=7,
        groups="per-sequence", qkv_seed=1008, literal_source="gzip", text_seed=7,
        head_groups=True),
    "long-context": dict(
        B=1, H=16, N=65536, d=128, block=128, dtype=BF16, causal=True,
        win_before=2, win_after=0, win_clamp=False, global_blocks=[0, 1, 2, 3],
        num_random=0, literal_mode="pair", literal_p=0.15, mask_seed=5,
        groups="shared", qkv_seed=1005),
}

# Offset workload: 16 calls, one per alpha of a linear ramp 1 -> 2.
OFFSET_WORKLOAD = dict(B=8, H=8, d=64, lengths=(2048, 8192), W=8, dtype=BF16,
                       alphas=tuple(1.0 + l / 15.0 for l in range(16)),
                       qkv_seed_base={2048: 1400, 8192: 1500})

# Variants of the offset pattern ("Depth-Staggered Fibonacci Spacing for Sparse
# Attention", Sec. 2), 16 calls each on the shape above at N = 2048:
#  * stagger-ratio: Fibonacci base, alpha_l = 0.5 + l/15 held exactly (its rungs
#    that land on a half round up);
#  * power2-stagger: the power-of-2 control base with the same alpha ramp;
#  * interp: continuous alpha_l = 0.5 + sigmoid(theta_l) with theta_l drawn
#    N(0, 0.05^2) (a per-layer scalar that stays near its initialisation alpha
#    = 1), so every rung is an interpolated gather.
OFFSET_VARIANTS = {
    "stagger-ratio": dict(base="fibonacci", ratios=tuple((15 + 2 * l, 30) for l in range(16)), qkv_seed_base=1600),
    "power2-stagger": dict(base="power2", ratios=tuple((15 + 2 * l, 30) for l in range(16)), qkv_seed_base=1700),
    "interp": dict(base="fibonacci", theta_seed=1800, theta_sd=0.05, qkv_seed_base=1800),
}


def interp_alphas(v, L=16):
    """alpha_l = 0.5 + sigmoid(theta_l), theta_l ~ N(0, sd^2) from the variant's seed."""
    g = np.random.default_rng(v["theta_seed"])
    th = g.normal(0.0, v["theta_sd"], size=L)
    return [0.5 + 1.0 / (1.0 + float(np.exp(-t))) for t in th]


def mask_spec(w, **over):
    """Plain-dict mask description of a block workload (block units)."""
    B, H = w["B"], w["H"]
    if w["groups"] == "shared":
        G, mbs, mhs = 1, 0, 0
    elif w["groups"] == "per-sequence":
        G, mbs, mhs = B, 1, 0
    else:
        raise ValueError(w["groups"])
    spec = dict(num_blocks=w["N"] // w["block"], num_groups=G, causal=w["causal"],
                win_before=w["win_before"], win_after=w["win_after"],
                win_clamp=w["win_clamp"], global_blocks=list(w["global_blocks"]),
                num_random=w["num_random"], random_blocks=None,
                literal_mode=w["literal_mode"], literal_flags=None,
                literal_p=w["literal_p"], seed=w["mask_seed"],
                mask_batch_stride=mbs, mask_head_stride=mhs)
    spec.update(over)
    return spec


def torch_dtype(name):
    return {BF16: torch.bfloat16, F32: torch.float32}[name]


def make_qkv(B, H, N, d, dtype, seed, H_kv=None):
    """Seeded CPU tensors q [B,H,N,d], k, v [B,H_kv,N,d] in ``dtype``."""
    H_kv = H if H_kv is None else H_kv
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H_kv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H_kv, N, d), generator=g, dtype=torch.float32)
    td = torch_dtype(dtype) if isinstance(dtype, str) else dtype
    return q.to(td), k.to(td), v.to(td)


def random_flags(G, nb, p, seed):
    """Seeded explicit literal flags uint8 [G, nb] (torch generator draws)."""
    g = torch.Generator().manual_seed(seed)
    return (torch.rand((G, nb), generator=g) < p).to(torch.uint8)


def random_draws(G, nb, r, causal, seed):
    """Seeded explicit random-block draws int32 [G, nb, r]: for each row a prefix
    of a random permutation of the allowed range (earlier blocks when causal),
    padded with -1 when fewer than r blocks are available."""
    g = torch.Generator().manual_seed(seed)
    out = torch.full((G, nb, r), -1, dtype=torch.int32)
    for gi in range(G):
        for i in range(nb):
            n = i if causal else nb
            if n <= 0:
                continue
            perm = torch.randperm(n, generator=g)[:r]
            out[gi, i, :perm.numel()] = perm.to(torch.int32)
    return out


# Regimes of synthetic byte blocks: highly repetitive, prose-like, dense.
_REGIMES = ("repetitive", "prose", "dense")


def synthetic_bytes(G, n_bytes, block_bytes, seed):
    """Byte streams [G, n_bytes] (uint8) with block-level variation in redundancy.

    Stand-in for book text: each block is written in one regime -- a short
    phrase repeated (repetitive), words drawn with Zipf-like frequencies from a
    fixed vocabulary (prose), or uniform printable characters (dense).  The
    regime persists from block to block with probability 0.6, so literal
    blocks come in runs as in real text.  Deterministic in ``seed``.
    """
    rng = np.random.default_rng(seed)
    letters = np.frombuffer(b"abcdefghijklmnopqrstuvwxyz", dtype=np.uint8)
    vocab = [bytes(rng.choice(letters, size=int(rng.integers(2, 10)))) for _ in range(300)]
    zipf = 1.0 / np.arange(1, len(vocab) + 1)
    zipf /= zipf.sum()
    out = np.zeros((G, n_bytes), dtype=np.uint8)
    nb = n_bytes // block_bytes
    for g in range(G):
        regime = int(rng.integers(0, 3))
        for i in range(nb):
            if i > 0 and rng.random() >= 0.6:
                regime = int(rng.integers(0, 3))
            kind = _REGIMES[regime]
            if kind == "repetitive":
                phrase = b" ".join(vocab[int(j)] for j in rng.integers(0, 20, size=int(rng.integers(1, 3)))) + b". "
                blk = (phrase * (block_bytes // len(phrase) + 1))[:block_bytes]
            elif kind == "prose":
                blk = b""
                while len(blk) < block_bytes:
                    blk += vocab[int(rng.choice(len(vocab), p=zipf))] + b" "
                blk = blk[:block_bytes]
            else:
                blk = bytes(rng.integers(32, 127, size=block_bytes, dtype=np.uint8))
            out[g, i * block_bytes:(i + 1) * block_bytes] = np.frombuffer(blk, dtype=np.uint8)
        out[g, nb * block_bytes:] = 32
    return out
