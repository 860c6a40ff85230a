"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic and imports neither the HIP library nor the
oracle: it only draws numbers and lays out shapes.  Both sides of every parity check take
their inputs from here.

Recipe: torch CPU generator seeded with 42 + an offset per tensor, standard normal draws
in float32, cast to float16 with round-to-nearest-even where the workload is fp16.  Shapes
follow the pages' workloads (24-layer model with 14 query heads, 2 key-value heads,
head_dim 64; xformers varlen demo seqlens (37, 120, 8, 200); paged pool of 16-token
blocks).  No public dataset is involved: the pages measure on the authors' own prompts.
"""
from dataclasses import dataclass, field

import torch

SEED = 42
BLOCK = 16
HEAD_DIM = 64


def gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(shape, seed, dtype=torch.float16):
    """N(0,1) draws in fp32 on the CPU generator, then cast (RNE) to `dtype`."""
    x = torch.randn(*shape, generator=gen(seed), dtype=torch.float32)
    return x.to(dtype)


def randn_device(shape, seed, dtype, device):
    """Same recipe on a device generator (used for sizes too large to draw on the host;
    the values differ from the CPU stream but both sides of a check read the same
    tensor)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device).to(dtype)


# ---------------------------------------------------------------------------------------
# model shapes
# ---------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Model:
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: torch.dtype


MODEL_24L = Model(layers=24, q_heads=14, kv_heads=2, head_dim=64, dtype=torch.float16)
SINGLE_HEAD_F32 = Model(layers=1, q_heads=1, kv_heads=1, head_dim=64, dtype=torch.float32)


# ---------------------------------------------------------------------------------------
# single head fp32: 40-token prompt then 48 decode steps
# ---------------------------------------------------------------------------------------
SINGLE_PROMPT = 40
SINGLE_STEPS = 48


def single_head_sequence(seed=SEED):
    """q, k, v [88, 1, 64] fp32 for the 40 + 48 token single-head run."""
    n = SINGLE_PROMPT + SINGLE_STEPS
    return (randn((n, 1, HEAD_DIM), seed, torch.float32),
            randn((n, 1, HEAD_DIM), seed + 1, torch.float32),
            randn((n, 1, HEAD_DIM), seed + 2, torch.float32))


# ---------------------------------------------------------------------------------------
# packed varlen prefill
# ---------------------------------------------------------------------------------------
VARLEN_SEQLENS = (37, 120, 8, 200)


def cu_seqlens(seqlens):
    cu = [0]
    for s in seqlens:
        cu.append(cu[-1] + int(s))
    return torch.tensor(cu, dtype=torch.int32)


def varlen_inputs(seqlens, hq, hkv, seed=SEED + 100, dtype=torch.float16, head_dim=HEAD_DIM):
    T = int(sum(seqlens))
    d = head_dim
    return (randn((T, hq, d), seed, dtype), randn((T, hkv, d), seed + 1, dtype),
            randn((T, hkv, d), seed + 2, dtype), cu_seqlens(seqlens))


# ---------------------------------------------------------------------------------------
# batched decode over a paged cache with shared prefixes
# ---------------------------------------------------------------------------------------
@dataclass
class PagedBatch:
    """Request structure of a paged decode batch.

    ctx_before[i]   tokens cached before the step (the step appends one more)
    group[i]        sharing group of request i (requests 8g .. 8g+7)
    prefix          tokens of the group prefix (block aligned); request i reads
                    min(ctx_before[i], prefix) of them
    """
    ctx_before: list
    group: list
    prefix: int
    group_size: int = 8
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.ctx_before)


def paged_batch(batch, lo=128, hi=2048, prefix=512, group_size=8, seed=SEED + 200):
    """Context lengths uniform on the integers lo..hi; groups of `group_size` consecutive
    requests share a `prefix`-token prefix."""
    g = gen(seed + batch)
    ctx = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    group = [i // group_size for i in range(batch)]
    return PagedBatch(ctx_before=ctx, group=group, prefix=prefix, group_size=group_size)


def uniform_batch(batch, ctx, seed=SEED + 300):
    """Every request holds `ctx` tokens, no sharing."""
    return PagedBatch(ctx_before=[int(ctx)] * batch, group=list(range(batch)), prefix=0,
                      group_size=1)


def free_list_permutation(num_blocks, seed=SEED + 400):
    """Seeded shuffle of the pool's block ids, so that tables come out scattered."""
    return torch.randperm(num_blocks, generator=gen(seed)).to(torch.int32)


def group_prefix_kv(pb: PagedBatch, hkv, seed, dtype=torch.float16, layer=0, head_dim=HEAD_DIM):
    """{group: (K, V)} of shape [hkv, prefix, d]: the rows every member of a sharing group
    holds in common."""
    base = seed + 1000 * layer
    pref = {}
    if pb.prefix > 0:
        for gi in sorted(set(pb.group)):
            pref[gi] = (randn((hkv, pb.prefix, head_dim), base + 2 * gi, dtype),
                        randn((hkv, pb.prefix, head_dim), base + 2 * gi + 1, dtype))
    return pref


def logical_kv(pb: PagedBatch, hkv, lmax, seed, dtype=torch.float16, layer=0, head_dim=HEAD_DIM):
    """Logical (contiguous) K and V [B, hkv, lmax, d] for one layer: positions below the
    prefix are the group's shared rows, the rest are private to each request; positions
    at or beyond ctx_before+1 are zero padding (never read)."""
    B = pb.batch
    K = torch.zeros((B, hkv, lmax, head_dim), dtype=dtype)
    V = torch.zeros_like(K)
    base = seed + 1000 * layer
    pref = group_prefix_kv(pb, hkv, seed, dtype, layer, head_dim)
    for i in range(B):
        n = pb.ctx_before[i] + 1
        shared = min(pb.ctx_before[i], pb.prefix)
        if shared > 0:
            pk, pv = pref[pb.group[i]]
            K[i, :, :shared] = pk[:, :shared]
            V[i, :, :shared] = pv[:, :shared]
        if n > shared:
            s = base + 100000 + 2 * i
            K[i, :, shared:n] = randn((hkv, n - shared, head_dim), s, dtype)
            V[i, :, shared:n] = randn((hkv, n - shared, head_dim), s + 1, dtype)
    return K, V


def decode_q(batch, hq, seed, dtype=torch.float16, layer=0, head_dim=HEAD_DIM):
    return randn((batch, hq, head_dim), seed + 7919 * (layer + 1), dtype)
