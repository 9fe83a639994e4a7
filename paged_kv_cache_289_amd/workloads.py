"""Seeded synthetic inputs for paged decode attention.

This module builds the *inputs* only: context lengths, a physical block pool
with its per-sequence block tables, and q/K/V values.  It holds none of the
attention arithmetic.  Both the CPU oracle's tests and the HIP path's tests and
benchmark draw their inputs from here, so that the two see identical data.

Structure follows the pages' description of paged KV storage: the cache of each
sequence lives in fixed-size blocks (16 tokens by default) scattered through a
shared physical pool, reached through a per-sequence table of physical block ids
("Local_LLM_03_vLLM_Architecture", PagedAttention slide; "vLLM: LLM Inference
That Doesn't Waste Your GPU", section "PagedAttention: virtual memory for KV").
Sequences that share a prompt prefix point at the same physical blocks
("Scaling inference with vLLM", prefix-sharing paragraph).

Pool layout: ``k_cache`` and ``v_cache`` are separate arrays of shape
``[num_blocks, num_kv_heads, block_size, head_dim]``.  Token ``t`` of sequence
``s`` sits in physical block ``block_tables[s, t // block_size]`` at slot
``t % block_size``; the allocator below writes that placement and records the
slots it left unused (free blocks, the tail of each last block, table padding)
so that tests can poison them.

Values are N(0, 1), drawn in float32 and rounded to the storage dtype with
round-to-nearest-even.  bf16 values are carried on the host as ``uint16`` bit
patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


# --------------------------------------------------------------------------
# structure
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PagedStructure:
    """Shapes, context lengths, block tables and pool bookkeeping of one call.

    ``q_lens[s]`` is the number of query tokens of sequence ``s`` (1 for a
    decode step).  ``context_lens[s]`` counts every key the queries of ``s``
    may see, the new tokens included (their K/V are already in the pool).
    """

    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [S]
    q_lens: np.ndarray                # int32 [S]
    block_tables: np.ndarray          # int32 [S, max_blocks_per_seq]
    scale: float
    seed: int
    layers: int = 1
    free_blocks: np.ndarray = dataclasses.field(default_factory=lambda: np.zeros(0, np.int32))
    pad_block: int = 0                # block id written into unused table entries
    shared_prefix_blocks: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def q_offsets(self) -> np.ndarray:
        off = np.zeros(self.num_seqs + 1, np.int32)
        np.cumsum(self.q_lens, out=off[1:])
        return off

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.q_lens == 1))

    def blocks_used(self, s: int) -> int:
        return -(-int(self.context_lens[s]) // self.block_size)

    def tail_slots(self) -> List[tuple]:
        """(block id, first unused slot) for every sequence's last, partly filled block."""
        out = []
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            r = L % self.block_size
            if L > 0 and r != 0:
                out.append((int(self.block_tables[s, L // self.block_size]), r))
        return out

    def summary(self) -> dict:
        return {
            "workload": self.name, "dtype": self.dtype, "num_seqs": self.num_seqs,
            "num_heads": self.num_heads, "num_kv_heads": self.num_kv_heads,
            "head_dim": self.head_dim, "block_size": self.block_size,
            "num_blocks": self.num_blocks, "max_blocks_per_seq": self.max_blocks_per_seq,
            "sum_context": int(self.context_lens.sum()), "max_context": self.max_context_len,
            "total_q": self.total_q, "layers": self.layers, "seed": self.seed,
        }


def _rngs(seed: int):
    ss = np.random.SeedSequence(seed)
    a, b = ss.spawn(2)
    return np.random.default_rng(a), np.random.default_rng(b)


def allocate(name: str, dtype: str, context_lens: Sequence[int], q_lens: Sequence[int],
             num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
             rng: np.random.Generator, seed: int, *, pool_extra: float = 0.10,
             exact_pool: Optional[int] = None, shared_prefix_blocks: int = 0,
             max_blocks_per_seq: Optional[int] = None, scale: Optional[float] = None,
             layers: int = 1) -> PagedStructure:
    """Place every sequence's blocks at random spots of one physical pool.

    The pool holds ``ceil((1 + pool_extra) * needed)`` blocks (or exactly
    ``exact_pool``).  A random permutation of the pool is consumed in order:
    first the shared-prefix blocks (if any), then each sequence's own blocks.
    Blocks never consumed stay free.  Table entries past a sequence's last
    block hold ``pad_block`` (a free block when there is one).
    """
    L = np.asarray(context_lens, dtype=np.int64)
    n = np.asarray(q_lens, dtype=np.int64)
    S = L.shape[0]
    assert n.shape == (S,)
    assert np.all(L >= 0) and np.all(n >= 0)
    nb = -(-L // block_size)
    P = shared_prefix_blocks
    if P:
        assert np.all(nb >= P), "every sequence must cover the shared prefix"
    needed = P + int((nb - P).sum()) if S else 0
    pool = exact_pool if exact_pool is not None else max(1, math.ceil((1.0 + pool_extra) * needed))
    assert pool >= needed
    perm = rng.permutation(pool).astype(np.int32)
    mb = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, int(nb.max()) if S else 1)
    assert mb >= (int(nb.max()) if S else 0)
    free = perm[needed:]
    pad = int(free[0]) if free.size else 0
    tables = np.full((S, mb), pad, dtype=np.int32)
    cur = P
    prefix = perm[:P]
    for s in range(S):
        k = int(nb[s])
        if P:
            tables[s, :P] = prefix
            own = k - P
            tables[s, P:k] = perm[cur:cur + own]
            cur += own
        else:
            tables[s, :k] = perm[cur:cur + k]
            cur += k
    assert cur == needed
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PagedStructure(
        name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, num_blocks=pool,
        context_lens=L.astype(np.int32), q_lens=n.astype(np.int32), block_tables=tables,
        scale=float(scale), seed=seed, layers=layers, free_blocks=free.copy(), pad_block=pad,
        shared_prefix_blocks=P)


# --------------------------------------------------------------------------
# the named workloads (Llama-like shapes; values synthetic)
# --------------------------------------------------------------------------

def tiny_fp32(seed: int = 0, dtype: str = "f32") -> PagedStructure:
    """4 sequences, contexts {1, 17, 33, 100}, 4 query / 2 KV heads, head_dim 64,
    16-token blocks, a 64-block pool placed by one seeded permutation, scale 1/8."""
    srng, _ = _rngs(seed)
    return allocate("tiny_fp32_gqa2_d64", dtype, [1, 17, 33, 100], [1, 1, 1, 1], 4, 2, 64, 16,
                    srng, seed, exact_pool=64, scale=1.0 / 8.0)


def llama3_8b_decode(seed: int = 0, num_seqs: int = 64, ctx_lo: int = 128, ctx_hi: int = 4096,
                     block_size: int = 16, dtype: str = "bf16") -> PagedStructure:
    """Decode layer of a Llama-3-8B-like model: 32 query / 8 KV heads, head_dim 128,
    contexts uniform in [ctx_lo, ctx_hi] (inclusive), pool = needed + 10% free."""
    srng, _ = _rngs(seed)
    L = srng.integers(ctx_lo, ctx_hi + 1, size=num_seqs)
    return allocate(f"llama3_8b_decode_b{num_seqs}", dtype, L, np.ones_like(L), 32, 8, 128,
                    block_size, srng, seed, max_blocks_per_seq=-(-ctx_hi // block_size))


def llama3_70b_decode(seed: int = 0, num_seqs: int = 32, ctx: int = 8192, layers: int = 80,
                      num_heads: int = 64, dtype: str = "bf16") -> PagedStructure:
    """Decode of a Llama-3-70B-like model: 64 query / 8 KV heads, head_dim 128, every
    context at ``ctx`` tokens, one block table shared by ``layers`` per-layer pools
    with no free blocks (32 x 8192 tokens x 4 KiB x 80 layers = 80 GiB)."""
    srng, _ = _rngs(seed)
    L = np.full(num_seqs, ctx)
    nb = -(-ctx // 16) * num_seqs
    return allocate(f"llama3_70b_decode_b{num_seqs}_ctx{ctx}", dtype, L, np.ones_like(L),
                    num_heads, 8, 128, 16, srng, seed, exact_pool=nb, layers=layers)


def shared_prefix_mix(seed: int = 0, num_seqs: int = 256, prefix_blocks: int = 128,
                      tail_median: float = 256.0, tail_sigma: float = 1.0, tail_max: int = 6144,
                      dtype: str = "bf16") -> PagedStructure:
    """Every table starts with the same ``prefix_blocks`` physical blocks (2048 tokens),
    then a unique tail of clip(rint(LogNormal(ln median, sigma)), 1, tail_max) tokens."""
    srng, _ = _rngs(seed)
    tail = np.clip(np.rint(srng.lognormal(math.log(tail_median), tail_sigma, size=num_seqs)),
                   1, tail_max).astype(np.int64)
    L = prefix_blocks * 16 + tail
    mb = prefix_blocks + -(-tail_max // 16)
    return allocate(f"shared_prefix_mix_b{num_seqs}", dtype, L, np.ones_like(L), 32, 8, 128, 16,
                    srng, seed, shared_prefix_blocks=prefix_blocks, max_blocks_per_seq=mb)


def spec_verify(seed: int = 0, num_seqs: int = 64, n_new: int = 5, ctx_lo: int = 1024,
                ctx_hi: int = 8192, dtype: str = "bf16") -> PagedStructure:
    """Speculative verification: ``n_new`` query tokens per sequence with a causal mask
    over them; contexts (new tokens included) uniform in [ctx_lo, ctx_hi]."""
    srng, _ = _rngs(seed)
    L = srng.integers(ctx_lo, ctx_hi + 1, size=num_seqs)
    return allocate(f"spec_verify_b{num_seqs}_n{n_new}", dtype, L, np.full_like(L, n_new), 32, 8,
                    128, 16, srng, seed, max_blocks_per_seq=-(-ctx_hi // 16))


def chunked_prefill(seed: int = 0, cached: int = 4096, chunk: int = 512,
                    dtype: str = "bf16") -> PagedStructure:
    """One ``chunk``-token prefill chunk over ``cached`` paged tokens; the chunk's own
    K/V are in the pool, so the context is cached + chunk (4608)."""
    srng, _ = _rngs(seed)
    return allocate(f"chunked_prefill_{chunk}_over_{cached}", dtype, [cached + chunk], [chunk],
                    32, 8, 128, 16, srng, seed)


def random_small(seed: int, *, num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, ctx_lo: int, ctx_hi: int, q_len_max: int = 1,
                 dtype: str = "f32", pool_extra: float = 0.25, scale: Optional[float] = None,
                 shared_prefix_blocks: int = 0) -> PagedStructure:
    """Small random case for property tests: ragged contexts, optional multi-token queries
    (1..q_len_max, never more than the context), optional shared prefix."""
    srng, _ = _rngs(seed)
    lo = max(ctx_lo, shared_prefix_blocks * block_size)
    L = srng.integers(lo, max(lo, ctx_hi) + 1, size=num_seqs)
    n = np.minimum(srng.integers(1, q_len_max + 1, size=num_seqs), np.maximum(L, 1))
    return allocate(f"random_small_{seed}", dtype, L, n, num_heads, num_kv_heads, head_dim,
                    block_size, srng, seed, pool_extra=pool_extra, scale=scale,
                    shared_prefix_blocks=shared_prefix_blocks)


def kv_append_chunk(seed: int = 0, num_seqs: int = 64, chunk: int = 512, ctx_lo: int = 512,
                    ctx_hi: int = 4096, dtype: str = "bf16") -> PagedStructure:
    """Appending a ``chunk``-token prefill chunk to each of ``num_seqs`` sequences of the
    Llama-3-8B-like layout (8 KV heads, head_dim 128, 16-token blocks): contexts
    uniform in [ctx_lo, ctx_hi] count the chunk, whose tokens are the last ones."""
    srng, _ = _rngs(seed)
    L = srng.integers(ctx_lo, ctx_hi + 1, size=num_seqs)
    return allocate(f"kv_append_chunk{chunk}_b{num_seqs}", dtype, L, np.full_like(L, chunk), 32,
                    8, 128, 16, srng, seed, max_blocks_per_seq=-(-ctx_hi // 16))


NAMED = {
    "tiny_fp32": tiny_fp32,
    "llama3_8b_decode": llama3_8b_decode,
    "llama3_70b_decode": llama3_70b_decode,
    "shared_prefix_mix": shared_prefix_mix,
    "spec_verify": spec_verify,
    "chunked_prefill": chunked_prefill,
    "kv_append": kv_append_chunk,
}


# --------------------------------------------------------------------------
# values
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bits.
    Inputs here are finite normals; NaN is handled by forcing a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32, copy=False)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def storage_nan(dtype: str):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]


def host_values(st: PagedStructure, layer: int = 0) -> Dict[str, np.ndarray]:
    """q [total_q, H, D] and the K/V pool [num_blocks, Hk, B, D] on the host, in the
    storage dtype (bf16 as uint16 bits).  Seeded by (seed, layer)."""
    _, vrng = _rngs(st.seed)
    if layer:
        vrng = np.random.default_rng(np.random.SeedSequence([st.seed, layer, 0x5eed]))
    shp = (st.num_blocks, st.num_kv_heads, st.block_size, st.head_dim)
    q = vrng.standard_normal((st.total_q, st.num_heads, st.head_dim), dtype=np.float32)
    k = vrng.standard_normal(shp, dtype=np.float32)
    v = vrng.standard_normal(shp, dtype=np.float32)
    return {"q": _to_storage(q, st.dtype), "k_cache": _to_storage(k, st.dtype),
            "v_cache": _to_storage(v, st.dtype)}


def poison_unused(st: PagedStructure, vals: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Copy of ``vals`` whose pool slots that no visible token occupies hold NaN:
    every free block (the table padding points at one when the pool has any) and
    the unused tail slots of each sequence's last block."""
    nan = storage_nan(st.dtype)
    out = {k: v.copy() for k, v in vals.items()}
    for name in ("k_cache", "v_cache"):
        c = out[name]
        if st.free_blocks.size:
            c[st.free_blocks] = nan
        for b, r in st.tail_slots():
            c[b, :, r:, :] = nan
    return out


def device_values(st: PagedStructure, device, layer: int = 0):
    """The same kind of inputs generated on a torch device with a seeded device RNG
    (used where host generation would be too slow or too large)."""
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[st.dtype]
    g = torch.Generator(device=device)
    g.manual_seed(int(st.seed) * 1000003 + int(layer) * 7919 + 17)
    shp = (st.num_blocks, st.num_kv_heads, st.block_size, st.head_dim)

    def randn(shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(tdt)

    q = randn((st.total_q, st.num_heads, st.head_dim))
    k = randn(shp)
    v = randn(shp)
    return {"q": q, "k_cache": k, "v_cache": v}


def host_to_torch(vals: Dict[str, np.ndarray], dtype: str, device="cpu"):
    """Wrap host storage arrays as torch tensors of the matching dtype (bf16 bits are
    reinterpreted, not converted)."""
    import torch
    out = {}
    for k, a in vals.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype == "bf16" and a.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        out[k] = t.to(device)
    return out


def torch_to_host(t, dtype: str) -> np.ndarray:
    """Inverse of :func:`host_to_torch` for one tensor."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# --------------------------------------------------------------------------
# re-packing the same logical cache (for invariance tests)
# --------------------------------------------------------------------------

def permute_placement(st: PagedStructure, vals: Dict[str, np.ndarray], seed: int):
    """Move every physical block to a new random id and rewrite the tables to match.
    The logical content of every sequence is unchanged."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xB10C]))
    perm = rng.permutation(st.num_blocks).astype(np.int32)   # old id -> new id
    new_vals = dict(vals)
    for name in ("k_cache", "v_cache"):
        c = np.empty_like(vals[name])
        c[perm] = vals[name]
        new_vals[name] = c
    new_st = dataclasses.replace(st, block_tables=perm[st.block_tables],
                                 free_blocks=perm[st.free_blocks], pad_block=int(perm[st.pad_block]))
    return new_st, new_vals


def unshare_prefix(st: PagedStructure, vals: Dict[str, np.ndarray]):
    """Give every sequence its own copy of the shared-prefix blocks (appended at the
    end of the pool), so that no two tables point at the same block."""
    P = st.shared_prefix_blocks
    assert P > 0
    S = st.num_seqs
    extra = (S - 1) * P
    new_vals = dict(vals)
    for name in ("k_cache", "v_cache"):
        c = vals[name]
        new_vals[name] = np.concatenate([c, np.empty((extra,) + c.shape[1:], c.dtype)], axis=0)
    tables = st.block_tables.copy()
    nxt = st.num_blocks
    for s in range(1, S):
        for j in range(P):
            src = int(st.block_tables[s, j])
            for name in ("k_cache", "v_cache"):
                new_vals[name][nxt] = vals[name][src]
            tables[s, j] = nxt
            nxt += 1
    new_st = dataclasses.replace(st, num_blocks=st.num_blocks + extra, block_tables=tables,
                                 shared_prefix_blocks=0)
    return new_st, new_vals


def pack_logical(name: str, dtype: str, k_seqs: List[np.ndarray], v_seqs: List[np.ndarray],
                 q: np.ndarray, q_lens: Sequence[int], num_heads: int, block_size: int, seed: int,
                 scale: float, pool_extra: float = 0.25):
    """Write per-sequence contiguous K/V (``[L_s, Hk, D]`` storage arrays) into a freshly
    allocated paged pool with the given block size.  Returns (structure, values).
    Unused slots are left zero."""
    lens = [int(k.shape[0]) for k in k_seqs]
    Hk, D = k_seqs[0].shape[1], k_seqs[0].shape[2]
    rng = np.random.default_rng(np.random.SeedSequence([seed, block_size, 0xFACE]))
    st = allocate(name, dtype, lens, q_lens, num_heads, Hk, D, block_size, rng, seed,
                  pool_extra=pool_extra, scale=scale)
    kc = np.zeros((st.num_blocks, Hk, block_size, D), k_seqs[0].dtype)
    vc = np.zeros_like(kc)
    for s, (ks, vs) in enumerate(zip(k_seqs, v_seqs)):
        for j in range(st.blocks_used(s)):
            b = int(st.block_tables[s, j])
            lo, hi = j * block_size, min((j + 1) * block_size, lens[s])
            kc[b, :, :hi - lo, :] = ks[lo:hi].transpose(1, 0, 2)
            vc[b, :, :hi - lo, :] = vs[lo:hi].transpose(1, 0, 2)
    return st, {"q": q, "k_cache": kc, "v_cache": vc}
