"""fp64 oracle of paged attention (test infrastructure only; see the package header).

What is computed
----------------
The pages describe paged KV storage as a change of *where* the cache bytes live,
not of what attention computes: the cache is cut into fixed-size blocks scattered
through physical memory, and a per-sequence table maps logical positions to
physical blocks ("Local_LLM_03_vLLM_Architecture", PagedAttention slide; "vLLM:
LLM Inference That Doesn't Waste Your GPU", section "PagedAttention: virtual
memory for KV"; "Scaling inference with vLLM", paging paragraph).  Decoding
attends each new token over every prior token's cached K and V
("Local_LLM_03_vLLM_Architecture", KV-cache slide; "vLLM: LLM Inference That
Doesn't Waste Your GPU", section "KV cache, in one picture").

So the oracle is the plain definition, in two steps:

1. **Gather** each sequence's K/V through its block table into contiguous arrays
   ordered by logical position.
2. **Attend** with textbook softmax attention, in fp64.

Readings taken where the pages are silent (each also listed in the design notes):

* pool layout ``[num_blocks, num_kv_heads, block_size, head_dim]``, K and V apart;
* grouped-query attention with contiguous groups: query head ``h`` reads KV head
  ``h // (num_heads // num_kv_heads)`` (the pages name "GQA-8" only);
* ``context_lens[s]`` counts every key, including the query tokens' own, whose
  K/V are already in the pool;
* multi-token queries (speculative verification, a prefill chunk) are the last
  ``n_s`` positions of the context; with the causal mask, query row ``i`` sees
  keys ``t <= L_s - n_s + i`` ("Scaling inference with vLLM", speculative
  decoding paragraph: the target verifies all guessed tokens in one pass;
  "Local_LLM_03_vLLM_Architecture", chunked-prefill slide);
* a sequence with no visible key yields a zero output row.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# storage -> fp64
# --------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored values to fp64.

    bf16 is carried as uint16 bit patterns: the upper half of an IEEE binary32,
    so ``bits << 16`` reinterpreted as float32 is the value, exactly.
    """
    if dtype == "bf16":
        x = np.asarray(x)
        assert x.dtype == np.uint16, "bf16 arrays are uint16 bit patterns"
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "fp8e4m3":
        return widen_fp8e4m3(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def widen_fp8e4m3(codes: np.ndarray) -> np.ndarray:
    """Exact values of 8-bit floating-point codes in the E4M3 format with no
    infinities (the OCP 8-bit format): sign bit, 4 exponent bits with bias 7, 3
    mantissa bits.  Exponent field 0 holds the subnormals m/8 * 2^-6; the code
    with all exponent and mantissa bits set is NaN."""
    c = np.asarray(codes)
    assert c.dtype == np.uint8, "fp8 arrays are uint8 codes"
    c = c.astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def paged_decode_quant_kv(q: np.ndarray, q_dtype: str, k_cache: np.ndarray, v_cache: np.ndarray,
                          kv_dtype: str, k_scale: float, v_scale: float, block_tables: np.ndarray,
                          context_lens: np.ndarray, block_size: int, scale: float,
                          seqs: Optional[Sequence[int]] = None) -> np.ndarray:
    """Decode over a cache stored in a reduced-precision format with one scale per
    tensor: the keys are ``k_scale * widen(k)`` and the values ``v_scale * widen(v)``;
    the query keeps its own type.  Otherwise the same gather and attention."""
    S, H, D = q.shape
    out = np.zeros((S, H, D), np.float64)
    idx = list(range(S)) if seqs is None else list(seqs)
    for s, (Ks, Vs) in zip(idx, gather_contiguous(k_cache, v_cache, block_tables, context_lens,
                                                  block_size, idx)):
        L = int(context_lens[s])
        out[s:s + 1] = attend_rows(widen(q[s:s + 1], q_dtype), k_scale * widen(Ks, kv_dtype),
                                   v_scale * widen(Vs, kv_dtype), scale, [L])
    return out


# --------------------------------------------------------------------------
# step 1: gather through the block table
# --------------------------------------------------------------------------

def gather_contiguous(k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                      context_lens: np.ndarray, block_size: int,
                      seqs: Optional[Sequence[int]] = None) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Per sequence, its K and V as ``[L_s, num_kv_heads, head_dim]`` arrays in logical order.

    Token ``t`` lives in physical block ``block_tables[s, t // block_size]`` at
    slot ``t % block_size`` (the per-sequence table mapping logical positions to
    physical blocks).  Values are returned in the storage dtype (no widening), so
    the result can be compared bit for bit with a device gather.
    """
    out = []
    idx = range(len(context_lens)) if seqs is None else seqs
    for s in idx:
        L = int(context_lens[s])
        t = np.arange(L)
        phys = np.asarray(block_tables[s])[t // block_size]
        slot = t % block_size
        # k_cache[phys, :, slot, :] -> [L, Hk, D]
        out.append((k_cache[phys, :, slot, :], v_cache[phys, :, slot, :]))
    return out


# --------------------------------------------------------------------------
# step 2: textbook softmax attention
# --------------------------------------------------------------------------

def attend_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                visible: Sequence[int], return_lse: bool = False):
    """Softmax attention for a handful of query rows of one sequence, in fp64.

    ``q``: ``[n, H, D]``; ``K``, ``V``: ``[L, Hk, D]``; ``visible[i]``: the number of
    leading keys row ``i`` may see.  For query head ``h`` of KV group ``g``:
    ``z_t = scale * <q_h, k_t>``, ``w_t = exp(z_t - max z)``,
    ``out = sum_t w_t v_t / sum_t w_t`` and ``lse = max z + log(sum_t w_t)``.
    """
    n, H, D = q.shape
    Hk = K.shape[1]
    G = H // Hk
    out = np.zeros((n, H, D), np.float64)
    lse = np.full((n, H), -np.inf, np.float64)
    for i in range(n):
        T = int(visible[i])
        if T <= 0:
            continue
        for g in range(Hk):
            qg = q[i, g * G:(g + 1) * G, :]            # [G, D]
            Kg = K[:T, g, :]                           # [T, D]
            Vg = V[:T, g, :]
            z = scale * (qg @ Kg.T)                    # [G, T]
            m = z.max(axis=1, keepdims=True)
            w = np.exp(z - m)
            den = w.sum(axis=1, keepdims=True)
            out[i, g * G:(g + 1) * G, :] = (w @ Vg) / den
            lse[i, g * G:(g + 1) * G] = (m + np.log(den))[:, 0]
    return (out, lse) if return_lse else out


def paged_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    block_tables: np.ndarray, context_lens: np.ndarray, q_offsets: np.ndarray,
                    block_size: int, scale: float, dtype: str, causal: bool = True,
                    seqs: Optional[Sequence[int]] = None, return_lse: bool = False):
    """Paged attention for ``q`` rows ``[total_q, H, D]`` grouped by ``q_offsets`` (``[S+1]``).

    Row ``i`` of sequence ``s`` (of ``n_s = q_offsets[s+1] - q_offsets[s]`` rows)
    sees keys ``t <= L_s - n_s + i`` when ``causal``, otherwise all ``L_s`` keys.
    Returns fp64 ``[total_q, H, D]`` (rows of sequences not in ``seqs`` stay zero).
    """
    total_q, H, D = q.shape
    out = np.zeros((total_q, H, D), np.float64)
    lse = np.full((total_q, H), -np.inf, np.float64)
    S = len(context_lens)
    idx = list(range(S)) if seqs is None else list(seqs)
    gathered = gather_contiguous(k_cache, v_cache, block_tables, context_lens, block_size, idx)
    for s, (Ks, Vs) in zip(idx, gathered):
        a, b = int(q_offsets[s]), int(q_offsets[s + 1])
        n, L = b - a, int(context_lens[s])
        if n == 0:
            continue
        vis = [L - n + i + 1 if causal else L for i in range(n)]
        vis = [max(0, min(L, x)) for x in vis]
        o, l = attend_rows(widen(q[a:b], dtype), widen(Ks, dtype), widen(Vs, dtype), scale,
                           vis, return_lse=True)
        out[a:b] = o
        lse[a:b] = l
    return (out, lse) if return_lse else out


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, dtype,
                 seqs=None, return_lse=False):
    """Decode step: one query row per sequence (``q``: ``[S, H, D]``) over all ``L_s`` keys."""
    S = len(context_lens)
    q_offsets = np.arange(S + 1, dtype=np.int64)
    return paged_attention(q, k_cache, v_cache, block_tables, context_lens, q_offsets,
                           block_size, scale, dtype, causal=False, seqs=seqs, return_lse=return_lse)


def paged_multiq(q, k_cache, v_cache, block_tables, context_lens, q_offsets, block_size, scale,
                 dtype, causal=True, seqs=None, return_lse=False):
    """Several query rows per sequence (speculative verification or a prefill chunk)."""
    return paged_attention(q, k_cache, v_cache, block_tables, context_lens, q_offsets,
                           block_size, scale, dtype, causal=causal, seqs=seqs,
                           return_lse=return_lse)


# --------------------------------------------------------------------------
# second, independent formulation for tiny inputs
# --------------------------------------------------------------------------

def brute_force_paged_attention(q, k_cache, v_cache, block_tables, context_lens, q_offsets,
                                block_size, scale, dtype, causal=True):
    """Pure-Python loops over (sequence, row, head, key) that read the pool through the
    block table one element at a time; never builds a contiguous copy, never calls a
    matrix routine.  Softmax is evaluated as ``exp(z_t) / sum exp(z_u)`` after
    subtracting the maximum, with ``math.fsum`` sums.  For tiny inputs only."""
    import math
    qf, kf, vf = widen(q, dtype), widen(k_cache, dtype), widen(v_cache, dtype)
    total_q, H, D = qf.shape
    Hk = kf.shape[1]
    G = H // Hk
    out = np.zeros((total_q, H, D), np.float64)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        a, b = int(q_offsets[s]), int(q_offsets[s + 1])
        n = b - a
        for i in range(n):
            T = (L - n + i + 1) if causal else L
            T = max(0, min(L, T))
            if T == 0:
                continue
            for h in range(H):
                g = h // G
                scores = []
                for t in range(T):
                    blk = int(block_tables[s][t // block_size])
                    r = t % block_size
                    scores.append(scale * math.fsum(qf[a + i, h, d] * kf[blk, g, r, d]
                                                    for d in range(D)))
                mx = max(scores)
                w = [math.exp(z - mx) for z in scores]
                den = math.fsum(w)
                for d in range(D):
                    num = math.fsum(w[t] * vf[int(block_tables[s][t // block_size]), g,
                                               t % block_size, d] for t in range(T))
                    out[a + i, h, d] = num / den
    return out


# --------------------------------------------------------------------------
# KV byte accounting
# --------------------------------------------------------------------------

def kv_bytes_per_token(layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V for one token across ``layers``: 2 * layers * (num_kv_heads * head_dim) * bytes.

    This is the pages' own KV-size arithmetic for Llama-3-70B with GQA-8
    ("Local_LLM_03_vLLM_Architecture", KV-cache sizing slide), and the product
    "context x layers x kv-heads x head_dim x dtype bytes" per tensor ("vLLM: LLM
    Inference That Doesn't Waste Your GPU", section "KV cache, in one picture")
    counted once for K and once for V."""
    return 2 * layers * num_kv_heads * head_dim * elem_bytes


def kv_bytes_for_context(context_lens, layers: int, num_kv_heads: int, head_dim: int,
                         elem_bytes: int) -> int:
    """KV bytes that attention over these contexts must read: every visible token once."""
    return int(np.sum(np.asarray(context_lens, dtype=np.int64))) * \
        kv_bytes_per_token(layers, num_kv_heads, head_dim, elem_bytes)
