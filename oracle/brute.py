"""Second, independent oracle route for small inputs -- TEST INFRASTRUCTURE (numpy, fp64).

Where the C oracle walks each sequence forward through its block table, this route starts from the pool:
for every physical block it finds which logical block numbers of the sequence point at it, turns each slot of
such a block into a logical position j * block_size + offset, keeps the positions below the sequence length,
and so rebuilds the dense per-sequence K and V. A plain dense softmax attention follows (vLLM PagedAttention,
page 1 section 3.1 for the contiguous [batch, heads, max_len, head_dim] cache the paged one replaces; section
3.2 for the block table). Pure-Python loops: use it on tiny inputs only.
"""

from __future__ import annotations

import numpy as np


def _e4m3_as_f32(c: np.ndarray) -> np.ndarray:
    """E4M3 codes rebuilt as fp32 bit patterns: the exponent is re-biased (7 -> 127) and the 3 mantissa bits
    moved to the top of the fp32 mantissa; subnormals (exponent 0) are m / 512, which numpy computes exactly;
    exponent 15 with mantissa 7 is NaN."""
    c = c.astype(np.uint32)
    sign, e, m = c >> 7, (c >> 3) & 15, c & 7
    normal = ((sign << 31) | ((e + 120) << 23) | (m << 20)).view(np.float32)
    sub = np.where(sign == 1, -1.0, 1.0).astype(np.float32) * (m.astype(np.float32) / np.float32(512.0))
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.float32(np.nan), out)


def to_f64(a: np.ndarray) -> np.ndarray:
    """float32 arrays widen exactly; uint16 arrays are bf16 bit patterns (the high half of an fp32); uint8
    arrays are OCP FP8 E4M3 codes."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype == np.uint8:
        return _e4m3_as_f32(a).astype(np.float64)
    raise TypeError(a.dtype)


def dense_kv(key_cache, value_cache, block_table_row, length, k_scale=1.0, v_scale=1.0):
    """Dense [L, Hkv, D] K and V of one sequence, rebuilt by scanning every physical block of the pool."""
    NB, bs, Hkv, D = key_cache.shape
    nblk = -(-int(length) // bs)
    live = np.asarray(block_table_row[:nblk])
    k = np.full((int(length), Hkv, D), np.nan)
    v = np.full((int(length), Hkv, D), np.nan)
    seen = np.zeros(int(length), dtype=bool)
    for b in range(NB):
        for j in np.nonzero(live == b)[0]:
            for off in range(bs):
                t = int(j) * bs + off
                if t < length:
                    k[t] = to_f64(key_cache[b, off]) * k_scale
                    v[t] = to_f64(value_cache[b, off]) * v_scale
                    seen[t] = True
    if not seen.all():
        raise ValueError("a live logical position maps to no physical block of the pool")
    return k, v


def decode(query, key_cache, value_cache, block_tables, context_lens, scale, k_scale=1.0, v_scale=1.0):
    q = to_f64(np.asarray(query))
    B, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        k, v = dense_kv(key_cache, value_cache, block_tables[s], L, k_scale, v_scale)
        for h in range(Hq):
            z = (k[:, h // G, :] @ q[s, h]) * scale
            w = np.exp(z - z.max())
            out[s, h] = (w @ v[:, h // G, :]) / w.sum()
    return out


def contiguous_decode(query, k_contig, v_contig, context_lens, scale):
    """Attention over a contiguous cache [B, Hkv, max_len, D] (the layout paging replaces), fp64 numpy."""
    q = to_f64(np.asarray(query))
    kc = to_f64(np.asarray(k_contig))
    vc = to_f64(np.asarray(v_contig))
    B, Hq, D = q.shape
    G = Hq // kc.shape[1]
    out = np.zeros((B, Hq, D))
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        for h in range(Hq):
            z = (kc[s, h // G, :L] @ q[s, h]) * scale
            w = np.exp(z - z.max())
            out[s, h] = (w @ vc[s, h // G, :L]) / w.sum()
    return out


def decode_multi(query, key_cache, value_cache, block_tables, context_lens, query_start, scale, k_scale=1.0,
                 v_scale=1.0):
    """Several new tokens per sequence: row j of sequence s's QL rows attends over its first L - QL + j + 1
    positions (none when that count is not positive), from the dense K/V rebuilt by scanning the pool."""
    q = to_f64(np.asarray(query))
    T, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        if L == 0 or q1 == q0:
            continue
        k, v = dense_kv(key_cache, value_cache, block_tables[s], L, k_scale, v_scale)
        for j in range(q1 - q0):
            E = L - (q1 - q0) + j + 1
            if E <= 0:
                continue
            for h in range(Hq):
                z = (k[:E, h // G, :] @ q[q0 + j, h]) * scale
                w = np.exp(z - z.max())
                out[q0 + j, h] = (w @ v[:E, h // G, :]) / w.sum()
    return out

