"""Plain float64 definition of decode attention over a host/HBM split KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is blocked,
fused or reordered beyond what the definition says; numpy supplies the
elementwise maths and the dot products.

Sources (page title, section):
  * DirectKV README, introduction: KV lives in CPU-pinned memory; one kernel
    does K/V projection, Neox RoPE rotation and multi-head attention.
  * DirectKV README, Attribution: online softmax of FlashAttention, streaming KV
    from CPU-pinned memory without a GPU staging buffer.
  * DirectKV README, Step 6 (correctness tests): new K and V are checked after
    projection, O after attention.
  * SplitKernel README, Overview / Key Features / Usage: the KV cache is
    partitioned between host and device memory by an offloading ratio.

Readings where the pages are silent (each listed again in the design notes):
  * Neox RoPE = rotate-half pairing (i, i + D/2), f_i = theta^(-2i/D).
  * Keys are rotated once, at append, and stored as bfloat16 (round to nearest
    even); attention reads the stored keys.  The query is rotated at its own
    position.  Values are stored unrotated.
  * The query of sequence b sits at position N_b - 1 and attends to all N_b
    cached tokens (itself included); scale = 1/sqrt(D); no mask or soft-cap.
  * LSE is the natural log of the sum of exp(scaled score); partial outputs
    are normalised; an empty partition is (o, lse) = (0, -inf).
  * GQA: query head h reads KV head floor(h / g), g = Hq / Hkv.
  * Contiguous split: the oldest floor(r * L) tokens (IEEE double product) are
    host-resident; paged layout: entry = phys << 1 | tier, row = phys * P + t % P.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------- bfloat16

def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_rne_bits(x) -> np.ndarray:
    """Round float64 values once to bfloat16, nearest with ties to even.

    bfloat16 keeps 8 significant bits.  For a normal value x = m * 2^e with
    0.5 <= |m| < 1, the nearest bfloat16 is rint(m * 2^8) * 2^(e - 8), where
    rint rounds halves to even.  Below the smallest normal (2^-126) the grid
    is the fixed quantum 2^-133.  The rounded value is exactly representable
    in float32, whose upper 16 bits are the bfloat16 pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
    r = np.where(np.abs(x) < 2.0 ** -126, sub, normal)
    f = r.astype(np.float32)  # exact: r has at most 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- RoPE (Neox)

def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """f_i = theta^(-2i/D), i = 0 .. D/2 - 1 (Neox RoPE named in the DirectKV
    README introduction; the frequency ladder is the rotary-embedding one)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / head_dim)


def rope_neox(x, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE of x[..., D] at integer positions ``pos`` (broadcast
    against x[..., 0]).  Pairs (i, i + D/2) rotate by angle pos * f_i:
        y_i        = x_i cos a - x_{i+D/2} sin a
        y_{i+D/2}  = x_{i+D/2} cos a + x_i sin a
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    f = rope_inv_freq(D, theta)
    pos = np.asarray(pos, dtype=np.float64)
    if np.broadcast_shapes(pos.shape, x.shape[:-1]) != x.shape[:-1]:
        raise ValueError(f"positions {pos.shape} do not broadcast to the vectors {x.shape[:-1]}")
    a = pos[..., None] * f
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------- projection

def project(x, w) -> np.ndarray:
    """New-token projection k = x W (DirectKV README introduction: the fused
    kernel projects K and V).  x [n, hidden], W [hidden, Hkv*D] row-major with
    output column h*D + d; no bias."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


# ---------------------------------------------------------------- attention

def attention(q_rot, k, v, scale: float):
    """Softmax attention of every query head over all N tokens.

    q_rot [Hq, D] (already rotated), k and v [N, Hkv, D].  Returns o [Hq, D]
    and lse [Hq] (natural log of sum_t exp(s_t)).
    """
    q_rot = np.asarray(q_rot, dtype=np.float64)
    Hq, D = q_rot.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    o = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    for h in range(Hq):
        kvh = h // g
        kh = np.asarray(k[:, kvh, :], dtype=np.float64)
        vh = np.asarray(v[:, kvh, :], dtype=np.float64)
        s = scale * (kh @ q_rot[h])
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        o[h] = (e / z) @ vh
        lse[h] = m + math.log(z)
    return o, lse


def attention_subset(q_rot, k, v, idx, scale: float):
    """Attention restricted to token indices ``idx``; empty -> (0, -inf)."""
    idx = np.asarray(idx, dtype=np.int64)
    Hq, D = np.asarray(q_rot).shape
    if idx.size == 0:
        return np.zeros((Hq, D)), np.full(Hq, -np.inf)
    return attention(q_rot, k[idx], v[idx], scale)


def merge_lse(os_, lses):
    """Combine normalised partials (o_i, lse_i) into the full result:
    M = max lse_i, w_i = exp(lse_i - M), o = sum w_i o_i / sum w_i,
    lse = M + ln sum w_i.  Partials with lse = -inf carry weight 0.
    os_ [n, Hq, D], lses [n, Hq]."""
    os_ = np.asarray(os_, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    n, Hq, D = os_.shape
    o = np.zeros((Hq, D))
    lse = np.full(Hq, -np.inf)
    for h in range(Hq):
        col = lses[:, h]
        if np.all(np.isneginf(col)):
            continue
        M = col.max()
        w = np.where(np.isneginf(col), 0.0, np.exp(col - M))
        o[h] = (w[:, None] * os_[:, h, :]).sum(axis=0) / w.sum()
        lse[h] = M + math.log(w.sum())
    return o, lse


# ---------------------------------------------------------------- placement

def contig_split_point(ratio: float, length: int) -> int:
    """Number of leading (oldest) tokens held in host memory: floor(r * L),
    the product taken in IEEE double (SplitKernel README, Usage: placement
    and offloading-ratio utilities)."""
    return int(math.floor(float(ratio) * float(length)))


def contig_slot(b: int, t: int, length: int, ratio: float, host_stride: int, dev_stride: int):
    """(tier, row) of token t of sequence b in the contiguous-split layout.
    tier 1 = host pool row b*host_stride + t; tier 0 = device pool row
    b*dev_stride + (t - n_host)."""
    n_host = contig_split_point(ratio, length)
    if t < n_host:
        return 1, b * host_stride + t
    return 0, b * dev_stride + (t - n_host)


def paged_slot(table, b: int, t: int, page: int):
    """(tier, row) of token t of sequence b in the paged layout."""
    e = int(table[b][t // page])
    return e & 1, (e >> 1) * page + t % page


# ---------------------------------------------------------------- decode

def _stored_keys(k_raw_bits, theta, rounded=True, positions=None):
    k = bf16_to_f64(k_raw_bits)
    n = k.shape[0]
    pos = np.arange(n) if positions is None else np.asarray(positions)
    kr = rope_neox(k, pos[:, None], theta)
    if rounded:
        kr = bf16_to_f64(bf16_rne_bits(kr))
    return kr


def decode_sequence(q_bits, k_raw_bits, v_bits, q_pos: int, theta: float, scale: float,
                    heads=None, rounded_keys: bool = True, key_positions=None):
    """Decode attention of one sequence over its whole cache.

    q_bits [Hq, D], k_raw_bits / v_bits [N, Hkv, D] (bf16 bits, keys before
    RoPE).  Token t's key is rotated at position t; the query at ``q_pos``.
    With ``rounded_keys`` the attention reads bf16-rounded rotated keys, as
    held in the cache after append.  ``heads`` restricts the query heads (for
    sampling at full size); the KV work is done one KV head at a time.
    ``key_positions`` overrides the rotation position of each cached token
    (default: token t at position t).
    Returns o [len(heads), D], lse [len(heads)].
    """
    q = bf16_to_f64(q_bits)
    Hq, D = q.shape
    Hkv = k_raw_bits.shape[1]
    g = Hq // Hkv
    heads = list(range(Hq)) if heads is None else list(heads)
    q_rot = rope_neox(q, np.full(Hq, q_pos), theta)
    o = np.zeros((len(heads), D))
    lse = np.zeros(len(heads))
    by_kv = {}
    for j, h in enumerate(heads):
        by_kv.setdefault(h // g, []).append((j, h))
    for kvh, hs in by_kv.items():
        kk = _stored_keys(k_raw_bits[:, kvh:kvh + 1, :], theta, rounded_keys, key_positions)
        vv = bf16_to_f64(v_bits[:, kvh:kvh + 1, :])
        sub_q = np.stack([q_rot[h] for _, h in hs])
        oo, ll = attention(sub_q, kk, vv, scale)
        for r, (j, _) in enumerate(hs):
            o[j], lse[j] = oo[r], ll[r]
    return o, lse


def decode_sequence_split(q_bits, k_raw_bits, v_bits, q_pos: int, theta: float, scale: float,
                          parts, rounded_keys: bool = True):
    """Same result assembled from partitions: attention over each token set in
    ``parts`` (a list of index arrays, possibly empty) then the LSE merge."""
    q = bf16_to_f64(q_bits)
    Hq = q.shape[0]
    q_rot = rope_neox(q, np.full(Hq, q_pos), theta)
    kk = _stored_keys(k_raw_bits, theta, rounded_keys)
    vv = bf16_to_f64(v_bits)
    os_, ls = [], []
    for idx in parts:
        o, l = attention_subset(q_rot, kk, vv, idx, scale)
        os_.append(o)
        ls.append(l)
    return merge_lse(np.stack(os_), np.stack(ls))


def decode_batch(q_bits, caches, q_pos, theta: float, scale: float, rounded_keys: bool = True):
    """q_bits [B, Hq, D]; caches[b] = (k_raw_bits [N_b,Hkv,D], v_bits [N_b,Hkv,D])."""
    outs, lses = [], []
    for b, (kb, vb) in enumerate(caches):
        o, l = decode_sequence(q_bits[b], kb, vb, int(q_pos[b]), theta, scale,
                               rounded_keys=rounded_keys)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def append_expected_rows(k_new, v_new, pos, theta: float, k_is_bits: bool = True):
    """Rows written by an append of one new token at position ``pos``.

    k_new / v_new [Hkv, D]: bf16 bits (no-projection mode) or float64 values
    from :func:`project` (projection mode, ``k_is_bits=False``).  Returns the
    stored bit patterns: bf16(RoPE(k, pos)) and bf16(v), each rounded once.
    """
    if k_is_bits:
        k = bf16_to_f64(k_new)
        v_bits = np.asarray(v_new, dtype=np.uint16)
    else:
        k = np.asarray(k_new, dtype=np.float64)
        v_bits = bf16_rne_bits(v_new)
    kr = rope_neox(k, np.full(k.shape[0], pos), theta)
    return bf16_rne_bits(kr), v_bits


# ---------------------------------------------------------------- prefill

def prefill_sequence(q_bits, k_raw_bits, v_bits, q_pos0: int, theta: float, scale: float,
                     heads=None, rounded_keys: bool = True, row_block: int = 256):
    """Causal attention of n new query tokens over a sequence's cache.

    DirectKV README, introduction (one kernel projects, rotates and attends)
    and Step 6 ("Prefill (all new KV)" cases).  Query row j sits at position
    p_j = q_pos0 + j, is rotated there, and attends to cached tokens
    0 .. p_j (its own key included).  q_bits [n, Hq, D]; k_raw_bits / v_bits
    [N, Hkv, D] with N >= q_pos0 + n (keys before RoPE, rotated at their own
    positions and stored as bf16 when ``rounded_keys``).
    Returns o [n, len(heads), D], lse [n, len(heads)].
    """
    q = bf16_to_f64(q_bits)
    n, Hq, D = q.shape
    N, Hkv = k_raw_bits.shape[0], k_raw_bits.shape[1]
    g = Hq // Hkv
    heads = list(range(Hq)) if heads is None else list(heads)
    assert q_pos0 + n <= N, "every query position must be in the cache"
    pos = q_pos0 + np.arange(n)
    q_rot = rope_neox(q, np.repeat(pos[:, None], Hq, axis=1), theta)
    o = np.zeros((n, len(heads), D))
    lse = np.zeros((n, len(heads)))
    by_kv = {}
    for j, h in enumerate(heads):
        by_kv.setdefault(h // g, []).append((j, h))
    last = q_pos0 + n
    for kvh, hs in by_kv.items():
        kk = _stored_keys(k_raw_bits[:last, kvh:kvh + 1, :], theta, rounded_keys)[:, 0, :]
        vv = bf16_to_f64(v_bits[:last, kvh, :])
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            for j, h in hs:
                s = scale * (q_rot[r0:r1, h, :] @ kk.T)          # [rows, last]
                mask = np.arange(last)[None, :] > pos[r0:r1, None]
                s = np.where(mask, -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                o[r0:r1, j, :] = (e / z) @ vv
                lse[r0:r1, j] = (m + np.log(z))[:, 0]
    return o, lse


# ---------------------------------------------------------------- offloaded linear

def linear(x_bits, w_bits) -> np.ndarray:
    """Offloaded linear layer, y = x W^T (SplitKernel README, Overview and Key
    Features: weights fetched directly from the remote tier for an offloaded
    linear).  Reading: W is stored like a PyTorch linear weight, [out][in]
    bf16; x is [M][in] bf16; no bias; y [M][out] in float64."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T


def linear_split_rows(ratio: float, out_features: int) -> int:
    """Output rows of W held in host memory: the first floor(r * N) rows (the
    same IEEE-double rule as the KV split; SplitKernel README, Usage:
    placement and offloading-ratio utilities)."""
    return contig_split_point(ratio, out_features)


def linear_split(x_bits, w_host_bits, w_dev_bits) -> np.ndarray:
    """y for W split by output rows: host rows first, then HBM rows."""
    return np.concatenate([linear(x_bits, w_host_bits), linear(x_bits, w_dev_bits)], axis=1)
