"""Plain fp64 CPU oracle for MLA speculative-decoding verify attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP kernels (its bf16 decode, gather, masking, softmax and
split/merge are written here, independently).

What it computes (the pages' subject, restated):
  * "Verify attention" is the speculative-decoding step in which the target
    model checks the drafter's proposed tokens (magik.net, "The Decisive A/B",
    section "The Context: A Custom Kernel in Production").  Several draft
    tokens of one request are scored in one pass, every head attending over
    the request's cached keys.
  * The cache is MLA (Multi-head Latent Attention): all heads share one latent
    row per token (magik.net, "The Moment of Truth", opening section).  Each
    row holds 512 latent dims followed by 64 rope dims; q and k are 576-wide
    and v is the first 512 dims of the same row.
  * The cache is paged with page_size = 1, so every token is its own scattered
    slot and is fetched through a slot index ("The Decisive A/B", "The
    Context").
  * The pages' kernel splits the keys of a request into chunks ("KV-split
    flash-decode"), computes a partial result per chunk and then reduces the
    partials ("The Decisive A/B", "The Context" and "What This Reveals About
    the Bottleneck").  The split is an exact regrouping of one softmax, so the
    unsplit definition below is the result; `verify_attention_split` follows
    the partial + reduce steps for the split/unsplit pin.

Readings where the pages are silent:
  * seq_lens[b] counts the request's draft tokens; their rows are the last
    q_lens[b] entries of the request's slot list.
  * Causal within the draft block, inclusive: draft t (0-based) sees keys
    j <= L - Q + t, i.e. n_t = L - Q + t + 1 keys.
  * scores s_j = scale * q . k_j with scale = 1/sqrt(192); lse is the natural
    log of sum_j exp(s_j), with the scale included.
  * q is token-major [T_q, H, 576], requests concatenated in order; slot_idx is
    packed [sum L]; out is [T_q, H, 512]; lse is [T_q, H].

All arithmetic is float64 on bf16-decoded inputs.
"""
from __future__ import annotations

import numpy as np

D_QK = 576
D_V = 512


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly: a bf16 value is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def visible_count(seq_len: int, q_len: int, t: int) -> int:
    """Number of keys draft token t may attend to: the prefix plus drafts 0..t."""
    return seq_len - q_len + t + 1


def _offsets(lens: np.ndarray) -> np.ndarray:
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return out


def _gather_keys(kv_pool: np.ndarray, slot_idx: np.ndarray, start: int, count: int) -> np.ndarray:
    """Fetch the request's latent rows through its slot list (page_size = 1)."""
    slots = np.asarray(slot_idx[start:start + count], dtype=np.int64)
    return bf16_bits_to_f64(kv_pool[slots])


def _scores(q_rows: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s[h, j] = scale * sum_d q[h, d] k[j, d] over all 576 dims."""
    return scale * (q_rows @ keys.T)


def _softmax_stats(s: np.ndarray):
    """Row-wise max-shifted exponentials: returns (e, m, z) with e = exp(s - m), z = sum e."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e, m[..., 0], z[..., 0]


def _attend(q_rows: np.ndarray, keys: np.ndarray, scale: float):
    """Softmax attention of q_rows [H, 576] over keys [n, 576] (v = keys[:, :512]).

    Returns out [H, 512] and lse [H].  n == 0 gives out = 0 and lse = -inf.
    """
    h = q_rows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((h, D_V)), np.full(h, -np.inf)
    s = _scores(q_rows, keys, scale)
    e, m, z = _softmax_stats(s)
    out = (e / z[:, None]) @ keys[:, :D_V]
    lse = m + np.log(z)
    return out, lse


def verify_attention(q, kv_pool, slot_idx, seq_lens, q_lens, scale):
    """Unsplit definition.  q: uint16 [T_q, H, 576]; kv_pool: uint16 [slots, 576].

    Returns (out float64 [T_q, H, 512], lse float64 [T_q, H]).
    """
    q = np.asarray(q)
    t_q, heads, _ = q.shape
    out = np.zeros((t_q, heads, D_V))
    lse = np.full((t_q, heads), -np.inf)
    ko = _offsets(seq_lens)
    qo = _offsets(q_lens)
    for b in range(len(seq_lens)):
        L, Q = int(seq_lens[b]), int(q_lens[b])
        if Q == 0:
            continue
        keys = _gather_keys(kv_pool, slot_idx, int(ko[b]), L)
        for t in range(Q):
            n = visible_count(L, Q, t)
            row = int(qo[b]) + t
            out[row], lse[row] = _attend(bf16_bits_to_f64(q[row]), keys[:n], scale)
    return out, lse


def verify_attention_rows(q, kv_pool, slot_idx, seq_lens, q_lens, scale, rows):
    """The same definition evaluated only at the (token, head) pairs in `rows`.

    rows: iterable of (token_row, head).  Returns (out [len(rows), 512], lse [len(rows)]).
    Used to check full-size runs at sampled outputs.
    """
    ko = _offsets(seq_lens)
    qo = _offsets(q_lens)
    req_of_token = np.repeat(np.arange(len(q_lens)), np.asarray(q_lens, dtype=np.int64))
    rows = list(rows)
    out = np.zeros((len(rows), D_V))
    lse = np.zeros(len(rows))
    cache = {}
    for i, (tok, h) in enumerate(rows):
        b = int(req_of_token[tok])
        L, Q = int(seq_lens[b]), int(q_lens[b])
        if b not in cache:
            cache.clear()
            cache[b] = _gather_keys(kv_pool, slot_idx, int(ko[b]), L)
        t = tok - int(qo[b])
        n = visible_count(L, Q, t)
        o, s = _attend(bf16_bits_to_f64(q[tok, h:h + 1]), cache[b][:n], scale)
        out[i], lse[i] = o[0], s[0]
    return out, lse


def split_bounds(seq_len: int, nsplit: int):
    """Contiguous key chunks of c = ceil(L / nsplit) keys; trailing chunks may be empty."""
    c = -(-seq_len // nsplit) if seq_len > 0 else 0
    return [(min(s * c, seq_len), min((s + 1) * c, seq_len)) for s in range(nsplit)]


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Reduce per-split partials: lse = logsumexp_s lse_s; out = sum_s exp(lse_s - lse) o_s.

    o_parts [S, ..., 512], lse_parts [S, ...]; -inf partials carry no weight.
    All -inf gives out = 0 and lse = -inf.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)
    z = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(z > 0, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    out = np.einsum("s...,s...d->...d", w / np.where(z > 0, z, 1.0), o_parts)
    return out, lse


def verify_attention_split(q, kv_pool, slot_idx, seq_lens, q_lens, scale, nsplit, return_partials=False):
    """KV-split form: per-chunk partials (o_s normalised within the chunk, lse_s), then the reduce.

    Returns (out, lse) and, if asked, the partials as arrays
    o_part [T_q, H, nsplit, 512] and lse_part [T_q, H, nsplit].
    """
    q = np.asarray(q)
    t_q, heads, _ = q.shape
    o_part = np.zeros((t_q, heads, nsplit, D_V))
    lse_part = np.full((t_q, heads, nsplit), -np.inf)
    ko = _offsets(seq_lens)
    qo = _offsets(q_lens)
    for b in range(len(seq_lens)):
        L, Q = int(seq_lens[b]), int(q_lens[b])
        if Q == 0:
            continue
        keys = _gather_keys(kv_pool, slot_idx, int(ko[b]), L)
        bounds = split_bounds(L, nsplit)
        for t in range(Q):
            n = visible_count(L, Q, t)
            row = int(qo[b]) + t
            qr = bf16_bits_to_f64(q[row])
            for s, (lo, hi) in enumerate(bounds):
                hi = min(hi, n)
                lo = min(lo, hi)
                o_part[row, :, s], lse_part[row, :, s] = _attend(qr, keys[lo:hi], scale)
    out, lse = merge_partials(np.moveaxis(o_part, 2, 0), np.moveaxis(lse_part, 2, 0))
    if return_partials:
        return out, lse, o_part, lse_part
    return out, lse


__all__ = [
    "bf16_bits_to_f64", "visible_count", "verify_attention", "verify_attention_rows",
    "verify_attention_split", "merge_partials", "split_bounds",
]
