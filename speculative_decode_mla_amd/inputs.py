"""Seeded synthetic inputs for MLA speculative-decoding verify attention.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It draws random numbers and encodes them to bf16; it holds none
of the attention arithmetic (no scores, no softmax, no gather).

Workloads (all bf16 q/kv drawn from N(0, 1), page_size = 1, so every token of
a request owns one scattered row of the latent KV pool; each row is 512 latent
dims followed by 64 rope dims, and v is the first 512 dims):

  tiny      B=1,  H=16, Q=4,  L=256,   4096-slot pool,  nsplit=1
  ctx4k     B=1,  H=64, Q=8,  L=4096,  1M-slot pool,    nsplit=8
  ctx23k    B=1,  H=64, Q=16, L=23000, 1M-slot pool,    nsplit=16
  ctx64k    B=1,  H=64, Q=16, L=65536, 2M-slot pool,    nsplit=32
  ctx91k    B=1,  H=64, Q=16, L=91000, 2M-slot pool,    nsplit=32
  batch16   B=16, H=64, Q=16, L_b log-uniform in [1k, 64k], 4M-slot pool, nsplit=32
  ctx64k_sink  ctx64k's inputs, then one planted dominant key in every 2,048-key chunk (below)

Draw order for a seed (fixed, so that every consumer sees the same bytes):
  1. rng = numpy.random.default_rng(seed)
  2. ragged batch only: L = rint(exp(uniform(ln 1024, ln 65536, B)))
  3. slots = rng.permutation(num_slots)[:sum(L)]; request b takes the next L_b
  4. kv rows = standard_normal((sum(L), 576), float32) -> bf16 (RNE)
  5. q = standard_normal((sum(Q), H, 576), float32) -> bf16 (RNE)
  6. planted keys (workloads with sink_nats > 0 only, after all of the above, so the
     other draws are those of the plain workload): in every chunk of sink_every keys of
     request 0, key chunk_start + 32 + integers(0, sink_every - 32) (never in the chunk's
     first 32 keys) becomes bf16(c * q[t, h]) for a random (token, head) row (t, h), with
     c = sink_nats / (scale * |q[t, h]|^2): that row's score for the key is about sink_nats
     nats, far above the scores of N(0, 1) keys (a few nats), like an attention sink.
Pool rows that no request references hold the bf16 quiet NaN 0x7FC0, so a
stray read shows up as NaN in the result.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

D_QK = 576          # 512 latent + 64 rope
D_V = 512           # v is the first 512 dims of each latent row
BF16_QNAN = 0x7FC0
SM_SCALE = 1.0 / math.sqrt(192.0)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    q_len: int
    ctx: int | None          # None: ragged, log-uniform lengths drawn from the seed
    num_slots: int
    nsplit: int
    seed: int
    ctx_lo: int = 1024
    ctx_hi: int = 65536
    sink_nats: float = 0.0   # > 0: plant one dominant key per chunk of sink_every keys (draw step 6)
    sink_every: int = 2048


WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 4, 256, 4096, 1, 0),
    "ctx4k": Workload("ctx4k", 1, 64, 8, 4096, 1 << 20, 8, 1),
    "ctx23k": Workload("ctx23k", 1, 64, 16, 23000, 1 << 20, 16, 2),
    "ctx64k": Workload("ctx64k", 1, 64, 16, 65536, 1 << 21, 32, 3),
    "ctx91k": Workload("ctx91k", 1, 64, 16, 91000, 1 << 21, 32, 4),
    "batch16": Workload("batch16", 16, 64, 16, None, 1 << 22, 32, 5),
    # q_len = 1 decode steps (one token per request, no drafts to verify)
    "decode64k": Workload("decode64k", 1, 64, 1, 65536, 1 << 21, 128, 6),
    # ctx64k with one key per 2,048-key chunk (one split each at nsplit 32) scoring ~60 nats for one row
    "ctx64k_sink": Workload("ctx64k_sink", 1, 64, 16, 65536, 1 << 21, 32, 3, sink_nats=60.0),
    "decode_batch16": Workload("decode_batch16", 16, 64, 1, None, 1 << 22, 32, 7),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_QNAN
    return rounded


@dataclasses.dataclass
class VerifyInputs:
    """Host-side inputs of one verify call.  Arrays are numpy, bf16 kept as uint16 bits."""
    q: np.ndarray            # uint16 [T_q, H, 576]
    kv_rows: np.ndarray      # uint16 [sum(L), 576], request-major: request b's L_b rows in key order
    slot_idx: np.ndarray     # int32  [sum(L)], pool slot of each kv row
    seq_lens: np.ndarray     # int32  [B]
    q_lens: np.ndarray       # int32  [B]
    num_slots: int
    heads: int
    scale: float = SM_SCALE

    def pool(self) -> np.ndarray:
        """Materialise the full host pool: referenced rows scattered to their slots, the rest NaN."""
        pool = np.full((self.num_slots, D_QK), BF16_QNAN, dtype=np.uint16)
        pool[self.slot_idx] = self.kv_rows
        return pool

    def sparse_pool(self) -> "SparsePool":
        """The same pool without materialising the unreferenced rows (for large pools)."""
        return SparsePool(self.kv_rows, self.slot_idx, self.num_slots)


class SparsePool:
    """Indexable like the host pool (pool[slots] -> rows); unreferenced slots read as NaN rows."""

    def __init__(self, kv_rows: np.ndarray, slot_idx: np.ndarray, num_slots: int):
        self.kv_rows = kv_rows
        self.row_of_slot = np.full(num_slots, -1, dtype=np.int64)
        self.row_of_slot[slot_idx] = np.arange(len(slot_idx))
        self.shape = (num_slots, D_QK)

    def __getitem__(self, slots):
        r = self.row_of_slot[np.asarray(slots, dtype=np.int64)]
        out = self.kv_rows[np.maximum(r, 0)]
        out[r < 0] = BF16_QNAN
        return out


def ragged_lengths(rng: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    return np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), batch))).astype(np.int64)


def make_inputs(w: Workload | str, seed: int | None = None) -> VerifyInputs:
    """Draw the inputs of workload `w` (see the module docstring for the draw order)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if w.ctx is None:
        lens = ragged_lengths(rng, w.batch, w.ctx_lo, w.ctx_hi)
    else:
        lens = np.full(w.batch, w.ctx, dtype=np.int64)
    qlens = np.full(w.batch, w.q_len, dtype=np.int64)
    x = make_custom(rng, lens, qlens, w.heads, w.num_slots)
    if w.sink_nats > 0:
        plant_dominant_keys(rng, x, w.sink_nats, w.sink_every)
    return x


def plant_dominant_keys(rng: np.random.Generator, x: VerifyInputs, nats: float, every: int) -> None:
    """Draw step 6: in every chunk of `every` keys of request 0, one key (not among the chunk's
    first 32) becomes bf16(c * q[t, h]) for a random row, c = nats / (scale * |q[t, h]|^2)."""
    L, Q = int(x.seq_lens[0]), int(x.q_lens[0])
    for start in range(0, L, every):
        span = min(every, L - start)
        if span <= 32:
            break
        j = start + 32 + int(rng.integers(0, span - 32))
        t, h = int(rng.integers(0, Q)), int(rng.integers(0, x.heads))
        qv = (x.q[t, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        c = nats / (x.scale * float(np.dot(qv, qv)))
        x.kv_rows[j] = f32_to_bf16_bits((c * qv).astype(np.float32))


def make_custom(rng: np.random.Generator, seq_lens, q_lens, heads: int, num_slots: int,
                scale: float = SM_SCALE) -> VerifyInputs:
    """Inputs with explicit per-request lengths, drawn in the fixed order from `rng`."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    total = int(seq_lens.sum())
    if total > num_slots:
        raise ValueError(f"pool of {num_slots} slots cannot hold {total} rows")
    if np.any(q_lens > seq_lens) or np.any(q_lens < 0):
        raise ValueError("each request needs 0 <= q_len <= seq_len")
    slots = rng.permutation(num_slots)[:total].astype(np.int32)
    kv = f32_to_bf16_bits(rng.standard_normal((total, D_QK), dtype=np.float32))
    t_q = int(q_lens.sum())
    q = f32_to_bf16_bits(rng.standard_normal((t_q, heads, D_QK), dtype=np.float32))
    return VerifyInputs(q=q, kv_rows=kv, slot_idx=slots, seq_lens=seq_lens.astype(np.int32),
                        q_lens=q_lens.astype(np.int32), num_slots=num_slots, heads=heads, scale=scale)
