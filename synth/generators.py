"""Seeded input generators (numpy only).

Every function takes an explicit seed and returns host arrays. Values that the
device stores in bfloat16 are drawn in float32 and rounded to bfloat16 with
round-to-nearest-even; both the raw 16-bit patterns (for upload) and their
exact float32 values (for the oracle) are returned, so that both sides see the
identical numbers.

Layouts (row-major, C order):
  two-stream Q      [batch, 2L, n_q_heads, head_dim]
  two-stream K, V   [batch, 2L, n_kv_heads, head_dim]
  decode q          [S, B, n_q_heads, head_dim]
  decode k_new/v_new[S, B, n_kv_heads, head_dim]
  K cache pages     [num_pages, n_kv_heads, page_size, head_dim] (one more
                    leading layers dim in layered_commit_inputs)
  V cache pages     [num_pages, n_kv_heads, head_dim, page_size]  (V is stored
                    transposed inside each page)
  block_table       [S, max_pages] int32, page ids of each sequence's pages
  cache_len         [S] int32
  hidden            [N, D],   lm-head weight W [V, D]
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_CHUNK = 1 << 26


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for s in range(0, flat.size, _CHUNK):
        u = flat[s:s + _CHUNK].view(np.uint32)
        r = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
        out[s:s + _CHUNK] = ((u + r) >> 16).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


@dataclass
class Tensor:
    """A generated tensor: exact float32 values plus, for bfloat16, the bits."""
    f32: np.ndarray
    bits: np.ndarray | None  # uint16 bf16 patterns, or None for float32 storage

    @property
    def shape(self):
        return self.f32.shape


def _make(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "f32":
        return Tensor(np.ascontiguousarray(x, dtype=np.float32), None)
    if dtype == "bf16":
        bits = bf16_round(x)
        return Tensor(bf16_bits_to_f32(bits), bits)
    raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")


def two_stream_qkv(seed: int, batch: int, L: int, n_q_heads: int, n_kv_heads: int,
                   head_dim: int, dtype: str = "bf16"):
    """Q/K/V over z = [x; x~] (length 2L), entries N(0, 1)."""
    rng = np.random.default_rng(seed)
    q = _make(_normal(rng, (batch, 2 * L, n_q_heads, head_dim)), dtype)
    k = _make(_normal(rng, (batch, 2 * L, n_kv_heads, head_dim)), dtype)
    v = _make(_normal(rng, (batch, 2 * L, n_kv_heads, head_dim)), dtype)
    return q, k, v


def sequence_qkv(seed: int, batch: int, T: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, dtype: str = "bf16"):
    """Q/K/V over one sequence of T positions (any T), entries N(0, 1)."""
    rng = np.random.default_rng([seed, 104729])
    q = _make(_normal(rng, (batch, T, n_q_heads, head_dim)), dtype)
    k = _make(_normal(rng, (batch, T, n_kv_heads, head_dim)), dtype)
    v = _make(_normal(rng, (batch, T, n_kv_heads, head_dim)), dtype)
    return q, k, v


@dataclass
class DecodeInputs:
    q: Tensor
    k_new: Tensor
    v_new: Tensor
    k_cache: Tensor          # [num_pages, Hkv, page, d]
    v_cache: Tensor          # [num_pages, Hkv, d, page]
    block_table: np.ndarray  # [S, max_pages] int32
    cache_len: np.ndarray    # [S] int32
    page_size: int
    max_pages: int
    num_pages: int


def decode_step_tensors(seed: int, step: int, S: int, B: int, n_q_heads: int,
                        n_kv_heads: int, head_dim: int, dtype: str = "bf16"):
    """Fresh q / k_new / v_new for one decode step, entries N(0, 1)."""
    rng = np.random.default_rng([seed, 7919, step])
    q = _make(_normal(rng, (S, B, n_q_heads, head_dim)), dtype)
    kn = _make(_normal(rng, (S, B, n_kv_heads, head_dim)), dtype)
    vn = _make(_normal(rng, (S, B, n_kv_heads, head_dim)), dtype)
    return q, kn, vn


def decode_inputs(seed: int, S: int, B: int, n_q_heads: int, n_kv_heads: int,
                  head_dim: int, len_lo: int, len_hi: int, page_size: int,
                  extra_capacity: int = 0, dtype: str = "bf16") -> DecodeInputs:
    """A paged KV cache with seeded prefix lengths ~ U{len_lo..len_hi} (inclusive).

    Every sequence owns ceil((len_hi + extra_capacity) / page_size) pages; the
    page ids are a seeded permutation, so logically adjacent pages are scattered
    in memory. All cache slots (used or not) hold N(0, 1) values.
    """
    rng = np.random.default_rng(seed)
    cache_len = rng.integers(len_lo, len_hi + 1, size=S).astype(np.int32)
    cap = len_hi + extra_capacity
    max_pages = max(1, -(-cap // page_size))
    num_pages = S * max_pages
    block_table = rng.permutation(num_pages).astype(np.int32).reshape(S, max_pages)
    k_cache = _make(_normal(rng, (num_pages, n_kv_heads, page_size, head_dim)), dtype)
    v_logical = _normal(rng, (num_pages, n_kv_heads, page_size, head_dim))
    v_cache = _make(np.ascontiguousarray(v_logical.transpose(0, 1, 3, 2)), dtype)
    del v_logical
    q, kn, vn = decode_step_tensors(seed, 0, S, B, n_q_heads, n_kv_heads, head_dim, dtype)
    return DecodeInputs(q, kn, vn, k_cache, v_cache, block_table, cache_len,
                        page_size, max_pages, num_pages)


@dataclass
class LayeredCommitInputs:
    k_new: Tensor        # [layers, S, B, n_kv_heads, head_dim]
    v_new: Tensor
    k_cache: Tensor      # [layers, num_pages, n_kv_heads, page_size, head_dim]
    v_cache: Tensor      # [layers, num_pages, n_kv_heads, head_dim, page_size]
    block_table: np.ndarray
    cache_len: np.ndarray
    page_size: int
    max_pages: int
    num_pages: int


def layered_commit_inputs(seed: int, layers: int, S: int, B: int, n_kv_heads: int,
                          head_dim: int, len_lo: int, len_hi: int, page_size: int,
                          extra_capacity: int = 0, dtype: str = "bf16") -> LayeredCommitInputs:
    """One paged KV cache per layer sharing one block table and one length per sequence.

    Lengths ~ U{len_lo..len_hi}; each sequence owns ceil((len_hi + extra_capacity)
    / page_size) pages whose ids are a seeded permutation; cache slots and the new
    rows of every layer hold N(0, 1) values.
    """
    rng = np.random.default_rng([seed, 104729])
    cache_len = rng.integers(len_lo, len_hi + 1, size=S).astype(np.int32)
    max_pages = max(1, -(-(len_hi + extra_capacity) // page_size))
    num_pages = S * max_pages
    block_table = rng.permutation(num_pages).astype(np.int32).reshape(S, max_pages)
    shape = (layers, num_pages, n_kv_heads, page_size, head_dim)
    k_cache = _make(_normal(rng, shape), dtype)
    v_cache = _make(np.ascontiguousarray(_normal(rng, shape).transpose(0, 1, 2, 4, 3)), dtype)
    rows = (layers, S, B, n_kv_heads, head_dim)
    k_new = _make(_normal(rng, rows), dtype)
    v_new = _make(_normal(rng, rows), dtype)
    return LayeredCommitInputs(k_new, v_new, k_cache, v_cache, block_table, cache_len,
                               page_size, max_pages, num_pages)


def lmhead_inputs(seed: int, N: int, D: int, V: int, w_std: float = 0.02):
    """hidden [N, D] ~ N(0, 1) and W [V, D] ~ N(0, w_std), both bfloat16."""
    rng = np.random.default_rng(seed)
    hidden = _make(_normal(rng, (N, D)), "bf16")
    w = _make(_normal(rng, (V, D), w_std), "bf16")
    return hidden, w


def normal_logits(seed: int, N: int, V: int, std: float) -> np.ndarray:
    """float32 logits [N, V] ~ N(0, std) (std is the standard deviation)."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (N, V), std)


class PeakedLogitsPool:
    """Logits with one planted peak per row whose max-probability is a chosen target.

    A fixed N(0, 1) noise pool [N, V] (float32) is drawn once. For each step a
    peak id is drawn uniformly per row, and a target probability
    p = U^(1/5) ~ Beta(5, 1). The peak logit is set to ln(p / (1 - p) * S_rest),
    where S_rest is the row's sum of exp over the other (noise) entries, so the
    softmax weight of the peak equals p up to the float32 rounding of the
    stored logit. Targets closer than `margin` to any threshold in `taus` are
    redrawn, which keeps realised probabilities far outside the 1e-6 guard.
    """

    def __init__(self, seed: int, N: int, V: int, taus=(0.9, 0.6), margin: float = 1e-4,
                 beta_a: float = 5.0):
        self.seed, self.N, self.V = seed, N, V
        self.taus = tuple(float(t) for t in taus)
        self.margin = margin
        self.beta_a = beta_a
        rng = np.random.default_rng([seed, 1])
        self.pool = _normal(rng, (N, V))
        self.row_expsum = np.empty(N, dtype=np.float64)
        for s in range(0, N, 64):
            self.row_expsum[s:s + 64] = np.exp(self.pool[s:s + 64].astype(np.float64)).sum(axis=1)

    def peaks(self, step: int):
        """(peak_ids int64 [N], peak_logits float32 [N], target_p float64 [N]) for a step."""
        rng = np.random.default_rng([self.seed, 2, step])
        ids = rng.integers(0, self.V, size=self.N)
        p = rng.random(self.N) ** (1.0 / self.beta_a)
        while True:
            bad = np.zeros(self.N, dtype=bool)
            for t in self.taus:
                bad |= np.abs(p - t) < self.margin
            bad |= p >= 1.0 - 1e-9
            if not bad.any():
                break
            p[bad] = rng.random(int(bad.sum())) ** (1.0 / self.beta_a)
        rest = self.row_expsum - np.exp(self.pool[np.arange(self.N), ids].astype(np.float64))
        peak = np.log(p / (1.0 - p) * rest).astype(np.float32)
        return ids, peak, p

    def logits(self, step: int) -> np.ndarray:
        """The full float32 logits [N, V] of a step (pool with the peaks planted)."""
        ids, peak, _ = self.peaks(step)
        out = self.pool.copy()
        out[np.arange(self.N), ids] = peak
        return out


def tau_schedule(S: int, step: int, switch_step: int = 32, before: float = 0.9,
                 after: float = 0.6) -> np.ndarray:
    """Per-sequence thresholds for a step: `before` until `switch_step`, then `after`."""
    return np.full(S, before if step < switch_step else after, dtype=np.float32)


def sample_pairs(seed: int, batch: int, n_heads: int, count: int):
    """`count` distinct (batch, head) pairs drawn from the seed."""
    rng = np.random.default_rng([seed, 3])
    flat = rng.choice(batch * n_heads, size=min(count, batch * n_heads), replace=False)
    return [(int(f // n_heads), int(f % n_heads)) for f in flat]
