"""Seeded synthetic inputs for paged latent attention (MLA).

This module only *draws* inputs: lengths, page tables and bf16 normal
samples.  It holds none of the attention arithmetic, so both the fp64 CPU
oracle (``oracle/``) and the HIP library can be fed from it without sharing
any of the method's code.

Layout conventions (m-star "flashinfer_mla" page, FlashInferMLAWrapper.plan /
run):

* ``qo_indptr[B+1]``: query tokens of row b are ``qo_indptr[b]:qo_indptr[b+1]``.
* ``kv_indptr[B+1]`` / ``kv_indices[nnz]``: the pages of row b, in key order.
* ``kv_last_page_len[B]``: valid slots of the row's last page, so the row
  holds ``(n_pages - 1) * page_size + last`` keys.
* ``kv_cache[num_pages, page_size, 576]``: one ``[ckv(512) | kpe(64)]`` latent
  per token.
* ``q_nope[T, H, 512]`` (absorbed), ``q_pe[T, H, 64]``.

All floating point tensors are returned as raw bf16 bit patterns (uint16).
fp32 normal samples are rounded to bf16 with round-to-nearest-even.

Slots a row does not own (the tail of its last page, pages no row names) are
filled with a large finite "poison" value, so a kernel that reads them
produces a visibly wrong result.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64
LATENT_DIM = KV_LORA_RANK + QK_ROPE_HEAD_DIM
# Softmax scale of the original (pre-absorption) query/key head dim 128 + 64.
SM_SCALE = float(np.float32(192.0 ** -0.5))
POISON_BF16 = 0x4100  # bf16 bit pattern of +8.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the bits.

    Inputs must be finite (the generators only produce normal samples).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_normals(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) fp32 samples rounded to bf16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24  # bound the fp32 temporary
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


@dataclass
class Workload:
    """One batch of paged-MLA inputs (host numpy arrays)."""

    name: str
    seed: int
    num_heads: int
    page_size: int
    causal: bool
    sm_scale: float
    return_lse: bool
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    kv_last_page_len: np.ndarray
    q_nope: np.ndarray  # uint16 [T, H, 512]
    q_pe: np.ndarray    # uint16 [T, H, 64]
    kv_cache: np.ndarray  # uint16 [num_pages, page_size, 576]
    # A second key segment for the same queries (merged through the LSE).
    extra: Optional["Workload"] = None
    notes: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.qo_indptr.shape[0] - 1)

    @property
    def num_tokens(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def num_pages(self) -> int:
        return int(self.kv_cache.shape[0])

    def kv_lens(self) -> np.ndarray:
        n = np.diff(self.kv_indptr).astype(np.int64)
        last = self.kv_last_page_len.astype(np.int64)
        return np.where(n > 0, (n - 1) * self.page_size + last, 0)

    def qo_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr).astype(np.int64)


def _page_table(kv_lens, page_size, pool_pages, rng, pool_perm=None):
    """Assign pages to rows in row order from a shuffled pool."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    need = (kv_lens + page_size - 1) // page_size
    total = int(need.sum())
    if pool_pages is None:
        pool_pages = total
    if total > pool_pages:
        raise ValueError("page pool too small")
    perm = rng.permutation(pool_pages) if pool_perm is None else pool_perm
    kv_indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(need)
    kv_indices = perm[:total].astype(np.int32)
    last = np.where(need > 0, kv_lens - (need - 1) * page_size, 0).astype(np.int32)
    return kv_indptr, kv_indices, last, pool_pages


def _poison_unowned(kv_cache, kv_indptr, kv_indices, last, page_size):
    """Overwrite every slot no row owns with the poison value."""
    num_pages = kv_cache.shape[0]
    owned_pages = np.zeros(num_pages, dtype=bool)
    owned_pages[kv_indices] = True
    kv_cache[~owned_pages] = POISON_BF16
    B = len(last)
    for b in range(B):
        s, e = int(kv_indptr[b]), int(kv_indptr[b + 1])
        if e > s and last[b] < page_size:
            kv_cache[kv_indices[e - 1], int(last[b]):, :] = POISON_BF16


def make_workload(
    name: str,
    seed: int,
    kv_lens,
    qo_lens,
    num_heads: int,
    page_size: int,
    causal: bool = True,
    return_lse: bool = True,
    pool_pages: Optional[int] = None,
    rng: Optional[np.random.Generator] = None,
    sm_scale: float = SM_SCALE,
    q_nope: Optional[np.ndarray] = None,
    q_pe: Optional[np.ndarray] = None,
) -> Workload:
    """Build one workload.

    Draw order from ``rng`` (``default_rng(seed)`` unless given): page
    permutation, then q_nope, q_pe, kv_cache normals.  Pages are a shuffled
    pool (``pool_pages`` pages, default: exactly the pages the rows need)
    handed to the rows in row order.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    qo_lens = np.asarray(qo_lens, dtype=np.int64)
    if kv_lens.shape != qo_lens.shape:
        raise ValueError("kv_lens and qo_lens differ in length")
    kv_indptr, kv_indices, last, pool = _page_table(kv_lens, page_size, pool_pages, rng)
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    T = int(qo_indptr[-1])
    if q_nope is None:
        q_nope = bf16_normals(rng, (T, num_heads, KV_LORA_RANK))
    if q_pe is None:
        q_pe = bf16_normals(rng, (T, num_heads, QK_ROPE_HEAD_DIM))
    kv_cache = bf16_normals(rng, (pool, page_size, LATENT_DIM))
    _poison_unowned(kv_cache, kv_indptr, kv_indices, last, page_size)
    return Workload(
        name=name, seed=seed, num_heads=num_heads, page_size=page_size,
        causal=causal, sm_scale=sm_scale, return_lse=return_lse,
        qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
        kv_last_page_len=last, q_nope=q_nope, q_pe=q_pe, kv_cache=kv_cache,
    )


# ---------------------------------------------------------------------------
# The five named workloads.  Seed = 1000 + workload number.  Integer ranges
# are inclusive.
# ---------------------------------------------------------------------------

def tiny(seed: int = 1001) -> Workload:
    """2 rows, H=16, page_size 16, kv lens 37 (decode) and 100 (causal
    prefill of 5 queries), pages from a seeded permutation of a 16-page pool:
    row 0 takes the first 3 ids, row 1 the next 7; 6 pool pages stay unused
    (and poisoned)."""
    rng = np.random.default_rng(seed)
    w = make_workload("tiny", seed, [37, 100], [1, 5], 16, 16, causal=True,
                      pool_pages=16, rng=rng)
    return w


def decode_batch(seed: int = 1002, batch: int = 64, num_heads: int = 128) -> Workload:
    """64 decode rows, H=128, page_size 64, kv lens uniform in [512, 4096]."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(512, 4096, size=batch, endpoint=True)
    return make_workload("decode_b64_h128", seed, kv, np.ones(batch, np.int64),
                         num_heads, 64, causal=True, rng=rng)


def long_decode(seed: int = 1003) -> Workload:
    """16 decode rows, H=16, kv len 32768 each, page_size 64, random pages."""
    rng = np.random.default_rng(seed)
    kv = np.full(16, 32768, dtype=np.int64)
    return make_workload("long_decode_b16_h16_32k", seed, kv, np.ones(16, np.int64),
                         16, 64, causal=True, rng=rng)


def chunked_prefill(seed: int = 1004) -> Workload:
    """8 rows of 512 queries each; cached prefix uniform in [0, 8192]; each
    row's keys are its prefix plus its own 512 tokens; causal; H=128;
    page_size 64."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, 8192, size=8, endpoint=True)
    return make_workload("chunked_prefill_b8_q512_h128", seed, prefix + 512,
                         np.full(8, 512, np.int64), 128, 64, causal=True, rng=rng)


def mixed(seed: int = 1005, with_extra: bool = True) -> Workload:
    """32 decode rows (kv uniform in [1024, 16384]) followed by 4 causal
    prefill rows of 1024 queries (prefix uniform in [0, 4096]), one
    qo_indptr; H=128; page_size 1.  ``extra``: a second, non-causal segment of
    2048 fresh keys per row (its own page pool), for an LSE merge."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(1024, 16384, size=32, endpoint=True)
    pre = rng.integers(0, 4096, size=4, endpoint=True) + 1024
    kv = np.concatenate([dec, pre])
    qo = np.concatenate([np.ones(32, np.int64), np.full(4, 1024, np.int64)])
    w = make_workload("mixed_b36_p1_h128", seed, kv, qo, 128, 1, causal=True, rng=rng)
    if with_extra:
        w.extra = make_workload("mixed_extra_segment", seed, np.full(36, 2048), qo, 128, 1,
                                causal=False, rng=rng, q_nope=w.q_nope, q_pe=w.q_pe)
    return w


WORKLOADS = {
    "tiny": tiny,
    "decode": decode_batch,
    "long_decode": long_decode,
    "prefill": chunked_prefill,
    "mixed": mixed,
}


def fp8_cache_codes(kv_cache_bits: np.ndarray, kv_scale: float) -> np.ndarray:
    """An fp8 (E4M3) latent cache standing for a bf16 one: the bf16 values
    divided by kv_scale, clamped to +-448 and converted by PyTorch's
    float8_e4m3fn rounding; returns the codes (uint8), same shape."""
    import torch
    f = (np.ascontiguousarray(kv_cache_bits).astype(np.uint32) << np.uint32(16)).view(np.float32)
    t = torch.from_numpy(f / np.float32(kv_scale)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
