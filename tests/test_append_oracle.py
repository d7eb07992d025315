"""Pins for the oracle's KV append (write this step's latent rows into the
paged cache before attention; page "mstar.engine.resources.attn.base",
AttentionManager.requires_kv_write).  Each test checks the oracle against
something other than its own formula: a page walk that counts slots, the
attention oracle reading the rows back, relabelled page tables, and the
cases it must reject."""

import numpy as np
import pytest

import oracle
import workloads as W


def _case(seed, page_size, rows, num_pages=None):
    """rows: list of (kv_len, q_len).  Pages are a seeded permutation of a
    pool with one spare page; the cache and the new rows are random bf16."""
    rng = np.random.default_rng(seed)
    n_pages = [0 if L == 0 else -(-L // page_size) for L, _ in rows]
    total = sum(n_pages)
    num_pages = num_pages or total + 1
    perm = rng.permutation(num_pages)
    kv_indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    kv_indices = perm[:total].astype(np.int32)
    last = np.array([0 if L == 0 else L - (n - 1) * page_size for (L, _), n in zip(rows, n_pages)],
                    dtype=np.int32)
    qo = np.concatenate([[0], np.cumsum([q for _, q in rows])]).astype(np.int32)
    T = int(qo[-1])
    cache = W.f32_to_bf16_bits(rng.standard_normal((num_pages, page_size, 576), dtype=np.float32))
    ckv = W.f32_to_bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    kpe = W.f32_to_bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
    return cache, ckv, kpe, qo, kv_indptr, kv_indices, last


def _walk(cache, ckv, kpe, qo, kv_indptr, kv_indices, last, page_size):
    """Brute force: list the row's (page, slot) pairs by walking its pages in
    order, slot by slot, and give the last Q of them to the row's tokens."""
    out = cache.copy()
    for b in range(len(qo) - 1):
        slots = []
        pages = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
        for k, p in enumerate(pages):
            fill = last[b] if k == len(pages) - 1 else page_size
            for s in range(fill):
                slots.append((int(p), s))
        q = int(qo[b + 1] - qo[b])
        for i, (p, s) in enumerate(slots[len(slots) - q:] if q else []):
            t = int(qo[b]) + i
            out[p, s, :512] = ckv[t]
            out[p, s, 512:] = kpe[t]
    return out


@pytest.mark.parametrize("page_size", [1, 3, 16, 64])
def test_append_matches_page_walk(page_size):
    rows = [(37, 1), (100, 5), (0, 0), (64, 64), (5, 2), (129, 0)]
    c = _case(7 + page_size, page_size, rows)
    got = oracle.append_kv(*c, page_size)
    want = _walk(*c, page_size)
    assert np.array_equal(got, want)
    # every slot the step does not own is untouched
    changed = np.any(got != c[0], axis=-1)
    assert changed.sum() <= sum(q for _, q in rows)


def test_append_then_attend_reads_the_new_rows():
    """A decode token whose own appended key is a needle (its score dwarfs
    the others) attends to that row; a one-key row returns it exactly."""
    P = 16
    rows = [(50, 1), (1, 1), (33, 3)]
    cache, ckv, kpe, qo, kvp, idx, last = _case(3, P, rows)
    H = 2
    rng = np.random.default_rng(11)
    q_nope = W.f32_to_bf16_bits(rng.standard_normal((5, H, 512), dtype=np.float32) * 0.01)
    q_pe = W.f32_to_bf16_bits(rng.standard_normal((5, H, 64), dtype=np.float32))
    # needle: token 0's new kpe aligned with its q_pe, large
    qp0 = oracle.widen(q_pe[0, 0])
    kpe[0] = W.f32_to_bf16_bits((np.sign(qp0) * 64.0).astype(np.float32))
    new = oracle.append_kv(cache, ckv, kpe, qo, kvp, idx, last, P)
    o, lse = oracle.attention(q_nope, q_pe, new, qo, kvp, idx, last, P, True, 192 ** -0.5)
    assert np.abs(o[0, 0] - oracle.widen(ckv[0])).max() < 1e-6
    assert np.array_equal(o[1], np.broadcast_to(oracle.widen(ckv[1]), (H, 512)))
    # before the append the needle is absent: the output differs
    o0, _ = oracle.attention(q_nope, q_pe, cache, qo, kvp, idx, last, P, True, 192 ** -0.5)
    assert np.abs(o0[0, 0] - oracle.widen(ckv[0])).max() > 1e-2


def test_append_is_invariant_under_page_relabelling():
    P = 4
    c = _case(5, P, [(9, 3), (14, 2)], num_pages=12)
    cache, ckv, kpe, qo, kvp, idx, last = c
    sigma = np.random.default_rng(1).permutation(cache.shape[0])
    moved = np.empty_like(cache)
    moved[sigma] = cache
    got = oracle.append_kv(moved, ckv, kpe, qo, kvp, sigma[idx].astype(np.int32), last, P)
    ref = oracle.append_kv(*c, P)
    assert np.array_equal(got[sigma], ref)


def test_append_rejects_more_tokens_than_keys():
    c = _case(2, 8, [(3, 4)])
    with pytest.raises(ValueError):
        oracle.append_kv(*c, 8)


def test_append_rejects_two_tokens_in_one_slot():
    cache, ckv, kpe, qo, kvp, idx, last = _case(4, 4, [(4, 1), (4, 1)])
    idx = np.array([idx[0], idx[0]], dtype=np.int32)  # both rows end in the same slot
    with pytest.raises(ValueError):
        oracle.append_kv(cache, ckv, kpe, qo, kvp, idx, last, 4)
