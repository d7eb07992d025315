"""Pins for the fp64 oracle: each test checks it against something other than
itself (a different formulation, a library routine, a closed form or brute
force), so that a dropped term, a wrong sign, a wrong index or a mask
off-by-one in the oracle fails at least one of them."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

SM = W.SM_SCALE


def _bits(rng, shape, scale=1.0):
    return W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _run(w, tokens=None, **kw):
    return oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                            w.kv_indices, w.kv_last_page_len, w.page_size, w.causal,
                            w.sm_scale, tokens=tokens, **kw)


def _keys_by_walking_pages(w, row):
    """Gather a row's keys page by page, slot by slot (independent of the
    oracle's vectorised gather)."""
    cache = oracle.widen(w.kv_cache)
    lens = w.kv_lens()
    out = []
    s, e = int(w.kv_indptr[row]), int(w.kv_indptr[row + 1])
    for pi, p in enumerate(w.kv_indices[s:e]):
        n_slots = w.page_size if pi < e - s - 1 else int(w.kv_last_page_len[row])
        for slot in range(n_slots):
            out.append(cache[int(p), slot])
    assert len(out) == lens[row]
    return np.array(out).reshape(-1, W.LATENT_DIM)


# ---------------------------------------------------------------------------
# Brute-force, non-absorbed attention with random projection weights.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("page_size,kv_lens,qo_lens,causal", [
    (1, [7, 3], [1, 3], True),
    (4, [13, 1, 9], [5, 1, 2], True),
    (16, [40, 17], [1, 4], False),
    (16, [37, 100], [1, 5], True),
])
def test_absorbed_equals_non_absorbed(page_size, kv_lens, qo_lens, causal):
    """The layer computes attention with 128-wide nope heads (k_nope = W_UK ckv,
    v = W_UV ckv) plus 64-wide rope parts; absorbing W_UK into the query and
    applying W_UV after the latent output must give the same result."""
    rng = np.random.default_rng(7)
    H, d_nope, d_v = 3, 128, 128
    w = W.make_workload("bf", 7, kv_lens, qo_lens, H, page_size, causal=causal, rng=rng)
    T = w.num_tokens
    W_UK = rng.standard_normal((H, d_nope, W.KV_LORA_RANK)) / math.sqrt(W.KV_LORA_RANK)
    W_UV = rng.standard_normal((H, W.KV_LORA_RANK, d_v)) / math.sqrt(W.KV_LORA_RANK)
    q_orig = rng.standard_normal((T, H, d_nope))
    q_pe = oracle.widen(w.q_pe)
    # absorbed query: q_nope @ W_UK, kv_lora_rank wide (the oracle's
    # projections, pinned here by the non-absorbed brute force below)
    q_abs = oracle.absorb_query(q_orig, W_UK)
    o_lat, lse = oracle.attention(q_abs, q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                                  w.kv_indices, w.kv_last_page_len, page_size, causal, SM)
    o_abs = oracle.up_project(o_lat, W_UV)

    sm = float(np.float32(SM))
    for b in range(w.batch):
        keys = _keys_by_walking_pages(w, b)
        L, Q = keys.shape[0], int(qo_lens[b])
        ckv, kpe = keys[:, :512], keys[:, 512:]
        for i in range(Q):
            t = int(w.qo_indptr[b]) + i
            pos = L - Q + i  # position of the query among the keys
            for h in range(H):
                k_nope = ckv @ W_UK[h].T      # [L, 128]
                v = ckv @ W_UV[h]             # [L, 128]
                s = sm * (k_nope @ q_orig[t, h] + kpe @ q_pe[t, h])
                vis = np.array([(not causal) or j <= pos for j in range(L)])
                if not vis.any():
                    assert np.all(o_abs[t, h] == 0) and lse[t, h] == -np.inf
                    continue
                sv = s[vis]
                p = np.exp(sv - sv.max())
                ref = (p / p.sum()) @ v[vis]
                np.testing.assert_allclose(o_abs[t, h], ref, rtol=1e-10, atol=1e-12)
                assert abs(lse[t, h] - (sv.max() + math.log(p.sum()))) < 1e-10


# ---------------------------------------------------------------------------
# Library routine: PyTorch fp64 scaled_dot_product_attention with an explicit
# bottom-right causal mask (its is_causal flag is top-left aligned).
# ---------------------------------------------------------------------------

def test_matches_torch_sdpa_bottom_right_mask():
    rng = np.random.default_rng(11)
    w = W.make_workload("sdpa", 11, [50, 9, 33], [6, 9, 1], 4, 8, causal=True, rng=rng)
    o, lse = _run(w)
    sm = float(np.float32(SM))
    for b in range(w.batch):
        keys = torch.from_numpy(_keys_by_walking_pages(w, b))
        L = keys.shape[0]
        q0, q1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        Q = q1 - q0
        q = torch.from_numpy(np.concatenate([oracle.widen(w.q_nope[q0:q1]),
                                             oracle.widen(w.q_pe[q0:q1])], -1))  # [Q,H,576]
        q = q.permute(1, 0, 2).contiguous()  # [H,Q,576]
        k = keys.unsqueeze(0).expand(q.shape[0], L, 576).contiguous()
        v = keys[:, :512].unsqueeze(0).expand(q.shape[0], L, 512).contiguous()
        mask = torch.ones(Q, L, dtype=torch.bool).tril(diagonal=L - Q)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=sm)
        scores = torch.einsum("hqd,hkd->hqk", q, k) * sm
        ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
        np.testing.assert_allclose(o[q0:q1], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[q0:q1], ref_lse.T.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Invariants and closed forms.
# ---------------------------------------------------------------------------

def test_page_permutation_invariance():
    """Relabelling the pages (and moving their contents) changes nothing,
    bit for bit: the oracle's summation order depends only on key order."""
    w = W.tiny()
    o1, l1 = _run(w)
    rng = np.random.default_rng(3)
    sigma = rng.permutation(w.num_pages)
    cache2 = np.empty_like(w.kv_cache)
    cache2[sigma] = w.kv_cache
    o2, l2 = oracle.attention(w.q_nope, w.q_pe, cache2, w.qo_indptr, w.kv_indptr,
                              sigma[w.kv_indices].astype(np.int32), w.kv_last_page_len,
                              w.page_size, w.causal, w.sm_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_single_key_returns_that_row():
    rng = np.random.default_rng(5)
    w = W.make_workload("one", 5, [1, 1], [1, 1], 8, 16, rng=rng)
    o, lse = _run(w)
    sm = float(np.float32(SM))
    for b in range(2):
        key = oracle.widen(w.kv_cache[w.kv_indices[b], 0])
        assert np.array_equal(o[b], np.broadcast_to(key[:512], o[b].shape))
        s = sm * (oracle.widen(w.q_nope[b]) @ key[:512] + oracle.widen(w.q_pe[b]) @ key[512:])
        np.testing.assert_allclose(lse[b], s, rtol=0, atol=1e-12)


def test_zero_query_gives_mean_and_log_count():
    """q = 0: every visible score is 0, so o is the mean of the visible ckv
    rows and lse = ln(#visible)."""
    rng = np.random.default_rng(9)
    w = W.make_workload("zq", 9, [23, 64], [4, 2], 2, 4, rng=rng)
    w.q_nope[:] = 0
    w.q_pe[:] = 0
    o, lse = _run(w)
    for b in range(w.batch):
        keys = _keys_by_walking_pages(w, b)
        L, Q = keys.shape[0], int(w.qo_lens()[b])
        for i in range(Q):
            t = int(w.qo_indptr[b]) + i
            n = L - Q + i + 1
            np.testing.assert_allclose(o[t], np.broadcast_to(keys[:n, :512].mean(0), o[t].shape),
                                       rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(lse[t], math.log(n), rtol=1e-14)


def test_identical_keys():
    """n identical keys: o is that key's ckv and lse = s + ln n."""
    rng = np.random.default_rng(13)
    w = W.make_workload("same", 13, [19], [1], 4, 8, rng=rng)
    key = w.kv_cache[w.kv_indices[0], 0].copy()
    w.kv_cache[w.kv_indices, :, :] = key
    o, lse = _run(w)
    k = oracle.widen(key)
    s = float(np.float32(SM)) * (oracle.widen(w.q_nope[0]) @ k[:512] + oracle.widen(w.q_pe[0]) @ k[512:])
    np.testing.assert_allclose(o[0], np.broadcast_to(k[:512], o[0].shape), rtol=1e-13)
    np.testing.assert_allclose(lse[0], s + math.log(19), rtol=1e-13)


def test_two_segment_merge_identity():
    """Attention over keys A ++ B equals the LSE merge of attention over A
    (fully visible prefix) and over B (causal, |B| >= Q)."""
    rng = np.random.default_rng(17)
    H, P = 4, 4
    lenA, lenB, Q = [12, 30, 5], [9, 6, 3], [4, 6, 1]
    w_full = W.make_workload("ab", 17, np.add(lenA, lenB), Q, H, P, causal=True, rng=rng)
    # Split each row's keys into the first lenA (segment A) and the rest (B).
    keysA, keysB = [], []
    for b in range(3):
        k = _keys_by_walking_pages(w_full, b)
        keysA.append(k[:lenA[b]])
        keysB.append(k[lenA[b]:])

    def as_cache(keys_list):
        cache, indptr, idx, last = [], [0], [], []
        for k in keys_list:
            n = (k.shape[0] + P - 1) // P
            for p in range(n):
                page = np.full((P, 576), 0x4100, dtype=np.uint16)
                chunk = W.f32_to_bf16_bits(k[p * P:(p + 1) * P].astype(np.float32))
                page[:chunk.shape[0]] = chunk
                idx.append(len(cache))
                cache.append(page)
            indptr.append(indptr[-1] + n)
            last.append(k.shape[0] - (n - 1) * P if n else 0)
        return (np.array(cache), np.array(indptr, np.int32), np.array(idx, np.int32),
                np.array(last, np.int32))

    cA, ipA, ixA, lA = as_cache(keysA)
    cB, ipB, ixB, lB = as_cache(keysB)
    o_all, s_all = _run(w_full)
    oA, sA = oracle.attention(w_full.q_nope, w_full.q_pe, cA, w_full.qo_indptr, ipA, ixA, lA, P,
                              False, SM)
    oB, sB = oracle.attention(w_full.q_nope, w_full.q_pe, cB, w_full.qo_indptr, ipB, ixB, lB, P,
                              True, SM)
    om, sm_ = oracle.merge_state(oA, sA, oB, sB)
    np.testing.assert_allclose(om, o_all, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sm_, s_all, rtol=1e-12, atol=1e-12)


def test_merge_state_closed_forms():
    """Equal LSEs average the values (s grows by ln 2); an empty side is the
    identity; two empty sides give (0, -inf)."""
    rng = np.random.default_rng(19)
    va, vb = rng.standard_normal((3, 2, 8)), rng.standard_normal((3, 2, 8))
    s = rng.standard_normal((3, 2))
    v, sout = oracle.merge_state(va, s, vb, s)
    np.testing.assert_allclose(v, (va + vb) / 2, rtol=1e-14)
    np.testing.assert_allclose(sout, s + math.log(2), rtol=1e-14)
    ninf = np.full((3, 2), -np.inf)
    v, sout = oracle.merge_state(va, s, vb, ninf)
    np.testing.assert_array_equal(v, va)
    np.testing.assert_array_equal(sout, s)
    v, sout = oracle.merge_state(va, ninf, vb, ninf)
    assert np.all(v == 0) and np.all(np.isneginf(sout))
    # weights e^{s_a} : e^{s_b}
    sa, sb = np.zeros((3, 2)), np.full((3, 2), math.log(3.0))
    v, sout = oracle.merge_state(va, sa, vb, sb)
    np.testing.assert_allclose(v, 0.25 * va + 0.75 * vb, rtol=1e-14)
    np.testing.assert_allclose(sout, math.log(4.0), rtol=1e-14)


def test_empty_rows_and_queries_without_keys():
    """A row with no keys, and causal queries that precede every key
    (Q > L), give o = 0 and lse = -inf."""
    rng = np.random.default_rng(23)
    w = W.make_workload("empty", 23, [0, 2, 5], [2, 4, 0], 2, 4, rng=rng)
    o, lse = _run(w)
    assert np.all(o[0:2] == 0) and np.all(np.isneginf(lse[0:2]))
    # row 1: L=2, Q=4 -> queries 0 and 1 see nothing, 2 sees 1 key, 3 sees 2
    assert np.all(o[2:4] == 0) and np.all(np.isneginf(lse[2:4]))
    assert np.all(np.isfinite(lse[4:6]))
    k0 = oracle.widen(w.kv_cache[w.kv_indices[w.kv_indptr[1]], 0])
    assert np.array_equal(o[4], np.broadcast_to(k0[:512], o[4].shape))


@pytest.mark.parametrize("visible", [True, False])
def test_needle_key(visible):
    """A key whose score dwarfs the rest dominates the output when visible and
    changes nothing (bit for bit) when the causal mask hides it."""
    rng = np.random.default_rng(29)
    L, Q, H = 40, 5, 2
    w = W.make_workload("needle", 29, [L], [Q], H, 8, rng=rng)
    o0, l0 = _run(w)
    i = 2                      # query index; it sees keys 0 .. L - Q + i
    last_vis = L - Q + i
    j = last_vis if visible else last_vis + 1
    q = oracle.widen(w.q_nope[i])  # [H, 512]
    needle = np.where(q[0] >= 0, 4.0, -4.0)  # large score for head 0
    page, slot = w.kv_indices[j // 8], j % 8
    w.kv_cache[page, slot, :512] = W.f32_to_bf16_bits(needle.astype(np.float32))
    o1, l1 = _run(w)
    if visible:
        np.testing.assert_allclose(o1[i, 0], needle, rtol=1e-6, atol=1e-6)
        assert l1[i, 0] > l0[i, 0] + 50
    else:
        assert np.array_equal(o1[i], o0[i]) and np.array_equal(l1[i], l0[i])
    # queries before i never see key j either way when j > their last visible key
    assert np.array_equal(o1[0], o0[0]) or j <= L - Q


def test_vectorised_equals_loops_tiny():
    """The vectorised oracle against a pure-loop transcription on the tiny
    workload's shapes (fewer heads to keep the loops quick)."""
    rng = np.random.default_rng(31)
    w = W.make_workload("loops", 31, [37, 100, 0], [1, 5, 2], 2, 16, pool_pages=16, rng=rng)
    o1, l1 = _run(w)
    o2, l2 = oracle.attention_loops(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                                    w.kv_indices, w.kv_last_page_len, w.page_size, w.causal,
                                    w.sm_scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=0)


def test_token_subset_matches_full():
    w = W.tiny()
    o, l = _run(w)
    sel = np.array([5, 0, 3])
    o2, l2 = _run(w, tokens=sel)
    assert np.array_equal(o2, o[sel]) and np.array_equal(l2, l[sel])


def test_poisoned_slots_are_never_read():
    """Changing every slot no row owns leaves the result bit-identical."""
    w = W.tiny()
    o1, l1 = _run(w)
    owned = np.zeros(w.kv_cache.shape[:2], dtype=bool)
    lens = w.kv_lens()
    for b in range(w.batch):
        for j in range(int(lens[b])):
            owned[w.kv_indices[w.kv_indptr[b] + j // 16], j % 16] = True
    w.kv_cache[~owned] = 0x7F00  # a huge finite bf16 value
    o2, l2 = _run(w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("bad", ["qo0", "kvdec", "last0", "lastbig", "page", "short"])
def test_validate_rejects(bad):
    qo = np.array([0, 1, 3], np.int32)
    kv = np.array([0, 2, 3], np.int32)
    idx = np.array([0, 1, 2], np.int32)
    last = np.array([3, 4], np.int32)
    if bad == "qo0":
        qo = np.array([1, 1, 3], np.int32)
    elif bad == "kvdec":
        kv = np.array([0, 3, 2], np.int32)
    elif bad == "last0":
        last = np.array([0, 4], np.int32)
    elif bad == "lastbig":
        last = np.array([5, 4], np.int32)
    elif bad == "page":
        idx = np.array([0, 9, 2], np.int32)
    elif bad == "short":
        idx = np.array([0, 1], np.int32)
    with pytest.raises(ValueError):
        oracle.validate(qo, kv, idx, last, 4, 4)
    oracle.validate(np.array([0, 1, 3], np.int32), np.array([0, 2, 3], np.int32),
                    np.array([0, 1, 2], np.int32), np.array([3, 4], np.int32), 4, 4)


def test_bf16_widening_is_exact():
    """bf16 -> fp64 widening against torch's own bf16 -> fp64 conversion,
    over every finite bf16 bit pattern."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    ours = oracle.widen(bits)
    fin = np.isfinite(t)
    assert np.array_equal(ours[fin], t[fin])


def test_generator_rounding_matches_torch():
    rng = np.random.default_rng(37)
    x = rng.standard_normal(100000).astype(np.float32) * 10
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generators_are_deterministic():
    a, b = W.tiny(), W.tiny()
    for f in ("q_nope", "q_pe", "kv_cache", "kv_indices", "kv_indptr", "kv_last_page_len"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    # the tiny layout: 16-page pool, row 0 three pages (last 5), row 1 seven (last 4)
    assert a.num_pages == 16
    assert list(a.kv_indptr) == [0, 3, 10] and list(a.kv_last_page_len) == [5, 4]
    assert list(a.kv_lens()) == [37, 100] and list(a.qo_indptr) == [0, 1, 6]


def test_golden_tiny_fixture():
    """The oracle still reproduces the stored tiny-workload values."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    doc = json.load(open(path))
    o, lse = _run(W.tiny())
    np.testing.assert_allclose(lse, np.array(doc["lse"]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[:, :, doc["cols"]], np.array(doc["o_cols"]), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# The projections on their own: closed forms and loops.
# ---------------------------------------------------------------------------

def test_projection_closed_forms_and_loops():
    rng = np.random.default_rng(3)
    T, H = 5, 3
    q = W.f32_to_bf16_bits(rng.standard_normal((T, H, 128), dtype=np.float32))
    # W_UK[h] = [I_128 | 0] (head 0), a column permutation (head 1), 2 I (head 2)
    w = np.zeros((H, 128, 512))
    w[0, :, :128] = np.eye(128)
    perm = rng.permutation(512)[:128]
    w[1, np.arange(128), perm] = 1.0
    w[2, :, 256:384] = 2.0 * np.eye(128)
    out = oracle.absorb_query(q, w)
    qf = oracle.widen(q)
    assert np.array_equal(out[:, 0, :128], qf[:, 0]) and not out[:, 0, 128:].any()
    assert np.array_equal(out[:, 1, perm], qf[:, 1])
    assert np.array_equal(out[:, 2, 256:384], 2.0 * qf[:, 2])
    # up-projection by explicit loops
    o = rng.standard_normal((2, 2, 512))
    wv = rng.standard_normal((2, 512, 128))
    ref = np.zeros((2, 2, 128))
    for t in range(2):
        for h in range(2):
            for n in range(128):
                ref[t, h, n] = sum(o[t, h, k] * wv[h, k, n] for k in range(512))
    np.testing.assert_allclose(oracle.up_project(o, wv), ref, rtol=1e-12, atol=1e-12)
