"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Small cases compare every output; the full-size workloads compare every
output where the oracle is quick (decode, long decode) and sampled tokens
elsewhere (first, last and random queries of every row)."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (assert_close, from_dev_bf16, oracle_of, run_library, sample_tokens,
                      split_tokens, to_dev_bf16)

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    pm.library()  # raises if the HIP library is not built


def test_tiny_workload():
    w = W.tiny()
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, "tiny")


def test_tiny_golden_fixture():
    """The stored oracle values for the tiny workload (tests/golden)."""
    import json
    import os
    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")))
    o, lse = run_library(W.tiny())
    ow = oracle.widen(o)[:, :, doc["cols"]]
    ref = np.array(doc["o_cols"])
    assert np.all(np.abs(ow - ref) <= 1e-2 + 1e-2 * np.abs(ref))
    assert np.abs(lse - np.array(doc["lse"])).max() <= 2e-3


@pytest.mark.parametrize("heads", [1, 16, 24, 32, 40, 64, 100, 128])
@pytest.mark.parametrize("page_size", [1, 16, 33, 64])
def test_ragged_small(heads, page_size):
    """Ragged rows spanning several 32-key tiles with ragged tails, a row
    without keys, a row with more queries than keys, decode and prefill rows."""
    rng = np.random.default_rng(100 + heads + page_size)
    kv = [1, 95, 0, 300, 64, 7]
    qo = [1, 3, 2, 40, 1, 9]
    w = W.make_workload("ragged", 0, kv, qo, heads, page_size, causal=True, rng=rng)
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, f"ragged H={heads} P={page_size}")


@pytest.mark.parametrize("causal", [False, True])
def test_non_causal_and_causal(causal):
    rng = np.random.default_rng(7)
    w = W.make_workload("nc", 0, [130, 33, 500], [17, 33, 2], 128, 16, causal=causal, rng=rng)
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, f"causal={causal}")


def test_without_lse():
    w = W.tiny()
    o, lse = run_library(w, return_lse=False)
    assert lse is None
    o_ref, _ = oracle_of(w)
    assert_close(o, None, o_ref, None, "no lse")


def test_single_key_is_exact():
    """One visible key: the output is that key's ckv row, bit for bit."""
    rng = np.random.default_rng(9)
    w = W.make_workload("one", 0, [1, 1, 1], [1, 1, 1], 128, 64, rng=rng)
    o, lse = run_library(w)
    for b in range(3):
        key = w.kv_cache[w.kv_indices[b], 0, :512]
        assert np.array_equal(o[b], np.broadcast_to(key, o[b].shape))
    _, l_ref = oracle_of(w)
    assert np.abs(lse - l_ref).max() <= 2e-3


def test_page_permutation_bitwise():
    """Relabelling pages (and moving their data) leaves the output bitwise
    unchanged: the schedule depends only on lengths."""
    rng = np.random.default_rng(11)
    w = W.make_workload("perm", 0, [700, 33, 1500], [1, 5, 64], 64, 16, rng=rng)
    o1, l1 = run_library(w)
    sigma = np.random.default_rng(12).permutation(w.num_pages)
    cache2 = np.empty_like(w.kv_cache)
    cache2[sigma] = w.kv_cache
    w.kv_cache = cache2
    w.kv_indices = sigma[w.kv_indices].astype(np.int32)
    o2, l2 = run_library(w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("visible", [True, False])
def test_needle_causal_boundary(visible):
    """A key with a dominant score right at (or just past) a query's causal
    limit: it must dominate that query's output when visible and have no
    effect when masked."""
    rng = np.random.default_rng(13)
    L, Q, H = 200, 40, 32
    w = W.make_workload("needle", 0, [L], [Q], H, 16, rng=rng)
    i = 17
    j = L - Q + i + (0 if visible else 1)
    q = oracle.widen(w.q_nope[i])
    needle = np.where(q[0] >= 0, 4.0, -4.0).astype(np.float32)
    w.kv_cache[w.kv_indices[j // 16], j % 16, :512] = W.f32_to_bf16_bits(needle)
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, f"needle visible={visible}")
    ow = oracle.widen(o[i, 0])
    if visible:
        assert np.abs(ow - needle).max() < 0.05
    else:
        assert np.abs(ow - needle).max() > 1.0


def _redo_items(w, sched, c_of_key, qscale):
    """Work items whose first tile's largest base-2 score sits more than 64
    below a later score of the item (the kernel redoes such items with a new
    reference maximum).  Scores here are qscale[h] * 512 * c_j * sm_scale."""
    lens = w.kv_lens()
    n = 0
    for it in sched["items"]:
        kb, ke = int(it[2]), int(it[3])
        if ke <= kb:
            continue
        c = c_of_key[int(it[1])][kb:ke]
        s2 = 512 * float(np.float32(w.sm_scale)) / np.log(2.0) * qscale.max()
        if (c.max() - c[:32].max()) * s2 > 64:
            n += 1
    return n


@pytest.mark.parametrize("heads", [5, 16, 32, 64, 128])
@pytest.mark.parametrize("page_size", [32, 33])
def test_extreme_score_range_redo(heads, page_size):
    """Scores that jump by far more than 2^64 after a work item's first tile
    (the kernel's reference-maximum redo path) still match the oracle, in
    every kernel instantiation (the two-wave kernel of 16 head slots, one,
    two and four waves; tiles inside pages and tiles spanning pages), for a
    decode row and a causal prefill row.
    The schedule is checked on the host to contain items that take the redo."""
    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(17 + heads + page_size)
    kv, qo = [256, 300], [1, 24]
    w = W.make_workload("extreme", 0, kv, qo, heads, page_size, causal=True, rng=rng)
    qscale = 1.0 + np.arange(heads) / heads  # heads differ
    q = np.broadcast_to(qscale[None, :, None], (w.num_tokens, heads, 512)).astype(np.float32)
    w.q_nope[:] = W.f32_to_bf16_bits(q)
    w.q_pe[:] = 0
    c_of_key = []
    for b, L in enumerate(kv):
        c = np.where(np.arange(L) < 32, 0.01, np.where(np.arange(L) < 40, 0.5, 3.0))
        c_of_key.append(c)
        for j in range(L):
            pg = w.kv_indices[w.kv_indptr[b] + j // page_size]
            w.kv_cache[pg, j % page_size, :512] = W.f32_to_bf16_bits(
                np.full(512, c[j], np.float32))
    plan = pm.MLAPlan(heads, page_size)
    o, lse = run_library(w, plan=plan)
    sched = pm.schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, page_size,
                        w.num_pages, heads, plan.stats()["num_workers"], causal=True)
    plan.close()
    assert _redo_items(w, sched, c_of_key, qscale) > 0, "no item reaches the redo branch"
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, f"extreme H={heads} P={page_size}")


def test_replan_reuses_buffers():
    """Plan a large batch, then a smaller one, then the large one again on
    the same handle; each run matches the oracle."""
    import paged_mla_attention_amd as pm
    plan = pm.MLAPlan(64, 16)
    big = W.make_workload("big", 0, [900, 40, 2000], [1, 40, 3], 64, 16,
                          rng=np.random.default_rng(21))
    small = W.make_workload("small", 0, [50], [2], 64, 16, rng=np.random.default_rng(22))
    for w in (big, small, big):
        o, lse = run_library(w, plan=plan)
        o_ref, l_ref = oracle_of(w)
        assert_close(o, lse, o_ref, l_ref, w.name)
    plan.close()


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

def test_decode_b64_h128_full():
    w = W.decode_batch()
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, "decode B=64 H=128")


def test_long_decode_full():
    w = W.long_decode()
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, "long decode")


def test_chunked_prefill_sampled():
    w = W.chunked_prefill()
    o, lse = run_library(w)
    toks = np.union1d(sample_tokens(w, per_row=5), split_tokens(w))
    o_ref, l_ref = oracle_of(w, tokens=toks)
    assert_close(o[toks], lse[toks], o_ref, l_ref, "chunked prefill")


def test_mixed_with_extra_segment_merge():
    """Main causal run, extra non-causal 2048-key segment, merge_state; the
    merged result must equal the oracle on (extra keys ++ main keys), causal."""
    import paged_mla_attention_amd as pm
    w = W.mixed()
    e = w.extra
    q = (to_dev_bf16(w.q_nope), to_dev_bf16(w.q_pe))
    plan = pm.MLAPlan(w.num_heads, w.page_size)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=True,
              sm_scale=w.sm_scale, num_cache_pages=w.num_pages)
    o_main, s_main = plan.run(q[0], q[1], to_dev_bf16(w.kv_cache), return_lse=True)
    plan.plan(e.qo_indptr, e.kv_indptr, e.kv_indices, e.kv_last_page_len, causal=False,
              sm_scale=e.sm_scale, num_cache_pages=e.num_pages)
    o_ext, s_ext = plan.run(q[0], q[1], to_dev_bf16(e.kv_cache), return_lse=True)
    o_m, s_m = pm.merge_state(o_main, s_main, o_ext, s_ext)
    torch.cuda.synchronize()
    plan.close()
    toks = np.union1d(sample_tokens(w, per_row=3), split_tokens(w))
    # main segment alone
    o_ref, l_ref = oracle_of(w, tokens=toks)
    assert_close(from_dev_bf16(o_main)[toks], s_main.cpu().numpy()[toks], o_ref, l_ref, "mixed main")
    # the merge against the oracle on the concatenated key sequence
    B = w.batch
    lens_m, lens_e = w.kv_lens(), e.kv_lens()
    cache = np.concatenate([e.kv_cache, w.kv_cache])  # page_size 1: one key per page
    indptr = np.zeros(B + 1, np.int32)
    idx = []
    for b in range(B):
        idx.extend(e.kv_indices[e.kv_indptr[b]:e.kv_indptr[b + 1]].tolist())
        idx.extend((w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]] + e.num_pages).tolist())
        indptr[b + 1] = len(idx)
    assert np.array_equal(np.diff(indptr), lens_m + lens_e)
    o_ref, l_ref = oracle.attention(w.q_nope, w.q_pe, cache, w.qo_indptr, indptr,
                                    np.array(idx, np.int32), np.ones(B, np.int32), 1, True,
                                    w.sm_scale, tokens=toks)
    assert_close(from_dev_bf16(o_m)[toks], s_m.cpu().numpy()[toks], o_ref, l_ref, "mixed merged")


# ---------------------------------------------------------------------------
# mla_merge_state
# ---------------------------------------------------------------------------

def _merge_inputs(T, H, seed):
    rng = np.random.default_rng(seed)
    va = W.bf16_normals(rng, (T, H, 512))
    vb = W.bf16_normals(rng, (T, H, 512))
    sa = (rng.standard_normal((T, H)) * 3).astype(np.float32)
    sb = (rng.standard_normal((T, H)) * 3).astype(np.float32)
    sa[0, :3] = -np.inf          # one side empty
    sb[1, :2] = -np.inf
    sa[2, 0] = sb[2, 0] = -np.inf  # both empty
    sa[3, 1] = sb[3, 1] = 5.0      # equal
    return va, sa, vb, sb


@pytest.mark.parametrize("T,H", [(4, 16), (37, 128), (1000, 8)])
def test_merge_state(T, H):
    import paged_mla_attention_amd as pm
    va, sa, vb, sb = _merge_inputs(T, H, T)
    v, s = pm.merge_state(to_dev_bf16(va), torch.from_numpy(sa).cuda(), to_dev_bf16(vb),
                          torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    v_ref, s_ref = oracle.merge_state(va, sa.astype(np.float64), vb, sb.astype(np.float64))
    assert_close(from_dev_bf16(v), s.cpu().numpy(), v_ref, s_ref, "merge_state")
    # both-empty entries are exactly zero
    assert np.all(oracle.widen(from_dev_bf16(v))[2, 0] == 0)


def test_merge_state_in_place():
    import paged_mla_attention_amd as pm
    va, sa, vb, sb = _merge_inputs(64, 32, 5)
    a_v, a_s = to_dev_bf16(va), torch.from_numpy(sa).cuda()
    pm.merge_state(a_v, a_s, to_dev_bf16(vb), torch.from_numpy(sb).cuda(), v_out=a_v, s_out=a_s)
    torch.cuda.synchronize()
    v_ref, s_ref = oracle.merge_state(va, sa.astype(np.float64), vb, sb.astype(np.float64))
    assert_close(from_dev_bf16(a_v), a_s.cpu().numpy(), v_ref, s_ref, "merge_state in place")


# ---------------------------------------------------------------------------
# Error paths through the C ABI (all decided on the host)
# ---------------------------------------------------------------------------

def test_error_paths():
    import ctypes

    import paged_mla_attention_amd as pm
    from paged_mla_attention_amd import _native
    lib = pm.library()
    h = ctypes.c_void_p()
    assert lib.mla_plan_create(ctypes.byref(h), 0, 16, 256, 64, 16) == 2  # unsupported rank
    assert lib.mla_plan_create(ctypes.byref(h), 0, 129, 512, 64, 16) == 2
    assert lib.mla_plan_create(ctypes.byref(h), 99, 16, 512, 64, 16) == 1
    assert lib.mla_plan_create(ctypes.byref(h), 0, 16, 512, 64, 16) == 0
    # run before plan
    assert lib.mla_run(h, 1, 1, 1, 1, None, None) == 3
    assert b"before" in lib.mla_last_error()
    with pytest.raises(_native.MLAError, match="kv_indices"):
        pm.mla_plan(h.value, [0, 1], [0, 1], [5], [1], True, 0.1, 4, 0)
    with pytest.raises(_native.MLAError, match="sm_scale"):
        pm.mla_plan(h.value, [0, 1], [0, 1], [0], [1], True, float("nan"), 4, 0)
    # a failed plan leaves the handle unplanned
    assert lib.mla_run(h, 1, 1, 1, 1, None, None) == 3
    lib.mla_plan_destroy(h)


def test_identical_replan_is_kept_and_a_change_is_not():
    """An identical re-plan keeps the schedule (same output, bit for bit); a
    table that differs in one entry is planned afresh (matches the oracle for
    the new table)."""
    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(31)
    w = W.make_workload("replan", 0, [300, 70, 1000], [1, 1, 1], 64, 16, rng=rng)
    plan = pm.MLAPlan(64, 16)
    o1, l1 = run_library(w, plan=plan)
    o2, l2 = run_library(w, plan=plan)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # shorten the second row by three keys (a different last_page_len)
    w.kv_last_page_len = w.kv_last_page_len.copy()
    w.kv_last_page_len[1] -= 3
    assert w.kv_last_page_len[1] >= 1
    o3, l3 = run_library(w, plan=plan)
    o_ref, l_ref = oracle_of(w)
    assert_close(o3, l3, o_ref, l_ref, "re-planned table")
    assert not np.array_equal(o3[1], o1[1])
    plan.close()
