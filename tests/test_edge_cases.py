"""Edge cases through the C ABI against the fp64 oracle: rows longer than the
longest work item (split at the item cap as well as for balance), with tiles
inside pages and with per-key page ids, batches whose queries see no keys,
an empty batch, a single head, many short prefill items per worker, and
the shared pool of whole-token items."""

import numpy as np
import pytest

import workloads as W
from gpu_util import assert_close, oracle_of, run_library

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    pm.library()


@pytest.mark.parametrize("page_size", [64, 1])
def test_rows_longer_than_an_item(page_size):
    """100,000 keys (over 3,000 tiles; an item holds at most 1,024) in one
    decode row next to a short one, 16 heads."""
    rng = np.random.default_rng(71 + page_size)
    w = W.make_workload("long_rows", 0, [100_000, 40], [1, 1], 16, page_size, rng=rng)
    import paged_mla_attention_amd as pm
    s = pm.schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, page_size,
                    w.num_pages, 16, 256)
    lens = s["items"][:, 3] - s["items"][:, 2]
    assert lens.max() <= 1024 * 32 and len(s["merges"]) >= 1
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, f"100k keys P={page_size}")


def test_no_query_sees_a_key():
    """Every row is empty or has more causal queries than keys at the front:
    the outputs are zero and the LSEs -inf exactly where the oracle says."""
    rng = np.random.default_rng(5)
    w = W.make_workload("empty_rows", 0, [0, 0, 3], [2, 1, 6], 32, 16, rng=rng)
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert np.isneginf(l_ref).any()
    assert_close(o, lse, o_ref, l_ref, "empty rows")


@pytest.mark.parametrize("heads", [32, 64, 128])
def test_empty_item_after_a_full_one_on_one_worker(heads):
    """A query with no visible key right after a token with keys, on the same
    worker (checked on the host schedule): the empty item's finish must not
    disturb the previous item's output, for every wave count."""
    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(31 + heads)
    w = W.make_workload("empty_after", 0, [10, 0, 40, 0, 75, 0], [1, 1, 1, 1, 1, 1], heads, 16,
                        rng=rng)
    workers = torch.cuda.get_device_properties(0).multi_processor_count
    s = pm.schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, 16, w.num_pages,
                    heads, workers)
    wi, items = s["worker_indptr"], s["items"]
    pairs = [k for k in range(workers) for i in range(wi[k], wi[k + 1] - 1)
             if items[i, 3] > items[i, 2] and items[i + 1, 3] == items[i + 1, 2]]
    assert pairs, "no worker runs an empty item after one with keys"
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, f"empty after full H={heads}")


def test_empty_batch():
    import paged_mla_attention_amd as pm
    plan = pm.MLAPlan(16, 16)
    plan.plan([0], [0], [], [], num_cache_pages=1)
    kv = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((0, 16, 512), dtype=torch.bfloat16, device="cuda")
    qp = torch.zeros((0, 16, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = plan.run(q, qp, kv, return_lse=True)
    torch.cuda.synchronize()
    assert o.shape == (0, 16, 512) and lse.shape == (0, 16)
    plan.close()


def test_single_head():
    rng = np.random.default_rng(9)
    w = W.make_workload("one_head", 0, [130, 7, 64], [1, 4, 64], 1, 32, rng=rng)
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, "H=1")


def test_many_short_prefill_items_one_wave():
    """600 causal queries over short rows, 24 heads (one wave per
    workgroup): several items per worker, many of them a single tile."""
    rng = np.random.default_rng(13)
    kv = [40, 200, 33, 500, 96]
    qo = [40, 150, 10, 300, 100]
    w = W.make_workload("short_prefill", 0, kv, qo, 24, 16, rng=rng)
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, "short prefill H=24")


def test_reserved_plan_takes_a_long_causal_prefix():
    """A reserved plan sized for 516 tokens and a 64K-key row accepts a
    causal prefill of 512 tokens over that row (every token re-walks the
    prefix, in several items each) and matches the oracle on sampled tokens."""
    import paged_mla_attention_amd as pm
    from gpu_util import sample_tokens, split_tokens, to_dev_bf16
    rng = np.random.default_rng(77)
    w = W.make_workload("long_prefix", 0, [65536 + 512, 100], [512, 4], 16, 64, rng=rng)
    plan = pm.MLAPlan(16, 64)
    plan.reserve(2, w.num_tokens, int(w.kv_indptr[-1]))
    o, lse = run_library(w, plan=plan)
    plan.close()
    toks = np.union1d(sample_tokens(w, per_row=4), split_tokens(w)[:16])
    o_ref, l_ref = oracle_of(w, tokens=toks)
    assert_close(o[toks], lse[toks], o_ref, l_ref, "reserved long causal prefix")


@pytest.mark.parametrize("heads,page_size", [(64, 64), (128, 16), (32, 64)])
def test_shared_pool_every_token_and_counter_reset(heads, page_size):
    """A batch with enough query tokens for the shared pool (whole-token items
    that workgroups draw from a device counter once their own lists are done):
    every token checked against the oracle, over two runs of one plan with
    other queries, so a counter not left at zero by the first run would skip
    pool items in the second."""
    import paged_mla_attention_amd as pm
    from gpu_util import to_dev_bf16
    rng = np.random.default_rng(97 + heads)
    workers = torch.cuda.get_device_properties(0).multi_processor_count * (2 if heads <= 32 else 1)
    n_rows = 8
    q_len = (4 * workers + n_rows - 1) // n_rows + 3
    # rows whose first queries see few keys (small items), next to long ones
    kv = q_len + np.array([0, 1200, 40, 1500, 10, 900, 0, 1300])
    w = W.make_workload("pool", 0, kv, [q_len] * n_rows, heads, page_size, rng=rng)
    s = pm.schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, page_size,
                    w.num_pages, heads, workers)
    wi = s["worker_indptr"]
    assert wi[workers + 1] - wi[workers] > workers, "no shared pool for this batch"
    plan = pm.MLAPlan(heads, page_size)
    kv_dev = to_dev_bf16(w.kv_cache)
    try:
        for rep in range(2):
            if rep:
                w.q_nope = W.bf16_normals(rng, w.q_nope.shape)
                w.q_pe = W.bf16_normals(rng, w.q_pe.shape)
            o, lse = run_library(w, plan=plan, kv_cache=kv_dev)
            o_ref, l_ref = oracle_of(w)
            assert_close(o, lse, o_ref, l_ref, f"shared pool H={heads} P={page_size} run {rep}")
    finally:
        plan.close()


@pytest.mark.parametrize("heads,rows,keys", [(128, 8, 20000), (16, 8, 40000)])
def test_host_slot_first_items_beyond_staged_pages(heads, rows, keys):
    """A decode batch small enough for the pinned host slot whose first items
    span more pages than the slot stages per worker (page size 32, about 20
    pages each): those workgroups load the page list from the slot's copy of
    the page table instead.  Every token against the oracle."""
    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(61 + heads)
    w = W.make_workload("hs_pages", 0, [keys] * rows, [1] * rows, heads, 32, rng=rng)
    workers = torch.cuda.get_device_properties(0).multi_processor_count * (2 if heads <= 32 else 1)
    s = pm.schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, 32, w.num_pages,
                    heads, workers)
    it, wi = s["items"], s["worker_indptr"]
    assert len(it) <= 2 * workers and len(s["merges"]) <= 192  # (read from the host slot)
    pages = [(it[wi[k]][3] - 1) // 32 - it[wi[k]][2] // 32 + 1
             for k in range(workers) if wi[k + 1] > wi[k]]
    assert max(pages) > 16
    o, lse = run_library(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, f"host slot, first items beyond staged pages, H={heads}")
