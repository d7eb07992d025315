"""mla_run captured in a HIP graph and replayed: every replay, with eager
work and synchronisations between the replays, matches the eager result bit
for bit.  Covers a schedule the kernels read from the pinned host slot
(decode-sized, released by the kernels' flags), one read from the device
copy (prefill-sized) and one with a shared pool of whole-token items."""

import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("shape,heads", [("decode", 128), ("prefill", 128), ("pool", 128),
                                         ("decode", 16), ("pool", 16)])
def test_graph_replays_match_eager(shape, heads):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    if shape == "decode":
        w = W.make_workload("g_decode", 0, [700, 33, 1500, 64], [1, 1, 1, 1], heads, 64,
                            rng=np.random.default_rng(41))
    elif shape == "pool":
        # enough query tokens (and small whole-token items) for the shared
        # pool, whose device counter every run must leave at zero
        workers = torch.cuda.get_device_properties(0).multi_processor_count * (2 if heads <= 32 else 1)
        q_len = (4 * workers + 7) // 8 + 3
        kv = q_len + np.array([0, 1200, 40, 1500, 10, 900, 0, 1300])
        w = W.make_workload("g_pool", 0, kv, [q_len] * 8, heads, 64, rng=np.random.default_rng(43))
    else:
        w = W.make_workload("g_prefill", 0, [1200, 300, 2100], [256, 300, 128], heads, 64,
                            rng=np.random.default_rng(42))
    T, H = w.num_tokens, w.num_heads
    qn, qp, kv = _dev(w.q_nope), _dev(w.q_pe), _dev(w.kv_cache)
    plan = pm.MLAPlan(H, w.page_size)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=True,
              sm_scale=w.sm_scale, num_cache_pages=w.num_pages)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    plan.run(qn, qp, kv, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    stats = plan.stats()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        plan.run(qn, qp, kv, out=out, lse=lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(qn, qp, kv, out=out, lse=lse)
    for k in range(4):
        out.fill_(0)
        lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {k}: output differs"
        assert torch.equal(lse, ref_l), f"replay {k}: lse differs"
        # eager work between replays
        plan.run(qn, qp, kv, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o)
    # A replay after the eager runs, then two fresh plans (each refills a
    # staging slot, waiting for the runs that read it) and the plan's
    # release: none of them may wait on the captured run.
    g.replay()
    torch.cuda.synchronize()
    last = w.kv_last_page_len.copy()
    for k in range(2):
        last[0] = w.kv_last_page_len[0] - 1 - k
        plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, last, causal=True,
                  sm_scale=w.sm_scale, num_cache_pages=w.num_pages)
        plan.run(qn, qp, kv, out=out, lse=lse)
    torch.cuda.synchronize()
    plan.close()
    assert stats["num_workers"] > 0


def test_reserved_plan_graph_survives_replans():
    """A plan with reserved capacity: mla_run captured once, then replayed
    after plans of three different batches (decode, prefill and mixed rows,
    different lengths and token counts), each replay matching the oracle for
    the batch planned last."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    import oracle
    from gpu_util import assert_close
    H, P = 64, 16
    batches = [
        W.make_workload("r1", 0, [300, 70, 1000], [1, 1, 1], H, P, rng=np.random.default_rng(1)),
        W.make_workload("r2", 0, [2000, 50], [16, 50], H, P, rng=np.random.default_rng(2)),
        W.make_workload("r3", 0, [40, 900, 123, 777], [5, 1, 1, 30], H, P,
                        rng=np.random.default_rng(3)),
    ]
    max_t, max_pages = 96, max(w.num_pages for w in batches)
    max_nnz = max(int(w.kv_indptr[-1]) for w in batches)
    q_pool = torch.zeros((max_t, H, 512), dtype=torch.bfloat16, device="cuda")
    qp_pool = torch.zeros((max_t, H, 64), dtype=torch.bfloat16, device="cuda")
    kv_pool = torch.zeros((max_pages, P, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((max_t, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((max_t, H), dtype=torch.float32, device="cuda")
    plan = pm.MLAPlan(H, P)
    plan.reserve(8, max_t, max_nnz)

    def load(w):
        T = w.num_tokens
        q_pool[:T].copy_(_dev(w.q_nope))
        qp_pool[:T].copy_(_dev(w.q_pe))
        kv_pool[:w.num_pages].copy_(_dev(w.kv_cache))
        plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=True,
                  sm_scale=w.sm_scale, num_cache_pages=max_pages)

    load(batches[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.run(q_pool, qp_pool, kv_pool, out=out, lse=lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(q_pool, qp_pool, kv_pool, out=out, lse=lse)
    torch.cuda.synchronize()
    for w in batches + [batches[0]]:
        load(w)
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        T = w.num_tokens
        o = out[:T].view(torch.int16).cpu().numpy().view(np.uint16)
        o_ref, l_ref = oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                                        w.kv_indices, w.kv_last_page_len, P, True, w.sm_scale)
        assert_close(o, lse[:T].cpu().numpy(), o_ref, l_ref, f"replay after planning {w.name}")
    with pytest.raises(Exception):  # beyond the reserved capacity
        big = W.make_workload("big", 0, [100] * 9, [1] * 9, H, P, rng=np.random.default_rng(4))
        plan.plan(big.qo_indptr, big.kv_indptr, big.kv_indices, big.kv_last_page_len,
                  num_cache_pages=big.num_pages)
    plan.close()


def test_reserved_plan_graph_with_shared_pool():
    """A captured run of a plan with reserved capacity, replayed after plans
    that alternate between a batch with a shared pool of whole-token items
    and one without: the pool's range comes from the device copy of the
    schedule and its counters are left at zero by every replay."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    import oracle
    from gpu_util import assert_close
    H, P = 64, 16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    q_len = (4 * cus + 7) // 8 + 3
    kv = q_len + np.array([0, 1200, 40, 1500, 10, 900, 0, 1300])
    pooled = W.make_workload("rp1", 0, kv, [q_len] * 8, H, P, rng=np.random.default_rng(11))
    plain = W.make_workload("rp2", 0, [700, 90, 1500], [1, 30, 2], H, P,
                            rng=np.random.default_rng(12))
    s = pm.schedule(pooled.qo_indptr, pooled.kv_indptr, pooled.kv_indices,
                    pooled.kv_last_page_len, P, pooled.num_pages, H, cus)
    assert s["worker_indptr"][cus + 1] > s["worker_indptr"][cus], "no shared pool"
    batches = [pooled, plain, pooled]
    max_t = max(w.num_tokens for w in batches)
    max_pages = max(w.num_pages for w in batches)
    max_nnz = max(int(w.kv_indptr[-1]) for w in batches)
    q_buf = torch.zeros((max_t, H, 512), dtype=torch.bfloat16, device="cuda")
    qp_buf = torch.zeros((max_t, H, 64), dtype=torch.bfloat16, device="cuda")
    kv_buf = torch.zeros((max_pages, P, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((max_t, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((max_t, H), dtype=torch.float32, device="cuda")
    plan = pm.MLAPlan(H, P)
    plan.reserve(8, max_t, max_nnz)

    def load(w):
        T = w.num_tokens
        q_buf[:T].copy_(_dev(w.q_nope))
        qp_buf[:T].copy_(_dev(w.q_pe))
        kv_buf[:w.num_pages].copy_(_dev(w.kv_cache))
        plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=True,
                  sm_scale=w.sm_scale, num_cache_pages=max_pages)

    load(plain)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        plan.run(q_buf, qp_buf, kv_buf, out=out, lse=lse, stream=st)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(q_buf, qp_buf, kv_buf, out=out, lse=lse)
    torch.cuda.synchronize()
    try:
        for w in batches:
            load(w)
            out.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            T = w.num_tokens
            o = out[:T].view(torch.int16).cpu().numpy().view(np.uint16)
            o_ref, l_ref = oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr,
                                            w.kv_indptr, w.kv_indices, w.kv_last_page_len, P,
                                            True, w.sm_scale)
            assert_close(o, lse[:T].cpu().numpy(), o_ref, l_ref, f"replay after planning {w.name}")
    finally:
        plan.close()
