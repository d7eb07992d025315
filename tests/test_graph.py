"""mla_run captured in a HIP graph and replayed: every replay, with eager
work and synchronisations between the replays, matches the eager result bit
for bit.  Covers a schedule the kernels read from the pinned host slot
(decode-sized, released by the kernels' flags) and one read from the
device copy (prefill-sized)."""

import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("shape", ["decode", "prefill"])
def test_graph_replays_match_eager(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    if shape == "decode":
        w = W.make_workload("g_decode", 0, [700, 33, 1500, 64], [1, 1, 1, 1], 128, 64,
                            rng=np.random.default_rng(41))
    else:
        w = W.make_workload("g_prefill", 0, [1200, 300, 2100], [256, 300, 128], 128, 64,
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
    plan.close()
    assert stats["num_workers"] > 0
