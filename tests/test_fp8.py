"""fp8 (E4M3) latent cache on the GPU, through the C ABI (mla_run_fp8,
mla_append_kv_fp8), against the fp64 oracle: ragged batches over every
kernel variant (one, two and four waves; tiles inside pages and per-key
pages), the full decode and long-decode batches, the overflow-redo path,
a batch with a shared pool of whole-token items, HIP-graph replays, and the
quantising append bit for bit."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_close, from_dev_bf16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    pm.library()


def _dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run_fp8(w, codes, scale, plan=None):
    import paged_mla_attention_amd as pm
    own = plan is None
    if own:
        plan = pm.MLAPlan(w.num_heads, w.page_size)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=w.causal,
              sm_scale=w.sm_scale, num_cache_pages=w.num_pages, kv_dtype="fp8_e4m3")
    kv = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    o, lse = plan.run(_dev_bits(w.q_nope), _dev_bits(w.q_pe), kv, return_lse=True, kv_scale=scale)
    torch.cuda.synchronize()
    if own:
        plan.close()
    return from_dev_bf16(o), lse.cpu().numpy()


def _oracle_fp8(w, codes, scale, tokens=None):
    return oracle.attention_fp8(w.q_nope, w.q_pe, codes, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                w.kv_last_page_len, w.page_size, w.causal, w.sm_scale, scale,
                                tokens=tokens)


@pytest.mark.parametrize("heads", [1, 16, 24, 32, 40, 64, 100, 128])
@pytest.mark.parametrize("page_size", [1, 16, 33, 64])
def test_fp8_ragged_small(heads, page_size):
    rng = np.random.default_rng(300 + heads + page_size)
    w = W.make_workload("fp8_ragged", 0, [1, 95, 0, 300, 64, 7], [1, 3, 2, 40, 1, 9], heads,
                        page_size, rng=rng)
    scale = 0.37 if heads % 32 == 0 else 1 / 16
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    o, lse = _run_fp8(w, codes, scale)
    o_ref, l_ref = _oracle_fp8(w, codes, scale)
    assert_close(o, lse, o_ref, l_ref, f"fp8 ragged H={heads} P={page_size}")


def test_fp8_decode_b64_h128_full():
    w = W.decode_batch()
    scale = 1 / 32
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    o, lse = _run_fp8(w, codes, scale)
    o_ref, l_ref = _oracle_fp8(w, codes, scale)
    assert_close(o, lse, o_ref, l_ref, "fp8 decode B=64 H=128")


def test_fp8_long_decode_full():
    w = W.long_decode()
    scale = 0.05
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    o, lse = _run_fp8(w, codes, scale)
    o_ref, l_ref = _oracle_fp8(w, codes, scale)
    assert_close(o, lse, o_ref, l_ref, "fp8 long decode")


@pytest.mark.parametrize("heads", [16, 32, 128])
@pytest.mark.parametrize("page_size", [32, 33])
def test_fp8_extreme_score_range_redo(heads, page_size):
    """Scores jumping by far more than 2^64 after an item's first tile (the
    redo path) over an fp8 cache."""
    rng = np.random.default_rng(41 + heads + page_size)
    kv, qo = [256, 300], [1, 24]
    w = W.make_workload("fp8_extreme", 0, kv, qo, heads, page_size, rng=rng)
    qscale = 1.0 + np.arange(heads) / heads
    w.q_nope[:] = W.f32_to_bf16_bits(np.broadcast_to(
        qscale[None, :, None], (w.num_tokens, heads, 512)).astype(np.float32))
    w.q_pe[:] = 0
    for b, L in enumerate(kv):
        c = np.where(np.arange(L) < 32, 0.01, np.where(np.arange(L) < 40, 0.5, 3.0))
        for j in range(L):
            pg = w.kv_indices[w.kv_indptr[b] + j // page_size]
            w.kv_cache[pg, j % page_size, :512] = W.f32_to_bf16_bits(np.full(512, c[j], np.float32))
    scale = 1 / 64
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    o, lse = _run_fp8(w, codes, scale)
    o_ref, l_ref = _oracle_fp8(w, codes, scale)
    assert_close(o, lse, o_ref, l_ref, f"fp8 extreme H={heads} P={page_size}")


@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_fp8_append_bit_exact(page_size):
    """The quantising append writes the oracle's codes, byte for byte, and
    leaves every other byte of the cache alone."""
    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(60 + page_size)
    w = W.make_workload("fp8_append", 0, [40, 3, 700, 129], [2, 3, 1, 64], 16, page_size, rng=rng)
    scale = 0.3
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    T = w.num_tokens
    ckv = W.bf16_normals(rng, (T, 512))
    kpe = W.bf16_normals(rng, (T, 64))
    ckv[0, :8] = W.f32_to_bf16_bits(np.array([1000, -1000, 1e-30, -1e-30, 0, 134.4, 67.2, -0.0],
                                             np.float32))
    plan = pm.MLAPlan(16, page_size)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len,
              num_cache_pages=w.num_pages, kv_dtype="fp8_e4m3")
    kv = torch.from_numpy(codes.copy()).cuda()
    plan.append_kv(_dev_bits(ckv), _dev_bits(kpe), kv, kv_scale=scale)
    torch.cuda.synchronize()
    plan.close()
    want = oracle.append_kv_fp8(codes, ckv, kpe, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                w.kv_last_page_len, page_size, scale)
    got = kv.cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).sum())} bytes differ"


def test_fp8_append_then_attend_decode():
    """Decode batch: append each row's new token into the fp8 cache, then
    attend; the result matches the oracle's append + attention."""
    import paged_mla_attention_amd as pm
    w = W.decode_batch()
    scale = 1 / 32
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    rng = np.random.default_rng(77)
    ckv, kpe = W.bf16_normals(rng, (64, 512)), W.bf16_normals(rng, (64, 64))
    plan = pm.MLAPlan(128, 64)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len,
              num_cache_pages=w.num_pages, kv_dtype="fp8_e4m3")
    kv = torch.from_numpy(codes.copy()).cuda()
    plan.append_kv(_dev_bits(ckv), _dev_bits(kpe), kv, kv_scale=scale)
    o, lse = plan.run(_dev_bits(w.q_nope), _dev_bits(w.q_pe), kv, return_lse=True,
                      kv_scale=scale)
    torch.cuda.synchronize()
    plan.close()
    want = oracle.append_kv_fp8(codes, ckv, kpe, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                w.kv_last_page_len, 64, scale)
    assert np.array_equal(kv.cpu().numpy(), want)
    o_ref, l_ref = _oracle_fp8(w, want, scale)
    assert_close(from_dev_bf16(o), lse.cpu().numpy(), o_ref, l_ref, "fp8 append + decode")


def test_fp8_rejects_bad_scale():
    import paged_mla_attention_amd as pm
    from paged_mla_attention_amd import _native
    w = W.tiny()
    codes = W.fp8_cache_codes(w.kv_cache, 1.0)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(_native.MLAError, match="kv_scale"):
            _run_fp8(w, codes, bad)


@pytest.mark.parametrize("heads,page_size", [(128, 64), (32, 16), (16, 64)])
def test_fp8_shared_pool_every_token(heads, page_size):
    """A batch with a shared pool of whole-token items over an fp8 cache:
    every token against the fp8 oracle, over two runs of one plan."""
    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(410 + heads)
    workers = torch.cuda.get_device_properties(0).multi_processor_count * (2 if heads <= 32 else 1)
    q_len = (4 * workers + 7) // 8 + 3
    kv = q_len + np.array([0, 1200, 40, 1500, 10, 900, 0, 1300])
    w = W.make_workload("fp8_pool", 0, kv, [q_len] * 8, heads, page_size, rng=rng)
    s = pm.schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, page_size,
                    w.num_pages, heads, workers)
    assert s["worker_indptr"][workers + 1] - s["worker_indptr"][workers] > workers
    scale = 0.21
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    plan = pm.MLAPlan(heads, page_size)
    try:
        for rep in range(2):
            if rep:
                w.q_nope = W.bf16_normals(rng, w.q_nope.shape)
            o, lse = _run_fp8(w, codes, scale, plan=plan)
            o_ref, l_ref = _oracle_fp8(w, codes, scale)
            assert_close(o, lse, o_ref, l_ref, f"fp8 shared pool H={heads} P={page_size} run {rep}")
    finally:
        plan.close()


@pytest.mark.parametrize("heads,page_size,shape", [(16, 64, "decode"), (32, 16, "pool"),
                                                   (128, 64, "decode")])
def test_fp8_graph_replays_match_eager(heads, page_size, shape):
    """mla_run_fp8 captured in a HIP graph and replayed, with eager runs
    between the replays: every replay equals the eager result bit for bit
    (the two-wave split kernel up to 32 heads, from the host slot and with a
    shared pool; the four-wave kernel at 128 heads)."""
    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(520 + heads + page_size)
    if shape == "decode":
        w = W.make_workload("fp8_g", 0, [700, 33, 1500, 64, 2100], [1] * 5, heads, page_size,
                            rng=rng)
    else:
        workers = torch.cuda.get_device_properties(0).multi_processor_count * 2
        q_len = (4 * workers + 7) // 8 + 3
        kv = q_len + np.array([0, 1200, 40, 1500, 10, 900, 0, 1300])
        w = W.make_workload("fp8_gp", 0, kv, [q_len] * 8, heads, page_size, rng=rng)
    scale = 0.11
    codes = torch.from_numpy(np.ascontiguousarray(W.fp8_cache_codes(w.kv_cache, scale))).cuda()
    qn, qp = _dev_bits(w.q_nope), _dev_bits(w.q_pe)
    T, H = w.num_tokens, heads
    plan = pm.MLAPlan(H, page_size)
    try:
        plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=True,
                  sm_scale=w.sm_scale, num_cache_pages=w.num_pages, kv_dtype="fp8_e4m3")
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
        plan.run(qn, qp, codes, out=out, lse=lse, kv_scale=scale)
        torch.cuda.synchronize()
        ref_o, ref_l = out.clone(), lse.clone()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            plan.run(qn, qp, codes, out=out, lse=lse, stream=st, kv_scale=scale)
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(qn, qp, codes, out=out, lse=lse, kv_scale=scale)
        for k in range(3):
            out.fill_(0)
            lse.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o), f"replay {k}: output differs"
            assert torch.equal(lse, ref_l), f"replay {k}: lse differs"
            plan.run(qn, qp, codes, out=out, lse=lse, kv_scale=scale)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o)
        o_ref, l_ref = _oracle_fp8(w, W.fp8_cache_codes(w.kv_cache, scale), scale)
        assert_close(from_dev_bf16(ref_o), ref_l.cpu().numpy(), o_ref, l_ref,
                     f"fp8 graph H={heads} P={page_size}")
    finally:
        plan.close()


def test_fp8_host_slot_first_items_beyond_staged_pages():
    """The two-wave fp8 kernel on a host-slot schedule whose first items span
    about 20 pages (more than the slot stages per worker): the producer wave
    loads those page lists from the slot's page table."""
    rng = np.random.default_rng(611)
    w = W.make_workload("fp8_hs_pages", 0, [40000] * 8, [1] * 8, 16, 32, rng=rng)
    scale = 0.07
    codes = W.fp8_cache_codes(w.kv_cache, scale)
    o, lse = _run_fp8(w, codes, scale)
    o_ref, l_ref = _oracle_fp8(w, codes, scale)
    assert_close(o, lse, o_ref, l_ref, "fp8 host slot, first items beyond staged pages")
