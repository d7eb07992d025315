"""KV append (mla_append_kv): the planner's destination rows on the CPU, and
the HIP scatter through the C ABI against the oracle's append, bit for bit,
followed by attention over the appended cache."""

import numpy as np
import pytest

import oracle
import workloads as W
from test_append_oracle import _case, _walk

torch = pytest.importorskip("torch")


def _rows_by_walk(qo, kv_indptr, kv_indices, last, page_size):
    """Cache rows of the step's tokens by walking each row's pages slot by
    slot (no division), the last Q slots for the row's Q tokens."""
    out = []
    for b in range(len(qo) - 1):
        slots = []
        pages = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
        for k, p in enumerate(pages):
            fill = last[b] if k == len(pages) - 1 else page_size
            slots += [int(p) * page_size + s for s in range(fill)]
        q = int(qo[b + 1] - qo[b])
        out += slots[len(slots) - q:] if q else []
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("page_size", [1, 3, 16, 64])
def test_planner_append_rows_match_page_walk(page_size):
    import paged_mla_attention_amd as pm
    rows = [(37, 1), (100, 5), (0, 0), (64, 64), (5, 2), (129, 0)]
    _, _, _, qo, kvp, idx, last = _case(17 + page_size, page_size, rows)
    from paged_mla_attention_amd import _native
    got = pm.append_rows(qo, kvp, idx, last, page_size, int(idx.max()) + 2,
                         lib_path=_native.HOST_LIB_PATH)
    assert np.array_equal(got.astype(np.int64), _rows_by_walk(qo, kvp, idx, last, page_size))


def test_planner_append_rejects_bad_tables():
    import paged_mla_attention_amd as pm
    from paged_mla_attention_amd import _native
    with pytest.raises(_native.MLAError, match="query tokens"):
        pm.append_rows([0, 4], [0, 1], [0], [3], 8, 4, lib_path=_native.HOST_LIB_PATH)
    with pytest.raises(_native.MLAError, match="same|cache row"):
        pm.append_rows([0, 1, 2], [0, 1, 2], [2, 2], [4, 4], 4, 4,
                       lib_path=_native.HOST_LIB_PATH)


# ---------------------------------------------------------------- GPU parity

def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    pm.library()
    return pm


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _append_gpu(pm, c, page_size, num_heads=16, plan=None):
    cache, ckv, kpe, qo, kvp, idx, last = c
    own = plan is None
    if own:
        plan = pm.MLAPlan(num_heads, page_size)
    plan.plan(qo, kvp, idx, last, causal=True, sm_scale=192 ** -0.5,
              num_cache_pages=cache.shape[0])
    kv = _dev(cache)
    plan.append_kv(_dev(ckv), _dev(kpe), kv)
    torch.cuda.synchronize()
    if own:
        plan.close()
    return kv


@pytest.mark.gpu
@pytest.mark.parametrize("page_size", [1, 3, 16, 64])
def test_append_bitwise(page_size):
    pm = _gpu()
    rows = [(37, 1), (100, 5), (0, 0), (64, 64), (5, 2), (129, 0), (2000, 300)]
    c = _case(31 + page_size, page_size, rows)
    got = _host(_append_gpu(pm, c, page_size))
    assert np.array_equal(got, oracle.append_kv(*c, page_size))


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["decode_batch", "chunked_prefill"])
def test_append_full_size_then_attend(name):
    """The workload's own queries are this step's tokens: append fresh rows
    for them (bit-exact against the oracle), then attention over the new
    cache matches the oracle on sampled tokens."""
    pm = _gpu()
    from gpu_util import assert_close, from_dev_bf16, sample_tokens
    w = getattr(W, name)()
    rng = np.random.default_rng(99)
    T = w.num_tokens
    ckv = W.bf16_normals(rng, (T, 512))
    kpe = W.bf16_normals(rng, (T, 64))
    c = (w.kv_cache, ckv, kpe, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len)
    plan = pm.MLAPlan(w.num_heads, w.page_size)
    kv = _append_gpu(pm, c, w.page_size, plan=plan)
    ref_cache = oracle.append_kv(*c, w.page_size)
    assert np.array_equal(_host(kv), ref_cache)
    o, lse = plan.run(_dev(w.q_nope), _dev(w.q_pe), kv, return_lse=True)
    torch.cuda.synchronize()
    plan.close()
    toks = sample_tokens(w, per_row=2, seed=5)
    o_ref, l_ref = oracle.attention(w.q_nope, w.q_pe, ref_cache, w.qo_indptr, w.kv_indptr,
                                    w.kv_indices, w.kv_last_page_len, w.page_size, w.causal,
                                    w.sm_scale, tokens=toks)
    assert_close(from_dev_bf16(o)[toks], lse.cpu().numpy()[toks], o_ref, l_ref, name)


@pytest.mark.gpu
def test_append_errors():
    pm = _gpu()
    from paged_mla_attention_amd import _native
    plan = pm.MLAPlan(16, 4)
    z = torch.zeros((2, 512), dtype=torch.bfloat16, device="cuda")
    zp = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((4, 4, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        plan.append_kv(z, zp, kv)  # before plan
    plan.plan([0, 1, 2], [0, 1, 2], [2, 2], [4, 4], num_cache_pages=4)
    with pytest.raises(_native.MLAError, match="cache row"):
        plan.append_kv(z, zp, kv)  # both tokens land in page 2 slot 3
    plan.plan([0, 2], [0, 1], [1], [1], num_cache_pages=4)
    with pytest.raises(_native.MLAError, match="query tokens"):
        plan.append_kv(z, zp, kv)
    plan.close()
