"""Per-head projections (mla_absorb_query, mla_up_project) through the C ABI
against the fp64 oracle: several token blocks with a ragged tail, head counts
up to 128, the decode and chunked-prefill shapes (sampled tokens), and the
chain absorb -> attention -> up-projection stage by stage."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import O_ATOL, O_RTOL, assert_close, from_dev_bf16, to_dev_bf16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    pm.library()
    return pm


def _bf16(rng, shape, scale=1.0):
    return W.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _check(got_bits, ref, what):
    got = oracle.widen(got_bits)
    err = np.abs(got - ref)
    bad = err > O_ATOL + O_RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"


@pytest.mark.parametrize("T,H", [(1, 1), (37, 3), (128, 16), (300, 8), (129, 128)])
def test_absorb_and_up_project(T, H):
    pm = _gpu()
    rng = np.random.default_rng(T * 131 + H)
    q = _bf16(rng, (T, H, 128))
    w_uk = _bf16(rng, (H, 128, 512), 128 ** -0.5)
    o = _bf16(rng, (T, H, 512))
    w_uv = _bf16(rng, (H, 512, 128), 512 ** -0.5)
    qa = pm.absorb_query(to_dev_bf16(q), to_dev_bf16(w_uk))
    v = pm.up_project(to_dev_bf16(o), to_dev_bf16(w_uv))
    torch.cuda.synchronize()
    _check(from_dev_bf16(qa), oracle.absorb_query(q, w_uk), "absorb")
    _check(from_dev_bf16(v), oracle.up_project(o, w_uv), "up-projection")


@pytest.mark.parametrize("T", [64, 4096])
def test_full_shapes_sampled(T):
    pm = _gpu()
    H = 128
    rng = np.random.default_rng(T)
    q = _bf16(rng, (T, H, 128))
    w_uk = _bf16(rng, (H, 128, 512), 128 ** -0.5)
    o = _bf16(rng, (T, H, 512))
    w_uv = _bf16(rng, (H, 512, 128), 512 ** -0.5)
    qa = from_dev_bf16(pm.absorb_query(to_dev_bf16(q), to_dev_bf16(w_uk)))
    v = from_dev_bf16(pm.up_project(to_dev_bf16(o), to_dev_bf16(w_uv)))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 40)]))
    _check(qa[toks], oracle.absorb_query(q[toks], w_uk), "absorb")
    _check(v[toks], oracle.up_project(o[toks], w_uv), "up-projection")


def test_chain_absorb_attend_up_project():
    """Each stage of the layer's attention on its own inputs: the absorbed
    query the GPU produced feeds the oracle's attention, and the latent output
    the GPU produced feeds the oracle's up-projection."""
    pm = _gpu()
    w = W.tiny()
    rng = np.random.default_rng(5)
    T, H = w.num_tokens, w.num_heads
    q_orig = _bf16(rng, (T, H, 128))
    w_uk = _bf16(rng, (H, 128, 512), 128 ** -0.5)
    w_uv = _bf16(rng, (H, 512, 128), 512 ** -0.5)
    qa = pm.absorb_query(to_dev_bf16(q_orig), to_dev_bf16(w_uk))
    plan = pm.MLAPlan(H, w.page_size)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=True,
              sm_scale=w.sm_scale, num_cache_pages=w.num_pages)
    o, lse = plan.run(qa, to_dev_bf16(w.q_pe), to_dev_bf16(w.kv_cache), return_lse=True)
    v = pm.up_project(o, to_dev_bf16(w_uv))
    torch.cuda.synchronize()
    plan.close()
    qa_bits, o_bits = from_dev_bf16(qa), from_dev_bf16(o)
    _check(qa_bits, oracle.absorb_query(q_orig, w_uk), "absorb")
    o_ref, l_ref = oracle.attention(qa_bits, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                                    w.kv_indices, w.kv_last_page_len, w.page_size, True,
                                    w.sm_scale)
    assert_close(o_bits, lse.cpu().numpy(), o_ref, l_ref, "attention")
    _check(from_dev_bf16(v), oracle.up_project(o_bits, w_uv), "up-projection")


def test_projection_errors():
    pm = _gpu()
    from paged_mla_attention_amd import _native
    lib = pm.library()
    assert lib.mla_absorb_query(None, None, None, 0, 4, None) == 0  # nothing to do
    assert lib.mla_absorb_query(None, None, None, 3, 4, None) == 1
    assert lib.mla_up_project(1, 1, 1, -1, 4, None) == 1
    assert lib.mla_up_project(1, 1, 1, 3, 0, None) == 1
    with pytest.raises(ValueError):
        pm.absorb_query(torch.zeros((2, 4, 64), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((4, 128, 512), dtype=torch.bfloat16, device="cuda"))
    assert _native is not None
