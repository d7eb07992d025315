"""Helpers shared by the GPU tests: upload a workload, run the library,
compare with the oracle at the stated tolerances."""

import numpy as np
import torch

import oracle

# Tolerances: bf16 output |err| <= 1e-2 + 1e-2 |ref|, LSE |err| <= 2e-3.
O_ATOL, O_RTOL, LSE_ATOL = 1e-2, 1e-2, 2e-3


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def run_library(w, plan=None, return_lse=True, kv_cache=None, q=None):
    """Plan and run workload `w` through the C ABI; returns (o bits, lse)."""
    import paged_mla_attention_amd as pm
    own = plan is None
    if own:
        plan = pm.MLAPlan(w.num_heads, w.page_size)
    qn, qp = q if q is not None else (to_dev_bf16(w.q_nope), to_dev_bf16(w.q_pe))
    kv = kv_cache if kv_cache is not None else to_dev_bf16(w.kv_cache)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=w.causal,
              sm_scale=w.sm_scale, num_cache_pages=w.num_pages)
    res = plan.run(qn, qp, kv, return_lse=return_lse)
    torch.cuda.synchronize()
    if own:
        plan.close()
    if return_lse:
        o, lse = res
        return from_dev_bf16(o), lse.cpu().numpy()
    return from_dev_bf16(res), None


def assert_close(o_bits, lse, o_ref, lse_ref, what=""):
    """Element-wise check against the fp64 oracle."""
    o = oracle.widen(o_bits)
    assert not np.isnan(o).any(), f"{what}: NaN in output"
    err = np.abs(o - o_ref)
    bound = O_ATOL + O_RTOL * np.abs(o_ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} output elements out of tolerance, "
                             f"max err {err.max():.3e}; first at {idx.tolist()}")
    if lse is not None:
        assert not np.isnan(lse).any(), f"{what}: NaN in lse"
        ninf_ref = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse), ninf_ref), f"{what}: -inf pattern differs"
        fin = ~ninf_ref
        if fin.any():
            lerr = np.abs(lse[fin] - lse_ref[fin]).max()
            assert lerr <= LSE_ATOL, f"{what}: lse max err {lerr:.3e}"


def oracle_of(w, tokens=None):
    return oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                            w.kv_indices, w.kv_last_page_len, w.page_size, w.causal,
                            w.sm_scale, tokens=tokens)


def sample_tokens(w, per_row=6, seed=0):
    """First, last and a few random query tokens of every row."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(w.batch):
        s, e = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        if e == s:
            continue
        pick = {s, e - 1}
        if e - s > 2:
            pick.update(rng.integers(s, e, size=min(per_row, e - s)).tolist())
        out.extend(sorted(pick))
    return np.array(out, dtype=np.int64)


def split_tokens(w, workers=None):
    """Query tokens whose keys the planner splits over several work items
    (their results go through the split-KV merge), for a plan on this
    device (one worker per compute unit) unless `workers` is given."""
    import paged_mla_attention_amd as pm
    if workers is None:
        workers = torch.cuda.get_device_properties(0).multi_processor_count
    s = pm.schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.page_size,
                    w.num_pages, w.num_heads, workers, causal=w.causal)
    return np.unique(s["merges"][:, 0]).astype(np.int64)
