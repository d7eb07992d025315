"""Host planner tests (CPU): schedule invariants, validation errors, and a
replay of the schedule through the oracle (each work item's key range
attended on its own, then the partials merged through their LSEs) that must
reproduce the oracle's result on the whole row."""

import os

import numpy as np
import pytest

import oracle
import workloads as W
from paged_mla_attention_amd import _native, schedule
from paged_mla_attention_amd.build import build_host_planner

TILE = 32


@pytest.fixture(scope="module")
def host_lib():
    if not os.path.exists(_native.HOST_LIB_PATH):
        build_host_planner()
    return _native.HOST_LIB_PATH


def _sched(w, workers, host_lib, causal=None):
    return schedule(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.page_size,
                    w.num_pages, w.num_heads, workers,
                    causal=w.causal if causal is None else causal, lib_path=host_lib)


def _check_invariants(w, s, workers):
    items, merges, wi = s["items"], s["merges"], s["worker_indptr"]
    assert wi.shape == (workers + 2,) and wi[0] == 0 and wi[-1] == items.shape[0]
    assert np.all(np.diff(wi) >= 0)
    # the shared pool: whole tokens (final outputs), largest first
    pool = items[wi[workers]:wi[workers + 1]]
    assert np.all(pool[:, 4] == -1) and np.all(pool[:, 2] == 0)
    ptiles = (pool[:, 3] + TILE - 1) // TILE
    assert np.all(np.diff(ptiles) <= 0)
    T = w.num_tokens
    lens = w.kv_lens()
    qo = w.qo_indptr
    # expected visible keys per token
    vis = np.zeros(T, np.int64)
    row_of = np.zeros(T, np.int64)
    for b in range(w.batch):
        Q = int(qo[b + 1] - qo[b])
        for i in range(Q):
            vis[qo[b] + i] = oracle.visible_keys(i, Q, int(lens[b]), w.causal)
            row_of[qo[b] + i] = b
    covered = [[] for _ in range(T)]
    for it in items:
        t, row, kb, ke, slot = (int(x) for x in it[:5])
        assert 0 <= t < T and row == row_of[t]
        assert int(it[5]) == int(w.kv_indptr[row])  # the row's page-list base
        assert kb % TILE == 0 and 0 <= kb <= ke <= vis[t]
        covered[t].append((kb, ke, slot))
    slot_seen = set()
    split_tokens = {int(m[0]): (int(m[1]), int(m[2])) for m in merges}
    for t in range(T):
        rngs = sorted(covered[t])
        assert rngs, f"token {t} has no item"
        # exactly-once coverage of [0, vis)
        pos = 0
        for kb, ke, _ in rngs:
            assert kb == pos
            pos = ke
        assert pos == vis[t]
        if len(rngs) == 1:
            assert rngs[0][2] == -1 and t not in split_tokens
        else:
            first, n = split_tokens[t]
            assert n == len(rngs)
            slots = sorted(r[2] for r in rngs)
            assert slots == list(range(first, first + n))
            slot_seen.update(slots)
            assert all(ke > kb for kb, ke, _ in rngs)  # no empty pieces
    assert len(slot_seen) == s["num_slots"]


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "long_decode"])
@pytest.mark.parametrize("workers", [1, 7, 256])
def test_schedule_invariants(name, workers, host_lib):
    gen = {"tiny": W.tiny,
           "decode": lambda: W.decode_batch(batch=16, num_heads=8),
           "prefill": lambda: W.make_workload("p", 3, [700, 512, 0, 1300], [512, 64, 3, 100], 8,
                                              64, rng=np.random.default_rng(3)),
           "long_decode": lambda: W.make_workload("l", 4, [4096] * 3, [1] * 3, 16, 64,
                                                  rng=np.random.default_rng(4))}[name]
    w = gen()
    s = _sched(w, workers, host_lib)
    _check_invariants(w, s, workers)


def test_schedule_balances_full_workloads(host_lib):
    """At the decode and prefill workloads' page tables (no tensors needed),
    the most loaded worker's own list carries at most 25% more key tiles than
    the mean of the lists."""
    for w in (W.decode_batch(), W.chunked_prefill()):
        s = _sched(w, 256, host_lib)
        _check_invariants(w, s, 256)
        it, wi = s["items"], s["worker_indptr"]
        tiles = (it[:, 3] - it[:, 2] + TILE - 1) // TILE
        own = tiles[:wi[256]]
        per = np.add.reduceat(np.r_[own, 0], wi[:256])[:256] * (np.diff(wi[:257]) > 0)
        assert per.max() <= 1.25 * own.sum() / 256 + 8


def test_shared_pool_sizes(host_lib):
    """A batch of many query tokens keeps its smallest whole tokens, about a
    tenth of the work and each small against a worker's share, in the shared
    pool; a decode batch (fewer tokens than four per worker) has none."""
    item_cost = 7.0  # the cost model's fixed part of an item at 128 heads, in tiles
    s = _sched(W.decode_batch(), 256, host_lib)
    assert s["worker_indptr"][256] == s["worker_indptr"][257]
    w = W.chunked_prefill()
    s = _sched(w, 256, host_lib)
    it, wi = s["items"], s["worker_indptr"]
    cost = (it[:, 3] - it[:, 2] + TILE - 1) // TILE + item_cost
    pool = cost[wi[256]:wi[257]]
    assert 0.08 * cost.sum() <= pool.sum() <= 0.10 * cost.sum()
    assert pool.max() <= cost.sum() / 256 / 8
    # every pooled token is no longer than any whole token left in the lists
    own = it[:wi[256]]
    whole = own[own[:, 4] == -1]
    assert pool.max() - item_cost <= ((whole[:, 3] + TILE - 1) // TILE).min() or len(whole) == 0


@pytest.mark.parametrize("workers", [3, 64])
def test_plan_replay_matches_oracle(workers, host_lib):
    """Attend every work item's key range with the oracle, merge the partial
    results of split tokens with the oracle merge, and compare with the oracle
    on whole rows."""
    rng = np.random.default_rng(41)
    w = W.make_workload("replay", 41, [300, 37, 0, 129, 1000], [1, 5, 2, 40, 1], 2, 16,
                        rng=rng)
    s = _sched(w, workers, host_lib)
    _check_invariants(w, s, workers)
    o_ref, l_ref = oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                                    w.kv_indices, w.kv_last_page_len, w.page_size, True,
                                    w.sm_scale)
    H = w.num_heads
    parts = {}
    for it in s["items"]:
        t, row, kb, ke, slot = (int(x) for x in it[:5])
        # a one-row, one-token problem over the keys [kb, ke) of `row`
        keys = oracle.gather_row_keys(w.kv_cache, w.kv_indptr, w.kv_indices, row, ke,
                                      w.page_size)[kb:]
        n = keys.shape[0]
        cache = keys.reshape(n, 1, 576) if n else np.zeros((1, 1, 576))
        o, l = oracle.attention(w.q_nope[t:t + 1], w.q_pe[t:t + 1], cache,
                                np.array([0, 1], np.int32), np.array([0, n], np.int32),
                                np.arange(max(n, 1), dtype=np.int32), np.array([1], np.int32),
                                1, False, w.sm_scale)
        parts.setdefault(t, []).append((slot, o[0], l[0]))
    for t in range(w.num_tokens):
        p = sorted(parts[t], key=lambda x: x[0])
        o, l = p[0][1], p[0][2]
        for _, o2, l2 in p[1:]:
            o, l = oracle.merge_state(o, l, o2, l2)
        np.testing.assert_allclose(o, o_ref[t], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(l, l_ref[t], rtol=1e-12, atol=1e-12)
    assert H == 2


@pytest.mark.parametrize("bad,msg", [
    ("qo0", r"qo_indptr\[0\]"), ("kvdec", "kv_indptr decreases"), ("last0", "kv_last_page_len"),
    ("lastbig", "kv_last_page_len"), ("page", "kv_indices"), ("neg_page", "kv_indices"),
    ("heads", "num_heads"), ("rows", "2\\^31 cache rows"),
])
def test_schedule_rejects_bad_tables(bad, msg, host_lib):
    qo = np.array([0, 1, 3], np.int32)
    kv = np.array([0, 2, 3], np.int32)
    idx = np.array([0, 1, 2], np.int32)
    last = np.array([3, 4], np.int32)
    heads, pages = 16, 4
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
    elif bad == "neg_page":
        idx = np.array([0, -1, 2], np.int32)
    elif bad == "heads":
        heads = 129
    elif bad == "rows":
        pages = (1 << 29) + 1  # x 4 slots per page: one row past 2^31
    with pytest.raises(_native.MLAError, match=msg):
        schedule(qo, kv, idx, last, 4, pages, heads, 8, lib_path=host_lib)


def test_empty_batch(host_lib):
    s = schedule(np.array([0], np.int32), np.array([0], np.int32), np.zeros(0, np.int32),
                 np.zeros(0, np.int32), 16, 0, 16, 8, lib_path=host_lib)
    assert s["items"].shape[0] == 0 and s["num_slots"] == 0


def test_planner_under_sanitizers(tmp_path):
    """Build the planner with AddressSanitizer + UBSan and drive it from a
    small C++ program over random and adversarial page tables."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = os.path.join(root, "tests", "planner_fuzz.cpp")
    exe = str(tmp_path / "planner_fuzz")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-I", os.path.join(root, "include"),
                        src, os.path.join(root, "paged_mla_attention_amd", "csrc", "planner.cpp"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "300"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


def test_slot_wait_has_a_deadline(tmp_path):
    """The host's wait for the kernels to release a staging slot ends at its
    deadline when a flag never arrives (and returns at once when they have)."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "host_wait_check")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-pthread", "-I",
                        os.path.join(root, "paged_mla_attention_amd", "csrc"),
                        os.path.join(root, "tests", "host_wait_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def test_item_count_within_reserved_bound(host_lib):
    """A causal prefill over a 64K-key prefix: every query token re-walks
    its row's prefix, so the item count grows with tokens times the prefix's
    item cuts.  It stays within what a reserved plan sizes for:
    tokens * (1 + (max_keys - 1) // (32 * 1024)) + 2 * workers + 8."""
    P, workers = 64, 256
    kv_lens, qo_lens = [65536 + 512, 100], [512, 4]
    pages = [(L + P - 1) // P for L in kv_lens]
    kv_indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    kv_indices = np.random.default_rng(3).permutation(kv_indptr[-1]).astype(np.int32)
    last = np.array([L - (n - 1) * P for L, n in zip(kv_lens, pages)], np.int32)
    s = schedule(qo_indptr, kv_indptr, kv_indices, last, P, int(kv_indptr[-1]), 16, workers,
                 causal=True, lib_path=host_lib)
    T = int(qo_indptr[-1])
    max_keys = int(kv_indptr[-1]) * P
    bound = T * (1 + (max_keys - 1) // (TILE * 1024)) + 2 * workers + 8
    assert s["items"].shape[0] <= bound
    # the bound a reserved plan used to make (one cut per cached key) is exceeded
    assert s["items"].shape[0] > T + 2 * workers + max_keys // (TILE * 1024) + 8
