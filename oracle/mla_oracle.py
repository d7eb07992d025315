"""Plain fp64 CPU oracle for paged latent attention (MLA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes (sources are the m-star documentation pages):

* "mstar.engine.resources.attn.flashinfer_mla", module description: the cache
  holds one ``[ckv | kpe]`` latent per token; the query is the absorbed
  ``q_nope`` (kv_lora_rank wide) plus the un-rotated ``q_pe``; the output
  stays in the latent space ``[tokens, heads, kv_lora_rank]``.
* same page, ``FlashInferMLAWrapper.run``: shapes ``q_nope [T,H,512]``,
  ``q_pe [T,H,64]``, ``kv_cache_layer [pages, page_size, latent]``, output
  ``[T,H,512]`` and, optionally, the natural-log log-sum-exp of the scores
  ``[T,H]``.
* same page, ``FlashInferMLAWrapper`` parameters: ``sm_scale`` is the softmax
  scale of the original head dim (192 ** -0.5); ``plan`` takes the CSR page
  table (qo_indptr, paged_kv_indptr, paged_kv_indices,
  paged_kv_last_page_len) with ``causal=True`` by default.
* "mstar.engine.resources.attn.ragged.wrappers", ``PrefixedPrefillWrapper``:
  a causal query block is aligned to the end of its keys.
* ``FlashInferMLAManager.run``: the LSE exists to merge with another key
  segment (``merge_state`` below).

Score for token t, head h and key j:
``s_j = sm_scale * (q_nope[t,h] . ckv_j + q_pe[t,h] . kpe_j)``;
``o = sum_j softmax(s)_j ckv_j``; ``lse = ln sum_j exp(s_j)``.

Readings where the pages are silent (each also listed in the design notes):
row length ``L = (n_pages - 1) * page_size + last_page_len``; query i of a
row with Q queries sees keys ``j < min(L, i + L - Q + 1)`` when causal, all
``L`` keys otherwise; a query with no visible key gives ``o = 0`` and
``lse = -inf``; the LSE is over the *scaled* scores; ``sm_scale`` is used
at the fp32 value the kernel receives.

Appending the step's latent rows (page "mstar.engine.resources.attn.base",
``AttentionManager.requires_kv_write``: a layer writes this step's K/V through
the KV resource, then runs attention over the cache): reading, the step's Q
tokens of a row are its last Q keys (the same end alignment as the causal
query block; the page on ``kv_len_buf`` says a row's queries and the entries
the step appends start at the end of its stored context), so token i of the
row is key ``L - Q + i``.

The projections either side of the kernel (module description of the
flashinfer_mla page: the cache is the latent, the query is absorbed as
``q_nope @ W_UK``, and the latent output is brought back to the value heads
by ``W_UV``): per head, ``q_abs[t,h,:] = q_nope[t,h,:] @ W_UK[h]`` with
``W_UK [H, d_nope, 512]`` and ``v[t,h,:] = o[t,h,:] @ W_UV[h]`` with
``W_UV [H, 512, d_v]``; reading (the pages state only the 192-wide scale):
``d_nope = d_v = 128``.

An fp8 latent cache (the wrapper's ``plan`` takes a ``kv_dtype``, default
``None``, i.e. the bf16 of ``dtype``; the pages name no fp8 format or
scale).  Reading: the cache holds OCP FP8 E4M3 codes (1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities, the
all-ones magnitude is NaN, largest finite 448) and one fp32 dequantisation
scale for the whole cache, shared by ckv and kpe: a cached value is
``decode(code) * kv_scale``.  Appending a bf16 row quantises
``fp32(x / kv_scale)`` (IEEE fp32 division) to the nearest code, ties to the
even mantissa, saturating at +-448, keeping the sign of zero.  Attention over such a cache is the
attention above over the dequantised values.

Parity pins: every function here is checked by the CPU tests against
something other than itself (brute-force non-absorbed attention, page
permutation invariance, the two-segment merge identity, the single-key and
closed-form cases, PyTorch's fp64 scaled_dot_product_attention with an
explicit bottom-right mask, and a pure-loop version).  Parity unpinned: none.
"""

from __future__ import annotations

import math

import numpy as np

KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64


def widen(x) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values; other arrays -> fp64.

    A bf16 value is the upper half of an fp32 word, so shifting its 16 bits
    left by 16 gives the fp32 bit pattern, which widens exactly to fp64.
    """
    a = np.asarray(x)
    if a.dtype == np.uint16:
        with np.errstate(invalid="ignore"):  # NaN bit patterns stay NaN
            return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def validate(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size, num_pages):
    """Check the CSR page table.  Raises ValueError.

    indptr arrays start at 0 and never decrease (the ragged-wrapper page
    states ``[0] == 0`` for its cu_seqlens); ``1 <= last <= page_size`` for
    rows that own pages; page ids lie in ``[0, num_pages)``.
    """
    qo = np.asarray(qo_indptr, dtype=np.int64)
    kv = np.asarray(kv_indptr, dtype=np.int64)
    idx = np.asarray(kv_indices, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    if page_size < 1:
        raise ValueError("page_size must be >= 1")
    if qo.ndim != 1 or kv.shape != qo.shape or last.shape != (qo.shape[0] - 1,):
        raise ValueError("indptr / last_page_len shapes disagree")
    if qo[0] != 0 or kv[0] != 0:
        raise ValueError("indptr[0] must be 0")
    if np.any(np.diff(qo) < 0) or np.any(np.diff(kv) < 0):
        raise ValueError("indptr must be non-decreasing")
    if idx.shape[0] < kv[-1]:
        raise ValueError("kv_indices shorter than kv_indptr[-1]")
    n = np.diff(kv)
    if np.any((n > 0) & ((last < 1) | (last > page_size))):
        raise ValueError("last_page_len out of [1, page_size]")
    used = idx[: kv[-1]]
    if used.size and (used.min() < 0 or used.max() >= num_pages):
        raise ValueError("page id out of range")


def kv_lengths(kv_indptr, kv_last_page_len, page_size) -> np.ndarray:
    """Keys per row: ``(n - 1) * page_size + last`` for n > 0 pages, else 0."""
    n = np.diff(np.asarray(kv_indptr, dtype=np.int64))
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    return np.where(n > 0, (n - 1) * page_size + last, 0)


def visible_keys(i, q_len, kv_len, causal) -> int:
    """Number of keys query i of a row sees (prefix of the row's keys).

    Causal alignment to the end of the keys: query i sits at key position
    ``i + kv_len - q_len``, so it sees keys ``0 .. i + kv_len - q_len``.
    """
    if not causal:
        return int(kv_len)
    return int(min(kv_len, max(0, i + kv_len - q_len + 1)))


def gather_row_keys(kv_cache, kv_indptr, kv_indices, row, kv_len, page_size) -> np.ndarray:
    """The row's keys in key order, fp64 ``[L, 576]``: key j lives in page
    ``kv_indices[kv_indptr[row] + j // page_size]`` at slot ``j % page_size``."""
    j = np.arange(int(kv_len))
    pages = np.asarray(kv_indices)[int(kv_indptr[row]) + j // page_size]
    slots = j % page_size
    return widen(np.asarray(kv_cache)[pages, slots, :])


def attention(q_nope, q_pe, kv_cache, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
              page_size, causal, sm_scale, tokens=None, validate_inputs=True,
              max_block_elems=1 << 24):
    """Paged latent attention in fp64.

    Returns ``(o [n, H, 512], lse [n, H])`` for the requested ``tokens``
    (all tokens when None, in order).  bf16 inputs are given as uint16 bit
    patterns; float arrays are used as they are (in fp64).
    """
    kv_cache_a = np.asarray(kv_cache)
    num_pages = kv_cache_a.shape[0]
    if validate_inputs:
        validate(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size, num_pages)
    qo = np.asarray(qo_indptr, dtype=np.int64)
    T = int(qo[-1])
    H = np.asarray(q_nope).shape[1]
    sm = float(np.float32(sm_scale))
    lens = kv_lengths(kv_indptr, kv_last_page_len, page_size)
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    rows_of = np.searchsorted(qo, tokens, side="right") - 1
    o = np.zeros((tokens.shape[0], H, KV_LORA_RANK))
    lse = np.full((tokens.shape[0], H), -np.inf)
    for row in np.unique(rows_of):
        sel = np.nonzero(rows_of == row)[0]
        L = int(lens[row])
        Q = int(qo[row + 1] - qo[row])
        if L == 0:
            continue
        K = gather_row_keys(kv_cache_a, kv_indptr, kv_indices, row, L, page_size)
        ckv, kpe = K[:, :KV_LORA_RANK], K[:, KV_LORA_RANK:]
        per = max(1, max_block_elems // max(1, H * L))
        for s in range(0, sel.shape[0], per):
            part = sel[s:s + per]
            t = tokens[part]
            qn = widen(np.asarray(q_nope)[t])  # [n, H, 512]
            qp = widen(np.asarray(q_pe)[t])    # [n, H, 64]
            scores = sm * (qn @ ckv.T + qp @ kpe.T)  # [n, H, L]
            vis = np.array([visible_keys(int(x - qo[row]), Q, L, causal) for x in t])
            mask = np.arange(L)[None, :] < vis[:, None]  # [n, L]
            scores = np.where(mask[:, None, :], scores, -np.inf)
            has = vis > 0
            if not np.any(has):
                continue
            hs = part[has]
            sc = scores[has]
            m = sc.max(axis=-1, keepdims=True)
            w = np.exp(sc - m)
            z = w.sum(axis=-1, keepdims=True)
            o[hs] = (w @ ckv) / z
            lse[hs] = (m + np.log(z))[..., 0]
    return o, lse


def merge_state(v_a, s_a, v_b, s_b):
    """Merge two attention results over disjoint key segments, in fp64.

    ``(v, s)`` pairs are a normalised output and its natural-log LSE.  With
    ``M = max(s_a, s_b)``: ``w = exp(s - M)``, ``s = M + ln(w_a + w_b)``,
    ``v = (w_a v_a + w_b v_b) / (w_a + w_b)``; two empty segments
    (``s = -inf``) give ``(0, -inf)``.
    """
    va, vb = widen(v_a), widen(v_b)
    sa, sb = widen(s_a), widen(s_b)
    M = np.maximum(sa, sb)
    empty = np.isneginf(M)
    Mf = np.where(empty, 0.0, M)
    wa = np.where(np.isneginf(sa), 0.0, np.exp(sa - Mf))
    wb = np.where(np.isneginf(sb), 0.0, np.exp(sb - Mf))
    z = wa + wb
    zs = np.where(empty, 1.0, z)
    v = (wa[..., None] * va + wb[..., None] * vb) / zs[..., None]
    v = np.where(empty[..., None], 0.0, v)
    s = np.where(empty, -np.inf, Mf + np.log(zs))
    return v, s


def attention_loops(q_nope, q_pe, kv_cache, qo_indptr, kv_indptr, kv_indices,
                    kv_last_page_len, page_size, causal, sm_scale):
    """The same definition with plain Python loops (tiny inputs only)."""
    qn_all, qp_all, cache = widen(q_nope), widen(q_pe), widen(kv_cache)
    sm = float(np.float32(sm_scale))
    B = len(qo_indptr) - 1
    T, H = qn_all.shape[0], qn_all.shape[1]
    o = [[[0.0] * KV_LORA_RANK for _ in range(H)] for _ in range(T)]
    lse = [[-math.inf] * H for _ in range(T)]
    for b in range(B):
        n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        L = 0 if n == 0 else (n - 1) * page_size + int(kv_last_page_len[b])
        Q = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        for i in range(Q):
            t = int(qo_indptr[b]) + i
            nvis = L if not causal else min(L, max(0, i + L - Q + 1))
            for h in range(H):
                scores = []
                rows = []
                for j in range(nvis):
                    page = int(kv_indices[int(kv_indptr[b]) + j // page_size])
                    key = cache[page, j % page_size]
                    dot = 0.0
                    for d in range(KV_LORA_RANK):
                        dot += qn_all[t, h, d] * key[d]
                    for d in range(QK_ROPE_HEAD_DIM):
                        dot += qp_all[t, h, d] * key[KV_LORA_RANK + d]
                    scores.append(sm * dot)
                    rows.append(key[:KV_LORA_RANK])
                if not scores:
                    continue
                m = max(scores)
                ws = [math.exp(s - m) for s in scores]
                z = sum(ws)
                acc = [0.0] * KV_LORA_RANK
                for w, r in zip(ws, rows):
                    for d in range(KV_LORA_RANK):
                        acc[d] += w * r[d]
                o[t][h] = [a / z for a in acc]
                lse[t][h] = m + math.log(z)
    return np.array(o, dtype=np.float64), np.array(lse, dtype=np.float64)


def append_kv(kv_cache, ckv, kpe, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
              page_size):
    """The cache after this step's latent rows are written (a new array).

    ``kv_cache`` is uint16 bf16 bits ``[pages, page_size, 576]``; ``ckv``
    ``[T, 512]`` and ``kpe`` ``[T, 64]`` hold the step's rows for the tokens
    of ``qo_indptr``.  Token ``t = qo_indptr[b] + i`` becomes key
    ``j = L_b - Q_b + i`` of row b: ``[ckv[t] | kpe[t]]`` is stored at slot
    ``j % page_size`` of page ``kv_indices[kv_indptr[b] + j // page_size]``.
    Raises ValueError when a row has more tokens than keys, or when two
    tokens would land in the same slot.
    """
    cache = np.array(kv_cache, copy=True)
    num_pages = cache.shape[0]
    validate(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size, num_pages)
    qo = np.asarray(qo_indptr, dtype=np.int64)
    lens = kv_lengths(kv_indptr, kv_last_page_len, page_size)
    idx = np.asarray(kv_indices, dtype=np.int64)
    written = set()
    for b in range(qo.shape[0] - 1):
        Q = int(qo[b + 1] - qo[b])
        L = int(lens[b])
        if Q > L:
            raise ValueError(f"row {b} has {Q} tokens but only {L} keys")
        for i in range(Q):
            j = L - Q + i
            page = int(idx[int(kv_indptr[b]) + j // page_size])
            slot = j % page_size
            if (page, slot) in written:
                raise ValueError(f"two tokens write page {page} slot {slot}")
            written.add((page, slot))
            t = int(qo[b]) + i
            cache[page, slot, :KV_LORA_RANK] = ckv[t]
            cache[page, slot, KV_LORA_RANK:] = kpe[t]
    return cache


def head_matmul(x, w):
    """Per-head product ``out[t, h, :] = x[t, h, :] @ w[h]`` in fp64.

    ``x [T, H, K]`` and ``w [H, K, N]`` are bf16 bit patterns (uint16) or
    float arrays; returns ``[T, H, N]`` fp64.
    """
    xf, wf = widen(x), widen(w)
    return np.einsum("thk,hkn->thn", xf, wf)


def absorb_query(q_nope, w_uk):
    """The absorbed query ``q_nope @ W_UK`` per head: ``[T, H, 128] x
    [H, 128, 512] -> [T, H, 512]`` (fp64)."""
    return head_matmul(q_nope, w_uk)


def up_project(o, w_uv):
    """The latent output brought to the value heads, ``o @ W_UV`` per head:
    ``[T, H, 512] x [H, 512, 128] -> [T, H, 128]`` (fp64)."""
    return head_matmul(o, w_uv)


# ---------------------------------------------------------------------------
# fp8 (OCP E4M3) latent cache
# ---------------------------------------------------------------------------

FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode(codes) -> np.ndarray:
    """fp64 values of FP8 E4M3 codes (uint8), by the format's definition:
    sign s, exponent field e (bias 7), mantissa field m; e = 0 gives the
    subnormal ``m / 8 * 2**-6``, otherwise ``(1 + m / 8) * 2**(e - 7)``;
    e = 15 with m = 7 is NaN (there are no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def fp8_e4m3_encode(x) -> np.ndarray:
    """FP8 E4M3 code (uint8) nearest to each finite value of ``x``, ties to
    the even code, magnitudes beyond 448 saturated to 448; the sign is kept,
    also for a value that rounds to zero (-0).

    Written as a search over the 127 non-negative finite codes (their
    values increase with the code): the two neighbours of |x| and the
    distance to each decide, a tie goes to the code with an even mantissa."""
    v = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("fp8 encode takes finite values only")
    grid = fp8_e4m3_decode(np.arange(127, dtype=np.uint8))  # 0 .. 448, increasing
    a = np.minimum(np.abs(v), FP8_E4M3_MAX)
    hi = np.searchsorted(grid, a, side="left")  # first grid value >= a
    hi = np.minimum(hi, 126)
    lo = np.where(grid[hi] == a, hi, np.maximum(hi - 1, 0))
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def fp8_quantize_rows(x_bits, kv_scale) -> np.ndarray:
    """Codes of bf16 values (uint16 bits) stored in an fp8 cache with scale
    ``kv_scale``: the fp32 quotient ``x / kv_scale`` rounded to a code."""
    q = (widen(x_bits).astype(np.float32) / np.float32(kv_scale)).astype(np.float64)
    return fp8_e4m3_encode(q)


def dequantize_cache(kv_cache_fp8, kv_scale) -> np.ndarray:
    """The values an fp8 cache holds, fp64: ``decode(code) * kv_scale``."""
    return fp8_e4m3_decode(kv_cache_fp8) * float(np.float32(kv_scale))


def attention_fp8(q_nope, q_pe, kv_cache_fp8, qo_indptr, kv_indptr, kv_indices,
                  kv_last_page_len, page_size, causal, sm_scale, kv_scale, tokens=None):
    """Paged latent attention over an fp8 cache (codes ``[pages, P, 576]``
    uint8): the attention above on the dequantised cache."""
    return attention(q_nope, q_pe, dequantize_cache(kv_cache_fp8, kv_scale), qo_indptr,
                     kv_indptr, kv_indices, kv_last_page_len, page_size, causal, sm_scale,
                     tokens=tokens)


def append_kv_fp8(kv_cache_fp8, ckv, kpe, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                  page_size, kv_scale):
    """The fp8 cache after this step's bf16 rows are quantised and written
    to the slots ``append_kv`` gives them (a new array)."""
    return append_kv(kv_cache_fp8, fp8_quantize_rows(ckv, kv_scale),
                     fp8_quantize_rows(kpe, kv_scale), qo_indptr, kv_indptr, kv_indices,
                     kv_last_page_len, page_size)
