"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares nothing with the HIP path: no kernels, no headers, no helpers.

Every function widens its inputs losslessly to float64 and materialises the
whole N x N score matrix of each (batch, head) pair, which is exactly what the
IO-aware method avoids.  It is slow on purpose and meant to be read against
the pages:

* The result: Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V -- "FlashAttention
  (EL)", section on the problem of standard attention (the displayed formula).
  The scale is passed in explicitly; 1/sqrt(d) is the caller's default.
* The method is exact, not an approximation -- "Flash Attention uitgelegd"
  (datacamp), section "Standaard attention vs Flash attention".  So the oracle
  is that definition written out.
* Causal masking is the decoder-only variant -- "Flash Attention: Ako
  transformery zvladaju ..." section 5 ("Limity"), and ``is_causal=True`` in
  its section 6 usage example.  Reading used here: key j is visible to query i
  iff j <= i (top-left aligned; identical to bottom-right for square inputs).
* The backward pass recomputes scores instead of storing them -- datacamp page,
  section "Recomputation"; Slovak page section 2.  The pages state no gradient
  formulas, so ``ref_bwd`` is the plain chain rule through the definition.
* The saved per-row statistic is the natural-log log-sum-exp of the scaled,
  masked scores (the pages only say "running max and sum of exponentials":
  Greek page, section "Online υπολογισμός Softmax").

``ref_fwd_tiled`` is a second, independent forward that follows the pages'
tile-by-tile description literally (tiling: datacamp "Tiling", Slovak page
section 2, Greek page "Tiling"; online softmax with a running max and a running
sum: Slovak page section 2, Greek page "Online υπολογισμός Softmax").  It exists
so that a brute-force test can show tiled == naive.

Fully masked rows (unreachable for square causal inputs, where the diagonal is
always visible) are defined as O = 0 and LSE = -inf.

Grouped-query and multi-query attention (GQA/MQA) are named by the Slovak page
(section 5, "Limity a co dalej") and by the Greek page's FlashAttention-2
section (MQA), without a definition.  Reading used here: K and V carry Hkv
heads, Hkv divides the H query heads, and query head h attends with K/V head
h // (H / Hkv) (MQA: Hkv = 1; Hkv = H is ordinary multi-head attention).  The
gradient of a shared K/V head is then the sum over the query heads that use it.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head",
    "causal_visible",
    "attention_probs",
    "ref_fwd",
    "ref_fwd_rows",
    "ref_fwd_tiled",
    "ref_bwd",
    "ref_decode",
    "ref_decode_paged",
    "ref_merge_partials",
]


def kv_head(h: int, n_heads: int, n_kv_heads: int) -> int:
    """K/V head used by query head h: h // (H / Hkv) (reading in the module docstring)."""
    if n_kv_heads < 1 or n_heads % n_kv_heads:
        raise ValueError(f"{n_kv_heads} K/V heads do not divide {n_heads} query heads")
    return h // (n_heads // n_kv_heads)


def _f64(x) -> np.ndarray:
    """Widen to float64 without rounding (bf16 and fp32 are subsets of fp64)."""
    a = np.asarray(x)
    if a.dtype == np.float64:
        return a
    return a.astype(np.float64)


def causal_visible(query_rows: np.ndarray, n_keys: int) -> np.ndarray:
    """Boolean [len(query_rows), n_keys]: key j visible to query row i iff j <= i.

    Reading of the pages' causal mask (Slovak page, section 5; ``is_causal``
    in its section 6): top-left aligned, so row i sees keys 0..i.
    """
    rows = np.asarray(query_rows, dtype=np.int64).reshape(-1, 1)
    cols = np.arange(n_keys, dtype=np.int64).reshape(1, -1)
    return cols <= rows


def _scores(qh: np.ndarray, kh: np.ndarray, scale: float,
            visible: np.ndarray | None) -> np.ndarray:
    """S = scale * Q K^T for one head, with invisible entries set to -inf."""
    s = scale * (qh @ kh.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    return s


def _softmax_rows(s: np.ndarray):
    """Row softmax of S with its log-sum-exp; fully masked rows -> P = 0, LSE = -inf."""
    m = np.max(s, axis=-1, keepdims=True, initial=-np.inf)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe)                  # exp(-inf) = 0 for masked entries
    l = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(dead, 0.0, e / np.where(dead, 1.0, l))
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, l)))
    return p, lse[..., 0]


def attention_probs(q, k, causal: bool, scale: float) -> np.ndarray:
    """P = softmax(scale * Q K^T) with the optional causal mask, [..., Nq, Nk] fp64.

    Materialises the full score matrix (Greek page, problem section: the N x N
    matrix S that standard attention stores).  Leading dims are looped over.
    """
    q64, k64 = _f64(q), _f64(k)
    lead = q64.shape[:-2]
    nq, nk = q64.shape[-2], k64.shape[-2]
    qf = q64.reshape((-1, nq, q64.shape[-1]))
    kf = k64.reshape((-1, nk, k64.shape[-1]))
    out = np.empty((qf.shape[0], nq, nk), dtype=np.float64)
    vis = causal_visible(np.arange(nq), nk) if causal else None
    for i in range(qf.shape[0]):
        out[i], _ = _softmax_rows(_scores(qf[i], kf[i], scale, vis))
    return out.reshape(lead + (nq, nk))


def ref_fwd(q, k, v, causal: bool, scale: float):
    """Forward definition: O = softmax(scale Q K^T [masked]) V and LSE per row.

    Shapes: q [B,H,Nq,d], k and v [B,Hkv,Nk,d] with Hkv dividing H (query head
    h uses K/V head ``kv_head(h, H, Hkv)``) -> O [B,H,Nq,d], LSE [B,H,Nq], both
    float64.  LSE_i = m_i + ln(sum_j exp(S_ij - m_i)) (natural log).
    Source: the displayed formula of the Greek page's problem section; causal
    variant and GQA reading as in the module docstring.
    """
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, nq, _ = q64.shape
    Hkv, nk = k64.shape[1], k64.shape[2]
    o = np.empty(q64.shape[:3] + (v64.shape[-1],), dtype=np.float64)
    lse = np.empty((B, H, nq), dtype=np.float64)
    vis = causal_visible(np.arange(nq), nk) if causal else None
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            p, lse[b, h] = _softmax_rows(_scores(q64[b, h], k64[b, g], scale, vis))
            o[b, h] = p @ v64[b, g]
    return o, lse


def ref_fwd_rows(q, k, v, causal: bool, scale: float, rows):
    """Forward definition evaluated only for the query rows ``rows``.

    Same result as ``ref_fwd(...)[..., rows, :]`` (each output row depends only
    on its own query row and on all keys/values), but costs O(len(rows) * N)
    per head, which makes sampled checks at N = 16384 affordable.
    Returns O [B,H,R,d] and LSE [B,H,R] in float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    q64 = _f64(np.asarray(q)[:, :, rows, :])
    k64, v64 = _f64(k), _f64(v)
    B, H = q64.shape[:2]
    Hkv, nk = k64.shape[1], k64.shape[2]
    vis = causal_visible(rows, nk) if causal else None
    o = np.empty((B, H, rows.size, v64.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, rows.size), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            p, lse[b, h] = _softmax_rows(_scores(q64[b, h], k64[b, g], scale, vis))
            o[b, h] = p @ v64[b, g]
    return o, lse


def ref_fwd_tiled(q, k, v, causal: bool, scale: float, br: int, bc: int):
    """The pages' blockwise algorithm, written out step by step (fp64).

    Q is cut into row blocks of ``br`` rows and K/V into blocks of ``bc`` keys
    (tiling).  For every query block the key blocks are visited in order; per
    row a running maximum m, a running sum of exponentials l and an unnormalised
    output acc are kept (the "two intermediate values" of the Greek page's
    online-softmax section, plus the output being updated block by block as its
    tiling section describes).  For each key block:

        m_new = max(m, rowmax(S_blk))
        alpha = exp(m - m_new)          # rescales what was accumulated so far
        p     = exp(S_blk - m_new)
        l     = alpha * l + rowsum(p)
        acc   = alpha * acc + p V_blk

    At the end O = acc / l and LSE = m + ln l.  Used only to show, by brute
    force on tiny inputs, that the tiled method equals the definition.
    """
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, nq, _ = q64.shape
    Hkv, nk = k64.shape[1], k64.shape[2]
    dv = v64.shape[-1]
    o = np.zeros((B, H, nq, dv), dtype=np.float64)
    lse = np.full((B, H, nq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            for r0 in range(0, nq, br):
                r1 = min(nq, r0 + br)
                rows = np.arange(r0, r1)
                m = np.full(r1 - r0, -np.inf)
                l = np.zeros(r1 - r0)
                acc = np.zeros((r1 - r0, dv))
                for c0 in range(0, nk, bc):
                    c1 = min(nk, c0 + bc)
                    s = scale * (q64[b, h, r0:r1] @ k64[b, g, c0:c1].T)
                    if causal:
                        vis = np.arange(c0, c1)[None, :] <= rows[:, None]
                        s = np.where(vis, s, -np.inf)
                    m_new = np.maximum(m, np.max(s, axis=1))
                    # rows with nothing visible yet keep m = -inf; use 0 as the
                    # reference point so that exp(-inf - (-inf)) never appears
                    ref = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                    p = np.exp(s - ref[:, None])
                    l = alpha * l + np.sum(p, axis=1)
                    acc = alpha[:, None] * acc + p @ v64[b, g, c0:c1]
                    m = m_new
                live = l > 0
                o[b, h, r0:r1] = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse


def ref_bwd(q, k, v, do, causal: bool, scale: float, return_ds: bool = False):
    """Gradients of O = softmax(scale Q K^T [masked]) V by the plain chain rule.

    The pages give no gradient formulas (they only say that backward recomputes
    the scores instead of storing them: datacamp "Recomputation", Slovak page
    section 2), so this is ordinary calculus through ``ref_fwd``'s definition,
    with the row-softmax Jacobian diag(p) - p p^T, using the oracle's own fp64
    P and O:

        dV = P^T dO
        dP = dO V^T
        D_i = sum_k dO_ik O_ik        (= sum_j P_ij dP_ij)
        dS = P * (dP - D 1^T)
        dQ = scale dS K,  dK = scale dS^T Q

    Shapes: q, do [B,H,N,d]; k, v [B,Hkv,N,d] (GQA reading of the module
    docstring: a K/V head's dK and dV sum the contributions of the query heads
    that use it); float64 out.  With ``return_ds`` the per-query-head dS
    [B,H,Nq,Nk] is returned as a fourth value (used by invariant tests).
    """
    q64, k64, v64, do64 = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, nq, _ = q64.shape
    Hkv, nk = k64.shape[1], k64.shape[2]
    dq = np.empty_like(q64)
    dk = np.zeros_like(k64)
    dvv = np.zeros_like(v64)
    ds_all = np.empty((B, H, nq, nk)) if return_ds else None
    vis = causal_visible(np.arange(nq), nk) if causal else None
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            p, _ = _softmax_rows(_scores(q64[b, h], k64[b, g], scale, vis))
            o = p @ v64[b, g]
            dvv[b, g] += p.T @ do64[b, h]
            dp = do64[b, h] @ v64[b, g].T
            dd = np.sum(do64[b, h] * o, axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[b, h] = scale * (ds @ k64[b, g])
            dk[b, g] += scale * (ds.T @ q64[b, h])
            if return_ds:
                ds_all[b, h] = ds
    if return_ds:
        return dq, dk, dvv, ds_all
    return dq, dk, dvv


def ref_decode(q, k_cache, v_cache, scale: float):
    """One decode step against a KV cache: the forward definition with one query.

    q [B,H,1,d]; k_cache, v_cache [B,Hkv,L,d] (all cached keys visible, no
    mask; query head h reads cache head h // (H / Hkv)) -> O [B,H,1,d] and
    LSE [B,H] in float64.  The KV cache is the one the
    attention-backend page describes for generation; the decode result is the
    same softmax(q K^T * scale) V over the L cached tokens.
    """
    o, lse = ref_fwd(q, k_cache, v_cache, causal=False, scale=scale)
    return o, lse[:, :, 0]


def ref_decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: float):
    """Decode step against a paged KV cache.

    The attention-backend page (sections "Wat is het precies?" and "Voorbeelden
    uit de praktijk", PagedAttention) describes cutting the KV cache into small
    blocks allocated from a pool instead of one contiguous reservation, with the
    same mathematical result.  Reading used here: the pool holds P pages of
    ``page_size`` tokens per K/V head, k_pool and v_pool [P, Hkv, page_size, d];
    sequence b owns the pages block_table[b, 0], block_table[b, 1], ... in
    token order, and its first seq_lens[b] tokens are its cache.  The result is
    ``ref_decode`` over that token sequence.  A sequence of length 0 gets
    O = 0 and LSE = -inf (the fully-masked convention).

    q [B,H,1,d] -> O [B,H,1,d], LSE [B,H] in float64.
    """
    q64 = _f64(q)
    kp, vp = _f64(k_pool), _f64(v_pool)
    bt = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B, H, _, d = q64.shape
    Hkv, ps = kp.shape[1], kp.shape[2]
    o = np.zeros((B, H, 1, vp.shape[-1]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n_tok = int(lens[b])
        n_pg = -(-n_tok // ps)
        pages = bt[b, :n_pg]
        # gather the sequence's pages in order: [Hkv, n_pg * ps, d], then cut to its length
        kb = np.concatenate([kp[p] for p in pages], axis=1)[:, :n_tok] if n_pg else np.zeros((Hkv, 0, d))
        vb = np.concatenate([vp[p] for p in pages], axis=1)[:, :n_tok] if n_pg else np.zeros((Hkv, 0, d))
        ob, lb = ref_fwd(q64[b:b + 1], kb[None], vb[None], causal=False, scale=scale)
        o[b], lse[b] = ob[0], lb[0, :, 0]
    return o, lse


def ref_merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key subsets by their LSEs.

    o_parts [..., S, d] are the normalised outputs over S disjoint key subsets
    and lse_parts [..., S] their log-sum-exps.  This is the online-softmax
    rescaling (Slovak page section 2; Greek page "Online υπολογισμός Softmax")
    applied to whole subsets:

        M   = max_s lse_s
        lse = M + ln sum_s exp(lse_s - M)
        O   = sum_s exp(lse_s - lse) o_s

    Subsets that saw no key carry lse = -inf and weight 0.
    """
    o64, l64 = _f64(o_parts), _f64(lse_parts)
    M = np.max(l64, axis=-1, keepdims=True)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(l64 - M_safe)
    tot = np.sum(w, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, M_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
        wn = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    o = np.sum(wn[..., None] * o64, axis=-2)
    return o, lse[..., 0]
