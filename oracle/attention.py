"""Dense attention oracle (float64).  Test infrastructure only.

Definition followed, for sequence b of a packed batch (query rows
[cq_b, cq_{b+1}), key rows [ck_b, ck_{b+1}), lengths L_q, L_k), query head h
and its key/value head g = h // (Hq / Hkv):

    s_ij = scale * sum_c q[i,h,c] k[j,g,c]
    allowed(i, j) = True                       (non-causal)
                  = j <= i + (L_k - L_q)       (causal, bottom-right aligned)
    m_i = max_{allowed} s_ij,   l_i = sum_{allowed} exp(s_ij - m_i)
    o_i = sum_{allowed} exp(s_ij - m_i) / l_i * v[j,g,:],   lse_i = m_i + ln l_i
    a row with no allowed key gives o_i = 0, lse_i = -inf.

Sources:
* query pieces computed one after another, S -> softmax -> P V, rows mapped
  back to their global index: [3090] section 三 (fix table and the sentence
  after it).  The piece split never changes the values, so the oracle does
  not split.
* masked keys are excluded (weight exactly zero), not given a finite bias:
  [MI250] sections 3.3 and 6.2.
* variable-length batches through cu_seqlens_q / cu_seqlens_k, each sequence
  bounded by its own key length: [SGLang] sections 2.2 and 3.2.
* the per-row log-sum-exp output ("softmax_lse"): [SGLang] section 3.2.
* the blockwise online merge reaches this same value: [V32] section
  进一步探索, eq. (1)(2).

The computation is organised per (sequence, head, block of query rows) only to
bound memory and to let independent units run on several host threads
(``workers``); every row is evaluated by the definition above on its own.  A
block of a causal sequence forms its logits only over the keys some row of
the block may see (keys past the block's last allowed key are masked for every
row, so leaving them out changes no value).
"""
from __future__ import annotations

import numpy as np

from oracle.pool import run_units

__all__ = ["attention", "attn_probs", "allowed_key_count", "kv_head", "attention_paged"]


def kv_head(h: int, num_heads_q: int, num_heads_kv: int) -> int:
    """Key/value head of query head h: contiguous groups of Hq/Hkv query heads
    share one key/value head (grouped-query attention)."""
    return h // (num_heads_q // num_heads_kv)


def masked_softmax_stats(logits: np.ndarray, mask: np.ndarray):
    """Two-pass softmax statistics of rows that have at least one allowed key.

    Returns (e, m, l): e = exp(logits - m) on allowed entries and 0 elsewhere,
    m = row max over allowed entries, l = row sum of e.
    """
    lg = np.where(mask, logits, -np.inf)
    m = lg.max(axis=1)                                   # pass 1: row max
    e = np.where(mask, np.exp(lg - m[:, None]), 0.0)
    return e, m, e.sum(axis=1)                           # pass 2: row sum


def finish_rows(e: np.ndarray, m: np.ndarray, l_sum: np.ndarray, vv: np.ndarray):
    """o = (e V) / l and lse = m + ln l for rows with allowed keys."""
    return (e @ vv) / l_sum[:, None], m + np.log(l_sum)


def allowed_key_count(i_local: np.ndarray, len_q: int, len_k: int, causal: bool) -> np.ndarray:
    """Number of keys query row ``i_local`` (0-based inside its sequence) may attend to.

    Causal alignment is bottom-right: the queries are the last L_q positions of
    the L_k keys, so row i sees keys 0 .. i + (L_k - L_q).
    """
    i_local = np.asarray(i_local, dtype=np.int64)
    if not causal:
        return np.full(i_local.shape, len_k, dtype=np.int64)
    return np.clip(i_local + (len_k - len_q) + 1, 0, len_k)


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _rows_of_seq(rows_global: np.ndarray, cq: np.ndarray, b: int) -> np.ndarray:
    lo, hi = int(cq[b]), int(cq[b + 1])
    return rows_global[(rows_global >= lo) & (rows_global < hi)]


def attention(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool, scale: float,
              rows=None, heads=None, row_block: int = 512, workers: int = 1):
    """Plain float64 attention over a packed variable-length batch.

    Args:
      q: [total_q, Hq, d];  k: [total_k, Hkv, d];  v: [total_k, Hkv, d_v]
         (any real dtype; converted to float64 exactly).
      cu_seqlens_q, cu_seqlens_k: int [B+1] prefix offsets, cu[0] = 0.
      causal: bottom-right causal mask when True.
      scale: logit scale (a float32 value passed to a kernel is represented
         exactly as a float64 here).
      rows: optional 1-D array of global query rows to evaluate (others are
         left as NaN in ``out`` and ``lse``); None = all rows.
      heads: optional list of query heads to evaluate; None = all.
      row_block: rows evaluated together (memory bound only; long key ranges
         use smaller blocks so one block's logits stay near 2^24 values).
      workers: host threads evaluating (sequence, head, row block) units.

    Returns:
      out [total_q, Hq, d_v] float64, lse [Hq, total_q] float64 (natural log).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    total_q, hq, d = q.shape
    hkv = k.shape[1]
    dv = v.shape[2]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    scale = float(scale)
    all_rows = np.arange(total_q, dtype=np.int64) if rows is None else np.unique(np.asarray(rows, np.int64))
    head_list = range(hq) if heads is None else list(heads)

    fill = 0.0 if rows is None and heads is None else np.nan
    out = np.full((total_q, hq, dv), fill, dtype=np.float64)
    lse = np.full((hq, total_q), fill, dtype=np.float64)

    units = []
    for b in range(len(cq) - 1):
        len_k = int(ck[b + 1] - ck[b])
        sel = _rows_of_seq(all_rows, cq, b)
        blk = max(16, min(row_block, (1 << 24) // max(len_k, 1)))
        for h in head_list:
            for s in range(0, sel.size, blk):
                units.append((b, h, sel[s:s + blk]))

    def unit(u):
        b, h, r = u
        q0, k0 = int(cq[b]), int(ck[b])
        len_q, len_k = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        g = kv_head(h, hq, hkv)
        il = r - q0                                  # local row indices
        n_allowed = allowed_key_count(il, len_q, len_k, causal)
        nk = int(n_allowed.max()) if n_allowed.size else 0   # keys some row of the block sees
        kk = k[k0:k0 + nk, g, :]                     # [nk, d]
        vv = v[k0:k0 + nk, g, :]                     # [nk, d_v]
        o_blk = np.zeros((r.size, dv))
        lse_blk = np.full(r.size, -np.inf)
        has = n_allowed > 0
        if has.any():
            logits = scale * (q[r[has], h, :] @ kk.T)        # [n, nk]
            mask = np.arange(nk)[None, :] < n_allowed[has][:, None]
            e, m, l_sum = masked_softmax_stats(logits, mask)
            o_blk[has], lse_blk[has] = finish_rows(e, m, l_sum, vv)
        out[r, h, :] = o_blk
        lse[h, r] = lse_blk

    run_units(unit, units, workers)
    return out, lse


def attn_probs(q, k, cu_seqlens_q, cu_seqlens_k, causal: bool, scale: float, head: int,
               seq: int, q0: int, rows: int, num_heads_kv: int = None):
    """Probability matrix P of one query piece of one head (float64).

    P[r, j] = exp(s_ij - m_i) / l_i for the piece's local rows
    i = q0 .. q0 + rows - 1 of sequence ``seq``, over that sequence's keys
    j = 0 .. L_k - 1; masked entries are 0, a row with no key is all zeros.

    The piece is returned starting at its own row 0 — the piece-local
    addressing fix of [3090] section 三 (S/P buffers indexed from the piece
    base, not from q0 * N).
    """
    q, k = _as64(q), _as64(k)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    hq = q.shape[1]
    hkv = k.shape[1] if num_heads_kv is None else num_heads_kv
    g = kv_head(head, hq, hkv)
    len_q, len_k = int(cq[seq + 1] - cq[seq]), int(ck[seq + 1] - ck[seq])
    if not (0 <= q0 and q0 + rows <= len_q):
        raise ValueError("piece outside its sequence")
    r = np.arange(q0, q0 + rows) + int(cq[seq])
    kk = k[int(ck[seq]):int(ck[seq]) + len_k, g, :]
    logits = float(scale) * (q[r, head, :] @ kk.T)
    n_allowed = allowed_key_count(np.arange(q0, q0 + rows), len_q, len_k, causal)
    mask = np.arange(len_k)[None, :] < n_allowed[:, None]
    p = np.zeros((rows, len_k))
    has = n_allowed > 0
    if has.any():
        e, _, l_sum = masked_softmax_stats(logits[has], mask[has])
        p[has] = e / l_sum[:, None]
    return p


def attention_paged(q, k_cache, v_cache, block_table, page_size: int, cu_seqlens_q, cu_seqlens_k, causal: bool,
                    scale: float, rows=None, heads=None):
    """attention() over paged K/V caches: sequence b's key position j is token
    row block_table[b, j // page_size] * page_size + j % page_size of
    k_cache / v_cache ([num_pages * page_size, Hkv, d]); cu_seqlens_k gives
    the key lengths.  The logical K/V of every sequence are gathered and
    packed, then the plain definition applies."""
    from oracle.paging import paged_rows
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    idx = [paged_rows(bt[b], page_size, int(ck[b + 1] - ck[b])) for b in range(len(ck) - 1)]
    idx = np.concatenate(idx) if idx else np.zeros(0, np.int64)
    kc, vc = np.asarray(k_cache), np.asarray(v_cache)
    return attention(q, kc[idx], vc[idx], cu_seqlens_q, cu_seqlens_k, causal, scale, rows=rows, heads=heads)
