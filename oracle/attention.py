"""fp64 oracle for causal / sliding-window GQA softmax attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
-------
* Scaled dot-product softmax attention: weights are the softmax over keys of
  ``q_i . k_j`` times a scale, and the output is the weighted sum of values
  [vinija.ai Gemma 4 primer, "Why long context is difficult" (attention
  equation) and "Sliding-window attention" (alpha_ij equation)].  The scale
  is an argument: the primer uses ``1/sqrt(d_k)``, while the PyTorch port
  says QK-norm replaces that factor [gemma4-pt-claude README, "Key
  architectural features"].
* Sliding-window (local) layers: token ``i`` attends only to keys in a
  window of size ``w`` ending at ``i`` [vinija.ai Gemma 4 primer, "Local
  attention" and "Sliding-window attention", window equations]; windows are
  512 on E2B/E4B and 1024 on 31B/26B ["Window sizes by model family"].
* Global layers: every earlier key is visible, and the layer stays causal
  [vinija.ai Gemma 4 primer, "Global attention layers"; Gemma 4 Keras docs,
  "What changed from Gemma 3" (causal masking kept on global layers)].
* GQA: several query heads share one key/value head [Gemma 4 Keras docs,
  ``Gemma4Model`` table, ``num_kv_heads``; gemma4-pt-claude README,
  "Supported Models"].
* Decode over a KV cache: the new query attends over the stored keys and
  values of every earlier token [vinija.ai Gemma 4 primer, "KV cache and
  long-context scaling"; gemma4-pt-claude README, "KV Cache"].
* Image blocks attend bidirectionally within themselves on the
  sliding-window layers [Gemma 4 Keras docs, "What changed from Gemma 3",
  NaViT vision tower, and ``use_bidirectional_vision``]: a row inside an
  image block also sees every key of its block.
* Sliding layers keep a window-sized cache [gemma4-pt-claude README, "KV
  Cache": sliding-layer caches hold the window, global ones grow]; decoding
  past the window must agree with the uncached forward pass [same page,
  "Tests" list].

Readings where the pages are silent or disagree
-----------------------------------------------
* Window boundary: key ``j`` is visible from row ``i`` iff ``0 <= i - j < w``
  (``w`` keys including the token itself).  The primer's sum runs from
  ``i - w`` (``w + 1`` keys); the PyTorch port keeps ``w`` cache slots per
  sliding layer, which fits ``w`` keys.  ``w = 0`` means global (``j <= i``).
* GQA grouping is contiguous: query head ``h`` uses KV head
  ``h // (Hq // Hkv)``.
* LSE is the natural log of the softmax denominator, ``log sum_j exp(s_ij)``.
* A row with no visible key (never produced by these masks) outputs zeros
  and ``lse = -inf``.
* Decode: the cache holds post-prologue keys and values; the query attends
  over the first ``n_b`` rows of its sequence's cache (``n_b`` includes the
  new token's own slot).
* Rolling cache of a sliding layer: ``w`` slots, position ``p`` stored in
  slot ``p mod w`` (each write replaces the position ``w`` earlier).

Pins (tests/test_oracle_attention.py)
-------------------------------------
* The band oracle against the brute-force explicit-mask oracle on tiny
  shapes across window, GQA and length edges (brute force);
* both against ``torch.nn.functional.scaled_dot_product_attention`` in
  float64 with a mask built from ``torch.tril`` (a library routine), GQA via
  repeated KV heads;
* closed forms: softmax rows sum to 1; visible-key count ``min(i+1, w)``;
  ``w = 1`` gives ``out = v``; ``S <= w`` equals the global result; a
  scale of 0 gives ``lse = log(count)``; decode of the last row equals the
  prefill row.
* Rolling cache: the slot contents after sequential writes against the
  closed form ``p = L - ((L - s) mod w)``; decode over the ring equals the
  sliding prefill's row ``L`` (the uncached forward) for lengths below, at
  and far past the window.
* Chunked prefill over caches equals the rows ``pos0 .. pos0 + qlen - 1``
  of the whole-sequence prefill (the batched/chunked forward equals the
  single one), padded rows stay empty.
* Span masks: degenerate spans give the plain mask; the masked oracle
  against torch SDPA with the same boolean mask; one span over a whole
  global sequence gives unmasked attention; inside a block the mask is all
  true, outside it the window mask.
"""

import numpy as np


def visible(i, j, window):
    """Mask predicate: may query row ``i`` see key ``j``?

    Global (``window == 0``): ``j <= i``.  Sliding: ``0 <= i - j < window``.
    """
    d = i - j
    if window == 0:
        return d >= 0
    return (d >= 0) & (d < window)


def mask_bruteforce(S, window):
    """Explicit ``S x S`` boolean mask built element by element."""
    m = np.zeros((S, S), dtype=bool)
    for i in range(S):
        for j in range(S):
            m[i, j] = bool(visible(i, j, window))
    return m


def _kv_head(h, Hq, Hkv):
    return h // (Hq // Hkv)


def attention_bruteforce(q, k, v, scale, window):
    """Brute-force attention over the full ``S x S`` logit matrix.

    ``q``: ``[B, S, Hq, D]``; ``k``, ``v``: ``[B, S, Hkv, D]`` (any real
    dtype, widened to fp64).  Returns ``(out [B,S,Hq,D], lse [B,Hq,S],
    weights [B,Hq,S,S])``.  For tiny shapes only.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    mask = mask_bruteforce(S, window)
    out = np.zeros((B, S, Hq, D))
    lse = np.full((B, Hq, S), -np.inf)
    weights = np.zeros((B, Hq, S, S))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
            s = np.where(mask, s, -np.inf)
            for i in range(S):
                if not mask[i].any():
                    continue
                mx = np.max(s[i])
                e = np.exp(s[i] - mx)
                den = np.sum(e)
                weights[b, h, i] = e / den
                lse[b, h, i] = mx + np.log(den)
            out[b, :, h, :] = weights[b, h] @ v[b, :, g, :]
    return out, lse, weights


def _band_rows(q_rows, k_band, v_band, rows, key0, scale, window):
    """Softmax attention of the given query rows over one key band."""
    s = scale * (q_rows @ k_band.T)                       # [nr, nk]
    keys = key0 + np.arange(k_band.shape[0])
    m = visible(rows[:, None], keys[None, :], window)
    s = np.where(m, s, -np.inf)
    has = m.any(axis=1)
    mx = np.where(has, np.max(s, axis=1), 0.0)
    e = np.where(m, np.exp(s - mx[:, None]), 0.0)
    den = e.sum(axis=1)
    safe = np.where(has, den, 1.0)
    o = (e @ v_band) / safe[:, None]
    o[~has] = 0.0
    lse = np.where(has, mx + np.log(safe), -np.inf)
    return o, lse


def attention_band(q, k, v, scale, window, rows=None, block=256):
    """Row-blocked attention that only touches keys inside each row's band.

    Same contract as :func:`attention_bruteforce` minus the weights.  If
    ``rows`` (a sorted 1-D array of query rows) is given, only those rows are
    computed and the results have ``len(rows)`` in place of ``S``:
    ``out [B, R, Hq, D]``, ``lse [B, Hq, R]``.
    """
    q = np.asarray(q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = np.zeros((B, R, Hq, D))
    lse = np.full((B, Hq, R), -np.inf)
    for b in range(B):
        for g in range(Hkv):
            heads = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == g]
            for r0 in range(0, R, block):
                rr = rows[r0:r0 + block]
                hi = int(rr[-1]) + 1
                lo = 0 if window == 0 else max(0, int(rr[0]) - window + 1)
                kb = np.asarray(k[b, lo:hi, g, :], np.float64)
                vb = np.asarray(v[b, lo:hi, g, :], np.float64)
                for h in heads:
                    qr = np.asarray(q[b, rr, h, :], np.float64)
                    o, l_ = _band_rows(qr, kb, vb, rr, lo, scale, window)
                    out[b, r0:r0 + block, h, :] = o
                    lse[b, h, r0:r0 + block] = l_
    return out, lse


def decode_attention(q, k_cache, v_cache, n, scale, heads=None, batch=None):
    """Single-token decode: query ``q[b, h]`` over cache rows ``[0, n[b])``.

    ``q``: ``[B, Hq, D]`` (post-prologue); ``k_cache``, ``v_cache``:
    ``[B, Hkv, cap, D]`` (``v_cache`` may be the same array as ``k_cache``);
    ``n``: ``[B]`` visible lengths.  ``batch`` / ``heads`` restrict the work
    to a subset (results are indexed ``[len(batch), len(heads)]``).
    Returns ``(out [B', H', D], lse [B', H'])``.
    """
    Bq, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    batch = list(range(Bq)) if batch is None else list(batch)
    heads = list(range(Hq)) if heads is None else list(heads)
    out = np.zeros((len(batch), len(heads), D))
    lse = np.full((len(batch), len(heads)), -np.inf)
    for bi, b in enumerate(batch):
        nb = int(n[b])
        for hi, h in enumerate(heads):
            g = _kv_head(h, Hq, Hkv)
            if nb <= 0:
                continue
            kk = np.asarray(k_cache[b, g, :nb, :], np.float64)
            vv = kk if v_cache is k_cache else np.asarray(v_cache[b, g, :nb, :], np.float64)
            s = scale * (kk @ np.asarray(q[b, h], np.float64))
            mx = np.max(s)
            e = np.exp(s - mx)
            den = np.sum(e)
            out[bi, hi] = (e @ vv) / den
            lse[bi, hi] = mx + np.log(den)
    return out, lse


def visible_count(S, window, span_lo=None, span_hi=None, block=512):
    """Number of keys each prefill row sees, by enumeration of the mask.

    Every (row, key) pair of the ``S x S`` grid is tested with
    :func:`visible` (and, with spans, the span rule of :func:`mask_spans`),
    a block of rows at a time so that long sequences stay within memory.
    """
    counts = np.zeros(S, dtype=np.int64)
    j = np.arange(S)[None, :]
    for r0 in range(0, S, block):
        i = np.arange(r0, min(S, r0 + block))[:, None]
        m = visible(i, j, window)
        if span_lo is not None:
            lo = np.asarray(span_lo)[r0:r0 + block][:, None]
            hi = np.asarray(span_hi)[r0:r0 + block][:, None]
            m = m | ((j >= lo) & (j <= hi))
        counts[r0:r0 + block] = m.sum(axis=1)
    return counts


def visible_pairs(S, window):
    """Total visible (row, key) pairs of one head: the per-row counts summed."""
    return int(visible_count(S, window).sum())


def ring_positions(n, window):
    """Position held by each slot of a ``window``-slot rolling cache after
    positions ``0 .. n-1`` were written in order (slot ``p mod window``);
    -1 for a slot never written."""
    pos = np.full(window, -1, dtype=np.int64)
    for p in range(int(n)):
        pos[p % window] = p
    return pos


def sliding_decode_ring(q, k_ring, v_ring, n, scale, window):
    """Single-token decode of a sliding layer over rolling caches.

    ``q``: ``[B, Hq, D]`` (the new token at position ``n[b] - 1``);
    ``k_ring``, ``v_ring``: ``[B, Hkv, window, D]`` with position ``p`` in
    slot ``p mod window``; ``n``: ``[B]`` positions so far, the new token
    included.  The query sees the slots whose position ``p`` satisfies
    ``0 <= (n[b] - 1) - p < window``.  Returns ``(out [B, Hq, D], lse [B, Hq])``.
    """
    Bq, Hq, D = q.shape
    Hkv = k_ring.shape[1]
    out = np.zeros((Bq, Hq, D))
    lse = np.full((Bq, Hq), -np.inf)
    for b in range(Bq):
        pos = ring_positions(n[b], window)
        last = int(n[b]) - 1
        vis = [s for s in range(window) if pos[s] >= 0 and visible(last, int(pos[s]), window)]
        if not vis:
            continue
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kk = np.asarray(k_ring[b, g, vis, :], np.float64)
            vv = np.asarray(v_ring[b, g, vis, :], np.float64)
            sc = scale * (kk @ np.asarray(q[b, h], np.float64))
            mx = np.max(sc)
            e = np.exp(sc - mx)
            den = np.sum(e)
            out[b, h] = (e @ vv) / den
            lse[b, h] = mx + np.log(den)
    return out, lse


def prefill_over_cache(q, k_cache, v_cache, pos0, qlen, scale, window):
    """A chunk of new query rows over caches (chunked prefill, padded batches).

    Row ``t < qlen[b]`` of ``q [B, S, Hq, D]`` is position ``p = pos0[b] + t``
    and sees cache rows ``j`` of ``k_cache``/``v_cache [B, Hkv, cap, D]`` with
    :func:`visible` ``(p, j, window)``.  Rows ``t >= qlen[b]`` are padding:
    zeros and ``lse = -inf``.  Returns ``(out [B, S, Hq, D], lse [B, Hq, S])``.
    """
    q = np.asarray(q)
    B, S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((B, S, Hq, D))
    lse = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        for t in range(int(qlen[b])):
            p = int(pos0[b]) + t
            lo = 0 if window == 0 else max(0, p - window + 1)
            for h in range(Hq):
                g = _kv_head(h, Hq, Hkv)
                kk = np.asarray(k_cache[b, g, lo:p + 1, :], np.float64)
                vv = np.asarray(v_cache[b, g, lo:p + 1, :], np.float64)
                sc = scale * (kk @ np.asarray(q[b, t, h], np.float64))
                mx = np.max(sc)
                e = np.exp(sc - mx)
                den = np.sum(e)
                out[b, t, h] = (e @ vv) / den
                lse[b, h, t] = mx + np.log(den)
    return out, lse


def mask_spans(S, window, span_lo, span_hi):
    """Visibility with bidirectional spans: ``visible(i, j, window)`` or
    ``span_lo[i] <= j <= span_hi[i]`` (row ``i``'s own image block; a text
    row has ``span_lo = span_hi = i``)."""
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    lo = np.asarray(span_lo)[:, None]
    hi = np.asarray(span_hi)[:, None]
    return visible(i, j, window) | ((j >= lo) & (j <= hi))


def attention_masked(q, k, v, scale, mask):
    """Brute-force attention under an explicit boolean mask ``[S, S]`` (shared
    by every batch and head).  Returns ``(out [B, S, Hq, D], lse [B, Hq, S])``."""
    q = np.asarray(q, np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    out = np.zeros((B, S, Hq, D))
    lse = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = scale * (q[b, :, h, :] @ np.asarray(k[b, :, g, :], np.float64).T)
            s = np.where(mask, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - np.where(np.isfinite(mx), mx, 0.0))
            den = e.sum(axis=1)
            out[b, :, h, :] = (e @ np.asarray(v[b, :, g, :], np.float64)) / den[:, None]
            lse[b, h, :] = mx[:, 0] + np.log(den)
    return out, lse


def span_rows(S, images):
    """``span_lo``, ``span_hi`` of one sequence whose image blocks are
    ``(start, length)`` pairs; text rows get ``lo = hi = i``."""
    lo = np.arange(S)
    hi = np.arange(S)
    for st, n in images:
        lo[st:st + n] = st
        hi[st:st + n] = st + n - 1
    return lo, hi
