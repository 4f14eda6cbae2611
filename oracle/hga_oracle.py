"""Plain CPU oracle of Hierarchical Global Attention (HGA) routed attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library never routes through it, and the two share no code: this file imports
numpy and nothing else of this repository.

Everything is float64 on the exactly representable (bf16- or fp32-rounded)
inputs.  The steps follow the method as the pages state it:

* HGA technical summary, Italian page (gist.science/it/paper/2606.30709),
  section "Meccanismo Core", items 1-4, and section "Architettura della Memoria";
* the same paper's French page (gist.science/fr/paper/2606.30709), section
  "Mécanisme Central", which restates the same four items.

Below these are cited as [HGA-it, Meccanismo Core, item N] and
[HGA-fr, Mécanisme Central, ...].

Where the pages leave a step open, the plainest reading consistent with the rest
is taken; each such reading is marked "Reading:" at the place it is used:

* Q and K arrive post-RoPE (as a RoPE'd cache holds them); the raw projected key
  is reached by exact de-rotation.  ``k_is_rotated=False`` takes raw keys.
* RoPE pairs are half-split, pair i = (x[i], x[i + d/2]), theta_i = base^(-2i/d).
* A pair is high-frequency iff theta_i * C > tau (tau = 1 rad by default); the
  same set of pairs is used for chunk and for group summaries.
* The representative position of a span [a, a+L) is its centre a + (L-1)/2.
* A summary is a plain mean (no normalisation).
* The score of a chunk or group is the max over the routing unit's query
  vectors of q.s / sqrt(d).  One routing unit per (batch, KV head, query chunk)
  in prefill and per (batch, KV head) in decode; the max runs over all query
  heads that share the KV head.
* Candidates for chunk routing are the intermediate chunks [n_sink, j - n_local);
  sink, local and current chunks are always visible and never routed.
* Group routing looks only at the groups of routed chunks.
* Ties go to the lower index; index lists are ascending and padded with -1.
* Fewer candidates than k (or groups than g): all of them are taken.
* Decode: the query sits at position seq_len - 1, whose K/V is already cached.
* NaN scores rank below every number (as -inf, then by index).

Parity unpinned: the readings of the pair layout, the RoPE base of the decode
workloads, the representative position and the GQA max-aggregation are choices
with no external value to check them against; they are pinned only for
internal consistency (the literal and relative summary forms agree, closed forms
for one-token spans and constant keys hold).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# --------------------------------------------------------------------------- #
# parameters
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class HGAConfig:
    """Method parameters [HGA-it, Meccanismo Core, items 1-3]."""

    head_dim: int
    chunk_size: int          # C
    group_size: int          # G, divides C
    n_sink: int              # sink chunks, always visible
    n_local: int             # recent chunks before the current one, always visible
    top_k: int               # routed chunks per unit
    top_g: int               # routed groups per unit
    rope_base: float = 10000.0
    hf_threshold: float = 1.0  # radians; pair i is high-frequency iff theta_i*C > this

    @property
    def groups_per_chunk(self) -> int:
        return self.chunk_size // self.group_size


def rope_thetas(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d), i < d/2 (standard RoPE frequencies)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def high_freq_pairs(cfg: HGAConfig) -> np.ndarray:
    """Boolean mask over RoPE pairs: high-frequency iff theta_i * C > tau.

    [HGA-it, Meccanismo Core, item 3] splits pairs into high- and low-frequency
    ones without a numeric rule; Reading: the pair turns by more than tau radians
    across one chunk.
    """
    return rope_thetas(cfg.head_dim, cfg.rope_base) * cfg.chunk_size > cfg.hf_threshold


def rotate_pairs(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Rotate every half-split pair (x_i, x_{i+d/2}) of x[..., d] by phi[..., d/2]."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = np.cos(phi), np.sin(phi)
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# --------------------------------------------------------------------------- #
# step 1: RoPE-aware chunk / group key summaries
# --------------------------------------------------------------------------- #
def span_summary_literal(k_raw: np.ndarray, start: int, cfg: HGAConfig) -> np.ndarray:
    """Summary of one span of RAW (un-rotated) keys k_raw[L, d] starting at ``start``.

    [HGA-it, Meccanismo Core, item 3]: high-frequency pairs are rotated per
    token (to the token's own position) before the mean; low-frequency pairs are
    averaged in raw key space and the mean is rotated to the span's
    representative position.
    """
    L = k_raw.shape[0]
    th = rope_thetas(cfg.head_dim, cfg.rope_base)
    hf = high_freq_pairs(cfg)
    t = start + np.arange(L, dtype=np.float64)
    per_token = rotate_pairs(k_raw, np.outer(t, th)).mean(axis=0)
    p_rep = start + (L - 1) / 2.0
    pooled = rotate_pairs(k_raw.mean(axis=0), th * p_rep)
    mask = np.concatenate([hf, hf])
    return np.where(mask, per_token, pooled)


def span_summary_relative(k_rot: np.ndarray, start: int, cfg: HGAConfig) -> np.ndarray:
    """Same summary computed from POST-RoPE keys k_rot[L, d].

    Rotations of one pair compose additively, so the literal form equals:
    high-frequency pairs -> plain mean of the rotated keys; low-frequency pairs
    -> mean of each rotated key turned by theta_i * (p_rep - t).  Only angles of
    at most theta_i*(L-1)/2 appear.
    """
    L = k_rot.shape[0]
    th = rope_thetas(cfg.head_dim, cfg.rope_base)
    hf = high_freq_pairs(cfg)
    t = start + np.arange(L, dtype=np.float64)
    p_rep = start + (L - 1) / 2.0
    rel = rotate_pairs(k_rot, np.outer(p_rep - t, th)).mean(axis=0)
    mask = np.concatenate([hf, hf])
    return np.where(mask, k_rot.mean(axis=0), rel)


def apply_rope(x: np.ndarray, positions: np.ndarray, cfg: HGAConfig) -> np.ndarray:
    """x[..., L, d] at positions[L] -> RoPE'd copy (half-split pairs)."""
    th = rope_thetas(cfg.head_dim, cfg.rope_base)
    return rotate_pairs(x, np.outer(np.asarray(positions, dtype=np.float64), th))


def build_summaries(K, cfg: HGAConfig, n_tokens: int | None = None,
                    k_is_rotated: bool = True, form: str = "relative"):
    """Chunk and group summaries for every COMPLETE chunk of K[B, H, n, d].

    Returns (chunk_sum[B, H, nC, d], group_sum[B, H, nC*m, d]) in float64 where
    nC = n_tokens // C.  Groups are the m = C/G sub-spans of each chunk
    [HGA-it, Meccanismo Core, item 1].  A partial chunk is never a routing
    candidate, so it gets no summary.
    """
    K = np.asarray(K)
    B, H, n, d = K.shape
    n = n if n_tokens is None else n_tokens
    C, G = cfg.chunk_size, cfg.group_size
    nC, m = n // C, C // G
    cs = np.zeros((B, H, nC, d))
    gs = np.zeros((B, H, nC * m, d))
    for b in range(B):
        for h in range(H):
            kk = K[b, h, : nC * C].astype(np.float64)
            if form == "relative":
                if not k_is_rotated:
                    kk = apply_rope(kk, np.arange(nC * C), cfg)
                f = span_summary_relative
            elif form == "literal":
                if k_is_rotated:  # de-rotate to raw key space, exactly
                    kk = apply_rope(kk, -np.arange(nC * C, dtype=np.float64), cfg)
                f = span_summary_literal
            else:
                raise ValueError(form)
            for c in range(nC):
                cs[b, h, c] = f(kk[c * C:(c + 1) * C], c * C, cfg)
            for g in range(nC * m):
                gs[b, h, g] = f(kk[g * G:(g + 1) * G], g * G, cfg)
    return cs, gs


# --------------------------------------------------------------------------- #
# steps 2-3: two-level routing
# --------------------------------------------------------------------------- #
def select_top(scores: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """First min(k, n) ids under (score descending, id ascending), returned ascending.

    NaN scores count as -inf.
    """
    s = np.where(np.isnan(scores), -np.inf, scores)
    order = np.lexsort((ids, -s))  # primary: -score, secondary: id
    return np.sort(ids[order[: min(k, len(ids))]])


def boundary_gap(scores: np.ndarray, k: int) -> float:
    """Relative gap between the k-th and (k+1)-th best scores; inf if no boundary."""
    if k <= 0 or len(scores) <= k:
        return math.inf
    s = np.sort(np.where(np.isnan(scores), -np.inf, scores))[::-1]
    hi, lo = s[k - 1], s[k]
    den = max(abs(hi), abs(lo))
    if den == 0.0:
        return 0.0
    return float((hi - lo) / den)


def chunk_candidates(j: int, cfg: HGAConfig) -> np.ndarray:
    """Content-routed candidates of query chunk j: [n_sink, j - n_local).

    [HGA-it, Meccanismo Core, item 2] and the key contribution "Policy di
    Routing a Due Livelli": content retrieval works on the intermediate context;
    sink and local chunks are visible by rule.
    """
    lo, hi = cfg.n_sink, j - cfg.n_local
    return np.arange(lo, max(lo, hi), dtype=np.int64)


def route_unit(Uq: np.ndarray, chunk_sum: np.ndarray, group_sum: np.ndarray,
               j: int, cfg: HGAConfig):
    """Route one unit: query vectors Uq[nu, d] of query chunk j (one KV head).

    Level 1 [HGA-it, Meccanismo Core, item 2, first bullet]: score every
    candidate chunk summary, keep the top-k.  Level 2 (second bullet): score the
    group summaries inside the kept chunks, keep the top-g.
    Returns (chunk ids ascending, group ids ascending, diagnostics dict).
    """
    d = Uq.shape[-1]
    scale = 1.0 / math.sqrt(d)
    m = cfg.groups_per_chunk
    cand = chunk_candidates(j, cfg)
    if len(cand):
        sc = (Uq @ chunk_sum[cand].T).max(axis=0) * scale
    else:
        sc = np.zeros(0)
    R = select_top(sc, cand, cfg.top_k)
    gids = (R[:, None] * m + np.arange(m)[None, :]).reshape(-1)
    if len(gids):
        gsc = (Uq @ group_sum[gids].T).max(axis=0) * scale
    else:
        gsc = np.zeros(0)
    Gsel = select_top(gsc, gids, cfg.top_g)
    diag = {
        "chunk_scores": sc, "chunk_cand": cand, "group_scores": gsc, "group_cand": gids,
        "chunk_gap": boundary_gap(sc, cfg.top_k), "group_gap": boundary_gap(gsc, cfg.top_g),
    }
    return R, Gsel, diag


def _pad(ids: np.ndarray, n: int) -> np.ndarray:
    out = np.full(n, -1, dtype=np.int32)
    out[: len(ids)] = ids
    return out


def route(Q, q_pos, chunk_sum, group_sum, cfg: HGAConfig, n_kv_heads: int,
          units: list | None = None):
    """Route every unit of Q[B, Hq, nq, d].

    Prefill (nq > 1): nq is a multiple of C and q_pos[b] is C-aligned; unit u of
    batch b is query chunk q_pos[b]/C + u with query vectors = all g_q*C rows of
    the KV head's query heads in that chunk.  Decode (nq == 1): one unit, chunk
    floor(q_pos[b]/C), query vectors = the g_q heads' rows.
    Returns chunk_idx[B, Hkv, nU, k], group_idx[B, Hkv, nU, g] (int32, -1 padded)
    and a dict of diagnostics keyed by (b, h, u).  ``units`` restricts work to a
    list of (b, h, u) triples (other entries stay -1).
    """
    Q = np.asarray(Q)
    B, Hq, nq, d = Q.shape
    gq = Hq // n_kv_heads
    C = cfg.chunk_size
    nU = 1 if nq == 1 else nq // C
    ci = np.full((B, n_kv_heads, nU, max(cfg.top_k, 0)), -1, dtype=np.int32)
    gi = np.full((B, n_kv_heads, nU, max(cfg.top_g, 0)), -1, dtype=np.int32)
    diags = {}
    todo = units if units is not None else [(b, h, u) for b in range(B)
                                            for h in range(n_kv_heads) for u in range(nU)]
    for (b, h, u) in todo:
        if nq == 1:
            j = int(q_pos[b]) // C
            Uq = Q[b, h * gq:(h + 1) * gq, 0].astype(np.float64)
        else:
            j = int(q_pos[b]) // C + u
            Uq = Q[b, h * gq:(h + 1) * gq, u * C:(u + 1) * C].astype(np.float64).reshape(-1, d)
        R, Gs, dg = route_unit(Uq, np.asarray(chunk_sum[b, h], dtype=np.float64),
                               np.asarray(group_sum[b, h], dtype=np.float64), j, cfg)
        ci[b, h, u] = _pad(R, cfg.top_k)
        gi[b, h, u] = _pad(Gs, cfg.top_g)
        diags[(b, h, u)] = dg
    return ci, gi, diags


# --------------------------------------------------------------------------- #
# step 4: deterministic visibility
# --------------------------------------------------------------------------- #
def forced_chunks(j: int, cfg: HGAConfig) -> np.ndarray:
    """Always-visible chunks of query chunk j: sink, recent local, current.

    [HGA-it, Meccanismo Core, item 2, third bullet].  Reading: the n_local chunks
    right before j, plus j itself; overlaps early in the sequence count once.
    """
    s = set(range(min(cfg.n_sink, j + 1))) | set(range(max(0, j - cfg.n_local), j + 1))
    return np.array(sorted(s), dtype=np.int64)


def visible_tokens(t: int, group_ids: np.ndarray, cfg: HGAConfig) -> np.ndarray:
    """Exact token set T(t) of a query at position t (ascending).

    The union, as a set, of the forced chunks' tokens and the listed groups'
    tokens, keeping only tokens u <= t.  Reading: the causal mask applies to
    every visible token; it only bites in the current chunk for lists that
    routing produced (their groups lie before the local window), and it drops
    any later group of a list given by a caller.  Negative ids are holes.
    """
    C, G = cfg.chunk_size, cfg.group_size
    j = t // C
    parts = [np.arange(c * C, c * C + C) for c in forced_chunks(j, cfg)]
    toks = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    g = np.asarray(group_ids)
    g = g[g >= 0]
    if len(g):
        toks = np.concatenate([toks, (g[:, None] * G + np.arange(G)[None, :]).reshape(-1)])
    toks = np.unique(toks)
    return toks[toks <= t]


# --------------------------------------------------------------------------- #
# step 5: exact token-level softmax attention
# --------------------------------------------------------------------------- #
def softmax_attend(q: np.ndarray, Kt: np.ndarray, Vt: np.ndarray):
    """o = sum_u softmax(q.k_u / sqrt(d)) v_u over the given rows; returns (o, lse).

    [HGA-it, Meccanismo Core, item 4]: standard softmax over the bounded exact
    token set, original K/V only.
    """
    d = q.shape[-1]
    z = (Kt @ q) / math.sqrt(d)
    zmax = z.max()
    w = np.exp(z - zmax)
    den = w.sum()
    return (w @ Vt) / den, float(zmax + math.log(den))


def attend(Q, q_pos, K, V, group_idx, cfg: HGAConfig, n_kv_heads: int,
           rows: list | None = None):
    """Exact attention of every query row over its visible set.

    Q[B, Hq, nq, d] at positions q_pos[b] + i; K, V[B, Hkv, n_cap, d];
    group_idx[B, Hkv, nU, g] as produced by ``route`` (or by any other router:
    this scores a given index set).  Returns O[B, Hq, nq, d] float64 and
    lse[B, Hq, nq].  ``rows`` restricts work to (b, hq, i) triples.
    """
    Q = np.asarray(Q)
    B, Hq, nq, d = Q.shape
    gq = Hq // n_kv_heads
    C = cfg.chunk_size
    O = np.zeros((B, Hq, nq, d))
    lse = np.zeros((B, Hq, nq))
    todo = rows if rows is not None else [(b, hq, i) for b in range(B)
                                          for hq in range(Hq) for i in range(nq)]
    for (b, hq, i) in todo:
        h = hq // gq
        t = int(q_pos[b]) + i
        u = 0 if nq == 1 else (t // C - int(q_pos[b]) // C)
        toks = visible_tokens(t, group_idx[b, h, u], cfg)
        o, l = softmax_attend(Q[b, hq, i].astype(np.float64),
                              np.asarray(K[b, h, toks], dtype=np.float64),
                              np.asarray(V[b, h, toks], dtype=np.float64))
        O[b, hq, i] = o
        lse[b, hq, i] = l
    return O, lse


def attend_unit_block(Q, q_pos, K, V, group_idx, cfg: HGAConfig, n_kv_heads: int,
                      b: int, h: int, u: int):
    """Attention for all g_q*C rows of one prefill unit at once (same result as
    ``attend`` on those rows; one matrix product instead of a loop).

    Returns O[g_q, C, d] and lse[g_q, C].
    """
    Q = np.asarray(Q)
    _, Hq, nq, d = Q.shape
    gq = Hq // n_kv_heads
    C = cfg.chunk_size
    t0 = int(q_pos[b]) + u * C
    j = t0 // C
    toks = visible_tokens(t0 + C - 1, group_idx[b, h, u], cfg)
    Kt = np.asarray(K[b, h, toks], dtype=np.float64)
    Vt = np.asarray(V[b, h, toks], dtype=np.float64)
    q = Q[b, h * gq:(h + 1) * gq, u * C:(u + 1) * C].astype(np.float64)  # [gq, C, d]
    z = np.einsum("gcd,td->gct", q, Kt) / math.sqrt(d)
    pos = t0 + np.arange(C)
    z = np.where(toks[None, None, :] <= pos[None, :, None], z, -np.inf)  # causal in chunk j
    zmax = z.max(axis=-1, keepdims=True)
    w = np.exp(z - zmax)
    den = w.sum(axis=-1, keepdims=True)
    assert j == t0 // C
    return (w @ Vt) / den, (zmax + np.log(den))[..., 0]


def attend_backward(Q, q_pos, K, V, group_idx, dO, cfg: HGAConfig, n_kv_heads: int):
    """Gradients of ``attend``'s O with respect to Q, K and V for an upstream
    gradient dO, with the selection held fixed.

    [HGA-it, Meccanismo Core, item 4]: O is an exact softmax over the selected
    tokens.  Reading: routing is a piecewise-constant function of Q and of the
    summaries, so no gradient flows through it; the gradient is that of the
    softmax attention over the fixed token set T(t) of every query row.  For one
    row with scores z_u = q.k_u / sqrt(d), p = softmax(z), o = sum_u p_u v_u:
        dv_u += p_u do;   dp_u = do.v_u;   dz_u = p_u (dp_u - sum_w p_w dp_w);
        dq = sum_u dz_u k_u / sqrt(d);   dk_u += dz_u q / sqrt(d).
    Returns dQ[B, Hq, nq, d], dK and dV[B, Hkv, n_cap, d] (float64).
    """
    Q = np.asarray(Q, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, Hq, nq, d = Q.shape
    gq = Hq // n_kv_heads
    C = cfg.chunk_size
    Kf = np.asarray(K, dtype=np.float64)
    Vf = np.asarray(V, dtype=np.float64)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(Kf)
    dV = np.zeros_like(Vf)
    sc = 1.0 / math.sqrt(d)
    for b in range(B):
        for hq in range(Hq):
            h = hq // gq
            for i in range(nq):
                t = int(q_pos[b]) + i
                u = 0 if nq == 1 else (t // C - int(q_pos[b]) // C)
                toks = visible_tokens(t, group_idx[b, h, u], cfg)
                Kt, Vt = Kf[b, h, toks], Vf[b, h, toks]
                q, do = Q[b, hq, i], dO[b, hq, i]
                z = (Kt @ q) * sc
                p = np.exp(z - z.max())
                p /= p.sum()
                dp = Vt @ do
                dz = p * (dp - p @ dp)
                dQ[b, hq, i] = (dz @ Kt) * sc
                dK[b, h, toks] += np.outer(dz, q) * sc
                dV[b, h, toks] += np.outer(p, do)
    return dQ, dK, dV


# --------------------------------------------------------------------------- #
# warm tier: a bounded LRU of recently routed groups
# --------------------------------------------------------------------------- #
def warm_lru_step(tags, stamps, clock: int, group_ids, n_groups_cap: int):
    """One step of the warm tier of one (batch, KV head) unit.

    [HGA-it, Architettura della Memoria: a bounded LRU cache in device memory
    holds the recently routed chunks; the full K/V history lives in host
    memory.]  Readings:
    * the cached unit is the routed group, the unit the cold tier copies;
    * a step's routed groups are used together (one time stamp per step);
    * a group already cached keeps its slot (a hit; the lowest such slot);
    * the missing groups take the least recently used slots that this step has
      not used: smallest stamp first (an empty slot has stamp 0), the lower slot
      on equal stamps; the j-th missing group in list order gets the j-th of
      those slots in slot order;
    * list entries outside [0, n_groups_cap) are ignored.

    tags[s]: group held by slot s, or -1; stamps[s]: the last step that used it;
    clock: the steps so far.  Requires len(tags) >= the number of valid
    entries.  Returns (slot_of, misses, tags, stamps, clock) after the step:
    slot_of[i] is the slot of entry i (-1 if ignored); misses lists the
    (slot, group) pairs to copy in from host memory, in list order.
    """
    tags = [int(x) for x in tags]
    stamps = [int(x) for x in stamps]
    now = int(clock) + 1
    slot_of = [-1] * len(group_ids)
    pending = []
    for i, g in enumerate(int(x) for x in group_ids):
        if not 0 <= g < n_groups_cap:
            continue
        if g in tags:
            s = tags.index(g)
            slot_of[i] = s
            stamps[s] = now
        else:
            pending.append((i, g))
    # evict: the len(pending) least recently used slots not used by this step
    order = sorted((stamps[s], s) for s in range(len(tags)) if stamps[s] != now)
    victims = sorted(s for _, s in order[:len(pending)])
    assert len(victims) == len(pending), "more groups than slots"
    misses = []
    for (i, g), s in zip(pending, victims):
        tags[s] = g
        stamps[s] = now
        slot_of[i] = s
        misses.append((s, g))
    return slot_of, misses, tags, stamps, now


# --------------------------------------------------------------------------- #
# whole passes
# --------------------------------------------------------------------------- #
def prefill(Q, K, V, cfg: HGAConfig, n_kv_heads: int):
    """Full causal prefill of n tokens (q_pos = 0): summaries, routing, attention."""
    Q = np.asarray(Q)
    B, Hq, n, d = Q.shape
    gq = Hq // n_kv_heads
    cs, gs = build_summaries(K, cfg, n_tokens=n)
    q_pos = np.zeros(B, dtype=np.int64)
    ci, gi, diags = route(Q, q_pos, cs, gs, cfg, n_kv_heads)
    O = np.zeros((B, Hq, n, d))
    lse = np.zeros((B, Hq, n))
    C = cfg.chunk_size
    for b in range(B):
        for h in range(n_kv_heads):
            for u in range(n // C):
                o, l = attend_unit_block(Q, q_pos, K, V, gi, cfg, n_kv_heads, b, h, u)
                O[b, h * gq:(h + 1) * gq, u * C:(u + 1) * C] = o
                lse[b, h * gq:(h + 1) * gq, u * C:(u + 1) * C] = l
    return {"O": O, "lse": lse, "chunk_sum": cs, "group_sum": gs,
            "chunk_idx": ci, "group_idx": gi, "diags": diags}


def decode(Q, K, V, seq_len, chunk_sum, group_sum, cfg: HGAConfig, n_kv_heads: int):
    """One decode step: query b at position seq_len[b]-1 (its K/V already cached).

    chunk_sum/group_sum must hold every candidate chunk (all chunks before
    floor((seq_len-1)/C) - n_local).
    """
    q_pos = np.asarray(seq_len, dtype=np.int64) - 1
    ci, gi, diags = route(Q, q_pos, chunk_sum, group_sum, cfg, n_kv_heads)
    O, lse = attend(Q, q_pos, K, V, gi, cfg, n_kv_heads)
    return {"O": O, "lse": lse, "chunk_idx": ci, "group_idx": gi, "diags": diags}


def dense_causal(Q, K, V, n_kv_heads: int):
    """Dense causal softmax attention (GQA) — the top-k-covers-everything limit."""
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, n, d = Q.shape
    gq = Hq // n_kv_heads
    O = np.zeros_like(Q)
    for b in range(B):
        for hq in range(Hq):
            h = hq // gq
            for t in range(n):
                o, _ = softmax_attend(Q[b, hq, t], np.asarray(K[b, h, : t + 1], np.float64),
                                      np.asarray(V[b, h, : t + 1], np.float64))
                O[b, hq, t] = o
    return O
