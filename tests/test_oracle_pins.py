"""Pins of the CPU oracle against facts fixed outside it (closed forms, brute force,
library routines, invariants the HGA pages state).  CPU only.

Every check below is written independently of the oracle's own code: rotations
are redone with complex numbers, top-k with Python's ``sorted``, attention with
``torch.nn.functional.scaled_dot_product_attention``.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def cfg(**kw):
    base = dict(head_dim=16, chunk_size=8, group_size=4, n_sink=1, n_local=1, top_k=2,
                top_g=3, rope_base=100.0, hf_threshold=1.0)
    base.update(kw)
    return O.HGAConfig(**base)


def as_complex(x):
    h = x.shape[-1] // 2
    return x[..., :h] + 1j * x[..., h:]


def from_complex(z):
    return np.concatenate([z.real, z.imag], axis=-1)


# --------------------------------------------------------------------------- #
# high-frequency pair split: closed form
# --------------------------------------------------------------------------- #
def test_hf_pair_counts_closed_form():
    gold = json.load(open(GOLD))["hf_pair_counts"]["cases"]
    for c in gold:
        cf = O.HGAConfig(head_dim=c["d"], chunk_size=c["C"], group_size=16, n_sink=1, n_local=1,
                         top_k=1, top_g=1, rope_base=c["base"], hf_threshold=c["tau"])
        hf = O.high_freq_pairs(cf)
        assert int(hf.sum()) == c["count"], c
        # the high-frequency pairs are a prefix (theta decreases with i)
        assert hf[: c["count"]].all()


# --------------------------------------------------------------------------- #
# summaries
# --------------------------------------------------------------------------- #
def _raw_and_rot(rng, L, start, cf):
    d = cf.head_dim
    raw = rng.standard_normal((L, d))
    th = 1.0 / cf.rope_base ** (np.arange(d // 2) * 2.0 / d)
    t = start + np.arange(L)
    rot = from_complex(as_complex(raw) * np.exp(1j * np.outer(t, th)))
    return raw, rot, th


@pytest.mark.parametrize("start,L", [(0, 8), (24, 8), (1000, 4), (77, 5)])
def test_all_pairs_high_freq_gives_mean_of_rotated_keys(start, L):
    """tau = 0 -> every pair high-frequency -> summary = mean of per-token rotated keys."""
    cf = cfg(hf_threshold=0.0)
    rng = np.random.default_rng(1 + start)
    raw, rot, _ = _raw_and_rot(rng, L, start, cf)
    want = rot.mean(axis=0)
    np.testing.assert_allclose(O.span_summary_literal(raw, start, cf), want, atol=1e-12)
    np.testing.assert_allclose(O.span_summary_relative(rot, start, cf), want, atol=1e-12)


@pytest.mark.parametrize("start,L", [(0, 8), (40, 8), (4096, 16)])
def test_all_pairs_low_freq_gives_rotated_raw_mean(start, L):
    """tau huge -> every pair low-frequency -> raw mean rotated to the span centre."""
    cf = cfg(hf_threshold=1e9)
    rng = np.random.default_rng(7 + start)
    raw, rot, th = _raw_and_rot(rng, L, start, cf)
    p = start + (L - 1) / 2
    want = from_complex(as_complex(raw.mean(axis=0)) * np.exp(1j * th * p))
    np.testing.assert_allclose(O.span_summary_literal(raw, start, cf), want, atol=1e-12)
    np.testing.assert_allclose(O.span_summary_relative(rot, start, cf), want, atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 0.5, 1.0, 3.0, 1e9])
def test_single_token_span_is_the_rotated_key(tau):
    cf = cfg(hf_threshold=tau)
    rng = np.random.default_rng(3)
    for start in (0, 5, 12345):
        raw, rot, _ = _raw_and_rot(rng, 1, start, cf)
        np.testing.assert_allclose(O.span_summary_literal(raw, start, cf), rot[0], atol=1e-12)
        np.testing.assert_allclose(O.span_summary_relative(rot, start, cf), rot[0], atol=1e-12)


def test_constant_raw_key_geometric_series():
    """Constant raw key k over [a, a+L): HF pair -> k * mean_t e^{i theta t} (geometric
    series); LF pair -> k * e^{i theta p}."""
    cf = cfg(head_dim=32, chunk_size=16, group_size=4, rope_base=50.0, hf_threshold=1.0)
    rng = np.random.default_rng(11)
    a, L = 48, 16
    k = rng.standard_normal(32)
    raw = np.tile(k, (L, 1))
    th = 1.0 / 50.0 ** (np.arange(16) * 2.0 / 32)
    hf = th * 16 > 1.0
    assert hf.any() and (~hf).any()
    z = np.exp(1j * th)
    geo = np.exp(1j * th * a) * (1 - z ** L) / (L * (1 - z))
    kc = as_complex(k)
    want_c = np.where(hf, kc * geo, kc * np.exp(1j * th * (a + (L - 1) / 2)))
    want = from_complex(want_c)
    rot = from_complex(as_complex(raw) * np.exp(1j * np.outer(a + np.arange(L), th)))
    np.testing.assert_allclose(O.span_summary_literal(raw, a, cf), want, atol=1e-12)
    np.testing.assert_allclose(O.span_summary_relative(rot, a, cf), want, atol=1e-12)


@pytest.mark.parametrize("k_is_rotated", [True, False])
def test_literal_and_relative_forms_agree(k_is_rotated):
    cf = cfg(head_dim=32, chunk_size=16, group_size=4, rope_base=10000.0)
    rng = np.random.default_rng(5)
    K = rng.standard_normal((2, 2, 100, 32))
    a = O.build_summaries(K, cf, k_is_rotated=k_is_rotated, form="literal")
    b = O.build_summaries(K, cf, k_is_rotated=k_is_rotated, form="relative")
    for x, y in zip(a, b):
        assert x.shape == y.shape
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)
    assert a[0].shape == (2, 2, 6, 32) and a[1].shape == (2, 2, 24, 32)


def test_summaries_use_existing_keys_only_and_are_means():
    """A summary is linear in the span's keys and ignores keys outside the span."""
    cf = cfg(head_dim=16, chunk_size=8, group_size=4)
    rng = np.random.default_rng(9)
    K = rng.standard_normal((1, 1, 32, 16))
    cs, gs = O.build_summaries(K, cf)
    K2 = K.copy()
    K2[0, 0, 8:16] *= 3.0
    cs2, gs2 = O.build_summaries(K2, cf)
    np.testing.assert_allclose(cs2[0, 0, 1], 3.0 * cs[0, 0, 1], atol=1e-12)
    np.testing.assert_allclose(np.delete(cs2[0, 0], 1, 0), np.delete(cs[0, 0], 1, 0), atol=0)
    np.testing.assert_allclose(gs2[0, 0, 2:4], 3.0 * gs[0, 0, 2:4], atol=1e-12)


# --------------------------------------------------------------------------- #
# routing
# --------------------------------------------------------------------------- #
def test_select_top_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(200):
        n = int(rng.integers(0, 20))
        ids = np.sort(rng.choice(1000, size=n, replace=False))
        sc = rng.integers(-3, 3, size=n).astype(np.float64)  # many ties
        k = int(rng.integers(0, 25))
        want = sorted(sorted(zip(ids.tolist(), sc.tolist()), key=lambda p: (-p[1], p[0]))[:k])
        got = O.select_top(sc, ids, k)
        assert got.tolist() == [p[0] for p in want]


def _brute_route(Uq, cs, gs, j, cf):
    d = Uq.shape[1]
    m = cf.groups_per_chunk
    cand = list(range(cf.n_sink, max(cf.n_sink, j - cf.n_local)))

    def score(s):
        return max(sum(float(q[i]) * float(s[i]) for i in range(d)) for q in Uq) / math.sqrt(d)

    csc = {c: score(cs[c]) for c in cand}
    R = sorted(sorted(cand, key=lambda c: (-csc[c], c))[: cf.top_k])
    gcand = [c * m + r for c in R for r in range(m)]
    gsc = {g: score(gs[g]) for g in gcand}
    Gs = sorted(sorted(gcand, key=lambda g: (-gsc[g], g))[: cf.top_g])
    return R, Gs


def test_route_unit_matches_brute_force():
    cf = cfg(head_dim=8, chunk_size=4, group_size=2, n_sink=1, n_local=2, top_k=3, top_g=4)
    rng = np.random.default_rng(21)
    cs = rng.standard_normal((12, 8))
    gs = rng.standard_normal((24, 8))
    for j in range(12):
        Uq = rng.standard_normal((5, 8))
        R, Gs, _ = O.route_unit(Uq, cs, gs, j, cf)
        bR, bG = _brute_route(Uq, cs, gs, j, cf)
        assert R.tolist() == bR and Gs.tolist() == bG, j


def test_boundary_gap_hand_computed():
    """The relative gap at the k-th boundary on hand-derived cases: ties, negative
    scores, a zero denominator, NaN ranking last, no boundary."""
    for c in json.load(open(GOLD))["boundary_gap"]["cases"]:
        sc = np.array([float(x) for x in c["scores"]])
        want = math.inf if c["gap"] == "inf" else float(c["gap"])
        got = O.boundary_gap(sc, c["k"])
        assert (got == want) if math.isinf(want) else abs(got - want) < 1e-15, (c, got)


def _brute_route_heads(Q, q_pos, cs, gs, cf, n_kv_heads, group_of):
    """Decode routing of every (b, h) by brute force, with query head hq serving
    KV head group_of(hq)."""
    B, Hq = Q.shape[:2]
    out = {}
    for b in range(B):
        j = int(q_pos[b]) // cf.chunk_size
        for h in range(n_kv_heads):
            Uq = np.stack([Q[b, hq, 0] for hq in range(Hq) if group_of(hq) == h])
            out[(b, h)] = _brute_route(Uq, cs[b, h], gs[b, h], j, cf)
    return out


def test_route_groups_query_heads_contiguously():
    """GQA: KV head h serves query heads [h*gq, (h+1)*gq) (the layout of Q, K and V
    in the pages' GQA models); with two KV heads and a binding top-k, routing
    equals a brute force over those heads, and differs from an interleaved
    (hq % Hkv) grouping on this input."""
    cf = cfg(head_dim=8, chunk_size=4, group_size=2, n_sink=1, n_local=1, top_k=2, top_g=3)
    rng = np.random.default_rng(5)
    B, Hq, H, d, nC = 2, 4, 2, 8, 10
    cs = rng.standard_normal((B, H, nC, d))
    gs = rng.standard_normal((B, H, nC * 2, d))
    Q = rng.standard_normal((B, Hq, 1, d)) * 0.1
    # query head 2 points hard at chunk 3 of KV head 0, query head 1 at chunk 6 of
    # KV head 1: a grouping error moves those needles to the wrong KV head
    Q[:, 2, 0] = 8.0 * cs[:, 0, 3]
    Q[:, 1, 0] = 8.0 * cs[:, 1, 6]
    q_pos = np.array([39, 38])
    ci, gi, _ = O.route(Q, q_pos, cs, gs, cf, H)
    want = _brute_route_heads(Q, q_pos, cs, gs, cf, H, lambda hq: hq // (Hq // H))
    other = _brute_route_heads(Q, q_pos, cs, gs, cf, H, lambda hq: hq % H)
    differs = False
    for (b, h), (R, Gs) in want.items():
        assert ci[b, h, 0].tolist() == R and gi[b, h, 0].tolist() == Gs, (b, h)
        differs |= other[(b, h)] != (R, Gs)
    assert differs


def test_visible_set_with_given_lists_is_a_causal_union():
    """A caller's group list may repeat a group, name groups inside the forced
    chunks, groups after the query and holes: the visible set is the union of
    the forced tokens and the listed groups' tokens, each token once, up to the
    query's position (brute force with Python sets)."""
    cf = cfg(chunk_size=8, group_size=4, n_sink=1, n_local=1)
    t = 37  # chunk 4; forced chunks 0, 3, 4
    lst = np.array([5, -1, 5, 1, 7, 9, 8, 2, 11, -3, 4])
    want = {u for c in (0, 3, 4) for u in range(8 * c, 8 * c + 8)}
    want |= {u for g in lst.tolist() if g >= 0 for u in range(4 * g, 4 * g + 4)}
    want = sorted(u for u in want if u <= t)
    assert O.visible_tokens(t, lst, cf).tolist() == want
    # attention over that set counts every token once
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((1, 1, 1, 16))
    K = rng.standard_normal((1, 1, 64, 16))
    V = rng.standard_normal((1, 1, 64, 16))
    o, _ = O.attend(Q, np.array([t]), K, V, lst.reshape(1, 1, 1, -1), cf, 1)
    z = K[0, 0, want] @ Q[0, 0, 0] / 4.0
    w = np.exp(z - z.max())
    np.testing.assert_allclose(o[0, 0, 0], w @ V[0, 0, want] / w.sum(), atol=1e-12)


def test_unit_block_attention_matches_masked_softmax_per_row():
    """The prefill oracle's per-unit form (all g_q*C rows of a query chunk at
    once) against a mask built row by row from the rule (sink chunks, local
    chunks, the current chunk up to the row, the listed groups) and a float64
    masked softmax in torch: GQA head grouping, causality inside the current
    chunk, holes, repeats and a listed group inside a forced chunk."""
    cf = cfg(chunk_size=8, group_size=4, n_sink=1, n_local=1, top_g=4)
    Hkv, gq, d, n = 2, 2, 16, 64
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((1, Hkv * gq, n, d))
    K = rng.standard_normal((1, Hkv, n, d))
    V = rng.standard_normal((1, Hkv, n, d))
    nU = n // 8
    gi = np.full((1, Hkv, nU, 4), -1, dtype=np.int64)
    for h in range(Hkv):
        for u in range(nU):
            cands = list(range(1 * 2, max(1, u - 1) * 2))  # groups of chunks [1, u - 1)
            pick = rng.permutation(cands)[:3].tolist() if cands else []
            row = pick + [pick[0] if pick else -1]     # a repeat (or a hole)
            if u >= 3:
                row[-1] = 2 * (u - 1)                   # a group of the local chunk u - 1
            gi[0, h, u, :len(row)] = row
    for h in range(Hkv):
        for u in range(nU):
            o, lse = O.attend_unit_block(Q, np.array([0]), K, V, gi, cf, Hkv, 0, h, u)
            listed = {int(g) for g in gi[0, h, u] if g >= 0}
            for hh in range(gq):
                for c in range(8):
                    t = 8 * u + c
                    s = torch.arange(n)
                    vis = (s < 8) | (s >= 8 * (u - 1))
                    vis |= torch.tensor([(x // 4) in listed for x in range(n)])
                    vis &= s <= t  # causal: nothing after the row
                    q = torch.from_numpy(Q[0, h * gq + hh, t])
                    z = torch.from_numpy(K[0, h]) @ q / math.sqrt(d)
                    z = torch.where(vis, z, torch.tensor(-math.inf, dtype=torch.float64))
                    w = torch.softmax(z, dim=0)
                    want = (w @ torch.from_numpy(V[0, h])).numpy()
                    np.testing.assert_allclose(o[hh, c], want, atol=1e-12)
                    np.testing.assert_allclose(lse[hh, c], torch.logsumexp(z, dim=0).item(), atol=1e-12)


def test_route_takes_all_when_fewer_candidates():
    cf = cfg(head_dim=8, chunk_size=4, group_size=2, n_sink=1, n_local=1, top_k=50, top_g=500)
    rng = np.random.default_rng(2)
    cs, gs = rng.standard_normal((10, 8)), rng.standard_normal((20, 8))
    R, Gs, dg = O.route_unit(rng.standard_normal((3, 8)), cs, gs, 9, cf)
    assert R.tolist() == list(range(1, 8))
    assert Gs.tolist() == list(range(2, 16))
    assert dg["chunk_gap"] == math.inf and dg["group_gap"] == math.inf


def test_chunk_and_group_size_one_is_token_topk_attention():
    """C = G = 1 reduces HGA to textbook top-k token attention plus the current token."""
    n, d, k = 40, 8, 5
    cf = O.HGAConfig(head_dim=d, chunk_size=1, group_size=1, n_sink=0, n_local=0,
                     top_k=k, top_g=k, rope_base=10000.0)
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((1, 1, n, d))
    K = rng.standard_normal((1, 1, n, d))
    V = rng.standard_normal((1, 1, n, d))
    res = O.prefill(Q, K, V, cf, n_kv_heads=1)
    q, kk, v = (torch.tensor(x[0, 0]) for x in (Q, K, V))
    s = q @ kk.T / math.sqrt(d)
    for t in range(n):
        prev = s[t, :t]
        sel = torch.topk(prev, min(k, t)).indices.tolist() if t else []
        keep = torch.zeros(n, dtype=torch.bool)
        keep[sel] = True
        keep[t] = True
        w = torch.softmax(s[t].masked_fill(~keep, float("-inf")), dim=0)
        np.testing.assert_allclose(res["O"][0, 0, t], (w @ v).numpy(), atol=1e-12)


# --------------------------------------------------------------------------- #
# visibility + attention invariants
# --------------------------------------------------------------------------- #
def _sdpa_causal(Q, K, V, hkv):
    gq = Q.shape[1] // hkv
    k = torch.tensor(K).repeat_interleave(gq, dim=1)
    v = torch.tensor(V).repeat_interleave(gq, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Q), k, v, is_causal=True).numpy()


@pytest.mark.parametrize("C,G,ns,nl", [(8, 4, 1, 1), (8, 2, 0, 0), (4, 4, 2, 3), (16, 4, 1, 0)])
def test_full_topk_equals_dense_causal(C, G, ns, nl):
    n, d, hq, hkv = 64, 16, 4, 2
    cf = O.HGAConfig(head_dim=d, chunk_size=C, group_size=G, n_sink=ns, n_local=nl,
                     top_k=n, top_g=n, rope_base=100.0)
    rng = np.random.default_rng(C * 7 + G)
    Q = rng.standard_normal((2, hq, n, d))
    K = rng.standard_normal((2, hkv, n, d))
    V = rng.standard_normal((2, hkv, n, d))
    res = O.prefill(Q, K, V, cf, n_kv_heads=hkv)
    np.testing.assert_allclose(res["O"], _sdpa_causal(Q, K, V, hkv), atol=1e-10)
    np.testing.assert_allclose(res["O"], O.dense_causal(Q, K, V, hkv), atol=1e-12)


def test_full_topk_decode_equals_dense():
    L, d, hq, hkv = 77, 16, 4, 1
    cf = O.HGAConfig(head_dim=d, chunk_size=8, group_size=4, n_sink=1, n_local=1,
                     top_k=100, top_g=100, rope_base=100.0)
    rng = np.random.default_rng(12)
    Q = rng.standard_normal((1, hq, 1, d))
    K = rng.standard_normal((1, hkv, 80, d))
    V = rng.standard_normal((1, hkv, 80, d))
    cs, gs = O.build_summaries(K, cf, n_tokens=L)
    res = O.decode(Q, K, V, np.array([L]), cs, gs, cf, hkv)
    k = torch.tensor(K[:, :, :L]).expand(1, hq, L, d)
    v = torch.tensor(V[:, :, :L]).expand(1, hq, L, d)
    want = torch.nn.functional.scaled_dot_product_attention(torch.tensor(Q), k, v).numpy()
    np.testing.assert_allclose(res["O"], want, atol=1e-12)


def test_forced_windows_visible_under_adversarial_keys():
    """Sink, local and current tokens stay in the softmax even when their keys point
    away from every query; V one-hot exposes every token's weight."""
    n, d = 48, 64
    cf = O.HGAConfig(head_dim=d, chunk_size=8, group_size=4, n_sink=1, n_local=2,
                     top_k=1, top_g=1, rope_base=100.0)
    rng = np.random.default_rng(6)
    q = rng.standard_normal(d)
    Q = np.tile(q, (1, 1, n, 1))
    K = rng.standard_normal((1, 1, n, d)) + 1.5 * q  # aligned keys everywhere...
    forced_tok = [u for c in (0, 3, 4, 5) for u in range(c * 8, c * 8 + 8)]
    K[0, 0, forced_tok] = -3.0 * q / np.linalg.norm(q)  # ...except sink/local/current of j=5
    V = np.zeros((1, 1, n, d))
    V[0, 0, np.arange(n), np.arange(n)] = 1.0
    res = O.prefill(Q, K, V, cf, n_kv_heads=1)
    t = n - 1
    w = res["O"][0, 0, t, :n]
    for u in forced_tok:
        assert w[u] > 0.0, u
    assert np.count_nonzero(w > 0) == len(forced_tok) + 4  # + one routed group of 4


def test_attention_never_reads_summaries():
    """NaN-poisoned summaries after routing leave the output unchanged and finite."""
    cf = cfg(head_dim=16, chunk_size=8, group_size=4, top_k=2, top_g=3)
    rng = np.random.default_rng(8)
    Q = rng.standard_normal((1, 2, 1, 16))
    K = rng.standard_normal((1, 1, 96, 16))
    V = rng.standard_normal((1, 1, 96, 16))
    cs, gs = O.build_summaries(K, cf)
    res = O.decode(Q, K, V, np.array([96]), cs, gs, cf, 1)
    cs[:] = np.nan
    gs[:] = np.nan
    O2, _ = O.attend(Q, np.array([95]), K, V, res["group_idx"], cf, 1)
    assert np.isfinite(O2).all()
    np.testing.assert_array_equal(O2, res["O"])


def test_constant_keys_one_hot_values_expose_exact_set_and_tiebreak():
    """K constant -> every score ties -> the lowest candidate indices win; with V one-hot
    the output is indicator(T)/|T|."""
    n, d = 64, 64
    cf = O.HGAConfig(head_dim=d, chunk_size=8, group_size=2, n_sink=1, n_local=1,
                     top_k=2, top_g=3, rope_base=100.0, hf_threshold=0.0)
    rng = np.random.default_rng(10)
    Q = rng.standard_normal((1, 1, n, d))
    K = np.tile(rng.standard_normal(d), (1, 1, n, 1))
    V = np.eye(n)[None, None]
    res = O.prefill(Q, K, V, cf, n_kv_heads=1)
    for t in (63, 40, 30, 17):
        j = t // 8
        R = [c for c in range(1, max(1, j - 1))][:2]
        gids = sorted([c * 4 + r for c in R for r in range(4)])[:3]
        forced = sorted(set(range(min(1, j + 1))) | set(range(max(0, j - 1), j + 1)))
        T = {u for c in forced for u in range(c * 8, c * 8 + 8) if u <= t}
        T |= {u for g in gids for u in range(g * 2, g * 2 + 2)}
        want = np.zeros(n)
        want[sorted(T)] = 1.0 / len(T)
        np.testing.assert_allclose(res["O"][0, 0, t], want, atol=1e-12)
        assert res["chunk_idx"][0, 0, j].tolist()[: len(R)] == R


def test_softmax_is_a_set_function():
    rng = np.random.default_rng(13)
    q = rng.standard_normal(32)
    Kt, Vt = rng.standard_normal((50, 32)), rng.standard_normal((50, 32))
    o, l = O.softmax_attend(q, Kt, Vt)
    for _ in range(5):
        p = rng.permutation(50)
        o2, l2 = O.softmax_attend(q, Kt[p], Vt[p])
        np.testing.assert_allclose(o2, o, atol=1e-12)
        assert abs(l2 - l) < 1e-12


def test_two_key_closed_form():
    d = 4
    q = np.array([1.0, 0.5, -0.25, 2.0])
    k0, k1 = np.array([0.3, 0.1, 0.0, 0.7]), np.array([-0.2, 0.4, 1.0, 0.1])
    v0, v1 = np.array([1.0, -2.0, 3.0, 0.5]), np.array([-1.0, 4.0, 0.0, 2.5])
    z0, z1 = q @ k0 / 2.0, q @ k1 / 2.0
    delta = z0 - z1
    want = (v0 + math.exp(-delta) * v1) / (1 + math.exp(-delta))
    o, lse = O.softmax_attend(q, np.stack([k0, k1]), np.stack([v0, v1]))
    np.testing.assert_allclose(o, want, atol=1e-14)
    assert abs(lse - (z0 + math.log(1 + math.exp(-delta)))) < 1e-14


def test_visible_token_counts_closed_form():
    gold = json.load(open(GOLD))
    from hierarchical_sparse_attention_build_amd import workloads as W
    for c in gold["decode_visible_tokens"]["cases"]:
        s = W.spec(c["workload"])
        cf = O.HGAConfig(**W.hga_config_kwargs(s))
        t = s.n_tokens - 1
        j = t // s.chunk_size
        assert len(O.chunk_candidates(j, cf)) == c["candidates"]
        forced = O.visible_tokens(t, np.array([], dtype=np.int64), cf)
        assert len(forced) == c["forced"]
        m = s.chunk_size // s.group_size
        groups = np.arange(min(s.top_g, s.top_k * m)) * 3 + 4 * m  # any disjoint routed groups
        assert len(O.visible_tokens(t, groups, cf)) == c["total"]
        assert 0.019 <= c["total"] / s.n_tokens <= 0.125
    for c in gold["prefill_last_row_tokens"]["cases"]:
        s = W.spec(c["workload"])
        cf = O.HGAConfig(**W.hga_config_kwargs(s))
        t = s.n_tokens - 1
        m = s.chunk_size // s.group_size
        ng = min(s.top_g, s.top_k * m)
        groups = np.arange(ng) + s.n_sink * m
        assert len(O.visible_tokens(t, groups, cf)) == c["total"]


def test_forced_chunks_enumeration():
    cf = cfg(n_sink=2, n_local=3)
    assert O.forced_chunks(0, cf).tolist() == [0]
    assert O.forced_chunks(1, cf).tolist() == [0, 1]
    assert O.forced_chunks(4, cf).tolist() == [0, 1, 2, 3, 4]
    assert O.forced_chunks(6, cf).tolist() == [0, 1, 3, 4, 5, 6]
    assert O.chunk_candidates(6, cf).tolist() == [2]
    assert O.chunk_candidates(5, cf).tolist() == []
    assert O.chunk_candidates(10, cf).tolist() == [2, 3, 4, 5, 6]


# --------------------------------------------------------------------------- #
# warm tier: bounded LRU of routed groups
# --------------------------------------------------------------------------- #
def _lru_run(steps, slots, n_groups_cap=1 << 20):
    tags, stamps, clock = [-1] * slots, [0] * slots, 0
    out = []
    for g in steps:
        so, mi, tags, stamps, clock = O.warm_lru_step(tags, stamps, clock, g, n_groups_cap)
        out.append((so, mi, list(tags), list(stamps)))
    return out


def test_warm_lru_textbook_sequence():
    """Two slots, one group per step, accesses 5 7 5 9: least recently used is
    evicted, so 9 replaces 7 (a FIFO cache would replace 5)."""
    r = _lru_run([[5], [7], [5], [9]], 2)
    assert [m for _, m, _, _ in r] == [[(0, 5)], [(1, 7)], [], [(1, 9)]]
    assert sorted(r[-1][2]) == [5, 9]
    assert r[2][0] == [0]          # the hit keeps its slot


def test_warm_lru_matches_recency_list_one_group_per_step():
    """With one group per step every stamp is distinct, and the cached set after
    each step is the textbook LRU set: the `slots` most recently used distinct
    groups (kept here as a plain recency list)."""
    rng = np.random.default_rng(11)
    for slots in (1, 3, 8):
        seq = rng.integers(0, 12, size=300)
        r = _lru_run([[int(g)] for g in seq], slots)
        recency = []
        hits = 0
        for g, (so, mi, tags, _) in zip(seq, r):
            g = int(g)
            hit = g in recency
            hits += hit
            if hit:
                recency.remove(g)
            recency.insert(0, g)
            del recency[slots:]
            assert (mi == []) == hit
            assert sorted(t for t in tags if t >= 0) == sorted(recency)
            assert tags[so[0]] == g
        assert 0 < hits < len(seq)


def test_warm_lru_invariants_many_groups_per_step():
    """Several groups per step: every routed group is cached after its step, only
    missing groups are copied (each into a slot nobody in the step uses), hits
    keep their slots, and an evicted slot was never more recently used than a
    slot that survives."""
    rng = np.random.default_rng(12)
    slots, per_step, cap = 12, 5, 40
    tags, stamps, clock = [-1] * slots, [0] * slots, 0
    for _ in range(400):
        g = rng.choice(cap, per_step, replace=False).tolist()
        g[rng.integers(per_step)] = -1 if rng.random() < 0.3 else g[0]  # holes and a repeat
        g = [x if x != g[0] or i == 0 else -1 for i, x in enumerate(g)]   # keep entries distinct
        before_tags, before_stamps = list(tags), list(stamps)
        so, mi, tags, stamps, clock = O.warm_lru_step(tags, stamps, clock, g, cap)
        valid = [x for x in g if 0 <= x < cap]
        for i, x in enumerate(g):
            if 0 <= x < cap:
                assert tags[so[i]] == x and stamps[so[i]] == clock
            else:
                assert so[i] == -1
        missing = [x for x in valid if x not in before_tags]
        assert [x for _, x in mi] == missing
        assert len({s for s, _ in mi} | {so[i] for i, x in enumerate(g) if x in before_tags and x >= 0}) == len(valid)
        evicted = [s for s, _ in mi]
        kept = [s for s in range(slots) if s not in evicted and stamps[s] != clock]
        for s in evicted:
            for k in kept:
                assert (before_stamps[s], s) <= (before_stamps[k], k) or before_tags[s] == -1


def test_warm_lru_ignores_out_of_range_entries():
    so, mi, tags, stamps, clock = O.warm_lru_step([-1] * 4, [0] * 4, 0, [3, -1, 99, 2], 10)
    assert so[1] == -1 and so[2] == -1
    assert [g for _, g in mi] == [3, 2] and clock == 1


# --------------------------------------------------------------------------- #
# backward through the selected-set attention
# --------------------------------------------------------------------------- #
def _bwd_case(seed=21):
    cf = cfg(head_dim=8, chunk_size=4, group_size=2, n_sink=1, n_local=1, top_k=2, top_g=2)
    rng = np.random.default_rng(seed)
    B, Hq, H, n, d = 1, 2, 1, 24, 8
    Q = rng.standard_normal((B, Hq, n, d))
    K = rng.standard_normal((B, H, n, d))
    V = rng.standard_normal((B, H, n, d))
    q_pos = np.zeros(B, dtype=np.int64)
    cs, gs = O.build_summaries(K, cf)
    _, gi, _ = O.route(Q, q_pos, cs, gs, cf, H)
    dO = rng.standard_normal((B, Hq, n, d))
    return cf, Q, K, V, q_pos, gi, dO, H


def test_attend_backward_matches_central_differences():
    """Each gradient entry against a central difference of sum(dO * O) with the
    routed lists held fixed (step 1e-6 in float64)."""
    cf, Q, K, V, q_pos, gi, dO, H = _bwd_case()
    dQ, dK, dV = O.attend_backward(Q, q_pos, K, V, gi, dO, cf, H)
    f = lambda Q_, K_, V_: float((O.attend(Q_, q_pos, K_, V_, gi, cf, H)[0] * dO).sum())
    rng = np.random.default_rng(1)
    h = 1e-6
    for X, G, k in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        for _ in range(12):
            idx = tuple(int(rng.integers(s)) for s in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[k], args_m[k] = Xp, Xm
            num = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(num - G[idx]) <= 1e-6 * max(1.0, abs(num)), (k, idx, num, G[idx])


def test_attend_backward_matches_torch_autograd():
    """The same gradients from torch autograd (CPU, float64) of a masked softmax
    attention whose mask is the visible sets."""
    cf, Q, K, V, q_pos, gi, dO, H = _bwd_case(22)
    dQ, dK, dV = O.attend_backward(Q, q_pos, K, V, gi, dO, cf, H)
    B, Hq, n, d = Q.shape
    gq = Hq // H
    mask = np.zeros((B, Hq, n, n), dtype=bool)
    for b in range(B):
        for hq in range(Hq):
            for i in range(n):
                mask[b, hq, i, O.visible_tokens(i, gi[b, hq // gq, i // cf.chunk_size], cf)] = True
    Qt = torch.tensor(Q, requires_grad=True)
    Kt = torch.tensor(K, requires_grad=True)
    Vt = torch.tensor(V, requires_grad=True)
    Ke = Kt.repeat_interleave(gq, dim=1)
    Ve = Vt.repeat_interleave(gq, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(Qt, Ke, Ve, attn_mask=torch.tensor(mask))
    (out * torch.tensor(dO)).sum().backward()
    assert np.abs(Qt.grad.numpy() - dQ).max() < 1e-10
    assert np.abs(Kt.grad.numpy() - dK).max() < 1e-10
    assert np.abs(Vt.grad.numpy() - dV).max() < 1e-10
