"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every case prints its name, shape and seed before touching the GPU.  Inputs are
the seeded workloads; the oracle runs in float64 on the same rounded values.
"""
import numpy as np
import pytest

import oracle as O
from hierarchical_sparse_attention_build_amd import workloads as W
from tests.hga_testutil import (GAP, TOL, cfg_of, check_routing, dev, f64, max_abs, messy_group_lists,
                                params_of, say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_sparse_attention_build_amd import hga as H
    H.lib()
    return H


def _summ_tables(s):
    nC = s.n_tokens // s.chunk_size
    m = s.chunk_size // s.group_size
    cs = torch.full((s.batch, s.n_kv_heads, nC, s.head_dim), float("nan"), device="cuda")
    gs = torch.full((s.batch, s.n_kv_heads, nC * m, s.head_dim), float("nan"), device="cuda")
    return cs, gs


# --------------------------------------------------------------------------- summaries
@pytest.mark.parametrize("name,over", [
    ("tiny_prefill_fp32", {}),
    ("decode_32k", {"batch": 2, "n_tokens": 4096}),
    ("tiny_prefill_fp32", {"group_size": 1, "n_tokens": 256}),
    ("decode_32k", {"batch": 1, "n_tokens": 2048, "chunk_size": 32, "group_size": 8, "head_dim": 64}),
])
def test_summaries(hga, name, over):
    s = W.spec(name, **over)
    say(f"[summaries] {name} {over} seed={s.seed}")
    w = W.make(s)
    p = params_of(s)
    K = dev(w.K, s.dtype)
    cs, gs = _summ_tables(s)
    nC = s.n_tokens // s.chunk_size
    hga.build_summaries(p, K, s.n_tokens, 0, nC, cs, gs)
    torch.cuda.synchronize()
    ocs, ogs = O.build_summaries(f64(w.K, s.dtype), cfg_of(s))
    e1, e2 = max_abs(cs.cpu().numpy(), ocs), max_abs(gs.cpu().numpy(), ogs)
    say(f"  chunk max-abs {e1:.3e}  group max-abs {e2:.3e}")
    assert e1 < 1e-5 and e2 < 1e-5


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_summaries_raw_keys(hga, dtype):
    """Raw projected keys: literal form with absolute angles, plus the RoPE'd copy."""
    s = W.spec("tiny_prefill_fp32", dtype=dtype, n_tokens=2048, chunk_size=64, group_size=16)
    say(f"[summaries raw] dtype={dtype} seed={s.seed}")
    w = W.make(s)
    p = params_of(s)
    K = dev(w.K, s.dtype)
    Krot = torch.empty_like(K)
    cs, gs = _summ_tables(s)
    nC = s.n_tokens // s.chunk_size
    # a sub-range first: only chunks [3, nC) are written
    hga.build_summaries(p, K, s.n_tokens, 3, nC, cs, gs, k_is_rotated=False, K_rot_out=Krot)
    torch.cuda.synchronize()
    cfg = cfg_of(s)
    Kf = f64(w.K, s.dtype)
    ocs, ogs = O.build_summaries(Kf, cfg, k_is_rotated=False, form="literal")
    m = s.chunk_size // s.group_size
    e1 = max_abs(cs[:, :, 3:].cpu().numpy(), ocs[:, :, 3:])
    e2 = max_abs(gs[:, :, 3 * m:].cpu().numpy(), ogs[:, :, 3 * m:])
    assert torch.isnan(cs[:, :, :3]).all()
    rot = O.apply_rope(Kf, np.arange(s.n_tokens), cfg)
    kr = Krot.float().cpu().numpy()
    t0 = 3 * s.chunk_size
    if dtype == "fp32":
        e3 = max_abs(kr[:, :, t0:], rot[:, :, t0:])
        assert e3 < 1e-5, e3
    else:  # one bf16 rounding of a value within fp32 error of the exact one
        err = np.abs(kr[:, :, t0:] - rot[:, :, t0:])
        scale = np.abs(Kf[:, :, t0:]).max()
        assert np.all(err <= np.abs(rot[:, :, t0:]) * 2.0 ** -7 + 1e-6 * scale)
    say(f"  chunk {e1:.3e} group {e2:.3e}")
    assert e1 < 2e-5 and e2 < 2e-5


# --------------------------------------------------------------------------- routing
def _decode_inputs(s, w):
    q_pos = (w.seq_len - 1).astype(np.int32)
    return q_pos


@pytest.mark.parametrize("name,over", [
    ("decode_32k", {"batch": 2, "n_tokens": 8192}),
    ("decode_64k", {"batch": 1, "n_tokens": 16384}),
    ("offload_decode_128k", {"batch": 1, "n_tokens": 16384}),
])
def test_route_decode(hga, name, over):
    s = W.spec(name, **over)
    say(f"[route decode] {name} {over} seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    ocs, ogs = O.build_summaries(f64(w.K, s.dtype), cfg)
    cs32, gs32 = ocs.astype(np.float32), ogs.astype(np.float32)
    q_pos = _decode_inputs(s, w)
    or_ci, or_gi, diags = O.route(f64(w.Q, s.dtype), q_pos, cs32.astype(np.float64),
                                  gs32.astype(np.float64), cfg, s.n_kv_heads)
    p = params_of(s)
    B, H = s.batch, s.n_kv_heads
    ci = torch.empty((B, H, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device="cuda")
    sc = torch.full((B, H, s.n_tokens // s.chunk_size), float("nan"), device="cuda")
    ws = hga.workspace(p, hga.OP_ROUTE, 1, s.n_tokens)
    hga.route(p, dev(w.Q, s.dtype), 1, torch.from_numpy(q_pos).cuda(), torch.from_numpy(cs32).cuda(),
              torch.from_numpy(gs32).cuda(), s.n_tokens, ci, gi, ws, scores_out=sc)
    torch.cuda.synchronize()
    n, unique = check_routing(ci.cpu().numpy(), gi.cpu().numpy(), or_ci, or_gi, diags, s.top_k, s.top_g)
    say(f"  units {n}, unique {len(unique)}")
    scn = sc.cpu().numpy()
    for (b, h, u), dg in diags.items():
        got = scn[b, h, dg["chunk_cand"]]
        np.testing.assert_allclose(got, dg["chunk_scores"], rtol=1e-5, atol=1e-6)
    # second call on the same workspace (counters reset themselves)
    hga.route(p, dev(w.Q, s.dtype), 1, torch.from_numpy(q_pos).cuda(), torch.from_numpy(cs32).cuda(),
              torch.from_numpy(gs32).cuda(), s.n_tokens, ci, gi, ws)
    torch.cuda.synchronize()
    check_routing(ci.cpu().numpy(), gi.cpu().numpy(), or_ci, or_gi, diags, s.top_k, s.top_g)
    assert int(ws[:64].sum()) == 0


# --------------------------------------------------------------------------- attention
@pytest.mark.parametrize("name,over", [
    ("decode_32k", {"batch": 2, "n_tokens": 8192}),
    ("decode_32k", {"batch": 2, "n_tokens": 4096, "dtype": "fp32"}),
    ("offload_decode_128k", {"batch": 1, "n_tokens": 8192}),
])
def test_attend_decode_given_indices(hga, name, over):
    """Attention alone, on index sets chosen by the oracle (given to both sides)."""
    s = W.spec(name, **over)
    say(f"[attend decode] {name} {over} seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    ocs, ogs = O.build_summaries(Kf, cfg)
    q_pos = _decode_inputs(s, w)
    _, or_gi, _ = O.route(Qf, q_pos, ocs, ogs, cfg, s.n_kv_heads)
    Oo, lse_o = O.attend(Qf, q_pos, Kf, Vf, or_gi, cfg, s.n_kv_heads)
    p = params_of(s)
    out = torch.empty((s.batch, s.n_q_heads, 1, s.head_dim), device="cuda")
    lse = torch.empty((s.batch, s.n_q_heads, 1), device="cuda")
    ws = hga.workspace(p, hga.OP_ATTEND, 1, s.n_tokens)
    hga.attend(p, dev(w.Q, s.dtype), 1, torch.from_numpy(q_pos).cuda(), dev(w.K, s.dtype),
               dev(w.V, s.dtype), s.n_tokens, torch.from_numpy(or_gi).cuda(), out, ws, lse_out=lse)
    torch.cuda.synchronize()
    e = max_abs(out.cpu().numpy(), Oo)
    el = max_abs(lse.cpu().numpy(), lse_o)
    say(f"  O max-abs {e:.3e}  lse max-abs {el:.3e}")
    assert e <= TOL[s.dtype] and el <= 10 * TOL[s.dtype]


# --------------------------------------------------------------------------- end to end
def _run_decode_e2e(hga, s, w):
    cfg = cfg_of(s)
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    p = params_of(s)
    B, H, n = s.batch, s.n_kv_heads, s.n_tokens
    K, V, Q = dev(w.K, s.dtype), dev(w.V, s.dtype), dev(w.Q, s.dtype)
    cs, gs = _summ_tables(s)
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).cuda()
    # tables for every complete chunk before the query's chunk (a decode loop's state)
    jq = int((w.seq_len.min() - 1) // s.chunk_size)
    hga.build_summaries(p, K, n, 0, jq, cs, gs)
    ci = torch.empty((B, H, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.n_q_heads, 1, s.head_dim), device="cuda")
    ws = hga.workspace(p, hga.OP_DECODE, 1, n)
    hga.decode(p, Q, K, V, n, seq, cs, gs, out, ws, chunk_idx=ci, group_idx=gi)
    torch.cuda.synchronize()
    ocs, ogs = O.build_summaries(Kf, cfg)
    q_pos = (w.seq_len - 1).astype(np.int64)
    or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, H)
    gi_n = gi.cpu().numpy()
    n_units, unique = check_routing(ci.cpu().numpy(), gi_n, or_ci, or_gi, diags, s.top_k, s.top_g)
    # every row, against the oracle's attention over the GPU's validated lists
    Oo, _ = O.attend(Qf, q_pos, Kf, Vf, gi_n, cfg, H)
    e = max_abs(out.cpu().numpy(), Oo)
    say(f"  units {n_units} unique routing {len(unique)}  O max-abs over all units {e:.3e}")
    assert e <= TOL[s.dtype]
    # the step completed chunk (L-1)/C: its summaries were written
    csn = cs.cpu().numpy()
    for b in range(B):
        L = int(w.seq_len[b])
        if L % s.chunk_size == 0:
            c = L // s.chunk_size - 1
            assert max_abs(csn[b, :, c], ocs[b, :, c]) < 1e-5
    return ws


@pytest.mark.parametrize("name,over", [
    ("decode_32k", {"batch": 2, "n_tokens": 8192}),
    ("decode_64k", {"batch": 2, "n_tokens": 16384}),
    ("decode_32k", {"batch": 2, "n_tokens": 4096, "dtype": "fp32"}),
    ("decode_32k", {"batch": 2, "n_tokens": 4096, "n_q_heads": 8, "n_kv_heads": 8}),
    ("decode_32k", {"batch": 1, "n_tokens": 4096, "n_q_heads": 16, "n_kv_heads": 1, "head_dim": 64}),
    # 88 units: too many for two routing workgroups and one forced each on a
    # 256-CU device (one routing and one forced workgroup per unit instead)
    ("decode_32k", {"batch": 11, "n_tokens": 2048}),
    # 136 units: one routing and two forced workgroups per unit
    ("decode_32k", {"batch": 17, "n_tokens": 2048}),
    # 2042 candidate chunks: four keys per lane in each wave's share of the chunk selection
    ("decode_32k", {"batch": 1, "n_tokens": 131072}),
    # top_k = 32: the second selection phase takes 8 x 32 winners, four keys per lane
    ("decode_32k", {"batch": 2, "n_tokens": 16384, "top_k": 32}),
])
def test_decode_end_to_end(hga, name, over):
    s = W.spec(name, **over)
    say(f"[decode e2e] {name} {over} seed={s.seed}")
    w = W.make(s)
    _run_decode_e2e(hga, s, w)


def test_decode_full_size_32k(hga):
    """The benchmarked decode workload at full size (B=8, 32K context)."""
    s = W.spec("decode_32k")
    say(f"[decode e2e full] decode_32k seed={s.seed}")
    w = W.make(s)
    _run_decode_e2e(hga, s, w)


@pytest.mark.timeout(300)
def test_decode_full_size_64k_sampled(hga):
    """The long-context decode workload at full size (B=16, 64K context, 128
    units, in the launch shape that is benchmarked); the routing and output of
    six sampled units against the oracle, computed on those units' own slices
    of Q, K and V."""
    s = W.spec("decode_64k")
    say(f"[decode e2e full, sampled units] decode_64k seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    p = params_of(s)
    B, H, n = s.batch, s.n_kv_heads, s.n_tokens
    gq = s.n_q_heads // H
    K, V, Q = dev(w.K, s.dtype), dev(w.V, s.dtype), dev(w.Q, s.dtype)
    cs, gs = _summ_tables(s)
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).cuda()
    jq = int((w.seq_len.min() - 1) // s.chunk_size)
    hga.build_summaries(p, K, n, 0, jq, cs, gs)
    ci = torch.empty((B, H, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.n_q_heads, 1, s.head_dim), device="cuda")
    hga.decode(p, Q, K, V, n, seq, cs, gs, out, hga.workspace(p, hga.OP_DECODE, 1, n), chunk_idx=ci, group_idx=gi)
    torch.cuda.synchronize()
    ci_n, gi_n, got = ci.cpu().numpy(), gi.cpu().numpy(), out.cpu().numpy()
    assert np.isfinite(got).all()
    rng = np.random.default_rng(s.seed)
    sample = list(zip(rng.choice(B, 6, replace=False).tolist(), rng.integers(0, H, 6).tolist()))
    for b, h in sample:
        Kf, Vf = f64(w.K[b:b + 1, h:h + 1], s.dtype), f64(w.V[b:b + 1, h:h + 1], s.dtype)
        Qf = f64(w.Q[b:b + 1, h * gq:(h + 1) * gq], s.dtype)
        q_pos = (w.seq_len[b:b + 1] - 1).astype(np.int64)
        ocs, ogs = O.build_summaries(Kf, cfg)
        or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, 1)
        _, unique = check_routing(ci_n[b:b + 1, h:h + 1], gi_n[b:b + 1, h:h + 1], or_ci, or_gi, diags,
                                  s.top_k, s.top_g)
        Oo, _ = O.attend(Qf, q_pos, Kf, Vf, gi_n[b:b + 1, h:h + 1], cfg, 1)
        e = max_abs(got[b, h * gq:(h + 1) * gq, 0], Oo[0, :, 0])
        say(f"  unit (b={b}, h={h}): unique routing {bool(unique)}, O max-abs {e:.3e}")
        assert e <= TOL[s.dtype]


def test_decode_ragged_and_short(hga):
    """Per-sequence lengths from 1 token up to the capacity, partial current chunks,
    sequences with no routing candidates yet."""
    s = W.spec("decode_32k", batch=6, n_tokens=4096, needles=0)
    say(f"[decode ragged] seed={s.seed}")
    w = W.make(s)
    w.seq_len = np.array([1, 64, 65, 300, 1000, 4096], dtype=np.int32)
    cfg = cfg_of(s)
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    p = params_of(s)
    n = s.n_tokens
    K, V, Q = dev(w.K, s.dtype), dev(w.V, s.dtype), dev(w.Q, s.dtype)
    cs, gs = _summ_tables(s)
    hga.build_summaries(p, K, n, 0, n // s.chunk_size, cs, gs)
    seq = torch.from_numpy(w.seq_len).cuda()
    ci = torch.empty((s.batch, s.n_kv_heads, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((s.batch, s.n_kv_heads, 1, s.top_g), dtype=torch.int32, device="cuda")
    out = torch.empty((s.batch, s.n_q_heads, 1, s.head_dim), device="cuda")
    ws = hga.workspace(p, hga.OP_DECODE, 1, n)
    hga.decode(p, Q, K, V, n, seq, cs, gs, out, ws, chunk_idx=ci, group_idx=gi)
    torch.cuda.synchronize()
    ocs, ogs = O.build_summaries(Kf, cfg)
    q_pos = (w.seq_len - 1).astype(np.int64)
    or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, s.n_kv_heads)
    gi_n = gi.cpu().numpy()
    check_routing(ci.cpu().numpy(), gi_n, or_ci, or_gi, diags, s.top_k, s.top_g)
    Oo, _ = O.attend(Qf, q_pos, Kf, Vf, gi_n, cfg, s.n_kv_heads)
    got = out.cpu().numpy()
    for b in range(s.batch):
        assert max_abs(got[b], Oo[b]) <= TOL[s.dtype], b
    # first sequences have no candidates: empty routing
    assert (ci.cpu().numpy()[0] == -1).all() and (gi.cpu().numpy()[0] == -1).all()
    assert np.isfinite(got).all()


@pytest.mark.parametrize("over", [{}, {"n_sink": 0, "n_local": 0}, {"top_k": 0, "top_g": 0},
                                  {"group_size": 64, "top_g": 5}, {"head_dim": 64, "n_q_heads": 16},
                                  {"n_q_heads": 8, "n_sink": 3, "n_local": 1, "top_k": 40, "top_g": 100},
                                  {"chunk_size": 32, "group_size": 8, "top_k": 7, "top_g": 9}])
def test_decode_step_matches_route_then_attend(hga, over):
    """The one-launch decode step and the separate routing + attention calls
    agree: index lists bit for bit (same exact selection over the same fp32
    scores), outputs to fp32 rounding (the softmax sums are split differently).
    Lengths are ragged, with partial chunks and sequences without candidates."""
    s = W.spec("decode_32k", batch=4, n_tokens=4096, **over)
    say(f"[decode step vs route+attend] {over} seed={s.seed}")
    w = W.make(s)
    w.seq_len = np.array([1, 700, 2049, 4096], dtype=np.int32)
    p = params_of(s)
    n = s.n_tokens
    K, V, Q = dev(w.K, s.dtype), dev(w.V, s.dtype), dev(w.Q, s.dtype)
    cs, gs = _summ_tables(s)
    hga.build_summaries(p, K, n, 0, n // s.chunk_size, cs, gs)
    seq = torch.from_numpy(w.seq_len).cuda()
    shape_i = lambda k: (s.batch, s.n_kv_heads, 1, max(1, k))
    ci = torch.full(shape_i(s.top_k), -7, dtype=torch.int32, device="cuda")
    gi = torch.full(shape_i(s.top_g), -7, dtype=torch.int32, device="cuda")
    ci2, gi2 = ci.clone(), gi.clone()
    out = torch.empty((s.batch, s.n_q_heads, 1, s.head_dim), device="cuda")
    out2 = torch.empty_like(out)
    hga.decode(p, Q, K, V, n, seq, cs, gs, out, hga.workspace(p, hga.OP_DECODE, 1, n), chunk_idx=ci, group_idx=gi)
    hga.route(p, Q, 1, seq - 1, cs, gs, n, ci2, gi2, hga.workspace(p, hga.OP_ROUTE, 1, n))
    hga.attend(p, Q, 1, seq - 1, K, V, n, gi2, out2, hga.workspace(p, hga.OP_ATTEND, 1, n))
    torch.cuda.synchronize()
    if s.top_k > 0:
        assert torch.equal(ci, ci2)
    if s.top_g > 0:
        assert torch.equal(gi, gi2)
    assert torch.isfinite(out).all()
    assert max_abs(out.cpu().numpy(), out2.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("over", [{}, {"n_tokens": 512}, {"top_k": 0, "top_g": 0, "n_tokens": 512},
                                  {"n_sink": 0, "n_local": 0, "n_tokens": 512},
                                  {"group_size": 64, "top_g": 3, "n_tokens": 512}])
def test_prefill_tiny_fp32(hga, over):
    s = W.spec("tiny_prefill_fp32", **over)
    say(f"[prefill fp32] {over} seed={s.seed}")
    w = W.make(s)
    _run_prefill(hga, s, w)


@pytest.mark.parametrize("over", [{"n_tokens": 2048}, {"n_tokens": 4096, "batch": 1},
                                  {"n_tokens": 2048, "head_dim": 64, "n_q_heads": 16},
                                  {"n_tokens": 2048, "n_q_heads": 8, "top_g": 40},
                                  # k > 64: the routing kernel's general variant (large LDS arrays)
                                  {"n_tokens": 8192, "top_k": 72, "top_g": 96}])
def test_prefill_bf16(hga, over):
    s = W.spec("prefill_32k", **over)
    say(f"[prefill bf16] {over} seed={s.seed}")
    w = W.make(s)
    _run_prefill(hga, s, w)


@pytest.mark.parametrize("over", [
    {},                                                # 4 query heads per KV head, G = 16
    {"n_q_heads": 16, "head_dim": 64},                 # 2 per KV head, d = 64
    {"n_q_heads": 8, "group_size": 32, "top_g": 12},   # 1 per KV head, groups of two 16-key blocks
    {"group_size": 64, "top_g": 5},                    # whole-chunk groups, a partly filled last tile
    {"group_size": 8, "top_g": 24},                    # groups of 8 keys
    {"top_k": 0, "top_g": 0},                          # no routed groups: forced chunks only
    {"n_sink": 0, "n_local": 0, "top_g": 16},          # the current chunk and the routed groups only
    {"n_q_heads": 8, "head_dim": 64, "top_g": 20},     # 1 query head per KV head, d = 64
])
def test_prefill_attend_given_lists(hga, over):
    """hga_attend for a block of prefill queries appended at a position offset
    (chunked prefill), with given group lists that have holes (-1 entries),
    against the oracle's unit blocks: O and the log-sum-exp of every row."""
    s = W.spec("prefill_32k", batch=2, n_tokens=2048, **over)
    say(f"[prefill attend, given lists] {over} seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    B, Hq, H, d, n, C = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size
    m = C // s.group_size
    nq = 512
    nU = nq // C
    q_pos = np.array([1024, 1536], dtype=np.int64)
    Qs = np.stack([w.Q[b, :, q_pos[b]:q_pos[b] + nq] for b in range(B)])
    rng = np.random.default_rng(11)
    gi = np.full((B, H, nU, max(1, s.top_g)), -1, dtype=np.int32)[..., :s.top_g]
    for b in range(B):
        for h in range(H):
            for u in range(nU):
                j = int(q_pos[b]) // C + u
                pool = np.arange(s.n_sink * m, max(s.n_sink, j - s.n_local) * m)
                pick = np.sort(rng.choice(pool, min(s.top_g, len(pool)), replace=False))
                pick = np.where(rng.random(len(pick)) < 0.7, pick, -1)
                gi[b, h, u, :len(pick)] = pick
    p = params_of(s)
    out = torch.empty((B, Hq, nq, d), device="cuda")
    lse = torch.empty((B, Hq, nq), device="cuda")
    ws = hga.workspace(p, hga.OP_ATTEND, nq, n)
    hga.attend(p, dev(Qs, s.dtype), nq, torch.from_numpy(q_pos.astype(np.int32)).cuda(), dev(w.K, s.dtype),
               dev(w.V, s.dtype), n, torch.from_numpy(gi).cuda(), out, ws, lse_out=lse)
    torch.cuda.synchronize()
    Qf, Kf, Vf = f64(Qs, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
    gq = Hq // H
    eo = el = 0.0
    for b in range(B):
        for h in range(H):
            for u in range(nU):
                o, l = O.attend_unit_block(Qf, q_pos, Kf, Vf, gi, cfg, H, b, h, u)
                rows = slice(u * C, (u + 1) * C)
                eo = max(eo, max_abs(got[b, h * gq:(h + 1) * gq, rows], o))
                el = max(el, max_abs(got_lse[b, h * gq:(h + 1) * gq, rows], l))
    say(f"  O max-abs {eo:.3e}  lse max-abs {el:.3e}")
    assert eo <= TOL[s.dtype] and el <= TOL[s.dtype]


def _run_prefill(hga, s, w, units=None):
    cfg = cfg_of(s)
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    p = params_of(s)
    B, H, n = s.batch, s.n_kv_heads, s.n_tokens
    nU = n // s.chunk_size
    cs, gs = _summ_tables(s)
    ci = torch.empty((B, H, nU, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, nU, max(1, s.top_g)), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.n_q_heads, n, s.head_dim), device="cuda")
    ws = hga.workspace(p, hga.OP_PREFILL, n, n)
    hga.prefill(p, dev(w.Q, s.dtype), dev(w.K, s.dtype), dev(w.V, s.dtype), n, cs, gs, out, ws,
                chunk_idx=ci, group_idx=gi)
    torch.cuda.synchronize()
    ocs, ogs = O.build_summaries(Kf, cfg)
    assert max_abs(cs.cpu().numpy(), ocs) < 1e-5
    assert max_abs(gs.cpu().numpy(), ogs) < 1e-5
    q_pos = np.zeros(B, dtype=np.int64)
    or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, H, units=units)
    gi_n = gi.cpu().numpy()[..., :s.top_g] if s.top_g else np.zeros((B, H, nU, 0), np.int32)
    n_units, unique = check_routing(ci.cpu().numpy(), gi_n, or_ci, or_gi, diags, s.top_k, s.top_g)
    got = out.cpu().numpy()
    gq = s.n_q_heads // H
    emax = 0.0
    for (b, h, u) in sorted(diags):
        o, _ = O.attend_unit_block(Qf, q_pos, Kf, Vf, gi_n, cfg, H, b, h, u)
        g = got[b, h * gq:(h + 1) * gq, u * s.chunk_size:(u + 1) * s.chunk_size]
        emax = max(emax, max_abs(g, o))
    say(f"  units {n_units} unique routing {len(unique)}  O max-abs over all units {emax:.3e}")
    assert emax <= TOL[s.dtype]
    return out


@pytest.mark.parametrize("name,over", [
    ("tiny_prefill_fp32", {"n_tokens": 512}),
    ("prefill_32k", {"n_tokens": 512, "n_q_heads": 8, "n_kv_heads": 2}),
    ("prefill_32k", {"n_tokens": 384, "n_q_heads": 4, "n_kv_heads": 4, "head_dim": 64, "top_g": 0,
                     "top_k": 0}),
])
def test_prefill_backward(hga, name, over):
    """dQ, dK, dV of the prefill attention against the oracle's gradients, on
    index sets the oracle routed (given to both sides)."""
    s = W.spec(name, **over)
    say(f"[prefill backward] {name} {over} seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    B, H, n, d = s.batch, s.n_kv_heads, s.n_tokens, s.head_dim
    q_pos = np.zeros(B, dtype=np.int64)
    ocs, ogs = O.build_summaries(Kf, cfg)
    _, or_gi, _ = O.route(Qf, q_pos, ocs, ogs, cfg, H)
    rng = np.random.default_rng(9)
    dO = rng.standard_normal((B, s.n_q_heads, n, d)).astype(np.float32)
    rdQ, rdK, rdV = O.attend_backward(Qf, q_pos, Kf, Vf, or_gi, dO.astype(np.float64), cfg, H)
    p = params_of(s)
    gi = torch.from_numpy(np.ascontiguousarray(or_gi if s.top_g else np.zeros((B, H, n // s.chunk_size, 1)),
                                               dtype=np.int32)).cuda()
    dQ = torch.empty((B, s.n_q_heads, n, d), device="cuda")
    dK = torch.full((B, H, n, d), float("nan"), device="cuda")
    dV = torch.full_like(dK, float("nan"))
    ws = hga.workspace(p, hga.OP_PREFILL_BACKWARD, n, n)
    hga.prefill_backward(p, dev(w.Q, s.dtype), dev(w.K, s.dtype), dev(w.V, s.dtype), n, gi,
                         torch.from_numpy(dO).cuda(), dQ, dK, dV, ws)
    torch.cuda.synchronize()
    for nm, got, ref in (("dQ", dQ, rdQ), ("dK", dK, rdK), ("dV", dV, rdV)):
        e = max_abs(got.cpu().numpy(), ref)
        scale = max(1.0, float(np.abs(ref).max()))
        say(f"  {nm} max-abs {e:.3e} (scale {scale:.2f})")
        assert e <= 1e-4 * scale, nm


def test_offload_decode(hga):
    """Cold tier: K/V in pinned host memory, hot windows in HBM, routed groups copied."""
    s = W.spec("offload_decode_128k", batch=2, n_tokens=16384)
    say(f"[offload decode] seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    p = params_of(s)
    B, H, n, C, d = s.batch, s.n_kv_heads, s.n_tokens, s.chunk_size, s.head_dim
    Kf, Vf, Qf = f64(w.K, s.dtype), f64(w.V, s.dtype), f64(w.Q, s.dtype)
    K_host = W.to_torch(w.K, s.dtype, pin=True)
    V_host = W.to_torch(w.V, s.dtype, pin=True)
    hot_chunks = s.n_sink + s.n_local + 1
    Kt, Vt = W.to_torch(w.K, s.dtype), W.to_torch(w.V, s.dtype)
    K_hot = torch.zeros((B, H, hot_chunks * C, d), dtype=Kt.dtype)
    V_hot = torch.zeros_like(K_hot)
    j = (n - 1) // C
    for c in list(range(s.n_sink)) + list(range(j - s.n_local, j + 1)):
        sl = hga.hot_slot(c, s.n_sink, s.n_local)
        K_hot[:, :, sl * C:(sl + 1) * C] = Kt[:, :, c * C:(c + 1) * C]
        V_hot[:, :, sl * C:(sl + 1) * C] = Vt[:, :, c * C:(c + 1) * C]
    K_hot, V_hot = K_hot.cuda(), V_hot.cuda()
    cs, gs = _summ_tables(s)
    hga.build_summaries(p, dev(w.K, s.dtype), n, 0, j, cs, gs)
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).cuda()
    out = torch.empty((B, s.n_q_heads, 1, d), device="cuda")
    ci = torch.empty((B, H, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device="cuda")
    staging = torch.empty(2 * B * H * s.top_g * s.group_size * d * 2, dtype=torch.uint8, device="cuda")
    ws = hga.workspace(p, hga.OP_DECODE_OFFLOAD, 1, n)
    copy_stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    hga.decode_offload(p, dev(w.Q, s.dtype), K_host, V_host, K_hot, V_hot, n, seq, cs, gs, out,
                       staging, ws, chunk_idx=ci, group_idx=gi, copy_stream=copy_stream.cuda_stream)
    torch.cuda.synchronize()
    ocs, ogs = O.build_summaries(Kf, cfg)
    q_pos = (w.seq_len - 1).astype(np.int64)
    or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, H)
    gi_n = gi.cpu().numpy()
    _, unique = check_routing(ci.cpu().numpy(), gi_n, or_ci, or_gi, diags, s.top_k, s.top_g)
    Oo, _ = O.attend(Qf, q_pos, Kf, Vf, gi_n, cfg, H)
    e = max_abs(out.cpu().numpy(), Oo)
    say(f"  unique routing {len(unique)} of {len(diags)}  O max-abs over all units {e:.3e}")
    assert e <= TOL[s.dtype]
    # the step completed the last chunk: summary built from the hot window
    assert max_abs(cs.cpu().numpy()[:, :, j], ocs[:, :, j]) < 1e-5


@pytest.mark.timeout(300)
def test_offload_decode_full_size_sampled(hga):
    """Cold tier on the full 128K offload workload (B=4, 64/8 heads, top_k 64,
    top_g 128), K/V in pinned host memory: the routing, output and completed
    chunk's summary of six sampled units against the oracle, computed on
    those units' own slices of Q, K and V."""
    s = W.spec("offload_decode_128k")
    say(f"[offload decode full, sampled units] seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    p = params_of(s)
    B, H, n, C, d = s.batch, s.n_kv_heads, s.n_tokens, s.chunk_size, s.head_dim
    gq = s.n_q_heads // H
    K_host = W.to_torch(w.K, s.dtype, pin=True)
    V_host = W.to_torch(w.V, s.dtype, pin=True)
    hot_chunks = s.n_sink + s.n_local + 1
    K_hot = torch.zeros((B, H, hot_chunks * C, d), dtype=K_host.dtype)
    V_hot = torch.zeros_like(K_hot)
    j = (n - 1) // C
    for c in list(range(s.n_sink)) + list(range(j - s.n_local, j + 1)):
        sl = hga.hot_slot(c, s.n_sink, s.n_local)
        K_hot[:, :, sl * C:(sl + 1) * C] = K_host[:, :, c * C:(c + 1) * C]
        V_hot[:, :, sl * C:(sl + 1) * C] = V_host[:, :, c * C:(c + 1) * C]
    K_hot, V_hot = K_hot.cuda(), V_hot.cuda()
    cs, gs = _summ_tables(s)
    hga.build_summaries(p, K_host.cuda(), n, 0, j, cs, gs)
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).cuda()
    out = torch.empty((B, s.n_q_heads, 1, d), device="cuda")
    ci = torch.empty((B, H, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device="cuda")
    staging = torch.empty(2 * B * H * s.top_g * s.group_size * d * 2, dtype=torch.uint8, device="cuda")
    ws = hga.workspace(p, hga.OP_DECODE_OFFLOAD, 1, n)
    copy_stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    hga.decode_offload(p, dev(w.Q, s.dtype), K_host, V_host, K_hot, V_hot, n, seq, cs, gs, out,
                       staging, ws, chunk_idx=ci, group_idx=gi, copy_stream=copy_stream.cuda_stream)
    torch.cuda.synchronize()
    ci_n, gi_n, got, cs_n = ci.cpu().numpy(), gi.cpu().numpy(), out.cpu().numpy(), cs.cpu().numpy()
    assert np.isfinite(got).all()
    rng = np.random.default_rng(s.seed)
    sample = list(zip(rng.choice(B, 6, replace=True).tolist(), rng.choice(H, 6, replace=False).tolist()))
    for b, h in sample:
        Kf, Vf = f64(w.K[b:b + 1, h:h + 1], s.dtype), f64(w.V[b:b + 1, h:h + 1], s.dtype)
        Qf = f64(w.Q[b:b + 1, h * gq:(h + 1) * gq], s.dtype)
        q_pos = (w.seq_len[b:b + 1] - 1).astype(np.int64)
        ocs, ogs = O.build_summaries(Kf, cfg)
        if int(w.seq_len[b]) % C == 0:
            # the step completed chunk j: its summary was built from the hot window
            assert max_abs(cs_n[b, h, j], ocs[0, 0, j]) < 1e-5
        or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, 1)
        _, unique = check_routing(ci_n[b:b + 1, h:h + 1], gi_n[b:b + 1, h:h + 1], or_ci, or_gi, diags,
                                  s.top_k, s.top_g)
        Oo, _ = O.attend(Qf, q_pos, Kf, Vf, gi_n[b:b + 1, h:h + 1], cfg, 1)
        e = max_abs(got[b, h * gq:(h + 1) * gq, 0], Oo[0, :, 0])
        say(f"  unit (b={b}, h={h}): unique routing {bool(unique)}, O max-abs {e:.3e}")
        assert e <= TOL[s.dtype]


@pytest.mark.parametrize("batch,n_tokens,steps", [
    (2, 16384, 6),           # 1024 groups per (b, kv head): the lookup's group-to-slot map
    (1, 8192 * 16 + 4096, 3),  # 8448 groups: above the map's 8192, the slot scan
])
def test_offload_warm_tier_steps(hga, batch, n_tokens, steps):
    """Warm tier over several decode steps with drifting queries: per step the
    output equals the staging path's bit for bit and the oracle's attention over
    the step's routed lists, the LRU state (tags, stamps, clock) and the hit and
    miss counts equal the oracle's LRU fed with the same routed lists, and every
    cached slot holds its group's rows."""
    s = W.spec("offload_decode_128k", batch=batch, n_tokens=n_tokens)
    say(f"[offload warm tier] B={batch} n={n_tokens} seed={s.seed}")
    w = W.make(s)
    p = params_of(s)
    cfg = cfg_of(s)
    Kf, Vf = f64(w.K, s.dtype), f64(w.V, s.dtype)
    B, H, n, C, G, d = s.batch, s.n_kv_heads, s.n_tokens, s.chunk_size, s.group_size, s.head_dim
    K_host = W.to_torch(w.K, s.dtype, pin=True)
    V_host = W.to_torch(w.V, s.dtype, pin=True)
    hot_chunks = s.n_sink + s.n_local + 1
    Kt, Vt = W.to_torch(w.K, s.dtype), W.to_torch(w.V, s.dtype)
    K_hot = torch.zeros((B, H, hot_chunks * C, d), dtype=Kt.dtype)
    V_hot = torch.zeros_like(K_hot)
    j = (n - 1) // C
    for c in list(range(s.n_sink)) + list(range(j - s.n_local, j + 1)):
        sl = hga.hot_slot(c, s.n_sink, s.n_local)
        K_hot[:, :, sl * C:(sl + 1) * C] = Kt[:, :, c * C:(c + 1) * C]
        V_hot[:, :, sl * C:(sl + 1) * C] = Vt[:, :, c * C:(c + 1) * C]
    K_hot, V_hot = K_hot.cuda(), V_hot.cuda()
    cs, gs = _summ_tables(s)
    hga.build_summaries(p, dev(w.K, s.dtype), n, 0, j, cs, gs)
    slots = s.top_g + 8
    warm = hga.warm_state(p, slots)
    ws_w = hga.workspace(p, hga.OP_DECODE_OFFLOAD, 1, n)
    ws_s = hga.workspace(p, hga.OP_DECODE_OFFLOAD, 1, n)
    staging = torch.empty(2 * B * H * s.top_g * G * d * 2, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    gi = torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device="cuda")
    out_w = torch.empty((B, s.n_q_heads, 1, d), device="cuda")
    out_s = torch.empty_like(out_w)
    state = {(b, h): ([-1] * slots, [0] * slots, 0) for b in range(B) for h in range(H)}
    rng = np.random.default_rng(5)
    Q0 = W.to_f64(w.Q, s.dtype).astype(np.float32)
    n_groups_cap = n // G
    tot_hits = tot_miss = 0
    for step in range(steps):
        q = Q0 + 0.5 * rng.standard_normal(Q0.shape).astype(np.float32)
        Qs = W.to_torch(W.bf16_bits(q), "bf16").cuda()
        seq = torch.full((B,), n - 5 + step, dtype=torch.int32, device="cuda")  # positions inside chunk j
        say(f"  step {step}")
        hga.decode_offload_warm(p, Qs, K_host, V_host, K_hot, V_hot, n, seq, cs, gs, out_w, warm, ws_w,
                                group_idx=gi, copy_stream=copy_stream.cuda_stream)
        hga.decode_offload(p, Qs, K_host, V_host, K_hot, V_hot, n, seq, cs, gs, out_s, staging, ws_s,
                           copy_stream=copy_stream.cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(out_w, out_s)
        g_np = gi.cpu().numpy()
        # the output against the oracle's attention over this step's routed lists
        Oo, _ = O.attend(W.to_f64(W.bf16_bits(q), "bf16"), seq.cpu().numpy().astype(np.int64) - 1, Kf, Vf,
                         g_np, cfg, H)
        e = max_abs(out_w.cpu().numpy(), Oo)
        say(f"    O max-abs {e:.3e}")
        assert e <= TOL[s.dtype]
        tags, stamps, clock = warm["tags"].cpu().numpy(), warm["stamps"].cpu().numpy(), warm["clock"].cpu().numpy()
        hits, misses = warm["hits"].cpu().numpy(), warm["misses"].cpu().numpy()
        for b in range(B):
            for h in range(H):
                t0, s0, c0 = state[(b, h)]
                so, mi, t1, s1, c1 = O.warm_lru_step(t0, s0, c0, g_np[b, h, 0], n_groups_cap)
                state[(b, h)] = (t1, s1, c1)
                assert tags[b, h].tolist() == t1 and stamps[b, h].tolist() == s1 and clock[b, h] == c1
                n_valid = sum(1 for x in g_np[b, h, 0] if 0 <= x < n_groups_cap)
                assert misses[b, h] == len(mi) and hits[b, h] == n_valid - len(mi)
                tot_hits += int(hits[b, h])
                tot_miss += int(misses[b, h])
    # every cached slot holds its group's K and V rows
    Kw, Vw = warm["K"].cpu(), warm["V"].cpu()
    for b in range(B):
        for h in range(H):
            for sl, g in enumerate(state[(b, h)][0]):
                if g >= 0:
                    assert torch.equal(Kw[b, h, sl], Kt[b, h, g * G:(g + 1) * G])
                    assert torch.equal(Vw[b, h, sl], Vt[b, h, g * G:(g + 1) * G])
    say(f"  hits {tot_hits} misses {tot_miss}")
    assert tot_hits > 0 and tot_miss > B * H * s.top_g  # both paths taken, evictions included


def test_decode_step_is_deterministic(hga):
    """Repeated decode steps on the same inputs give the same lists and
    bit-identical outputs: the partial results of a unit's workgroups are
    merged in a fixed order, whichever workgroup finishes last."""
    s = W.spec("decode_32k", batch=8, n_tokens=4096)
    say(f"[decode deterministic] seed={s.seed}")
    w = W.make(s)
    p = params_of(s)
    n = s.n_tokens
    K, V, Q = dev(w.K, s.dtype), dev(w.V, s.dtype), dev(w.Q, s.dtype)
    cs, gs = _summ_tables(s)
    hga.build_summaries(p, K, n, 0, n // s.chunk_size, cs, gs)
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).cuda()
    ws = hga.workspace(p, hga.OP_DECODE, 1, n)
    outs, lists = [], []
    for _ in range(6):
        gi = torch.empty((s.batch, s.n_kv_heads, 1, s.top_g), dtype=torch.int32, device="cuda")
        ci = torch.empty((s.batch, s.n_kv_heads, 1, s.top_k), dtype=torch.int32, device="cuda")
        out = torch.empty((s.batch, s.n_q_heads, 1, s.head_dim), device="cuda")
        hga.decode(p, Q, K, V, n, seq - 1, cs, gs, out, ws, chunk_idx=ci, group_idx=gi)
        outs.append(out)
        lists.append((ci, gi))
    torch.cuda.synchronize()
    for out, (ci, gi) in zip(outs[1:], lists[1:]):
        assert torch.equal(ci, lists[0][0]) and torch.equal(gi, lists[0][1])
        assert torch.equal(out, outs[0])


def test_nan_summaries_after_routing_leave_output_unchanged(hga):
    """No summary value enters the output: poisoning the tables after routing
    changes nothing in a second attention pass."""
    s = W.spec("decode_32k", batch=2, n_tokens=4096)
    say(f"[nan summaries] seed={s.seed}")
    w = W.make(s)
    p = params_of(s)
    n = s.n_tokens
    K, V, Q = dev(w.K, s.dtype), dev(w.V, s.dtype), dev(w.Q, s.dtype)
    cs, gs = _summ_tables(s)
    hga.build_summaries(p, K, n, 0, n // s.chunk_size, cs, gs)
    gi = torch.empty((s.batch, s.n_kv_heads, 1, s.top_g), dtype=torch.int32, device="cuda")
    ci = torch.empty((s.batch, s.n_kv_heads, 1, s.top_k), dtype=torch.int32, device="cuda")
    out1 = torch.empty((s.batch, s.n_q_heads, 1, s.head_dim), device="cuda")
    out2 = torch.empty_like(out1)
    ws = hga.workspace(p, hga.OP_DECODE, 1, n)
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).cuda()
    hga.decode(p, Q, K, V, n, seq - 1, cs, gs, out1, ws, chunk_idx=ci, group_idx=gi)
    ws2 = hga.workspace(p, hga.OP_ATTEND, 1, n)
    out0 = torch.empty_like(out1)
    hga.attend(p, Q, 1, seq - 2, K, V, n, gi, out0, ws2)
    cs.fill_(float("nan"))
    gs.fill_(float("nan"))
    hga.attend(p, Q, 1, seq - 2, K, V, n, gi, out2, ws2)
    torch.cuda.synchronize()
    assert torch.isfinite(out2).all()
    # the same attention launch before and after poisoning: bit-identical
    assert torch.equal(out0, out2)
    # the decode step splits the softmax sums differently: equal up to fp32 rounding
    assert max_abs(out1.cpu().numpy(), out2.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("case", ["all_tied_small", "all_tied_large", "two_levels", "nan_rows"])
def test_route_ties_and_nan(hga, case):
    """Selections on hand-made summary tables: exact ties go to the lower index
    (both the bucket path and the radix path of the top-k), NaN scores rank
    with -inf."""
    n = 131072 if case == "all_tied_large" else 8192
    s = W.spec("decode_32k", batch=1, n_q_heads=2, n_kv_heads=1, n_tokens=n, top_k=40, top_g=100)
    say(f"[route ties] {case} n={n}")
    rng = np.random.default_rng(7)
    d, C, G = s.head_dim, s.chunk_size, s.group_size
    nC, m = n // C, C // G
    Q = rng.standard_normal((1, 2, 1, d)).astype(np.float32)
    Qb = W.bf16_bits(Q)
    Qf = W.to_f64(Qb, "bf16")
    if case.startswith("all_tied"):
        cs = np.tile(rng.standard_normal(d), (1, 1, nC, 1))
        gs = np.tile(rng.standard_normal(d), (1, 1, nC * m, 1))
    elif case == "two_levels":
        base = rng.standard_normal(d)
        cs = np.tile(base, (1, 1, nC, 1)) * np.where(rng.random(nC) < 0.5, 1.0, 2.0)[None, None, :, None]
        gs = rng.standard_normal((1, 1, nC * m, d))
    else:
        cs = rng.standard_normal((1, 1, nC, d))
        gs = rng.standard_normal((1, 1, nC * m, d))
        cs[0, 0, rng.choice(nC, 50, replace=False)] = np.nan
        gs[0, 0, rng.choice(nC * m, 200, replace=False)] = np.nan
    cs32, gs32 = cs.astype(np.float32), gs.astype(np.float32)
    cfg = cfg_of(s)
    q_pos = np.array([n - 1], dtype=np.int32)
    or_ci, or_gi, diags = O.route(Qf, q_pos, cs32.astype(np.float64), gs32.astype(np.float64), cfg, 1)
    p = params_of(s)
    ci = torch.empty((1, 1, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((1, 1, 1, s.top_g), dtype=torch.int32, device="cuda")
    ws = hga.workspace(p, hga.OP_ROUTE, 1, n)
    hga.route(p, dev(Qb, "bf16"), 1, torch.from_numpy(q_pos).cuda(), torch.from_numpy(cs32).cuda(),
              torch.from_numpy(gs32).cuda(), n, ci, gi, ws)
    torch.cuda.synchronize()
    g_ci, g_gi = ci.cpu().numpy(), gi.cpu().numpy()
    if case in ("all_tied_small", "all_tied_large", "nan_rows"):
        # ties are exact on both sides: the sets must be identical
        np.testing.assert_array_equal(g_ci, or_ci)
        np.testing.assert_array_equal(g_gi, or_gi)
    else:
        check_routing(g_ci, g_gi, or_ci, or_gi, diags, s.top_k, s.top_g)
    if case.startswith("all_tied"):
        assert g_ci[0, 0, 0].tolist() == list(range(s.n_sink, s.n_sink + s.top_k))


def test_attend_masks_holes_in_group_list(hga):
    """-1 entries anywhere in a group list contribute nothing."""
    s = W.spec("decode_32k", batch=2, n_tokens=4096)
    say(f"[attend holes] seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    rng = np.random.default_rng(3)
    q_pos = (w.seq_len - 1).astype(np.int32)
    j = int(q_pos[0]) // s.chunk_size
    m = s.chunk_size // s.group_size
    gi = np.full((s.batch, s.n_kv_heads, 1, s.top_g), -1, dtype=np.int32)
    for b in range(s.batch):
        for h in range(s.n_kv_heads):
            pool = np.arange(s.n_sink * m, (j - s.n_local) * m)
            pick = np.sort(rng.choice(pool, s.top_g, replace=False))
            keep = rng.random(s.top_g) < 0.6
            gi[b, h, 0] = np.where(keep, pick, -1)
    Oo, _ = O.attend(Qf, q_pos, Kf, Vf, gi, cfg, s.n_kv_heads)
    p = params_of(s)
    out = torch.empty((s.batch, s.n_q_heads, 1, s.head_dim), device="cuda")
    ws = hga.workspace(p, hga.OP_ATTEND, 1, s.n_tokens)
    hga.attend(p, dev(w.Q, s.dtype), 1, torch.from_numpy(q_pos).cuda(), dev(w.K, s.dtype), dev(w.V, s.dtype),
               s.n_tokens, torch.from_numpy(gi).cuda(), out, ws)
    torch.cuda.synchronize()
    e = max_abs(out.cpu().numpy(), Oo)
    say(f"  O max-abs {e:.3e}")
    assert e <= TOL[s.dtype]


def test_route_once_attend_many(hga):
    """Route once, attend many: the group lists that a decode step routes for
    one layer are reused by hga_attend for another layer (its own Q, K, V).
    The second layer's output is the exact attention of its queries over the
    union of its forced windows and the first layer's routed groups."""
    s0 = W.spec("decode_32k", batch=2, n_tokens=4096)
    s1 = W.spec("decode_32k", batch=2, n_tokens=4096, seed=s0.seed + 1)
    say(f"[route once, attend many] seeds={s0.seed},{s1.seed}")
    w0, w1 = W.make(s0), W.make(s1)
    cfg = cfg_of(s1)
    p = params_of(s0)
    n = s0.n_tokens
    seq = torch.from_numpy(w0.seq_len).cuda()
    K0 = dev(w0.K, s0.dtype)
    cs, gs = _summ_tables(s0)
    hga.build_summaries(p, K0, n, 0, n // s0.chunk_size, cs, gs)
    gi = torch.full((s0.batch, s0.n_kv_heads, 1, s0.top_g), -7, dtype=torch.int32, device="cuda")
    out0 = torch.empty((s0.batch, s0.n_q_heads, 1, s0.head_dim), device="cuda")
    hga.decode(p, dev(w0.Q, s0.dtype), K0, dev(w0.V, s0.dtype), n, seq, cs, gs, out0,
               hga.workspace(p, hga.OP_DECODE, 1, n), group_idx=gi)
    out1 = torch.empty_like(out0)
    hga.attend(p, dev(w1.Q, s1.dtype), 1, seq - 1, dev(w1.K, s1.dtype), dev(w1.V, s1.dtype), n, gi, out1,
               hga.workspace(p, hga.OP_ATTEND, 1, n))
    torch.cuda.synchronize()
    gin = gi.cpu().numpy()
    assert (gin >= 0).sum() > 0
    Oo, _ = O.attend(f64(w1.Q, s1.dtype), (w1.seq_len - 1).astype(np.int32), f64(w1.K, s1.dtype),
                     f64(w1.V, s1.dtype), gin, cfg, s1.n_kv_heads)
    e = max_abs(out1.cpu().numpy(), Oo)
    say(f"  layer-1 O max-abs {e:.3e}")
    assert e <= TOL[s1.dtype]


def test_prefill_full_size_32k(hga):
    """The benchmarked prefill workload at full size (32K tokens, 32/8 heads),
    checked on a sample of units spread over the sequence and the heads."""
    s = W.spec("prefill_32k")
    say(f"[prefill full] prefill_32k seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    p = params_of(s)
    B, H, n, C = s.batch, s.n_kv_heads, s.n_tokens, s.chunk_size
    nU = n // C
    cs, gs = _summ_tables(s)
    ci = torch.empty((B, H, nU, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, nU, s.top_g), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.n_q_heads, n, s.head_dim), device="cuda")
    ws = hga.workspace(p, hga.OP_PREFILL, n, n)
    hga.prefill(p, dev(w.Q, s.dtype), dev(w.K, s.dtype), dev(w.V, s.dtype), n, cs, gs, out, ws,
                chunk_idx=ci, group_idx=gi)
    torch.cuda.synchronize()
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    ocs, ogs = O.build_summaries(Kf, cfg)
    assert max_abs(cs.cpu().numpy(), ocs) < 1e-5
    assert max_abs(gs.cpu().numpy(), ogs) < 1e-5
    rng = np.random.default_rng(0)
    units = [(0, h, u) for h in range(H) for u in sorted(rng.choice(nU, 5, replace=False).tolist())]
    units += [(0, 0, 0), (0, 3, 1), (0, 5, 2), (0, 7, nU - 1)]
    q_pos = np.zeros(B, dtype=np.int64)
    or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, H, units=units)
    gi_n = gi.cpu().numpy()
    n_units, unique = check_routing(ci.cpu().numpy(), gi_n, or_ci, or_gi, diags, s.top_k, s.top_g)
    got = out.cpu().numpy()
    gq = s.n_q_heads // H
    emax = 0.0
    for (b, h, u) in sorted(diags):
        o, _ = O.attend_unit_block(Qf, q_pos, Kf, Vf, gi_n, cfg, H, b, h, u)
        emax = max(emax, max_abs(got[b, h * gq:(h + 1) * gq, u * C:(u + 1) * C], o))
    say(f"  sampled units {n_units} unique routing {len(unique)}  O max-abs over all sampled units {emax:.3e}")
    assert emax <= TOL[s.dtype]
    assert np.isfinite(got).all()


def test_decode_streaming_heads_full_size(hga):
    """Streaming heads (top_k = top_g = 0: the sink, local and current chunks
    only) on the full decode_32k shape, in the one-launch decode step, against
    the oracle."""
    s = W.spec("decode_32k", top_k=0, top_g=0)
    say(f"[decode streaming heads, full size] seed={s.seed}")
    w = W.make(s)
    _run_decode_e2e(hga, s, w)


@pytest.mark.parametrize("path", ["decode_step", "decode_splitk", "prefill_pipe", "prefill_g8"])
def test_attend_given_lists_with_repeats_and_forced_groups(hga, path):
    """hga_attend with lists as a caller might give them (any order, holes,
    repeated groups, groups inside the sink, local and current chunks, after
    the query's chunk, past the cache): every token counts once, against the
    oracle's set union.  decode_step: one query per sequence (the one-launch
    kernel); decode_splitk: the same with the log-sum-exp requested (the
    split-K kernel); prefill_pipe / prefill_g8: a block of prefill queries
    (groups of 16 and of 8 keys)."""
    over = {"group_size": 8, "top_g": 40} if path == "prefill_g8" else {}
    decode = path.startswith("decode")
    s = W.spec("decode_32k" if decode else "prefill_32k", batch=2, n_tokens=4096, **over)
    say(f"[attend given lists, messy] {path} seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    B, Hq, H, d, n, C = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size
    rng = np.random.default_rng(17)
    p = params_of(s)
    if decode:
        q_pos = np.array([n - 1, 2500], dtype=np.int64)
        Qs, nq, nU = w.Q, 1, 1
        gi = messy_group_lists(rng, B, H, 1, s.top_g, lambda b, u: int(q_pos[b]) // C, s, n)
    else:
        q_pos = np.array([1024, 2048], dtype=np.int64)
        nq = 512
        nU = nq // C
        Qs = np.stack([w.Q[b, :, q_pos[b]:q_pos[b] + nq] for b in range(B)])
        gi = messy_group_lists(rng, B, H, nU, s.top_g, lambda b, u: int(q_pos[b]) // C + u, s, n)
    out = torch.empty((B, Hq, nq, d), device="cuda")
    lse = torch.empty((B, Hq, nq), device="cuda") if path != "decode_step" else None
    ws = hga.workspace(p, hga.OP_ATTEND, nq, n)
    gi_d = torch.from_numpy(gi).cuda()
    hga.attend(p, dev(Qs, s.dtype), nq, torch.from_numpy(q_pos.astype(np.int32)).cuda(), dev(w.K, s.dtype),
               dev(w.V, s.dtype), n, gi_d, out, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(gi_d.cpu(), torch.from_numpy(gi))  # the caller's list is left as given
    Qf, Kf, Vf = f64(Qs, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    got = out.cpu().numpy()
    if decode:
        Oo, lo = O.attend(Qf, q_pos, Kf, Vf, gi, cfg, H)
        eo = max_abs(got, Oo)
        el = max_abs(lse.cpu().numpy(), lo) if lse is not None else 0.0
    else:
        gq = Hq // H
        eo = el = 0.0
        for b in range(B):
            for h in range(H):
                for u in range(nU):
                    o, l = O.attend_unit_block(Qf, q_pos, Kf, Vf, gi, cfg, H, b, h, u)
                    rows = slice(u * C, (u + 1) * C)
                    eo = max(eo, max_abs(got[b, h * gq:(h + 1) * gq, rows], o))
                    el = max(el, max_abs(lse.cpu().numpy()[b, h * gq:(h + 1) * gq, rows], l))
    say(f"  O max-abs {eo:.3e}  lse max-abs {el:.3e}")
    assert eo <= TOL[s.dtype] and el <= TOL[s.dtype]


def test_prefill_backward_given_lists_with_repeats(hga):
    """hga_prefill_backward with messy caller lists (repeats, forced-chunk and
    later groups, holes, ids past the cache): gradients of the attention over
    the set union, against the oracle."""
    s = W.spec("prefill_32k", n_tokens=512, n_q_heads=8, n_kv_heads=2)
    say(f"[prefill backward, messy lists] seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    Qf, Kf, Vf = f64(w.Q, s.dtype), f64(w.K, s.dtype), f64(w.V, s.dtype)
    B, H, n, d, C = s.batch, s.n_kv_heads, s.n_tokens, s.head_dim, s.chunk_size
    nU = n // C
    rng = np.random.default_rng(23)
    gi = messy_group_lists(rng, B, H, nU, s.top_g, lambda b, u: u, s, n)
    dO = rng.standard_normal((B, s.n_q_heads, n, d)).astype(np.float32)
    rdQ, rdK, rdV = O.attend_backward(Qf, np.zeros(B, np.int64), Kf, Vf, gi, dO.astype(np.float64), cfg, H)
    p = params_of(s)
    dQ = torch.empty((B, s.n_q_heads, n, d), device="cuda")
    dK = torch.full((B, H, n, d), float("nan"), device="cuda")
    dV = torch.full_like(dK, float("nan"))
    ws = hga.workspace(p, hga.OP_PREFILL_BACKWARD, n, n)
    hga.prefill_backward(p, dev(w.Q, s.dtype), dev(w.K, s.dtype), dev(w.V, s.dtype), n, torch.from_numpy(gi).cuda(),
                         torch.from_numpy(dO).cuda(), dQ, dK, dV, ws)
    torch.cuda.synchronize()
    for nm, got, ref in (("dQ", dQ, rdQ), ("dK", dK, rdK), ("dV", dV, rdV)):
        e = max_abs(got.cpu().numpy(), ref)
        scale = max(1.0, float(np.abs(ref).max()))
        say(f"  {nm} max-abs {e:.3e} (scale {scale:.2f})")
        assert e <= 1e-4 * scale, nm


@pytest.mark.timeout(300)
def test_prefill_64k_single_call_sampled(hga):
    """A 64K-token causal prefill in one hga_prefill call (B=1, 32/8 heads,
    d=128): the summary tables in full and the routing and output of sampled
    units against the oracle."""
    s = W.spec("prefill_32k", n_tokens=65536)
    say(f"[prefill 64K, one call, sampled units] seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    p = params_of(s)
    B, H, n, C = s.batch, s.n_kv_heads, s.n_tokens, s.chunk_size
    nU = n // C
    cs, gs = _summ_tables(s)
    ci = torch.empty((B, H, nU, s.top_k), dtype=torch.int32, device="cuda")
    gi = torch.empty((B, H, nU, s.top_g), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.n_q_heads, n, s.head_dim), device="cuda")
    ws = hga.workspace(p, hga.OP_PREFILL, n, n)
    hga.prefill(p, dev(w.Q, s.dtype), dev(w.K, s.dtype), dev(w.V, s.dtype), n, cs, gs, out, ws,
                chunk_idx=ci, group_idx=gi)
    torch.cuda.synchronize()
    # float32 views of the bf16 values (exact); the oracle converts the slices it reads to float64
    Qf = W.bf16_to_f32(w.Q)
    Kf, Vf = W.bf16_to_f32(w.K), W.bf16_to_f32(w.V)
    ocs, ogs = O.build_summaries(Kf, cfg)
    assert max_abs(cs.cpu().numpy(), ocs) < 1e-5
    assert max_abs(gs.cpu().numpy(), ogs) < 1e-5
    rng = np.random.default_rng(1)
    units = [(0, h, u) for h in range(H) for u in sorted(rng.choice(nU, 3, replace=False).tolist())]
    units += [(0, 0, nU - 1), (0, 7, nU // 2)]
    q_pos = np.zeros(B, dtype=np.int64)
    or_ci, or_gi, diags = O.route(Qf, q_pos, ocs, ogs, cfg, H, units=units)
    gi_n = gi.cpu().numpy()
    n_units, unique = check_routing(ci.cpu().numpy(), gi_n, or_ci, or_gi, diags, s.top_k, s.top_g)
    gq = s.n_q_heads // H
    emax = 0.0
    for (b, h, u) in sorted(diags):
        o, _ = O.attend_unit_block(Qf, q_pos, Kf, Vf, gi_n, cfg, H, b, h, u)
        emax = max(emax, max_abs(out[b, h * gq:(h + 1) * gq, u * C:(u + 1) * C].cpu().numpy(), o))
    say(f"  sampled units {n_units} unique routing {len(unique)}  O max-abs {emax:.3e}")
    assert emax <= TOL[s.dtype]
    assert torch.isfinite(out).all()


def test_prefill_backward_full_size_sampled(hga):
    """The benchmarked backward at full size (32K tokens, 32/8 heads, the lists
    of the GPU's own routing), against the oracle's gradients on samples: dQ of
    whole query chunks (a row's gradient depends on its own visible set only),
    and dK, dV of whole key chunks, summed over every query chunk that sees
    them (routed or forced, any KV head)."""
    s = W.spec("prefill_32k")
    say(f"[prefill backward full] prefill_32k seed={s.seed}")
    w = W.make(s)
    cfg = cfg_of(s)
    p = params_of(s)
    B, H, n, C, d, m = s.batch, s.n_kv_heads, s.n_tokens, s.chunk_size, s.head_dim, s.chunk_size // s.group_size
    nU = n // C
    cs, gs = _summ_tables(s)
    gi = torch.empty((B, H, nU, s.top_g), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.n_q_heads, n, d), device="cuda")
    Qd, Kd, Vd = dev(w.Q, s.dtype), dev(w.K, s.dtype), dev(w.V, s.dtype)
    hga.prefill(p, Qd, Kd, Vd, n, cs, gs, out, hga.workspace(p, hga.OP_PREFILL, n, n), group_idx=gi)
    g = torch.Generator(device="cuda").manual_seed(s.seed + 5)
    dO = torch.randn((B, s.n_q_heads, n, d), device="cuda", generator=g)
    dQ = torch.empty_like(dO)
    dK = torch.empty((B, H, n, d), device="cuda")
    dV = torch.empty_like(dK)
    hga.prefill_backward(p, Qd, Kd, Vd, n, gi, dO, dQ, dK, dV, hga.workspace(p, hga.OP_PREFILL_BACKWARD, n, n))
    torch.cuda.synchronize()
    gi_n = gi.cpu().numpy()
    dO_n = dO.cpu().numpy().astype(np.float64)
    Kf, Vf = f64(w.K, s.dtype), f64(w.V, s.dtype)
    Qb = w.Q  # bf16 bits; rows converted per sampled chunk

    def oracle_block(j):
        """The oracle's gradients from the 64 query rows of chunk j (all heads)."""
        rows = slice(j * C, (j + 1) * C)
        Qj = W.to_f64(Qb[:, :, rows], s.dtype)
        return O.attend_backward(Qj, np.full(B, j * C, dtype=np.int64), Kf, Vf, gi_n[:, :, j:j + 1],
                                 dO_n[:, :, rows], cfg, H)

    # dQ of sampled query chunks
    eq, scq = 0.0, 1.0
    got_q = dQ.cpu().numpy()
    for j in (2, 257, nU - 1):
        rdQ, _, _ = oracle_block(j)
        eq = max(eq, max_abs(got_q[:, :, j * C:(j + 1) * C], rdQ))
        scq = max(scq, float(np.abs(rdQ).max()))
    say(f"  dQ (3 query chunks) max-abs {eq:.3e} (scale {scq:.2f})")
    assert eq <= 1e-4 * scq

    # dK, dV of sampled key chunks: every query chunk that sees a block of c
    got_k, got_v = dK.cpu().numpy(), dV.cpu().numpy()
    for c in (nU - 6, 3 * nU // 4):
        seers = []
        for j in range(c, nU):
            forced = c < s.n_sink or j - c <= s.n_local
            routed = any((x >= 0 and x // m == c) for x in gi_n[:, :, j].ravel())
            if forced or routed:
                seers.append(j)
        rK = np.zeros((B, H, C, d))
        rV = np.zeros((B, H, C, d))
        for j in seers:
            _, pk, pv = oracle_block(j)
            rK += pk[:, :, c * C:(c + 1) * C]
            rV += pv[:, :, c * C:(c + 1) * C]
        ek = max_abs(got_k[:, :, c * C:(c + 1) * C], rK)
        ev = max_abs(got_v[:, :, c * C:(c + 1) * C], rV)
        sk, sv = max(1.0, float(np.abs(rK).max())), max(1.0, float(np.abs(rV).max()))
        say(f"  key chunk {c} (seen by {len(seers)} query chunks): dK max-abs {ek:.3e} (scale {sk:.2f}), "
            f"dV max-abs {ev:.3e} (scale {sv:.2f})")
        assert ek <= 1e-4 * sk and ev <= 1e-4 * sv
    assert np.isfinite(got_q).all() and np.isfinite(got_k).all() and np.isfinite(got_v).all()
