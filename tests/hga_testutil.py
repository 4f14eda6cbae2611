"""Shared helpers of the GPU parity tests: moving seeded workloads to the device,
running the oracle on the same rounded inputs, and the parity rules.

Parity rules (floating-point routing decides integers, so index sets are unique
only where the scores are clearly separated):
  1. chunk index sets are bit-exact for every unit whose oracle gap at the k-th
     boundary exceeds 1e-3 (relative to the larger of the two boundary scores);
     group sets are compared where the chunk sets agree and the group gap
     exceeds 1e-3;
  2. where a gap is <= 1e-3 the GPU's selection must still be a valid one: the
     right count, and no selected candidate scoring clearly below an unselected one;
  3. the output O of every row is compared with the oracle's attention over the
     GPU's own index lists (which rules 1 and 2 have just validated): max-abs
     2e-3 for bf16 inputs, 1e-5 for fp32.  Where the routing is unique those
     lists are the oracle's own, so O then also equals the end-to-end oracle.
"""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle as O
from hierarchical_sparse_attention_build_amd import workloads as W

GAP = 1e-3
TOL = {"bf16": 2e-3, "fp32": 1e-5}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def cfg_of(s: W.Spec) -> O.HGAConfig:
    return O.HGAConfig(**W.hga_config_kwargs(s))


def params_of(s: W.Spec, out_dtype=None):
    from hierarchical_sparse_attention_build_amd import hga
    dt = hga.HGA_BF16 if s.dtype == "bf16" else hga.HGA_F32
    return hga.params(s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.chunk_size, s.group_size,
                      s.n_sink, s.n_local, s.top_k, s.top_g, s.rope_base, s.hf_threshold,
                      qkv_dtype=dt, out_dtype=hga.HGA_F32 if out_dtype is None else out_dtype)


def dev(arr, dtype, device="cuda"):
    return W.to_torch(arr, dtype).to(device)


def f64(arr, dtype):
    return W.to_f64(arr, dtype)


def check_routing(gpu_ci, gpu_gi, or_ci, or_gi, diags, top_k, top_g):
    """Rules 1 and 2.  Returns (units, units with unique routing) and the set of
    unique units."""
    unique = set()
    n_units = 0
    for key, dg in diags.items():
        b, h, u = key
        n_units += 1
        g_ci = gpu_ci[b, h, u]
        o_ci = or_ci[b, h, u]
        ncand = len(dg["chunk_cand"])
        # rule 2: count and validity of the chunk selection
        cnt = int((g_ci >= 0).sum())
        assert cnt == min(top_k, ncand), (key, cnt, ncand)
        sel = g_ci[:cnt]
        assert np.all(np.diff(sel) > 0), (key, "not ascending", sel)
        assert np.all(g_ci[cnt:] == -1)
        if ncand:
            sc = dict(zip(dg["chunk_cand"].tolist(), dg["chunk_scores"].tolist()))
            assert set(sel.tolist()) <= set(sc), (key, "selected a non-candidate")
            if 0 < cnt < ncand:
                worst_in = min(sc[c] for c in sel.tolist())
                best_out = max(v for c, v in sc.items() if c not in set(sel.tolist()))
                den = max(abs(worst_in), abs(best_out), 1e-30)
                assert (best_out - worst_in) / den <= GAP, (key, worst_in, best_out)
        chunk_same = np.array_equal(g_ci, o_ci)
        if dg["chunk_gap"] > GAP:
            assert chunk_same, (key, "chunk set differs with gap", dg["chunk_gap"], g_ci, o_ci)
        if not chunk_same:
            continue
        g_gi = gpu_gi[b, h, u]
        o_gi = or_gi[b, h, u]
        gcnt = int((g_gi >= 0).sum())
        assert gcnt == min(top_g, len(dg["group_cand"])), (key, gcnt)
        gsel = g_gi[:gcnt]
        assert np.all(np.diff(gsel) > 0)
        gsc = dict(zip(dg["group_cand"].tolist(), dg["group_scores"].tolist()))
        assert set(gsel.tolist()) <= set(gsc)
        if 0 < gcnt < len(gsc):
            worst_in = min(gsc[g] for g in gsel.tolist())
            best_out = max(v for g, v in gsc.items() if g not in set(gsel.tolist()))
            den = max(abs(worst_in), abs(best_out), 1e-30)
            assert (best_out - worst_in) / den <= GAP, (key, "group", worst_in, best_out)
        group_same = np.array_equal(g_gi, o_gi)
        if dg["group_gap"] > GAP:
            assert group_same, (key, "group set differs with gap", dg["group_gap"], g_gi, o_gi)
        if dg["chunk_gap"] > GAP and dg["group_gap"] > GAP:
            unique.add(key)
    return n_units, unique


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def messy_group_lists(rng, B, H, n_units, top_g, unit_chunk, s, n_cap):
    """Group lists as a caller might pass them: candidate groups in random order,
    mixed with holes, repeats, groups inside the sink, local and current chunks,
    groups after the query chunk and ids past the cache.  unit_chunk(b, u) is the
    query chunk of unit u of sequence b."""
    m = s.chunk_size // s.group_size
    n_groups = n_cap // s.group_size
    gi = np.full((B, H, n_units, top_g), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for u in range(n_units):
                j = unit_chunk(b, u)
                pool = np.arange(s.n_sink * m, max(s.n_sink, j - s.n_local) * m)
                k = min(len(pool), max(1, top_g // 2))
                lst = list(rng.choice(pool, k, replace=False)) if k else []
                extra = [int(rng.integers(0, max(1, s.n_sink) * m)),          # sink chunk
                         j * m + int(rng.integers(0, m)),                     # current chunk
                         max(0, j - 1) * m + int(rng.integers(0, m)),         # local window
                         (j + 1) * m + int(rng.integers(0, m)),               # after the query chunk
                         n_groups + 3, -1, -5]
                if lst:
                    extra += [int(lst[0]), int(lst[-1])]                      # repeats
                lst = [int(x) for x in lst] + extra
                rng.shuffle(lst)
                lst = lst[:top_g]
                gi[b, h, u, :len(lst)] = lst
    return gi
