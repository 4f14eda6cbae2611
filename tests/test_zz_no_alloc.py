"""hga_decode_static (the decode step with the library's static device scratch,
no workspace) against hga_decode on the same inputs, through the C ABI: calls
in a row on one device, the later ones with smaller inputs, so that each call
finds the scratch as the previous, larger one left it."""
import numpy as np
import pytest

from hierarchical_sparse_attention_build_amd import workloads as W
from tests.hga_testutil import TOL, dev, max_abs, params_of, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_sparse_attention_build_amd import hga as H
    H.lib()
    return H


def _decode_both(hga, s, lists):
    w = W.make(s)
    p = params_of(s)
    B, H, n, C, d = s.batch, s.n_kv_heads, s.n_tokens, s.chunk_size, s.head_dim
    K, V, Q = dev(w.K, s.dtype), dev(w.V, s.dtype), dev(w.Q, s.dtype)
    nC = n // C
    m = C // s.group_size
    cs = torch.zeros((B, H, nC, d), device="cuda")
    gs = torch.zeros((B, H, nC * m, d), device="cuda")
    hga.build_summaries(p, K, n, 0, nC, cs, gs)
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).cuda()
    # hga_decode writes the completed chunk's summaries: each call gets its own tables
    cs2, gs2 = cs.clone(), gs.clone()
    out_r = torch.empty((B, s.n_q_heads, 1, d), device="cuda")
    out_s = torch.full_like(out_r, float("nan"))
    ci_r = torch.empty((B, H, 1, s.top_k), dtype=torch.int32, device="cuda")
    gi_r = torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device="cuda")
    ci_s = torch.full_like(ci_r, -7) if lists else None
    gi_s = torch.full_like(gi_r, -7) if lists else None
    hga.decode(p, Q, K, V, n, seq, cs, gs, out_r, hga.workspace(p, hga.OP_DECODE, 1, n),
               chunk_idx=ci_r, group_idx=gi_r)
    hga.decode_static(p, Q, K, V, n, seq, cs2, gs2, out_s, chunk_idx=ci_s, group_idx=gi_s)
    torch.cuda.synchronize()
    e = max_abs(out_s.cpu().numpy(), out_r.cpu().numpy())
    say(f"  B={B} n={n}: O max-abs {e:.3e} (bit-identical: {torch.equal(out_s, out_r)})")
    assert torch.isfinite(out_s).all()
    assert e <= TOL[s.dtype]
    if lists:
        assert torch.equal(ci_s, ci_r) and torch.equal(gi_s, gi_r)
    assert torch.equal(cs2, cs) and torch.equal(gs2, gs)


def test_decode_static_matches_decode_on_calls_in_a_row(hga):
    say("[decode static] calls in a row, larger then smaller inputs")
    for over, lists in (({"batch": 8, "n_tokens": 8192}, True),
                        ({"batch": 2, "n_tokens": 4096}, False),
                        ({"batch": 3, "n_tokens": 2048, "n_q_heads": 16, "n_kv_heads": 8}, True),
                        ({"batch": 1, "n_tokens": 1024, "top_k": 0, "top_g": 0}, False)):
        s = W.spec("decode_32k", **over)
        say(f"  {over} lists={lists} seed={s.seed}")
        _decode_both(hga, s, lists)
