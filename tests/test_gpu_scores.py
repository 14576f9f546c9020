"""GPU check of the indexer's fused scores, float against float (the pages'
alignment order puts the sparse index selection right after the states:
"Day 0 Inference Adaptation and Performance Optimization for Hybrid Attention
LLMs", section "Engineering Execution", item 2).

dsa_indexer_scores runs the indexer kernel of dsa_indexer_topk and writes each
score as the selection compares it.  The oracle's fp64 score is the reference.
Bound: every product of the dot products is exact in fp32 (bf16 x bf16 and
e4m3 x e4m3 have at most 16 significant bits), so the kernel's error comes
from fp32 additions and multiplications, at most a few hundred of them along
any path (128-term dot products, 64 heads, the key and query scales); each
rounds by at most 2^-24 of a value bounded by
A[p] = sum_h |w'_h| * sum_d |q_hd k_pd| (dequantized).  The test allows
2^-16 * A[p]: 256 times the first-order bound of 256 roundings; a dropped or
doubled head, a wrong scale or a wrong key moves the score by about A / 64 or
more."""
import numpy as np
import pytest
import torch

from gpu_cases import query_case, say
from oracle import dsa_oracle as O
from sparse_attention_07_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_attention_07_amd import dsa
DEV = "cuda"


def spec(name, **kw):
    base = dict(H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=16)
    base.update(kw)
    return synth.CaseSpec(name, **base)


CASES = [
    spec("sc_bf16_d64", idx_dtype="bf16", D_idx=64, H_idx=4, lens=[4096, 777], seed=61),
    spec("sc_bf16_d128", idx_dtype="bf16", lens=[9000, 64, 3000], seed=62),
    spec("sc_fp8", lens=[20000, 1000, 5], seed=63),
    spec("sc_fp8_16heads", H_idx=16, lens=[7000, 130], seed=64),
    spec("sc_mxfp8", idx_dtype="mxfp8", lens=[12000, 2500], seed=65),
    # several queries per sequence: two queries share each key load
    spec("sc_fp8_pairs", lens=[6000, 3000], queries_per_seq=[9, 8], seed=66),
    spec("sc_bf16_pairs", idx_dtype="bf16", lens=[5000], queries_per_seq=[11], seed=67),
]


@pytest.mark.parametrize("sp", CASES, ids=[c.name for c in CASES])
def test_indexer_scores_match_oracle(sp):
    say(f"[case] {sp.name}")
    case = synth.build_case(sp, device=DEV)
    got = dsa.indexer_scores(case.q_idx, case.w, case.k_idx_pool, case.block_table, case.seq_lens,
                             q_idx_scale=case.q_idx_scale, q_seq=case.q_seq, q_visible=case.q_visible,
                             max_q_per_seq=case.max_q_per_seq)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    worst = 0.0
    for t in range(case.T):
        d, phys = query_case(case, t, kv_positions=())
        S, _ = O.query_scores(d, 0)
        n = S.shape[0]
        # magnitude bound A[p] from the dequantized operands
        b, _, slots = O.query_geometry(d, 0)
        qv = O.index_query(d["q_idx"][0], None if d["q_idx_scale"] is None else d["q_idx_scale"][0], d["idx_dtype"])
        keys = O.index_keys(d["k_idx_pool"], d["idx_dtype"], d["D_idx"], slots)
        A = (np.abs(keys) @ np.abs(qv).T) @ np.abs(np.asarray(d["w"][0], np.float64))
        g = got[t, :n]
        assert np.isfinite(g).all(), f"query {t}: a visible position has no score"
        assert np.isnan(got[t, n:]).all(), f"query {t}: a score past the horizon was written"
        err = np.abs(g - S)
        tol = 2.0 ** -16 * A + 1e-30
        r = float((err / tol).max()) if n else 0.0
        worst = max(worst, r)
        assert (err <= tol).all(), f"query {t}: worst error {err.max():.3g} at {int(err.argmax())}, ratio {r:.3g}"
    say(f"  {case.T} queries: worst error / bound = {worst:.3g}")
