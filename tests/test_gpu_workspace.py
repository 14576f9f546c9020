"""GPU: one workspace shared by calls of different shapes, in a row.

The Top-K merges count list arrivals in the workspace's counter region, which
must be zero before a workspace's first use and which every call leaves zero
again; calls of at most 64 queries plan inside the indexer and rely on that,
larger ones run the planning kernel.  Here one workspace, cleared once by
dsa_workspace_init, serves a sequence of indexer, layer and attention calls of
different shapes (one query list per query, lists merged in one and in two
levels, paired speculative queries, a prefill chunk planned by its own
kernel); every call must give exactly the indices a fresh workspace gives,
and the first calls are checked against the oracle."""
import numpy as np
import pytest
import torch

from gpu_cases import check_queries, say
from sparse_attention_07_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_attention_07_amd import dsa
DEV = "cuda"


def spec(name, **kw):
    base = dict(H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128)
    base.update(kw)
    return synth.CaseSpec(name, **base)


def topk_on(case, workspace=None):
    return dsa.indexer_topk(case.q_idx, case.w, case.k_idx_pool, case.block_table, case.seq_lens, case.spec.K,
                            q_idx_scale=case.q_idx_scale, q_seq=case.q_seq, q_visible=case.q_visible,
                            max_q_per_seq=case.max_q_per_seq, workspace=workspace)


def layer_on(case, workspace):
    """dsa_layer through the C ABI on the given (shared) workspace."""
    lay = dsa.layer_from_case(case)
    need = lay.workspace.numel()
    assert workspace.numel() >= need
    out = torch.empty_like(lay.out)
    idx = torch.empty_like(lay.indices)
    st = dsa.LIB.dsa_layer(dsa.ctypes.byref(lay.idx), dsa.ctypes.byref(lay.mla), lay.K, lay.scale,
                           dsa._ptr(idx), dsa._ptr(out), dsa._ptr(workspace), workspace.numel(), dsa._stream())
    assert st == 0, dsa.LIB.dsa_status_str(st)
    return idx, out


def test_one_workspace_many_shapes():
    cases = {
        # 40000 keys: ten 4096-key lists, merged in two levels (per-query counter)
        "two_level": synth.build_case(spec("ws_two_level", lens=[40000, 1000, 3], seed=61), device=DEV),
        # 8 speculative queries on one sequence: paired queries, their lists merged in one level
        "pairs": synth.build_case(spec("ws_pairs", lens=[20000, 9000], queries_per_seq=[8, 1], seed=62),
                                  device=DEV),
        # 2048 queries of a prefill chunk: more than 64, planned by the planning kernel
        "prefill": synth.build_case(spec("ws_prefill", prefill=(6000, 2048), K=512, H=64, seed=63), device=DEV,
                                    prefill_chunk=1),
        # one query per list: no merge at all
        "single": synth.build_case(spec("ws_single", idx_dtype="bf16", lens=[3000, 64, 4000], seed=64),
                                   device=DEV),
    }
    # fresh workspaces (each initialised on allocation): the reference results
    fresh = {k: topk_on(c) for k, c in cases.items()}
    need = 0
    for c in cases.values():
        lay = dsa.layer_from_case(c)
        need = max(need, lay.workspace.numel())
        del lay
    ws = dsa.workspace_init(torch.empty(need, dtype=torch.uint8, device=DEV))
    order = ["two_level", "pairs", "prefill", "two_level", "single", "pairs", "prefill", "two_level"]
    for step, name in enumerate(order):
        c = cases[name]
        got = topk_on(c, workspace=ws)
        torch.cuda.synchronize()
        same = torch.equal(got, fresh[name])
        say(f"  call {step} ({name}, T={c.T}) on the shared workspace: indices equal to a fresh workspace's: {same}")
        assert same, f"call {step} ({name}) on the shared workspace differs from a fresh workspace"
        # the layer and the attention alone on the same workspace, between indexer calls
        if step in (1, 4):
            idx, out = layer_on(c, ws)
            torch.cuda.synchronize()
            assert torch.equal(idx, fresh[name])
            o2 = dsa.sparse_mla_attn(c.q, c.kv_pool, idx, c.spec.scale, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(o2, out), "attention alone on the shared workspace differs from the layer's"
    # every query of the merge-heavy cases against the oracle
    for name in ("two_level", "pairs"):
        c = cases[name]
        idx, out = layer_on(c, ws)
        torch.cuda.synchronize()
        say(f"[oracle] {name}")
        check_queries(c, idx, out, range(c.T))
    # the counter region is zero again after the last call
    torch.cuda.synchronize()
    head = ws[: dsa.WS_RESERVED_BYTES].cpu().numpy()
    assert not np.any(head), "the counter region is not clear after the calls"
