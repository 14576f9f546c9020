"""Helpers for GPU parity tests: run the HIP path through the C ABI and check
sampled (or all) queries against the CPU oracle with the comparison rules."""
from __future__ import annotations

import numpy as np
import torch

from dsa_check import check_index_row, check_outputs
from oracle import dsa_oracle as O
from sparse_attention_07_amd import synth


def say(*a):
    print(*a, flush=True)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def latent_pages(case: synth.Case, t: int, positions=None) -> np.ndarray:
    """The latent rows of query t's sequence, re-paged in logical order (row p =
    logical position p), as the oracle reads them (bf16 bits, or FP8 row bytes).
    With `positions`, only the 64-token pages holding them are copied from the
    device; the other rows stay zero (untouched, lazily zeroed host memory), so
    long sequences cost only what the checks read."""
    b = int(case.q_seq[t])
    L = int(case.seq_lens[b])
    nblk = (L + 63) // 64
    fp8 = case.spec.kv_dtype == "fp8"
    row_w = synth.KV_FP8_ROW if fp8 else synth.LATENT
    dt = np.uint8 if fp8 else np.uint16
    if positions is None:
        lp = np.arange(nblk, dtype=np.int64)
    else:
        lp = np.unique(np.asarray(positions, dtype=np.int64) // 64)
    kv = np.zeros((nblk * 64, row_w), dt)
    if lp.size:
        phys = case.block_table[b].cpu().long()[torch.from_numpy(lp)]
        rows = case.kv_pool.view(-1, 64, row_w)[phys.to(case.kv_pool.device)]
        rows = rows.cpu().numpy() if fp8 else bits16(rows)
        kv.reshape(nblk, 64, row_w)[lp] = rows.reshape(-1, 64, row_w)
    return kv


def query_case(case: synth.Case, t: int, kv_positions=None):
    """Oracle-format data for query t, with the query's sequence re-paged in
    logical order (mini slot = logical position).  Returns (dict, phys_slots)
    where phys_slots[p] is the real pool slot of logical position p.  The
    latent rows are those of `latent_pages` (all of them by default; with
    kv_positions=(), none: fill d["kv_pool"] before attending)."""
    b = int(case.q_seq[t])
    L = int(case.seq_lens[b])
    nblk = (L + 63) // 64
    pages = case.block_table[b, :nblk].long()
    spec = case.spec
    if spec.idx_dtype == "bf16":
        kp = bits16(case.k_idx_pool[pages]) if nblk else np.zeros((0, 64, spec.D_idx), np.uint16)
    else:
        kp = case.k_idx_pool[pages].cpu().numpy() if nblk else np.zeros((0, 64 * spec.D_idx + 256), np.uint8)
    kv = latent_pages(case, t, kv_positions)
    d = dict(T=1, B=1, H_idx=spec.H_idx, D_idx=spec.D_idx, idx_dtype=spec.idx_dtype, K=spec.K, H=spec.H,
             scale=spec.scale, num_blocks=max(nblk, 1),
             seq_lens=np.array([L], np.int32), block_table=np.arange(max(nblk, 1), dtype=np.int32)[None],
             q_seq=np.array([0], np.int32), q_visible=np.array([int(case.q_visible[t])], np.int32),
             w=case.w[t:t + 1].cpu().numpy(), q=bits16(case.q[t:t + 1]), k_idx_pool=kp,
             kv_pool=kv, kv_dtype=spec.kv_dtype)
    if spec.idx_dtype == "bf16":
        d["q_idx"], d["q_idx_scale"] = bits16(case.q_idx[t:t + 1]), None
    else:
        d["q_idx"], d["q_idx_scale"] = case.q_idx[t:t + 1].cpu().numpy(), case.q_idx_scale[t:t + 1].cpu().numpy()
    phys = O.logical_slots(case.block_table[b].cpu().numpy(), L)
    return d, phys


def assert_ascending_positions(row, phys):
    """The valid entries of an index row are in ascending logical position
    (the order the C ABI promises for dsa_indexer_topk's output)."""
    pos_of = {int(s): p for p, s in enumerate(phys)}
    gp = [pos_of[int(s)] for s in row if s >= 0]
    assert all(a < b for a, b in zip(gp, gp[1:])), "valid entries are not in ascending position order"


def check_queries(case: synth.Case, indices: torch.Tensor, out: torch.Tensor, queries, *, mla_unit=None,
                  order=True):
    """Index-set rule and attention rule for the listed queries, and the
    ascending-position order of each index row.  `mla_unit`, if given, is a
    callable(indices_tensor) -> out used to feed the oracle's own index sets
    through the sparse MLA alone."""
    idx_cpu = indices.cpu().numpy()
    out_cpu = out.float().cpu().numpy()
    K = case.spec.K
    got_o, ref_o = [], []
    oracle_rows = {}
    for t in queries:
        d, phys = query_case(case, t, kv_positions=())
        S, _ = O.query_scores(d, 0)
        ok, msg = check_index_row(idx_cpu[t], S, phys, K)
        say(f"  query {t}: n={S.shape[0]} index set: {msg}")
        assert ok, f"query {t}: {msg}"
        if order:
            assert_ascending_positions(idx_cpu[t], phys)
        # oracle attention over the GPU's own set (positions = mini slots)
        pos_of = {int(s): p for p, s in enumerate(phys)}
        gpos = np.array([pos_of[int(s)] for s in idx_cpu[t] if s >= 0], dtype=np.int64)
        opos = O.topk_positions(S, K)
        d["kv_pool"] = latent_pages(case, t, np.concatenate([gpos, opos]))
        ref = O.mla_query(d, 0, gpos)
        got_o.append(out_cpu[t])
        ref_o.append(ref)
        row = np.full(K, -1, np.int64)
        row[: opos.shape[0]] = phys[opos]
        oracle_rows[t] = (row, O.mla_query(d, 0, opos))
    ok, msg = check_outputs(np.stack(got_o), np.stack(ref_o))
    say(f"  layer output vs oracle on the GPU's index sets: {msg}")
    assert ok, msg
    if mla_unit is not None:
        fed = indices.clone()
        for t, (row, _) in oracle_rows.items():
            fed[t] = torch.from_numpy(row.astype(np.int32)).to(fed.device)
        o2 = mla_unit(fed).float().cpu().numpy()
        ok, msg = check_outputs(np.stack([o2[t] for t in oracle_rows]), np.stack([r for _, r in oracle_rows.values()]))
        say(f"  sparse MLA fed the oracle's index sets: {msg}")
        assert ok, msg
