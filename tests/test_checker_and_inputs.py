"""CPU tests of the comparison rules (mistakes planted in candidate results)
and of the synthetic input recipe."""
import numpy as np
import pytest
import torch

from dsa_check import check_index_row, check_outputs
from oracle import dsa_oracle as O
from sparse_attention_07_amd import synth


def _row_from_positions(pos, slots, K):
    row = np.full(K, -1, np.int64)
    row[: len(pos)] = np.asarray(slots)[np.asarray(pos, dtype=np.int64)]
    return row


def test_checker_accepts_exact_and_reordered():
    rng = np.random.default_rng(0)
    S = rng.standard_normal(500)
    slots = rng.permutation(4096)[:500]
    pos = O.topk_positions(S, 32)
    assert check_index_row(_row_from_positions(pos, slots, 32), S, slots, 32)[0]
    assert check_index_row(_row_from_positions(pos[::-1], slots, 32), S, slots, 32)[0]


def test_checker_near_tie_passes_clear_swap_fails():
    S = np.array([10.0, 9.0, 8.0, 7.0, 6.99999, 1.0])
    slots = np.arange(6) + 100
    # oracle top-4 = {0,1,2,3}; swapping 3 for 4 is a 1.4e-6 relative gap -> ok
    assert check_index_row(_row_from_positions([0, 1, 2, 4], slots, 4), S, slots, 4)[0]
    # swapping 3 for 5 is a large gap -> fail
    assert not check_index_row(_row_from_positions([0, 1, 2, 5], slots, 4), S, slots, 4)[0]


def test_checker_exact_ties_pass_either_way():
    S = np.array([5.0, 3.0, 3.0, 3.0, 1.0])
    slots = np.arange(5)
    assert check_index_row(_row_from_positions([0, 3], slots, 2), S, slots, 2)[0]


def test_checker_rejects_structural_mistakes():
    S = np.arange(10, dtype=np.float64)
    slots = np.arange(10) * 3
    good = _row_from_positions([9, 8, 7], slots, 5)
    good[3:] = -1
    assert check_index_row(good, S, slots, 3)[0] is False  # wrong K length
    assert check_index_row(_row_from_positions([9, 8, 7], slots, 3), S, slots, 3)[0]
    dup = _row_from_positions([9, 9, 7], slots, 3)
    assert not check_index_row(dup, S, slots, 3)[0]
    outside = _row_from_positions([9, 8, 7], slots, 3)
    outside[0] = 1  # slot 1 is not a visible position
    assert not check_index_row(outside, S, slots, 3)[0]
    hole = np.array([27, -1, 21, -1])
    assert not check_index_row(hole, S, slots, 4)[0]
    short = np.array([27, 24, -1])  # k_t=3 but only 2 valid
    assert not check_index_row(short, S, slots, 3)[0]
    # n < K: all n must be selected and the rest -1
    S2 = np.array([1.0, 2.0])
    assert check_index_row(np.array([1, 0, -1, -1]), S2, np.array([0, 1]), 4)[0]
    assert not check_index_row(np.array([1, -1, -1, -1]), S2, np.array([0, 1]), 4)[0]


def test_checker_absolute_floor_for_zero_scores():
    S = np.array([4.0, 0.0, 0.0, -0.0, -3.0])
    slots = np.arange(5)
    assert check_index_row(_row_from_positions([0, 2], slots, 2), S, slots, 2)[0]
    S3 = np.array([4.0, 1e-9, -1e-9, -3.0])
    assert check_index_row(_row_from_positions([0, 2], np.arange(4), 2), S3, np.arange(4), 2)[0]


def test_output_check():
    ref = np.ones((2, 4, 512))
    assert check_outputs(ref + 0.01, ref)[0]
    assert not check_outputs(ref + 0.03, ref)[0]
    bad = ref.copy()
    bad[0, 0, :100] += 0.019  # within max-abs but check rel L2 too
    assert check_outputs(bad, ref)[0]


# ----------------------------------------------------------------------------- input recipe
def test_synth_tiny_decode_layout():
    c = synth.build_case(synth.PRESETS["tiny_decode"])
    assert c.T == 1 and c.B == 1 and c.num_blocks == 64
    assert c.k_idx_pool.shape == (64, 64, 64) and c.k_idx_pool.dtype == torch.bfloat16
    assert c.kv_pool.shape == (64 * 64, 576)
    assert sorted(c.block_table[0].tolist()) == list(range(64))
    assert c.q_visible.tolist() == [4096]
    assert c.q.shape == (1, 16, 576) and c.w.shape == (1, 4)


def test_synth_fp8_quantization_roundtrip():
    spec = synth.CaseSpec("t", H_idx=8, D_idx=128, idx_dtype="fp8", K=16, H=16, lens=[100, 64, 1])
    c = synth.build_case(spec)
    d = synth.to_numpy(c)
    assert c.k_idx_pool.shape == (c.num_blocks, 8448)
    # dequantized keys are within e4m3 rounding (2^-4 relative, 2^-9*scale absolute) of the bf16 draw
    gen = torch.Generator().manual_seed(1)
    raw = synth._randn_bf16(gen, (c.num_blocks, 64, 128), "cpu").to(torch.float64).numpy().reshape(-1, 128)
    for b, L in enumerate([100, 64, 1]):
        slots = O.logical_slots(d["block_table"][b], L)
        deq = O.index_keys(d["k_idx_pool"], "fp8", 128, slots)
        x = raw[slots]
        amax = np.abs(x).max(1, keepdims=True)
        assert np.all(np.abs(deq - x) <= np.abs(x) * 2 ** -4 + amax / 448 * 2 ** -9 + 1e-12)
        assert np.allclose(np.abs(deq).max(1), amax[:, 0], rtol=1e-6)


def test_synth_mxfp8_quantization_roundtrip():
    spec = synth.CaseSpec("t", H_idx=8, D_idx=128, idx_dtype="mxfp8", K=16, H=16, lens=[100, 64, 1])
    c = synth.build_case(spec)
    d = synth.to_numpy(c)
    assert c.k_idx_pool.shape == (c.num_blocks, 8448)
    assert c.q_idx_scale.shape == (c.T, 8, 4) and c.q_idx_scale.dtype == torch.uint8
    assert int(c.k_idx_pool[:, 8192:].max()) < 255 and int(c.q_idx_scale.max()) < 255
    gen = torch.Generator().manual_seed(1)
    raw = synth._randn_bf16(gen, (c.num_blocks, 64, 128), "cpu").to(torch.float64).numpy().reshape(-1, 128)
    for b, L in enumerate([100, 64, 1]):
        slots = O.logical_slots(d["block_table"][b], L)
        deq = O.index_keys(d["k_idx_pool"], "mxfp8", 128, slots)
        x = raw[slots].reshape(L, 4, 32)
        amax = np.abs(x).max(2, keepdims=True)
        scale = np.exp2(np.floor(np.log2(amax)) - 8)          # the group's power of two
        err = np.abs(deq.reshape(L, 4, 32) - x)
        bound = np.abs(x) * 2 ** -4 + scale * 2 ** -9 + np.maximum(np.abs(x) - 448 * scale, 0) + 1e-12
        assert np.all(err <= bound)
        assert np.all(amax / scale >= 256) and np.all(amax / scale < 512)


def test_synth_fp8_latent_roundtrip():
    # the same draw in bf16 and in FP8 latent form: dequantized rows (oracle decode) sit within the e4m3
    # rounding of the bf16 rows, rope dims unchanged, tile amax mapped to +-448 * scale
    kw = dict(H_idx=8, D_idx=128, idx_dtype="fp8", K=16, H=16, lens=[100, 64, 1])
    cb = synth.build_case(synth.CaseSpec("t", **kw))
    cf = synth.build_case(synth.CaseSpec("t", kv_dtype="fp8", **kw))
    assert cf.kv_pool.shape == (cb.kv_pool.shape[0], 656) and cf.kv_pool.dtype == torch.uint8
    assert torch.equal(cb.q, cf.q) and torch.equal(cb.k_idx_pool, cf.k_idx_pool)
    x = O.bf16_to_f64(synth.to_numpy(cb)["kv_pool"]).reshape(-1, 576)
    deq = O.latent_rows(synth.to_numpy(cf), np.arange(x.shape[0]))
    assert np.array_equal(deq[:, 512:], x[:, 512:])
    xt = x[:, :512].reshape(-1, 4, 128)
    amax = np.abs(xt).max(2, keepdims=True)
    err = np.abs(deq[:, :512].reshape(-1, 4, 128) - xt)
    assert np.all(err <= np.abs(xt) * 2 ** -4 + amax / 448 * 2 ** -9 + 1e-12)
    live = amax[:, :, 0] > 0
    assert np.allclose(np.abs(deq[:, :512].reshape(-1, 4, 128)).max(2)[live], amax[:, :, 0][live], rtol=1e-6)


def test_synth_speculative_and_prefill_horizons():
    spec = synth.CaseSpec("t", H_idx=4, D_idx=64, idx_dtype="bf16", K=8, H=16, lens=[70, 300],
                          queries_per_seq=[1, 4])
    c = synth.build_case(spec)
    assert c.q_seq.tolist() == [0, 1, 1, 1, 1]
    assert c.q_visible.tolist() == [70, 297, 298, 299, 300]
    assert c.max_q_per_seq == 4
    p = synth.CaseSpec("p", H_idx=4, D_idx=64, idx_dtype="bf16", K=8, H=16, prefill=(300, 128))
    c2 = synth.build_case(p, prefill_chunk=2)
    assert c2.T == 44 and c2.seq_lens.tolist() == [300]
    assert c2.q_visible.tolist() == list(range(257, 301))
    c1 = synth.build_case(p, prefill_chunk=1)
    assert c1.seq_lens.tolist() == [256]
    # same draws across chunks: chunk 1's first query equals row 128 of the full query draw
    c0 = synth.build_case(p, prefill_chunk=0)
    assert torch.equal(c0.kv_pool, c1.kv_pool)


def test_synth_is_deterministic():
    a = synth.build_case(synth.PRESETS["tiny_decode"])
    b = synth.build_case(synth.PRESETS["tiny_decode"])
    for f in ("k_idx_pool", "kv_pool", "q_idx", "w", "q", "block_table"):
        assert torch.equal(getattr(a, f), getattr(b, f))
