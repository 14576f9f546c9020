"""Pins for the CPU oracle: each oracle function is checked against something
other than itself -- a library routine (torch's float8/bf16 decode, torch's
float64 scaled_dot_product_attention), hand-worked values, closed forms, brute
force with Python's own sorting, or an invariant.  The pages print no worked
example, so no value here comes from them."""
import math

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O


def bf16_bits(x):
    """float values (exactly representable in bf16) -> uint16 bit patterns."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(t.to(torch.float32), torch.tensor(np.asarray(x, dtype=np.float32))), "not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def make_case(idx_dtype, D, H_idx, k_rows, q_idx, w, seq_len, block_row, NB, q_scale=None, k_scales=None,
              K=4, H=2, q=None, kv=None, q_visible=None):
    """A one-query case dict in the oracle's array format."""
    if idx_dtype == "bf16":
        pool = np.zeros((NB * 64, D), dtype=np.uint16)
        pool[O.logical_slots(block_row, len(k_rows))] = bf16_bits(k_rows)
        pool = pool.reshape(NB, 64, D)
    elif idx_dtype == "mxfp8":
        ng = D // 32
        pool = np.zeros((NB, 64 * D + 64 * ng), dtype=np.uint8)
        slots = O.logical_slots(block_row, len(k_rows))
        for p, s in enumerate(slots):
            pg, r = divmod(int(s), 64)
            pool[pg, r * D:(r + 1) * D] = np.asarray(k_rows[p], dtype=np.uint8)
            pool[pg, 64 * D + ng * r: 64 * D + ng * (r + 1)] = np.asarray(k_scales[p], dtype=np.uint8)
    else:
        pool = np.zeros((NB, 64 * D + 256), dtype=np.uint8)
        slots = O.logical_slots(block_row, len(k_rows))
        for p, s in enumerate(slots):
            pg, r = divmod(int(s), 64)
            pool[pg, r * D:(r + 1) * D] = np.asarray(k_rows[p], dtype=np.uint8)
            pool[pg, 64 * D + 4 * r: 64 * D + 4 * r + 4] = np.frombuffer(np.float32(k_scales[p]).tobytes(), np.uint8)
    if q is None:
        q = np.zeros((1, H, 576), dtype=np.uint16)
    if kv is None:
        kv = np.zeros((NB * 64, 576), dtype=np.uint16)
    return dict(
        T=1, B=1, H_idx=H_idx, D_idx=D, idx_dtype=idx_dtype, K=K, H=H, scale=1 / math.sqrt(576), num_blocks=NB,
        seq_lens=np.array([seq_len], np.int32), block_table=np.array([block_row], np.int32),
        q_seq=np.array([0], np.int32), q_visible=np.array([seq_len if q_visible is None else q_visible], np.int32),
        w=np.array([w], np.float32),
        q_idx=(bf16_bits([q_idx]) if idx_dtype == "bf16" else np.array([q_idx], np.uint8)),
        q_idx_scale=None if q_scale is None else np.array([q_scale], np.uint8 if idx_dtype == "mxfp8" else np.float32),
        k_idx_pool=pool, q=q, kv_pool=kv)


# ----------------------------------------------------------------------------- decoders
def test_fp8_decode_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2  # 0x7f and 0xff only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert O.fp8_e4m3fn_to_f64(np.uint8(0x7E)) == 448.0
    assert O.fp8_e4m3fn_to_f64(np.uint8(0x01)) == 2.0 ** -9


def test_e8m0_decode_all_256_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = O.e8m0_to_f64(b)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert [math.ldexp(1.0, int(x) - 127) for x in b[:255]] == ours[:255].tolist()


def test_mxfp8_dequant_group_boundaries():
    # 64 codes of 1.0 with group scales 2^1 and 2^-3: the first 32 decode to 2,
    # the next 32 to 1/8 (a shifted or transposed group index fails)
    codes = np.full((1, 64), 0x38, dtype=np.uint8)
    v = O.mxfp8_to_f64(codes, np.array([[128, 124]], dtype=np.uint8))
    assert v[0, :32].tolist() == [2.0] * 32 and v[0, 32:].tolist() == [0.125] * 32


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 65536, 4096).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = O.bf16_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


# ----------------------------------------------------------------------------- indexer scores
def test_scores_hand_worked_bf16():
    # q0=[1,2,0], q1=[0,-1,3], w=[0.5,-2]
    # k0=[1,1,1]:    d=(3, 2)     -> 0.5*3 - 2*2      = -2.5
    # k1=[2,0,-1]:   d=(2,-3)     -> 0.5*2 - 2*0      =  1.0
    # k2=[0,-1,-1]:  d=(-2,-2)    -> 0                =  0.0
    # k3=[-1,.5,2]:  d=(0, 5.5)   -> 0.5*0 - 2*5.5    = -11.0
    keys = [[1, 1, 1], [2, 0, -1], [0, -1, -1], [-1, 0.5, 2]]
    case = make_case("bf16", 3, 2, keys, [[1, 2, 0], [0, -1, 3]], [0.5, -2.0], 4, [0], 1)
    S, slots = O.query_scores(case, 0)
    assert S.tolist() == [-2.5, 1.0, 0.0, -11.0]
    assert slots.tolist() == [0, 1, 2, 3]
    assert O.topk_positions(S, 2).tolist() == [1, 2]


def test_scores_hand_worked_fp8():
    # e4m3fn codes: 0x38=1, 0x40=2, 0x44=3, 0xB8=-1
    # q0 = [1,2]*0.5 = [0.5,1];  q1 = [3,-1]*2 = [6,-2];  w = [1,-0.25]
    # k0 = [2,1]*4 = [8,4]:      d=(8, 40)     -> 8 - 10     = -2
    # k1 = [1,3]*0.5 = [.5,1.5]: d=(1.75, 0)   -> 1.75
    q_codes = [[0x38, 0x40], [0x44, 0xB8]]
    k_codes = [[0x40, 0x38], [0x38, 0x44]]
    case = make_case("fp8", 2, 2, k_codes, q_codes, [1.0, -0.25], 2, [3], 4, q_scale=[0.5, 2.0],
                     k_scales=[4.0, 0.5])
    S, slots = O.query_scores(case, 0)
    assert S.tolist() == [-2.0, 1.75]
    assert slots.tolist() == [192, 193]


def test_scores_hand_worked_mxfp8():
    # D = 64: two groups of 32.  e4m3fn codes 0x38=1, 0x40=2, 0x44=3, 0xB8=-1;
    # E8M0 bytes 125=1/4, 126=1/2, 127=1, 128=2, 129=4, 130=8.
    # q head 0: dim 0 = 1 (x2), dim 32 = 2 (x1/2)  -> [2 @0, 1 @32]
    # q head 1: dim 1 = 2 (x1)                     -> [2 @1]
    # k0: dim 0 = 3, dim 1 = 1 (group x1/4), dim 32 = -1 (x8) -> [.75 @0, .25 @1, -8 @32]
    # k1: dim 0 = 1 (x1), dim 32 = 1 (x4)                    -> [1 @0, 4 @32]
    # head dots: k0 (1.5 - 8 = -6.5, 0.5), k1 (2 + 4 = 6, 0); w = [1.5, -2]
    # S0 = 1.5*0 - 2*0.5 = -1;  S1 = 1.5*6 - 2*0 = 9
    D = 64
    q = np.zeros((2, D), np.uint8)
    q[0, 0], q[0, 32], q[1, 1] = 0x38, 0x40, 0x40
    k = np.zeros((2, D), np.uint8)
    k[0, 0], k[0, 1], k[0, 32] = 0x44, 0x38, 0xB8
    k[1, 0], k[1, 32] = 0x38, 0x38
    case = make_case("mxfp8", D, 2, k, q, [1.5, -2.0], 2, [1], 2, q_scale=[[128, 126], [127, 127]],
                     k_scales=[[125, 130], [127, 129]])
    S, slots = O.query_scores(case, 0)
    assert S.tolist() == [-1.0, 9.0]
    assert slots.tolist() == [64, 65]


def test_mxfp8_with_equal_group_scales_equals_fp8_per_token():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, (5, 128)).astype(np.uint8) | (rng.integers(0, 2, (5, 128)) << 7).astype(np.uint8)
    byte = rng.integers(110, 140, 5).astype(np.uint8)
    mx = O.mxfp8_to_f64(codes, np.repeat(byte[:, None], 4, axis=1))
    fp = O.fp8_e4m3fn_to_f64(codes) * np.exp2(byte.astype(np.float64) - 127)[:, None]
    assert np.array_equal(mx, fp)


def test_mxfp8_key_group_scale_only_touches_its_group():
    rng = np.random.default_rng(4)
    D = 128
    k = rng.integers(0, 0x60, (3, D)).astype(np.uint8)
    ks = rng.integers(120, 135, (3, 4)).astype(np.uint8)
    q = np.zeros((1, D), np.uint8)
    q[0, 64:96] = rng.integers(0x20, 0x50, 32)  # query lives in group 2 only
    base = make_case("mxfp8", D, 1, k, q, [1.0], 3, [0], 1, q_scale=[[127, 127, 127, 127]], k_scales=ks)
    S0, _ = O.query_scores(base, 0)
    ks2 = ks.copy()
    ks2[:, [0, 1, 3]] += 3      # other groups: no effect
    S1, _ = O.query_scores(make_case("mxfp8", D, 1, k, q, [1.0], 3, [0], 1, q_scale=[[127] * 4], k_scales=ks2), 0)
    assert np.array_equal(S0, S1)
    ks3 = ks.copy()
    ks3[:, 2] += 2              # its own group: the (positive) scores scale by 4
    S2, _ = O.query_scores(make_case("mxfp8", D, 1, k, q, [1.0], 3, [0], 1, q_scale=[[127] * 4], k_scales=ks3), 0)
    assert np.array_equal(S2, 4 * S0) and (S0 > 0).all()


def test_scores_closed_form_ramp_through_permuted_pages():
    # H=1, w=1, q=e0, k_p=(p+1)/256 e0 -> S_p=(p+1)/256; Top-K = last K positions
    n, D = 256, 4
    keys = np.zeros((n, D))
    keys[:, 0] = (np.arange(n) + 1) / 256.0
    block_row = [5, 2, 7, 0]
    case = make_case("bf16", D, 1, keys, [[1, 0, 0, 0]], [1.0], n, block_row, 8, K=10)
    S, slots = O.query_scores(case, 0)
    assert np.array_equal(S, (np.arange(n) + 1) / 256.0)
    res = O.layer_query(case, 0)
    assert res["positions"].tolist() == list(range(255, 245, -1))
    expect_slots = [block_row[p // 64] * 64 + p % 64 for p in range(255, 245, -1)]
    assert res["indices"].tolist() == expect_slots


def test_scores_positive_homogeneity():
    rng = np.random.default_rng(1)
    H, D, n = 4, 8, 64
    qv = rng.standard_normal((H, D))
    w = rng.standard_normal(H)
    keys = rng.standard_normal((n, D))
    S = O.indexer_scores(qv, w, keys)
    for a in (0.25, 3.0):
        np.testing.assert_allclose(O.indexer_scores(qv * a, w, keys), a * S, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(O.indexer_scores(qv, w * a, keys), a * S, rtol=1e-12, atol=1e-12)
        assert set(O.topk_positions(O.indexer_scores(qv * a, w, keys), 9)) == set(O.topk_positions(S, 9))


def test_scores_brute_force_loops_tiny():
    # scalar Python loops over heads and dims: catches a transposed q or a dropped head
    rng = np.random.default_rng(2)
    H, D, n = 3, 5, 7
    qv = rng.standard_normal((H, D))
    w = rng.standard_normal(H)
    keys = rng.standard_normal((n, D))
    S = O.indexer_scores(qv, w, keys)
    for p in range(n):
        acc = 0.0
        for h in range(H):
            dot = math.fsum(qv[h, d] * keys[p, d] for d in range(D))
            acc += w[h] * (dot if dot > 0 else 0.0)
        assert abs(acc - S[p]) < 1e-12


# ----------------------------------------------------------------------------- Top-K
@pytest.mark.parametrize("n,K", [(1, 4), (5, 5), (37, 8), (300, 64), (64, 300)])
def test_topk_matches_python_sorted_with_ties(n, K):
    rng = np.random.default_rng(n * 7 + K)
    S = rng.integers(-5, 6, n).astype(np.float64)  # many exact ties
    S[rng.integers(0, n, max(1, n // 4))] = 0.0
    ours = O.topk_positions(S, K)
    ref = sorted(range(n), key=lambda p: (-S[p], p))[: min(K, n)]
    assert ours.tolist() == ref


def test_topk_selected_dominate_unselected():
    rng = np.random.default_rng(3)
    S = rng.standard_normal(5000)
    pos = O.topk_positions(S, 123)
    mask = np.zeros(5000, bool)
    mask[pos] = True
    assert S[mask].min() >= S[~mask].max()
    assert len(set(pos.tolist())) == 123


def test_causal_horizon_hides_later_positions():
    # position 9 has the largest key but query sees only 0..7
    n, D = 10, 2
    keys = np.zeros((n, D))
    keys[:, 0] = np.arange(n)
    keys[9, 0] = 100
    case = make_case("bf16", D, 1, keys, [[1, 0]], [1.0], n, [0], 1, K=3, q_visible=8)
    res = O.layer_query(case, 0)
    assert res["positions"].tolist() == [7, 6, 5]
    assert res["indices"].tolist() == [7, 6, 5]


def test_zero_visible_gives_padding_and_zero_output():
    case = make_case("bf16", 2, 1, np.zeros((4, 2)), [[1, 0]], [1.0], 4, [0], 1, K=3, q_visible=0)
    res = O.layer_query(case, 0)
    assert res["indices"].tolist() == [-1, -1, -1]
    assert not res["out"].any()


# ----------------------------------------------------------------------------- sparse MLA
def sdpa_f64(qh, rows, scale):
    q = torch.from_numpy(qh)[:, None, :]                               # [H, 1, 576]
    k = torch.from_numpy(rows)[None].expand(qh.shape[0], -1, -1)      # [H, k, 576]
    v = torch.from_numpy(rows[:, :512])[None].expand(qh.shape[0], -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(q, k.contiguous(), v, scale=scale)[:, 0].numpy()


def test_mla_matches_torch_sdpa_float64():
    rng = np.random.default_rng(4)
    qh = rng.standard_normal((6, 576))
    rows = rng.standard_normal((37, 576))
    scale = 1 / math.sqrt(576)
    np.testing.assert_allclose(O.sparse_mla(qh, rows, scale), sdpa_f64(qh, rows, scale), rtol=1e-12, atol=1e-13)


def test_mla_identical_rows_return_the_row():
    rng = np.random.default_rng(5)
    c = rng.standard_normal(576)
    rows = np.tile(c, (11, 1))
    out = O.sparse_mla(rng.standard_normal((3, 576)), rows, 0.1)
    np.testing.assert_allclose(out, np.tile(c[:512], (3, 1)), rtol=1e-14, atol=1e-14)


def test_mla_zero_query_is_mean_of_values():
    rng = np.random.default_rng(6)
    rows = rng.standard_normal((9, 576))
    out = O.sparse_mla(np.zeros((2, 576)), rows, 0.3)
    np.testing.assert_allclose(out, np.tile(rows[:, :512].mean(0), (2, 1)), rtol=1e-13, atol=1e-14)


def test_mla_single_row_and_empty():
    rng = np.random.default_rng(7)
    r = rng.standard_normal((1, 576))
    np.testing.assert_array_equal(O.sparse_mla(rng.standard_normal((4, 576)), r, 1.0), np.tile(r[0, :512], (4, 1)))
    assert not O.sparse_mla(rng.standard_normal((4, 576)), np.zeros((0, 576)), 1.0).any()


def test_mla_softmax_weights_sum_to_one():
    rng = np.random.default_rng(8)
    _, P = O.sparse_mla(rng.standard_normal((5, 576)) * 3, rng.standard_normal((50, 576)), 1 / 24, True)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-12)
    assert (P >= 0).all()


# ----------------------------------------------------------------------------- whole layer
def random_layer_case(rng, n, NB, block_row, K, H=4, idx_dtype="bf16"):
    D, H_idx = 8, 3
    keys = rng.standard_normal((n, D)).astype(np.float32)
    keys = torch.tensor(keys).to(torch.bfloat16).to(torch.float32).numpy()
    q_idx = torch.tensor(rng.standard_normal((H_idx, D)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    q = bf16_bits(torch.tensor(rng.standard_normal((1, H, 576)).astype(np.float32)).to(torch.bfloat16).float().numpy())
    kv = np.zeros((NB * 64, 576), np.uint16)
    lat = torch.tensor(rng.standard_normal((n, 576)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    kv[O.logical_slots(block_row, n)] = bf16_bits(lat)
    return make_case(idx_dtype, D, H_idx, keys, q_idx, rng.standard_normal(H_idx) * 0.5, n, block_row, NB,
                     K=K, H=H, q=q, kv=kv), lat


def test_layer_with_K_at_least_n_equals_dense_attention():
    rng = np.random.default_rng(9)
    n = 150
    case, lat = random_layer_case(rng, n, 3, [2, 0, 1], K=256)
    res = O.layer_query(case, 0)
    assert sorted(res["positions"].tolist()) == list(range(n))
    qh = O.bf16_to_f64(case["q"][0])
    dense = sdpa_f64(qh, lat.astype(np.float64), case["scale"])
    np.testing.assert_allclose(res["out"], dense, rtol=1e-11, atol=1e-12)


def test_layer_invariant_under_page_permutation():
    rng = np.random.default_rng(10)
    n = 200
    case_a, _ = random_layer_case(np.random.default_rng(11), n, 4, [0, 1, 2, 3], K=17)
    case_b, _ = random_layer_case(np.random.default_rng(11), n, 4, [3, 1, 0, 2], K=17)
    ra, rb = O.layer_query(case_a, 0), O.layer_query(case_b, 0)
    assert ra["positions"].tolist() == rb["positions"].tolist()
    np.testing.assert_array_equal(ra["out"], rb["out"])
    assert ra["indices"].tolist() != rb["indices"].tolist()  # slots differ, positions do not


# --------------------------------------------------------------------------- index-query quantization
def _all_e4m3_midpoints():
    pos = O.fp8_e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))   # 0 .. 448, ascending
    mids = (pos[1:] + pos[:-1]) / 2                                # exact in float32 (one more bit)
    return np.concatenate([mids, -mids]).astype(np.float32)


def test_e4m3_encode_matches_torch_float8_including_every_tie():
    # library routine: torch's round-to-nearest-even float -> float8_e4m3fn cast
    rng = np.random.default_rng(11)
    y = np.concatenate([rng.uniform(-448, 448, 100_000), rng.uniform(-0.02, 0.02, 100_000),
                        rng.normal(0, 1, 100_000), _all_e4m3_midpoints(), [0.0, -0.0, 448.0, -448.0, 2.0 ** -9,
                                                                          2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3fn_encode(y), ref)


def test_e4m3_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(O.e4m3fn_encode(O.fp8_e4m3fn_to_f64(codes)), codes)


def test_quantize_fp8_hand_worked_row():
    # amax 896 -> s = 2; x/s = 448, 0.5, -1.5, 0.25, 8.5 (a tie: 8 and 9 -> 8), 9.5 (tie -> 10)
    x = np.array([896.0, 1.0, -3.0, 0.5, 17.0, 19.0, 0.0, -896.0], np.float32)
    codes, s = O.quantize_fp8_per_row(x[None])
    assert s.tolist() == [2.0]
    # 448 = 0x7e; 0.5 = 2^-1 -> exp field 6; -1.5 -> 0x80 | (7 << 3) | 4; 0.25 -> field 5;
    # 8 = 2^3 -> field 10; 10 = 1.25 * 2^3 -> field 10, mantissa 2
    assert codes[0].tolist() == [0x7E, 0x30, 0xBC, 0x28, 0x50, 0x52, 0x00, 0xFE]


def test_quantize_fp8_zero_row_and_subnormal_codes():
    codes, s = O.quantize_fp8_per_row(np.zeros((2, 64), np.float32))
    assert s.tolist() == [1.0, 1.0] and not codes.any()
    # amax 448 -> s = 1.  Subnormals are n * 2^-9: 2^-7 is n = 4; 3 * 2^-10 is the tie n = 1.5 -> 2;
    # 7 * 2^-10 the tie n = 3.5 -> 4; 2^-10 the tie n = 0.5 -> 0
    x = np.zeros((1, 32), np.float32)
    x[0, :5] = [448.0, 2.0 ** -7, 3 * 2.0 ** -10, 7 * 2.0 ** -10, -(2.0 ** -10)]
    codes, s = O.quantize_fp8_per_row(x)
    assert s.tolist() == [1.0] and codes[0, :5].tolist() == [0x7E, 0x04, 0x02, 0x04, 0x80]


def test_quantize_fp8_error_bound_and_amax_code():
    rng = np.random.default_rng(12)
    x = (rng.normal(0, 1, (500, 128)) * np.exp(rng.normal(0, 3, (500, 1)))).astype(np.float32)
    codes, s = O.quantize_fp8_per_row(x)
    y = x.astype(np.float64) / s[:, None].astype(np.float64)
    deq = O.fp8_e4m3fn_to_f64(codes)
    # round to nearest: half an e4m3 ulp (2^-4 relative for normals, 2^-10 absolute below 2^-6), plus
    # the float32 rounding of x/s
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6) + np.abs(y) * 2.0 ** -23
    assert np.all(np.abs(deq - np.clip(y, -448, 448)) <= bound)
    # the element holding amax lands on +-448 (code 0x7e or 0xfe)
    am = np.abs(x).argmax(axis=1)
    assert np.all((codes[np.arange(500), am] & 0x7F) == 0x7E)


def test_quantize_mxfp8_hand_worked_groups():
    x = np.zeros((1, 128), np.float32)
    x[0, :3] = [1.0, -0.75, 2.0 ** -7]          # group 0: amax 1 -> e = -8, x * 256 = 256, -192, 2
    x[0, 64:66] = [500.0, 3.0]                  # group 2: amax 500 -> e = 0; 500 clamps to 448
    x[0, 96] = 2.0 ** -130                      # group 3: float32 subnormal amax -> e clamps to -127
    codes, sc = O.quantize_mxfp8(x)
    assert sc[0].tolist() == [119, 127, 127, 0]   # group 1 is all zero -> byte 127
    assert codes[0, :3].tolist() == [0x78, 0xF4, 0x40]
    assert not codes[0, 32:64].any()
    assert codes[0, 64:66].tolist() == [0x7E, 0x44]   # 3 = 1.5 * 2^1 -> exp field 8, mantissa 4
    assert codes[0, 96] == 0x20                  # 2^-130 * 2^127 = 2^-3 -> exp field 4


def test_quantize_mxfp8_scale_is_power_of_two_below_amax_and_error_bound():
    rng = np.random.default_rng(13)
    x = (rng.normal(0, 1, (300, 128)) * np.exp(rng.normal(0, 4, (300, 4))).repeat(32, axis=1)).astype(np.float32)
    codes, sc = O.quantize_mxfp8(x)
    amax = np.abs(x.astype(np.float64)).reshape(300, 4, 32).max(axis=2)
    e = sc.astype(np.int64) - 127
    for a, ee in zip(amax.ravel(), e.ravel()):
        m, ex = math.frexp(float(a))             # a = m * 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
        assert ee == ex - 1 - 8
    y = x.astype(np.float64) / np.exp2(e.astype(np.float64)).repeat(32, axis=1)
    deq = O.fp8_e4m3fn_to_f64(codes)
    assert np.all(np.abs(y) < 512)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-9)
    clipped = np.clip(y, -448, 448)
    assert np.all(np.abs(deq - clipped) <= bound)


def test_quantizers_agree_with_the_input_generators_recipe():
    # the seeded generators quantize their own inputs with torch ops; the oracle's
    # bit-level quantizers must give the same codes on bf16 data
    from sparse_attention_07_amd import synth
    g = torch.Generator().manual_seed(14)
    xb = (torch.randn(64, 64, 128, generator=g) * torch.exp(torch.randn(64, 64, 1, generator=g) * 2)).to(torch.bfloat16)
    x = xb.float().numpy()
    c_t, s_t = synth.quantize_fp8_rows(xb)
    c_o, s_o = O.quantize_fp8_per_row(x)
    assert np.array_equal(c_t.numpy(), c_o) and np.array_equal(s_t.numpy(), s_o)
    m_t, e_t = synth.quantize_mxfp8_rows(xb)
    m_o, e_o = O.quantize_mxfp8(x)
    assert np.array_equal(m_t.numpy(), m_o) and np.array_equal(e_t.numpy(), e_o)


# --------------------------------------------------------------------------- FP8 latent KV (tile 128)
def bf16_round_bits(x):
    """float values -> bf16 bit patterns, rounded to nearest even."""
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp8_kv_row(codes, scales, rope_bf16_bits):
    r = np.zeros(O.KV_FP8_ROW, np.uint8)
    r[:512] = codes
    r[512:528] = np.asarray(scales, "<f4").view(np.uint8)
    r[528:656] = np.asarray(rope_bf16_bits, "<u2").view(np.uint8)
    return r


def test_fp8_kv_row_layout_hand_worked():
    codes = np.zeros(512, np.uint8)
    codes[0] = 0x38            # 1.0
    codes[127] = 0xC0          # -2.0 (last dim of tile 0)
    codes[128] = 0x38          # first dim of tile 1
    codes[511] = 0x01          # smallest subnormal 2^-9, tile 3
    rope = bf16_bits([3.0] + [0.0] * 62 + [-0.5])
    row = fp8_kv_row(codes, [2.0, 0.25, 1.0, 8.0], rope)
    assert row.size == 656
    x = O.latent_rows_fp8(row[None])[0]
    assert x.shape == (576,)
    assert x[0] == 2.0 and x[127] == -4.0 and x[128] == 0.25 and x[511] == 8.0 * 2.0 ** -9
    assert x[1:127].tolist() == [0.0] * 126
    assert x[512] == 3.0 and x[575] == -0.5          # rope untouched by the scales


def test_fp8_kv_tile_scale_moves_only_its_tile():
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 0x7E, 512).astype(np.uint8) | (rng.integers(0, 2, 512).astype(np.uint8) << 7)
    rope = bf16_round_bits(rng.normal(0, 1, 64))
    base = O.latent_rows_fp8(fp8_kv_row(codes, [1.0, 1.0, 1.0, 1.0], rope)[None])[0]
    for t in range(4):
        sc = [1.0] * 4
        sc[t] = 4.0
        x = O.latent_rows_fp8(fp8_kv_row(codes, sc, rope)[None])[0]
        moved = np.flatnonzero(x != base)
        assert set(moved) <= set(range(128 * t, 128 * t + 128))
        assert np.array_equal(x[128 * t: 128 * t + 128], 4.0 * base[128 * t: 128 * t + 128])


def test_fp8_kv_attention_equals_bf16_attention_on_representable_rows():
    # rows whose nope values are e4m3 codes times a power-of-two tile scale are exact in bf16 too:
    # the FP8 and bf16 caches must then give identical attention
    rng = np.random.default_rng(22)
    n, H = 40, 4
    codes = rng.integers(0, 0x7E, (n, 512)).astype(np.uint8) | (rng.integers(0, 2, (n, 512)).astype(np.uint8) << 7)
    scales = 2.0 ** rng.integers(-8, 3, (n, 4))
    rope = bf16_round_bits(rng.normal(0, 1, (n, 64)))
    fp8_pool = np.stack([fp8_kv_row(codes[i], scales[i], rope[i]) for i in range(n)])
    vals = O.fp8_e4m3fn_to_f64(codes) * np.repeat(scales, 128, axis=1)
    bf_pool = np.concatenate([bf16_bits(vals), rope], axis=1)
    assert np.array_equal(O.bf16_to_f64(bf_pool[:, :512]), vals)      # representable, so exact
    q = bf16_round_bits(rng.normal(0, 1, (1, H, 576)))
    slots = rng.permutation(n)[:25]
    a = O.mla_query(dict(q=q, kv_pool=fp8_pool, kv_dtype="fp8", scale=0.05), 0, slots)
    b = O.mla_query(dict(q=q, kv_pool=bf_pool, scale=0.05), 0, slots)
    assert np.array_equal(a, b)


def test_fp8_kv_rows_follow_slots_and_skip_padding():
    rng = np.random.default_rng(23)
    n = 6
    pool = np.stack([fp8_kv_row(np.full(512, 0x38, np.uint8), [float(i + 1)] * 4, bf16_bits(np.full(64, float(i))))
                     for i in range(n)])
    rows = O.latent_rows(dict(kv_pool=pool, kv_dtype="fp8"), np.array([4, 1]))
    assert rows[0, 0] == 5.0 and rows[1, 0] == 2.0 and rows[0, 512 + 24] == 4.0
    # the attention of a single selected row returns that row's value dims whatever the query
    q = bf16_round_bits(rng.normal(0, 1, (1, 2, 576)))
    out = O.mla_query(dict(q=q, kv_pool=pool, kv_dtype="fp8", scale=0.1), 0, np.array([-1, 3, -1]))
    assert np.array_equal(out, np.tile(O.latent_rows(dict(kv_pool=pool, kv_dtype="fp8"), [3])[0, :512], (2, 1)))


# --------------------------------------------------------------------------- residual + RMSNorm after the attention
def test_residual_rmsnorm_matches_torch_rms_norm_float64():
    # library routine: torch's RMSNorm over the last dim, in float64
    rng = np.random.default_rng(31)
    T, H = 3, 4
    attn, res = rng.normal(0, 1, (T, H, 512)), rng.normal(0, 2, (T, H, 512))
    gamma = rng.normal(1, 0.3, H * 512)
    y, out = O.residual_rmsnorm(attn, res, gamma, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(attn + res).reshape(T, -1), (H * 512,),
                                       torch.from_numpy(gamma), eps=1e-6).reshape(T, H, 512).numpy()
    assert np.array_equal(y, attn + res)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_residual_rmsnorm_closed_forms():
    H = 2
    # a constant row c: mean(y^2) = c^2, so out = c / sqrt(c^2 + eps) * gamma
    attn = np.full((1, H, 512), 1.5)
    res = np.full((1, H, 512), -3.5)
    gamma = np.linspace(-2, 2, H * 512)
    y, out = O.residual_rmsnorm(attn, res, gamma, 0.25)
    assert np.all(y == -2.0)
    assert np.allclose(out.reshape(-1), -2.0 / np.sqrt(4.0 + 0.25) * gamma, rtol=1e-15, atol=0)
    # one non-zero entry v in N values: mean = v^2/N, out there = v / sqrt(v^2/N) = sqrt(N) (eps = 0)
    attn = np.zeros((1, H, 512))
    attn[0, 1, 7] = 3.0
    _, out = O.residual_rmsnorm(attn, np.zeros_like(attn), np.ones(H * 512), 0.0)
    assert np.isclose(out[0, 1, 7], np.sqrt(H * 512)) and np.count_nonzero(out) == 1
    # tokens are normalized separately, and scaling a token (eps = 0) changes nothing
    rng = np.random.default_rng(32)
    a = rng.normal(0, 1, (2, H, 512))
    _, o1 = O.residual_rmsnorm(a, np.zeros_like(a), np.ones(H * 512), 0.0)
    a2 = a.copy()
    a2[1] *= 1000.0
    _, o2 = O.residual_rmsnorm(a2, np.zeros_like(a2), np.ones(H * 512), 0.0)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(np.mean(o1.reshape(2, -1) ** 2, axis=1), 1.0, rtol=1e-12)
