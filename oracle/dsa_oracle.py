"""CPU oracle for the DSA sparse-attention layer: lightning indexer, Top-K, sparse MLA.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, fp64 definition of
what the GPU path computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and this
module imports nothing from the library (it works on numpy arrays only).

What it follows (pages: five articles on hybrid-attention LLM inference):
  * "Day 0 Inference Adaptation and Performance Optimization for Hybrid
    Attention LLMs", section "Index-Selected Sparse Attention": an indexer scores
    all historical positions, the Top-K most relevant are kept, the sparse
    attention reads only the latent KV at those positions.
  * "Hybrid Attention LLM Inference Acceleration ...", section 2 (sparse
    attention path): scoring, head-weight weighting and Top-K selection over the
    paged K cache; attention only over the Top-K positions.
  * "Optimizing Inference for Hybrid-Architecture LLMs ...", section 2.2 and
    section 3.1 (indexer three-in-one fusion): scores are weighted by head
    weights and compared for Top-K.
The exact formula is S[p] = sum_h w_h * ReLU(q_h . k_p) over indexer heads h,
MLA attention over the 576-wide latent rows (512 "nope" + 64 rope) with value =
the first 512 dims and softmax scale 1/sqrt(576).

Readings where the pages are silent:
  * one index key per token, shared by all indexer heads; w is per query token;
  * FP8 data is OCP e4m3fn codes times an fp32 scale (per token for keys, per
    (token, head) for queries), dequantized before the dot product;
  * MXFP8 data ("Optimizing Inference for Hybrid-Architecture LLMs", section
    4.2: one shared scale per group of 32 elements) is OCP microscaling:
    e4m3fn codes times the group's E8M0 scale 2^(byte - 127);
  * quantizing a query: an FP8 scale is amax/448 in float32 (1 for an
    all-zero row), an MXFP8 group scale 2^(floor(log2 amax) - 8) (2^0 for an
    all-zero group); values are divided by the scale, clamped to +-448 and
    rounded to nearest even e4m3fn;
  * Top-K keeps k_t = min(K, n_t) positions; ties go to the lower logical
    position; outputs are physical pool slots, valid ones first, then -1;
  * a query with no visible position attends over nothing and outputs zeros;
  * FP8 latent KV: per token, 4 scales over the 512 nope dims (tiles of 128),
    the 64 rope dims kept in bf16; attention runs over the dequantized rows;
  * residual + RMSNorm after the attention: over the token's H x 512 output
    values (no output projection is part of the layer), with a given norm
    weight and epsilon.

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, hand-worked values, a library routine (torch's float8 decode and its
float64 scaled_dot_product_attention), brute force on tiny inputs, or an
invariant.  No function is left "parity unpinned".
"""
from __future__ import annotations

import numpy as np

PAGE = 64
LATENT = 576
VDIM = 512
KV_TILE = 128                       # FP8 latent: one scale per 128 nope elements of a token
KV_FP8_ROW = VDIM + 4 * (VDIM // KV_TILE) + 2 * (LATENT - VDIM)   # 656 bytes per token


# --------------------------------------------------------------------------- decoding
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 (bf16 is the top half of an fp32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def fp8_e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn code -> float64, decoded bit by bit: sign bit, 4-bit exponent
    with bias 7, 3-bit mantissa; exponent 0 is subnormal (m/8 * 2^-6); no
    infinities; S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, v)


MX_GROUP = 32


def e8m0_to_f64(scale_bytes: np.ndarray) -> np.ndarray:
    """E8M0 scale byte b -> 2^(b - 127) as float64 (an exponent-only format
    with bias 127); b = 255 is NaN."""
    b = np.asarray(scale_bytes, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def mxfp8_to_f64(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """MXFP8 dequantization along the last axis: each run of MX_GROUP
    consecutive e4m3fn codes is multiplied by the E8M0 scale of its group.
    codes [..., D], scale_bytes [..., D / MX_GROUP]."""
    return fp8_e4m3fn_to_f64(codes) * np.repeat(e8m0_to_f64(scale_bytes), MX_GROUP, axis=-1)


# --------------------------------------------------------------------------- index-query quantization
# The step before the path: the projected indexer query (bf16) becomes e4m3fn
# codes plus scales ("Inference Acceleration for a New Domestic LLM
# Architecture", section 3: a Q-quantization launch in the index pre-stage;
# "Optimizing Inference for Hybrid-Architecture LLMs", sections 3.2 and 4.2;
# "Hybrid Attention LLM Inference Acceleration", sections 4 and 5).  The pages
# give the group size (32) but no scale rule: a per-(token, head) scale is
# amax/448, an MX group scale the power of two that puts amax's exponent at
# e4m3's largest (8).  Scale arithmetic is float32, as an fp32 device computes
# it, so the integer codes are decided in the same precision on both sides;
# the e4m3 rounding itself is exact.
E4M3_MAX = 448.0


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of finite values with |y| <= 448 to OCP e4m3fn
    codes (bit patterns), from the format's definition: subnormals are
    multiples of 2^-9 below 2^-6; a normal value 2^e (1 + m/8) has exponent
    field e + 7 (1..15) and mantissa m; ties go to the even mantissa."""
    y = np.asarray(y, dtype=np.float64)
    sign = (np.signbit(y)).astype(np.int64) << 7
    a = np.abs(y)
    codes = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal: n = RNE(a / 2^-9), n in 0..8 (8 = the smallest normal, code 0x08)
    codes[sub] = np.round(a[sub] * 2.0 ** 9).astype(np.int64)   # np.round is half-to-even
    nrm = ~sub
    e = np.floor(np.log2(a[nrm])).astype(np.int64)
    frac = a[nrm] / np.exp2(e.astype(np.float64))                 # in [1, 2), exact
    m = np.round((frac - 1.0) * 8.0).astype(np.int64)             # 0..8, half-to-even
    e = e + (m == 8)
    m = np.where(m == 8, 0, m)
    codes[nrm] = ((e + 7) << 3) | m
    return (codes | sign).astype(np.uint8)


def quantize_fp8_per_row(x: np.ndarray):
    """Per-row e4m3fn quantization of float values x [..., D]: s = amax/448 in
    float32 (1 when amax = 0); codes = e4m3(RNE(clamp(x/s, +-448))) with x/s
    rounded to float32.  Returns (uint8 codes, float32 scales [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    y = np.clip((x32 / s[..., None]).astype(np.float32), -E4M3_MAX, E4M3_MAX)
    return e4m3fn_encode(y), s


def quantize_mxfp8(x: np.ndarray):
    """OCP microscaling e4m3 along the last axis in groups of 32: group scale
    2^e with e = floor(log2(amax)) - 8 (8 = e4m3's largest exponent; e = 0 when
    amax = 0; clamped to [-127, 127]); codes = e4m3(RNE(clamp(x / 2^e, +-448))).
    Returns (uint8 codes, uint8 E8M0 bytes e + 127)."""
    x32 = np.asarray(x, dtype=np.float32)
    g = x32.reshape(*x32.shape[:-1], x32.shape[-1] // MX_GROUP, MX_GROUP).astype(np.float64)
    amax = np.abs(g).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0).astype(np.int64)
    e = np.clip(e, -127, 127)
    y = np.clip(g / np.exp2(e.astype(np.float64))[..., None], -E4M3_MAX, E4M3_MAX)   # exact: power of two
    return e4m3fn_encode(y).reshape(x32.shape), (e + 127).astype(np.uint8)


# --------------------------------------------------------------------------- paged cache access
def logical_slots(block_row: np.ndarray, n: int) -> np.ndarray:
    """Physical slot of logical positions 0..n-1 of one sequence: the page id
    from the block table times 64, plus the offset inside the 64-token page."""
    p = np.arange(n, dtype=np.int64)
    return np.asarray(block_row, dtype=np.int64)[p // PAGE] * PAGE + p % PAGE


def index_keys(k_idx_pool: np.ndarray, idx_dtype: str, D: int, slots: np.ndarray) -> np.ndarray:
    """Dequantized index keys [len(slots), D] (float64) at the given pool slots."""
    slots = np.asarray(slots, dtype=np.int64)
    if idx_dtype == "bf16":
        pool = np.asarray(k_idx_pool).reshape(-1, D)
        return bf16_to_f64(pool[slots])
    if idx_dtype == "fp8":
        pages = np.asarray(k_idx_pool, dtype=np.uint8)
        page, row = slots // PAGE, slots % PAGE
        cols = row[:, None] * D + np.arange(D)[None, :]
        codes = pages[page[:, None], cols]
        sbytes = pages[page[:, None], PAGE * D + 4 * row[:, None] + np.arange(4)[None, :]]
        scale = np.ascontiguousarray(sbytes).view("<f4").reshape(-1).astype(np.float64)
        return fp8_e4m3fn_to_f64(codes) * scale[:, None]
    if idx_dtype == "mxfp8":
        pages = np.asarray(k_idx_pool, dtype=np.uint8)
        page, row = slots // PAGE, slots % PAGE
        ng = D // MX_GROUP
        codes = pages[page[:, None], row[:, None] * D + np.arange(D)[None, :]]
        sbytes = pages[page[:, None], PAGE * D + ng * row[:, None] + np.arange(ng)[None, :]]
        return mxfp8_to_f64(codes, sbytes)
    raise ValueError(idx_dtype)


def index_query(q_idx_t: np.ndarray, q_scale_t, idx_dtype: str) -> np.ndarray:
    """Dequantized indexer query of one token, [H_idx, D] float64."""
    if idx_dtype == "bf16":
        return bf16_to_f64(q_idx_t)
    if idx_dtype == "mxfp8":
        return mxfp8_to_f64(q_idx_t, q_scale_t)
    return fp8_e4m3fn_to_f64(q_idx_t) * np.asarray(q_scale_t, dtype=np.float64)[:, None]


# --------------------------------------------------------------------------- the three steps
def indexer_scores(qv: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """S[p] = sum_h w[h] * max(0, q[h] . k[p]) for every key row p (float64)."""
    dots = keys @ qv.T                      # [n, H_idx]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def topk_positions(S: np.ndarray, K: int) -> np.ndarray:
    """The min(K, n) positions with the largest S, ties to the lower position,
    by a full stable sort on (-S, position)."""
    n = S.shape[0]
    order = np.lexsort((np.arange(n), -S))
    return order[: min(K, n)]


def sparse_mla(qh: np.ndarray, rows: np.ndarray, scale: float, return_probs: bool = False):
    """Dense softmax attention of the H query heads over the gathered latent rows:
    Z = scale * q . row (576-wide), P = softmax over rows, out = P @ rows[:, :512].
    No rows -> zeros."""
    H = qh.shape[0]
    if rows.shape[0] == 0:
        out = np.zeros((H, VDIM))
        return (out, np.zeros((H, 0))) if return_probs else out
    Z = scale * (qh @ rows.T)
    Z = Z - Z.max(axis=1, keepdims=True)
    E = np.exp(Z)
    P = E / E.sum(axis=1, keepdims=True)
    out = P @ rows[:, :VDIM]
    return (out, P) if return_probs else out


# --------------------------------------------------------------------------- per-query drivers
def query_geometry(case: dict, t: int):
    """(sequence b, visible count n_t, slots of positions 0..n_t-1)."""
    b = int(case["q_seq"][t])
    n = int(min(case["q_visible"][t], case["seq_lens"][b]))
    n = max(n, 0)
    return b, n, logical_slots(case["block_table"][b], n)


def query_scores(case: dict, t: int):
    """Indexer scores of query t over its visible positions, plus their slots."""
    b, n, slots = query_geometry(case, t)
    qv = index_query(case["q_idx"][t], None if case["q_idx_scale"] is None else case["q_idx_scale"][t],
                     case["idx_dtype"])
    keys = index_keys(case["k_idx_pool"], case["idx_dtype"], case["D_idx"], slots)
    return indexer_scores(qv, case["w"][t], keys), slots


def latent_rows_fp8(rows: np.ndarray) -> np.ndarray:
    """FP8 latent rows (uint8 [n][656]) -> float64 [n][576].  The main attention
    KV is FP8 with one scale per token and 128-element tile ("Hybrid Attention
    LLM Inference Acceleration", section 5 table; "Inference Acceleration for a
    New Domestic LLM Architecture", section 4).  A token's row: 512 e4m3fn codes
    of the nope dims, then 4 little-endian fp32 scales (tile t covers dims
    128t..128t+127), then the 64 rope dims in bf16 (the pages do not say how
    rope dims are stored; kept in bf16).  Nope dim d = e4m3(code[d]) * scale[d // 128]."""
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8).reshape(-1, KV_FP8_ROW))
    ntile = VDIM // KV_TILE
    scales = r[:, VDIM: VDIM + 4 * ntile].copy().view("<f4").astype(np.float64)
    rope = r[:, VDIM + 4 * ntile:].copy().view("<u2")
    nope = fp8_e4m3fn_to_f64(r[:, :VDIM]) * np.repeat(scales, KV_TILE, axis=1)
    return np.concatenate([nope, bf16_to_f64(rope)], axis=1)


def latent_rows(case: dict, slots: np.ndarray) -> np.ndarray:
    slots = np.asarray(slots, dtype=np.int64)
    if case.get("kv_dtype", "bf16") == "fp8":
        return latent_rows_fp8(np.asarray(case["kv_pool"]).reshape(-1, KV_FP8_ROW)[slots])
    return bf16_to_f64(np.asarray(case["kv_pool"]).reshape(-1, LATENT)[slots])


def mla_query(case: dict, t: int, slots) -> np.ndarray:
    """Sparse MLA output [H, 512] of query t over the given slots (-1 entries skipped)."""
    slots = np.asarray(slots, dtype=np.int64)
    slots = slots[slots >= 0]
    qh = bf16_to_f64(np.asarray(case["q"][t]))
    return sparse_mla(qh, latent_rows(case, slots), case["scale"])


def residual_rmsnorm(attn: np.ndarray, residual: np.ndarray, gamma: np.ndarray, eps: float):
    """The step after the attention ("Day-0 Inference Adaptation for LLMs",
    operator section 2: the residual connection and normalization that follow
    sparse attention, fused into its tail).  Per query token, over the token's
    whole output vector (H heads x 512, flattened): y = attn + residual (the new
    residual stream), out = y / sqrt(mean(y^2) + eps) * gamma.  Returns (y, out)
    as float64, same shapes as attn."""
    a = np.asarray(attn, dtype=np.float64)
    T = a.shape[0]
    y = a.reshape(T, -1) + np.asarray(residual, dtype=np.float64).reshape(T, -1)
    ms = np.mean(y * y, axis=1, keepdims=True)
    out = y / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64).reshape(1, -1)
    return y.reshape(a.shape), out.reshape(a.shape)


def layer_query(case: dict, t: int) -> dict:
    """The whole layer for query t: scores, Top-K slots (padded to K with -1), output."""
    S, slots = query_scores(case, t)
    pos = topk_positions(S, case["K"])
    sel = np.full(case["K"], -1, dtype=np.int64)
    sel[: pos.shape[0]] = slots[pos]
    return dict(scores=S, slots=slots, positions=pos, indices=sel, out=mla_query(case, t, sel))


def layer_all(case: dict) -> dict:
    """layer_query for every query of a (small) case."""
    res = [layer_query(case, t) for t in range(case["T"])]
    return dict(indices=np.stack([r["indices"] for r in res]), out=np.stack([r["out"] for r in res]),
                per_query=res)
