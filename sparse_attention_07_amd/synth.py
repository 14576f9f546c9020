"""Seeded synthetic inputs for the DSA sparse-attention layer.

This module only *draws* inputs: sequence lengths, the page permutation of the
paged caches, the index-K cache, the 576-wide latent cache, the indexer queries
and head weights, and the MLA queries.  It holds none of the layer's
arithmetic (no scoring, no selection, no attention) and imports neither the
oracle nor the HIP binding, so both sides can consume the same tensors.

Workloads follow the pages' long-context decode and chunked-prefill setting
("Day 0 Inference Adaptation ... Hybrid Attention LLMs", section
"Index-Selected Sparse Attention"; "Optimizing Inference for Hybrid-Architecture
LLMs", section 2.2) at the five named sizes below.  Values are N(0,1) drawn in
fp32 and rounded to bf16 (round-to-nearest-even); head weights are N(0,1)/2.

FP8 index data (keys: one fp32 scale per token; queries: one fp32 scale per
(token, head)) is produced with scale = amax/448 and torch's
round-to-nearest-even float8_e4m3fn conversion after clamping to +-448
(scale 1 when amax is 0).  MXFP8 index data (one E8M0 power-of-two scale per
32 consecutive elements, "Optimizing Inference for Hybrid-Architecture LLMs",
section 4.2) follows the OCP microscaling recipe: the group scale is
2^(floor(log2(amax)) - 8) (8 = the largest e4m3 exponent; 2^0 for an all-zero
group), elements are x / scale rounded to nearest-even e4m3fn after clamping
to +-448.  This is input preparation; the method consumes the codes and scales
as given.

Layouts (all contiguous):
  * index-K pool, bf16:  [NB, 64, D_idx] bf16
  * index-K pool, fp8:   [NB, 64*D_idx + 64*4] uint8 per page: 64 rows of
    D_idx e4m3fn codes, then 64 little-endian fp32 scales (8448 B for D_idx=128)
  * index-K pool, mxfp8: [NB, 64*D_idx + 64*D_idx/32] uint8 per page: 64 rows of
    D_idx e4m3fn codes, then per row D_idx/32 E8M0 group-scale bytes
  * latent pool:          [NB*64, 576] bf16 (512 nope + 64 rope), or with kv_dtype
                          "fp8" uint8 [NB*64, 656]: 512 e4m3fn codes, 4 fp32 scales
                          (one per 128 nope dims), 64 bf16 rope dims
  * block_table:          [B, max_blocks] int32 (unused entries are 0)
  * seq_lens:             [B] int32
  * q_idx:                [T, H_idx, D_idx] bf16, or uint8 codes + q_idx_scale [T, H_idx] fp32
                          (fp8) or [T, H_idx, D_idx/32] uint8 E8M0 (mxfp8)
  * q_idx_src:            [T, H_idx, D_idx] bf16 index query before quantization
  * w:                    [T, H_idx] fp32
  * q:                    [T, H, 576] bf16
  * q_seq / q_visible:    [T] int32 (query -> sequence, causal horizon)
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

PAGE = 64
LATENT = 576
VDIM = 512
FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class CaseSpec:
    """A synthetic workload.  ``lens`` fixes each sequence's cached length; when
    it is None, ``B`` lengths are drawn uniformly from ``len_range`` (inclusive).
    ``queries_per_seq`` gives the number of decode queries per sequence (the
    last ones sit on the last cached positions, speculative-decoding style).
    ``prefill`` = (total_len, chunk): one sequence whose queries are its own
    positions, processed in chunks of ``chunk`` queries."""
    name: str
    H_idx: int
    D_idx: int
    idx_dtype: str  # "bf16" | "fp8" | "mxfp8"
    K: int
    H: int
    lens: Optional[Sequence[int]] = None
    len_range: Optional[Sequence[int]] = None
    B: int = 0
    queries_per_seq: Optional[Sequence[int]] = None
    prefill: Optional[Sequence[int]] = None
    seed: int = 0
    scale: float = 1.0 / math.sqrt(LATENT)
    permute_pages: bool = True
    kv_dtype: str = "bf16"  # "bf16" | "fp8" (e4m3fn nope dims, one fp32 scale per 128, bf16 rope)


# The five workloads the pages' path is measured on.
PRESETS = {
    "tiny_decode": CaseSpec("tiny_decode", H_idx=4, D_idx=64, idx_dtype="bf16", K=256, H=16, lens=[4096]),
    "decode_b32_32k": CaseSpec("decode_b32_32k", H_idx=64, D_idx=128, idx_dtype="bf16", K=2048, H=128,
                               lens=[32768] * 32),
    "decode_b64_128k_fp8": CaseSpec("decode_b64_128k_fp8", H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128,
                                    len_range=(65536, 131072), B=64),
    # the benchmark decode shape with the pages' MXFP8 (group-32) index quantization
    "decode_b64_128k_mxfp8": CaseSpec("decode_b64_128k_mxfp8", H_idx=64, D_idx=128, idx_dtype="mxfp8", K=2048,
                                      H=128, len_range=(65536, 131072), B=64),
    # the benchmark decode shape with the latent cache in FP8 (one scale per token and 128 nope dims)
    "decode_b64_128k_fp8kv": CaseSpec("decode_b64_128k_fp8kv", H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128,
                                      len_range=(65536, 131072), B=64, kv_dtype="fp8"),
    "prefill_16k": CaseSpec("prefill_16k", H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128,
                            prefill=(16384, 4096)),
    "mixed_1m": CaseSpec("mixed_1m", H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128,
                         lens=[4096, 16384, 65536, 131072, 262144, 524288, 786432, 1048576],
                         queries_per_seq=[1, 1, 1, 1, 1, 1, 1, 4]),
}


@dataclasses.dataclass
class Case:
    spec: CaseSpec
    seq_lens: torch.Tensor
    block_table: torch.Tensor
    num_blocks: int
    k_idx_pool: torch.Tensor
    kv_pool: torch.Tensor
    q_idx: torch.Tensor
    q_idx_scale: Optional[torch.Tensor]
    w: torch.Tensor
    q: torch.Tensor
    q_seq: torch.Tensor
    q_visible: torch.Tensor
    max_q_per_seq: int
    # the bf16 index query the codes were quantized from (== q_idx for bf16)
    q_idx_src: Optional[torch.Tensor] = None

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])


def _randn_bf16(gen: torch.Generator, shape, device, scale: float = 1.0, chunk_elems: int = 1 << 26) -> torch.Tensor:
    """N(0,1)*scale drawn in fp32 in fixed-size pieces (bounded temporaries), rounded to bf16."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[s:e] = x.to(torch.bfloat16)
    return out


def quantize_fp8_rows(x: torch.Tensor):
    """Per-row e4m3fn quantization: scale = amax/448 (1 if amax == 0),
    codes = RNE(x/scale) after clamping to +-448.  Returns (uint8 codes, fp32 scales)."""
    xf = x.to(torch.float32)
    amax = xf.abs().amax(dim=-1)
    scale = amax / FP8_MAX
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    y = (xf / scale.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


MX_GROUP = 32
E4M3_EMAX = 8  # largest e4m3 exponent: 448 = 1.75 * 2^8


def quantize_mxfp8_rows(x: torch.Tensor):
    """OCP microscaling e4m3 along the last dim (a multiple of 32): per group of
    32, scale = 2^(floor(log2(amax)) - 8) (2^0 if amax == 0, exponent clamped
    to [-127, 127]); codes = RNE(x/scale) after clamping to +-448.  Returns
    (uint8 codes, uint8 E8M0 scale bytes = exponent + 127, one per group)."""
    xf = x.to(torch.float32)
    g = xf.reshape(*xf.shape[:-1], xf.shape[-1] // MX_GROUP, MX_GROUP)
    amax = g.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    e = torch.where(amax > 0, ex - 1 - E4M3_EMAX, torch.zeros_like(ex)).clamp_(-127, 127)
    scale = torch.ldexp(torch.ones_like(amax), e)
    y = (g / scale.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(xf.shape)
    return codes, (e + 127).to(torch.uint8)


KV_TILE = 128
KV_FP8_ROW = VDIM + 4 * (VDIM // KV_TILE) + 2 * (LATENT - VDIM)  # 656 bytes per token


def pack_fp8_latent(kv: torch.Tensor) -> torch.Tensor:
    """bf16 latent rows [N, 576] -> FP8 rows uint8 [N, 656]: the 512 nope dims as
    e4m3fn codes with one fp32 scale per 128 (scale = amax/448 of the tile, as
    for the index data), then the 4 scales, then the 64 rope dims unchanged."""
    N = kv.shape[0]
    out = torch.empty(N, KV_FP8_ROW, dtype=torch.uint8, device=kv.device)
    step = 1 << 20
    for a in range(0, N, step):
        b = min(N, a + step)
        nope = kv[a:b, :VDIM].reshape(b - a, VDIM // KV_TILE, KV_TILE)
        codes, sc = quantize_fp8_rows(nope)
        out[a:b, :VDIM] = codes.reshape(b - a, VDIM)
        out[a:b, VDIM: VDIM + 4 * (VDIM // KV_TILE)] = sc.contiguous().view(torch.uint8).reshape(b - a, -1)
        out[a:b, VDIM + 4 * (VDIM // KV_TILE):] = kv[a:b, VDIM:].contiguous().view(torch.uint8)
    return out


def _page_bytes(D: int, idx_dtype: str = "fp8") -> int:
    return PAGE * D + (PAGE * D // MX_GROUP if idx_dtype == "mxfp8" else PAGE * 4)


def build_case(spec: CaseSpec, device="cpu", prefill_chunk: Optional[int] = None) -> Case:
    """Draw the case's tensors on ``device``.  Draw order: lengths, page
    permutation, index keys, latent rows, index queries, head weights, MLA
    queries.  For a prefill spec, ``prefill_chunk`` selects which chunk of
    queries the call covers (the caches hold the positions up to that chunk's
    end)."""
    # structure (lengths, page permutation) and values come from two generators
    cpu_gen = torch.Generator(device="cpu")
    cpu_gen.manual_seed(spec.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed + 1)

    # ---- lengths and query layout
    if spec.prefill is not None:
        total, chunk = spec.prefill
        c = 0 if prefill_chunk is None else prefill_chunk
        assert 0 <= c * chunk < total
        q_lo, q_hi = c * chunk, min(total, (c + 1) * chunk)
        lens = [total]
    elif spec.lens is not None:
        lens = list(spec.lens)
    else:
        lo, hi = spec.len_range
        lens = torch.randint(lo, hi + 1, (spec.B,), generator=cpu_gen).tolist()
    B = len(lens)
    nblk = [(L + PAGE - 1) // PAGE for L in lens]
    NB = max(1, sum(nblk))
    max_blocks = max(1, max(nblk))

    # ---- page placement: one pool, pages of all sequences randomly permuted
    perm = torch.randperm(NB, generator=cpu_gen) if spec.permute_pages else torch.arange(NB)
    bt = torch.zeros(B, max_blocks, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, : nblk[b]] = perm[off: off + nblk[b]].to(torch.int32)
        off += nblk[b]

    # ---- index-K cache (tail of each sequence's last page stays zero)
    D = spec.D_idx
    kf = _randn_bf16(gen, (NB, PAGE, D), device)
    valid = torch.zeros(NB * PAGE, dtype=torch.bool)
    for b in range(B):
        pos = torch.arange(lens[b])
        valid[(bt[b, pos // PAGE].long() * PAGE + pos % PAGE)] = True
    valid_d = valid.to(device).view(NB, PAGE)
    kf.masked_fill_(~valid_d.unsqueeze(-1), 0)
    if spec.idx_dtype == "bf16":
        k_pool = kf
    elif spec.idx_dtype == "fp8":
        codes, ks = quantize_fp8_rows(kf)
        k_pool = torch.empty(NB, _page_bytes(D), dtype=torch.uint8, device=device)
        k_pool[:, : PAGE * D] = codes.reshape(NB, PAGE * D)
        k_pool[:, PAGE * D:] = ks.contiguous().view(torch.uint8).reshape(NB, PAGE * 4)
        del codes, ks
    elif spec.idx_dtype == "mxfp8":
        codes, ks = quantize_mxfp8_rows(kf)
        k_pool = torch.empty(NB, _page_bytes(D, "mxfp8"), dtype=torch.uint8, device=device)
        k_pool[:, : PAGE * D] = codes.reshape(NB, PAGE * D)
        k_pool[:, PAGE * D:] = ks.reshape(NB, PAGE * D // MX_GROUP)
        del codes, ks
    else:
        raise ValueError(spec.idx_dtype)
    del kf

    # ---- latent cache
    kv = _randn_bf16(gen, (NB * PAGE, LATENT), device)
    kv.masked_fill_(~valid.to(device).unsqueeze(-1), 0)
    if spec.kv_dtype == "fp8":
        kv = pack_fp8_latent(kv)
    elif spec.kv_dtype != "bf16":
        raise ValueError(spec.kv_dtype)

    # ---- queries
    if spec.prefill is not None:
        T_all = spec.prefill[0]
        q_seq_all = torch.zeros(T_all, dtype=torch.int32)
        q_vis_all = torch.arange(1, T_all + 1, dtype=torch.int32)
        sel = slice(q_lo, q_hi)
        max_q = T_all
    else:
        qps = list(spec.queries_per_seq) if spec.queries_per_seq is not None else [1] * B
        seq_ids, vis = [], []
        for b in range(B):
            n = qps[b]
            for j in range(n):
                seq_ids.append(b)
                vis.append(lens[b] - n + 1 + j)
        T_all = len(seq_ids)
        q_seq_all = torch.tensor(seq_ids, dtype=torch.int32)
        q_vis_all = torch.tensor(vis, dtype=torch.int32)
        sel = slice(0, T_all)
        max_q = max(qps) if qps else 1

    H_i = spec.H_idx
    qi = _randn_bf16(gen, (T_all, H_i, D), device)
    if spec.idx_dtype == "fp8":
        qcodes, qscale = quantize_fp8_rows(qi)
        q_idx, q_idx_scale = qcodes, qscale
    elif spec.idx_dtype == "mxfp8":
        q_idx, q_idx_scale = quantize_mxfp8_rows(qi)
    else:
        q_idx, q_idx_scale = qi, None
    w = torch.randn(T_all, H_i, generator=gen, device=device, dtype=torch.float32) * 0.5
    q = _randn_bf16(gen, (T_all, spec.H, LATENT), device)

    seq_lens = torch.tensor(lens, dtype=torch.int32)
    if spec.prefill is not None:
        # the cache holds the positions written so far: up to this chunk's end
        seq_lens = torch.tensor([q_hi], dtype=torch.int32)

    def dev(t):
        return t.to(device).contiguous()

    return Case(
        spec=spec,
        seq_lens=dev(seq_lens),
        block_table=dev(bt),
        num_blocks=NB,
        k_idx_pool=k_pool.contiguous(),
        kv_pool=kv.contiguous(),
        q_idx=q_idx[sel].contiguous(),
        q_idx_scale=None if q_idx_scale is None else q_idx_scale[sel].contiguous(),
        w=w[sel].contiguous(),
        q=q[sel].contiguous(),
        q_seq=dev(q_seq_all[sel]),
        q_visible=dev(q_vis_all[sel]),
        max_q_per_seq=min(max_q, sel.stop - sel.start),
        q_idx_src=qi[sel].contiguous(),
    )


def to_numpy(case: Case) -> dict:
    """Host copies of a case as numpy arrays (bf16 as uint16 bit patterns)."""
    import numpy as np

    def bits16(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    d = dict(
        T=case.T, B=case.B, H_idx=case.spec.H_idx, D_idx=case.spec.D_idx, idx_dtype=case.spec.idx_dtype,
        K=case.spec.K, H=case.spec.H, scale=case.spec.scale, num_blocks=case.num_blocks,
        seq_lens=case.seq_lens.cpu().numpy(), block_table=case.block_table.cpu().numpy(),
        q_seq=case.q_seq.cpu().numpy(), q_visible=case.q_visible.cpu().numpy(),
        w=case.w.cpu().numpy(), q=bits16(case.q),
    )
    if case.spec.idx_dtype == "bf16":
        d["k_idx_pool"] = bits16(case.k_idx_pool)
        d["q_idx"] = bits16(case.q_idx)
        d["q_idx_scale"] = None
    else:
        d["k_idx_pool"] = case.k_idx_pool.cpu().numpy()
        d["q_idx"] = case.q_idx.cpu().numpy()
        d["q_idx_scale"] = case.q_idx_scale.cpu().numpy()
    if case.spec.kv_dtype == "fp8":
        d["kv_pool"] = case.kv_pool.cpu().numpy()
    else:
        d["kv_pool"] = bits16(case.kv_pool)
    d["kv_dtype"] = case.spec.kv_dtype
    return d
