"""Python binding of the DSA C ABI (include/dsa.h) via ctypes.

Argument marshalling only: every step of the layer runs in libdsa.so.  Torch
tensors supply device memory and the current HIP stream.  Importing this module
loads the library and fails loudly when it is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

IDX_BF16 = 0
IDX_FP8_E4M3FN = 1
IDX_MXFP8_E4M3 = 2
KV_BF16 = 0
KV_FP8_TILE128 = 1
KV_FP8_ROW = 656
PAGE = 64
LATENT = 576
VDIM = 512
MAX_K = 2048

# Every symbol the header declares (checked by the tests against include/dsa.h).
EXPORTS = ("dsa_workspace_bytes", "dsa_workspace_init", "dsa_indexer_topk", "dsa_indexer_scores", "dsa_sparse_mla_attn", "dsa_layer",
           "dsa_layer_static", "dsa_quantize_index_q", "dsa_check_tables", "dsa_status_str", "dsa_abi_version")
TABLE_NAMES = ("seq_lens", "block_table", "q_seq", "q_visible")
STATIC_SCRATCH_BYTES = 64 << 20
WS_RESERVED_BYTES = 32768  # counter region at the start of a workspace (zero before first use)


class DSAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dsa status {status}: {msg}")
        self.status = status


class IndexerArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("B", ctypes.c_int32), ("H_idx", ctypes.c_int32), ("D_idx", ctypes.c_int32),
        ("idx_dtype", ctypes.c_int32),
        ("q_idx", ctypes.c_void_p), ("q_idx_scale", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("k_idx_pool", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p), ("q_seq", ctypes.c_void_p), ("q_visible", ctypes.c_void_p),
        ("max_q_per_seq", ctypes.c_int32),
    ]


class MlaArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("q", ctypes.c_void_p), ("kv_pool", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64), ("kv_dtype", ctypes.c_int32),
        ("residual", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p), ("residual_out", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_07_amd.build`; "
                          "the DSA layer has no non-HIP path")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.dsa_workspace_bytes.restype = ctypes.c_size_t
    lib.dsa_workspace_bytes.argtypes = [P(IndexerArgs), P(MlaArgs), ctypes.c_int]
    lib.dsa_workspace_init.restype = ctypes.c_int
    lib.dsa_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.dsa_indexer_topk.restype = ctypes.c_int
    lib.dsa_indexer_topk.argtypes = [P(IndexerArgs), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
    lib.dsa_indexer_scores.restype = ctypes.c_int
    lib.dsa_indexer_scores.argtypes = [P(IndexerArgs), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
    lib.dsa_sparse_mla_attn.restype = ctypes.c_int
    lib.dsa_sparse_mla_attn.argtypes = [P(MlaArgs), ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.dsa_layer.restype = ctypes.c_int
    lib.dsa_layer.argtypes = [P(IndexerArgs), P(MlaArgs), ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.dsa_layer_static.restype = ctypes.c_int
    lib.dsa_layer_static.argtypes = [P(IndexerArgs), P(MlaArgs), ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_quantize_index_q.restype = ctypes.c_int
    lib.dsa_quantize_index_q.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_check_tables.restype = ctypes.c_int
    lib.dsa_check_tables.argtypes = [P(IndexerArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, P(ctypes.c_int32), P(ctypes.c_int64)]
    lib.dsa_status_str.restype = ctypes.c_char_p
    lib.dsa_status_str.argtypes = [ctypes.c_int]
    lib.dsa_abi_version.restype = ctypes.c_int
    lib.dsa_abi_version.argtypes = []
    return lib


LIB = _load()


def status_str(code: int) -> str:
    return LIB.dsa_status_str(code).decode()


def _check(code: int):
    if code != 0:
        raise DSAError(code, status_str(code))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def indexer_args(q_idx, w, k_idx_pool, block_table, seq_lens, *, q_idx_scale=None, q_seq=None, q_visible=None,
                 max_q_per_seq: int = 1, num_blocks: Optional[int] = None) -> IndexerArgs:
    """Build the C struct from tensors (no copies; tensors must stay alive)."""
    # uint8 codes with fp32 scales: FP8 (per token / head); with uint8 scales:
    # MXFP8 (E8M0 per 32 elements)
    fp8 = q_idx.dtype == torch.uint8
    mx = fp8 and q_idx_scale is not None and q_idx_scale.dtype == torch.uint8
    T, H_idx, D_idx = q_idx.shape
    a = IndexerArgs()
    a.T, a.B, a.H_idx, a.D_idx = T, seq_lens.shape[0], H_idx, D_idx
    a.idx_dtype = IDX_MXFP8_E4M3 if mx else (IDX_FP8_E4M3FN if fp8 else IDX_BF16)
    a.q_idx, a.q_idx_scale, a.w = _ptr(q_idx), _ptr(q_idx_scale), _ptr(w)
    a.k_idx_pool = _ptr(k_idx_pool)
    a.num_blocks = k_idx_pool.shape[0] if num_blocks is None else num_blocks
    a.block_table, a.max_blocks = _ptr(block_table), block_table.shape[1]
    a.seq_lens, a.q_seq, a.q_visible = _ptr(seq_lens), _ptr(q_seq), _ptr(q_visible)
    a.max_q_per_seq = max_q_per_seq
    return a


def mla_args(q, kv_pool, *, residual=None, norm_weight=None, residual_out=None, eps: float = 1e-6) -> MlaArgs:
    """kv_pool: bf16 [slots, 576], or uint8 [slots, 656] FP8 latent rows.  With
    `residual` ([T, H, 512] bf16), the output becomes RMSNorm(attn + residual) *
    norm_weight and residual_out receives attn + residual."""
    m = MlaArgs()
    m.T, m.H = q.shape[0], q.shape[1]
    m.q, m.kv_pool = _ptr(q), _ptr(kv_pool)
    m.num_blocks = kv_pool.shape[0] // PAGE
    m.kv_dtype = KV_FP8_TILE128 if kv_pool.dtype == torch.uint8 else KV_BF16
    m.residual, m.norm_weight, m.residual_out = _ptr(residual), _ptr(norm_weight), _ptr(residual_out)
    m.norm_eps = eps
    return m


def workspace_bytes(idx: Optional[IndexerArgs], mla: Optional[MlaArgs], K: int) -> int:
    return int(LIB.dsa_workspace_bytes(None if idx is None else ctypes.byref(idx),
                                       None if mla is None else ctypes.byref(mla), K))


def workspace_init(workspace: torch.Tensor) -> torch.Tensor:
    """dsa_workspace_init on the current stream: clears the counter region a
    new workspace must start with (once; calls leave it clear)."""
    _check(LIB.dsa_workspace_init(_ptr(workspace), workspace.numel(), _stream()))
    return workspace


def _workspace(nbytes: int, device) -> torch.Tensor:
    # 256-byte aligned by the caching allocator; only the counter region needs
    # initialising
    return workspace_init(torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device))


def indexer_topk(q_idx, w, k_idx_pool, block_table, seq_lens, K: int, *, q_idx_scale=None, q_seq=None,
                 q_visible=None, max_q_per_seq: int = 1, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer + Top-K: int32 [T, K] physical pool slots (ascending position), -1 padded.
    A `workspace` passed in must have been through workspace_init once."""
    a = indexer_args(q_idx, w, k_idx_pool, block_table, seq_lens, q_idx_scale=q_idx_scale, q_seq=q_seq,
                     q_visible=q_visible, max_q_per_seq=max_q_per_seq)
    if out is None:
        out = torch.empty(a.T, K, dtype=torch.int32, device=q_idx.device)
    need = workspace_bytes(a, None, K)
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, q_idx.device)
    _check(LIB.dsa_indexer_topk(ctypes.byref(a), K, _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


def indexer_scores(q_idx, w, k_idx_pool, block_table, seq_lens, *, q_idx_scale=None, q_seq=None, q_visible=None,
                   max_q_per_seq: int = 1, fill: float = float("nan")) -> torch.Tensor:
    """Debugging aid: the indexer's fused fp32 scores [T, 64 * max_blocks] as
    the Top-K compares them (positions not visible or on absent pages keep
    `fill`)."""
    a = indexer_args(q_idx, w, k_idx_pool, block_table, seq_lens, q_idx_scale=q_idx_scale, q_seq=q_seq,
                     q_visible=q_visible, max_q_per_seq=max_q_per_seq)
    ld = PAGE * a.max_blocks
    scores = torch.full((a.T, ld), fill, dtype=torch.float32, device=q_idx.device)
    workspace = _workspace(workspace_bytes(a, None, 1), q_idx.device)
    _check(LIB.dsa_indexer_scores(ctypes.byref(a), _ptr(scores), ld, _ptr(workspace), workspace.numel(), _stream()))
    return scores


def check_tables(q_idx, w, k_idx_pool, block_table, seq_lens, *, q_idx_scale=None, q_seq=None, q_visible=None,
                 max_q_per_seq: int = 1):
    """Debugging aid: checks host copies of the tables an indexer call reads
    (the arguments are those of indexer_topk).  Returns None when every entry
    is in range, else (table name, flat index) of the first bad entry."""
    a = indexer_args(q_idx, w, k_idx_pool, block_table, seq_lens, q_idx_scale=q_idx_scale, q_seq=q_seq,
                     q_visible=q_visible, max_q_per_seq=max_q_per_seq)
    host = [None if x is None else x.detach().to("cpu", torch.int32).contiguous()
            for x in (seq_lens, block_table, q_seq, q_visible)]
    table, index = ctypes.c_int32(-1), ctypes.c_int64(-1)
    code = LIB.dsa_check_tables(ctypes.byref(a), *[_ptr(x) for x in host], ctypes.byref(table), ctypes.byref(index))
    if code == 10:
        return TABLE_NAMES[table.value], int(index.value)
    _check(code)
    return None


def sparse_mla_attn(q, kv_pool, indices, scale: float, *, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, residual=None, norm_weight=None, residual_out=None,
                    eps: float = 1e-6) -> torch.Tensor:
    """Sparse MLA: bf16 [T, H, 512] over the latent rows at `indices` (-1 skipped);
    with `residual`, RMSNorm(attn + residual) * norm_weight (see mla_args)."""
    m = mla_args(q, kv_pool, residual=residual, norm_weight=norm_weight, residual_out=residual_out, eps=eps)
    K = indices.shape[1]
    if out is None:
        out = torch.empty(m.T, m.H, VDIM, dtype=torch.bfloat16, device=q.device)
    need = workspace_bytes(None, m, K)
    if need and (workspace is None or workspace.numel() < need):
        workspace = _workspace(need, q.device)
    _check(LIB.dsa_sparse_mla_attn(ctypes.byref(m), _ptr(indices), K, float(scale), _ptr(out),
                                   _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))
    return out


def quantize_index_q(q: torch.Tensor, idx_dtype: int = IDX_FP8_E4M3FN, *, codes: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None):
    """Index-query quantization of bf16 q [..., D]: returns (uint8 codes [..., D],
    scales) with scales fp32 [...] (FP8) or uint8 E8M0 [..., D/32] (MXFP8), the
    q_idx / q_idx_scale pair indexer_topk takes."""
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 tensor")
    D = q.shape[-1]
    lead = tuple(q.shape[:-1])
    if codes is None:
        codes = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    if scales is None:
        scales = (torch.empty(lead, dtype=torch.float32, device=q.device) if idx_dtype == IDX_FP8_E4M3FN
                  else torch.empty(lead + (max(D // 32, 1),), dtype=torch.uint8, device=q.device))
    rows = q.numel() // max(D, 1)
    _check(LIB.dsa_quantize_index_q(_ptr(q), rows, D, idx_dtype, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


class Layer:
    """The fused layer (indexer, Top-K, sparse MLA in one launch sequence) with
    its argument structs and workspace built once, so repeated calls only
    enqueue kernels."""

    def __init__(self, q_idx, w, k_idx_pool, block_table, seq_lens, q, kv_pool, K: int, scale: float, *,
                 q_idx_scale=None, q_seq=None, q_visible=None, max_q_per_seq: int = 1,
                 want_indices: bool = True, residual=None, norm_weight=None, residual_out=None, eps: float = 1e-6):
        self._keep = (q_idx, w, k_idx_pool, block_table, seq_lens, q, kv_pool, q_idx_scale, q_seq, q_visible,
                      residual, norm_weight, residual_out)
        self.idx = indexer_args(q_idx, w, k_idx_pool, block_table, seq_lens, q_idx_scale=q_idx_scale,
                                q_seq=q_seq, q_visible=q_visible, max_q_per_seq=max_q_per_seq)
        self.mla = mla_args(q, kv_pool, residual=residual, norm_weight=norm_weight, residual_out=residual_out,
                            eps=eps)
        self.K, self.scale = K, float(scale)
        dev = q.device
        self.out = torch.empty(self.mla.T, self.mla.H, VDIM, dtype=torch.bfloat16, device=dev)
        self.indices = torch.empty(self.idx.T, K, dtype=torch.int32, device=dev) if want_indices else None
        need = workspace_bytes(self.idx, self.mla, K)
        if need == 0:
            raise DSAError(3, "invalid layer arguments")
        self.workspace = _workspace(need, dev)

    def __call__(self):
        _check(LIB.dsa_layer(ctypes.byref(self.idx), ctypes.byref(self.mla), self.K, self.scale,
                             _ptr(self.indices), _ptr(self.out), _ptr(self.workspace), self.workspace.numel(),
                             _stream()))
        return self.out

    def call_static(self, out: Optional[torch.Tensor] = None, indices: Optional[torch.Tensor] = None):
        """The same layer through dsa_layer_static (the library's own scratch,
        no workspace); results go to `out` / `indices` (default: this layer's
        own buffers)."""
        out = self.out if out is None else out
        indices = self.indices if indices is None else indices
        _check(LIB.dsa_layer_static(ctypes.byref(self.idx), ctypes.byref(self.mla), self.K, self.scale,
                                    _ptr(indices), _ptr(out), _stream()))
        return out


def layer_from_case(case, want_indices: bool = True, **epilogue) -> Layer:
    """Layer over a synthetic case (see synth.py); `epilogue` takes residual,
    norm_weight, residual_out and eps."""
    s = case.spec
    return Layer(case.q_idx, case.w, case.k_idx_pool, case.block_table, case.seq_lens, case.q, case.kv_pool, s.K,
                 s.scale, q_idx_scale=case.q_idx_scale, q_seq=case.q_seq, q_visible=case.q_visible,
                 max_q_per_seq=case.max_q_per_seq, want_indices=want_indices, **epilogue)
