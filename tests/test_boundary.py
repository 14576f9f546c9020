"""CPU tests of the C ABI: the library loads, exports every function that
include/dsa.h declares, the ctypes structs match the C layout, and every
argument error is reported before anything is launched (no GPU needed: each
case below stops at a host-side check)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

dsa = pytest.importorskip("sparse_attention_07_amd.dsa", reason="libdsa.so not built")

OK, E_NULL, E_DTYPE, E_SHAPE, E_K, E_ALIGN, E_WS, E_UNSUP, E_HIP, E_TOO_LARGE, E_TABLE = range(11)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(dsa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(dsa.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(dsa.LIB, n)


def test_abi_version_and_status_strings():
    m = re.search(r"#define DSA_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == 8
    assert dsa.LIB.dsa_abi_version() == int(m.group(1))
    assert dsa.status_str(0) == "ok"
    for s in range(1, 11):
        assert dsa.status_str(s) and dsa.status_str(s) != "unknown status"
    assert dsa.status_str(99) == "unknown status"


def test_ctypes_structs_match_c_layout(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "dsa.h"
#define F(s, f) printf(#s "." #f " %zu\n", offsetof(s, f))
int main(void) {
  printf("dsa_indexer_args %zu\n", sizeof(dsa_indexer_args));
  printf("dsa_mla_args %zu\n", sizeof(dsa_mla_args));
  F(dsa_indexer_args, T); F(dsa_indexer_args, idx_dtype); F(dsa_indexer_args, q_idx);
  F(dsa_indexer_args, q_idx_scale); F(dsa_indexer_args, w); F(dsa_indexer_args, k_idx_pool);
  F(dsa_indexer_args, num_blocks); F(dsa_indexer_args, block_table); F(dsa_indexer_args, max_blocks);
  F(dsa_indexer_args, seq_lens); F(dsa_indexer_args, q_seq); F(dsa_indexer_args, q_visible);
  F(dsa_indexer_args, max_q_per_seq);
  F(dsa_mla_args, T); F(dsa_mla_args, H); F(dsa_mla_args, q); F(dsa_mla_args, kv_pool); F(dsa_mla_args, num_blocks);
  F(dsa_mla_args, kv_dtype); F(dsa_mla_args, residual); F(dsa_mla_args, norm_weight);
  F(dsa_mla_args, residual_out); F(dsa_mla_args, norm_eps);
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                         check=True).stdout.splitlines())
    assert int(got["dsa_indexer_args"]) == ctypes.sizeof(dsa.IndexerArgs)
    assert int(got["dsa_mla_args"]) == ctypes.sizeof(dsa.MlaArgs)
    for k, v in got.items():
        if "." in k:
            s, f = k.split(".")
            cls = dsa.IndexerArgs if s == "dsa_indexer_args" else dsa.MlaArgs
            assert getattr(cls, f).offset == int(v), k


# ---------------------------------------------------------------- validation (host-only paths)
_buf = ctypes.create_string_buffer(1 << 12)
_base = (ctypes.addressof(_buf) + 255) // 256 * 256  # aligned fake address, never dereferenced


def good_idx(**kw):
    a = dsa.IndexerArgs()
    a.T, a.B, a.H_idx, a.D_idx, a.idx_dtype = 4, 4, 64, 128, dsa.IDX_FP8_E4M3FN
    a.q_idx = a.q_idx_scale = a.w = a.k_idx_pool = a.block_table = a.seq_lens = _base
    a.num_blocks, a.max_blocks, a.max_q_per_seq = 100, 10, 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def good_mla(**kw):
    m = dsa.MlaArgs()
    m.T, m.H, m.q, m.kv_pool, m.num_blocks = 4, 128, _base, _base, 100
    for k, v in kw.items():
        setattr(m, k, v)
    return m


def call_idx(a, K=2048, out=_base, ws=None, ws_bytes=0):
    return dsa.LIB.dsa_indexer_topk(None if a is None else ctypes.byref(a), K, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,K,expect", [
    ({}, 0, E_K), ({}, 2049, E_K), ({}, -5, E_K),
    (dict(idx_dtype=7), 2048, E_DTYPE),
    (dict(q_idx=None), 2048, E_NULL), (dict(w=None), 2048, E_NULL), (dict(k_idx_pool=None), 2048, E_NULL),
    (dict(block_table=None), 2048, E_NULL), (dict(seq_lens=None), 2048, E_NULL),
    (dict(q_idx_scale=None), 2048, E_NULL),
    (dict(idx_dtype=dsa.IDX_BF16), 2048, E_DTYPE),  # bf16 with a scale pointer
    (dict(T=0), 2048, E_SHAPE), (dict(B=0), 2048, E_SHAPE), (dict(H_idx=0), 2048, E_SHAPE),
    (dict(H_idx=65), 2048, E_SHAPE), (dict(max_blocks=0), 2048, E_SHAPE), (dict(num_blocks=0), 2048, E_SHAPE),
    (dict(max_q_per_seq=0), 2048, E_SHAPE), (dict(T=5), 2048, E_SHAPE),  # no q_seq and T != B
    (dict(D_idx=64), 2048, E_UNSUP),  # FP8 with 64-wide heads
    (dict(idx_dtype=dsa.IDX_BF16, q_idx_scale=None, D_idx=96), 2048, E_SHAPE),
    (dict(q_idx=_base + 8), 2048, E_ALIGN), (dict(k_idx_pool=_base + 4), 2048, E_ALIGN),
    (dict(w=_base + 2), 2048, E_ALIGN), (dict(q_seq=_base + 1), 2048, E_ALIGN),
    (dict(num_blocks=1 << 26), 2048, E_SHAPE),
])
def test_indexer_argument_errors(kw, K, expect):
    assert call_idx(good_idx(**kw), K) == expect


def test_indexer_null_struct_output_and_workspace():
    assert call_idx(None) == E_NULL
    assert call_idx(good_idx(), out=None) == E_NULL
    assert call_idx(good_idx(), out=_base + 2) == E_ALIGN
    assert call_idx(good_idx(), ws=None) == E_WS
    need = dsa.workspace_bytes(good_idx(), None, 2048)
    assert need > 0
    assert call_idx(good_idx(), ws=_base, ws_bytes=need - 1) == E_WS
    assert call_idx(good_idx(), ws=_base + 16, ws_bytes=need) == E_WS  # workspace must be 256-B aligned


def test_indexer_scores_argument_errors():
    def call(a, scores=_base, ld=640, ws=None, ws_bytes=0):
        return dsa.LIB.dsa_indexer_scores(None if a is None else ctypes.byref(a), scores, ld, ws, ws_bytes, None)
    assert call(None) == E_NULL
    assert call(good_idx(), scores=None) == E_NULL
    assert call(good_idx(), scores=_base + 2) == E_ALIGN
    assert call(good_idx(), ld=639) == E_SHAPE  # a row must hold 64 * max_blocks positions
    assert call(good_idx(H_idx=0)) == E_SHAPE
    assert call(good_idx()) == E_WS
    need = dsa.workspace_bytes(good_idx(), None, 1)
    assert call(good_idx(), ws=_base, ws_bytes=need - 1) == E_WS


def call_mla(m, K=2048, idx=_base, out=_base, ws=None, ws_bytes=0):
    return dsa.LIB.dsa_sparse_mla_attn(None if m is None else ctypes.byref(m), idx, K, 0.04, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(H=48), E_SHAPE), (dict(H=256), E_SHAPE), (dict(T=0), E_SHAPE), (dict(num_blocks=0), E_SHAPE),
    (dict(q=None), E_NULL), (dict(kv_pool=None), E_NULL), (dict(q=_base + 8), E_ALIGN),
    (dict(kv_pool=_base + 2), E_ALIGN), (dict(kv_dtype=2), E_DTYPE), (dict(kv_dtype=-1), E_DTYPE),
    # residual + RMSNorm epilogue
    (dict(residual=_base), E_NULL), (dict(residual=_base, norm_weight=_base), E_NULL),
    (dict(residual=_base, norm_weight=_base, residual_out=_base, norm_eps=-1.0), E_SHAPE),
    (dict(residual=_base, norm_weight=_base, residual_out=_base, norm_eps=float("nan")), E_SHAPE),
    (dict(residual=_base, norm_weight=_base, residual_out=_base, norm_eps=float("inf")), E_SHAPE),
    (dict(residual=_base + 4, norm_weight=_base, residual_out=_base), E_ALIGN),
    (dict(residual=_base, norm_weight=_base + 2, residual_out=_base), E_ALIGN),
    (dict(residual=_base, norm_weight=_base, residual_out=_base + 4), E_ALIGN),
    (dict(residual=_base, norm_weight=_base + 8, residual_out=_base), E_ALIGN),
    (dict(residual=_base, norm_weight=_base, residual_out=_base + 8), E_ALIGN),
])
def test_mla_argument_errors(kw, expect):
    assert call_mla(good_mla(**kw)) == expect


def test_mla_null_and_workspace():
    assert call_mla(None) == E_NULL
    assert call_mla(good_mla(), idx=None) == E_NULL
    assert call_mla(good_mla(), out=None) == E_NULL
    assert call_mla(good_mla(), out=_base + 4) == E_ALIGN
    assert call_mla(good_mla(), K=0) == E_K
    # 4 queries -> the rows are split and partial results need workspace
    assert dsa.workspace_bytes(None, good_mla(), 2048) > 0
    assert call_mla(good_mla()) == E_WS
    # the residual epilogue adds one fp32 sum of squares per (query, head) when rows are split
    ep = dict(residual=_base, norm_weight=_base, residual_out=_base, norm_eps=1e-6)
    assert dsa.workspace_bytes(None, good_mla(**ep), 2048) >= dsa.workspace_bytes(None, good_mla(), 2048) + 4 * 128 * 4
    assert dsa.workspace_bytes(None, good_mla(T=1000, **ep), 2048) == dsa.workspace_bytes(None, good_mla(T=1000), 2048)


@pytest.mark.parametrize("T,H,K,splits", [
    (64, 128, 2048, 4),   # the 128K decode batch: 256 workgroups
    (32, 128, 2048, 8),   # 32 queries: 8 splits of 256 rows
    (11, 128, 2048, 8),   # at most 8 splits (the combine's width)
    (1, 16, 256, 8),      # a short list splits down to one 32-row tile per workgroup
    (1, 16, 100, 2),      # 100 rows: 3 splits asked for, 64-row (two-tile) splits give 2
    (1, 16, 40, 1),       # under two tiles: one split
    (4096, 128, 2048, 1), # a prefill chunk: one workgroup per query, no partials
])
def test_mla_split_count_sizes_the_partials(T, H, K, splits):
    # with S > 1 splits the workspace holds bf16 partials [T][S][H][512] and
    # fp32 (m, l) pairs [T][S][H][2], each region 256-byte aligned, past the
    # counter region an indexer call sharing the workspace keeps at its start
    def align(n):
        return (n + 255) // 256 * 256
    want = 0 if splits == 1 else (dsa.WS_RESERVED_BYTES + align(T * splits * H * 512 * 2)
                                  + align(T * splits * H * 2 * 4))
    assert dsa.workspace_bytes(None, good_mla(T=T, H=H), K) == want


def test_layer_argument_errors():
    def call(a, m, out=_base, ws=None, ws_bytes=0, idx_out=None):
        return dsa.LIB.dsa_layer(ctypes.byref(a), ctypes.byref(m), 2048, 0.04, idx_out, out, ws, ws_bytes, None)
    assert call(good_idx(), good_mla(T=3)) == E_SHAPE
    assert call(good_idx(), good_mla(num_blocks=99)) == E_SHAPE
    assert call(good_idx(), good_mla(), out=None) == E_NULL
    assert call(good_idx(), good_mla(), idx_out=_base + 1) == E_ALIGN
    assert call(good_idx(H_idx=0), good_mla()) == E_SHAPE
    assert call(good_idx(), good_mla(H=3)) == E_SHAPE
    need = dsa.workspace_bytes(good_idx(), good_mla(), 2048)
    assert need > dsa.workspace_bytes(good_idx(), None, 2048)
    assert call(good_idx(), good_mla(), ws=_base, ws_bytes=need - 256) == E_WS


def test_workspace_bytes_invalid_and_scaling():
    assert dsa.workspace_bytes(good_idx(T=0), None, 2048) == 0
    assert dsa.workspace_bytes(None, good_mla(H=7), 2048) == 0
    # 64 sequences of up to 128K tokens: bounded candidate storage (well under 1 GB)
    a = good_idx(T=64, B=64, max_blocks=2048, num_blocks=100000)
    n = dsa.workspace_bytes(a, good_mla(T=64, num_blocks=100000), 2048)
    assert 0 < n < (1 << 30)
    # a single short-context decode needs no candidate lists (one chunk per query):
    # the counter region and a few plan records
    small = dsa.workspace_bytes(good_idx(T=1, B=1, max_blocks=64), None, 256)
    assert dsa.WS_RESERVED_BYTES < small < dsa.WS_RESERVED_BYTES + 4096


def test_workspace_counter_region_constant_and_init_errors():
    m = re.search(r"#define DSA_WS_RESERVED_BYTES \(\(size_t\)(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) == dsa.WS_RESERVED_BYTES
    init = dsa.LIB.dsa_workspace_init
    assert init(None, 0, None) == 0           # nothing to clear: nothing enqueued
    assert init(None, 4096, None) == E_NULL
    assert init(_base + 16, 4096, None) == E_ALIGN


def test_keyspace_bound():
    # The indexer lays every query group's key range end to end in one space
    # counted in 64-key pages (32-bit): T * (max_blocks + 72) <= 2^30.
    # The last 4096-query chunk of a 1,048,576-token prefill (16,384 pages),
    # with paired queries and with one query per group at 600K tokens, fits.
    one_m = good_idx(T=4096, B=1, max_blocks=16384, num_blocks=16384, max_q_per_seq=4096, q_seq=_base,
                     q_visible=_base)
    assert dsa.workspace_bytes(one_m, None, 2048) > 0
    six = good_idx(T=4096, B=1, max_blocks=9375, num_blocks=9375, max_q_per_seq=1, q_seq=_base, q_visible=_base)
    assert dsa.workspace_bytes(six, None, 2048) > 0
    # at the bound, and one page past it
    edge = (1 << 30) // 4096 - 72
    assert dsa.workspace_bytes(good_idx(T=4096, B=1, max_blocks=edge, num_blocks=edge, q_seq=_base), None, 2048) > 0
    past = good_idx(T=4096, B=1, max_blocks=edge + 1, num_blocks=edge + 1, q_seq=_base)
    assert dsa.workspace_bytes(past, None, 2048) == 0
    assert call_idx(past) == E_SHAPE
    # 65,536 queries of a 1M-token sequence: about 1.08e9 pages, rejected
    big = good_idx(T=65536, B=1, max_blocks=16384, num_blocks=16384, q_seq=_base)
    assert call_idx(big) == E_SHAPE


def call_quant(q=_base, rows=64, D=128, dt=None, codes=_base, scales=_base):
    dt = dsa.IDX_FP8_E4M3FN if dt is None else dt
    return dsa.LIB.dsa_quantize_index_q(q, rows, D, dt, codes, scales, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dt=dsa.IDX_BF16), E_DTYPE), (dict(dt=9), E_DTYPE),
    (dict(D=96), E_SHAPE), (dict(D=16), E_SHAPE), (dict(D=1024), E_SHAPE), (dict(rows=-1), E_SHAPE),
    (dict(rows=1 << 40), E_SHAPE),
    (dict(q=None), E_NULL), (dict(codes=None), E_NULL), (dict(scales=None), E_NULL),
    (dict(q=_base + 8), E_ALIGN), (dict(codes=_base + 8), E_ALIGN), (dict(scales=_base + 2), E_ALIGN),
    (dict(rows=0, q=None, codes=None, scales=None), OK),   # nothing to do, nothing enqueued
])
def test_quantize_argument_errors(kw, expect):
    assert call_quant(**kw) == expect


def test_quantize_mxfp8_scale_bytes_need_no_alignment():
    # the E8M0 bytes are written one per group: any address; rows=0 stops before a launch
    assert call_quant(dt=dsa.IDX_MXFP8_E4M3, scales=_base + 1, rows=0) == OK
    assert call_quant(dt=dsa.IDX_MXFP8_E4M3, scales=_base + 1, q=_base + 4) == E_ALIGN


def test_check_tables_on_host_copies():
    import torch
    from sparse_attention_07_amd import synth
    case = synth.build_case(synth.CaseSpec("tables", H_idx=16, D_idx=128, idx_dtype="fp8", K=64, H=16,
                                           lens=[300, 64, 1], queries_per_seq=[2, 1, 1], seed=3))
    kw = dict(q_idx_scale=case.q_idx_scale, q_seq=case.q_seq, q_visible=case.q_visible,
              max_q_per_seq=case.max_q_per_seq)
    args = (case.q_idx, case.w, case.k_idx_pool, case.block_table, case.seq_lens)
    assert dsa.check_tables(*args, **kw) is None
    nb, mb = case.num_blocks, case.block_table.shape[1]

    def planted(name, index, value):
        t = {"seq_lens": case.seq_lens, "block_table": case.block_table, "q_seq": case.q_seq,
             "q_visible": case.q_visible}[name].clone()
        t.view(-1)[index] = value
        a = list(args)
        k = dict(kw)
        if name in ("seq_lens", "block_table"):
            a[4 if name == "seq_lens" else 3] = t
        else:
            k[name] = t
        return dsa.check_tables(*a, **k)
    assert planted("block_table", 0 * mb + 4, nb) == ("block_table", 4)    # page 4 of sequence 0 (position 256+)
    assert planted("block_table", 1 * mb + 0, -1) == ("block_table", mb)
    assert planted("block_table", 1 * mb + 1, -1) is None                  # past sequence 1's only page
    assert planted("seq_lens", 2, 64 * mb + 1) == ("seq_lens", 2)
    assert planted("q_seq", 3, 3) == ("q_seq", 3)
    assert planted("q_visible", 0, 301) == ("q_visible", 0)
    assert planted("q_visible", 2, -1) == ("q_visible", 2)
    # host copies missing where the call has device tables
    a = dsa.indexer_args(*args, **kw)
    st = dsa.LIB.dsa_check_tables(ctypes.byref(a), None, None, None, None, None, None)
    assert st == E_NULL
