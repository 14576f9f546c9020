"""dsa_layer_static (the layer with the library's own per-GPU scratch array,
for callers that cannot allocate) against dsa_layer with a caller workspace,
on the same inputs: two calls in a row, the second with a smaller input, then
the first again with the indices left in the scratch.  Same kernels, so the
index rows must be identical and the outputs within the attention tolerance
(they are in fact identical)."""
import pytest
import torch

from dsa_check import check_outputs
from gpu_cases import say
from sparse_attention_07_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_attention_07_amd import dsa
DEV = "cuda"


def spec(name, **kw):
    base = dict(H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128)
    base.update(kw)
    return synth.CaseSpec(name, **base)


def compare(layer, want_indices=True):
    layer()
    ref_out, ref_idx = layer.out.clone(), layer.indices.clone()
    out = torch.full_like(layer.out, float("nan"))
    idx = torch.full_like(layer.indices, -7) if want_indices else None
    layer.call_static(out=out, indices=idx)
    torch.cuda.synchronize()
    if want_indices:
        assert torch.equal(idx, ref_idx), "index rows differ"
    ok, msg = check_outputs(out.float().cpu().numpy(), ref_out.float().cpu().numpy())
    say(f"  static scratch vs workspace: {msg}; bitwise equal: "
        f"{torch.equal(out.view(torch.int16), ref_out.view(torch.int16))}")
    assert ok, msg


def test_static_scratch_layer_two_calls_then_smaller():
    # a 16-sequence decode batch up to 128K tokens (candidate lists, two merge
    # levels, 4 attention splits), then a smaller one, then the first again
    # with its indices kept in the scratch
    big = synth.build_case(spec("static_big", len_range=(65536, 131072), B=16, seed=71), device=DEV)
    small = synth.build_case(spec("static_small", lens=[5000, 300, 64], H=32, K=512, seed=72), device=DEV)
    lb, ls = dsa.layer_from_case(big), dsa.layer_from_case(small)
    say("[case] big")
    compare(lb)
    say("[case] smaller")
    compare(ls)
    say("[case] big, indices in the scratch")
    compare(lb, want_indices=False)


def test_static_scratch_rejects_oversized_calls():
    # 8192 queries x K=2048 of indices alone need 64 MiB: rejected before
    # anything is launched
    a = dsa.IndexerArgs()
    t = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    p = t.data_ptr()
    a.T, a.B, a.H_idx, a.D_idx, a.idx_dtype = 8192, 1, 64, 128, dsa.IDX_FP8_E4M3FN
    a.q_idx = a.q_idx_scale = a.w = a.k_idx_pool = a.block_table = a.seq_lens = a.q_seq = p
    a.num_blocks, a.max_blocks, a.max_q_per_seq = 128, 128, 8192
    m = dsa.MlaArgs()
    m.T, m.H, m.q, m.kv_pool, m.num_blocks = 8192, 128, p, p, 128
    assert dsa.workspace_bytes(a, m, 2048) > dsa.STATIC_SCRATCH_BYTES
    import ctypes
    st = dsa.LIB.dsa_layer_static(ctypes.byref(a), ctypes.byref(m), 2048, 0.04, None, p, None)
    assert st == 9, dsa.status_str(st)
