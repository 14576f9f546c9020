"""GPU parity of the residual + RMSNorm epilogue of the sparse attention (through
the C ABI) against the oracle: the oracle's attention over the GPU's own index
sets, then its residual + RMSNorm over each token's H x 512 values.  Covers the
split path (combine + norm kernels), the single-split path (norm inside the
attention kernel), a query with nothing visible, and an in-place residual."""
import numpy as np
import pytest
import torch

from gpu_cases import bits16, query_case, say
from oracle import dsa_oracle as O
from sparse_attention_07_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_attention_07_amd import dsa
DEV = "cuda"
EPS = 1e-6


def epilogue_inputs(T, H, seed):
    g = torch.Generator().manual_seed(seed)
    res = (torch.randn(T, H, 512, generator=g) * 2.0).to(torch.bfloat16)
    gamma = (1.0 + 0.3 * torch.randn(H * 512, generator=g)).to(torch.bfloat16)
    return res, gamma


def check_stored(got, ref):
    """The attention tolerance (max 2e-2, relative L2 1e-2) plus the bf16 storage
    of values of any size: half a bf16 ulp is at most 2^-8 of the value."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    worst = float(np.max(d - 2.0 ** -8 * np.abs(ref))) if d.size else 0.0
    ok = bool(np.all(d <= 2e-2 + 2.0 ** -8 * np.abs(ref))) and rel <= 1e-2
    return ok, f"max|d|={float(d.max()) if d.size else 0.0:.3g} (excess over 2^-8|ref| {worst:.3g}) relL2={rel:.3g}"


def check_epilogue(case, indices, res_out, out, res, gamma, queries):
    """Oracle attention over the GPU's index sets for the listed queries, then the
    oracle's residual + RMSNorm; compares residual_out and out."""
    idx = indices.cpu().numpy()
    attn = []
    for t in queries:
        d, phys = query_case(case, t)
        pos_of = {int(s): p for p, s in enumerate(phys)}
        gpos = [pos_of[int(s)] for s in idx[t] if s >= 0]
        attn.append(O.mla_query(d, 0, np.array(gpos, dtype=np.int64)))
    qs = list(queries)
    r = O.bf16_to_f64(bits16(res[qs]))
    y_ref, n_ref = O.residual_rmsnorm(np.stack(attn), r, O.bf16_to_f64(bits16(gamma)), EPS)
    ok, msg = check_stored(res_out[qs].float().cpu().numpy(), y_ref)
    say(f"  residual_out vs oracle: {msg}")
    assert ok, msg
    ok, msg = check_stored(out[qs].float().cpu().numpy(), n_ref)
    say(f"  normed out vs oracle: {msg}")
    assert ok, msg


def run_epilogue(spec, queries=None, prefill_chunk=None, in_place=False):
    say(f"[epilogue] {spec.name} chunk={prefill_chunk} in_place={in_place}")
    case = synth.build_case(spec, device=DEV, prefill_chunk=prefill_chunk)
    res, gamma = epilogue_inputs(case.T, spec.H, spec.seed + 100)
    res_d, gamma_d = res.to(DEV), gamma.to(DEV)
    res_out = res_d if in_place else torch.empty_like(res_d)
    layer = dsa.layer_from_case(case, residual=res_d, norm_weight=gamma_d, residual_out=res_out, eps=EPS)
    layer()
    torch.cuda.synchronize()
    qs = range(case.T) if queries is None else queries
    check_epilogue(case, layer.indices, res_out, layer.out, res, gamma, qs)
    return case, layer


def test_epilogue_split_decode_with_empty_query():
    # 8 splits per query (combine + norm kernels); the zero-length sequence attends over nothing
    sp = synth.CaseSpec("ep_split", H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128,
                        lens=[40000, 0, 3, 9000], seed=51)
    run_epilogue(sp)


def test_epilogue_single_split_prefill():
    # one split per query: the norm runs inside the attention kernel
    sp = synth.CaseSpec("ep_prefill", H_idx=64, D_idx=128, idx_dtype="fp8", K=512, H=128, prefill=(2048, 512),
                        seed=53)
    run_epilogue(sp, prefill_chunk=3, queries=[0, 1, 255, 511])


@pytest.mark.parametrize("H", [16, 64])
def test_epilogue_fewer_heads_fp8_latent(H):
    sp = synth.CaseSpec(f"ep_h{H}", H_idx=16, D_idx=128, idx_dtype="fp8", K=1024, H=H, lens=[5000, 700, 64],
                        seed=55 + H, kv_dtype="fp8")
    run_epilogue(sp)


def test_epilogue_in_place_residual():
    sp = synth.CaseSpec("ep_inplace", H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128, lens=[30000, 5000],
                        seed=57)
    run_epilogue(sp, in_place=True)


def test_epilogue_leaves_plain_attention_unchanged():
    # the same layer without the epilogue must still give the plain attention output, bit for bit across runs
    sp = synth.CaseSpec("ep_plain", H_idx=64, D_idx=128, idx_dtype="fp8", K=2048, H=128, lens=[20000, 7000],
                        seed=59)
    case = synth.build_case(sp, device=DEV)
    plain = dsa.layer_from_case(case)
    plain()
    o1 = plain.out.clone()
    res, gamma = epilogue_inputs(case.T, sp.H, 1)
    ep = dsa.layer_from_case(case, residual=res.to(DEV), norm_weight=gamma.to(DEV),
                             residual_out=torch.empty_like(res, device=DEV), eps=EPS)
    ep()
    plain()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), plain.out.view(torch.int16))
    assert torch.equal(plain.indices, ep.indices)
