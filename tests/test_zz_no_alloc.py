"""seer_sparse_decode_noalloc: the sparse decode with its split partials in the
library's static device scratch instead of a caller workspace.  Its results
must equal seer_sparse_decode's bit for bit (same kernels), on two calls in a
row with the second on a smaller input (the scratch keeps the first call's
contents), and match the fp64 oracle like every decode."""
import pytest
import torch

from block_sparse_attention_28_amd import seer
from block_sparse_attention_28_amd.workloads import DECODE_L64K_S90, DecodeWorkload

from gpu_util import build_and_run, check_sequence, oracle_sequence, sample_sequences, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    seer.load()


SMALL = DecodeWorkload(name="noalloc_small", B=3, Hq=16, Hkv=4, d=128, bs=64, budget=512, seed=61,
                       L_range=(700, 5000))


def both_forms(run, out_dtype):
    """(out, lse) of seer_sparse_decode (plan workspace) and of the allocation-free call, same inputs."""
    p, c = run.plan, run.cache
    p.decode(run.q, c["k"], c["v"], c["seqlens"])
    torch.cuda.synchronize()
    ref = (p.out.clone(), p.lse.clone())
    out = torch.full_like(p.out, float("nan"))
    lse = torch.full_like(p.lse, float("nan"))
    seer.seer_sparse_decode_noalloc(run.q, c["k"], c["v"], c["seqlens"], p.block_idx, p.n_sel, run.w.bs,
                                    p.softmax_scale, out, lse, num_splits=p.num_splits)
    torch.cuda.synchronize()
    return ref, (out, lse)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_workspace_call_twice_second_smaller(out_dtype):
    for w in (DECODE_L64K_S90, SMALL):
        run = build_and_run(w, out_dtype=out_dtype)
        say(f"  noalloc {w.name} splits={run.plan.num_splits} out={out_dtype}")
        assert seer.seer_sparse_decode_workspace_size(w.B, w.Hq, w.Hkv, w.d, w.k_max, w.bs,
                                                      run.plan.num_splits) <= 8 << 20
        (ro, rl), (o, l) = both_forms(run, out_dtype)
        assert torch.equal(ro, o) and torch.equal(rl, l), w.name
        # and the oracle's bar on sampled sequences, with the allocation-free output in place
        run.plan.out.copy_(o)
        run.plan.lse.copy_(l)
        for b in sample_sequences(w.B, seed=w.seed):
            check_sequence(run, b, oracle_sequence(run, b))


def test_noalloc_rejects_partials_beyond_the_scratch():
    w = DecodeWorkload(name="noalloc_big", B=64, Hq=64, Hkv=8, d=128, bs=64, budget=4096, seed=62, L=1024)
    need = seer.seer_sparse_decode_workspace_size(w.B, w.Hq, w.Hkv, w.d, w.k_max, w.bs, 16)
    assert need > 8 << 20
    q = torch.zeros((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((w.B, w.Hkv, 1024, w.d), dtype=torch.bfloat16, device="cuda")
    sl = torch.full((w.B,), 1024, dtype=torch.int32, device="cuda")
    idx = torch.zeros((w.B, w.Hkv, w.k_max), dtype=torch.int32, device="cuda")
    ns = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(seer.SeerError) as e:
        seer.seer_sparse_decode_noalloc(q, kv, kv, sl, idx, ns, w.bs, 0.088, out, num_splits=16)
    assert e.value.status == -3
