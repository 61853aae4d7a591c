"""paged_attn_decode_noalloc -- the decode call with its workspace in the library's own
device array, for callers that cannot allocate -- against paged_attn_decode with a
workspace of the caller's: the same outputs bit for bit, and both within the oracle's
tolerance, on two calls in a row where the second batch is smaller than the first
(the array keeps the first call's partial records, which must not leak into the
second's results)."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_common import assert_close, assert_lse_close
from tests.oracle_state import oracle_outputs, oracle_pool

pytestmark = pytest.mark.gpu

# (label, [(workload, overrides) of the first call, of the second, smaller call])
CASES = [
    ("balanced_bf16", [(2, dict(num_seqs=40, len_range=(1, 3000))), (2, dict(num_seqs=6, len_range=(1, 400)))]),
    ("fixed_splits", [(4, dict(num_seqs=3, context_len=5000, num_splits=9)),
                      (4, dict(num_seqs=1, context_len=900, num_splits=3))]),
    ("fp8_shared_prefix", [(5, dict(num_seqs=12, group_size=4, prefix_len=128, len_range=(129, 2000))),
                           (5, dict(num_seqs=4, group_size=2, prefix_len=64, len_range=(65, 300)))]),
    ("mxfp4", [(2, dict(num_seqs=20, len_range=(1, 2000), kv_dtype="mxfp4")),
               (2, dict(num_seqs=3, len_range=(1, 300), kv_dtype="mxfp4"))]),
]


def _one(B, cfg, over):
    from tests.device_batch import DeviceBatch
    wl = workloads.make(cfg, **over)
    print(f"[case] noalloc {wl.name} S={wl.num_seqs} Lmax={wl.max_context_len} splits={wl.num_splits}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.prepare_step()
    db.append_step()
    need = B.paged_attn_decode_workspace_size(db.cache, db.seqs_dec, db.q_code, wl.num_q_heads, db.num_splits)
    assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
    db.decode_step()                       # the existing entry point, caller's workspace
    out = torch.full_like(db.out_dec, float("nan"))
    lse = torch.full_like(db.lse_dec, float("nan"))
    B.paged_attn_decode_noalloc(db.cache, db.seqs_dec, db.q_dec, db.q_code, wl.num_q_heads, float(wl.sm_scale),
                                db.num_splits, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), db.out_dec.view(torch.int16)), "output differs from paged_attn_decode"
    assert torch.equal(lse.view(torch.int32), db.lse_dec.view(torch.int32)), "lse differs from paged_attn_decode"
    ref = oracle_outputs(wl, oracle_pool(wl))
    got = out.float().cpu().numpy().astype(np.float64)
    assert_close(got, ref[0], wl.kv_dtype, f"noalloc {wl.name}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref[1], wl.kv_dtype, f"noalloc {wl.name}")


@pytest.mark.parametrize("label,calls", CASES, ids=[c[0] for c in CASES])
def test_noalloc_decode_equals_decode_on_two_calls(gpu_lib, label, calls):
    for cfg, over in calls:
        _one(gpu_lib, cfg, over)


def test_noalloc_rejects_a_plan_larger_than_its_array(gpu_lib):
    """64 sequences in 64 fixed partitions of 32 query heads need about 68 MB of partial
    records: refused before anything is launched."""
    B = gpu_lib
    S, Hq, Hkv, D, P = 64, 32, 8, 128, 64
    pool = torch.zeros((4, 2, Hkv, P, D), dtype=torch.bfloat16, device="cuda")
    cache = B.make_cache(pool, P, Hkv, D, B.PKV_BF16)
    bt = torch.zeros((S, 128), dtype=torch.int32, device="cuda")
    lens = torch.full((S,), 8192, dtype=torch.int32, device="cuda")
    seqs = B.make_seqs(bt, lens, 8192)
    assert B.paged_attn_decode_workspace_size(cache, seqs, B.PKV_BF16, Hq, 64) > B.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(B.PagedKVError) as e:
        B.paged_attn_decode_noalloc(cache, seqs, q, B.PKV_BF16, Hq, 0.125, 64, out)
    assert e.value.code == B.PKV_EWORKSPACE and "scratch" in str(e.value)
