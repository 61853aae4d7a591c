"""Parity at the full sizes of the five workloads, in the launch configuration the
benchmark times (the workloads' own partition settings), on every output row.

Each workload runs on the GPU whole; the oracle then recomputes every decode sequence
and every query row of every prefill request, one sequence at a time from a compact
pool of its own pages (worker processes share the sequences; they never touch the
GPU), and compares them element by element at the same tolerances as the small parity
tests.  At full size the balanced decode schedule cuts and merges segments in a pattern
of its own, so no row is left out."""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_common import assert_close, assert_lse_close
from tests.oracle_state import oracle_sequence

pytestmark = pytest.mark.gpu

# (workload, overrides): the six workloads, the Llama batch and the mixed batch with an
# MXFP4 cache, and the mixed batch with an FP8 cache (the benchmark's other lines)
CASES = [(c, {}) for c in (1, 2, 3, 4, 5, 6)] + [(2, {"kv_dtype": "mxfp4"}), (3, {"kv_dtype": "mxfp4"}),
                                                 (3, {"kv_dtype": "fp8"})]


def _oracle_rows(cfg, over, scales, seqs):
    """Oracle outputs of sequences `seqs` (run in a worker process, with one BLAS thread:
    the workers already share the cores)."""
    from threadpoolctl import threadpool_limits
    wl = workloads.make(cfg, **over)
    if scales is not None:
        wl._scales = scales          # the batch-wide FP8 calibration, computed once by the parent
    out = {}
    with threadpool_limits(1):
        for s in seqs:
            out[s] = oracle_sequence(wl, s)
            wl.drop_cache()
    return out


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@pytest.mark.parametrize("cfg,over", CASES, ids=lambda x: str(x) if isinstance(x, int) else (x.get("kv_dtype") or "-"))
def test_full_size_every_row(gpu_lib, cfg, over):
    wl = workloads.make(cfg, **over)
    print(f"[case] full-size {wl.name} S={wl.num_seqs} tokens={int(wl.context_lens.sum())}", flush=True)
    scales = wl.fp8_scales() if wl.kv_dtype == "fp8" else None
    # the longest sequences first, spread over the workers in round-robin batches
    order = [int(s) for s in np.argsort(-wl.context_lens.astype(np.int64), kind="stable")]
    nw = _workers()
    batches = [order[i::nw * 4] for i in range(nw * 4) if order[i::nw * 4]]
    with ProcessPoolExecutor(nw, mp_context=mp.get_context("spawn")) as ex:
        futs = [ex.submit(_oracle_rows, cfg, over, scales, b) for b in batches]
        from tests.device_batch import DeviceBatch
        wl.prefetch()
        db = DeviceBatch(wl)
        db.fill_history()
        db.step()
        torch.cuda.synchronize()
        dec, dec_lse, pf, pf_lse = db.outputs_f64()
        del db
        wl.drop_cache()
        torch.cuda.empty_cache()
        ref = {}
        for f in futs:
            ref.update(f.result())
    npf = wl.num_prefill
    cu = wl.cu(wl.new_lens)
    err = {"decode": 0.0, "prefill": 0.0, "lse": 0.0}
    for s in range(wl.num_seqs):
        ref_o, ref_l = ref[s]
        if s < npf:
            got_o, got_l, kind = pf[cu[s]:cu[s + 1]], pf_lse[cu[s]:cu[s + 1]], "prefill"
        else:
            got_o, got_l, kind = dec[s - npf:s - npf + 1], dec_lse[s - npf:s - npf + 1], "decode"
        err[kind] = max(err[kind], assert_close(got_o, ref_o, wl.kv_dtype, f"{wl.name} {kind} seq {s}"))
        err["lse"] = max(err["lse"], assert_lse_close(got_l, ref_l, wl.kv_dtype, f"{wl.name} {kind} seq {s}"))
    print(f"[ok] {wl.name}: all {wl.num_seqs - npf} decode sequences and {int(cu[npf])} prefill rows of "
          f"{npf} requests; largest errors ({'abs' if wl.kv_dtype == 'f32' else 'rel'}) decode "
          f"{err['decode']:.2e}, prefill {err['prefill']:.2e}, lse (abs) {err['lse']:.2e}", flush=True)
