"""Shared helpers of the GPU parity tests: tolerances and comparisons against the
oracle (test infrastructure)."""
import numpy as np

# Tolerances: fp32 max-abs 1e-4; bf16 and FP8-KV outputs per (row, head)
# infinity-norm relative error 2e-2 and 5e-2.  The log-sum-exp is compared in
# absolute terms: the kernels accumulate it in fp32 from exact bf16/fp8 inputs.
TOL = {"f32": ("abs", 1e-4), "bf16": ("rel", 2e-2), "fp8": ("rel", 5e-2)}
LSE_ATOL = {"f32": 1e-4, "bf16": 2e-3, "fp8": 2e-3}


def rel_inf(got, ref):
    """max over (row, head) of ||got - ref||_inf / ||ref||_inf."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max()) if num.size else 0.0


def assert_close(got, ref, kv_dtype, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    kind, tol = TOL[kv_dtype]
    err = float(np.abs(got - ref).max()) if kind == "abs" else rel_inf(got, ref)
    assert err <= tol, f"{what}: {kind} error {err:.3e} > {tol:.1e}"
    return err


def assert_lse_close(got, ref, kv_dtype, what=""):
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    assert err <= LSE_ATOL[kv_dtype], f"{what}: lse error {err:.3e}"
    return err


def v_tiles_token_major(v_bits):
    """V tiles [N][H][P/S][D][S] (S = min(P, 32), the library's layout, stored in an
    array shaped [N][H][P][D]) re-indexed token-major [N][H][P][D]."""
    N, H, P, D = v_bits.shape
    S = min(P, 32)
    return v_bits.reshape(N, H, P // S, D, S).swapaxes(-1, -2).reshape(N, H, P, D)


def pool_token_major(bits):
    """The library's pool [page][K|V][kv_head][tile] (K tiles token-major [P][D], V tiles
    dim-major inside 32-slot sub-blocks) rearranged with both tiles token-major, the
    oracle's layout.  A pure re-indexing of the stored elements, for byte-exact
    comparison."""
    out = bits.copy()
    out[:, 1] = v_tiles_token_major(bits[:, 1])
    return out
