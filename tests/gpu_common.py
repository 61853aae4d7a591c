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


# Position of slot r inside a 32-slot V sub-block of the library's pool (slots 4c..4c+3
# at 8c..8c+3, slots 16+4c..16+4c+3 at 8c+4..8c+7).
VPOS = np.array([8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3) for r in range(32)])


def k_tiles_token_major(k_bits):
    """K tiles [N][H][D/32][P][32] (the library's layout, in an array shaped
    [N][H][P][D]) re-indexed token-major [N][H][P][D]."""
    N, H, P, D = k_bits.shape
    return k_bits.reshape(N, H, D // 32, P, 32).transpose(0, 1, 3, 2, 4).reshape(N, H, P, D)


def v_tiles_token_major(v_bits):
    """V tiles [N][H][P/S][D][S] (S = min(P, 32), slots of a 32-slot sub-block at
    positions VPOS) re-indexed token-major [N][H][P][D]."""
    N, H, P, D = v_bits.shape
    S = min(P, 32)
    x = v_bits.reshape(N, H, P // S, D, S)
    if S == 32:
        x = x[..., VPOS]
    return x.swapaxes(-1, -2).reshape(N, H, P, D)


def pool_token_major(bits):
    """The library's pool [page][K|V][kv_head][tile] rearranged with both tiles
    token-major [P][D], the oracle's layout.  A pure re-indexing of the stored
    elements, for byte-exact comparison."""
    out = bits.copy()
    out[:, 0] = k_tiles_token_major(bits[:, 0])
    out[:, 1] = v_tiles_token_major(bits[:, 1])
    return out


def pool_from_token_major(tm):
    """Inverse of pool_token_major."""
    N, _, H, P, D = tm.shape
    out = tm.copy()
    out[:, 0] = tm[:, 0].reshape(N, H, P, D // 32, 32).transpose(0, 1, 3, 2, 4).reshape(N, H, P, D)
    S = min(P, 32)
    x = tm[:, 1].reshape(N, H, P // S, S, D).swapaxes(-1, -2)
    if S == 32:
        y = np.empty_like(x)
        y[..., VPOS] = x
        x = y
    out[:, 1] = x.reshape(N, H, P, D)
    return out
