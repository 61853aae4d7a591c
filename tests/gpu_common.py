"""Shared helpers of the GPU parity tests: tolerances and comparisons against the
oracle (test infrastructure)."""
import numpy as np

# Tolerances: fp32 max-abs 1e-4; bf16 and FP8-KV outputs per (row, head)
# infinity-norm relative error 2e-2 and 5e-2; MXFP4-KV 2e-2 (its values decode to bf16
# exactly on both sides, so only the bf16 weights and the accumulation differ).  The log-sum-exp is compared in
# absolute terms: the kernels accumulate it in fp32 from exact bf16/fp8 inputs.
TOL = {"f32": ("abs", 1e-4), "bf16": ("rel", 2e-2), "fp8": ("rel", 5e-2), "mxfp4": ("rel", 2e-2)}
LSE_ATOL = {"f32": 1e-4, "bf16": 2e-3, "fp8": 2e-3, "mxfp4": 2e-3}


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


def mx_unpack(b):
    """uint8 array [..., n] -> [..., 2n] nibbles, the low nibble of each byte first."""
    b = np.asarray(b, np.uint8)
    return np.stack([b & 15, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))


def mx_pool_logical(bits, P, D):
    """The library's MXFP4 pool (uint8 [N][2][H][tile]) re-indexed into the oracle's
    logical rows [N][2][H][P][D + D/32]: the D E2M1 codes of a token row, one per byte,
    then its D/32 scale bytes.  A pure re-indexing of the stored nibbles and bytes.
      K codes: slot t's D/2 bytes; dims 32j + 8c + e are nibble e of word c*(D/32) + j
      V codes: 32-slot sub-blocks of 16*D bytes; dim 16u + m of the slot at position
               k = 8c + e (VPOS) is nibble e of word (4m + c)*(D/16) + u
      scales:  K [P][D/32]; V [P/32][32 positions][D/32], after the codes."""
    N, _, H, T = bits.shape
    J, C = D // 32, P * D // 2
    assert T == C + P * J
    k = mx_unpack(bits[:, 0, :, :C].reshape(N, H, P, 4, J, 4))       # [.., t, c, j, 8 e]
    k = k.transpose(0, 1, 2, 4, 3, 5).reshape(N, H, P, D)             # d = 32j + 8c + e
    ks = bits[:, 0, :, C:].reshape(N, H, P, J)
    v = mx_unpack(bits[:, 1, :, :C].reshape(N, H, P // 32, 16, 4, D // 16, 4))  # [.., m, c, u, 8 e]
    v = v.transpose(0, 1, 2, 4, 6, 5, 3).reshape(N, H, P // 32, 32, D)  # [.., k = 8c + e, d = 16u + m]
    v = v[:, :, :, VPOS, :].reshape(N, H, P, D)
    vs = bits[:, 1, :, C:].reshape(N, H, P // 32, 32, J)[:, :, :, VPOS, :].reshape(N, H, P, J)
    out = np.empty((N, 2, H, P, D + J), np.uint8)
    out[:, 0, :, :, :D], out[:, 0, :, :, D:] = k, ks
    out[:, 1, :, :, :D], out[:, 1, :, :, D:] = v, vs
    return out
