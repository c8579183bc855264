"""Shared helpers for the GPU parity tests (inputs to device, tolerances)."""

import numpy as np
import torch

from long_context_verify_tree_amd import synth


def to_dev(arr: np.ndarray, dtype: str):
    """numpy input (bf16 bits as uint16, or float32) -> device tensor."""
    if dtype == synth.BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to("cuda", non_blocking=False)


def device_inputs(x: synth.VerifyInputs):
    dt = x.cfg.dtype
    return dict(q=to_dev(x.q, dt), k_cache=to_dev(x.k_cache, dt), v_cache=to_dev(x.v_cache, dt),
                k_draft=to_dev(x.k_draft, dt), v_draft=to_dev(x.v_draft, dt),
                parent=torch.from_numpy(x.parent).to("cuda"))


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_rows(got, ref, got_lse, ref_lse, dtype, what=""):
    """Tolerances.  fp32: per row max|g-o| <= 1e-5 max|o|, lse within 1e-5 of
    max(|lse|, 1): its rounding comes from the fp32 scores (products summed
    over D, of magnitude ~ sqrt(D) scale for unit inputs), not from how close
    the lse itself lands to 0.  bf16 (fp32 accumulation): |g-o| <= 2e-2
    absolute, plus a normwise check per (b, h) slab (max|g-o| <= 2e-2 max|o|)
    and |lse_g - lse_o| <= 1e-3."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == synth.FP32:
        row_scale = np.abs(ref).max(axis=-1)
        bad = err.max(axis=-1) > 1e-5 * row_scale
        assert not bad.any(), f"{what}: fp32 rel err {float((err.max(-1) / row_scale).max()):.3e}"
        lerr = np.abs(got_lse - ref_lse)
        assert (lerr <= 1e-5 * np.maximum(np.abs(ref_lse), 1.0)).all(), f"{what}: lse err {lerr.max():.3e}"
    else:
        assert err.max() <= 2e-2, f"{what}: abs err {err.max():.3e}"
        slab = ref.reshape(-1, ref.shape[-2] * ref.shape[-1]) if ref.ndim >= 2 else ref[None]
        eslab = err.reshape(slab.shape)
        rel = eslab.max(axis=1) / np.maximum(np.abs(slab).max(axis=1), 1e-30)
        assert rel.max() <= 2e-2, f"{what}: normwise err {rel.max():.3e}"
        if got_lse is not None:
            lerr = np.abs(np.asarray(got_lse) - np.asarray(ref_lse))
            assert lerr.max() <= 1e-3, f"{what}: lse err {lerr.max():.3e}"
    return float(err.max())
