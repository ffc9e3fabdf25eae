"""Helpers for the GPU parity tests: device transfer and the parity bar.

Parity bar (from the workload statement, with a floor of 1 under the relative LSE error):
  * bf16 paths: max |O_gpu - O_ref| <= 2e-2 and
    max |lse_gpu - lse_ref| / max(|lse_ref|, 1) <= 1e-3;
  * fp32 path: max |O_gpu - O_ref| <= 1e-4 and max |lse_gpu - lse_ref| <= 1e-4;
  * rows with no visible key must be exactly o = 0 and lse = -inf on both sides.
O_ref is the fp64 oracle result, unrounded.
"""
import sys

import numpy as np

BF16_O_TOL = 2e-2
BF16_LSE_REL_TOL = 1e-3
F32_TOL = 1e-4


def say(*a):
    """Print and flush, so a GPU failure log names the case that was running."""
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_device(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def f32_to_device(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def compare(o_gpu, lse_gpu, o_ref, lse_ref, o_tol, lse_tol, lse_relative=True, label=""):
    """Assert the parity bar; returns (max |dO|, max lse error) for logging."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    lse_gpu = np.asarray(lse_gpu, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite output"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), f"{label}: empty-row pattern differs"
    if empty.any():
        assert np.all(o_gpu[empty] == 0.0), f"{label}: empty rows must be 0"
    do = float(np.max(np.abs(o_gpu - o_ref))) if o_gpu.size else 0.0
    fin = ~empty
    if fin.any():
        err = np.abs(lse_gpu[fin] - lse_ref[fin])
        if lse_relative:
            err = err / np.maximum(np.abs(lse_ref[fin]), 1.0)
        dl = float(np.max(err))
    else:
        dl = 0.0
    say(f"  {label}: max|dO| = {do:.3e} (tol {o_tol}), lse err = {dl:.3e} (tol {lse_tol})")
    assert do <= o_tol, f"{label}: max|dO| {do} > {o_tol}"
    assert dl <= lse_tol, f"{label}: lse error {dl} > {lse_tol}"
    return do, dl


def fwd_capped(q, k, v, causal, scale, max_workgroups, window=None, lib=None):
    """The bf16 prefill with a cap on its persistent grid, through the library's
    test hook fa_testing_fwd_capped (a per-call cap; results do not depend on
    it), on libfa.so or the library handle `lib`.  Returns (o, lse)."""
    import ctypes
    import torch
    from transformer_attention_fa_amd import api
    lib = lib or api.load()
    fn = lib.fa_testing_fwd_capped
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, vp]
    fn.restype = i
    B, H, N_q, d = q.shape
    _, H_kv, N_k, _ = k.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv, N_q, N_k, d,
            float(scale), int(bool(causal)), int(window or 0), int(max_workgroups), None,
            torch.cuda.current_stream(q.device).cuda_stream)
    assert st == api.FA_OK, (st, lib.fa_last_error().decode())
    return o, lse
