"""Shared helpers of the GPU parity tests: seeded inputs on the device, comparison
against the fp64 oracle, and an optional log of the observed error margins."""
import json
import os

import numpy as np
import torch

import synth

H, I = synth.HIDDEN, synth.INTERMEDIATE
BF16_TOL = 2e-2      # max |err| <= 2e-2 * RMS(ref), bf16 inputs with fp32 accumulation
FP32_TOL = 1e-5      # max |err| <= 1e-5 * RMS(ref), fp32 inputs

DEV = torch.device("cuda:0")


def f64(t: torch.Tensor) -> np.ndarray:
    return synth.to_f64(t)


def rms(a: np.ndarray) -> float:
    return float(np.sqrt(np.mean(a * a)))


def log_margin(label: str, err_over_rms: float, tol: float):
    path = os.environ.get("SMLP_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": label, "max_err_over_rms": err_over_rms, "tol": tol}) + "\n")


def assert_rms_close(got: torch.Tensor, ref: np.ndarray, tol: float, label: str, ref_rms=None):
    g = f64(got)
    assert g.shape == ref.shape, (label, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    r = rms(ref) if ref_rms is None else ref_rms
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    log_margin(label, err / r if r > 0 else err, tol)
    assert err <= tol * r, f"{label}: max|err| = {err:.3e} > {tol} * RMS {r:.3e} (ratio {err / r:.3e})"
    return err / r if r > 0 else 0.0


def workspace_for(M, H_, I_, dtype_code):
    from moe_shared_expert_amd import binding
    n = binding.shared_mlp_workspace_bytes(M, H_, I_, dtype_code)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)
