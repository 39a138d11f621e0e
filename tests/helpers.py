"""Shared helpers for the GPU parity tests (device transfer, error metrics)."""
import math
import sys

import numpy as np
import torch

from long_sequence_bidirectional_amd import inputs

# Tolerances.  The bf16 gates (max-abs 2e-2, mean-abs 2e-3 on O) and the f32
# gate (1e-5 max-abs on O and LSE) are the required ones; rel-L2 of O and the
# LSE bound for bf16 are self-imposed diagnostics that are much tighter than
# the mean-abs gate at long sequence lengths, where |O| ~ sqrt(e / Skv).
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL_L2 = 1e-2
BF16_LSE_MAX_ABS = 1e-3
F32_MAX_ABS = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor (bit-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def f64_of_bf16(bits: np.ndarray) -> np.ndarray:
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(o_gpu: np.ndarray, o_ref: np.ndarray):
    d = np.abs(o_gpu - o_ref)
    rel = float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    return float(d.max()), float(d.mean()), rel


def assert_bf16_parity(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    mx, mean, rel = errors(o_gpu, o_ref)
    lse_err = float(np.max(np.abs(lse_gpu - lse_ref)))
    log(f"  {what}: O max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}; LSE max-abs {lse_err:.3e}")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))
    assert mx <= BF16_MAX_ABS, f"{what}: O max-abs {mx}"
    assert mean <= BF16_MEAN_ABS, f"{what}: O mean-abs {mean}"
    assert rel <= BF16_REL_L2, f"{what}: O rel-L2 {rel}"
    assert lse_err <= BF16_LSE_MAX_ABS, f"{what}: LSE max-abs {lse_err}"


def assert_f32_parity(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    mx = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    lse_err = float(np.max(np.abs(lse_gpu - lse_ref))) if lse_ref.size else 0.0
    log(f"  {what}: O max-abs {mx:.3e}; LSE max-abs {lse_err:.3e}")
    assert mx <= F32_MAX_ABS, f"{what}: O max-abs {mx}"
    assert lse_err <= F32_MAX_ABS, f"{what}: LSE max-abs {lse_err}"


def scale_of(D):
    return 1.0 / math.sqrt(D)
