"""Small helpers shared by the GPU tests (device transfer, unit slicing)."""
import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 2e-3}


def tdtype(cfg_or_dtype):
    d = getattr(cfg_or_dtype, "dtype", cfg_or_dtype)
    return torch.float32 if d == "f32" else torch.bfloat16


def dev(x, dtype=torch.float32):
    """numpy -> contiguous device tensor (grid values are exact in bf16)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def unit_slices(cfg, unit):
    b, h = divmod(unit, cfg.n_kv_heads)
    G = cfg.group
    return b, h, slice(h * G, (h + 1) * G)


def zeros(shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def banner(msg):
    print(f"[gpu] {msg}", flush=True)
