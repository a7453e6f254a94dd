"""Test helpers: error measures and device transfer (no operator arithmetic)."""
import numpy as np
import torch


def rel_err(x, ref):
    """max |x - ref| / max |ref| over the whole tensor (max-norm relative error).

    Elementwise relative error is undefined where the reference is near zero,
    so the error is normalised by the tensor's largest reference magnitude."""
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values in the GPU result"
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def to_dev(inp, device="cuda"):
    """Move the generator's CPU tensors to the GPU (q/k/v keep their dtype)."""
    out = {}
    for key in ("q", "k", "v", "log_alpha", "b", "w", "S0", "dO", "dS_final"):
        t = inp.get(key)
        out[key] = None if t is None else t.to(device).contiguous()
    return out


def oracle_args(inp):
    return [inp["q32"], inp["k32"], inp["v32"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"]]


def device_cus():
    """Compute units of cuda:0 (the library sizes its launches from the same count)."""
    return torch.cuda.get_device_properties(0).multi_processor_count


def flags_bytes(items):
    """Bytes of the per-chunk strong-decay flags after a record buffer (rounded up to 256)."""
    return (items * 4 + 255) // 256 * 256


def sweeps_fuse(B, H, dk, dv, bf16=True):
    """Whether the library runs the two sweeps of a training step as one launch on this device:
    bf16 q/k/v, dk 64 or 128, dv a multiple of 64, and both sweeps' 64-column tiles at most one
    workgroup per CU."""
    return bf16 and dk in (64, 128) and dv % 64 == 0 and 2 * B * H * (dv // 64) <= device_cus()
