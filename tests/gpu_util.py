"""Helpers shared by the GPU parity tests (comparison, device transfer)."""
import numpy as np

# The parity bar for floating-point outputs: max relative error 2e-3, measured per tensor as
# max_i |gpu_i - oracle_i| / max_i |oracle_i| (weights bf16 or fp32, accumulation fp32).
TOL = 2e-3


def rel_err(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / (den if den > 0 else 1.0))


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def dev(a: np.ndarray):
    from autoregressive_decode_step_amd.loader import to_device
    return to_device(a, "cuda")


def say(msg: str) -> None:
    print(msg, flush=True)


_WEIGHTS = {}


def weights(shape, seed: int = 0) -> dict:
    """synth.model(shape, seed), kept for the next caller with the same weight shape (one set at a time: an
    8B-shaped set is 15 GB of host memory). The weights do not depend on max_seq."""
    import synth
    key = (shape.vocab, shape.d, shape.n_layer, shape.n_head, shape.n_kv, shape.head_dim, shape.hidden,
           shape.w_dtype, shape.w_std, seed)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        _WEIGHTS[key] = synth.model(shape, seed=seed)
    return _WEIGHTS[key]
