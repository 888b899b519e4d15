"""Host<->device glue for the GPU tests (no layer arithmetic here)."""
import numpy as np

from megatron_tensor_layer_amd import datagen


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray, dtype: str):
    """numpy float32 (bf16-representable when dtype == 'bf16') -> cuda tensor."""
    t = torch()
    if dtype == "bf16":
        bits = datagen.bf16_bits(a).view(np.int16)
        return t.from_numpy(bits).view(t.bfloat16).cuda()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host(x) -> np.ndarray:
    """cuda tensor (bf16 or fp32) -> numpy float64 (exact)."""
    t = torch()
    if x.dtype == t.bfloat16:
        u = x.contiguous().view(t.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return x.cpu().numpy().astype(np.float64)


def empty(shape, dtype: str, fill=float("nan")):
    """Device buffer pre-filled with a canary (NaN) so unwritten outputs show."""
    t = torch()
    td = t.bfloat16 if dtype == "bf16" else t.float32
    return t.full(tuple(shape), fill, dtype=td, device="cuda")


def tdtype(dtype: str):
    t = torch()
    return t.bfloat16 if dtype == "bf16" else t.float32
