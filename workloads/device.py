"""Raw-bit copies between host numpy arrays and device tensors.

Pure data movement: the bits a workload generator produced are copied to
the GPU unchanged (fp16/bf16 as int16, e4m3 as uint8, fp32 as int32), and
back.  No arithmetic of the method lives here.
"""
import numpy as np

_TORCH_NAME = {np.dtype(np.uint8): "uint8", np.dtype(np.uint16): "int16",
               np.dtype(np.uint32): "int32", np.dtype(np.uint64): "int64"}
_NP_SIGNED = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32,
              np.dtype(np.uint64): np.int64, np.dtype(np.uint8): np.uint8}


def to_dev(a: np.ndarray, pad_front: int = 0):
    """Copy raw bits to the GPU; pad_front extra elements in front shift the
    data off the allocation's alignment (the returned view starts there)."""
    import torch

    a = np.ascontiguousarray(a)
    flat = a.reshape(-1).view(_NP_SIGNED[a.dtype])
    t = torch.empty(flat.size + pad_front, dtype=getattr(torch, _TORCH_NAME[a.dtype]),
                    device="cuda")
    if pad_front:
        t[:pad_front] = 0
    t[pad_front:].copy_(torch.from_numpy(flat.copy()))
    return t[pad_front:]


def to_host(t, like: np.dtype) -> np.ndarray:
    """The device tensor's bits as a host array of dtype ``like``."""
    return t.cpu().numpy().view(like)
