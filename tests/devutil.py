"""Host <-> device helpers for the GPU tests (torch is only the allocator)."""
from __future__ import annotations

import numpy as np

TORCH_DT = None


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "i32": torch.int32}[dtype]


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to("cuda")


def to_host(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def empty(count: int, dtype: str, fill=None):
    import torch
    t = torch.empty(count, dtype=torch_dtype(dtype), device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def sync():
    import torch
    torch.cuda.synchronize()


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what=""):
    assert got.dtype == want.dtype and got.shape == want.shape, what
    if got.tobytes() != want.tobytes():
        g = got.view(np.uint16 if got.itemsize == 2 else np.uint32)
        w = want.view(np.uint16 if want.itemsize == 2 else np.uint32)
        bad = np.nonzero(g != w)[0]
        raise AssertionError("%s: %d of %d elements differ; first at %d: got %r want %r"
                             % (what, bad.size, got.size, bad[0], got[bad[0]], want[bad[0]]))
