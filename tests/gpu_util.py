"""Host <-> device helpers for the GPU tests (no arithmetic of the method)."""
import numpy as np
import torch

DEV = "cuda:0"
TORCH_DT = {"int32": torch.int32, "f32": torch.float32, "bf16": torch.bfloat16}
NP_DT = {"int32": np.int32, "f32": np.float32, "bf16": np.uint16}
ESIZE = {"int32": 4, "f32": 4, "bf16": 2}


def np_to_torch(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def torch_to_np(t, dtype):
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def alloc_ranks(N, L, dtype, pad=0, offset=0, fill=None):
    """[N, L] rank-strided view with row stride L+pad elements, starting
    `offset` elements into a fresh allocation."""
    S = L + pad
    buf = torch.empty(N * S + offset + 8, dtype=TORCH_DT[dtype], device=DEV)
    if fill is not None:
        buf.fill_(fill)
    else:
        buf.view(torch.uint8).fill_(0xA5)      # poison: unwritten outputs show up
    return buf[offset:offset + N * S].view(N, S)[:, :L]


def upload(xs, dtype, pad=0, offset=0):
    N, L = len(xs), len(xs[0])
    t = alloc_ranks(N, L, dtype, pad, offset)
    host = np_to_torch(np.stack([np.asarray(x, dtype=NP_DT[dtype]) for x in xs]), dtype)
    t.copy_(host.to(DEV))
    return t


def download(t, dtype):
    out = torch_to_np(t, dtype)
    return [out[r] for r in range(out.shape[0])]


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint8) if a.dtype != np.uint8 else a
