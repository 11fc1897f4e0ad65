"""Device-memory plumbing for the C ABI: torch CUDA tensors as buffers, numpy in and out.

Nothing here computes the method; it allocates, copies and calls ``frt``.
"""
import numpy as np
import torch

from . import frt

DEV = "cuda"


def to_dev(a):
    """numpy array -> contiguous CUDA tensor with the same bytes and dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV)


def to_np(t):
    return t.detach().cpu().numpy()


def empty_bytes(nbytes):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=DEV)


def empty_f32(*shape):
    return torch.empty(shape, dtype=torch.float32, device=DEV)


def pack_weight(w_bf16_bits, dtype, layout=frt.W_PLAIN, gamma=None, stream=None):
    """Pack a bf16 weight [K][N] (uint16 bits, numpy or CUDA tensor) on the GPU.

    Returns (packed uint8 tensor, colscale float32 tensor or None).
    """
    w = w_bf16_bits if isinstance(w_bf16_bits, torch.Tensor) else to_dev(np.asarray(w_bf16_bits, np.uint16).view(np.int16))
    K, N = w.shape
    packed = empty_bytes(frt.frt_weight_bytes(dtype, K, N))
    cs = empty_f32(N) if dtype == frt.E4M3 else None
    g = None if gamma is None else (gamma if isinstance(gamma, torch.Tensor) else to_dev(np.asarray(gamma, np.float32)))
    frt.frt_pack_weight(K, N, w, g, dtype, layout, packed, cs, stream=stream)
    return packed, cs


def operand_codes(packed, dtype, M, K):
    """Packed operand (CUDA tensor) -> logical codes [M][K] (numpy) via the host unpacker."""
    return frt.frt_operand_unpack_host(to_np(packed), dtype, M, K)


def weight_codes(packed, dtype, K, N, layout=frt.W_PLAIN):
    return frt.frt_weight_unpack_host(to_np(packed), dtype, K, N, layout)
