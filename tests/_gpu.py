"""Uploading synthetic layers to the GPU (bf16 bit patterns -> torch.bfloat16)."""
import numpy as np
import torch


def dev_tensor(vals32, bits, device="cuda"):
    if bits is not None:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(vals32, dtype=np.float32))
    return t.to(device)


def upload(layer, device="cuda"):
    W = dev_tensor(layer.W, layer.W_bits, device)
    has_x = layer.X is not None or layer.X_bits is not None
    X = dev_tensor(layer.X, layer.X_bits, device) if has_x else None
    H = torch.from_numpy(layer.H).to(device) if layer.H is not None else None
    return W, X, H


def to_np(t):
    return t.detach().cpu().numpy()
