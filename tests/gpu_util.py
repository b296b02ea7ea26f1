"""Helpers shared by the GPU tests: input upload, oracle runs, error metric."""
import numpy as np
import torch

from oracle import moe as omoe
from oracle import mx as omx
from workloads import gen


def rel_err(gpu, ref):
    """max |gpu - ref| / max |ref| (the acceptance metric)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(gpu - ref).max() / np.abs(ref).max())


def cpu_weights(shape, layer=0):
    """Oracle-side weights of expert e, regenerated on the CPU."""
    return lambda e: [t.numpy() for t in gen.expert_weights(shape, e, layer, "cpu")]


def device_weights(shape, layer=0, device="cuda"):
    return gen.all_expert_weights(shape, layer, device)


def x_as_f64(li):
    if li.x_codes is not None:
        return omoe.activations(x_codes=li.x_codes.numpy(), x_scales=li.x_scales.numpy())
    return omoe.activations(x_bf16=li.x_bf16.view(torch.int16).numpy())


def oracle_layer(shape, li, layer=0):
    return omoe.moe_layer(x_as_f64(li), li.logits, shape.k, cpu_weights(shape, layer), shape.layout,
                          return_intermediates=True)


def device_x(li, device="cuda"):
    if li.x_codes is not None:
        return li.x_codes.to(device), li.x_scales.to(device)
    return li.x_bf16.to(device), None
