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


# ------------------------------------------------- whole-output oracle runs

_FULL = {}


def full_oracle(shape, li, w_dev=None, label=""):
    """The oracle's layer over every token of a workload, computed once per
    workload shape in a test session and shared by the modules that need it.

    w_dev: the canonical MXFP4 weights as the workload generator made them on
    the device (the GPU path reads a tiled copy); each hit expert's bytes are
    copied to the host when the oracle asks for that expert, which is cheaper
    than regenerating them on the CPU.  Returns (out float64 [T][H], routing
    dict of ids / w / offsets / perm_src / dest_row).
    """
    if shape in _FULL:
        return _FULL[shape]
    import time
    t0 = time.time()
    done = [0]
    if w_dev is None:
        base = cpu_weights(shape)
    else:
        def base(e):
            return [t[e].cpu().numpy() for t in w_dev]

    def fetch(e):
        done[0] += 1
        if done[0] % 64 == 0:
            print(f"[oracle {label}] {done[0]} experts ({time.time() - t0:.0f}s)", flush=True)
        return base(e)

    out, it = omoe.moe_layer(x_as_f64(li), li.logits, shape.k, fetch, shape.layout, return_intermediates=True)
    it.pop("Y")
    print(f"[oracle {label}] whole layer: {done[0]} experts, {time.time() - t0:.1f}s", flush=True)
    _FULL[shape] = (out, it)
    return out, it


def generator_matches_on_cpu(shape, w_dev, experts):
    """The device-generated weights of the given experts equal the CPU generator's bytes."""
    for e in experts:
        cpu = gen.expert_weights(shape, int(e), 0, "cpu")
        for d, c in zip(w_dev, cpu):
            if not torch.equal(d[int(e)].cpu(), c):
                return False
    return True
