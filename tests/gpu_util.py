"""Helpers shared by the GPU parity tests: host <-> device copies and the
boundary-tolerant code comparison."""
import numpy as np

TOL_BOUNDARY = 1e-4      # code units: pre-round values this close to x.5 may round either way
TOL_OBJECTIVE = 1e-4     # relative


def torch_mod():
    import torch
    return torch


def dev():
    torch = torch_mod()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(a):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:      # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(a).to(dev())


def to_host(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def qz():
    import post_weight_quantization_05_amd as q
    q.lib()          # fails loudly if the HIP library is missing
    return q


def report(name, **kv):
    print(f"[{name}] " + " ".join(f"{k}={v}" for k, v in kv.items()), flush=True)
