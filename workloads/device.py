"""Host <-> device marshalling of workload arrays (no arithmetic).

bfloat16 arrays live on the host as uint16 bit patterns and on the device as
torch.bfloat16; the conversion is a reinterpretation of the bits.
"""

import numpy as np


def to_dev(a, device="cuda"):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t):
    import torch

    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
