"""Device-resident MoE layers: upload canonical expert tensors and pack them.

Plumbing around ``moe_pack_experts``: PyTorch allocates the slab and a staging
buffer on the GPU, the canonical tensors are copied over in chunks of experts,
and the library's pack kernel writes the records.  The canonical tensors come
from any ``source(first, n)`` callable returning an object with numpy
attributes ``gate``, ``up``, ``down``, ``scales``, ``biases`` stacked over the
experts [first, first + n) (expert id E is the shared expert).
"""
from dataclasses import dataclass, field

import torch

from . import make_desc, pack_experts, record_bytes, workspace_bytes, stack_extra_bytes


def upload_experts(source, n_total, bits, H, I, device="cuda", chunk=32, slab=None):
    rb = record_bytes(bits, H, I)
    if rb == 0:
        raise ValueError("unsupported expert shape bits=%d H=%d I=%d" % (bits, H, I))
    if slab is None:
        slab = torch.empty(n_total * rb, dtype=torch.uint8, device=device)
    staging = None
    for first in range(0, n_total, chunk):
        n = min(chunk, n_total - first)
        c = source(first, n)
        arrays = [torch.from_numpy(a.reshape(n, -1)) for a in (c.gate, c.up, c.down, c.scales, c.biases)]
        if staging is None or staging[0].shape[0] < n:
            staging = [torch.empty((n,) + tuple(a.shape[1:]), dtype=a.dtype, device=device) for a in arrays]
        dev = [s[:n] for s in staging]
        for d, a in zip(dev, arrays):
            d.copy_(a)
        pack_experts(bits, H, I, n, *dev, slab, first)
    torch.cuda.synchronize()
    return slab


@dataclass
class DeviceLayer:
    """One packed layer on the GPU plus the descriptor the C ABI takes."""
    H: int
    I: int
    E: int
    K: int
    bits: int
    slab: torch.Tensor
    w_router: torch.Tensor
    logit_bias: torch.Tensor = None
    shared_weight: float = 1.0
    renormalize: bool = True
    desc: object = field(init=False)

    def __post_init__(self):
        self.desc = make_desc(self.H, self.I, self.E, self.K, self.bits, self.slab, self.w_router,
                              self.logit_bias, self.shared_weight, self.renormalize)

    def record(self, e):
        rb = record_bytes(self.bits, self.H, self.I)
        return self.slab[e * rb:(e + 1) * rb]


def workspace(desc, B, device="cuda", stack=False):
    n = workspace_bytes(desc, B) + (stack_extra_bytes(B, desc.H) if stack else 0)
    if n == 0:
        raise ValueError("invalid layer descriptor or batch")
    return torch.zeros(n, dtype=torch.uint8, device=device), n
