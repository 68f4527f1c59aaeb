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

from . import (expert_ranges, make_desc, pack_experts, record_bytes, requant_4to2, workspace_bytes,
               stack_extra_bytes)


def upload_experts(source, n_total, bits, H, I, device="cuda", chunk=32, slab=None, group=64):
    rb = record_bytes(bits, H, I, group)
    if rb == 0:
        raise ValueError("unsupported expert shape bits=%d H=%d I=%d group=%d" % (bits, H, I, group))
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
        pack_experts(bits, H, I, n, *dev, slab, first, group=group)
    torch.cuda.synchronize()
    return slab


def host_store(source, n_total, bits, H, I, device="cuda", chunk=32, group=64):
    """The packed records of n_total experts in pinned host memory (the backing store of an
    expert cache): each chunk is packed on the GPU into a small device buffer and copied out,
    so the whole layer never has to fit in device memory."""
    rb = record_bytes(bits, H, I, group)
    store = torch.empty(n_total * rb, dtype=torch.uint8, pin_memory=True)
    buf = torch.empty(chunk * rb, dtype=torch.uint8, device=device)
    for first in range(0, n_total, chunk):
        n = min(chunk, n_total - first)
        c = source(first, n)
        arrays = [torch.from_numpy(a.reshape(n, -1)).to(device) for a in (c.gate, c.up, c.down, c.scales, c.biases)]
        pack_experts(bits, H, I, n, *arrays, buf, 0, group=group)
        store[first * rb:(first + n) * rb].copy_(buf[:n * rb])
    torch.cuda.synchronize()
    return store


def upload_requantized(source4, n_total, H, I, device="cuda", chunk=32, slab=None, group=64):
    """A 2-bit slab from canonical 4-bit experts: each chunk is uploaded, requantized on the
    GPU (moe_requant_4to2) and packed as 2-bit records.  source4(first, n) as for
    upload_experts, with 4-bit tensors."""
    rb = record_bytes(2, H, I, group)
    if slab is None:
        slab = torch.empty(n_total * rb, dtype=torch.uint8, device=device)
    for first in range(0, n_total, chunk):
        n = min(chunk, n_total - first)
        c = source4(first, n)
        g4, u4, d4, s4, b4 = [torch.from_numpy(a.reshape(n, -1)).to(device)
                              for a in (c.gate, c.up, c.down, c.scales, c.biases)]
        g2 = torch.empty((n, I * H // 4), dtype=torch.uint8, device=device)
        u2 = torch.empty_like(g2)
        d2 = torch.empty((n, H * I // 4), dtype=torch.uint8, device=device)
        s2, b2 = torch.empty_like(s4), torch.empty_like(b4)
        requant_4to2(H, I, n, g4, u4, d4, s4, b4, g2, u2, d2, s2, b2, group=group)
        pack_experts(2, H, I, n, g2, u2, d2, s2, b2, slab, first, group=group)
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
    range_flags: bool = True    # scan the records for the matrix-core range (moe_expert_ranges)
    group: int = 64             # weights per scale/bias group (64, 128 or 256)
    desc: object = field(init=False)
    expert_flags: torch.Tensor = field(init=False, default=None)

    def __post_init__(self):
        flags = None
        if self.range_flags:
            # on the GPU even when the records are a store in pinned host memory
            self.expert_flags = torch.empty(self.E + 1, dtype=torch.int32, device=self.w_router.device)
            expert_ranges(self.bits, self.H, self.I, self.slab, self.E + 1, self.expert_flags, group=self.group)
            # the descriptor carries the flags only when an expert is out of range: flags
            # that are all zero change nothing on the 4-bit paths, and would keep 2-bit
            # batches off the grouped path (one host read here, when the layer is built)
            if bool(self.expert_flags.any()):
                flags = self.expert_flags
        self.desc = make_desc(self.H, self.I, self.E, self.K, self.bits, self.slab, self.w_router,
                              self.logit_bias, self.shared_weight, self.renormalize, group=self.group,
                              expert_flags=flags)

    def record(self, e):
        rb = record_bytes(self.bits, self.H, self.I, self.group)
        return self.slab[e * rb:(e + 1) * rb]


def workspace(desc, B, device="cuda", stack=False):
    n = workspace_bytes(desc, B) + (stack_extra_bytes(B, desc.H) if stack else 0)
    if n == 0:
        raise ValueError("invalid layer descriptor or batch")
    return torch.zeros(n, dtype=torch.uint8, device=device), n
