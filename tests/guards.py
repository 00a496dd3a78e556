"""Guard canaries for GPU outputs and workspaces.

Every buffer handed to the library is a view into a larger allocation whose
leading and trailing PAD bytes hold a fixed byte pattern.  After each call the
test reads the pads back: any byte changed means a kernel wrote outside the
buffer it was given.
"""
import numpy as np
import torch

PAD = 4096
PATTERN = 0xA5


class GuardedAlloc:
    def __init__(self, device="cuda"):
        self.device = device
        self.items = []

    def empty(self, shape, dtype, name="buffer"):
        if isinstance(shape, int):
            shape = (shape,)
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((n + 2 * PAD,), PATTERN, dtype=torch.uint8, device=self.device)
        view = raw[PAD:PAD + n].view(dtype).view(shape)
        self.items.append((name, raw, n))
        return view

    def check(self, what=""):
        torch.cuda.synchronize()
        for name, raw, n in self.items:
            h = raw.cpu().numpy()
            lo, hi = h[:PAD], h[PAD + n:]
            assert (lo == PATTERN).all(), ("write before", name, what, int(np.argmax(lo != PATTERN)))
            assert (hi == PATTERN).all(), ("write past", name, what, int(np.argmax(hi != PATTERN)))
