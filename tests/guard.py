"""Device output buffers fenced by canary bytes: a kernel that writes past either end of its output
(a ragged M or N tile, a clamped row) changes a canary, and check() fails."""
import numpy as np

PAD = 256          # bytes on each side: keeps every output 256-byte aligned
CANARY = 0xC5


class Guarded:
    def __init__(self, shape, dtype, dev):
        import torch
        itemsize = torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(np.prod(shape)) * itemsize
        self.raw = torch.full((self.nbytes + 2 * PAD,), CANARY, dtype=torch.uint8, device=dev)
        self.tensor = self.raw[PAD:PAD + self.nbytes].view(dtype).view(*shape)

    def check(self, what=""):
        import torch
        torch.cuda.synchronize()
        head = self.raw[:PAD].cpu().numpy()
        tail = self.raw[PAD + self.nbytes:].cpu().numpy()
        assert np.all(head == CANARY), f"{what}: write before the start of the output"
        assert np.all(tail == CANARY), f"{what}: write past the end of the output"
