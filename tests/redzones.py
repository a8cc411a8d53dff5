"""Red zones around the buffers the GPU tests hand to the library.

Every output, workspace and expert-output buffer a GPU test allocates through
`poisoned()` is the middle of a larger device allocation whose GUARD bytes on
either side hold the same poison byte as the buffer. After each test,
`check()` reads the zones back: a byte that changed means some kernel wrote
past the start or the end of that buffer, and the test fails naming the
buffer and the first changed offset. This checks the shipped library itself
(no separate build, no device-side trap) on every parity case the suites run.
The zones catch writes that land within GUARD bytes of a buffer, which covers
an index one row or one element too far for rows of up to GUARD bytes and the
first GUARD bytes of a longer row.
"""
import numpy as np
import torch

GUARD = 4096   # bytes on each side; a multiple of every element size used

_live = []     # (base allocation, payload bytes, poison byte, label)


def poisoned(shape, dtype, byte, device):
    """An uninitialised-looking tensor of `shape` and `dtype` filled with
    `byte`, flanked by GUARD bytes of `byte` on each side."""
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    numel = int(np.prod(shape, dtype=np.int64)) if shape else 1
    nbytes = numel * torch.empty((), dtype=dtype).element_size()
    base = torch.empty(nbytes + 2 * GUARD, dtype=torch.uint8, device=device)
    base.fill_(byte)
    t = base[GUARD:GUARD + nbytes].view(dtype).view(shape)
    _live.append((base, nbytes, byte, f"{tuple(shape)} {dtype}"))
    return t


def check():
    """Fail if any red zone of the buffers allocated since the last check
    changed; forgets them either way."""
    live = list(_live)
    _live.clear()
    if not live:
        return
    if any(base.is_cuda for base, _, _, _ in live):
        torch.cuda.synchronize()
    bad = []
    for base, nbytes, byte, label in live:
        head = base[:GUARD].cpu().numpy()
        tail = base[GUARD + nbytes:].cpu().numpy()
        for side, zone in (("before", head), ("after", tail)):
            hit = np.flatnonzero(zone != byte)
            if hit.size:
                off = GUARD - hit[-1] if side == "before" else hit[0]
                bad.append(f"{label}: {hit.size} bytes changed {side} the buffer "
                           f"(nearest {off} bytes {side} it)")
    assert not bad, "writes outside their buffers: " + "; ".join(bad)
