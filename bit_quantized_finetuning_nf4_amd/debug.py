"""Debug mode of the binding, switched on by the environment: QLORA_DEBUG=1.

In debug mode every output tensor and workspace that the binding allocates
sits between two guard bands of GUARD_BYTES filled with a fixed byte, and
after every successful library call the binding synchronizes the device (so
a fault is reported at the call that caused it, not at some later
synchronization) and checks that no live guard band has changed (so a
kernel that writes past the end or before the start of its output is
caught at once).  Outputs the caller passes in are not guarded.

Off (the default) the allocation helper is a plain torch.empty and the
check is never called.
"""

import os
import weakref

import torch

ENABLED = os.environ.get("QLORA_DEBUG", "") == "1"
GUARD_BYTES = 256   # keeps the guarded view 256-byte aligned
PATTERN = 0xA5

_live = []   # weak references to guarded views


class CanaryError(RuntimeError):
    """A library call wrote into the guard band of a buffer."""


def empty(shape, dtype, device):
    """torch.empty(shape, dtype, device); in debug mode the tensor is a view
    into a larger buffer whose guard bands hold PATTERN."""
    if not ENABLED:
        return torch.empty(shape, dtype=dtype, device=device)
    if isinstance(shape, int):
        shape = (shape,)
    n = 1
    for d in shape:
        n *= int(d)
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    base = torch.full((nbytes + 2 * GUARD_BYTES,), PATTERN, dtype=torch.uint8, device=device)
    view = base[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(tuple(shape))
    view._qlora_guard = (base, nbytes)
    _live.append(weakref.ref(view))
    return view


def guards_intact(view):
    """True when both guard bands of a guarded view still hold PATTERN."""
    base, nbytes = view._qlora_guard
    lo = base[:GUARD_BYTES]
    hi = base[GUARD_BYTES + nbytes:]
    return bool(((lo == PATTERN).all() & (hi == PATTERN).all()).item())


def after_call(what):
    """Synchronize and check every live guard band; raise CanaryError naming
    the call when one has changed."""
    if any(ref() is not None and ref().is_cuda for ref in _live) or torch.cuda.is_initialized():
        torch.cuda.synchronize()
    alive = []
    bad = []
    for ref in _live:
        v = ref()
        if v is None:
            continue
        alive.append(ref)
        if not guards_intact(v):
            bad.append(tuple(v.shape))
    _live[:] = alive
    if bad:
        raise CanaryError(f"{what}: guard band changed around buffer(s) of shape {bad}")
