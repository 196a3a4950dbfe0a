"""Slot pool of fixed-size per-request recurrent states.

"Retrofitting Linear Attention into Diffusion Language Models", section 3.3:
the recurrent state is kept per query head beside the paged KV cache and
reuses its slot allocator; its size does not depend on how many tokens it
has absorbed, so a fixed memory budget admits a fixed number of requests.

One slot holds, for every head of one hybrid layer,
    S [H][2F][d] fp32   (sum of phi(k) v^T)
    Z [H][2F]    fp32   (sum of phi(k))
i.e. 4 H 2F (d + 1) bytes: 2,113,536 B at H = 16, F = d = 128.  The pool is
two dense tensors ``S[n_slots][H][2F][d]`` and ``Z[n_slots][H][2F]`` that the
kernels index with 64-bit offsets, plus a host-side free list.  Device
memory comes from torch's allocator; the HIP library itself allocates
nothing.
"""
from __future__ import annotations

import torch


def slot_bytes(heads: int, head_dim: int, feat: int) -> int:
    """Bytes of one slot (all heads of one layer): S and Z in fp32."""
    return 4 * heads * 2 * feat * (head_dim + 1)


def slots_for_budget(budget_bytes: int, heads: int, head_dim: int, feat: int, layers: int = 1) -> int:
    """How many requests' states fit in ``budget_bytes`` for ``layers`` hybrid layers."""
    per_req = slot_bytes(heads, head_dim, feat) * layers
    return int(budget_bytes // per_req)


class StatePool:
    """Fixed-size S/Z states for up to ``n_slots`` concurrent requests."""

    def __init__(self, n_slots: int, heads: int, head_dim: int, feat: int,
                 device="cuda", allocate: bool = True):
        if n_slots <= 0 or heads <= 0 or head_dim <= 0 or feat <= 0:
            raise ValueError("pool dimensions must be positive")
        self.n_slots, self.heads, self.head_dim, self.feat = n_slots, heads, head_dim, feat
        self.device = torch.device(device)
        self._free = list(range(n_slots - 1, -1, -1))   # pop() hands out the lowest slot
        self._used = set()
        self.S = self.Z = None
        if allocate:
            self.S = torch.zeros((n_slots, heads, 2 * feat, head_dim), dtype=torch.float32, device=self.device)
            self.Z = torch.zeros((n_slots, heads, 2 * feat), dtype=torch.float32, device=self.device)

    @property
    def nbytes(self) -> int:
        return self.n_slots * slot_bytes(self.heads, self.head_dim, self.feat)

    @property
    def free_slots(self) -> int:
        return len(self._free)

    def alloc(self, n: int) -> torch.Tensor:
        """Reserve ``n`` slots with empty (zero) states; returns them as int32
        on the pool's device, ready to pass as the ``slot`` map."""
        if n > len(self._free):
            raise MemoryError(f"state pool exhausted: {n} requested, {len(self._free)} free")
        got = [self._free.pop() for _ in range(n)]
        self._used.update(got)
        idx = torch.tensor(got, dtype=torch.int32)
        if self.S is not None and n:
            dev_idx = idx.to(self.device, dtype=torch.long)
            self.S.index_fill_(0, dev_idx, 0.0)
            self.Z.index_fill_(0, dev_idx, 0.0)
        return idx.to(self.device)

    def free(self, slots) -> None:
        """Return slots to the pool (their contents become garbage)."""
        for s in (int(x) for x in torch.as_tensor(slots).flatten().tolist()):
            if s not in self._used:
                raise ValueError(f"slot {s} is not allocated")
            self._used.remove(s)
            self._free.append(s)

    def save(self, slots):
        """Copy the states of ``slots`` out (checkpoint of a request's context)."""
        idx = torch.as_tensor(slots, device=self.device).long()
        return self.S.index_select(0, idx).clone(), self.Z.index_select(0, idx).clone()

    def restore(self, slots, saved) -> None:
        """Write saved states into ``slots`` (possibly other slots than saved from)."""
        idx = torch.as_tensor(slots, device=self.device).long()
        S, Z = saved
        self.S.index_copy_(0, idx, S)
        self.Z.index_copy_(0, idx, Z)
