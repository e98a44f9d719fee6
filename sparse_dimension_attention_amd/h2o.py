"""H2O decoding over a compact AQUA-Memory cache (AQUA combined with H2O heavy-hitter eviction:
abstract of arXiv 2509.11155; edgentiq blog, "Key Advantages").

Each (b, g) keeps ``heavy + recent`` slots.  A step is four libaqua calls on one stream (or the
single launch ``aqua_h2o_step``, which computes the same thing):

1. ``aqua_h2o_victim``: evict the non-recent slot ranked lowest by (mass desc, position asc) and
   claim it for the new position (its mass restarts at 0);
2. ``aqua_project_keys`` with ``slots = victim``: the new token's K' (first ``d_store`` dims) and V
   go into that slot;
3. ``aqua_select_dims``: every query head's q' and top-k mask over the first ``d_sel`` dims;
4. ``aqua_decode`` in mass mode over all slots: the attention output, and every slot's mass grows
   by the group's summed softmax weight.

Only one slot changes per step because a token outside the cache never gains mass while cached
ones only gain (non-negative fp32 additions), so the full-recompute heavy set of a step is the
previous set minus one member, plus the token that has just left the recent window.

:meth:`H2OCache.from_full` builds the starting state from a full-context cache and its mass
(the cumulative attention of earlier steps) with ``aqua_h2o_init``: the ``heavy`` positions of
highest mass among those older than the recent window, plus the ``recent`` latest positions.
Torch only allocates the compact state's tensors; every number in it comes from libaqua.
"""
from __future__ import annotations

import torch

from . import aqua as A


class H2OCache:
    """Compact per-(b, g) cache: K' ``[B][Hkv][d_store][n_slots]``, V ``[B][Hkv][n_slots][d]``,
    ``slot_pos`` int32 and ``mass`` fp32 ``[B][Hkv][n_slots]``, plus the decode workspace."""

    def __init__(self, kp, v, slot_pos, mass, heavy: int, recent: int):
        self.kp, self.v, self.slot_pos, self.mass = kp, v, slot_pos, mass
        self.heavy, self.recent = heavy, recent
        B, Hkv, _, n_slots = kp.shape
        self.cache = A.make_cache(kp, v, n_slots)
        self.victim = torch.empty(B, Hkv, dtype=torch.int32, device=kp.device)
        self.ws = None

    @classmethod
    def from_full(cls, kp_full, v_full, mass_full, length: int, heavy: int, recent: int):
        """Starting state after ``length`` tokens (positions 0..length-1) of a full cache
        ``kp_full [B][Hkv][d_store][T_cap]``, ``v_full [B][Hkv][T_cap][d]`` whose mass is
        ``mass_full [B][Hkv][T_cap]``.  Requires ``length - recent >= heavy``."""
        if length - recent < heavy:
            raise ValueError("fewer older tokens than heavy-hitter slots")
        B, Hkv, d_store, _ = kp_full.shape
        n_slots = heavy + recent
        kp = torch.empty(B, Hkv, d_store, n_slots, dtype=kp_full.dtype, device=kp_full.device)
        v = torch.empty(B, Hkv, n_slots, v_full.shape[-1], dtype=v_full.dtype,
                        device=v_full.device)
        mass = torch.empty(B, Hkv, n_slots, dtype=torch.float32, device=kp_full.device)
        pos = torch.empty(B, Hkv, n_slots, dtype=torch.int32, device=kp_full.device)
        A.aqua_h2o_init(A.make_cache(kp_full, v_full, length), mass_full, heavy, recent,
                        A.make_cache(kp, v, n_slots), mass, pos)
        return cls(kp, v, pos, mass, heavy, recent)

    def workspace(self, Hq: int):
        if self.ws is None:
            n = A.aqua_decode_workspace(self.cache, Hq)
            self.ws = torch.empty(n, dtype=torch.uint8, device=self.kp.device)  # no clearing needed
        return self.ws

    def step(self, q, k_new, v_new, P, t_new: int, d_sel: int, k: int, scale: float, out,
             q_proj, mask, stream=None, fused: bool = False):
        """One decode step for the token at position ``t_new``.
        q ``[B][Hq][d]``, k_new/v_new ``[B][Hkv][d]`` (raw, the cache's dtype); out ``[B][Hq][d]``
        fp32; q_proj ``[B][Hq][d]`` fp32 and mask ``[B][Hq][d/32]`` int32 are written.
        ``fused`` runs the step as the single launch ``aqua_h2o_step`` (the same results, bit for
        bit, as the four calls below)."""
        Hq = q.shape[1]
        ws = self.workspace(Hq)
        if fused:
            A.aqua_h2o_step(self.cache, Hq, q, k_new, v_new, P, d_sel, k, scale, self.mass,
                            self.slot_pos, t_new, self.recent, self.victim, out, ws,
                            q_proj_out=q_proj, mask_out=mask, stream=stream)
            return
        A.aqua_h2o_victim(self.mass, self.slot_pos, t_new, self.recent, self.victim, stream)
        A.aqua_project_keys(self.cache, k_new, v_new, P, 1, slots=self.victim, stream=stream)
        A.aqua_select_dims(q, P, d_sel, k, q_proj, mask, stream=stream)
        A.aqua_decode(self.cache, Hq, q_proj, mask, scale, out, ws, mass=self.mass, stream=stream)
