"""Host-side bookkeeping of a speculative run (no GPU, no method arithmetic).

Definitions follow the lucebox RTX 3090 run reported in "DFlash 深度解析"
(chenxutan.com/d/2993) §4.5: tokens per step is emitted tokens over draft
(verify) steps, and the "acceptance" percentage printed there is tokens per
step divided by the block length.  The community benchmark of the llama.cpp
merge reports draft acceptance as accepted drafts over drafted tokens; both are
returned.
"""
from __future__ import annotations


def spec_stats(emitted: int, steps: int, block: int, seconds: float = 0.0,
               accepted_drafts: int = 0, drafted: int = 0) -> dict:
    out = {
        "tokens_per_step": emitted / steps if steps else 0.0,
        "acceptance_per_block": (emitted / steps) / block if steps else 0.0,
        "draft_acceptance": accepted_drafts / drafted if drafted else 0.0,
    }
    if seconds > 0:
        out["tok_per_s"] = emitted / seconds
    return out
