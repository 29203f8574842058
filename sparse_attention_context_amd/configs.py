"""The five ISA workloads, as data.

Each is one in-context attention layer: B batches, H heads of width d,
Ns source-video tokens followed by Nc context tokens, block size b, the
fraction rho of context blocks kept and the fraction gamma of query blocks
routed to full attention.  ``clips`` splits the context into reference clips,
each with the scale its keys get in the synthetic inputs (low-saliency
context); ``sharp`` is the fraction of source queries sharpened towards a
source key.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    Ns: int
    Nc: int
    b: int
    rho: float
    gamma: float
    dtype: str            # "bf16" or "f32"
    seed: int
    clips: tuple = ((1.0, 0.5),)   # (fraction of Nc, key scale) per clip
    sharp: float = 0.20
    gammas: tuple = field(default=())  # extra gamma values swept on this shape


TINY = Workload("tiny_isa_check", 1, 2, 64, 256, 256, 16, 0.50, 0.25, "f32", 1, sharp=0.25)
SMALL = Workload("small_video_layer", 1, 12, 64, 4096, 4096, 64, 0.25, 0.20, "bf16", 2)
VIDEO_DIT = Workload("video_dit_layer", 1, 24, 128, 17550, 17550, 64, 0.25, 0.20, "bf16", 3)
LONG_CLIP = Workload("long_clip", 1, 24, 128, 32760, 32760, 64, 0.25, 0.0, "bf16", 4,
                     gammas=(0.0, 0.10, 0.30, 1.0))
MULTI_REF = Workload("multi_reference_icl", 1, 40, 128, 16384, 49152, 128, 0.15, 0.15, "bf16", 5,
                     clips=((1 / 3, 0.3), (1 / 3, 0.5), (1 / 3, 0.8)))

ALL = (TINY, SMALL, VIDEO_DIT, LONG_CLIP, MULTI_REF)
BY_NAME = {w.name: w for w in ALL}
