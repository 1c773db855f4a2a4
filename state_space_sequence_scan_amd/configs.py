"""The workloads the scan is measured and parity-tested on.

Shapes are those of the models the Mamba-3 pages describe: the 113M pure
Mamba-3 "nanomamba3" LM (d_model 768, 12 layers, MIMO rank 2, chunk 32:
the nanomamba3 article's model table) and 1.5B-scale layers with state size
128 (the Mamba-3 paper note, sections "Solution 3: MIMO" (R = 4) and
"Speed" (Table 6, state 128)).  d_model / d_inner are not consumed by the
scan (d_inner = H * P) and are kept only as labels.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    seqlen: int          # prefill length L
    nheads: int          # H
    headdim: int         # P
    dstate: int          # N
    rank: int            # R (1 = SISO)
    chunk: int           # Q
    ngroups: int = 1     # G (B, C, theta shared by H/G heads)
    io_dtype: str = "bf16"          # dtype of x, B, C, y ("fp32" or "bf16")
    theta_scale: float = 1.0
    decode_steps: int = 0
    seed: int = 1000
    label: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


CONFIGS = {
    "siso_l256_fp32": ScanConfig("siso_l256_fp32", batch=1, seqlen=256, nheads=4, headdim=16, dstate=16, rank=1,
                     chunk=32, io_dtype="fp32", seed=1000,
                     label="single SISO layer, fp32, L=256, H=4, P=16, N=16, chunk 32"),
    "nanomamba3": ScanConfig("nanomamba3", batch=4, seqlen=2048, nheads=24, headdim=64, dstate=128, rank=2,
                     chunk=32, seed=1001,
                     label="nanomamba3-shaped layer (d_model 768, d_inner 1536): 24 heads x P=64, "
                           "N=128, MIMO R=2, chunk 32, batch 4, L=2048"),
    "siso_l8192": ScanConfig("siso_l8192", batch=8, seqlen=8192, nheads=64, headdim=64, dstate=128, rank=1,
                     chunk=64, seed=1002,
                     label="1.5B-scale SISO layer (d_model 2048): 64 heads x P=64, N=128, R=1, "
                           "chunk 64, batch 8, L=8192"),
    "mimo4_l16384": ScanConfig("mimo4_l16384", batch=2, seqlen=16384, nheads=64, headdim=64, dstate=128, rank=4,
                     chunk=64, theta_scale=4.0, seed=1003,
                     label="1.5B-scale MIMO layer: 64 heads x P=64, N=128, R=4, chunk 64, batch 2, "
                           "L=16384, theta x4"),
    # The chunk of this workload's prefill is not fixed by the model: 32, the faster of the two
    # chunk sizes of the matrix-core path at R = 4 on this batch (chunk 64 is the other).
    "mimo4_decode_b256": ScanConfig("mimo4_decode_b256", batch=256, seqlen=1024, nheads=64, headdim=64, dstate=128, rank=4,
                     chunk=32, decode_steps=512, seed=1004,
                     label="1.5B-scale MIMO R=4 layer, batch 256: 1024-token chunked prefill (chunk 32), "
                           "then 512 single-token decode steps from its fp32 state"),
}


# Single-chunk sequences (L = Q) at the head shapes of the 1.5B-scale layers: each sequence is
# exactly one intra-chunk block (the masked C~B~^T product over the chunk) plus its chunk-state
# contraction, with no state passed between chunks.  They measure the intra-chunk contractions
# on their own; they are measurement workloads, not layers of the pages' models.
INTRA_CHUNK = {
    "mimo4_chunk64_b4096": ScanConfig("mimo4_chunk64_b4096", batch=4096, seqlen=64, nheads=64, headdim=64,
                                      dstate=128, rank=4, chunk=64, seed=1005,
                                      label="single-chunk sequences at the 1.5B MIMO head shape: 64 heads x P=64, "
                                            "N=128, R=4, L = chunk = 64, batch 4096"),
    "siso_chunk64_b4096": ScanConfig("siso_chunk64_b4096", batch=4096, seqlen=64, nheads=64, headdim=64,
                                     dstate=128, rank=1, chunk=64, seed=1006,
                                     label="single-chunk sequences at the 1.5B SISO head shape: 64 heads x P=64, "
                                           "N=128, R=1, L = chunk = 64, batch 4096"),
}


def scaled(cfg: ScanConfig, **kw) -> ScanConfig:
    """A copy with some fields replaced (smaller parity-test variants)."""
    return dataclasses.replace(cfg, **kw)


THETA_RANGE = math.pi
