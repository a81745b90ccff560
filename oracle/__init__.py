"""CPU oracle for the RaggedShard/DBuffer layout transform.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
statement of what the layout transform computes, written from the pages'
definitions (and, where they are silent, from one stated reading). Only the
tests, the smoke check and the bench's CPU-baseline leg may import it; the
product library never does, and nothing here imports the product package.

Floating point follows the rule "compute in float64, round once to float32":
for a single +, x or / of fp32 operands this equals the correctly rounded
fp32 result, because float64 carries more than 2*24+2 significand bits.

Sources cited in the modules:
  [summary]  "veScale-FSDP: Flexible and High-Performance FSDP at Scale"
             (bud-325 summary page), sections Key claims / Method.
  [walk]     "veScale-FSDP: flexible, structure-aware sharding at 10K-GPU
             scale" (feynmanwiki walkthrough); it has no section numbers, so
             a citation names the paragraph's topic.
  [OCP]      OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding.

Parity status: every function here is pinned by a CPU test except the
planner's choice among the valid plans beyond the 2x bound ("parity unpinned"
for optimality; validity and the bound are pinned).
"""
from . import adam, codes, plan, transform

__all__ = ["adam", "codes", "plan", "transform"]
