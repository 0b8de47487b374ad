"""MI355X (gfx950) library for one EAGLE-2 draft-tree verification step.

The compute path is the HIP library libeagle_tree.so (C ABI in
include/eagle_tree.h); `binding` marshals torch tensors to it, `step` sequences
its five calls, `workload` draws the seeded synthetic inputs.
"""
__all__ = ["binding", "step", "workload", "build"]
