"""MI355X (gfx950) SLA / SLA2 sparse-linear attention.

Hand-written HIP kernels behind the C ABI of include/sla.h. The forward pass:
router projection + block mean pooling, compressed scores + three-way block
classification, per-key-block linear state h_j / z_j, the marginal-block
sums (one MFMA product per head), and block-sparse online-softmax attention
over the critical blocks with the linear-branch output and the SLA2 mix (or
the SLA output fusion O = O_s + Proj(O_l)) fused into its epilogue. Also the
backward pass for a fixed mask (on its own, or from the state a saving
forward pass kept) and the SoftTop-k relaxation of the block selection. This package is the argument-marshalling binding.
"""

from ._binding import (  # noqa: F401
    LIB_PATH, HipEvents, Plan, SLAError, backward, backward_saved, backward_sla1, backward_sla1_saved, block_counts,
    forward, forward_noalloc, forward_sla1, forward_sla1_train, forward_train, load_library, make_problem,
    noalloc_scratch_bytes, soft_topk, workspace_bytes,
)

__all__ = ["forward", "forward_noalloc", "noalloc_scratch_bytes", "forward_sla1", "backward", "backward_sla1",
           "forward_train", "forward_sla1_train", "backward_saved", "backward_sla1_saved", "soft_topk", "Plan",
           "HipEvents", "block_counts", "workspace_bytes", "load_library", "make_problem", "SLAError", "LIB_PATH"]
