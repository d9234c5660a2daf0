"""ELSAA attention (sparse sortLSH branch + RACE low-rank branch + denominator-aware
fusion) on AMD MI355X (gfx950): hand-written HIP kernels behind a C ABI
(include/elsaa.h), with a thin torch binding."""
from .ops import (ElsaaConfig, ElsaaFunction, backward, check_orders, elsaa_attention, forward,
                  forward_fused,
                  gates, gates_backward, lowrank_summary, make_planes, select, select_noalloc,
                  topk)

__all__ = ["ElsaaConfig", "ElsaaFunction", "backward", "check_orders", "elsaa_attention",
           "forward", "forward_fused", "gates", "gates_backward", "lowrank_summary", "make_planes", "select",
           "select_noalloc", "topk"]
