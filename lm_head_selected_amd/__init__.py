"""MI355X-native fused LM-head GRPO / GSPO loss.

The computation lives in the gfx950 HIP library lib/libgrpo_head.so (C ABI in
include/grpo_head.h); `binding` is a thin ctypes layer over it.  Importing
`lm_head_selected_amd.binding` fails loudly when the library is missing.
"""
__all__ = ["binding"]
