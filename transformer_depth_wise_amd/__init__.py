"""MI355X-native depth-routing read of Attention Residuals (AttnRes / MHAR /
LR-AttnRes): HIP kernels for gfx950 behind the C ABI in include/attnres.h,
with a thin ctypes binding (``transformer_depth_wise_amd.attnres``)."""

__all__ = ["attnres"]
