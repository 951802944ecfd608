"""MI355X-native fused W-way reduce + residual add + RMSNorm (``libarrms``).

The compute lives in ``libarrms.so`` (hand-written HIP kernels for gfx950 behind
a C ABI, declared in ``include/arrms.h``).  ``tp_all_reduce_amd.arrms`` is the
thin ctypes binding with the same names; PyTorch only provides device memory
and streams.  The binding loads the library on first use and raises if it has
not been built: there is no CPU fallback.
"""

_BINDING_NAMES = (
    "ar_rms_plan", "ar_rms_plan_destroy", "ar_rms_plan_kernel", "ar_rms_one_stage",
    "ar_rms_run", "ar_rms_quant_run", "ar_qknorm_run", "ar_rms_last_error",
    "Plan", "ArrmsError", "OK", "EINVAL", "ENOTSUP", "EHIP", "ENOMEM",
    "BF16", "FP16", "FORCE_ROW", "FORCE_SPLIT", "ROUND_REDUCED", "KERNEL_ROW", "KERNEL_SPLIT",
    "fused_allreduce_rms_norm", "fused_allreduce_rms_norm_quant", "fused_qk_norm",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import arrms
        return getattr(arrms, name)
    raise AttributeError(name)
