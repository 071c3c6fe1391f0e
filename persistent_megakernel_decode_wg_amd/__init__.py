"""Python binding of libmbk, the batch-1 persistent-megakernel decoder for MI355X.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libmbk.so`` (see ``include/mbk.h``).  PyTorch provides device
memory (tensors) and the current stream.  If the library has not been built
the import of ``Decoder`` fails loudly; there is no fallback path.
"""
from .binding import (  # noqa: F401
    MBK_ERR_ARG, MBK_ERR_HIP, MBK_ERR_RANGE, MBK_ERR_SIZE, MBK_ERR_STATE, MBK_ERR_TIMEOUT, MBK_ERR_UNSUPPORTED,
    MBK_LAUNCH_COOPERATIVE, MBK_LAUNCH_PLAIN, MBK_OK, MBK_SYNC_BARRIER, MBK_SYNC_DATAFLOW, MBK_TOKEN_PREV,
    MBK_WEIGHTS_BF16, MBK_WEIGHTS_FP8_E4M3, Decoder,
    MbkError, lib, lib_path)
