"""MI355X (gfx950) pad-1 3x3 / 3x3x3 convolution with fused bias + ReLU / clamp epilogues.

A thin ctypes binding over the C ABI of libconv3x3.so (include/conv3x3.h): every function here
has the name of the C entry point it calls and only marshals arguments (device pointers, sizes,
the current HIP stream).  All arithmetic runs in the library's HIP kernels; there is no fallback.
"""
from .conv import (  # noqa: F401
    ABI_VERSION, ALGO_AUTO, ALGO_FUSED_HEAD, ALGO_MFMA, ALGO_SIMT, ALGO_SPLIT_HEAD, DTYPE_BF16, DTYPE_F16,
    EPI_CLAMP1, EPI_NONE, EPI_RELU, LAYOUT_CHANNELS_FIRST, LAYOUT_CHANNELS_LAST, ConvError,
    E_INVAL, E_LAUNCH, E_NODEVICE, E_UNSUPPORTED, E_WORKSPACE, OK, conv3x3_fwd,
    conv3x3_is_supported, conv3x3_select_algo, conv3x3x3_describe, conv3x3x3_fwd,
    conv3x3x3_fwd_noalloc, conv3x3x3_fwd_region, conv3x3x3_head_rgb8, conv3x3x3_is_supported,
    conv3x3x3_pack_weights,
    conv3x3x3_packed_weight_bytes, conv3x3x3_select_algo, conv3x3x3_workspace_bytes,
    conv_abi_version, conv_band_region, conv_calib_lds_dma, conv_calib_lds_read, conv_calib_mfma_bf16, conv_causal_region, conv_head_stencil, conv_head_temporal, conv_last_error, conv_out_size,
    conv_status_str, conv_video_rgb8, library, library_path)
