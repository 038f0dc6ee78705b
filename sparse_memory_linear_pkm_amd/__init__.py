"""Sparse Delta Memory hot path on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libsdm.so`` (C ABI in ``include/sdm.h``).  The
binding only marshals arguments: torch tensors provide device memory and
streams, and every step of the path runs in the HIP kernels of the library.
If the library has not been built, the first call raises ImportError; there
is no fallback implementation.
"""
from .binding import (SDM_OK, SDM_ERR_INVALID_ARG, SDM_ERR_UNSUPPORTED, SDM_ERR_HIP, SDM_F32,
                      SDM_BF16, SDM_NOALLOC_SCRATCH_BYTES, SdmDims, SdmError, dims_from, lib_path, load_library,
                      sdm_state_init, sdm_pkm_address, sdm_pkm_address_overlapped, sdm_scan_workspace_size, sdm_scan_forward,
                      sdm_decode_step, sdm_cow_bitmap_bytes, sdm_cow_reset, sdm_decode_step_cow,
                      sdm_cow_materialize, sdm_gates, sdm_output_norm_gate, sdm_gdn_dense_forward,
                      sdm_scan_forward_save, sdm_scan_backward, sdm_scan_backward_workspace_size, scan_forward_save,
                      scan_backward,
                      sdm_scan_forward_noalloc, scan_forward_noalloc, sdm_scan_forward_gated,
                      sdm_address_backward, sdm_address_backward_workspace_size, address_backward,
                      sdm_gates_backward, sdm_gates_backward_workspace_size, sdm_output_norm_gate_backward,
                      sdm_output_norm_gate_backward_workspace_size, gates_backward, output_norm_gate_backward,
                      sdm_status_string,
                      sdm_last_error, sdm_version, state_init, pkm_address, scan_forward, decode_step,
                      gates, output_norm_gate, gdn_dense_forward)
from .pipeline import prefill_chunks

__all__ = [n for n in dir() if n.startswith(("sdm_", "SDM_", "Sdm")) or n in (
    "dims_from", "lib_path", "load_library", "state_init", "pkm_address", "scan_forward",
    "decode_step", "gates", "output_norm_gate", "gdn_dense_forward", "scan_forward_save", "scan_backward",
    "address_backward", "gates_backward", "output_norm_gate_backward", "scan_forward_noalloc", "prefill_chunks")]
