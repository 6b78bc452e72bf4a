"""In-Place TTT fast-weight gated-MLP prefill on AMD Instinct MI355X (gfx950).

A thin ctypes binding over libttt_layer.so, whose C ABI is include/ttt.h.
PyTorch supplies device memory and the stream; every step of the layer runs
in the library's HIP kernels. There is no fallback: if the library is not
built, or a call fails, an exception is raised.

    O, W_final = layer_forward(H, X0, Wg, Wu, W_down0, conv_taps, W_target,
                               eta, chunk)
    grads = layer_backward(H, X0, Wg, Wu, W_down0, conv_taps, W_target,
                           eta, chunk, dO)
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    TTTError,
    backward_saved_workspace_size,
    backward_workspace_size,
    clipped_workspace_size,
    continue_workspace_size,
    copy_calibration,
    decode_begin,
    decode_state_size,
    decode_step,
    gated_activation,
    layer_backward,
    layer_forward,
    layer_forward_continue,
    layer_forward_packed,
    layer_forward_train,
    lib,
    lm_target,
    make_desc,
    packed_tables,
    packed_workspace_size,
    profile_enable,
    profile_read,
    train_workspace_size,
    workspace_size,
)

__all__ = ["layer_forward", "layer_forward_packed", "packed_workspace_size", "packed_tables",
           "layer_forward_continue", "continue_workspace_size", "clipped_workspace_size",
           "decode_state_size", "decode_begin", "decode_step",
           "gated_activation", "lm_target", "workspace_size",
           "layer_backward", "backward_workspace_size", "layer_forward_train",
           "train_workspace_size", "backward_saved_workspace_size",
           "copy_calibration",
           "make_desc", "profile_enable", "profile_read", "TTTError", "lib",
           "LIB_PATH"]
