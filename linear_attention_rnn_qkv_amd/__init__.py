"""MI355X-native (gfx950) forward layer core of Gated DeltaNet.

The compute path is the C-ABI library ``libgdn.so`` (hand-written HIP kernels);
``linear_attention_rnn_qkv_amd.gdn`` is its thin ctypes binding. Importing the
package itself loads nothing, so the seeded input generator ``synth`` can be
used without a GPU.
"""
__all__ = ["gdn", "synth"]
