"""MI355X (gfx950) decoder-block training hot path.

The computation lives in the HIP library libgdb.so (C ABI: include/gdb.h);
`ops` binds each entry point under its own name, `stack.DecoderStack` runs a
whole training step through it, `workmodel` counts the algorithmic FLOPs and
bytes.  Importing this package does not load the library; the first call
through `ops` does, and fails loudly if it has not been built
(`python -m gpt_decoder_block_amd.build`).
"""
__all__ = ["ops", "stack", "workmodel", "build"]
