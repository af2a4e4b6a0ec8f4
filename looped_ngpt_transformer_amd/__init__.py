"""Looped normalized-GPT forward pass on MI355X (gfx950).

The compute path is the HIP library libdory.so (C ABI: include/dory.h); `dory` is its
ctypes binding and `runtime` allocates device memory for it with torch.
"""
