"""DFlash block-diffusion drafting hot path for AMD Instinct MI355X (gfx950).

The compute lives in libdflash.so (HIP kernels behind the C ABI declared in
include/dflash.h).  ``binding`` mirrors that ABI one function per entry point;
``drafter.Drafter`` owns the device buffers of one handle.
"""
