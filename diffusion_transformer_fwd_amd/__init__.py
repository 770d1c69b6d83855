"""MI355X-native FLUX.2-[klein]-style DiT denoise step.

The compute path is the C-ABI library ``libdit.so`` (hand-written HIP for
gfx950); ``diffusion_transformer_fwd_amd.dit`` is its thin ctypes binding.
``synth`` draws seeded synthetic inputs. Importing this package does not load
the library; the binding loads it on first use and raises if it is missing.
"""
__all__ = ["synth"]
