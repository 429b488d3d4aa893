"""MI355X (gfx950) GPT-2 Pre-LN forward: HIP kernels behind a small C ABI.

    from gpt_pre_ln_amd.model import GPT2     # torch-managed device buffers
    from gpt_pre_ln_amd import binding        # the raw C ABI (ctypes)

Importing the package loads nothing; the library is loaded on first use and
fails loudly when it has not been built (python gpt_pre_ln_amd/build.py).
"""
