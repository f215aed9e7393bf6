"""MI355X (gfx950) tree-drafting hot path: block-diffusion drafter logits to
budget-optimal candidate trees (BASTION) and latent-mixture chain scores
(DBlast), as a C-ABI library (libbastion.so) with a thin Python binding.

    from block_diffusion_tree_amd import binding   # GPU entry points
    from block_diffusion_tree_amd import synth     # seeded synthetic inputs
"""
