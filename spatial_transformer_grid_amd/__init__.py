"""spatial_transformer_grid_amd -- MI355X-native spatial-transformer sampler.

Python face of libgsample (include/gsample.h): the grid generator
(AffineGrid), the 2D/3D sampler (GridSample), their fused composition and
Resize, all computed by hand-written HIP kernels for gfx950.  Tensors are
torch GPU tensors; torch supplies device memory and streams only.

    from spatial_transformer_grid_amd import affine_grid, grid_sample
    grid = affine_grid(theta, (N, C, H, W), align_corners=0)
    Y = grid_sample(X, grid, mode="linear", padding_mode="zeros")
"""

from ._binding import (  # noqa: F401
    GS_BF16,
    GS_F16,
    GS_F32,
    GSError,
    LIB_PATH,
    MODES,
    PADDINGS,
    affine_grid,
    affine_grid_sample_fused,
    grid_sample,
    lib,
    resize,
    resize_output_shape,
    resize_to,
)

__all__ = ["affine_grid", "grid_sample", "affine_grid_sample_fused", "resize",
           "resize_output_shape", "resize_to", "GSError", "lib"]
