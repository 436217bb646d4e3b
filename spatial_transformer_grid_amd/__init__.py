"""spatial_transformer_grid_amd -- MI355X-native spatial-transformer sampler.

Python face of libgsample (include/gsample.h): the grid generator
(AffineGrid), the sampler (GridSample) of any rank and type, their fused
composition, Resize and DeformConv, all computed by hand-written HIP kernels
for gfx950.  Tensors are
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
    deform_conv,
    deform_conv_noalloc,
    deform_conv_output_shape,
    deform_conv_workspace_size,
    dtype_code,
    grid_sample,
    grid_sample_2d_workspace_size,
    lib,
    resize,
    resize_output_shape,
    resize_to,
)

__all__ = ["affine_grid", "grid_sample", "affine_grid_sample_fused", "resize",
           "resize_output_shape", "resize_to", "deform_conv", "deform_conv_noalloc",
           "deform_conv_output_shape",
           "deform_conv_workspace_size", "dtype_code", "grid_sample_2d_workspace_size",
           "GSError", "lib"]
