"""Tile rasterizer for point primitives on AMD MI355X (gfx950).

The compute path is libsplat.so (HIP kernels behind a C ABI, include/splat.h);
`_lib` binds it with ctypes and `raster.Rasterizer` manages device buffers.
`scenes` draws the seeded synthetic inputs. Submodules are imported on use.
"""
__all__ = ["scenes", "raster", "build"]
