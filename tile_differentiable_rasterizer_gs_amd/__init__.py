"""MI355X-native forward 3D Gaussian-splatting rasterizer.

The compute path is the HIP library `libgsrast.so` (C ABI in include/gsrast.h);
`binding` marshals torch tensors into it.  `scenes` draws seeded synthetic
inputs.  Importing the package loads nothing: `Rasterizer` loads the library on
first use and raises if it is not built.
"""

__all__ = ["Rasterizer"]


def __getattr__(name):
    if name == "Rasterizer":
        import importlib

        return importlib.import_module(".binding", __name__).Rasterizer
    raise AttributeError(name)
