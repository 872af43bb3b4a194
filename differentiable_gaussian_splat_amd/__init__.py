"""MI355X-native tile-based 3D Gaussian splatting rasterizer (forward and backward).

The compute path is the HIP library ``libgsplat_hip.so`` (C ABI declared in
``include/gsplat.h``); :mod:`.raster` is its thin ctypes binding and
:mod:`.scenes` draws the seeded synthetic inputs. Importing this package loads
nothing: the library is opened on first use.
"""
__version__ = "0.1.0"
