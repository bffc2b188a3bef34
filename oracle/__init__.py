"""CPU oracle for the packed low-bit GEMV/GEMM path.

TEST INFRASTRUCTURE, NOT PRODUCT.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It
shares no code with the HIP library (no headers, helpers, tables or constant
generators) and never imports it.

* ``fp``     exact fp16 / bf16 bit-pattern decoding to float64
* ``layout`` packed sizes, the per-weight address of every sign / code / trit
             in the device layout, pack and unpack
* ``ref``    y = X (t*s)^T and a = |X| |t*s|^T in float64, acceptance bound
* ``mlx``    MLX's affine 1-bit g128 weights (a * q + b) and their exact
             Binary g128 form

Pins against something other than itself live in ``tests/test_oracle_*.py``.
Every function here is pinned; none is "parity unpinned".
"""
from . import fp, layout, mlx, ref  # noqa: F401
