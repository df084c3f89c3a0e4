"""MI355X-native Exact Flow Linear Attention (EFLA) hot path.

The kernels live in ``libefla.so`` (HIP for gfx950, C ABI in include/efla.h);
``efla`` is the thin ctypes binding, ``workloads`` the seeded input generators.
"""
from .efla import (EflaError, efla_chunk_fwd, efla_chunk_fwd_workspace_size,  # noqa: F401
                   efla_chunk_recurrence, efla_chunk_ut_transform, efla_coeff, efla_status_string,
                   efla_step, lib)
