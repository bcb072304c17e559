"""Seeded synthetic inputs (counter-based PRNG + workload builders).

Shared by the tests, the benchmark and the smoke check; it holds no
arithmetic of the RoPE / paged-store method and imports neither the HIP
library nor the CPU oracle."""
from . import prng, cases  # noqa: F401
