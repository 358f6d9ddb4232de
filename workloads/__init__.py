"""Synthetic DSA workloads: shapes of the measured/checked configurations
and the seeded input generators that both the HIP path and the CPU oracle
consume.  Nothing here computes any step of the method."""
from .configs import WORKLOADS, Workload, get  # noqa: F401
from .synth import make_inputs, make_scores  # noqa: F401
