"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark."""
from .dit import WORKLOADS, Workload, make_inputs, random_uniform_inputs, varying_need_inputs  # noqa: F401
