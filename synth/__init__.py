"""Seeded synthetic workloads (configs and input generators); no step of the method lives here."""
from . import configs, inputs  # noqa: F401
