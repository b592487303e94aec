"""Seeded synthetic inputs (canonical GALE format), shared by the oracle and the GPU harness."""
from .gen import *  # noqa: F401,F403
from .gen import n_outliers, CanonicalMatrix  # noqa: F401
