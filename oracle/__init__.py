"""CPU oracle (test infrastructure only): a plain, slow implementation of the balanced
expert-parallel hot path, used by the tests, the smoke check and the benchmark's CPU
baseline, and by nothing else."""

from . import moonep_oracle  # noqa: F401
