"""CPU oracle of the Lighthouse attention layer.  Test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the library."""
from . import lighthouse  # noqa: F401
