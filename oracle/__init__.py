"""CPU oracle (test infrastructure only): the plain definition of query-aware
sparse paged decode that the HIP library is checked against. Only tests, the
package smoke check and the benchmark's CPU-baseline leg import it."""
from .qsa_oracle import *  # noqa: F401,F403
