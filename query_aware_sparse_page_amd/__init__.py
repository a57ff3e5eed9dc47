"""query-aware sparse paged decode for MI355X: the libqsa HIP library and its
Python binding. Importing the package loads nothing; the binding loads
libqsa.so on first use and raises if it has not been built."""
from . import qsa  # noqa: F401

__all__ = ["qsa"]
