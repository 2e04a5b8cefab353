"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

Holds random draws, document-length recipes and tensor layouts only: no step of the
MSA method is computed here.  Both the HIP path and the CPU oracle consume what this
package produces; neither imports the other.
"""
from .workloads import *  # noqa: F401,F403
