"""CPU oracle of the WUSH-KV online path.  TEST INFRASTRUCTURE ONLY: imported by
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the
product package."""
from . import wushkv_ref, layout  # noqa: F401
