"""CPU oracle for position-independent KV splicing.  Test infrastructure only:
imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg."""
from .pic_oracle import *  # noqa: F401,F403
