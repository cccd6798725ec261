"""CPU oracle (test infrastructure only): see moe_oracle.py. Nothing on the GPU path may
import this package; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline do."""
