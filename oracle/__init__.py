"""Oracle of the TTS backbone hot path: plain fp64 CPU code, test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
"""
