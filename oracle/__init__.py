"""fp64 CPU oracle for the sparse MoE layer forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the library. It shares no
code with the HIP path.
"""
