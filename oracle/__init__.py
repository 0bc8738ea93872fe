"""Plain CPU oracle for NVFP4 quantize + block-scaled GEMM.

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the HIP library or its binding."""
