"""Independent fp64 CPU oracle for the link step.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import, call or execute anything in this
package. The product (position_independent_kv_legolink_amd) never imports it
and shares no code with it.

    plan.py       row selection, absolute positions, page ownership
    link.py       merged cache of a request and the link attention call
    attention.c   fp64 causal RoPE attention with explicit loops
    native.py     gcc build + ctypes loader for attention.c
"""
