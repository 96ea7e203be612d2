"""CPU oracle of the DeepSeek-V4-Flash-style routed-MoE FFN layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls, links or executes anything in
this package: it is used by ``tests/``, by ``__graft_entry__.smoke()`` (to check one small GPU call)
and by the ``cpu_baseline`` leg of ``bench.py``. It shares no code with the HIP library; the two
meet only in the seeded input generator ``synth`` (which holds none of the layer's arithmetic).

Modules
-------
``formats``  exact decoders/encoders of E2M1, E8M0, E4M3 and bf16 (NumPy, fp64).
``moe``      the layer, step by step: router, activation QDQ, expert FFN (packed and decoded-BF16
             arms), shared FP8 expert, fixed-order combine. fp64 dot products of exactly decoded
             values, rounded once to bf16; the fp32 steps the pages fix are emulated in fp32.
``exact``    an independent pure-Python brute force (integer arithmetic) of the same layer for tiny
             shapes, used to pin ``moe``.

Every function cites the passage it follows: the page
"Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Official semantics" and section 4 "Kernel
contract"; the paper "DeepSeek-V4-Flash on AMD gfx90a", section 6.1 for the E2M1 integer map.

Parity status: every function here is pinned by tests under ``tests/test_oracle_*.py`` (see each
function's docstring for its pin). The end-to-end layer at full size is pinned only through the
composition of pinned parts plus the brute-force agreement on tiny shapes.
"""
