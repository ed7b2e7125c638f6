"""Plain fp64 CPU oracle for the routed Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check and
the CPU-baseline leg of the benchmark use it.  It shares no code, tables or
helpers with the HIP library; it reads only the seeded inputs produced by the
``synth`` generator module.

Every function is written for a reader checking it against the FreeToken
pages by eye: no blocking, fusion or reordering beyond the plain definition.

Modules
-------
formats  BF16 and MXFP4 (e2m1 codes + e8m0 scale per 32) encode / decode
layer    router softmax + top-k, SwiGLU expert FFN, weighted combine,
         exact merge of two partial sums
cache    global LRU expert-cache simulation and the q* miss split

Parity status (what pins each function) is listed in each module header.
Functions whose result is not pinned by the pages or by mathematics say
"parity unpinned" there.
"""
