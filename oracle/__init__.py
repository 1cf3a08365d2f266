"""CPU oracle for the stream-K GEMM / conv-wgrad engine.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package
``implicit_gemm_conv_dp_amd`` and its HIP library) may import, call or link
anything here.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.

What it computes, each a plain definition evaluated in float64 (or an integer
algorithm written out step by step):

* ``codecs``    -- fp16 / bf16 / OCP fp8 e4m3 decode and round-to-nearest-even
                   encode, from the IEEE-754 and OCP 8-bit floating point
                   format definitions.
* ``gemm``      -- ``R[m][n] = sA[m] * sB[n] * sum_k a(m,k) b(k,n)`` for the
                   rcr layout (row-major A, column-major B).
* ``wgrad``     -- the backward-weight convolution by its definition (NHWC
                   activations, KRSC filter gradient, grouped, strided, padded).
* ``conv``      -- the forward convolution and the input gradient (dgrad) by
                   their definitions, same layouts.
* ``partition`` -- the data-parallel + stream-K split of output tiles and MAC
                   iterations over a CTA pool, plus a brute-force invariant
                   checker.
* ``simulate``  -- an in-order workgroup dispatch model of the linear / tree
                   hand-off that reports the smallest resident capacity with
                   which a plan completes.

Pins: every function here is checked against facts fixed by the pages or by
mathematics in ``tests/test_oracle_*.py`` (marked ``not gpu``).  Nothing is
"parity unpinned" except the statement, recorded in the GEMM tests, that the
GPU's fp32 summation order is not reproduced bit for bit on random data (the
oracle is fp64; the bar there is the tolerance).
"""

from . import codecs, gemm, wgrad, conv, partition, simulate  # noqa: F401
