"""CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's cpu_baseline leg may import this
package.  It shares no code with the HIP path; the seeded input generator is
the only module both sides use.

Contents (each function cites the passage it follows):
* seq        -- plain fp64 sequential recurrence (C, OpenMP), the reference,
                and its gradient (reverse-mode chain rule, token by token).
* gate       -- fp64 decay gate g = gmin * sigmoid(exp(A) * z) and the
                chunk-local inclusive cumulative sum of g.
* chunkwise  -- fp64 numpy chunkwise-parallel form and its gradient
                (independent checks of seq).
* brute      -- mpmath product-of-transitions form for tiny inputs.

Parity status: every function here is pinned by tests/test_oracle_*.py
(the gradient by finite differences of the forward, tests/test_oracle_bwd.py)
(brute force, closed forms, invariants); see the module headers.
"""
