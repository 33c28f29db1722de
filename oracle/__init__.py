"""CPU oracle for the Stacked Target Cross Attention (STCA) forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path: its only common dependency is ``stca_inputs`` (seeded draws, no STCA
arithmetic).

* ``oracle.stca``  -- numpy float64, one function per equation of the method,
  written from the pages' statement of it (see the module docstring for the
  sources and the readings taken where the pages are garbled or silent).
* ``oracle.brute`` -- an independent pure-Python scalar-loop version of the
  same equations, for tiny sizes only; the tests pin ``oracle.stca`` to it.
* ``oracle.sl``    -- stochastic-length training batches (eqs. (15)-(17), temporal
  suffix selection, two-step batch load balancing) in integer numpy.
* ``oracle.litm``  -- local same-ID token merging of a history (TM20K's LITM): grouping
  in plain Python, merged rows as float64 sums.
* ``oracle.grad``  -- gradients of the forward (eqs. (2)-(8)) for an upstream dZ: the chain
  rule written out in float64, pinned by central finite differences of ``oracle.stca``.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(library routines, closed forms, invariants the pages state, brute force).
The conventions the pages leave open (no residuals, per-layer encode from raw
X, query FFN weights shared with the history FFN of the same layer, no
LayerNorm in the query update) are fixed readings, shared with the HIP path
by definition; no page prints a number that could pin them ("parity unpinned"
for those readings only).
"""
from . import brute, grad, litm, sl, stca

__all__ = ["stca", "brute", "sl", "litm", "grad"]
