"""CPU oracle for exact attention: the forward pass and its gradients.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
C ABI or the Python binding in ``exact_attention_33_amd``) imports, calls or
links anything in this package.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.

Modules
-------
``attention``  the definition, written out plainly in fp64: materialise the
               scaled score matrix, mask it, three-pass safe softmax, multiply
               by V, log-sum-exp.  This is what the GPU path is compared with.
``backward``   the gradients dQ, dK, dV and the row statistic D, written out
               plainly in fp64 from the chain rule and the softmax Jacobian
               (every matrix of a head materialised).  What the GPU backward
               is compared with.
``streamed``   self-test helpers: the streamed forms the pages derive (online
               softmax in blocks, the per-key recurrence, the tiled forward,
               the split-and-merge of partial states).  They are checked
               against ``attention`` and against the printed numbers; they are
               never used for GPU parity.
``counting``   the HBM-byte / FLOP counting model of the explainer page, as
               closed forms.

Parity status per function: every public function here is pinned by a
``-m "not gpu"`` test against values or identities that the pages or the
mathematics fix (see ``tests/test_oracle_pins.py`` and
``tests/test_counting_model.py``; the backward by central finite
differences, the D shortcut identity, fp64 autograd and closed-form special
cases in ``tests/test_oracle_bwd.py``), except the bf16 tolerance, which the pages
do not address (they work in fp32/fp64 only).
"""
