"""CPU oracle for the flat-buffer Muon step -- TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``newton_schulz_flat_amd``) never imports, links or calls anything here, and
nothing here imports the product path: the two share no code.

Modules
-------
muon_oracle
    fp64 NumPy implementation of one Muon step over flat buffers.  The step
    follows the "Opt step" pseudocode of the page "Add initial Muon+M-FSDPv2
    implementation" (Megatron-LM PR #6425), steps 1, 2, 4 and 6, and the
    methods ``_compute_momentum_inputs``, ``_orthogonalize_updates`` and
    ``_apply_local_updates`` of ``FsdpMuon`` on the page
    "core.distributed.fsdp.src.megatron_fsdp.experimental.muon".
same_order
    float32 NumPy reference of the two elementwise phases (momentum/Nesterov
    input, decay + apply) that performs every IEEE operation in the same order
    as the device kernels, so that device results can be compared bit for bit.

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` against closed forms, invariants and brute force
(see each function's docstring for what pins it).  Two readings of the pages
(SGD-style momentum, decoupled weight decay) are choices the pages leave open;
they are pinned against their own closed forms but not against the pages.
"""
