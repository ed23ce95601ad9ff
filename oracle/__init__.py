"""fp64 CPU oracle of the MC-Sparse hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package.  It shares no
code, table or helper with the HIP path; both sides take their inputs from the
seeded generator in ``sparse_attention_diffusion_amd.workloads`` only.

Source for every definition: "MC-Sparse: Deconstructing and Closing the
Dense-Sparse Attention Gap in Diffusion Transformers" (agihunt.info summary of
arXiv 2610.06801), cited below by paragraph:

* "grouping paragraph"  - token-level KV picks gathered by index; PDDP cuts similar
  queries into groups of exactly C by principal-direction median splits.
* "selection paragraph" - per group, the K keys of largest summed attention weight,
  found by a two-pass kernel because flash attention hides the logits.
* "residual paragraph"  - the anchor stores dense minus sparse output; reuse steps
  add it to a fresh sparse call; groups, indices and residual refresh together.
* "gap paragraph"       - the discarded tail still carries weight (sparse softmax is
  renormalised over the kept keys, hence a residual exists).
* "limitations paragraph" - every anchor still runs full dense attention.

Every function says which readings it takes where the page is silent; the list of
readings is kept with the design notes of the repository.

Parity pins: every function here is checked against closed forms, library
routines or brute force in ``tests/test_oracle_*.py``; no function here is left
without such a pin.
"""
