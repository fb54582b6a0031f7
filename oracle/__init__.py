"""CPU oracle for the Psi-Spec draft-and-verify decode step.

This package is TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``lossless_decoding_uno_amd``) never imports, calls or links anything here, and
nothing here imports the product path.  The two share no code; the only common
dependency is the seeded input generator package ``synth``, which holds no
arithmetic of the method.

What it follows (page titles and sections of the pages that describe the method,
"Unlocking Lossless Speedups in LLMs via Discrete Diffusion"):

* model forward, fp64 (``oracle.model``): a pre-norm decoder whose linears carry
  rank-r LoRA "diffusion weights"; the draft pass uses AR + LoRA weights and the
  verify pass uses the AR weights alone (picx.dev summary, "Methodology /
  Architecture: Diffusion-Augmented LLMs"; paperglide reader, "The Uno Framework",
  "Sampler Extensions");
* draft block, verify block, accept, residual/bonus token, commit
  (``oracle.spec``): paperglide reader, "The Psi-Speculative Sampler" and
  "Sampler Extensions"; picx.dev summary, "Psi-Speculative Sampler";
* the integer-weight categorical sampler and the canonical exponential
  (``oracle.canonical``) and the Philox4x64-10 counter generator
  (``oracle.philox``).  The pages fix neither; they make "bit-exact" well defined
  and are this project's own reading, documented beside each function.

Every floating-point step of the model is fp64.  The sampler works in fp32 where
a float decides an integer (the pages do not fix that precision; fp32 is the
precision of the logits both sides hand to the sampler), and in exact integers
everywhere else.

Parity status: see each module's header.  ``oracle.model`` logit values are
"parity unpinned" against the pages (the pages print no logits); they are pinned
structurally (dense-merge LoRA identity, B = 0 reduction, cached == uncached,
independent torch-CPU routines for attention, RMSNorm, SiLU).
"""
