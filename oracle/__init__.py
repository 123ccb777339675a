"""fp64 CPU oracle for the denoise-step sampler hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.  The
product path (the HIP library and its Python binding) never imports it, and this package
never imports the product path: the two share no code.  Their only common input is the
seeded generator module ``denoise_step_sampler_amd.synth``, which holds no sampler
arithmetic.

What is computed, and where the pages define it:

* ``philox``      Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
                  "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), the noise source for
                  Gumbel-max sampling and uniform renoising.
* ``vocab_pass``  tied-unembedding logits, tempered softmax, entropy, argmax, Gumbel-max
                  sample and the self-conditioning expectation sum_v p_v E_v
                  (DiffusionGemma Technical Report part 2/6, sec. 3.2 eq. (6);
                  DiffusionGemma Explained, "Sampling" and "Self-conditioning").
* ``sampler``     entropy-bounded accept / uniform renoise / argmax-stability convergence
                  (Technical Report sec. 3.3; DiffusionGemma Explained, "Sampling";
                  vLLM blog "DiffusionGemma: the first dLLM natively supported in vLLM",
                  sampler section).
* ``q_sample``    closed-form forward corruption (Technical Report sec. 2.1.1 eq. (1);
                  DiffusionGemma-Lite DIFFUSION.html, forward process).

Every function is written from the definition, in fp64, with no blocking, fusion or
reordering beyond what the definition states.  Pins against closed forms, brute force and
published test vectors live in ``tests/test_oracle_*.py``.
"""
from . import philox, vocab_pass, sampler, q_sample  # noqa: F401
