"""CPU oracle for the VeriCache draft/verify path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy implementation of what the path computes:
full-KV greedy decoding of a pre-norm Llama-style decoder, the two compressor
families (token dropping by observed attention, per-group low-bit
quantization), compressed-KV drafting, full-KV verification and the
accept-until-first-mismatch rule, and sampled decoding with speculative
rejection sampling.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library or its
Python binding; the only common dependency is ``synth`` (seeded inputs).

Sources (the pages are cited by title and section):
  [VC1] "VeriCache: Making Lossy KV Compression Exact" (devshah.ca), section
        "The Core Idea": draft x tokens with the compressed cache, one
        verification pass with the full cache giving x + 1 predictions,
        accept until the first mismatch, insert the correction, keep a
        bonus token when all drafts match; worked example (Draft/Verify/Emit).
  [VC2] "VeriCache Guide: Lossless Inference with Lossy KV Caches"
        (aifetchly), sections "The Uniform Compressor Interface" and
        "Implementing VeriCache in Python and PyTorch" (compress(full_k,
        full_v) -> (ck, cv); kept indices sorted ascending).
  [VC3] "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference"
        (estelledc study note), section "实践案例" case 1 (draft / verify /
        accept_prefix_until_first_mismatch / resume loop).
  [VC2] also "Mathematical Guarantee of Lossless Correctness" (speculative
        rejection sampling; ``sampling.py``, whose uniforms come from
        Philox4x64-10, Salmon et al., "Parallel Random Numbers: As Easy as
        1, 2, 3", SC 2011).
  [KV4] "KV Cache and Speculative Decoding" (corecocept), section
        "Autoregressive Decoding and the KV Cache" (cached K/V are legal
        because causal attention never changes past rows).

Parity status of each function is stated in its docstring; functions with no
independent pin say "parity unpinned".
"""
