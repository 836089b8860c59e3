"""CPU oracle for the MT-NLG tensor-sliced decoder-layer shard and its Adam step.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 numpy/scipy
statement of what the GPU library computes. Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
it. The GPU library (``tensor_sliced_transformer_amd``) never imports, links or
calls anything here, and nothing here imports the GPU library: the two share no
code, constants or helpers. Inputs reach both sides from ``synth`` (seeded
random tensors only, none of the method's arithmetic).

Sources (cited by title and section; the pages carry no code):

* "Using DeepSpeed and Megatron to Train Megatron-Turing NLG 530B" -- Elamur
  Research summary page, sections "Summary" and "Key points" (dense
  left-to-right transformer; ~20 bytes/param mixed-precision Adam; gradient
  accumulation over 1920 micro-batches).
* "STRONGHOLD: Fast and Affordable Billion-scale Deep Learning Model Training"
  slide deck, slides 6-8 "Tensor (Intra-Layer) Model Parallelism" and the
  Megatron example (A split column-wise, Y = GeLU(XA); B split row-wise,
  Z = Dropout(YB); the conjugate operators f and g).
* jiqizhixin article on Megatron-Turing NLG (Chinese rendering of the
  NVIDIA/Microsoft MT-NLG blog), paragraph on the 3D-parallel system (8-way
  tensor slicing inside a node, 35-way pipeline, mixed precision, 105 layers,
  hidden 20480, 128 heads, throughput 126/121/113 TFLOP/s per GPU).

Where the pages are silent (LayerNorm placement and epsilon, the GeLU form,
biases, attention scale, head split, Adam details, clipping, loss scaling) the
readings taken are stated in the docstring of the function that uses them.

Modules:
  layer   -- LayerNorm, GeLU, causal attention, the two halves of a decoder
             layer shard (forward/backward), slicing of full parameters, the
             whole layer by summing slices.
  adam    -- fp32-gradient accumulation, global norm / clip / found-inf, and
             the Adam update with the bf16 weight copy.
  bf16    -- the oracle's own float -> bfloat16 round-to-nearest-even.
  pages   -- the pages' own arithmetic (parameter count, bytes/param,
             activation memory, throughput) for consistency pins.

Parity status: every function here is pinned by tests under tests/ against
closed forms, special cases, finite differences, brute force or the slicing
invariant; none is "parity unpinned" except the layer output values at MT-NLG
scale, which the pages do not print (the oracle is the definition there).
"""
