"""CPU oracle for the NF4 + double-quantized QLoRA frozen-base linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy (float64 / exact IEEE float32 steps) statement of what the GPU path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product library
(``bit_nf4_quantized_qlora_amd``) never imports, links or calls anything in
here, and nothing in here imports the product: the two share no code.

Modules
-------
``nf4_dq``   the storage encoding: NF4 codebook, blockwise absmax + nearest
             code, double quantization of the block constants, dequantization
             to BF16, and the bits-per-weight arithmetic.
``linear``   the fp64 forward / backward of the frozen-base linear layer with
             its LoRA adapters.
``merge``    folding trained adapters into the base (W_hat + s B A) and
             re-encoding the result.
``adamw``    one AdamW step on the adapters (the paged optimizer's update).
``mlp``      the gate / up / SwiGLU / down block around the linears.
``attention`` the causal attention core between the q/k/v and o projections.
``layer``    the decoder layer: the seven adapted projections, attention,
             SwiGLU and the two residual additions.
"""
