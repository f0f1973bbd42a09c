"""CPU oracle for the INT4 group-128 top-k MoE SwiGLU FFN forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, links or executes anything in this package; only the
test suite, the smoke check and the CPU-baseline leg of the benchmark do.  It
shares no code with the GPU path: no kernels, headers, helpers, tables or
constant generators.

Everything here is plain, slow and written to be checked by eye against the
pages it follows: NumPy in float64 for real arithmetic and int64 for integers,
with every rounding step of the method stated explicitly (float32 where the
method itself computes in float32, binary16 where it stores binary16).

Pages cited (by title; sections as printed on each page):

* "高效大语言模型推理实践：INT4量化与MoE架构的融合探索" (zingnex forum
  thread on the Efficient-LLM-Inference project) -- INT4 group quantisation
  with per-group scales; MoE slice mode.
* "Practical Exploration of Efficient Large Language Model Inference:
  Integration of INT4 Quantization and MoE Architecture" (English summary of
  the same project).
* "从FP32到INT4：大语言模型量化压缩实战指南" (practical FP32->INT4 guide) --
  §1.3 group-wise quantisation (group 128, per-group min/max scale, zero point
  only when asymmetric).
* "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" (W4A8 route for MoE
  inference) -- §2.3 the three-step W4A8 pipeline, §3.1 per-token activation
  quantisation, §3.2 router kept in floating point and the shared expert.
* "大模型之Dense、MoE与量化" (Dense, MoE and quantisation) -- MoE section:
  a Linear router scores experts, a few are picked, their outputs are
  combined in proportion to the scores; shared experts see every token.

Modules:

* ``quant``   -- symmetric / asymmetric INT4 g128 quantisation, nibble packing.
* ``layout``  -- the device tile layout, re-derived from its written spec.
* ``router``  -- fp64 router logits, top-k selection rule, renormalised weights.
* ``permute`` -- group-by-expert permutation (counts, offsets, perm, inv).
* ``ffn``     -- fp64 W4A16 and W4A8 FFN / MoE forward, per-token INT8
  activation quantisation, the INT32 group accumulators.
* ``lora``    -- LoRA-mode experts: low-rank adapters on the frozen INT4 dense FFN.

Parity status of each function is listed in its docstring ("pinned by" /
"parity unpinned").
"""
