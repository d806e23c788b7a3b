"""Oracle for the STEPQuant quantized gated-delta state step: plain, slow, float64, CPU.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library and its Python binding) never
calls it and shares no code with it; the only module both sides use is
``workloads`` (seeded random inputs, no arithmetic of the method).

Sources.  The method is described on the STEPQuant pages (Yao et al., 2026,
"STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent State
Quantization"): the hyper.ai summary (section 方法 / Method), the rcap.io post
(the decode-step pseudocode and the "Temporal" and "Spatial" paragraphs), and
the aiany.app summary ("Key method").  Each function cites the passage it
follows.  Where the pages leave a step open, the reading taken is stated in the
docstring.

Modules
-------
numerics    binary16 rounding written from the format's definition
recurrence  gated delta update and readout
quant       dual-axis quantizer / dequantizer and the uniform INT8 per-row comparator
step        one packed decode step (dequantize -> update -> readout -> requantize)
planner     lifetime-aware bit allocation, pivots, distortion, impact scores
"""
