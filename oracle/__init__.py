"""CPU oracle for the layer-streamed QLoRA step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation of what the streamed
step computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does.  It shares no code with the HIP library and imports nothing from the
package.

Streaming only changes when weights reach the device, not any value (page
"Soup ... radar note", section "In detail", reports zero difference against
the resident run), so the oracle is simply the un-streamed computation:
dequantise, run the decoder, back-propagate to the LoRA matrices.

Pins (what the oracle is checked against, in ``tests/test_oracle_*.py``):
  nf4.codebook      -- normal-CDF spacing of the levels (scipy ndtr), exact
                       +-1 ends and exact zero; values parity unpinned against
                       the pages, which print no table.
  nf4.quantize      -- exact-rational optimality of every chosen code, absmax
                       element maps to an end code, idempotence, zero blocks.
  nf4.dequant       -- exact product in float64 + independent integer rounding.
  nf4.double_quant  -- exact-rational nearest 8-bit code, group max -> 255, the
                       s/2 error bound, zero groups, and the 8B record size
                       against the pages' 3.60 GB / 32 layers.
  model.*           -- fp64 finite differences of the loss (LoRA A/B and the
                       embedded input), torch autograd on fp64, library
                       attention / cross-entropy, B = 0 identities, the
                       adapters-disabled reference pass, the DPO ln 2 closed
                       form.
  pref.head         -- closed forms where each sigmoid term is 1/2, ORPO odds
                       through p / (1 - p), float64 central differences of
                       every head (KTO with its reference point held).
  model.pref_step   -- float64 central differences of the step's LoRA
                       gradients per head, exact cancellation for chosen ==
                       rejected, the DPO head against the DPO step, KTO at
                       policy == reference.
  optim.adamw_step  -- torch.optim.AdamW in float64 over several steps (with and
                       without weight decay), the step-1 closed form, mirror
                       precision within float32 rounding of float64.
  model loss value  -- parity unpinned beyond the above: the pages print no
                       worked loss or gradient.
"""
