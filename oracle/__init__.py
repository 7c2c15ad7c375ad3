"""CPU oracle of the codebook-TTS decode path (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
shares no code, table or constant generator with it.  Its only shared input is
the seeded generator in ``synthetic``.

Parity status of each function (what pins it, in the CPU test suite):
* numerics.round_bf16          -- bit-level agreement with torch.bfloat16
* numerics.e4m3_*              -- exhaustive round trip of all 256 codes,
                                  every midpoint (ties to even), saturation,
                                  agreement with torch.float8_e4m3fn
* numerics.rmsnorm             -- closed form of the output rms, scale invariance
* numerics.rope                -- norm preservation, identity at p = 0,
                                  relative-position property, hd = 2 closed form
* numerics.attention_one       -- L = 1 gives v, equal keys give mean(V),
                                  split-K/LSE combine equals the one-pass form
* model.OracleModel            -- batched prefill equals step-by-step decode
                                  (causal-mask equivalence), GQA equals MHA with
                                  repeated K/V; mode E equals a torch library
                                  formulation (F.linear, F.rms_norm, complex RoPE,
                                  scaled_dot_product_attention) to 1e-10; mode S
                                  (BF16 and FP8) equals the same formulation with
                                  torch.bfloat16 / torch.float8_e4m3fn casts at
                                  the storage points to 1e-10 (rounding placement
                                  and the scale of each activation site);
                                  whole-model values beyond these: parity
                                  unpinned (no page prints a worked example)
* delay.*                      -- brute-force enumeration over every EOC step
                                  against an independent restatement; undelay
                                  inverts delay
* sampling.philox4x32_10       -- the generator's published known-answer vectors;
                                  array form equals the scalar form
* sampling.uniform / draw      -- 60000 draws per case follow torch.softmax over the
                                  allowed ids (chi-square, three temperatures, EOS
                                  allowed or not); a hand-worked inversion including
                                  an exact boundary; tiny-temperature argmax, NaN and
                                  single-id limits; the delay rule's forced codes
* model.calibrate              -- the per-site maxima equal those the torch
                                  formulation records on the same rows before
                                  rounding (1e-12; float32 scales bit-equal), and
                                  the quantised site maximum lands exactly on 448
"""
