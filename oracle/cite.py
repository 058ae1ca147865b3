"""Citation keys used in the oracle's docstrings.

The pages are public web articles on block-scaled FP4; a citation names the page
and the section (or table) on it.

  [V41-NVFP4]   "DeepSeek-V4.1-Flash-NVFP4" explainer (discosf.com news 5859265)
                  s1  why the 552B MoE needs NVFP4 (lossless MX->NV remap claim)
                  s2  NVFP4 format breakdown (E2M1 table, two-level scales,
                      group size 16, fp4_gemm_kernel description)
                  s3  which layers are quantized (routed experts w1/w2/w3;
                      Engram tables to MXFP4 with 32-element UE8M0 blocks)
                  s4  Model Optimizer and lossless conversion (activation scales
                      are calibrated; weights lossless != outputs identical)
                  s6  repository files (convert.py E2M1->E4M3 remap)
  [V4-ARCH]     "DeepSeek-V4" architecture article (cf-1.com news 2962809)
                  s6.3 FP4 QAT (1x32 tiles, FP4->FP8 lossless dequant, STE)
                  s2   model family (384 routed experts, 6 active)
                  s5.1 Muon (SwiGLU named), s6.1 wave-based EP dispatch/combine
  [V4-QAT]      "DeepSeek-V4 FP4 quantization-aware training" article
                (hotelren.com news 2972295)
                  s2.1 MXFP4 dynamic block scaling, E4M3 max 448
                  s3.1 QAT MoE snippet (top-k routing), s3.2 code stream + scale
                  array weight layout, s4.2 FP4->FP8 lossless dequant
  [R1-FP4]      "nvidia/DeepSeek-R1-FP4 on B200" article (cf-1.com news 2988385)
                  s2.3 weight_scale tensors next to the weights
  [FP4-101]     generic "what is an FP4 model" explainer (idctop.com)
                  s1 sign / exponent / mantissa split of a 4-bit float
"""
