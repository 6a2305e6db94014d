"""CPU oracle for the delta-W4A4 linear layer — test infrastructure only.

Only the test-suite, the package's smoke check and the CPU-baseline leg of
the benchmark may import or run anything in this package.  The product path
(the HIP library and its Python binding) never touches it, and it never
touches the product path: the two share no code, constants or tables.  Inputs
come from the seeded generators in `w4a4_quantized_linear_cube_amd.synth`,
which hold none of the method's arithmetic.

What it computes is the layer of the DeltaQuant notes ("DeltaQuant: 4-bit
Video Diffusion Models with Spatiotemporal Delta Smoothing", papernotes.org,
CVPR 2026), section 方法详解:
  * 关键设计 2: cut the (T, H, W) token grid into non-overlapping t*h*w cubes;
  * 关键设计 3: core = mean of a cube's tokens, delta = token - core
    (the core/delta equation);
  * 关键设计 4: core in FP8, delta in FP4, both times a 4-bit weight, with the
    weight split W = L1 L2 + R (the three-term equation) and the quantizer
    Q(X) = round(X / s) s, s = max|X| / q_max, q_max = 6 for 4-bit floats;
  * 损失函数/训练策略 (the implementation paragraph): FP8 cores, 4-bit
    weights and deltas, a low-rank branch of rank r.

Plain numpy, fp64 wherever a sum or product is formed, fp32 only where the
readings below fix fp32.  Readings taken where the pages are silent:
  R1  partial cubes at the high end of an axis are clipped; the mean is over
      the tokens present;
  R2  tokens are flattened row-major (T, H, W); a cube's tokens are taken in
      lexicographic (dt, dh, dw) order;
  R3  the core is an fp32 sum in that order, in blocks of 64 tokens (block
      partials summed in block order), divided by the count with one IEEE
      round-to-nearest-even division;
  R4  delta is taken against the unquantised fp32 core, delta = fl32(x - core);
  R5  s is the smallest power of two 2^e with max|X| <= q_max 2^e (never
      clips), e clamped to [-127, 127] and stored as an E8M0 code e + 127;
      groups are 32 consecutive channels (MX block format);
  R6  q_max = 448 for FP8 (OCP E4M3, max finite value);
  R7  "round" is round-to-nearest, ties to the even code; signs are kept, so
      negative values that round to zero give -0;
  R8  the core term multiplies Q4(R), not Q4(W), when the low-rank branch is on;
  R9  L1 = U_r sqrt(S_r), L2 = sqrt(S_r) V_r^T, each rounded to bf16, and R is
      formed from the rounded factors: R = fl32(W - L1 L2), the product summed
      in fp64 in rank order;
  R10 the low-rank branch is U = bf16(bf16(X) L1), then U L2, output fp32.
"""
