/*
 * foamd.h -- C ABI of the MI355X (gfx950) fused low-precision optimizer step.
 *
 * The library implements the optimizer step described on the FlashOptim
 * pages: parameters held as a 16-bit downcast weight theta' plus an N-bit
 * ULP-normalised error-correction code (ECC), optimizer states held as
 * companded 8-bit codes with one 16-bit scale per 32 elements, and fused
 * AdamW / momentum-SGD updates over lists of such tensors.
 *
 * Sources (titles and sections of the pages):
 *   [SPLIT]  Davis Blalock's FlashOptim thread, posts on weight splitting and
 *            on what the ECC bits hold; blog "FlashOptim: Breaking the Memory
 *            Wall with 24-bit Weights and Companded States", Methodology
 *            section 1 (ULP-based Weight Splitting).
 *   [STATE]  Same thread, posts on 8-bit codes with a 16-bit scale per 32
 *            elements and on companding; same blog, Methodology section 2
 *            (Companded Quantization) and Critical Insight.
 *   [UPDATE] Same thread, posts on computing the same updates as the usual
 *            optimizers, on gradients kept in backward precision and on
 *            gradient release; same blog, Conclusion & Perspective (drop-in
 *            torch.optim replacements).
 *   [LOWER]  Same blog, Conclusion & Perspective (Future Outlook): states
 *            below 8 bits as the next step, with no transform given; the
 *            4-bit codec keeps the 8-bit one's blocks, scales and companders.
 *
 * Numerical definitions.  The pages leave rounding modes, operation order,
 * scale format and compander formulas open; this library fixes them as
 * follows.  RN(.) is one IEEE binary32 rounding to nearest even; every
 * division and square root is the correctly rounded IEEE operation (the
 * kernels reach it through exact fast sequences, with IEEE fallbacks).
 *   Split: theta' = x rounded to the 16-bit format to nearest, ties away from
 *     zero; ECC = round_half_even((|x| - |theta'|) * 2^N / spacing), with the
 *     format's spacing on x's side of theta' (half the spacing above, below a
 *     power of two above the smallest normal), clamped to the N-bit range.
 *     NaN -> quiet NaN with ECC 0, +-Inf -> +-Inf with ECC 0, finite values
 *     past the format's range saturate to +-max with the ECC clamped.
 *   Blocks: 32 consecutive elements; the last block of a tensor holds n mod 32
 *     elements.  Scale = the smallest binary16 >= the block's maximum
 *     (momentum: max|m|; variance: RN(sqrt(max v))), saturating at 65504; the
 *     maximum ignores NaN elements, so a block whose valid elements are all
 *     NaN gets a NaN scale.
 *   Momentum codes (int8, [-127, 127]), companded: z = RN(m / s),
 *     q = sign(z) * round_half_even(127 * phi(min(|z|, 1))) with
 *     phi(a) = 2a / (1 + a), the rounding exact for the float z; decode
 *     RN(s * RN(q / (254 - |q|))) (code -128 decodes as -127).  Linear:
 *     q = clamp(rne(RN(127 * RN(m / s))), -127, 127); decode RN(D * q), D = RN(s / 127).
 *   Variance codes (uint8), companded: q = clamp(rne(RN(255 * RN(RN(sqrt(v)) / s))),
 *     0, 255); decode t = RN(D * q), D = RN(s / 255), v = RN(t * t).  Linear:
 *     q = clamp(rne(RN(255 * RN(v / RN(s * s)))), 0, 255); decode RN(D * q),
 *     D = RN(RN(s * s) / 255).
 *   4-bit companded codes [LOWER] (FO_COMPANDED4): as the companded codes
 *     with 7 for 127 (momentum codes in [-7, 7], decode RN(s * RN(q / (14 - |q|))),
 *     the pattern -8 decodes as -7) and 15 for 255 (variance codes in [0, 15],
 *     D = RN(s / 15)).  Two codes per byte: element 2i in the low nibble,
 *     2i+1 in the high one, momentum codes in 4-bit two's complement; a code
 *     array holds ceil(n/2) bytes and an odd n leaves the last high nibble 0.
 *   bfloat16 block scales [STATE] (FO_COMPANDED_BF16SCALE): the companded
 *     8-bit codes with scale = the smallest bfloat16 >= the block's maximum
 *     (subnormal values included), saturating at the largest finite
 *     bfloat16 (0x7F7F); NaN maximum -> 0x7FC0.  The pages fix a 16-bit scale
 *     without naming its format; this one keeps float32's exponent range.
 *   A NaN state element gets code 0 (the rule of saturating float-to-integer
 *   conversion); +-Inf takes the end codes.
 *   Updates: see fo_fused_adamw_step and fo_fused_sgdm_step.
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never frees or reallocates them.  Outputs are written in place.
 *   - Element arrays (weights, ECC, gradients, codes, f32 arrays) must be
 *     16-byte aligned; scale arrays must be 2-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous with respect to the host; kernel faults surface at the
 *     caller's next synchronisation.  Two exceptions block the host: the
 *     first call on a device that needs the codec tables builds them and
 *     synchronises `stream` once, and a launch-table cache miss that refills
 *     a slot waits for that slot's earlier launches.  A slot read only from
 *     `stream` is rewritten behind them in stream order (no wait, unless a
 *     larger table replaces its memory: then `stream` is synchronised); a
 *     slot read from another stream or device makes the call synchronise
 *     that slot's device.  Calls record no event, so steps on one stream
 *     follow one another with no gap.  Make one call per tensor list
 *     before capturing a HIP graph; later calls with the same list are
 *     capture-safe (no allocation, no synchronisation, no memset), and a
 *     call under capture with a list that has no launch table yet fails with
 *     FO_EINVAL.  A call made under capture pins its list's launch table
 *     until the process ends, so the graph stays valid however many other
 *     lists are stepped later; once all 1024 slots are pinned, a new list
 *     fails with FO_ENOMEM.
 *   - The library keeps, per device, one codec-table buffer and up to 1024
 *     cached launch tables (device + pinned host memory, a few KB each for
 *     ordinary lists), held until the process ends.
 *   - n == 0 is a no-op returning FO_OK.
 *   - Return value: FO_OK (0) or a negative FO_E* code; fo_last_error()
 *     returns a per-thread message for the last failing call.  Argument
 *     errors are detected on the host before anything is launched, so a
 *     failing call leaves all buffers untouched.
 *   - Blocks: element i of a tensor belongs to block i/32; a tensor of n
 *     elements has ceil(n/32) scales, the last one covering n mod 32
 *     elements when n is not a multiple of 32.
 */
#ifndef FOAMD_H
#define FOAMD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FO_ABI_VERSION 6   /* 2: l2_decay in fo_adamw_hparams; dampening, nesterov in fo_sgdm_hparams;
                              3: correctly rounded quotients in the update and the codecs, NaN codes 0,
                                 NaN-only short last blocks keep a NaN scale, SGD momentum 0 as torch;
                              4: fo_hbm_probe takes a chunk size (and an in-place mode);
                              5: FO_COMPANDED4, 4-bit state codes;
                              6: FO_COMPANDED_BF16SCALE, bfloat16 block scales */

enum fo_status {
  FO_OK = 0,
  FO_EINVAL = -1,   /* null/misaligned pointer, bad enum, n < 0, unsupported combination */
  FO_EALIAS = -2,   /* two arrays of a step's tensor list overlap */
  FO_EHIP = -3,     /* HIP runtime or launch error */
  FO_ENOMEM = -4    /* the library could not allocate its launch table */
};

/* 16-bit downcast format of theta' (and of the gradients). */
enum fo_wfmt { FO_BF16 = 0, FO_FP16 = 1 };
/* State code mapping: companded (softsign-like momentum, square-root
 * variance), the linear ablation with the same scales, the companded
 * mapping onto 4-bit codes, two per byte, or the companded 8-bit codes with
 * bfloat16 block scales instead of binary16 ones. */
enum fo_codec { FO_COMPANDED = 0, FO_LINEAR = 1, FO_COMPANDED4 = 2, FO_COMPANDED_BF16SCALE = 3 };
/* State kind: signed momentum-like (int8 codes in [-127,127]; [-7,7] as
 * 4-bit codes) or unsigned variance-like (uint8 codes in [0,255]; [0,15]). */
enum fo_kind { FO_MOMENTUM = 0, FO_VARIANCE = 1 };

/*
 * fo_split_weights -- [SPLIT]
 * Splits f32 master weights into the 16-bit downcast theta' and the ECC.
 *   w32      : n float32 (read)
 *   wfmt     : FO_BF16 or FO_FP16
 *   ecc_bits : 8 or 16; supported pairs are (BF16,8), (BF16,16), (FP16,8)
 *   w16_out  : n 16-bit patterns (bf16 or fp16) (written)
 *   ecc_out  : n int8 (ecc_bits 8) or int16 (ecc_bits 16) (written)
 * theta' = the input rounded to nearest, ties away from zero; ECC = the
 * signed offset of the input from theta' in units of 2^-N of the 16-bit
 * spacing on the input's side of theta', rounded half to even and clamped.
 * NaN -> quiet NaN, ECC 0; +-Inf -> +-Inf, ECC 0; finite values beyond the
 * 16-bit range saturate to +-max with the ECC clamped.
 */
int fo_split_weights(const float* w32, int64_t n, int wfmt, int ecc_bits,
                     void* w16_out, void* ecc_out, void* stream);

/*
 * fo_reconstruct_weights -- [SPLIT]
 * Rebuilds f32 master weights from (theta', ECC): |x| = |theta'| + ECC *
 * spacing * 2^-N with the sign of theta'.  Exact for bf16 + 16-bit ECC on
 * every finite value below the bf16 overflow threshold.  Defined on what
 * fo_split_weights writes (non-finite theta' must carry ECC 0, +-0 a
 * non-negative ECC); other inputs give unspecified values.
 *   w16, ecc : n elements each (read);  w32_out : n float32 (written)
 */
int fo_reconstruct_weights(const void* w16, const void* ecc, int64_t n, int wfmt,
                           int ecc_bits, float* w32_out, void* stream);

/*
 * fo_companded_quantize -- [STATE], [LOWER]
 * Quantises an f32 state to 8-bit (or 4-bit) codes plus one 16-bit scale per
 * 32 elements.
 *   x          : n float32 (read); variance states must be >= 0
 *   kind       : FO_MOMENTUM (int8 codes) or FO_VARIANCE (uint8 codes)
 *   codec      : FO_COMPANDED, FO_LINEAR, FO_COMPANDED4 or FO_COMPANDED_BF16SCALE
 *   codes_out  : n bytes, or ceil(n/2) under FO_COMPANDED4 (written)
 *   scales_out : ceil(n/32) fp16 bit patterns, bfloat16 ones under
 *                FO_COMPANDED_BF16SCALE (written)
 * Momentum scale = smallest fp16 >= max|x| of the block; variance scale =
 * smallest fp16 >= sqrt(max x) of the block (both saturate at 65504); under
 * FO_COMPANDED_BF16SCALE the smallest bfloat16 instead (saturating at its
 * largest finite value).
 */
int fo_companded_quantize(const float* x, int64_t n, int kind, int codec,
                          void* codes_out, uint16_t* scales_out, void* stream);

/*
 * fo_dequantize -- [STATE]
 * Decodes 8-bit (or 4-bit) codes and 16-bit block scales back to f32 (inverse
 * mapping of fo_companded_quantize for the same kind and codec).
 *   codes : n bytes, or ceil(n/2) under FO_COMPANDED4 (read);
 *   scales : ceil(n/32) fp16, or bfloat16 under FO_COMPANDED_BF16SCALE (read);
 *   x_out : n float32 (written)
 */
int fo_dequantize(const void* codes, const uint16_t* scales, int64_t n, int kind,
                  int codec, float* x_out, void* stream);

/* One tensor of a fused AdamW step.  All arrays hold n elements except the
 * scale arrays, which hold ceil(n/32), and the code arrays under
 * FO_COMPANDED4, which hold ceil(n/2) bytes.  w16/ecc/codes/scales are updated in
 * place; grad (same 16-bit format as w16) is only read. */
typedef struct fo_adamw_tensor {
  void*        w16;   /* theta', bf16 or fp16 */
  void*        ecc;   /* int8 or int16 */
  const void*  grad;  /* bf16 or fp16, same format as w16 */
  int8_t*      m_q;   /* momentum codes */
  uint16_t*    m_s;   /* momentum scales (fp16 bits; bfloat16 under FO_COMPANDED_BF16SCALE) */
  uint8_t*     v_q;   /* variance codes */
  uint16_t*    v_s;   /* variance scales (fp16 bits; bfloat16 under FO_COMPANDED_BF16SCALE) */
  int64_t      n;
} fo_adamw_tensor;

typedef struct fo_adamw_hparams {
  double  lr, beta1, beta2, eps, weight_decay;
  int64_t step;      /* 1-based step counter used for bias correction */
  int32_t wfmt;      /* fo_wfmt */
  int32_t ecc_bits;  /* 8 or 16 */
  int32_t codec;     /* fo_codec */
  int32_t l2_decay;  /* 0: AdamW (decoupled decay, theta *= 1 - lr*wd);
                        1: Adam (wd*theta added to the gradient, no decoupled decay) */
} fo_adamw_hparams;

/*
 * fo_fused_adamw_step -- [UPDATE] with [SPLIT] and [STATE]
 * One AdamW step (decoupled weight decay, bias correction, step >= 1) over a
 * list of `count` tensors, enqueued on `stream` as one kernel per range of
 * 2^18 wave tiles (2^29 elements; one kernel for most lists); with
 * hp->l2_decay = 1 the step is Adam with the weight decay added to the
 * gradient (torch.optim.Adam).  Per element: widen the gradient,
 * reconstruct the f32 master, decode m and v, update in float32, split the
 * new master into theta' + ECC, recompute the block scales of the new m and v
 * and re-encode them.  The update, with the f32 constants b1, b2, 1-b1, 1-b2,
 * decay = 1 - lr*wd (1 for Adam), step_size = lr / (1 - b1^t),
 * ibc2 = 1 / sqrt(1 - b2^t) computed in double and rounded once, is
 *   [Adam: g = g + wd*theta]  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g);
 *   theta = theta*decay;  d = sqrt(v)*ibc2 + eps;  theta = theta - step_size*(m/d)
 * with every operation rounded once (no fused multiply-add) and m/d, sqrt(v)
 * correctly rounded.  Blocks never cross
 * tensors; a short last block is handled per tensor.  Any sub-list (e.g. the
 * one tensor whose gradient just arrived) may be stepped on its own; the
 * result is bitwise identical to stepping it inside a larger list.
 * Errors: FO_EINVAL (see conventions; also step < 1, count < 0, list NULL
 * with count > 0), FO_EALIAS (arrays of the list overlap), FO_ENOMEM, FO_EHIP.
 */
int fo_fused_adamw_step(const fo_adamw_tensor* list, int32_t count,
                        const fo_adamw_hparams* hp, void* stream);

/*
 * fo_fused_adamw_step_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same step as fo_fused_adamw_step, bitwise, with no
 * hipMalloc, hipFree, pinned-host allocation, event or synchronisation.
 *   The codec tables and the call's launch table (descriptors and tile-bucket
 *   index) live in one fixed device array per GPU (438 KiB, held until the
 *   process ends), written on `stream` at every call: the descriptors travel
 *   as kernel arguments (3-KiB chunks) and the bucket index is computed on
 *   the device, so nothing on the host is read after the call returns and a
 *   call captured into a HIP graph replays its own table.  The first call on
 *   a device outside capture also builds the codec tables there (a captured
 *   call builds them in its graph).
 *   Limit: at most 2048 tensors per call (count > 2048 -> FO_EINVAL); sizes
 *   are otherwise unlimited.
 *   Calls and graph replays on one GPU share that array and must not
 *   overlap: order them on one stream (or order the streams); overlapping
 *   calls race.  The first call on a device must be ordered before any call
 *   on another stream.
 * Errors: as fo_fused_adamw_step, plus FO_EINVAL for lists over the limit.
 */
int fo_fused_adamw_step_noalloc(const fo_adamw_tensor* list, int32_t count,
                                const fo_adamw_hparams* hp, void* stream);

/* One tensor of a fused SGD-with-momentum step. */
typedef struct fo_sgdm_tensor {
  void*        w16;
  void*        ecc;
  const void*  grad;
  int8_t*      b_q;   /* momentum-buffer codes (ceil(n/2) bytes under FO_COMPANDED4) */
  uint16_t*    b_s;   /* momentum-buffer scales (fp16 bits; bfloat16 under FO_COMPANDED_BF16SCALE) */
  int64_t      n;
} fo_sgdm_tensor;

typedef struct fo_sgdm_hparams {
  double  lr, momentum, weight_decay, dampening;
  int64_t step;      /* 1-based; at step 1 the buffer is set to the decayed gradient */
  int32_t wfmt;
  int32_t ecc_bits;
  int32_t codec;
  int32_t nesterov;  /* 1: Nesterov momentum (needs momentum > 0, dampening 0) */
} fo_sgdm_hparams;

/*
 * fo_fused_sgdm_step -- [UPDATE] with [SPLIT] and [STATE]
 * One SGD-with-momentum step over a list of tensors, as torch.optim.SGD:
 * d = g + wd*theta; buffer = d at step 1 (and at every step when momentum is
 * 0, where torch keeps no buffer, so dampening has no effect), else
 * momentum*buffer + (1-dampening)*d; theta -= lr * (Nesterov ? d + momentum*buffer
 * : buffer), each operation rounded once in float32.  The momentum
 * buffer uses the momentum codec.  Same layout, ownership and error rules as
 * fo_fused_adamw_step (FO_EINVAL also for dampening outside [0,1] and for
 * Nesterov without momentum or with dampening).
 */
int fo_fused_sgdm_step(const fo_sgdm_tensor* list, int32_t count,
                       const fo_sgdm_hparams* hp, void* stream);

/*
 * fo_stream_probe -- measurement only.
 * Moves exactly the bytes one fused AdamW step moves (reads every array of
 * the list, writes back w16, ecc, codes and scales) with no arithmetic, in
 * the same launch configuration, to measure the attainable HBM ceiling.
 * `key` is XOR-ed into every written word; pass 0 to leave the data unchanged.
 */
int fo_stream_probe(const fo_adamw_tensor* list, int32_t count, int32_t wfmt,
                    int32_t ecc_bits, uint32_t key, void* stream);

/*
 * fo_hbm_probe -- measurement only.
 * Plain HBM streams in the fused kernels' access style (16-byte nontemporal
 * accesses, each instruction covering 1 KiB), one wave per chunk of
 * chunk_kib KiB (1, 2, 4 or 8), to measure the attainable bandwidth next to
 * the fused step:
 *   mode 0: read `bytes` of src (dst receives at most one 4-byte word, only
 *           if the XOR of all words read equals `key`);
 *   mode 1: write `key` over `bytes` of dst;
 *   mode 2: copy `bytes` from src to dst, each word XOR-ed with `key`;
 *   mode 3: update `bytes` of dst in place (each word XOR-ed with `key`;
 *           src is ignored).
 * bytes must be a multiple of the chunk; pointers 16-byte aligned device
 * memory.  Errors: FO_EINVAL, FO_EHIP.
 */
int fo_hbm_probe(void* dst, const void* src, int64_t bytes, int32_t mode, int32_t chunk_kib,
                 uint32_t key, void* stream);

/*
 * fo_selftest -- verification of the exact fast arithmetic the fused kernels
 * use on this device.  It counts (synchronously, into *mismatches):
 *   what 0: f32 patterns x in [lo, lo + count) where the Newton-refined
 *           hardware reciprocal differs from IEEE 1/x (the kernels use it for
 *           positive normal x < 2^126);
 *   what 1: patterns where the neighbour-corrected hardware square root
 *           differs from the IEEE square root (used for x = 0, x >= 2^-96);
 *   what 2: patterns where the hardware float-to-u8 conversion differs from
 *           clamp(round_half_even(x), 0, 255), NaN -> 0;
 *   what 3: of `count` pairs (a, b) drawn from a counter-based generator
 *           seeded by lo (b positive normal below 2^126, |a| in [2^-100,
 *           2^101) or 0; pairs whose quotient is neither 0 nor of magnitude
 *           in [2^-125, 2^120) are skipped), those where the
 *           residual-corrected quotient differs from IEEE a/b;
 *   what 4: the same with b a positive finite binary16 value and |a| <= b;
 *   what 5: as 3 over the pairs whose quotient is a nonzero subnormal, which
 *           the fused AdamW step keeps out of its fast form;
 *   what 6: as 1 for the square root from the estimate of the successor
 *           with one residual test (used for x = 0 and 2^-96 <= x <= 2^100).
 * Errors: FO_EINVAL (bad `what`, NULL output, a pattern range past 2^32),
 * FO_ENOMEM, FO_EHIP.
 */
int fo_selftest(int what, uint32_t lo, uint64_t count, uint64_t* mismatches, void* stream);

/* Number of launch-table cache slots pinned by calls made under HIP graph
 * capture (all devices).  Host-only query; never fails. */
int fo_cache_pinned(void);

/* Message of the last failing call on this thread ("" if none). */
const char* fo_last_error(void);
/* FO_ABI_VERSION of the loaded library. */
int fo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FOAMD_H */
