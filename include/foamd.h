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
 *
 * Numerical definitions (rounding modes, operation order, scale format,
 * compander formulas) are those of the CPU oracle shipped with the tests; the
 * pages leave them open and the chosen readings are documented with it.
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
 *     synchronises `stream` once, and a launch-table cache miss that evicts
 *     a slot waits for that slot's last use.  Make one call per tensor list
 *     before capturing a HIP graph; later calls with the same list are
 *     capture-safe (no allocation, no synchronisation, no memset).
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

#define FO_ABI_VERSION 2   /* 2: l2_decay in fo_adamw_hparams; dampening, nesterov in fo_sgdm_hparams */

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
 * variance) or the linear ablation with the same scales. */
enum fo_codec { FO_COMPANDED = 0, FO_LINEAR = 1 };
/* State kind: signed momentum-like (int8 codes in [-127,127]) or unsigned
 * variance-like (uint8 codes in [0,255]). */
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
 * fo_companded_quantize -- [STATE]
 * Quantises an f32 state to 8-bit codes plus one fp16 scale per 32 elements.
 *   x          : n float32 (read); variance states must be >= 0
 *   kind       : FO_MOMENTUM (int8 codes) or FO_VARIANCE (uint8 codes)
 *   codec      : FO_COMPANDED or FO_LINEAR
 *   codes_out  : n bytes (written)
 *   scales_out : ceil(n/32) fp16 bit patterns (written)
 * Momentum scale = smallest fp16 >= max|x| of the block; variance scale =
 * smallest fp16 >= sqrt(max x) of the block (both saturate at 65504).
 */
int fo_companded_quantize(const float* x, int64_t n, int kind, int codec,
                          void* codes_out, uint16_t* scales_out, void* stream);

/*
 * fo_dequantize -- [STATE]
 * Decodes 8-bit codes and fp16 block scales back to f32 (inverse mapping of
 * fo_companded_quantize for the same kind and codec).
 *   codes : n bytes (read);  scales : ceil(n/32) fp16 (read);  x_out : n float32 (written)
 */
int fo_dequantize(const void* codes, const uint16_t* scales, int64_t n, int kind,
                  int codec, float* x_out, void* stream);

/* One tensor of a fused AdamW step.  All arrays hold n elements except the
 * scale arrays, which hold ceil(n/32).  w16/ecc/codes/scales are updated in
 * place; grad (same 16-bit format as w16) is only read. */
typedef struct fo_adamw_tensor {
  void*        w16;   /* theta', bf16 or fp16 */
  void*        ecc;   /* int8 or int16 */
  const void*  grad;  /* bf16 or fp16, same format as w16 */
  int8_t*      m_q;   /* momentum codes */
  uint16_t*    m_s;   /* momentum scales (fp16 bits) */
  uint8_t*     v_q;   /* variance codes */
  uint16_t*    v_s;   /* variance scales (fp16 bits) */
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
 * reconstruct the f32 master, decode m and v, update in float32 with a fixed
 * operation order, split the new master into theta' + ECC, recompute the
 * block scales of the new m and v and re-encode them.  Blocks never cross
 * tensors; a short last block is handled per tensor.  Any sub-list (e.g. the
 * one tensor whose gradient just arrived) may be stepped on its own; the
 * result is bitwise identical to stepping it inside a larger list.
 * Errors: FO_EINVAL (see conventions; also step < 1, count < 0, list NULL
 * with count > 0), FO_EALIAS (arrays of the list overlap), FO_ENOMEM, FO_EHIP.
 */
int fo_fused_adamw_step(const fo_adamw_tensor* list, int32_t count,
                        const fo_adamw_hparams* hp, void* stream);

/* One tensor of a fused SGD-with-momentum step. */
typedef struct fo_sgdm_tensor {
  void*        w16;
  void*        ecc;
  const void*  grad;
  int8_t*      b_q;   /* momentum-buffer codes */
  uint16_t*    b_s;   /* momentum-buffer scales (fp16 bits) */
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
 * d = g + wd*theta; buffer = d at step 1, else momentum*buffer + (1-dampening)*d;
 * theta -= lr * (Nesterov ? d + momentum*buffer : buffer).  The momentum
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
 * fo_selftest -- verification of the exact fast arithmetic the fused kernels
 * use on this device.  Over the f32 bit patterns [lo, lo + count) it counts
 * (synchronously, into *mismatches) where
 *   what 0: the Newton-refined hardware reciprocal differs from IEEE 1/x
 *           (the kernels use it for positive normal x < 2^126);
 *   what 1: the neighbour-corrected hardware square root differs from the
 *           IEEE square root (used for x = 0 and x >= 2^-96);
 *   what 2: the hardware float-to-u8 conversion differs from
 *           clamp(round_half_even(x), 0, 255) (NaN skipped).
 * Errors: FO_EINVAL (bad `what`, NULL output, range past 2^32), FO_ENOMEM, FO_EHIP.
 */
int fo_selftest(int what, uint32_t lo, uint64_t count, uint64_t* mismatches, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* fo_last_error(void);
/* FO_ABI_VERSION of the loaded library. */
int fo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FOAMD_H */
