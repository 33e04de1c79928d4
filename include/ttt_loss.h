/*
 * ttt_loss.h - C ABI of the in-place masked softmax-loss gradient (MI355X / gfx950).
 *
 * The SpecForge paper review, "§3 Technical architecture -> Memory-efficient gradient
 * computation" and "§4 Core formulas -> Masked softmax loss / In-place backward", trains the
 * draft's LM head with a soft-target cross entropy whose gradient is written over the logits:
 *
 *   pi = softmax(z)   L = -sum_i p_i log pi_i   s = sum_i p_i g   z <- -(p g - pi s)
 *
 * per token row of the logits z [rows, vocab], target distribution p [rows, vocab] and
 * upstream gradient g, one weight per row (the token's loss-mask value times the loss
 * normaliser; a masked row has g = 0 and gets a zero gradient).  Rows of p need not sum to 1.
 *
 * Conventions (shared with ttt_attn.h): device pointers owned by the caller, 16-byte aligned
 * bases, work enqueued on `stream`, negative TTT_E_* codes (see ttt_attn.h) returned before
 * anything is launched, no allocation, no synchronisation, no state kept.
 */
#ifndef TTT_LOSS_H
#define TTT_LOSS_H

#include <stddef.h>
#include <stdint.h>

#include "ttt_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* rows >= 1; vocab >= 8 and a multiple of 8; dtype TTT_DTYPE_BF16 or TTT_DTYPE_F32
 * (z and p share it; g and loss are fp32). */
typedef struct ttt_loss_params {
  int64_t rows;
  int32_t vocab;
  int32_t dtype;
} ttt_loss_params;

/*
 * z      [rows, vocab] logits, overwritten in place with dL/dz = -(p g - softmax(z) s)
 *        (rounded to dtype; everything in between is fp32).
 * target [rows, vocab] target distribution p (read only).
 * g      [rows] fp32 upstream gradient per row.
 * loss   [rows] fp32 per-row loss -sum_i p_i log softmax(z)_i (unweighted), or NULL.
 * Errors: TTT_E_NULL (z, target or g NULL), TTT_E_SHAPE (rows < 1, vocab < 1,
 * rows * vocab >= 2^40), TTT_E_UNSUPPORTED (vocab % 8 != 0, unknown dtype), TTT_E_ALIGN,
 * TTT_E_HIP.  z and target must not overlap.
 */
int ttt_loss_grad_inplace(const ttt_loss_params* p, void* z, const void* target, const float* g,
                          float* loss, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_LOSS_H */
