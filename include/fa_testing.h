/*
 * fa_testing.h -- test hooks of libfa.so.  Not part of the computational
 * ABI in fa.h; they exist so that tests can drive rare paths from the host
 * while every kernel still runs to completion.
 */
#ifndef FA_TESTING_H
#define FA_TESTING_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Polls that the one-pass wide-row softmax (fa_softmax, out of place) makes
 * while waiting for the other chunks of its row before it computes the row's
 * statistics itself by streaming the row.  0 sends every workgroup straight
 * to that fallback; a negative value restores the default (65536).  Applies
 * to launches made after the call, process-wide; not thread-safe against
 * concurrent fa_softmax calls.
 */
void fa_testing_set_softmax_spin_limit(int limit);

/*
 * Rule by which the bf16 prefill (fa_forward with FA_BF16) moves each query
 * row's reference max and rescales o and l ('Online Softmax -- the
 * mathematical heart of FlashAttention', section 4; research-hub 'Online
 * Softmax' page, "Why it matters": FA-4 rescales only when the max shift
 * threatens stability):
 *   2 (default)  overflow guard: a tile's weights are taken against the
 *                current reference and kept unless a weight could reach 2^32;
 *                only then is the tile's max taken and the reference moved;
 *   1            threshold: every tile's max is taken, the reference moves
 *                when it grows by more than 8 (log2 units);
 *   0            eager: every tile's max is taken and o, l are rescaled on
 *                every tile (the plain recurrence).
 * All three give the same result up to rounding.  Any other value restores
 * the default.  Applies to launches made after the call, process-wide; for
 * measurement and tests.
 */
void fa_testing_set_rescale_rule(int rule);

#ifdef __cplusplus
}
#endif

#endif /* FA_TESTING_H */
