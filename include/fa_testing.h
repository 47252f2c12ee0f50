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

#ifdef __cplusplus
}
#endif

#endif /* FA_TESTING_H */
