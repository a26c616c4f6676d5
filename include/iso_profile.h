/*
 * iso_profile.h -- per-stage GPU timing of iso_fit_ex calls (libiso_mi355x.so).
 *
 * "Merge Hulls Without Copying Vertices: GPU Isotonic Regression" reports the fit's time per
 * stage (Section 7.5: chunk stage, merge levels, reconstruction, prefix sums).  These hooks give
 * the same breakdown on the caller's stream with HIP events, so a benchmark can time the
 * dominant kernel inside its own timed region.
 *
 * Stages: 0 whole-diagram chunks (k_increasing), 1 chunk pass (k_chunk; for rows of at most 4096
 * elements the one kernel that fits them: k_row, k_wave or k_tiny), 2 exact chunk
 * pass (k_chunk on the chunks whose turns the first pass could not decide), 3 chunk-start scan
 * (2 launches; 1 for rows of at most 1024 chunks), 4 merge levels (three levels of the tree per
 * launch: ceil(ceil(log2 m) / 3) launches for m chunks), 5 ends, 6 fit.  Rows of at most 4096
 * elements run stage 1 only.
 *
 * While enabled, every iso_fit_ex call records one event before its first kernel and one after
 * each stage, on its stream.  The state is process-global and not thread-safe: enable, run the
 * calls to time, read, disable -- from one host thread.
 */
#ifndef ISO_MI355X_PROFILE_H
#define ISO_MI355X_PROFILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ISO_PROF_STAGES = 7 };

/* Turn event recording on (1) or off (0).  Returns ISO_OK. */
int iso_prof_enable(int on);

/* Wait for the recorded events, add each stage's elapsed milliseconds and kernel launch count
 * since the last reset into ms[0..6] and launches[0..6] (arrays of ISO_PROF_STAGES entries
 * owned by the caller), store the number of timed calls in *calls, then forget the events.
 * Returns ISO_OK or ISO_EHIP. */
int iso_prof_read(double* ms, int64_t* launches, int64_t* calls);

/* Static name of a stage ("increasing", "chunk", "exact", "scan", "merge", "ends", "fit"), or "?". */
const char* iso_prof_stage_name(int stage);

/* Device-wide counts of rarely taken branches of the long-row path, kept whether or not timing is
 * enabled (one atomic add per event, on that branch only), for tests that must know a branch ran:
 *   [0] merges of the merge levels that fell back on the Overmars-van Leeuwen bisection after
 *       32 memory windows of one side ("Merge Hulls Without Copying Vertices", Section 5.2);
 *   [1] of those, bisections that rounding defeated, finished by single steps;
 *   [2] chunks processed by the exact chunk pass (Section 6 "Predicates": a turn of the first
 *       pass fell inside its error bound);
 *   [3] merges that walked in 256-vertex memory windows.
 * Copies the counts of the current device into out[0..3] (caller-owned, ISO_PROF_COUNTERS
 * entries) and zeroes them if reset != 0.  Waits for the device's work to finish (a synchronous
 * copy), so call it after the fits to be counted.  Counts from fits running concurrently on
 * several streams add up.  Returns ISO_OK, ISO_EINVAL (out NULL) or ISO_EHIP. */
enum { ISO_PROF_COUNTERS = 4 };
int iso_prof_counters(uint64_t* out, int reset);

#ifdef __cplusplus
}
#endif

#endif /* ISO_MI355X_PROFILE_H */
