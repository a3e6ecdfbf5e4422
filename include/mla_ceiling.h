/*
 * mla_ceiling.h -- C ABI of libmla_ceiling.so, the measurement probes that
 * the benchmark quotes the decode kernel against (MI355X, gfx950).
 *
 * This library is not part of the decode path and computes nothing of the
 * method: it measures, on the machine it runs on, the two ceilings a paged
 * MLA decode is bound by (the pages on FlashMLA name a memory-bound and a
 * compute-bound setting: the ygpos news page and the tweet quoted at the top
 * of "DeepSeek 开源记-第1天-FlashMLA").  The decode library does not link it.
 *
 * Conventions: device pointers of the current HIP device, owned by the
 * caller; calls only enqueue on `stream` (a hipStream_t, NULL = default);
 * status codes as in mla_decode.h (0 ok, -1 invalid argument, -4 HIP error);
 * arguments outside the stated ranges are rejected on the host before any
 * launch.
 */
#ifndef MLA_CEILING_H
#define MLA_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Each of num_workgroups workgroups streams the pages_per_workgroup cache
 * pages listed in pages[w * pages_per_workgroup + i] through a 4-slot LDS
 * ring of 36,864-byte stages with 16-byte LDS-DMA loads, two stages ahead, as
 * the decode kernel's 16-row tile does; no arithmetic.
 *   pool        device, num_pages pages of page_bytes bytes (one KV head)
 *   page_bytes  must be 73,728 (64 rows x 1152 B); num_pages * page_bytes
 *               must be below 2^31; a page index outside the pool loads
 *               zeros (no fault)
 *   pages       device int32 [num_workgroups, pages_per_workgroup]
 *   sink        device int32 [1]; written only in a case that does not occur
 *               for real data (it keeps the loads from being optimised away)
 * Bytes read = num_workgroups * pages_per_workgroup * page_bytes.
 */
int mla_ceiling_stream(const void *pool, int num_pages, int page_bytes, const int32_t *pages,
                       int num_workgroups, int pages_per_workgroup, int32_t *sink, void *stream);

/*
 * num_workgroups workgroups of 4 waves; each wave runs iters x 4 independent
 * 32x32x16 bf16 MFMAs (32768 flops each).
 *   sink             device float [1], same role as above
 *   random_operands  0: every MFMA reads the same small constant operands;
 *                    1: the MFMAs cycle through 8 pairs of operand fragments
 *                    of random bf16 values (magnitudes 1/8 .. 4, random signs
 *                    and mantissas), so consecutive MFMAs see new inputs as in
 *                    a kernel that streams cache rows; other values rejected
 * Flops = num_workgroups * 4 * iters * 4 * 32768.
 */
int mla_ceiling_mfma(float *sink, int num_workgroups, int iters, int random_operands, void *stream);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char *mla_ceiling_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CEILING_H */
