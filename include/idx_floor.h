/*
 * idx_floor.h -- reference launches that show the attainable floor of an
 * indexer call on the same GPU, at the same size.
 *
 * The pages time their score and top-K kernels at decode-step sizes ("Round 18
 * Track C ..." section 1, the per-kernel timing tables), where a call moves a
 * few MB: at that size the floor is a launch plus a short streaming read, not
 * the HBM bandwidth. These entry points measure that floor on the machine at
 * hand: an empty launch, and a plain streaming read of a byte range, optionally
 * followed by the same cross-workgroup arrival counter that the fused select
 * uses to hand a row to its last workgroup; and a run of back-to-back matrix
 * products, the rate the k-means assignment's products could reach at best.
 * They compute nothing of the method and serve only as measurement context.
 *
 * Conventions are those of idx.h: device pointers owned by the caller, `stream`
 * is a hipStream_t passed as void*, validation on the host before any launch,
 * negative status (IDX_ERR_*) on failure with nothing enqueued.
 */
#ifndef IDX_FLOOR_H
#define IDX_FLOOR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One launch of `blocks` workgroups of 64 threads that do nothing.
 * blocks in [1, 65536]. */
int idx_floor_empty(int blocks, void* stream);

/* Stream-read `bytes` bytes of `src` (16-byte aligned, bytes a multiple of 16)
 * with `blocks` workgroups of `threads` threads (256 or 1024), each reading one
 * contiguous share with 16-byte loads, and write one word per workgroup to
 * `sink` (device, at least `blocks` floats). If `ticket` is not NULL (device,
 * 4-byte aligned, one uint32 that is zero before the call), every workgroup
 * then takes a ticket on it after its loads have completed, and the last one
 * returns it to zero: the hand-off of the fused select, without the select.
 * blocks in [1, 65536]; bytes > 0. */
int idx_floor_read(const void* src, size_t bytes, float* sink, uint32_t* ticket, int blocks,
                   int threads, void* stream);

/* The matrix-core floor: `blocks` workgroups of 256 threads (four waves), each
 * wave issuing `iters` rounds (a multiple of 8) of four independent
 * v_mfma_f32_32x32x16_bf16 (2 * 32 * 32 * 16 * 4 * iters flops per wave) on
 * register operands read once from `frags` (device, 16 KiB: eight A fragments
 * then eight B fragments, each 64 lanes x 8 bf16, lane-major; round r uses A
 * fragment r % 8 and, in chain c, B fragment (r + c) % 8). Every thread then
 * writes the sum of its 64 accumulator words to `sink` (device, at least
 * 256 * blocks floats; with all-ones fragments each word is 1024 * iters). It
 * shows the bf16 matrix rate the chip sustains under load, which depends on
 * the clock that load allows and so on the operand data: random fragments
 * give the realistic figure. blocks in [1, 65536]; iters in [8, 16384]. */
int idx_floor_mfma(const void* frags, int blocks, int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IDX_FLOOR_H */
