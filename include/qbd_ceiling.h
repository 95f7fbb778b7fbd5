/* Reference kernels of libqbd_ceiling.so (measurement aids, not part of the
 * decode path): the streaming read for the memory roofline, and the cost of
 * one dependent step as a launch or as a grid-wide handoff.
 *
 * The weight streams of the block-quantized products read every weight byte
 * once.  qbd_read_ceiling reads a device buffer once with the same load pattern
 * and nothing else, so its time for B bytes is the practical ceiling of one
 * launch that streams B bytes on this GPU (launch, ramp and drain included),
 * beside the nominal HBM peak.
 *
 * Status codes are those of qbd.h: 0 ok, -1 null pointer, -2 bad size,
 * -3 misaligned pointer, -6 launch failure.
 */
#ifndef QBD_CEILING_H
#define QBD_CEILING_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words the sink of qbd_read_ceiling must hold (one per thread of its grid). */
int64_t qbd_read_ceiling_sink_words(void);

/* Reads bytes bytes at device pointer src (16-byte aligned; bytes a positive
 * multiple of 16) on stream, and writes sink[t] (device, 4-byte aligned,
 * qbd_read_ceiling_sink_words() words, caller-owned) so that the XOR of all
 * sink words equals the XOR of all 32-bit words of the buffer.  Asynchronous;
 * the buffers must stay valid until the stream has run it. */
int qbd_read_ceiling(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

/* Words of the device work buffer qbd_grid_handoff uses. */
int64_t qbd_grid_handoff_work_words(void);

/* Runs `phases` (0 .. 2^20) grid-wide handoffs of a 4 KB vector inside one
 * cooperative launch of 256 one-wave workgroups (one per CU), so that a
 * caller can time one handoff as the difference of two phase counts.  A
 * handoff is what a persistent kernel chaining dependent decode products
 * would pay per step: every workgroup writes its share of the vector,
 * arrives, waits for all others, then reads the whole vector.  mode 0: one
 * arrival counter; 1: 16 counters on separate lines; 2: one arrival word per
 * workgroup.  work: device, 256-byte aligned, qbd_grid_handoff_work_words()
 * words, caller-owned; the call clears its arrival and error words on
 * `stream` first (with a kernel).  After the stream has run it, work word W - 64 is nonzero
 * if a wait gave up (each is bounded) and word W - 63 counts vector values
 * read back wrong, W = qbd_grid_handoff_work_words(); both are zero in a
 * correct run.  Returns 0, -1 (null), -2 (mode or phases), -3 (alignment)
 * or -6 (the runtime refused the launch, e.g. the grid cannot be resident
 * at once). */
int qbd_grid_handoff(int mode, int phases, uint32_t* work, hipStream_t stream);

/* Words of the result buffer of qbd_grid_handoff_noalloc: 64 error words,
 * then the 1024 floats of the last phase's vector. */
int64_t qbd_grid_handoff_noalloc_result_words(void);

/* qbd_grid_handoff for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc):
 * the same handoff with its work buffer in a static 12.5 KB device array of
 * the library instead of a caller workspace.  Each GPU holds one such array
 * until the process ends; its address is looked up once per device, on the
 * first call with that device current.  No argument changes how much of it
 * is used, so no size can exceed it; mode and phases are checked as for
 * qbd_grid_handoff.  The call clears the arrival words with a kernel (no
 * memset), runs the handoff, then writes result (device, 4-byte aligned,
 * qbd_grid_handoff_noalloc_result_words() words, caller-owned): word 0 is
 * nonzero if a wait gave up, word 1 counts vector values read back wrong,
 * and words 64 .. 64 + 1023 hold the last phase's vector (not written when
 * phases is 0).  Calls that overlap on one GPU share the array and race.
 * Returns the codes of qbd_grid_handoff, and -5 if the array's address
 * cannot be looked up on the current device.  Allocates nothing. */
int qbd_grid_handoff_noalloc(int mode, int phases, uint32_t* result, hipStream_t stream);

/* Launches an empty kernel (one wave) on stream: the cost of one dependent
 * launch, timed over many launches replayed from a HIP graph. */
int qbd_empty_launch(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
