/* Streaming-read reference kernel for the memory roofline (measurement aid,
 * not part of the decode path; built into libqbd_ceiling.so).
 *
 * The weight streams of the block-quantized products read every weight byte
 * once.  This kernel reads a device buffer once with the same load pattern
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

#ifdef __cplusplus
}
#endif

#endif
