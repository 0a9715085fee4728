/*
 * deltalog_probe.h -- measurement kernels beside the DeltaLog library: what
 * the GPU streams at the access pattern of the decode kernels.
 *
 * The decode path is bound by HBM bandwidth (gist.science summary,
 * "Problema": eager decoding runs at an arithmetic intensity of about
 * 0.5-1 FLOP per byte, far below the machine balance).  The peak a datasheet
 * quotes is not what a given access pattern reaches, so these kernels
 * measure the two ceilings that bound the decode kernels from above, on the
 * same heads, workgroup shape, XCD mapping and 16-byte nontemporal loads and
 * stores: a read of every head (the most an append can do, since it reads
 * the base once) and an in-place copy of every head (the most the
 * decode-and-fold can do, since it reads and writes the base once).  A
 * write of every head, with no read, shows what the write side streams on
 * its own beside the copy that mixes reads and writes.  They compute nothing
 * of the method.
 *
 * Conventions as in deltalog.h: caller-owned device memory, the caller's
 * stream (void* hipStream_t), nothing allocated, nothing synchronised.
 */
#ifndef DELTALOG_PROBE_H
#define DELTALOG_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

#define DL_PROBE_READ 0 /* read every head once */
#define DL_PROBE_COPY 1 /* read every head and write it back in place, unchanged */
#define DL_PROBE_WRITE 2 /* overwrite every element of every head with 1.0f (no read; the values are lost) */

/* Enqueue one probe launch over the [B,H,dk,dv] fp32 tensor `state`
 * (16-byte aligned; DL_PROBE_COPY leaves its values unchanged,
 * DL_PROBE_WRITE replaces them all with 1.0f) with one
 * workgroup per head, shaped as the single-token append.  `sink` is one
 * float of device memory (4-byte aligned) that a read probe may write.
 * Returns 0, or a negative code as in dl_status (-1 argument, -2 shape,
 * -3 unsupported width, -4 launch refused) with dl_probe_last_error()
 * describing it.  B*H <= 2^23; dk and dv each 32, 64 or 128. */
int dl_probe_stream(int mode, float *state, int B, int H, int dk, int dv, float *sink, void *stream);

/* Message for the last error of dl_probe_stream on this thread ("" if none). */
const char *dl_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTALOG_PROBE_H */
