/* A plain streaming read of device memory, for measurement only.
 *
 * Not part of the decode path and not used by it.  The benchmark times this
 * read beside stage 1 of the decode so that the fraction of the nominal HBM
 * peak the decode reaches can be set against what a bare read of device
 * memory reaches on the same part: a large streaming read (the practical
 * read rate) and a cold read of exactly the decode's KV byte count (the
 * same start-up and tail costs, no page walk and no arithmetic).
 *
 * Built as its own library, libsplitkv_probe.so, so that the decode
 * library's exports stay the calls of attn_decode.h.
 */
#ifndef SPLITKV_READ_PROBE_H
#define SPLITKV_READ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues one kernel on `stream` (a hipStream_t; NULL = the null stream)
 * that reads `bytes` bytes starting at the device pointer `buf`, 16 bytes
 * per lane per load: `workgroups` workgroups of 256 lanes, each reading one
 * contiguous share of the buffer with eight loads in flight per lane (a
 * workgroup past the end reads nothing).  Nothing is written in
 * practice: the lanes fold what they read into one word and store it to
 * `sink` (device, at least `workgroups` 32-bit words) only if it equals a
 * fixed constant, which keeps the loads from being optimised away.
 *
 * Ownership: the caller owns `buf` and `sink`; nothing is allocated and
 * nothing is synchronised.
 * Returns 0 on success; -1 if buf or sink is null, buf is not 16-byte
 * aligned, bytes is not a positive multiple of 16 or workgroups is not
 * positive; otherwise the hipError_t of the launch.
 */
int32_t splitkv_read_probe(const void* buf, int64_t bytes, int32_t workgroups, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_READ_PROBE_H */
