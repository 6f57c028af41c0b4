/*
 * littlebit_probe.h -- measurement aid shipped beside the LittleBit library
 * (liblittlebit.so).  Not part of the method and not needed to use it: the
 * benchmark uses this call to measure the HBM read bandwidth plain loads reach
 * on the GPU, the reference its decode bandwidth is read against.
 */
#ifndef LITTLEBIT_PROBE_H
#define LITTLEBIT_PROBE_H

#include <stdint.h>

#include "littlebit.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues on `stream` one
 * read-only streaming pass over `bytes` bytes of device memory at `buf`
 * (16-byte loads, grid-stride), so that a caller timing it with events gets
 * the HBM read bandwidth plain loads reach on this GPU.  buf must be 16-byte
 * aligned and bytes a positive multiple of 16 (LB_ERR_ALIGNMENT /
 * LB_ERR_INVALID_ARGUMENT otherwise).  Reads only; writes nothing the caller
 * can see. */
lb_status lb_probe_stream_read(const void* buf, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LITTLEBIT_PROBE_H */
