/*
 * probe.h -- chip-peak probes of the benchmark (not part of the LoRA path).
 * They give the measured denominators printed beside the published MI355X
 * peaks (HBM3E 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).
 *
 * hrg_probe_read -- one launch of `blocks` x 256 threads that reads every
 *   16-byte vector of the device buffer buf[0, bytes) once.  sink: device
 *   uint32 [blocks * 4] (one word per wave is written).  Returns 0, 1 on a
 *   bad argument, 8 if the launch failed.  Asynchronous on `stream`.
 * hrg_probe_mfma -- one launch of `blocks` x 256 threads; every wave issues
 *   iters x 4 bf16 MFMAs of 32x32x16 (32768 flops each) on registers.  sink:
 *   device float [blocks * 256] (never written in practice).  Same returns.
 */
#ifndef HRG_PROBE_H
#define HRG_PROBE_H
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>
#ifdef __cplusplus
extern "C" {
#endif
int hrg_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream);
int hrg_probe_mfma(int iters, float* sink, int blocks, hipStream_t stream);
#ifdef __cplusplus
}
#endif
#endif /* HRG_PROBE_H */
