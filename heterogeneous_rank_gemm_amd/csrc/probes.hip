// Chip-peak probes for the roofline denominators: a streaming read of a
// device buffer (HBM bytes per second) and a register-resident loop of bf16
// MFMAs (dense matrix-core flops per second).  They are measurement aids of
// the benchmark, not part of the LoRA path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "probe.h"

namespace {

// Every thread reads 16-byte vectors with a grid stride and folds them into
// one word, so the loads cannot be dropped; one word per block is written.
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, size_t n, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i];
    const uint4 b = p[i + stride];
    const uint4 c = p[i + 2 * stride];
    const uint4 d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // one store per wave at most: the lanes fold first
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

// Each wave keeps four independent 32x32 accumulators and issues `iters`
// rounds of four 32x32x16 bf16 MFMAs on register operands.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u + lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(0x3c003c00u, 0x3c003c00u + lane, 0x3c003c00u, 0x3c003c00u));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = hrg::mfma32(a, b, c0);
    c1 = hrg::mfma32(b, a, c1);
    c2 = hrg::mfma32(a, a, c2);
    c3 = hrg::mfma32(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 1234.5f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // never true; keeps the loop
}

}  // namespace

extern "C" {

int hrg_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  if (!buf || !sink || blocks < 1 || bytes < 16) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<const uint4*>(buf),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

int hrg_probe_mfma(int iters, float* sink, int blocks, hipStream_t stream) {
  if (!sink || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

}  // extern "C"
