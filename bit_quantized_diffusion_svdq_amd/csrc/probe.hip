// Measurement helpers (no part of the layer's arithmetic): the shader clock
// the chip holds right now, and a read-only stream over a buffer (the floor
// a memory-bound kernel of that size can reach).
#include "common.h"

namespace {

// One lane counts shader-clock ticks (s_memtime) against the constant
// 100 MHz real-time counter (s_memrealtime) over a bounded busy loop.
__global__ void clock_probe_kernel(long long* out, int spins) {
    if (threadIdx.x != 0) return;
    const long long t0 = __builtin_amdgcn_s_memtime();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < spins; ++i) asm volatile("s_nop 7");
    const long long t1 = __builtin_amdgcn_s_memtime();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    out[0] = t1 - t0;
    out[1] = r1 - r0;
}

// Every 16-byte chunk of the buffer is read once (non-temporal), folded
// into a per-workgroup XOR that is stored so the loads cannot be dropped.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ buf, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
    const rsrc_t r = make_rsrc(buf, n16 * 16);
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(i * 16), 0, 2);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int t = 0; t < 256; ++t) s ^= red[t];
        sink[blockIdx.x] = s;
    }
}

}  // namespace

hipError_t launch_clock_probe(long long* out, int spins, hipStream_t stream) {
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, spins);
    return hipGetLastError();
}

hipError_t launch_read_probe(const uint8_t* buf, int64_t bytes, uint32_t* sink, int blocks,
                             hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, buf, bytes / 16, sink);
    return hipGetLastError();
}
