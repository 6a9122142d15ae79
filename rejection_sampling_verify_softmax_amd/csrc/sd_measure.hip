// sd_measure.hip -- a plain streaming read of device memory, the ceiling the
// verification kernels' row passes are measured against on the same device.
//
// Each workgroup reads one contiguous chunk (the layout of the row passes
// chunks) in 16-byte vectors with the load the row passes use (non-temporal by
// default), several in flight, and folds them with XOR; one word per
// workgroup is written so that no load can be dropped.
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {

namespace {

constexpr int kReadUnroll = 4;       // 16-byte vectors per thread per step

__global__ __launch_bounds__(kBlock) void k_stream_read(const uint4* __restrict__ data, int64_t nvec,
                                                        int64_t chunk, uint32_t* __restrict__ sink) {
    __shared__ uint32_t red[kWavesPerBlock];
    // workgroup g reads the contiguous vectors [g * chunk, (g + 1) * chunk), the
    // whole workgroup one contiguous round of kBlock * kReadUnroll vectors at a time
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = beg + chunk < nvec ? beg + chunk : nvec;
    const int64_t len = end > beg ? end - beg : 0;
    constexpr int step = kBlock * kReadUnroll;
    const uint4* base = data + beg;
    const int nsteps = (int)(len / step);
    uint32_t acc = 0u;
    pipelined_steps<kReadUnroll>(
        nsteps,
        [&](uint4 (&buf)[kReadUnroll], int s) {
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u)
                buf[u] = load16(base, (int64_t)s * step + u * kBlock + threadIdx.x);
        },
        [&](const uint4 (&buf)[kReadUnroll], int) {
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) acc ^= buf[u].x ^ buf[u].y ^ buf[u].z ^ buf[u].w;
        });
    for (int64_t i = (int64_t)nsteps * step + threadIdx.x; i < len; i += kBlock) {
        const uint4 v = load16(base, i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0u;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) r ^= red[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

hipError_t launch_stream_read(const void* data, int64_t bytes, uint32_t* sink, int n_blocks,
                              hipStream_t stream) {
    const int64_t nvec = bytes / 16;
    const int64_t chunk = (nvec + n_blocks - 1) / n_blocks;
    PassTimer::launch(k_stream_read, dim3((unsigned)n_blocks), dim3(kBlock), stream,
                      static_cast<const uint4*>(data), nvec, chunk, sink);
    return hipGetLastError();
}

}  // namespace sd
