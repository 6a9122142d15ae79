// sd_measure.hip -- a plain streaming read of device memory, the ceiling the
// verification kernels' row passes are measured against on the same device.
//
// Each workgroup reads one contiguous chunk in 16-byte vectors with the load
// the row passes use (non-temporal by default), several in flight, and folds
// them with XOR; one word per workgroup is written so that no load can be
// dropped. k_stream_read splits a flat buffer into equal chunks;
// k_stream_read_rows splits each row of a row-major matrix, as the row passes
// do (their row pitch is rarely a power of two, and chunk offsets that are
// read at a power-of-two spacing read slower).
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {

namespace {

constexpr int kReadUnroll = 4;       // 16-byte vectors per thread per step

// XOR fold of the 16-byte vectors [0, len) of `base` by one workgroup, one
// contiguous round of kBlock * kReadUnroll vectors at a time with the next
// round in flight; every thread returns the workgroup's fold.
__device__ uint32_t read_fold(const uint4* base, int64_t len, uint32_t* red) {
    constexpr int step = kBlock * kReadUnroll;
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
    uint32_t r = 0u;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) r ^= red[w];
    return r;
}

// workgroup g reads the contiguous vectors [g * chunk, (g + 1) * chunk)
__global__ __launch_bounds__(kBlock) void k_stream_read(const uint4* __restrict__ data, int64_t nvec,
                                                        int64_t chunk, uint32_t* __restrict__ sink) {
    __shared__ uint32_t red[kWavesPerBlock];
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = beg + chunk < nvec ? beg + chunk : nvec;
    const uint32_t r = read_fold(data + beg, end > beg ? end - beg : 0, red);
    if (threadIdx.x == 0) sink[blockIdx.x] = r;
}

// rows of row_vec vectors one after another, each split into chunks of
// chunk_vec vectors (the last one shorter): workgroup (row, chunk) reads its
// chunk, as the row passes read their rows
__global__ __launch_bounds__(kBlock) void k_stream_read_rows(const uint4* __restrict__ data, int64_t row_vec,
                                                             int64_t chunk_vec, int n_chunks,
                                                             uint32_t* __restrict__ sink) {
    __shared__ uint32_t red[kWavesPerBlock];
    const int64_t row = blockIdx.x / n_chunks;
    const int64_t beg = (blockIdx.x % n_chunks) * chunk_vec;
    const int64_t end = beg + chunk_vec < row_vec ? beg + chunk_vec : row_vec;
    const uint32_t r = read_fold(data + row * row_vec + beg, end - beg, red);
    if (threadIdx.x == 0) sink[blockIdx.x] = r;
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

hipError_t launch_stream_read_rows(const void* data, int64_t row_bytes, int n_rows, int64_t chunk_bytes,
                                   uint32_t* sink, hipStream_t stream) {
    const int64_t row_vec = row_bytes / 16, chunk_vec = chunk_bytes / 16;
    const int n_chunks = (int)((row_vec + chunk_vec - 1) / chunk_vec);
    PassTimer::launch(k_stream_read_rows, dim3((unsigned)((int64_t)n_rows * n_chunks)), dim3(kBlock), stream,
                      static_cast<const uint4*>(data), row_vec, chunk_vec, n_chunks, sink);
    return hipGetLastError();
}

}  // namespace sd
