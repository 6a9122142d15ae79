// sd_kv.hip -- accepted-path KV compaction after a tree walk.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io), §5 DDTree: after the walk the KV cache keeps only the
// accepted path. Draft node n (1 .. N-1) of sequence b wrote its keys and values
// to row base[b] + n - 1; the i-th node of the accepted path moves to row
// base[b] + i, so the accepted prefix becomes contiguous.
//
// Node ids grow along a path (a child is numbered after its parent), so the
// source of move i, base + path[i] - 1, is never below a destination of an
// earlier or equal move: moves taken in path order never read a row another
// move already wrote. One workgroup per (sequence, column tile of the row);
// each thread owns 16-byte columns and runs the moves in path order, so no
// barrier is needed.
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {

namespace {

constexpr int kKvWordsPerThread = 2;          // 16-byte words per thread per row
constexpr int kKvTile = kBlock * kKvWordsPerThread;
constexpr int kKvBatch = 4;                   // moves whose loads are issued together

typedef unsigned int kv_word __attribute__((ext_vector_type(4)));   // 16 bytes

__global__ __launch_bounds__(kBlock) void k_compact_kv(kv_word* __restrict__ kv, int64_t words,
                                                       const int64_t* __restrict__ base,
                                                       const int32_t* __restrict__ path,
                                                       const int32_t* __restrict__ alen, int N,
                                                       int n_tiles, int64_t n_rows) {
    const int b = blockIdx.x / n_tiles;
    const int tile = blockIdx.x % n_tiles;
    int A = alen[b];
    A = A < 0 ? 0 : (A > N - 1 ? N - 1 : A);
    const int64_t row0 = base[b];
    // a draft region outside the buffer is left alone
    if (A == 0 || row0 < 0 || row0 + (N - 1) > n_rows) return;
    const int32_t* p = path + (int64_t)b * N;
    const int64_t w0 = (int64_t)tile * kKvTile + threadIdx.x;
    for (int i0 = 0; i0 < A; i0 += kKvBatch) {
        // a batch: every source read before any destination of the batch is
        // written (a later move's source is never an earlier move's target)
        kv_word v[kKvBatch][kKvWordsPerThread];
        int src[kKvBatch];
#pragma unroll
        for (int j = 0; j < kKvBatch; ++j) {
            const int n = (i0 + j < A) ? p[i0 + j] : 0;
            src[j] = (n >= 1 && n <= N - 1) ? n : 0;          // 0: not a draft node, skipped
        }
#pragma unroll
        for (int j = 0; j < kKvBatch; ++j)
#pragma unroll
            for (int e = 0; e < kKvWordsPerThread; ++e) {
                const int64_t w = w0 + (int64_t)e * kBlock;
                if (src[j] != 0 && w < words) v[j][e] = kv[(row0 + src[j] - 1) * words + w];
            }
#pragma unroll
        for (int j = 0; j < kKvBatch; ++j)
#pragma unroll
            for (int e = 0; e < kKvWordsPerThread; ++e) {
                const int64_t w = w0 + (int64_t)e * kBlock;
                // (a node already in place needs no write)
                if (src[j] != 0 && src[j] - 1 != i0 + j && w < words)
                    kv[(row0 + i0 + j) * words + w] = v[j][e];
            }
    }
}

}  // namespace

hipError_t launch_compact_kv(void* kv, int64_t row_bytes, int64_t n_rows, const int64_t* base,
                             const int32_t* path, const int32_t* accepted_len, int B, int N,
                             hipStream_t stream) {
    const int64_t words = row_bytes / 16;
    const int n_tiles = (int)((words + kKvTile - 1) / kKvTile);
    PassTimer::launch(k_compact_kv, dim3((unsigned)((int64_t)B * n_tiles)), dim3(kBlock), stream,
                      static_cast<kv_word*>(kv), words, base, path, accepted_len, N, n_tiles, n_rows);
    return hipGetLastError();
}

}  // namespace sd
