// sd_select.hip -- DSpark-style choice of verify length.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io), §5 DSpark: with per-position confidences c_i, the
// chance that the prefix survives to position j is s_j = prod_{i<=j} c_i and the
// expected advance for verify length k is 1 + sum_{j<=k} s_j; the scheduler asks
// whether one more verified position is worth its cost.
//
// Each sequence's fp32 running product extends k while s_j beats the
// per-position cost (or maximises the objective of a cost table); the packed
// offsets cu_sel are the exclusive scan of the lengths, on the device, ready
// for a packed chain verify on the same stream without a host round trip.
// Batches up to 8192 sequences: one 1024-thread workgroup does both. Larger
// batches: one thread per sequence for the lengths, then one workgroup scans
// them.
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {

namespace {

// Up to this many sequences one workgroup does everything (their lengths kept
// in LDS for the offsets); larger batches take one thread per sequence for
// the lengths, then a scan workgroup.
constexpr int kOneBlockMaxB = 8192;
constexpr int kScanThreads = 1024;

// Length of sequence b. With `table` (the cost of verifying position j+1 at
// table[j]) it is the smallest maximiser of f(k) = 1 + sum_{j<=k} s_j -
// sum_{j<=k} table[j-1], both sums running in fp64 in position order; without
// it, the length extends while s_j > cost, which is that maximiser for a
// constant cost since s_j never increases. *sum receives sum_{j<=k} s_j.
__device__ __forceinline__ int seq_len(const float* __restrict__ conf, int64_t b, int K_max, float cost,
                                       const float* __restrict__ table, double* sum_out) {
    float s = 1.0f;
    double sum = 0.0;
    int k = 0;
    if (table == nullptr) {
        bool go = true;
#pragma unroll 8
        for (int j = 0; j < K_max; ++j) {
            s = s * conf[b * K_max + j];     // fp32, left to right
            if (go && s > cost) {
                k = j + 1;
                sum += (double)s;
            } else {
                go = false;
            }
        }
    } else {
        double run_s = 0.0, run_c = 0.0, best = 1.0;
        for (int j = 0; j < K_max; ++j) {
            s = s * conf[b * K_max + j];
            run_s += (double)s;
            run_c += (double)table[j];
            const double f = 1.0 + run_s - run_c;
            if (f > best) {
                best = f;
                k = j + 1;
                sum = run_s;
            }
        }
    }
    *sum_out = sum;
    return k;
}

// One workgroup: each thread takes a contiguous run of sequences (one while
// B <= 1024), then a block scan of the per-thread sums turns the lengths into
// packed offsets cu_sel (ready for a packed chain verify on the same stream,
// without a host round trip).
__global__ __launch_bounds__(kScanThreads) void k_select_len(const float* __restrict__ conf, int B,
                                                             int K_max, float cost,
                                                             const float* __restrict__ table,
                                                             int32_t* __restrict__ k_sel,
                                                             float* __restrict__ adv,
                                                             int32_t* __restrict__ cu_sel) {
    constexpr int kWaves = kScanThreads / kWave;
    __shared__ int wsum[kWaves];
    __shared__ int32_t sk[kOneBlockMaxB];     // the lengths again, for the offsets
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int per = (B + kScanThreads - 1) / kScanThreads;
    const int b0 = tid * per;
    const int b1 = min(B, b0 + per);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        double sum;
        const int k = seq_len(conf, b, K_max, cost, table, &sum);
        k_sel[b] = k;
        sk[b] = k;
        if (adv) adv[b] = (float)(1.0 + sum);
        local += k;
    }
    if (cu_sel == nullptr) return;
    const int incl = wave_incl_scan_int(local);
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int t = wsum[i];
        before += i < w ? t : 0;
        total += t;
    }
    int run = before + incl - local;
    for (int b = b0; b < b1; ++b) {
        cu_sel[b] = run;
        run += sk[b];                // (this thread's own stores)
    }
    if (tid == 0) cu_sel[B] = total;
}

// Large batches, step 1: one thread per sequence.
__global__ __launch_bounds__(kBlock) void k_select_len_wide(const float* __restrict__ conf, int B,
                                                            int K_max, float cost,
                                                            const float* __restrict__ table,
                                                            int32_t* __restrict__ k_sel,
                                                            float* __restrict__ adv) {
    const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (b >= B) return;
    double sum;
    k_sel[b] = seq_len(conf, b, K_max, cost, table, &sum);
    if (adv) adv[b] = (float)(1.0 + sum);
}

// Large batches, step 2: the exclusive scan of the lengths by one workgroup,
// 4 consecutive lengths per thread per round (one 16-byte span), a carry
// from round to round.
__global__ __launch_bounds__(kScanThreads) void k_scan_lengths(const int32_t* __restrict__ k_sel, int B,
                                                               int32_t* __restrict__ cu_sel) {
    constexpr int kWaves = kScanThreads / kWave;
    __shared__ int wsum[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    int carry = 0;
    for (int base = 0; base < B; base += 4 * kScanThreads) {
        const int i0 = base + 4 * tid;
        int v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (i0 + e < B) ? k_sel[i0 + e] : 0;
        const int mine = v[0] + v[1] + v[2] + v[3];
        const int incl = wave_incl_scan_int(mine);
        if (lane == kWave - 1) wsum[w] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            const int t = wsum[i];
            before += i < w ? t : 0;
            total += t;
        }
        int run = carry + before + incl - mine;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (i0 + e < B) cu_sel[i0 + e] = run;
            run += v[e];
        }
        carry += total;
        __syncthreads();                 // wsum is rewritten by the next round
    }
    if (tid == 0) cu_sel[B] = carry;
}

}  // namespace

hipError_t launch_select_len(const float* conf, int B, int K_max, float cost, const float* table,
                             int32_t* k_sel, float* adv, int32_t* cu_sel, hipStream_t stream) {
    if (B <= kOneBlockMaxB) {
        hipLaunchKernelGGL(k_select_len, dim3(1), dim3(kScanThreads), 0, stream, conf, B, K_max, cost,
                           table, k_sel, adv, cu_sel);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_select_len_wide, dim3((unsigned)((B + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       stream, conf, B, K_max, cost, table, k_sel, adv);
    if (cu_sel != nullptr)
        hipLaunchKernelGGL(k_scan_lengths, dim3(1), dim3(kScanThreads), 0, stream, k_sel, B, cu_sel);
    return hipGetLastError();
}

}  // namespace sd
