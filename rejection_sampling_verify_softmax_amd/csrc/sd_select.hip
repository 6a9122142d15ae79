// sd_select.hip -- DSpark-style choice of verify length.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io), §5 DSpark: with per-position confidences c_i, the
// chance that the prefix survives to position j is s_j = prod_{i<=j} c_i and the
// expected advance for verify length k is 1 + sum_{j<=k} s_j; the scheduler asks
// whether one more verified position is worth its cost.
//
// One workgroup: each thread takes a contiguous run of sequences, forms the
// fp32 running product, extends k while s_j beats the per-position cost, then a
// block scan turns the lengths into packed offsets cu_sel (ready for a packed
// chain verify on the same stream, without a host round trip).
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {

namespace {

constexpr int kSelectLds = 4096;         // lengths kept in LDS for the offsets

// With `table` (the cost of verifying position j+1 at table[j]) the length is
// the smallest maximiser of f(k) = 1 + sum_{j<=k} s_j - sum_{j<=k} table[j-1],
// both sums running in fp64 in position order; without it, the length extends
// while s_j > cost, which is that maximiser for a constant cost since s_j never
// increases.
__global__ __launch_bounds__(kBlock) void k_select_len(const float* __restrict__ conf, int B,
                                                       int K_max, float cost,
                                                       const float* __restrict__ table,
                                                       int32_t* __restrict__ k_sel,
                                                       float* __restrict__ adv,
                                                       int32_t* __restrict__ cu_sel) {
    __shared__ double scan_scratch[kWavesPerBlock];
    __shared__ int32_t sk[kSelectLds];       // the lengths again, for the offsets
    const int per = (B + kBlock - 1) / kBlock;
    const int b0 = threadIdx.x * per;
    const int b1 = min(B, b0 + per);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        float s = 1.0f;
        double sum = 0.0;
        int k = 0;
        if (table == nullptr) {
            bool go = true;
#pragma unroll 8
            for (int j = 0; j < K_max; ++j) {
                s = s * conf[(int64_t)b * K_max + j];     // fp32, left to right
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
                s = s * conf[(int64_t)b * K_max + j];
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
        k_sel[b] = k;
        if (b < kSelectLds) sk[b] = k;
        if (adv) adv[b] = (float)(1.0 + sum);
        local += k;
    }
    if (cu_sel == nullptr) return;
    double total;
    const double excl = block_exclusive_scan((double)local, scan_scratch, &total);
    int run = (int)excl;
    for (int b = b0; b < b1; ++b) {
        cu_sel[b] = run;
        run += b < kSelectLds ? sk[b] : k_sel[b];    // (this thread's own stores)
    }
    if (threadIdx.x == kBlock - 1) cu_sel[B] = (int)total;
}

}  // namespace

hipError_t launch_select_len(const float* conf, int B, int K_max, float cost, const float* table,
                             int32_t* k_sel, float* adv, int32_t* cu_sel, hipStream_t stream) {
    hipLaunchKernelGGL(k_select_len, dim3(1), dim3(kBlock), 0, stream, conf, B, K_max, cost, table,
                       k_sel, adv, cu_sel);
    return hipGetLastError();
}

}  // namespace sd
