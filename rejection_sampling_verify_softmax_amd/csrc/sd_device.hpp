// sd_device.hpp -- device helpers shared by the libsd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

constexpr int kWave = 64;
constexpr int kBlock = 256;            // threads per workgroup for the streaming kernels
constexpr int kWavesPerBlock = kBlock / kWave;

// ---------------------------------------------------------------------------
// Element access. Logit rows are fp32 or raw bf16 bit patterns; both are read
// in 16-byte vectors (8 bf16 or 4 fp32 per lane per load).
// ---------------------------------------------------------------------------
struct Bf16 {
    using raw = uint16_t;
    static constexpr int kVec = 8;
    __device__ static inline float at(const raw* p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
    __device__ static inline void unpack(const uint4& v, float (&f)[kVec]) {
        f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
        f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
        f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
    }
    // A vector of -inf (fills lanes past the end of a range).
    __device__ static inline uint4 neg_inf() {
        return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    }
};

struct F32 {
    using raw = float;
    static constexpr int kVec = 4;
    __device__ static inline float at(const raw* p, int64_t i) { return p[i]; }
    __device__ static inline void unpack(const uint4& v, float (&f)[kVec]) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ static inline uint4 neg_inf() {
        return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
    }
};

#ifndef SD_NT_LOADS
#define SD_NT_LOADS 1
#endif
// 16-byte load of vector `vec_index` of a row. Logit rows are streamed once, so
// the default marks the loads non-temporal (they bypass cache retention).
__device__ __forceinline__ uint4 load16(const void* base, int64_t vec_index) {
#if SD_NT_LOADS
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u r = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(base) + vec_index);
    return make_uint4(r.x, r.y, r.z, r.w);
#else
    return reinterpret_cast<const uint4*>(base)[vec_index];
#endif
}

// 16-byte load that is kept in the caches (for data read twice in a row).
__device__ __forceinline__ uint4 load16_cached(const void* base, int64_t vec_index) {
    return reinterpret_cast<const uint4*>(base)[vec_index];
}

// Runs steps 0..nsteps-1 with the next step's loads in flight while the
// current step is processed. Two buffers alternate by unrolling in pairs, so no
// register copy joins the steps and each step waits only for its own loads.
// load(buf, s) issues step s's loads into buf; proc(buf, s) consumes them.
template <int U, class Load, class Proc>
__device__ __forceinline__ void pipelined_steps(int nsteps, Load&& load, Proc&& proc) {
    if (nsteps <= 0) return;
    uint4 a[U], b[U];
    load(a, 0);
    int s = 0;
    for (; s + 2 < nsteps; s += 2) {
        load(b, s + 1);
        proc(a, s);
        load(a, s + 2);
        proc(b, s + 1);
    }
    if (s + 1 < nsteps) {
        load(b, s + 1);
        proc(a, s);
        proc(b, s + 1);
    } else {
        proc(a, s);
    }
}

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// NaN-ignoring maximum.
__device__ __forceinline__ float nmax(float a, float b) { return (b > a || a != a) ? b : a; }

// ---------------------------------------------------------------------------
// Wave and block reductions (fixed order, deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = nmax(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

// Exclusive prefix sum across the wave (lane order).
__device__ __forceinline__ double wave_excl_scan(double v) {
    const int lane = threadIdx.x & (kWave - 1);
    double incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    return incl - v;
}

// DPP row operations (no LDS round trip): v from lane i-n of the same row of
// 16 (row_shr:n; 0 where there is none), and the last lane of the previous
// row (row_bcast:15) or of the previous pair of rows (row_bcast:31) into the
// rows selected by the mask (0 elsewhere). The whole wave must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_from(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}

// Sum of a double over each row of 16 lanes by DPP rotations (no LDS round
// trip): every lane receives its row's sum (lanes may differ in the last bit,
// the order of the additions depending on the lane). The whole wave must be
// active.
// (lanes a DPP operation does not write, or whose source lies outside the
// row, receive +0.0)
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long b = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Inclusive prefix sum of a double across the wave (lane order) on DPP row
// shifts and row broadcasts. The whole wave must be active.
__device__ __forceinline__ double wave_incl_scan_f64(double v) {
    v += dpp_f64<0x111>(v);         // row_shr:1
    v += dpp_f64<0x112>(v);         // row_shr:2
    v += dpp_f64<0x114>(v);         // row_shr:4
    v += dpp_f64<0x118>(v);         // row_shr:8
    v += dpp_f64<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    return v;
}
__device__ __forceinline__ double row_sum_f64(double v) {
    v += dpp_f64<0x128>(v);     // row_ror:8
    v += dpp_f64<0x124>(v);     // row_ror:4
    v += dpp_f64<0x122>(v);     // row_ror:2
    v += dpp_f64<0x121>(v);     // row_ror:1
    return v;
}

// Maximum over the wave, returned to every lane.
// The wave's largest (hi, lo) pair, compared as one 64-bit key, returned to
// every lane: row_shr steps within each row of 16, then the last lanes of the
// earlier rows, then lane 63 read back.
template <int CTRL, int ROWS>
__device__ __forceinline__ void key64_step(uint32_t& hi, uint32_t& lo) {
    const uint32_t h = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, ROWS, 0xf, false);
    const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, ROWS, 0xf, false);
    const bool take = h > hi || (h == hi && l > lo);
    hi = take ? h : hi;
    lo = take ? l : lo;
}
__device__ __forceinline__ void wave_max_key64(uint32_t& hi, uint32_t& lo) {
    key64_step<0x111, 0xf>(hi, lo);
    key64_step<0x112, 0xf>(hi, lo);
    key64_step<0x114, 0xf>(hi, lo);
    key64_step<0x118, 0xf>(hi, lo);
    key64_step<0x142, 0xa>(hi, lo);
    key64_step<0x143, 0xc>(hi, lo);
    hi = __builtin_amdgcn_readlane(hi, kWave - 1);
    lo = __builtin_amdgcn_readlane(lo, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_from<0x111, 0xf>(v));
    v = max(v, dpp_from<0x112, 0xf>(v));
    v = max(v, dpp_from<0x114, 0xf>(v));
    v = max(v, dpp_from<0x118, 0xf>(v));
    v = max(v, dpp_from<0x142, 0xa>(v));
    v = max(v, dpp_from<0x143, 0xc>(v));
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

// The j-th largest (from 1) of the wave's 64 keys, bits LO and up (the rest
// 0), 0 when fewer than j keys are nonzero: the largest r that at least j
// keys reach, built bit by bit from the top.
template <int LO>
__device__ __forceinline__ uint32_t wave_jth_largest(uint32_t key, int j) {
    uint32_t r = 0u;
#pragma unroll
    for (int bit = 31; bit >= LO; --bit) {
        const uint32_t c = r | (1u << bit);
        if ((int)__popcll(__ballot(key >= c)) >= j) r = c;
    }
    return r;
}

// Inclusive prefix sum across the wave (lane order) of non-negative counts.
__device__ __forceinline__ int wave_incl_scan_int(int c) {
    uint32_t v = (uint32_t)c;
    v += dpp_from<0x111, 0xf>(v);
    v += dpp_from<0x112, 0xf>(v);
    v += dpp_from<0x114, 0xf>(v);
    v += dpp_from<0x118, 0xf>(v);
    v += dpp_from<0x142, 0xa>(v);
    v += dpp_from<0x143, 0xc>(v);
    return (int)v;
}

// ---------------------------------------------------------------------------
// Wave-level LDS sorting and ranking of 64-bit keys.
// ---------------------------------------------------------------------------
// Orders the wave's LDS traffic: every lane's earlier LDS writes are visible
// to every lane's later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bitonic sort (descending) of a[0..n) by one wave, n a power of two.
__device__ inline void wave_sort_desc(unsigned long long* a, int n) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            wave_lds_sync();
            for (int i = lane; i < n / 2; i += kWave) {
                const int lo = 2 * stride * (i / stride) + (i % stride);
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long x = a[lo], y = a[hi];
                if ((x < y) == desc) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
        }
    }
    wave_lds_sync();
}

// Number of keys in list[0..n) (sorted descending, distinct) above key.
__device__ __forceinline__ int count_above(const unsigned long long* list, int n,
                                           unsigned long long key) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (list[mid] > key) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Block-wide reductions for kBlock threads; `scratch` holds kWavesPerBlock entries.
// Every thread receives the result. Contains __syncthreads().
__device__ inline double block_sum(double v, double* scratch) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i) r += scratch[i];
    return r;
}
__device__ inline float block_max(float v, float* scratch) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    float r = scratch[0];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i) r = nmax(r, scratch[i]);
    return r;
}
__device__ inline int block_min_int(int v, int* scratch) {
    v = wave_min_int(v);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    int r = scratch[0];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i) r = min(r, scratch[i]);
    return r;
}
__device__ inline int block_max_int(int v, int* scratch) {
    v = wave_max_int(v);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    int r = scratch[0];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i) r = max(r, scratch[i]);
    return r;
}

// Exclusive prefix sum over the block (fp64, thread order). Contains barriers.
// `scratch` holds kWavesPerBlock entries.
__device__ inline double block_exclusive_scan(double v, double* scratch, double* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    double incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == kWave - 1) scratch[w] = incl;
    __syncthreads();
    double base = 0.0, tot = 0.0;
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i) {
        if (i < w) base += scratch[i];
        tot += scratch[i];
    }
    *total = tot;
    return base + incl - v;
}

// Draft-row offset and length of sequence b. A packed length outside
// [0, K_max] (an inconsistent cu) is clamped so that no kernel can index past
// the K_max+1 slots it was sized for.
__device__ __forceinline__ void seq_range(const int32_t* cu, int b, int K_max, int& d0, int& k) {
    if (cu) {
        d0 = cu[b];
        k = cu[b + 1] - d0;
        k = k < 0 ? 0 : (k > K_max ? K_max : k);
    } else {
        d0 = b * K_max;
        k = K_max;
    }
}

// Committed window of sequence b: its draft length k, or cap[b] clamped to
// [0, k] when a cap is given (the window is still verified in full).
__device__ __forceinline__ int committed_len(const int32_t* cap, int b, int k) {
    if (cap == nullptr) return k;
    const int c = cap[b];
    return c < 0 ? 0 : (c > k ? k : c);
}

// ---------------------------------------------------------------------------
// Softmax partials. A partial (o, S) of a set of logits x says
//   sum_x 2^(x*c - o) = S,  c = log2(e)/T rounded to fp32,
// where the reference o is an fp32 value (normally fl32(m*c) for some logit m).
// Partials of disjoint sets combine exactly in fp64 (see combine()).
// ---------------------------------------------------------------------------
struct alignas(16) Partial {
    float o;        // reference (fp32); -inf for an empty set
    float pad;
    double S;       // sum relative to o; 0 for an empty set, non-finite for a bad set
};

}  // namespace sd
