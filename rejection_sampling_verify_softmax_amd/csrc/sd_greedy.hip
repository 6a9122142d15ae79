// sd_greedy.hip -- greedy chain verification.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io), §1: greedy results follow the target argmax; the first
// mismatch ends the accepted prefix.
//
// Every position of a chain is tested at once, so every row is needed: k_argmax
// streams each (row, chunk) once with 16-byte loads and writes a (value, index)
// partial; a one-wave kernel per sequence then combines the partials and takes
// the first mismatch by a ballot. (The tree walk needs only the rows on its
// path and reads them on demand: sd_walk.hip.)
#include "sd_device.hpp"
#include "sd_internal.hpp"

#include <math.h>

namespace sd {

namespace {

struct ArgPartial {
    float v;      // maximum value (NaN ignored)
    int32_t i;    // lowest index reaching it; kNone if the chunk is all NaN
};
constexpr int32_t kNone = 0x7fffffff;
#ifndef SD_ARG_UNROLL
#define SD_ARG_UNROLL 2
#endif
constexpr int kArgUnroll = SD_ARG_UNROLL;
// Tokens per argmax workgroup: short rows of few sequences still give the
// launch thousands of workgroups.
#ifndef SD_ARG_CHUNK_BF16
#define SD_ARG_CHUNK_BF16 16384
#endif
#ifndef SD_ARG_CHUNK_F32
#define SD_ARG_CHUNK_F32 16384
#endif
inline int arg_chunk(int dtype) { return dtype == 1 ? SD_ARG_CHUNK_BF16 : SD_ARG_CHUNK_F32; }
inline int arg_chunks(int V, int dtype) { return (V + arg_chunk(dtype) - 1) / arg_chunk(dtype); }

__device__ __forceinline__ bool arg_better(float v, int i, float bv, int bi) {
    // (value desc, index asc); an empty candidate (kNone) never wins
    if (i == kNone) return false;
    if (bi == kNone) return true;
    return v > bv || (v == bv && i < bi);
}

// grid: (sequence, slot, chunk); slot s <= k_b is target row cu[b]+b+s.
template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) void k_argmax(const typename E::raw* __restrict__ rows,
                                                   const int32_t* __restrict__ aux, int slots,
                                                   int K_max, int V, int chunk, int n_chunks,
                                                   ArgPartial* __restrict__ out) {
    __shared__ unsigned long long skey[kWavesPerBlock];
    constexpr int EV = E::kVec;
    constexpr int U = kArgUnroll;
    const int ch = blockIdx.x % n_chunks;
    const int rest = blockIdx.x / n_chunks;
    const int s = rest % slots;
    const int b = rest / slots;
    int d0, k;
    seq_range(aux, b, K_max, d0, k);
    if (s > k) return;
    const int64_t row = (int64_t)d0 + b + s;
    const typename E::raw* rp = rows + row * (int64_t)V;
    const int beg = ch * chunk;
    const int end = min(V, beg + chunk);
    const int nvec = (end - beg + EV - 1) / EV;
    float best = -INFINITY;
    int bidx = kNone;
    // the best of one vector's elements, first index on ties; NaN-only
    // vectors leave vmax NaN and never win (fmaxf skips a NaN operand)
    auto consider = [&](const float (&f)[EV], int vi) {
        float vmax = f[0];
#pragma unroll
        for (int e = 1; e < EV; ++e) vmax = fmaxf(vmax, f[e]);
        if (vmax > best || (bidx == kNone && vmax == vmax)) {
            int e_hit = EV - 1;
#pragma unroll
            for (int e = EV - 1; e >= 0; --e)
                if (f[e] == vmax) e_hit = e;
            const int j = beg + vi * EV + e_hit;
            if (j < end) {
                best = vmax;
                bidx = j;
            }
        }
    };
    // whole steps: unchecked loads, the next step in flight. The same rule as
    // consider(), without branches: the lane keeps the best vector's maximum,
    // its index and its raw bits; the element is found once, after the steps.
    constexpr int kStep = kBlock * U;
    const int nsteps = VEC ? nvec / kStep : 0;
    float fbest = -INFINITY;
    int fvi = -1;
    uint4 fraw = make_uint4(0u, 0u, 0u, 0u);
    pipelined_steps<U>(
        nsteps,
        [&](uint4 (&buf)[U], int st) {
#pragma unroll
            for (int u = 0; u < U; ++u) buf[u] = load16(rp + beg, st * kStep + u * kBlock + threadIdx.x);
        },
        [&](const uint4 (&buf)[U], int st) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[EV];
                E::unpack(buf[u], f);
                float vmax = f[0];
#pragma unroll
                for (int e = 1; e < EV; ++e) vmax = fmaxf(vmax, f[e]);
                const bool take = vmax > fbest || (fvi < 0 && vmax == vmax);
                fbest = take ? vmax : fbest;
                fvi = take ? st * kStep + u * kBlock + (int)threadIdx.x : fvi;
                fraw.x = take ? buf[u].x : fraw.x;
                fraw.y = take ? buf[u].y : fraw.y;
                fraw.z = take ? buf[u].z : fraw.z;
                fraw.w = take ? buf[u].w : fraw.w;
            }
        });
    if (fvi >= 0) {
        float f[EV];
        E::unpack(fraw, f);
        int e_hit = EV - 1;
#pragma unroll
        for (int e = EV - 1; e >= 0; --e)
            if (f[e] == fbest) e_hit = e;
        best = fbest;
        bidx = beg + fvi * EV + e_hit;
    }
    // the ragged end (all of it in the element-wise path)
    for (int vi = nsteps * kStep + threadIdx.x; vi < nvec; vi += kBlock) {
        float f[EV];
        if (VEC) {
            E::unpack(load16(rp + beg, vi), f);
        } else {
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int j = beg + vi * EV + e;
                f[e] = j < end ? E::at(rp, j) : NAN;
            }
        }
        consider(f, vi);
    }
    // wave then block reduction of (value desc, index asc) as one 64-bit key,
    // larger is better (0: no value), on DPP row operations
    uint32_t khi = 0u, klo = 0u;
    if (bidx != kNone) {
        const uint32_t u = __float_as_uint(best == 0.f ? 0.f : best);
        khi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        klo = 0xffffffffu - (uint32_t)bidx;
    }
    wave_max_key64(khi, klo);
    if ((threadIdx.x & (kWave - 1)) == 0) skey[threadIdx.x / kWave] = ((unsigned long long)khi << 32) | klo;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long k = skey[0];
#pragma unroll
        for (int i = 1; i < kWavesPerBlock; ++i) k = skey[i] > k ? skey[i] : k;
        ArgPartial p;
        p.v = -INFINITY;
        p.i = kNone;
        if (k != 0ull) {
            const uint32_t h = (uint32_t)(k >> 32);
            p.v = __uint_as_float((h & 0x80000000u) ? (h & 0x7fffffffu) : ~h);
            p.i = (int32_t)(0xffffffffu - (uint32_t)k);
        }
        out[((int64_t)b * slots + s) * n_chunks + ch] = p;
    }
}

// The row's argmax from its chunk partials, in chunk order. The first
// kArgRegChunks partials are loaded together, without branches (an index past
// the row's chunks reads its last chunk again, and that copy is ignored), so
// that a row of up to that many chunks costs one round trip; longer rows
// continue one partial at a time.
constexpr int kArgRegChunks = 8;
__device__ int combine_arg(const ArgPartial* p, int n_chunks) {
    ArgPartial q[kArgRegChunks];
#pragma unroll
    for (int i = 0; i < kArgRegChunks; ++i) q[i] = p[i < n_chunks ? i : n_chunks - 1];
    float bv = -INFINITY;
    int bi = kNone;
#pragma unroll
    for (int i = 0; i < kArgRegChunks; ++i)
        if (i < n_chunks && arg_better(q[i].v, q[i].i, bv, bi)) {
            bv = q[i].v;
            bi = q[i].i;
        }
    for (int i = kArgRegChunks; i < n_chunks; ++i) {
        const ArgPartial t = p[i];
        if (arg_better(t.v, t.i, bv, bi)) {
            bv = t.v;
            bi = t.i;
        }
    }
    return bi == kNone ? -1 : bi;
}

__global__ __launch_bounds__(kWave) void k_greedy_decide(
    const ArgPartial* __restrict__ part, const int32_t* __restrict__ tok,
    const int32_t* __restrict__ cu, int K_max, int V, int n_chunks, int32_t* __restrict__ A_out,
    int32_t* __restrict__ next_out, int32_t* __restrict__ status_out, const int32_t* __restrict__ cap,
    int32_t* __restrict__ A_full_out) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int slots = K_max + 1;
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    const int64_t slot0 = (int64_t)b * slots;
    bool acc = true;
    int st = 0, g = -1;
    // lane s <= k combines slot s's argmax (slot k: the extra row), all in
    // one round of loads with the tokens
    if (lane <= k) g = combine_arg(part + (slot0 + lane) * n_chunks, n_chunks);
    if (lane < k) {
        const int y = tok[d0 + lane];
        const bool yok = (y >= 0 && y < V);
        acc = yok && g >= 0 && y == g;
        st = (yok ? 0 : 1) | (g >= 0 ? 0 : 2);
    }
    const unsigned long long rej = __ballot(!acc);
    const int A_full = rej ? (__ffsll(rej) - 1) : k;
    const int kc = committed_len(cap, b, k);
    const int A = A_full < kc ? A_full : kc;
    int mine = (lane < kc && lane <= A) ? st : 0;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) mine |= __shfl_xor(mine, o, kWave);
    // A <= kc <= k: the correction is the argmax at A, and after a full
    // accept the extra token is slot kc's
    int next = A < kWave ? __shfl(g, A, kWave) : combine_arg(part + (slot0 + A) * n_chunks, n_chunks);
    if (next < 0) mine |= 2;
    if (lane == 0) {
        A_out[b] = A;
        if (A_full_out) A_full_out[b] = A_full;
        next_out[b] = next;
        if (status_out) status_out[b] = mine;
    }
}

}  // namespace

size_t greedy_ws_bytes(int B, int K_max, int V, int dtype) {
    Carve cv;
    cv.take((size_t)B * (K_max + 1) * arg_chunks(V, dtype) * sizeof(ArgPartial));
    return cv.off;
}

template <class E, bool VEC>
static hipError_t greedy_impl(const void* target, const int32_t* tokens, const int32_t* cu, int B,
                              int K_max, int V, int dtype, int32_t* A, int32_t* next, int32_t* st,
                              const int32_t* cap, int32_t* A_full, void* ws, hipStream_t stream) {
    const int nc = arg_chunks(V, dtype);
    const int chunk = arg_chunk(dtype);
    ArgPartial* part = static_cast<ArgPartial*>(ws);
    const unsigned grid = (unsigned)((size_t)B * (K_max + 1) * nc);
    PassTimer::launch(k_argmax<E, VEC>, dim3(grid), dim3(kBlock), stream,
                      static_cast<const typename E::raw*>(target), cu, K_max + 1, K_max, V, chunk, nc,
                      part);
    hipLaunchKernelGGL(k_greedy_decide, dim3(B), dim3(kWave), 0, stream, part, tokens, cu, K_max, V,
                       nc, A, next, st, cap, A_full);
    return hipGetLastError();
}

hipError_t launch_greedy(const void* target, int dtype, const int32_t* tokens, const int32_t* cu,
                         int B, int K_max, int V, int32_t* accepted_len, int32_t* next_token,
                         int32_t* seq_status, const int32_t* cap, int32_t* accepted_full, void* ws,
                         hipStream_t stream) {
    if (dtype == 1) {
        if (V % Bf16::kVec == 0)
            return greedy_impl<Bf16, true>(target, tokens, cu, B, K_max, V, dtype, accepted_len,
                                           next_token, seq_status, cap, accepted_full, ws, stream);
        return greedy_impl<Bf16, false>(target, tokens, cu, B, K_max, V, dtype, accepted_len,
                                        next_token, seq_status, cap, accepted_full, ws, stream);
    }
    if (V % F32::kVec == 0)
        return greedy_impl<F32, true>(target, tokens, cu, B, K_max, V, dtype, accepted_len,
                                      next_token, seq_status, cap, accepted_full, ws, stream);
    return greedy_impl<F32, false>(target, tokens, cu, B, K_max, V, dtype, accepted_len, next_token,
                                   seq_status, cap, accepted_full, ws, stream);
}

}  // namespace sd
