// sd_chain.hip -- stochastic chain verification over the full vocabulary.
//
// Implements the chain rule of the page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、
// DDTree 与 DSpark" (chzhyang.github.io), §1: accept y_i iff u_i q_i(y_i) <= p_i(y_i)
// (the acceptance-probability equation alpha = min(1, p/q)), stop at the first
// rejection (the A B C D example), draw the correction token from the
// normalised positive residual [p - q]+ or, when all pass, the extra token from
// p; temperature is folded into both p and q.
//
// Four launches on the caller's stream:
//   1. k_chain_stats  grid (sequence, slot, chunk): one pass over every row.
//      Slot i < k_b streams target row i and draft row i together; slot k_b
//      streams the extra-token row. Each workgroup writes the softmax partial
//      (o, S) of its chunk of each row and, for chunk 0, the two logits at y_i.
//   2. k_chain_decide grid B, one wave: combines the partials of each row in
//      fp64, evaluates p_i(y_i) and q_i(y_i) in fp64, the accept bits, a
//      wave ballot for A, and the decision descriptor.
//   3. k_chain_mass   grid (sequence, chunk): for sequences that stopped on a
//      rejection only, the residual mass of each chunk of the decision row pair.
//   4. k_chain_sample grid B: finds the chunk that holds the inverse-CDF point
//      (chunk masses of the residual, or of p from the step-1 partials for an
//      extra token) and scans inside that one chunk.
#include "sd_device.hpp"
#include "sd_internal.hpp"

#include <math.h>

namespace sd {

namespace {

constexpr int kModeResidual = 0;
constexpr int kModeExtra = 1;
constexpr int kModeNone = 2;
constexpr int kStatsUnroll = 4;

struct ChainDesc {
    int32_t mode;
    int32_t A;
    int32_t t_row;      // target row the final token is drawn from
    int32_t d_row;      // draft row of the residual; -1 when q counts as 0
    int32_t slot;       // slot of the decision row (partials lookup)
    float u;            // the final uniform
    float O_p, O_q;     // row references
    double S_p, S_q;    // row sums relative to the references
};

struct RowStat {
    float O;
    double S;
    bool valid;
};

// Reads 16-byte vector `vi` of [beg, end) into f; entries past `end` are -inf.
template <class E, bool VEC>
__device__ __forceinline__ void load_vec(const typename E::raw* row, int beg, int end, int vi,
                                         float (&f)[E::kVec]) {
    if (VEC) {
        E::unpack(load16(row + beg, vi), f);
    } else {
#pragma unroll
        for (int e = 0; e < E::kVec; ++e) {
            const int j = beg + vi * E::kVec + e;
            f[e] = (j < end) ? E::at(row, j) : -INFINITY;
        }
    }
}

// Exact two-pass partial of row[beg, end): max first (NaN ignored, NaN presence
// recorded), then the sum relative to fl32(max * c). Used when the one-pass
// estimate is not finite.
template <class E, bool VEC>
__device__ Partial chunk_stats_exact(const typename E::raw* row, int beg, int end, float c,
                                     double* redd, float* redf, int* redi) {
    constexpr int EV = E::kVec;
    const int nvec = (end - beg + EV - 1) / EV;
    float m = -INFINITY;
    int nan_seen = 0;
    for (int vi = threadIdx.x; vi < nvec; vi += kBlock) {
        float f[EV];
        if (VEC) {
            E::unpack(load16(row + beg, vi), f);
        } else {
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int j = beg + vi * EV + e;
                f[e] = (j < end) ? E::at(row, j) : -INFINITY;
            }
        }
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            nan_seen |= (f[e] != f[e]);
            m = nmax(m, f[e]);
        }
    }
    m = block_max(m, redf);
    nan_seen = block_max_int(nan_seen, redi);
    Partial p;
    p.pad = 0.f;
    if (nan_seen || m == INFINITY) {
        p.o = 0.f;
        p.S = NAN;
        return p;
    }
    if (m == -INFINITY) {
        p.o = -INFINITY;
        p.S = 0.0;
        return p;
    }
    const float o = m * c;
    double s = 0.0;
    for (int vi = threadIdx.x; vi < nvec; vi += kBlock) {
        float f[EV];
        load_vec<E, VEC>(row, beg, end, vi, f);
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) t += fast_exp2(__builtin_fmaf(f[e], c, -o));
        s += (double)t;
    }
    p.o = o;
    p.S = block_sum(s, redd);
    return p;
}

// One-pass partials of NR rows over [beg, end). The reference of each row is
// fl32(m0 * c) with m0 the largest of the chunk's first 16-byte vector (read by
// every lane from one cache line); any overflow, -inf or NaN reference makes the
// sum non-finite and sends that row to the exact two-pass path.
template <class E, bool VEC, int NR>
__device__ void chunk_stats(const typename E::raw* const (&rows)[NR], int beg, int end, float c,
                            Partial (&out)[NR], double* redd, float* redf, int* redi) {
    constexpr int EV = E::kVec;
    constexpr int U = kStatsUnroll;
    const int nvec = (end - beg + EV - 1) / EV;
    float o[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float f[EV];
        load_vec<E, VEC>(rows[r], beg, end, 0, f);
        float m = f[0];
#pragma unroll
        for (int e = 1; e < EV; ++e) m = fmaxf(m, f[e]);
        o[r] = m * c;
    }
    float acc[NR][EV];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[r][e] = 0.f;

    for (int v0 = threadIdx.x; v0 < nvec; v0 += kBlock * U) {
        float f[NR][U][EV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = v0 + u * kBlock;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (VEC) {
                    uint4 w = (vi < nvec) ? load16(rows[r] + beg, vi) : E::neg_inf();
                    E::unpack(w, f[r][u]);
                } else {
                    if (vi < nvec) {
                        load_vec<E, VEC>(rows[r], beg, end, vi, f[r][u]);
                    } else {
#pragma unroll
                        for (int e = 0; e < EV; ++e) f[r][u][e] = -INFINITY;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int e = 0; e < EV; ++e)
                    acc[r][e] += fast_exp2(__builtin_fmaf(f[r][u][e], c, -o[r]));
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < EV; ++e) s += (double)acc[r][e];
        const double S = block_sum(s, redd);
        if (isfinite(S) && isfinite(o[r])) {
            out[r].o = o[r];
            out[r].pad = 0.f;
            out[r].S = S;
        } else {
            out[r] = chunk_stats_exact<E, VEC>(rows[r], beg, end, c, redd, redf, redi);
        }
    }
}

template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) void k_chain_stats(
    const typename E::raw* __restrict__ tgt, const typename E::raw* __restrict__ dft,
    const int32_t* __restrict__ tok, const int32_t* __restrict__ cu, int K_max, int V, int chunk,
    int n_chunks, float c, Partial* __restrict__ part_t, Partial* __restrict__ part_d,
    float* __restrict__ xy) {
    __shared__ double redd[kWavesPerBlock];
    __shared__ float redf[kWavesPerBlock];
    __shared__ int redi[kWavesPerBlock];
    const int slots = K_max + 1;
    const int ch = blockIdx.x % n_chunks;
    const int rest = blockIdx.x / n_chunks;
    const int s = rest % slots;
    const int b = rest / slots;
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    if (s > k) return;
    const int64_t slot_id = (int64_t)b * slots + s;
    const int64_t t_row = (int64_t)d0 + b + s;
    const int beg = ch * chunk;
    const int end = min(V, beg + chunk);
    const typename E::raw* tp = tgt + t_row * (int64_t)V;
    if (s < k) {
        const int64_t d_row = (int64_t)d0 + s;
        const typename E::raw* dp = dft + d_row * (int64_t)V;
        if (ch == 0 && threadIdx.x == 0) {
            const int y = tok[d_row];
            float xt = NAN, xd = NAN;
            if (y >= 0 && y < V) {
                xt = E::at(tp, y);
                xd = E::at(dp, y);
            }
            xy[slot_id * 2] = xt;
            xy[slot_id * 2 + 1] = xd;
        }
        const typename E::raw* rows[2] = {tp, dp};
        Partial out[2];
        chunk_stats<E, VEC, 2>(rows, beg, end, c, out, redd, redf, redi);
        if (threadIdx.x == 0) {
            part_t[slot_id * n_chunks + ch] = out[0];
            part_d[slot_id * n_chunks + ch] = out[1];
        }
    } else {
        const typename E::raw* rows[1] = {tp};
        Partial out[1];
        chunk_stats<E, VEC, 1>(rows, beg, end, c, out, redd, redf, redi);
        if (threadIdx.x == 0) part_t[slot_id * n_chunks + ch] = out[0];
    }
}

// Row statistics from its chunk partials (fixed chunk order, fp64).
__device__ RowStat combine_row(const Partial* p, int n_chunks) {
    RowStat r;
    r.O = -INFINITY;
    r.S = 0.0;
    r.valid = true;
    for (int i = 0; i < n_chunks; ++i) {
        const Partial q = p[i];
        if (!isfinite(q.S)) r.valid = false;
        if (q.S > 0.0) r.O = fmaxf(r.O, q.o);
    }
    if (!r.valid || r.O == -INFINITY) {
        r.valid = false;
        return r;
    }
    double S = 0.0;
    for (int i = 0; i < n_chunks; ++i) {
        const Partial q = p[i];
        if (q.S > 0.0) S += q.S * exp2((double)q.o - (double)r.O);
    }
    r.S = S;
    r.valid = isfinite(S) && S > 0.0;
    return r;
}

__global__ __launch_bounds__(kWave) void k_chain_decide(
    const Partial* __restrict__ part_t, const Partial* __restrict__ part_d,
    const float* __restrict__ xy, const int32_t* __restrict__ tok, const float* __restrict__ uni,
    const int32_t* __restrict__ cu, int K_max, int V, int n_chunks, float c,
    int32_t* __restrict__ A_out, float* __restrict__ probs_out, int32_t* __restrict__ status_out,
    ChainDesc* __restrict__ desc) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int slots = K_max + 1;
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    const int64_t slot0 = (int64_t)b * slots;
    bool acc = true;
    int st = 0;
    RowStat rp{-INFINITY, 0.0, false}, rq{-INFINITY, 0.0, false};
    if (lane < k) {
        rp = combine_row(part_t + (slot0 + lane) * n_chunks, n_chunks);
        rq = combine_row(part_d + (slot0 + lane) * n_chunks, n_chunks);
        const int y = tok[d0 + lane];
        const bool yok = (y >= 0 && y < V);
        double py = 0.0, qy = 0.0;
        if (yok && rp.valid) py = exp2((double)xy[(slot0 + lane) * 2] * (double)c - (double)rp.O) / rp.S;
        if (yok && rq.valid) qy = exp2((double)xy[(slot0 + lane) * 2 + 1] * (double)c - (double)rq.O) / rq.S;
        const double u = (double)uni[d0 + b + lane];
        acc = rp.valid && rq.valid && yok && py > 0.0 && u * qy <= py;
        st = (yok ? 0 : 1) | ((rp.valid && rq.valid) ? 0 : 2);
        if (probs_out) {
            probs_out[2 * (int64_t)(d0 + lane)] = (float)py;
            probs_out[2 * (int64_t)(d0 + lane) + 1] = (float)qy;
        }
    }
    const unsigned long long rej = __ballot(!acc);
    const int A = rej ? (__ffsll(rej) - 1) : k;
    int mine = (lane < k && lane <= A) ? st : 0;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) mine |= __shfl_xor(mine, o, kWave);
    // decision row statistics
    ChainDesc d;
    d.A = A;
    d.u = uni[d0 + b + k];
    if (A < k) {
        const float Op = __shfl(rp.O, A, kWave);
        const double Sp = __shfl(rp.S, A, kWave);
        const bool vp = __shfl((int)rp.valid, A, kWave) != 0;
        const float Oq = __shfl(rq.O, A, kWave);
        const double Sq = __shfl(rq.S, A, kWave);
        const bool vq = __shfl((int)rq.valid, A, kWave) != 0;
        d.mode = vp ? kModeResidual : kModeNone;
        d.t_row = d0 + b + A;
        d.d_row = vq ? d0 + A : -1;
        d.slot = A;
        d.O_p = Op;
        d.S_p = Sp;
        d.O_q = Oq;
        d.S_q = Sq;
    } else {
        RowStat rb = combine_row(part_t + (slot0 + k) * n_chunks, n_chunks);
        d.mode = rb.valid ? kModeExtra : kModeNone;
        if (!rb.valid) mine |= 2;
        d.t_row = d0 + b + k;
        d.d_row = -1;
        d.slot = k;
        d.O_p = rb.O;
        d.S_p = rb.S;
        d.O_q = 0.f;
        d.S_q = 0.0;
    }
    if (lane == 0) {
        A_out[b] = A;
        if (status_out) status_out[b] = mine;
        desc[b] = d;
    }
}

// Residual weight of one token: max(p - q, 0) in fp32 from the row statistics.
// Shared by the mass and sample kernels so both see identical values.
__device__ __forceinline__ float residual_w(float xp, float xq, float c, float Op, float ip,
                                            float Oq, float iq, bool has_q) {
    const float p = fast_exp2(__builtin_fmaf(xp, c, -Op)) * ip;
    const float q = has_q ? fast_exp2(__builtin_fmaf(xq, c, -Oq)) * iq : 0.f;
    return fmaxf(p - q, 0.f);
}

template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) void k_chain_mass(
    const typename E::raw* __restrict__ tgt, const typename E::raw* __restrict__ dft,
    const ChainDesc* __restrict__ desc, int V, int chunk, int n_chunks, float c,
    double* __restrict__ mass) {
    __shared__ double redd[kWavesPerBlock];
    constexpr int EV = E::kVec;
    const int b = blockIdx.x / n_chunks;
    const int ch = blockIdx.x % n_chunks;
    const ChainDesc d = desc[b];
    if (d.mode != kModeResidual) return;
    const int beg = ch * chunk;
    const int end = min(V, beg + chunk);
    const int nvec = (end - beg + EV - 1) / EV;
    const typename E::raw* tp = tgt + (int64_t)d.t_row * V;
    const bool has_q = d.d_row >= 0;
    const typename E::raw* dp = has_q ? dft + (int64_t)d.d_row * V : tp;
    const float ip = (float)(1.0 / d.S_p);
    const float iq = has_q ? (float)(1.0 / d.S_q) : 0.f;
    float acc[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] = 0.f;
    for (int vi = threadIdx.x; vi < nvec; vi += kBlock) {
        float fp[EV], fq[EV];
        load_vec<E, VEC>(tp, beg, end, vi, fp);
        load_vec<E, VEC>(dp, beg, end, vi, fq);
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[e] += residual_w(fp[e], fq[e], c, d.O_p, ip, d.O_q, iq, has_q);
    }
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < EV; ++e) s += (double)acc[e];
    s = block_sum(s, redd);
    if (threadIdx.x == 0) mass[(int64_t)b * n_chunks + ch] = s;
}

template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) void k_chain_sample(
    const typename E::raw* __restrict__ tgt, const typename E::raw* __restrict__ dft,
    const Partial* __restrict__ part_t, const ChainDesc* __restrict__ desc,
    const double* __restrict__ mass, int K_max, int V, int chunk, int n_chunks, float c,
    int32_t* __restrict__ next_out, float* __restrict__ R_out) {
    __shared__ double redd[kWavesPerBlock];
    __shared__ int redi[kWavesPerBlock];
    __shared__ double sh_before, sh_target;
    __shared__ int sh_chunk, sh_use_p;
    constexpr int EV = E::kVec;
    const int b = blockIdx.x;
    const ChainDesc d = desc[b];
    if (d.mode == kModeNone) {
        if (threadIdx.x == 0) {
            next_out[b] = -1;
            if (R_out) R_out[b] = 0.f;
        }
        return;
    }
    const int slots = K_max + 1;
    if (threadIdx.x == 0) {
        // chunk masses: residual, or p (extra token / residual with no mass)
        double R = 0.0;
        if (d.mode == kModeResidual)
            for (int i = 0; i < n_chunks; ++i) R += mass[(int64_t)b * n_chunks + i];
        const bool use_p = !(d.mode == kModeResidual && R > 0.0);
        const Partial* pp = part_t + ((int64_t)b * slots + d.slot) * n_chunks;
        double total = 0.0;
        if (use_p) {
            for (int i = 0; i < n_chunks; ++i)
                if (pp[i].S > 0.0) total += pp[i].S * exp2((double)pp[i].o - (double)d.O_p);
        } else {
            total = R;
        }
        const double target = (double)d.u * total;
        double cum = 0.0, before = 0.0;
        int found = -1, last_pos = -1;
        for (int i = 0; i < n_chunks; ++i) {
            double m;
            if (use_p)
                m = pp[i].S > 0.0 ? pp[i].S * exp2((double)pp[i].o - (double)d.O_p) : 0.0;
            else
                m = mass[(int64_t)b * n_chunks + i];
            if (m > 0.0) last_pos = i;
            if (found < 0 && cum + m > target && m > 0.0) {
                found = i;
                before = cum;
            }
            cum += m;
        }
        if (found < 0) {
            found = last_pos;
            before = 0.0;
            for (int i = 0; i < last_pos; ++i)
                before += use_p ? (pp[i].S > 0.0 ? pp[i].S * exp2((double)pp[i].o - (double)d.O_p) : 0.0)
                                : mass[(int64_t)b * n_chunks + i];
        }
        sh_before = before;
        sh_target = target;
        sh_chunk = found;
        sh_use_p = use_p ? 1 : 0;
        if (R_out) R_out[b] = (d.mode == kModeResidual) ? (float)R : 0.f;
    }
    __syncthreads();
    const int ch = sh_chunk;
    const bool use_p = sh_use_p != 0;
    const double target = sh_target;
    if (ch < 0) {
        if (threadIdx.x == 0) next_out[b] = -1;
        return;
    }
    // In-chunk scan: thread t owns a contiguous segment of `seg` elements.
    const int beg = ch * chunk;
    const int end = min(V, beg + chunk);
    const int seg = chunk / kBlock;                   // multiple of EV
    const int s0 = beg + threadIdx.x * seg;
    const int s1 = min(end, s0 + seg);
    const typename E::raw* tp = tgt + (int64_t)d.t_row * V;
    const bool has_q = !use_p && d.d_row >= 0;
    const typename E::raw* dp = has_q ? dft + (int64_t)d.d_row * V : tp;
    const float ip = (float)(1.0 / d.S_p);
    const float iq = has_q ? (float)(1.0 / d.S_q) : 0.f;
    double mysum = 0.0;
    int last_pos = -1;
    for (int j0 = s0; j0 < s1; j0 += EV) {
        float fp[EV], fq[EV];
        load_vec<E, false>(tp, j0, s1, 0, fp);
        if (has_q) load_vec<E, false>(dp, j0, s1, 0, fq);
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            if (j0 + e >= s1) break;
            const float w = use_p ? fast_exp2(__builtin_fmaf(fp[e], c, -d.O_p))
                                  : residual_w(fp[e], has_q ? fq[e] : 0.f, c, d.O_p, ip, d.O_q, iq, has_q);
            mysum += (double)w;
            if (w > 0.f) last_pos = j0 + e;
        }
    }
    double total;
    const double excl = block_exclusive_scan(mysum, redd, &total);
    const double start = sh_before + excl;
    const bool crosses = (s0 < s1) && (start + mysum > target);
    const int first = block_min_int(crosses ? (int)threadIdx.x : 0x7fffffff, redi);
    if (first == 0x7fffffff) {
        const int lp = block_max_int(last_pos, redi);
        if (threadIdx.x == 0) next_out[b] = lp;
        return;
    }
    if ((int)threadIdx.x == first) {
        double run = start;
        int pick = -1, lastp = -1;
        for (int j0 = s0; j0 < s1 && pick < 0; j0 += EV) {
            float fp[EV], fq[EV];
            load_vec<E, false>(tp, j0, s1, 0, fp);
            if (has_q) load_vec<E, false>(dp, j0, s1, 0, fq);
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                if (j0 + e >= s1 || pick >= 0) break;
                const float w = use_p ? fast_exp2(__builtin_fmaf(fp[e], c, -d.O_p))
                                      : residual_w(fp[e], has_q ? fq[e] : 0.f, c, d.O_p, ip, d.O_q, iq, has_q);
                run += (double)w;
                if (w > 0.f) lastp = j0 + e;
                if (run > target && w > 0.f) pick = j0 + e;
            }
        }
        next_out[b] = pick >= 0 ? pick : lastp;
    }
}

}  // namespace

size_t chain_full_ws_bytes(int B, int K_max, int V, int dtype) {
    const int nc = n_chunks_for(V, dtype);
    const size_t slots = (size_t)B * (K_max + 1);
    Carve cv;
    cv.take(slots * nc * sizeof(Partial));      // part_t
    cv.take(slots * nc * sizeof(Partial));      // part_d
    cv.take(slots * 2 * sizeof(float));         // xy
    cv.take((size_t)B * sizeof(ChainDesc));     // desc
    cv.take((size_t)B * nc * sizeof(double));   // mass
    return cv.off;
}

template <class E, bool VEC>
static hipError_t chain_full_impl(const ChainArgs& a) {
    const int nc = n_chunks_for(a.V, a.dtype);
    const int chunk = chunk_elems(a.dtype);
    const size_t slots = (size_t)a.B * (a.K_max + 1);
    Carve cv;
    char* ws = static_cast<char*>(a.ws);
    Partial* part_t = reinterpret_cast<Partial*>(ws + cv.take(slots * nc * sizeof(Partial)));
    Partial* part_d = reinterpret_cast<Partial*>(ws + cv.take(slots * nc * sizeof(Partial)));
    float* xy = reinterpret_cast<float*>(ws + cv.take(slots * 2 * sizeof(float)));
    ChainDesc* desc = reinterpret_cast<ChainDesc*>(ws + cv.take((size_t)a.B * sizeof(ChainDesc)));
    double* mass = reinterpret_cast<double*>(ws + cv.take((size_t)a.B * nc * sizeof(double)));
    const float c = (float)(1.4426950408889634 / (double)a.temperature);
    using raw = typename E::raw;
    const raw* tgt = static_cast<const raw*>(a.target);
    const raw* dft = static_cast<const raw*>(a.draft);
    const unsigned grid1 = (unsigned)(slots * nc);
    hipLaunchKernelGGL((k_chain_stats<E, VEC>), dim3(grid1), dim3(kBlock), 0, a.stream, tgt, dft,
                       a.tokens, a.cu, a.K_max, a.V, chunk, nc, c, part_t, part_d, xy);
    hipLaunchKernelGGL(k_chain_decide, dim3(a.B), dim3(kWave), 0, a.stream, part_t, part_d, xy,
                       a.tokens, a.uniforms, a.cu, a.K_max, a.V, nc, c, a.accepted_len, a.probs_out,
                       a.seq_status, desc);
    hipLaunchKernelGGL((k_chain_mass<E, VEC>), dim3((unsigned)((size_t)a.B * nc)), dim3(kBlock), 0,
                       a.stream, tgt, dft, desc, a.V, chunk, nc, c, mass);
    hipLaunchKernelGGL((k_chain_sample<E, VEC>), dim3(a.B), dim3(kBlock), 0, a.stream, tgt, dft,
                       part_t, desc, mass, a.K_max, a.V, chunk, nc, c, a.next_token, a.resid_mass_out);
    return hipGetLastError();
}

hipError_t launch_chain_full(const ChainArgs& a) {
    if (a.dtype == 1) {
        if (a.V % Bf16::kVec == 0) return chain_full_impl<Bf16, true>(a);
        return chain_full_impl<Bf16, false>(a);
    }
    if (a.V % F32::kVec == 0) return chain_full_impl<F32, true>(a);
    return chain_full_impl<F32, false>(a);
}

}  // namespace sd
