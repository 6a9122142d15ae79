// sd_walk.hip -- the DDTree walk with the rows read on demand, for a sampling
// target (T > 0) and for the argmax target (T = 0).
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io), §5 DDTree: verification walks along the token the
// target selects at each node; a node with no child carrying that token ends
// the walk and the token becomes the extra token. §1: temperature and
// truncation belong inside p, and the chain's ratio test is not a rule for a
// tree. Under sampling the target selects its token by drawing from its own
// row: the inverse CDF of softmax(x / T), in token-id order, at the node's
// uniform. The tree's nodes are fixed drafts, not samples from q, so no draft
// probability enters, and since no node is visited twice every draw uses a
// fresh uniform.
//
// Only the rows on the walk are ever needed, and the walk is sequential, so
// one 512-thread workgroup per sequence reads one row per step:
//   pass A  the row in 32768-token tiles (8 or 16 16-byte vectors per thread,
//           wave w holding a contiguous segment of each tile) -> the maximum
//           (sampling) or the lowest-id argmax (greedy);
//   pass B  (sampling) per-segment sums of 2^(x*c - m*c), c = log2(e)/T, from
//           the registers when the row is one tile, else re-read from L2;
//   pass C  (sampling) wave 0 finds the segment where the running sum passes
//           u * S, re-reads that segment and descends to the 64-vector step,
//           the lane and the element;
// then wave 0 matches the token against the node's children by a ballot.
#include "sd.h"
#include "sd_device.hpp"
#include "sd_internal.hpp"

#include <math.h>

namespace sd {

namespace {

constexpr int kWalkThreads = 512;
constexpr int kWalkWaves = kWalkThreads / kWave;
constexpr int kTileTokens = 32768;
constexpr int kMaxSeg = kWalkWaves * ((1 << 24) / kTileTokens);   // 4096 (V < 2^24)
constexpr int32_t kNoIdx = 0x7fffffff;

template <class E>
struct WalkShape {
    static constexpr int R = kTileTokens / (kWalkThreads * E::kVec);   // vectors per thread per tile
    static constexpr int kTileVec = kWalkThreads * R;
    static constexpr int kSegVec = kWave * R;                          // one wave's part of a tile
};

// Vector v of a row: 16-byte load when rows are vector aligned, else element
// loads; entries past the end of the row read as -inf.
template <class E, bool VEC>
__device__ __forceinline__ uint4 fetch_vec(const typename E::raw* rp, int64_t v, int V) {
    constexpr int EV = E::kVec;
    if (VEC) {
        if (v * EV < V) return load16_cached(rp, v);
        return E::neg_inf();
    }
    uint32_t w[4];
    if constexpr (EV == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t j = v * EV + 2 * k;
            const uint32_t lo = j < V ? (uint32_t)rp[j] : 0xff80u;
            const uint32_t hi = j + 1 < V ? (uint32_t)rp[j + 1] : 0xff80u;
            w[k] = lo | (hi << 16);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t j = v * EV + k;
            w[k] = j < V ? __float_as_uint(rp[j]) : 0xff800000u;
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Sum of one vector's weights 2^(x*c - mc), in element order (fp32).
template <class E>
__device__ __forceinline__ float vec_weight(const uint4& q, float c, float mc) {
    float f[E::kVec];
    E::unpack(q, f);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) s += fast_exp2(f[e] * c - mc);
    return s;
}

__device__ __forceinline__ bool idx_better(float v, int i, float bv, int bi) {
    // (value desc, index asc); an empty candidate never wins
    if (i == kNoIdx) return false;
    if (bi == kNoIdx) return true;
    return v > bv || (v == bv && i < bi);
}

// fp64 wave scans on DPP row operations (each half of the double moved by
// the same DPP control), so no step waits on an LDS permute. The whole wave
// must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long x = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = dpp_from<CTRL, ROWS>((uint32_t)x);
    const uint32_t hi = dpp_from<CTRL, ROWS>((uint32_t)(x >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Inclusive prefix sum across the wave (lane order): shifts of 1, 2, 4, 8
// inside each 16-lane row, then the row totals carried by row broadcasts.
__device__ __forceinline__ double wave_incl_scan_f64(double v) {
    v += dpp_f64<0x111, 0xf>(v);
    v += dpp_f64<0x112, 0xf>(v);
    v += dpp_f64<0x114, 0xf>(v);
    v += dpp_f64<0x118, 0xf>(v);
    v += dpp_f64<0x142, 0xa>(v);
    v += dpp_f64<0x143, 0xc>(v);
    return v;
}

// The previous lane's value (0 in lane 0): the exclusive scan from the inclusive one.
__device__ __forceinline__ double wave_prev_f64(double incl) { return dpp_f64<0x138, 0xf>(incl); }

// The last lane's value, in every lane (the wave total of an inclusive scan).
__device__ __forceinline__ double wave_last_f64(double incl) {
    const unsigned long long x = (unsigned long long)__double_as_longlong(incl);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)x, kWave - 1);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), kWave - 1);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double wave_total_f64(double v) { return wave_last_f64(wave_incl_scan_f64(v)); }

// The value of lane l (wave-uniform l), in every lane.
__device__ __forceinline__ double lane_f64(double v, int l) {
    const unsigned long long x = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// First index in [0, n) whose running sum of vals passes t, else the last
// index with a positive value (reached only through rounding), else -1.
// `rem` is t minus the running sum before the chosen index. Wave-uniform.
__device__ int wave_locate(const double* vals, int n, double t, double& rem) {
    const int lane = threadIdx.x & (kWave - 1);
    double base = 0.0;
    int last_pos = -1;
    double base_last = 0.0;
    for (int c0 = 0; c0 < n; c0 += kWave) {
        const int i = c0 + lane;
        const double v = i < n ? vals[i] : 0.0;
        const double incl = wave_incl_scan_f64(v);
        const double ex = wave_prev_f64(incl);
        const unsigned long long hit = __ballot(i < n && base + incl > t);
        if (hit) {
            const int l = __ffsll(hit) - 1;
            rem = t - (base + lane_f64(ex, l));
            return c0 + l;
        }
        const unsigned long long pos = __ballot(i < n && v > 0.0);
        if (pos) {
            const int l = 63 - __clzll(pos);
            last_pos = c0 + l;
            base_last = base + lane_f64(ex, l);
        }
        base += wave_last_f64(incl);
    }
    rem = t - base_last;
    return last_pos;
}

// The child of `node` carrying token g (the lowest node id), or -1: one
// ballot of the wave over the node table in LDS. Wave-uniform.
__device__ __forceinline__ int find_child(const int* tok, const int* par, int nn, int node, int g) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool hit = g >= 0 && lane >= 1 && lane < nn && par[lane] == node && tok[lane] == g;
    const unsigned long long h = __ballot(hit);
    return h ? (__ffsll(h) - 1) : -1;
}

template <class E, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kWalkThreads) void k_tree_walk_rows(
    const typename E::raw* __restrict__ rows, const int32_t* __restrict__ node_token,
    const int32_t* __restrict__ node_parent, const int32_t* __restrict__ n_nodes,
    const float* __restrict__ uniforms, int N, int V, float c, int32_t* __restrict__ path,
    int32_t* __restrict__ A_out, int32_t* __restrict__ next_out, int32_t* __restrict__ status_out) {
    using S = WalkShape<E>;
    constexpr int R = S::R;
    constexpr int EV = E::kVec;
    __shared__ int s_tok[SD_MAX_TREE_N];
    __shared__ int s_par[SD_MAX_TREE_N];
    __shared__ double s_seg[kMaxSeg];
    __shared__ float s_val[2][kWalkWaves];
    __shared__ int s_idx[2][kWalkWaves];
    __shared__ int s_out[2];   // token drawn (or -1: non-finite row), child (-1: none)

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    int nn = n_nodes[b];
    nn = nn < 1 ? 1 : (nn > N ? N : nn);
    if (tid < N) path[(int64_t)b * N + tid] = -1;
    const int64_t nvec = ((int64_t)V + EV - 1) / EV;
    const int ntiles = (int)((nvec + S::kTileVec - 1) / S::kTileVec);
    int node = 0, len = 0, next = -1, status = 0;
    // The node table goes to LDS after the root row's first loads are issued
    // (step 0 below); the barrier after pass A publishes it.
    auto load_node_table = [&]() {
        if (tid < N) {
            s_tok[tid] = node_token[(int64_t)b * N + tid];
            s_par[tid] = node_parent[(int64_t)b * N + tid];
        }
    };

    for (int step = 0; step < N; ++step) {
        const typename E::raw* rp = rows + ((int64_t)b * N + node) * (int64_t)V;
        const int par_buf = step & 1;
        // the node's uniform, issued first: it is consumed only after pass B
        const float u = GREEDY ? 0.0f : uniforms[(int64_t)b * N + node];
        uint4 q[R];
        auto load_tile = [&](int t) {
            const int64_t v0 = (int64_t)t * S::kTileVec + (int64_t)w * S::kSegVec + lane;
#pragma unroll
            for (int r = 0; r < R; ++r) q[r] = fetch_vec<E, VEC>(rp, v0 + r * kWave, V);
        };
        // pass A: maximum, or (value desc, index asc) argmax
        float best = -INFINITY;
        int bidx = kNoIdx;
        for (int t = 0; t < ntiles; ++t) {
            load_tile(t);
            if (step == 0 && t == 0) load_node_table();
            const int64_t v0 = (int64_t)t * S::kTileVec + (int64_t)w * S::kSegVec + lane;
            if (GREEDY) {
                // the thread's maximum over this tile (NaN skipped) from the
                // vectors' maxima, then its first occurrence: the first vector
                // that holds it, the first element there. Entries past the row
                // read as -inf and come after the row's own in this order, so
                // an occurrence past the row means the thread holds no value.
                float vmx[R];
                float M = NAN;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float f[EV];
                    E::unpack(q[r], f);
                    vmx[r] = f[0];
#pragma unroll
                    for (int e = 1; e < EV; ++e) vmx[r] = fmaxf(vmx[r], f[e]);
                    M = fmaxf(M, vmx[r]);
                }
                if (M == M) {
                    int rs = 0;
#pragma unroll
                    for (int r = R - 1; r >= 0; --r) rs = vmx[r] == M ? r : rs;
                    uint4 qs = q[0];
#pragma unroll
                    for (int r = 1; r < R; ++r) {
                        const bool t2 = rs == r;
                        qs.x = t2 ? q[r].x : qs.x;
                        qs.y = t2 ? q[r].y : qs.y;
                        qs.z = t2 ? q[r].z : qs.z;
                        qs.w = t2 ? q[r].w : qs.w;
                    }
                    float f[EV];
                    E::unpack(qs, f);
                    int es = 0;
#pragma unroll
                    for (int e = EV - 1; e >= 0; --e) es = f[e] == M ? e : es;
                    const int j = (int)((v0 + rs * kWave) * EV + es);
                    if (j < V && (M > best || bidx == kNoIdx)) {
                        best = M;
                        bidx = j;
                    }
                }
            } else {
                // NaN skipped (fmaxf returns the other operand); past the row -inf
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float f[EV];
                    E::unpack(q[r], f);
#pragma unroll
                    for (int e = 0; e < EV; ++e) best = fmaxf(best, f[e]);
                }
            }
        }
        if (GREEDY) {
            // (value desc, index asc) as one 64-bit key, larger is better
            // (0: no value), reduced over the wave on DPP row operations
            uint32_t khi = 0u, klo = 0u;
            if (bidx != kNoIdx) {
                const uint32_t u = __float_as_uint(best == 0.f ? 0.f : best);
                khi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
                klo = 0xffffffffu - (uint32_t)bidx;
            }
            wave_max_key64(khi, klo);
            if (khi != 0u) {
                const uint32_t u = (khi & 0x80000000u) ? (khi & 0x7fffffffu) : ~khi;
                best = __uint_as_float(u);
                bidx = (int)(0xffffffffu - klo);
            } else {
                best = -INFINITY;
                bidx = kNoIdx;
            }
        } else {
            best = wave_max(best);
        }
        // (double-buffered by step parity: the greedy walk has no other barrier
        // between one step's reads and the next step's writes)
        if (lane == 0) {
            s_val[par_buf][w] = best;
            s_idx[par_buf][w] = bidx;
        }
        __syncthreads();
        float m = s_val[par_buf][0];
        int mi = s_idx[par_buf][0];
#pragma unroll
        for (int i = 1; i < kWalkWaves; ++i) {
            if (GREEDY) {
                if (idx_better(s_val[par_buf][i], s_idx[par_buf][i], m, mi)) {
                    m = s_val[par_buf][i];
                    mi = s_idx[par_buf][i];
                }
            } else {
                m = nmax(m, s_val[par_buf][i]);
            }
        }
        int g, child;
        if (GREEDY) {
            // every wave finds the child itself (same LDS data, same answer)
            g = mi == kNoIdx ? -1 : mi;
            child = find_child(s_tok, s_par, nn, node, g);
        } else {
            const bool finite_m = isfinite(m);
            const float mc = m * c;
            // pass B: per-segment weight sums (segment = one wave's part of a
            // tile); the per-vector sums of the last tile stay in registers
            float lw[R];
#pragma unroll
            for (int r = 0; r < R; ++r) lw[r] = 0.0f;
            if (finite_m) {
                for (int t = 0; t < ntiles; ++t) {
                    if (ntiles > 1) load_tile(t);
                    double acc = 0.0;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        lw[r] = vec_weight<E>(q[r], c, mc);
                        acc += (double)lw[r];
                    }
                    acc = wave_total_f64(acc);
                    if (lane == 0) s_seg[t * kWalkWaves + w] = acc;
                }
            }
            __syncthreads();
            // every wave locates the segment (same LDS data, same answer); the
            // wave holding it descends from its registers
            const int nseg = ntiles * kWalkWaves;
            double tot = 0.0;
            for (int i = lane; i < nseg; i += kWave) tot += s_seg[i];
            tot = wave_total_f64(tot);
            const bool valid = finite_m && isfinite(tot) && tot > 0.0;
            double rem = 0.0;
            const int seg = valid ? wave_locate(s_seg, nseg, (double)u * tot, rem) : -1;
            const int owner = seg >= 0 ? seg % kWalkWaves : 0;
            if (w == owner) {
                int tok = -1;
                if (seg >= 0) {
                    const int tseg = seg / kWalkWaves;
                    if (tseg != ntiles - 1) {
                        load_tile(tseg);
#pragma unroll
                        for (int r = 0; r < R; ++r) lw[r] = vec_weight<E>(q[r], c, mc);
                    }
                    // the 64-vector step, then the lane, then the element
                    int rs = -1, last_pos = -1;
                    double base = 0.0, rem2 = 0.0, base_last = 0.0;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const double st = wave_total_f64((double)lw[r]);
                        if (rs < 0 && base + st > rem) {
                            rs = r;
                            rem2 = rem - base;
                        }
                        if (st > 0.0) {
                            last_pos = r;
                            base_last = base;
                        }
                        base += st;
                    }
                    if (rs < 0) {
                        rs = last_pos < 0 ? 0 : last_pos;
                        rem2 = rem - base_last;
                    }
                    uint4 mine = q[0];
                    float mw = lw[0];
#pragma unroll
                    for (int r = 1; r < R; ++r)
                        if (r == rs) {
                            mine = q[r];
                            mw = lw[r];
                        }
                    const double incl = wave_incl_scan_f64((double)mw);
                    const double ex = wave_prev_f64(incl);
                    const unsigned long long hit = __ballot(incl > rem2);
                    const unsigned long long pos = __ballot(mw > 0.0f);
                    const int l = hit ? (__ffsll(hit) - 1) : (pos ? 63 - __clzll(pos) : -1);
                    if (l >= 0) {
                        const double rem3 = rem2 - lane_f64(ex, l);
                        float f[EV];
                        E::unpack(mine, f);
                        int e_hit = -1, e_last = -1;
                        double cum = 0.0;
#pragma unroll
                        for (int e = 0; e < EV; ++e) {
                            const float we = fast_exp2(f[e] * c - mc);
                            cum += (double)we;
                            if (e_hit < 0 && cum > rem3) e_hit = e;
                            if (we > 0.0f) e_last = e;
                        }
                        const int e_sel = e_hit >= 0 ? e_hit : e_last;
                        const int64_t vsel = (int64_t)tseg * S::kTileVec + (int64_t)owner * S::kSegVec +
                                             (int64_t)rs * kWave + lane;
                        const int cand = e_sel >= 0 ? (int)(vsel * EV + e_sel) : -1;
                        tok = __shfl(cand, l, kWave);
                    }
                }
                const int ch = find_child(s_tok, s_par, nn, node, tok);
                if (lane == 0) {
                    s_out[0] = tok;
                    s_out[1] = ch;
                }
            }
            __syncthreads();
            g = s_out[0];
            child = s_out[1];
        }
        if (g < 0) {
            status |= SD_SEQ_NONFINITE;
            next = -1;
            break;
        }
        if (child < 0) {
            next = g;
            break;
        }
        if (tid == 0) path[(int64_t)b * N + len] = child;
        ++len;
        node = child;
    }
    if (tid == 0) {
        A_out[b] = len;
        next_out[b] = next;
        if (status_out) status_out[b] = status;
    }
}

template <class E, bool VEC>
hipError_t walk_impl(const void* target, const int32_t* tok, const int32_t* par, const int32_t* nn,
                     const float* uniforms, int B, int N, int V, float temperature, int32_t* path,
                     int32_t* A, int32_t* next, int32_t* status, hipStream_t stream) {
    const auto* rows = static_cast<const typename E::raw*>(target);
    if (temperature == 0.0f) {
        PassTimer::launch(k_tree_walk_rows<E, VEC, true>, dim3(B), dim3(kWalkThreads), stream, rows,
                          tok, par, nn, uniforms, N, V, 0.0f, path, A, next, status);
    } else {
        const float c = (float)(1.4426950408889634 / (double)temperature);
        PassTimer::launch(k_tree_walk_rows<E, VEC, false>, dim3(B), dim3(kWalkThreads), stream, rows,
                          tok, par, nn, uniforms, N, V, c, path, A, next, status);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_walk_rows(const void* target, int dtype, const int32_t* tok,
                                 const int32_t* par, const int32_t* n_nodes, const float* uniforms,
                                 int B, int N, int V, float temperature, int32_t* path,
                                 int32_t* accepted_len, int32_t* next_token, int32_t* seq_status,
                                 hipStream_t stream) {
    if (dtype == 1) {
        if (V % Bf16::kVec == 0)
            return walk_impl<Bf16, true>(target, tok, par, n_nodes, uniforms, B, N, V, temperature,
                                         path, accepted_len, next_token, seq_status, stream);
        return walk_impl<Bf16, false>(target, tok, par, n_nodes, uniforms, B, N, V, temperature,
                                      path, accepted_len, next_token, seq_status, stream);
    }
    if (V % F32::kVec == 0)
        return walk_impl<F32, true>(target, tok, par, n_nodes, uniforms, B, N, V, temperature, path,
                                    accepted_len, next_token, seq_status, stream);
    return walk_impl<F32, false>(target, tok, par, n_nodes, uniforms, B, N, V, temperature, path,
                                 accepted_len, next_token, seq_status, stream);
}

}  // namespace sd
