// sd_topk.hip -- exact top-k of long rows, the top-k chain decision, and the
// DDTree best-first tree build.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io): §1 (probability truncation must be folded into both p
// and q; accept test, first rejection, residual correction, extra token) and
// §5 DDTree (score Q(u) = prod q_i(u_i) of the displayed equation, prefixes
// chosen best-first with a heap under a node budget, numbered as chosen, each
// node seeing itself and its ancestors).
//
// k_topk_rows: one workgroup per row streams the row once. Each element whose
// key (value desc, id asc, NaN never kept) beats the workgroup's current k-th
// best key is appended to an LDS candidate buffer; when the buffer overflows it
// is sorted (bitonic, LDS) and cut back to k, which raises the threshold. The
// result is exact for any arrival order, because an element is dropped only
// when k kept elements already beat it.
#include "sd_device.hpp"
#include "sd_internal.hpp"

#include <math.h>

namespace sd {

namespace {

constexpr int kCap = 1024;          // candidate buffer entries (u64 keys) in LDS
constexpr int kTopkUnroll = 2;

struct TopEntry {
    int32_t idx;
    float x;
};

// Order-preserving 32-bit image of a non-NaN float; -0 and +0 map together.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
    if (x == 0.f) x = 0.f;
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}
// Larger key = better: higher value, then lower id.
__device__ __forceinline__ unsigned long long make_key(float x, int idx) {
    return ((unsigned long long)ordered_bits(x) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)idx);
}

// Sorts buf[0..kCap) descending (bitonic network). All kBlock threads call it.
__device__ void bitonic_desc(unsigned long long* buf) {
    for (int size = 2; size <= kCap; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < kCap / 2; i += kBlock) {
                const int lo = 2 * stride * (i / stride) + (i % stride);
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long a = buf[lo], b = buf[hi];
                if ((a < b) == desc) {
                    buf[lo] = b;
                    buf[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

// Row task -> row pointer. Chain: task = ((b * slots) + s) * 2 + side, side 0 =
// target row s (s <= k_b), side 1 = draft row s (s < k_b). Tree: task = b*K + d.
template <class E>
__device__ const typename E::raw* topk_row(const typename E::raw* tgt, const typename E::raw* dft,
                                           const int32_t* cu, int K_max, int V, int task,
                                           bool chain) {
    if (!chain) return tgt + (int64_t)task * V;
    const int side = task & 1;
    const int rest = task >> 1;
    const int slots = K_max + 1;
    const int s = rest % slots;
    const int b = rest / slots;
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    if (side == 0) return (s <= k) ? tgt + ((int64_t)d0 + b + s) * V : nullptr;
    return (s < k) ? dft + ((int64_t)d0 + s) * V : nullptr;
}

template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) void k_topk_rows(const typename E::raw* __restrict__ tgt,
                                                      const typename E::raw* __restrict__ dft,
                                                      const int32_t* __restrict__ cu, int K_max,
                                                      int V, int topk, int chain,
                                                      TopEntry* __restrict__ out,
                                                      int32_t* __restrict__ out_count) {
    __shared__ unsigned long long buf[kCap];
    __shared__ int cnt;
    __shared__ unsigned long long thr;
    constexpr int EV = E::kVec;
    constexpr int U = kTopkUnroll;
    const int task = blockIdx.x;
    const typename E::raw* row = topk_row<E>(tgt, dft, cu, K_max, V, task, chain != 0);
    if (row == nullptr) return;
    if (threadIdx.x == 0) {
        cnt = 0;
        thr = 0ull;
    }
    __syncthreads();
    const int nvec = (V + EV - 1) / EV;
    for (int v0 = 0; v0 < nvec; v0 += kBlock * U) {
        float f[U][EV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = v0 + u * kBlock + threadIdx.x;
            if (VEC) {
                if (vi < nvec) {
                    E::unpack(load16(row, vi), f[u]);
                } else {
#pragma unroll
                    for (int e = 0; e < EV; ++e) f[u][e] = NAN;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const int j = vi * EV + e;
                    f[u][e] = (vi < nvec && j < V) ? E::at(row, j) : NAN;
                }
            }
        }
        // pending bit per element: key beats the threshold and is not yet stored
        int n_now = 0;
        unsigned pending = 0;
        unsigned long long t = thr;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const float x = f[u][e];
                const int idx = (v0 + u * kBlock + threadIdx.x) * EV + e;
                if (x == x && make_key(x, idx) > t) pending |= 1u << (u * EV + e);
            }
        for (;;) {
            bool overflow = false;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const unsigned bit = 1u << (u * EV + e);
                    if (pending & bit) {
                        const int pos = atomicAdd(&cnt, 1);
                        if (pos < kCap) {
                            const int idx = (v0 + u * kBlock + threadIdx.x) * EV + e;
                            buf[pos] = make_key(f[u][e], idx);
                            pending &= ~bit;
                        } else {
                            overflow = true;
                        }
                    }
                }
            (void)overflow;
            __syncthreads();
            const int n = cnt;
            __syncthreads();            // every thread has read cnt before it changes
            if (n <= kCap) {
                n_now = n;
                break;
            }
            // overflow: sort the full buffer, keep the best topk, raise the threshold
            bitonic_desc(buf);
            for (int i = topk + threadIdx.x; i < kCap; i += kBlock) buf[i] = 0ull;
            if (threadIdx.x == 0) {
                cnt = topk;
                thr = buf[topk - 1];
            }
            __syncthreads();
            t = thr;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const unsigned bit = 1u << (u * EV + e);
                    if ((pending & bit) && !(make_key(f[u][e], (v0 + u * kBlock + threadIdx.x) * EV + e) > t))
                        pending &= ~bit;
                }
        }
        // Past half full: cut back to topk now, which raises the threshold, so
        // that later steps rarely overflow.
        if (n_now > kCap / 2) {
            for (int i = n_now + threadIdx.x; i < kCap; i += kBlock) buf[i] = 0ull;
            __syncthreads();
            bitonic_desc(buf);
            for (int i = topk + threadIdx.x; i < kCap; i += kBlock) buf[i] = 0ull;
            if (threadIdx.x == 0) {
                cnt = n_now < topk ? n_now : topk;
                if (n_now >= topk) thr = buf[topk - 1];
            }
            __syncthreads();
        }
    }
    // final sort and output
    const int n = cnt;
    for (int i = n + threadIdx.x; i < kCap; i += kBlock) buf[i] = 0ull;
    __syncthreads();
    bitonic_desc(buf);
    const int kept = n < topk ? n : topk;
    for (int i = threadIdx.x; i < topk; i += kBlock) {
        TopEntry te;
        if (i < kept) {
            const unsigned long long key = buf[i];
            te.idx = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
            te.x = from_ordered((uint32_t)(key >> 32));
        } else {
            te.idx = -1;
            te.x = -INFINITY;
        }
        out[(int64_t)task * topk + i] = te;
    }
    if (threadIdx.x == 0) out_count[task] = kept;
}

// ---------------------------------------------------------------------------
// Chain decision over top-k lists (fp64 throughout; the lists are tiny).
// ---------------------------------------------------------------------------
struct ListStat {
    double m;      // max of z = x / T over the kept set
    double S;      // sum of exp(z - m)
    bool valid;
};

// One wave: softmax statistics of a kept list.
__device__ ListStat list_stat(const TopEntry* L, int n, double T) {
    const int lane = threadIdx.x;
    ListStat r;
    r.valid = n > 0;
    if (!r.valid) {
        r.m = 0.0;
        r.S = 0.0;
        return r;
    }
    r.m = (double)L[0].x / T;           // list is sorted by value desc
    double s = 0.0;
    for (int i = lane; i < n; i += kWave) s += exp((double)L[i].x / T - r.m);
    s = wave_sum(s);
    r.S = s;
    r.valid = isfinite(r.m) && isfinite(s) && s > 0.0;
    return r;
}

// Probability of token y under a kept list (0 if not kept or invalid row).
__device__ double list_prob(const TopEntry* L, int n, const ListStat& st, int y, double T) {
    const int lane = threadIdx.x;
    double p = 0.0;
    for (int i = lane; i < n; i += kWave)
        if (L[i].idx == y) p = exp((double)L[i].x / T - st.m) / st.S;
    p = wave_sum(p);        // at most one lane holds y
    return st.valid ? p : 0.0;
}

// Inverse CDF in token-id order over the entries of target list P (at most
// SD_MAX_TOPK): weight w_j = p_j - q_j (clamped at 0) when D is given,
// otherwise p_j. Entries are ranked by id with a counting sort in LDS.
__device__ int list_inverse_cdf(const TopEntry* P, int np, const ListStat& sp, const TopEntry* D,
                                int nd, const ListStat& sq, bool residual, double T, double u,
                                double* wbuf, int* ibuf, double* R_out) {
    const int lane = threadIdx.x;
    for (int i = lane; i < np; i += kWave) {
        const int id = P[i].idx;
        double w = exp((double)P[i].x / T - sp.m) / sp.S;
        if (residual) {
            double q = 0.0;
            if (sq.valid)
                for (int j = 0; j < nd; ++j)
                    if (D[j].idx == id) q = exp((double)D[j].x / T - sq.m) / sq.S;
            w = w - q;
            if (!(w > 0.0)) w = 0.0;
        }
        int rank = 0;
        for (int j = 0; j < np; ++j) rank += (P[j].idx < id);
        wbuf[rank] = w;
        ibuf[rank] = id;
    }
    __syncthreads();
    int pick = -1;
    double R = 0.0;
    if (lane == 0) {
        for (int i = 0; i < np; ++i) R += wbuf[i];
        const double target = u * R;
        double C = 0.0;
        int last = -1;
        for (int i = 0; i < np; ++i) {
            C += wbuf[i];
            if (wbuf[i] > 0.0) last = ibuf[i];
            if (C > target && wbuf[i] > 0.0) {
                pick = ibuf[i];
                break;
            }
        }
        if (pick < 0) pick = last;
    }
    __syncthreads();
    *R_out = __shfl(R, 0, kWave);
    return __shfl(pick, 0, kWave);
}

__global__ __launch_bounds__(kWave) void k_chain_topk_decide(
    const TopEntry* __restrict__ lists, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ tok, const float* __restrict__ uni, const int32_t* __restrict__ cu,
    int K_max, int V, int topk, float temperature, int32_t* __restrict__ A_out,
    int32_t* __restrict__ next_out, float* __restrict__ probs_out, float* __restrict__ R_out,
    int32_t* __restrict__ status_out) {
    __shared__ double wbuf[kMaxTopk];
    __shared__ int ibuf[kMaxTopk];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int slots = K_max + 1;
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    const double T = (double)temperature;
    auto list_of = [&](int s, int side) { return lists + (((int64_t)b * slots + s) * 2 + side) * topk; };
    auto count_of = [&](int s, int side) { return counts[((int64_t)b * slots + s) * 2 + side]; };
    int A = k, status = 0;
    for (int i = 0; i < k; ++i) {
        const TopEntry* P = list_of(i, 0);
        const TopEntry* D = list_of(i, 1);
        const int np = count_of(i, 0), nd = count_of(i, 1);
        const ListStat sp = list_stat(P, np, T);
        const ListStat sq = list_stat(D, nd, T);
        const int y = tok[d0 + i];
        const bool yok = (y >= 0 && y < V);
        const double py = yok ? list_prob(P, np, sp, y, T) : 0.0;
        const double qy = yok ? list_prob(D, nd, sq, y, T) : 0.0;
        if (probs_out && lane == 0) {
            probs_out[2 * (int64_t)(d0 + i)] = (float)py;
            probs_out[2 * (int64_t)(d0 + i) + 1] = (float)qy;
        }
        if (A == k) {
            const double u = (double)uni[d0 + b + i];
            const bool acc = sp.valid && sq.valid && yok && py > 0.0 && u * qy <= py;
            if (!yok) status |= 1;
            if (!(sp.valid && sq.valid)) status |= 2;
            if (!acc) A = i;
        }
    }
    const double uf = (double)uni[d0 + b + k];
    int next = -1;
    double R = 0.0;
    if (A < k) {
        const TopEntry* P = list_of(A, 0);
        const TopEntry* D = list_of(A, 1);
        const int np = count_of(A, 0), nd = count_of(A, 1);
        const ListStat sp = list_stat(P, np, T);
        const ListStat sq = list_stat(D, nd, T);
        if (sp.valid) {
            next = list_inverse_cdf(P, np, sp, D, nd, sq, true, T, uf, wbuf, ibuf, &R);
            if (!(R > 0.0)) {
                double dummy;
                next = list_inverse_cdf(P, np, sp, D, nd, sq, false, T, uf, wbuf, ibuf, &dummy);
            }
        }
    } else {
        const TopEntry* P = list_of(k, 0);
        const int np = count_of(k, 0);
        const ListStat sp = list_stat(P, np, T);
        if (sp.valid) {
            double dummy;
            next = list_inverse_cdf(P, np, sp, P, 0, sp, false, T, uf, wbuf, ibuf, &dummy);
        } else {
            status |= 2;
        }
        R = 0.0;
    }
    if (lane == 0) {
        A_out[b] = A;
        next_out[b] = next;
        if (R_out) R_out[b] = (float)R;
        if (status_out) status_out[b] = status;
    }
}

// ---------------------------------------------------------------------------
// DDTree best-first build: one wave per sequence. The frontier (at most 64
// prefixes, one per lane) holds, for every popped node, its first child and
// its next sibling; a pop is a wave argmax under (Q desc, depth asc, rank tuple
// lexicographically asc). The rank tuple is packed 6 bits per depth, big-end
// first, in two 64-bit words, so equal-depth tuples compare as integers.
// ---------------------------------------------------------------------------
struct Front {
    float Q;
    int depth;
    unsigned long long w0, w1;
    int parent;
    int rank;        // rank at the last depth
    int valid;
};

__device__ __forceinline__ bool front_better(const Front& a, const Front& b) {
    if (!a.valid) return false;
    if (!b.valid) return true;
    if (a.Q != b.Q) return a.Q > b.Q;
    if (a.depth != b.depth) return a.depth < b.depth;
    if (a.w0 != b.w0) return a.w0 < b.w0;
    return a.w1 < b.w1;
}

__device__ __forceinline__ void set_rank(Front& f, int pos, int r) {
    if (pos < 10) {
        const int sh = 54 - 6 * pos;
        f.w0 = (f.w0 & ~(0x3full << sh)) | ((unsigned long long)r << sh);
    } else {
        const int sh = 54 - 6 * (pos - 10);
        f.w1 = (f.w1 & ~(0x3full << sh)) | ((unsigned long long)r << sh);
    }
}

__device__ Front shfl_front(const Front& f, int src) {
    Front r;
    r.Q = __shfl(f.Q, src, kWave);
    r.depth = __shfl(f.depth, src, kWave);
    r.w0 = __shfl(f.w0, src, kWave);
    r.w1 = __shfl(f.w1, src, kWave);
    r.parent = __shfl(f.parent, src, kWave);
    r.rank = __shfl(f.rank, src, kWave);
    r.valid = __shfl(f.valid, src, kWave);
    return r;
}

__global__ __launch_bounds__(kWave) void k_tree_build(
    const TopEntry* __restrict__ lists, const int32_t* __restrict__ counts, int K, int N, int W,
    int32_t* __restrict__ node_token, int32_t* __restrict__ node_parent,
    int32_t* __restrict__ node_depth, float* __restrict__ node_score,
    unsigned long long* __restrict__ node_anc, int32_t* __restrict__ n_nodes) {
    __shared__ float qv[kMaxTreeK][64];
    __shared__ int tv[kMaxTreeK][64];
    __shared__ int cntv[kMaxTreeK];
    __shared__ float nscore[64];
    __shared__ unsigned long long nanc[64];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    for (int d = 0; d < K; ++d) {
        const TopEntry* L = lists + ((int64_t)b * K + d) * W;
        if (lane < W) {
            qv[d][lane] = L[lane].x;
            tv[d][lane] = L[lane].idx;
        }
        if (lane == 0) cntv[d] = counts[(int64_t)b * K + d];
    }
    __shared__ int otok[64], opar[64], odep[64];
    if (lane < 64) {
        otok[lane] = -1;
        opar[lane] = -1;
        odep[lane] = 0;
        nscore[lane] = 0.f;
        nanc[lane] = 0ull;
    }
    __syncthreads();
    if (lane == 0) {
        nscore[0] = 1.0f;
        nanc[0] = 1ull;
    }
    Front f;
    f.valid = 0;
    f.Q = 0.f;
    f.depth = 0;
    f.w0 = 0ull;
    f.w1 = 0ull;
    f.parent = -1;
    f.rank = 0;
    if (lane == 0 && K > 0 && cntv[0] > 0) {
        f.valid = 1;
        f.Q = 1.0f * qv[0][0];
        f.depth = 1;
        f.parent = 0;
        f.rank = 0;
    }
    __syncthreads();
    int n = 1;
    while (n < N) {
        // wave argmax
        Front best = f;
        int best_lane = lane;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const Front other = shfl_front(best, lane ^ o);
            const int ol = __shfl_xor(best_lane, o, kWave);
            if (front_better(other, best)) {
                best = other;
                best_lane = ol;
            }
        }
        // every lane now holds the same winner
        if (!best.valid) break;
        const int m = best.depth;
        const int tokn = tv[m - 1][best.rank];
        const int par = best.parent;
        const unsigned long long anc = nanc[par] | (1ull << n);
        if (lane == 0) {
            otok[n] = tokn;
            opar[n] = par;
            odep[n] = m;
            nscore[n] = best.Q;
            nanc[n] = anc;
        }
        __syncthreads();
        // the winner's slot becomes the first child of node n
        if (lane == best_lane) {
            if (m < K && cntv[m] > 0) {
                f.Q = best.Q * qv[m][0];
                f.depth = m + 1;
                set_rank(f, m, 0);
                f.parent = n;
                f.rank = 0;
                f.valid = 1;
            } else {
                f.valid = 0;
            }
        }
        // the next sibling goes to the lowest free lane
        if (best.rank + 1 < cntv[m - 1]) {
            const unsigned long long freem = __ballot(!f.valid);
            const int dst = __ffsll(freem) - 1;
            if (lane == dst) {
                f = best;
                f.Q = nscore[par] * qv[m - 1][best.rank + 1];
                set_rank(f, m - 1, best.rank + 1);
                f.rank = best.rank + 1;
                f.valid = 1;
            }
        }
        ++n;
    }
    __syncthreads();
    const int64_t o0 = (int64_t)b * N;
    if (lane < N) {
        node_token[o0 + lane] = otok[lane];
        node_parent[o0 + lane] = opar[lane];
        node_depth[o0 + lane] = odep[lane];
        node_score[o0 + lane] = nscore[lane];
        node_anc[o0 + lane] = nanc[lane];
    }
    if (lane == 0) n_nodes[b] = n;
}

}  // namespace

size_t chain_topk_ws_bytes(int B, int K_max, int V, int top_k) {
    (void)V;
    const size_t tasks = (size_t)B * (K_max + 1) * 2;
    Carve cv;
    cv.take(tasks * top_k * sizeof(TopEntry));
    cv.take(tasks * sizeof(int32_t));
    return cv.off;
}

size_t tree_build_ws_bytes(int B, int K, int V, int N) {
    const int W = (N - 1) < V ? (N - 1) : V;
    const size_t tasks = (size_t)B * K;
    Carve cv;
    cv.take(tasks * W * sizeof(TopEntry));
    cv.take(tasks * sizeof(int32_t));
    return cv.off;
}

template <class E, bool VEC>
static hipError_t chain_topk_impl(const ChainArgs& a) {
    const size_t tasks = (size_t)a.B * (a.K_max + 1) * 2;
    Carve cv;
    char* ws = static_cast<char*>(a.ws);
    TopEntry* lists = reinterpret_cast<TopEntry*>(ws + cv.take(tasks * a.top_k * sizeof(TopEntry)));
    int32_t* counts = reinterpret_cast<int32_t*>(ws + cv.take(tasks * sizeof(int32_t)));
    using raw = typename E::raw;
    PassTimer::mark_before(a.stream);
    hipLaunchKernelGGL((k_topk_rows<E, VEC>), dim3((unsigned)tasks), dim3(kBlock), 0, a.stream,
                       static_cast<const raw*>(a.target), static_cast<const raw*>(a.draft), a.cu,
                       a.K_max, a.V, a.top_k, 1, lists, counts);
    PassTimer::mark_after(a.stream);
    hipLaunchKernelGGL(k_chain_topk_decide, dim3(a.B), dim3(kWave), 0, a.stream, lists, counts,
                       a.tokens, a.uniforms, a.cu, a.K_max, a.V, a.top_k, a.temperature,
                       a.accepted_len, a.next_token, a.probs_out, a.resid_mass_out, a.seq_status);
    return hipGetLastError();
}

hipError_t launch_chain_topk(const ChainArgs& a) {
    if (a.dtype == 1) {
        if (a.V % Bf16::kVec == 0) return chain_topk_impl<Bf16, true>(a);
        return chain_topk_impl<Bf16, false>(a);
    }
    if (a.V % F32::kVec == 0) return chain_topk_impl<F32, true>(a);
    return chain_topk_impl<F32, false>(a);
}

hipError_t launch_tree_build(const float* marg, int B, int K, int V, int N, int32_t* tok,
                             int32_t* par, int32_t* dep, float* score, uint64_t* anc,
                             int32_t* n_nodes, void* ws, hipStream_t stream) {
    const int W = (N - 1) < V ? (N - 1) : V;
    const size_t tasks = (size_t)B * K;
    Carve cv;
    char* w = static_cast<char*>(ws);
    TopEntry* lists = reinterpret_cast<TopEntry*>(w + cv.take(tasks * W * sizeof(TopEntry)));
    int32_t* counts = reinterpret_cast<int32_t*>(w + cv.take(tasks * sizeof(int32_t)));
    PassTimer::mark_before(stream);
    if (tasks > 0) {
        if (V % F32::kVec == 0)
            hipLaunchKernelGGL((k_topk_rows<F32, true>), dim3((unsigned)tasks), dim3(kBlock), 0,
                               stream, marg, marg, nullptr, 0, V, W, 0, lists, counts);
        else
            hipLaunchKernelGGL((k_topk_rows<F32, false>), dim3((unsigned)tasks), dim3(kBlock), 0,
                               stream, marg, marg, nullptr, 0, V, W, 0, lists, counts);
    }
    PassTimer::mark_after(stream);
    hipLaunchKernelGGL(k_tree_build, dim3(B), dim3(kWave), 0, stream, lists, counts, K, N, W, tok,
                       par, dep, score, reinterpret_cast<unsigned long long*>(anc), n_nodes);
    return hipGetLastError();
}

}  // namespace sd
