// sd_chain.hip -- stochastic chain verification over the full vocabulary.
//
// Implements the chain rule of the page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、
// DDTree 与 DSpark" (chzhyang.github.io), §1: accept y_i iff u_i q_i(y_i) <= p_i(y_i)
// (the acceptance-probability equation alpha = min(1, p/q)), stop at the first
// rejection (the A B C D example), draw the correction token from the
// normalised positive residual [p - q]+ or, when all pass, the extra token from
// p; temperature is folded into both p and q.
//
// Launches on the caller's stream:
//   1. k_chain_stats  grid (sequence, slot, [row,] chunk): the one pass over
//      every row. Slot i < k_b has target row i and draft row i, streamed by
//      one workgroup per row in the first phase and together in later phases;
//      slot k_b has the extra-token row. Each workgroup writes the softmax
//      partial (o, S) of its chunk of each of its rows and, for chunk 0 of the
//      target row, the two logits at y_i.
//   2. k_chain_decide one wave per sequence: combines the partials of each row
//      exactly (integer references: a power-of-two rescale), evaluates
//      p_i(y_i), q_i(y_i) in fp64, the accept bits and A (wave ballot), and the
//      descriptor of the decision row(s).
//   3. k_chain_mass   grid (sequence, 16K-token chunk): re-reads only the
//      decision row(s) for the weight mass of the residual (or of p for the
//      extra token) per 512-token piece.
//   4. k_chain_sample one wave per sequence: prefix over the piece masses, then
//      one piece scan for the final token.
// A large batch runs 2-4 of the last phase as one launch, k_chain_resolve,
// one workgroup per sequence; there an extra token's row is weighed only in
// the chunk that the row's chunk partials show to hold the draw. Phases: the positions are streamed in slot
// ranges (1 and 2 per range); a sequence rejected in an early range streams
// none of its later rows.
#include "sd_device.hpp"
#include "sd_internal.hpp"

#include <math.h>

#ifndef SD_STATS_UNROLL
#define SD_STATS_UNROLL 2
#endif

namespace sd {

namespace {

constexpr int kModeResidual = 0;
constexpr int kModeExtra = 1;
constexpr int kModeNone = 2;
constexpr int kU = SD_STATS_UNROLL;
#ifndef SD_MASS_DPP
#define SD_MASS_DPP 1
#endif
// Phase boundaries of a phased verification: phase i streams the slots
// (positions) from the previous boundary up to this one; the last phase runs
// to the end of the window.
#ifndef SD_PHASE_BOUNDS
#define SD_PHASE_BOUNDS 2
#endif
constexpr int kPhaseBounds[] = {SD_PHASE_BOUNDS};
constexpr int kMaxPhases = (int)(sizeof(kPhaseBounds) / sizeof(int)) + 1;
constexpr size_t kPhaseMinElems = size_t(1) << 24;     // logits in the window
// The first phase of a phased verification streams one row per workgroup (1)
// or a slot's target and draft rows together (0).
#ifndef SD_SPLIT_FIRST_PHASE
#define SD_SPLIT_FIRST_PHASE 1
#endif
constexpr int kSplitFirstPhase = SD_SPLIT_FIRST_PHASE;
// A one-pass chunk sum is kept only below 2^64 (its reference was then close
// enough to the chunk's maximum); otherwise the exact two-pass path runs.
constexpr double kFastSumLimit = 18446744073709551616.0;

struct ChainDesc {
    int32_t mode;
    int32_t A;
    int32_t t_row;      // target row the final token is drawn from
    int32_t d_row;      // draft row of the residual; -1 when q counts as 0
    float u;            // the final uniform
    float O_p, O_q;     // row references (integers)
    int32_t slot;       // extra token: the slot index (b * (K_max + 1) + kc) of its row; else -1
    double S_p, S_q;    // row sums relative to the references
};

// Per (sequence, slot), written by the chunk-0 workgroup of the slot: the two
// logits at the draft token, that position's uniform and whether the token is
// in range, so that the decision reads nothing that depends on the packed
// offsets. The extra-token slot carries only its uniform.
struct alignas(16) SlotRec {
    float xt, xd;
    float u;
    int32_t yok;
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

// Exact two-pass partial of row[beg, end): maximum first (NaN ignored, NaN
// presence recorded), then the sum relative to floor(max * c).
template <class E, bool VEC>
__device__ Partial chunk_stats_exact(const typename E::raw* row, int beg, int end, float c,
                                     double* redd, float* redf, int* redi) {
    constexpr int EV = E::kVec;
    const int nvec = (end - beg + EV - 1) / EV;
    float m = -INFINITY;
    int nan_seen = 0;
    for (int vi = threadIdx.x; vi < nvec; vi += kBlock) {
        float f[EV];
        load_vec<E, VEC>(row, beg, end, vi, f);
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
    const float o = floorf(m * c);
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

template <class E, int NR, int U>
__device__ __forceinline__ void accumulate(const uint4 (&v)[NR * U], const float (&o)[NR], float c,
                                           float (&acc)[NR][E::kVec]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float f[E::kVec];
            E::unpack(v[r * U + u], f);
#pragma unroll
            for (int e = 0; e < E::kVec; ++e) acc[r][e] += fast_exp2(__builtin_fmaf(f[e], c, -o[r]));
        }
}

// One-pass partials of NR rows over [beg, end). The reference of a row is the
// integer floor(m0 * c), m0 the largest logit of the chunk's first 16-byte
// vector (every lane reads that one cache line). A non-finite sum, a non-finite
// reference or a sum beyond 2^64 sends that row to the exact two-pass path.
template <class E, bool VEC, int NR, int U = kU>
__device__ void chunk_stats(const typename E::raw* const (&rows)[NR], int beg, int end, float c,
                            Partial (&out)[NR], double* redd, float* redf, int* redi) {
    constexpr int EV = E::kVec;
    const int nvec = (end - beg + EV - 1) / EV;
    float o[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float f[EV];
        load_vec<E, VEC>(rows[r], beg, end, 0, f);
        float m = f[0];
#pragma unroll
        for (int e = 1; e < EV; ++e) m = fmaxf(m, f[e]);
        o[r] = floorf(m * c);
    }
    float acc[NR][EV];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[r][e] = 0.f;

    int vdone = 0;
    if (VEC) {
        constexpr int step = kBlock * U;
        const int full = nvec / step;
        const typename E::raw* base[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) base[r] = rows[r] + beg;
        pipelined_steps<NR * U>(
            full,
            [&](uint4 (&buf)[NR * U], int rd) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int r = 0; r < NR; ++r)
                        buf[r * U + u] = load16(base[r], rd * step + u * kBlock + threadIdx.x);
            },
            [&](const uint4 (&buf)[NR * U], int) { accumulate<E, NR, U>(buf, o, c, acc); });
        vdone = full * step;
    }
    // ragged tail (the whole range in the element-wise path)
    for (int vi = vdone + threadIdx.x; vi < nvec; vi += kBlock) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float f[EV];
            load_vec<E, VEC>(rows[r], beg, end, vi, f);
#pragma unroll
            for (int e = 0; e < EV; ++e) acc[r][e] += fast_exp2(__builtin_fmaf(f[e], c, -o[r]));
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < EV; ++e) s += (double)acc[r][e];
        const double S = block_sum(s, redd);
        if (isfinite(o[r]) && isfinite(S) && S < kFastSumLimit) {
            out[r].o = o[r];
            out[r].pad = 0.f;
            out[r].S = S;
        } else {
            out[r] = chunk_stats_exact<E, VEC>(rows[r], beg, end, c, redd, redf, redi);
        }
    }
}

#ifndef SD_SPLIT_UNROLL
#define SD_SPLIT_UNROLL SD_STATS_UNROLL
#endif
constexpr int kSplitU = SD_SPLIT_UNROLL;

template <class E, bool VEC, bool SPLIT>
__global__ __launch_bounds__(kBlock) void k_chain_stats(
    const typename E::raw* __restrict__ tgt, const typename E::raw* __restrict__ dft,
    const int32_t* __restrict__ tok, const float* __restrict__ uni, const int32_t* __restrict__ cu,
    int K_max, int V, int chunk, int n_chunks, float c, Partial* __restrict__ part_t,
    Partial* __restrict__ part_d, SlotRec* __restrict__ rec, int slot_lo, int slot_span,
    const int32_t* __restrict__ alive) {
    __shared__ double redd[kWavesPerBlock];
    __shared__ float redf[kWavesPerBlock];
    __shared__ int redi[kWavesPerBlock];
    const int slots = K_max + 1;
    const int ch = blockIdx.x % n_chunks;
    // SPLIT: one row per workgroup (kind 0 the target row, kind 1 the draft
    // row); else the slot's target and draft rows in one workgroup (kind 2)
    const int kind = SPLIT ? (blockIdx.x / n_chunks) & 1 : 2;
    const int rest = blockIdx.x / n_chunks / (SPLIT ? 2 : 1);
    const int s = slot_lo + rest % slot_span;
    const int b = rest / slot_span;
    if (alive != nullptr && alive[b] == 0) return;     // decided in an earlier phase
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    if (s > k || (kind == 1 && s == k)) return;        // the extra row has no draft row
    const int64_t slot_id = (int64_t)b * slots + s;
    const int64_t t_row = (int64_t)d0 + b + s;
    const int64_t d_row = (int64_t)d0 + s;
    const int beg = ch * chunk;
    const int end = min(V, beg + chunk);
    const typename E::raw* tp = tgt + t_row * (int64_t)V;
    const typename E::raw* dp = s < k ? dft + d_row * (int64_t)V : nullptr;
    if (kind != 1 && ch == 0 && threadIdx.x == 0) {
        SlotRec r{NAN, NAN, uni[t_row], 0};
        if (s < k) {
            const int y = tok[d_row];
            if (y >= 0 && y < V) {
                r.xt = E::at(tp, y);
                r.xd = E::at(dp, y);
                r.yok = 1;
            }
        }
        rec[slot_id] = r;
    }
    if (!SPLIT && s < k) {
        const typename E::raw* rows[2] = {tp, dp};
        Partial out[2];
        chunk_stats<E, VEC, 2>(rows, beg, end, c, out, redd, redf, redi);
        if (threadIdx.x == 0) {
            part_t[slot_id * n_chunks + ch] = out[0];
            part_d[slot_id * n_chunks + ch] = out[1];
        }
    } else {
        const typename E::raw* rows[1] = {kind == 1 ? dp : tp};
        Partial out[1];
        chunk_stats<E, VEC, 1, SPLIT ? kSplitU : kU>(rows, beg, end, c, out, redd, redf, redi);
        if (threadIdx.x == 0) (kind == 1 ? part_d : part_t)[slot_id * n_chunks + ch] = out[0];
    }
}

constexpr int kRegChunks = 8;          // partials of a row loaded together

// The first kRegChunks partials of a row (n_chunks >= 1), loaded without
// branches so that several rows' loads are in flight together: an index past
// the row's chunks reads its last chunk again, and that copy is ignored.
__device__ __forceinline__ void load_partials(const Partial* p, int n_chunks, Partial (&q)[kRegChunks]) {
#pragma unroll
    for (int i = 0; i < kRegChunks; ++i) q[i] = p[i < n_chunks ? i : n_chunks - 1];
}

// Row statistics from its chunk partials (the first kRegChunks in q, the rest
// read from p). References are integers, so each partial is rescaled exactly
// by a power of two (fixed chunk order, fp64).
__device__ RowStat combine_loaded(const Partial (&q)[kRegChunks], const Partial* p, int n_chunks) {
    RowStat r;
    r.O = -INFINITY;
    r.S = 0.0;
    r.valid = true;
#pragma unroll
    for (int i = 0; i < kRegChunks; ++i)
        if (i < n_chunks) {
            if (!isfinite(q[i].S)) r.valid = false;
            if (q[i].S > 0.0) r.O = fmaxf(r.O, q[i].o);
        }
    for (int i = kRegChunks; i < n_chunks; ++i) {
        const Partial t = p[i];
        if (!isfinite(t.S)) r.valid = false;
        if (t.S > 0.0) r.O = fmaxf(r.O, t.o);
    }
    if (!r.valid || r.O == -INFINITY) {
        r.valid = false;
        return r;
    }
    double S = 0.0;
#pragma unroll
    for (int i = 0; i < kRegChunks; ++i)
        if (i < n_chunks && q[i].S > 0.0) S += ldexp(q[i].S, (int)fmaxf(q[i].o - r.O, -4096.f));
    for (int i = kRegChunks; i < n_chunks; ++i) {
        const Partial t = p[i];
        if (t.S > 0.0) S += ldexp(t.S, (int)fmaxf(t.o - r.O, -4096.f));
    }
    r.S = S;
    r.valid = isfinite(S) && S > 0.0;
    return r;
}

__device__ RowStat combine_row(const Partial* p, int n_chunks) {
    Partial q[kRegChunks];
    load_partials(p, n_chunks, q);
    return combine_loaded(q, p, n_chunks);
}

// Sampling weight of one token in fp32: the normalised residual max(p - q, 0)
// (Q), or p itself (!Q: the extra token, and a residual whose q counts as 0,
// since max(p - 0, 0) rounds to p). It is computed as scale * u with the
// unscaled u = max(e_p * r - e_q, 0), r = S_q / S_p, scale = 1 / S_q (Q), or
// u = e_p, scale = 1 / S_p (!Q), where e = 2^(x c - O): one multiply per
// 16-byte vector instead of one per token. The mass pass and the final scan
// form a lane's sum the same way (scale times the fp32 sum of u), so both see
// bit-identical lane sums. Q is a template argument: the streaming loops hold
// no per-token branch on the row kind.
struct WeightFn {
    float c, Op, Oq, r, scale;
    bool has_q;
};

template <bool Q>
__device__ __forceinline__ float weight_u(const WeightFn& w, float xp, float xq) {
    const float ep = fast_exp2(__builtin_fmaf(xp, w.c, -w.Op));
    if (!Q) return ep;
    const float eq = fast_exp2(__builtin_fmaf(xq, w.c, -w.Oq));
    return fmaxf(__builtin_fmaf(ep, w.r, -eq), 0.f);          // S_q * max(p - q, 0)
}

template <bool Q>
__device__ __forceinline__ float weight(const WeightFn& w, float xp, float xq) {
    return weight_u<Q>(w, xp, xq) * w.scale;
}

__device__ __forceinline__ WeightFn weight_fn(const ChainDesc& d, float c, bool use_p) {
    WeightFn w;
    w.c = c;
    w.Op = d.O_p;
    w.has_q = !use_p && d.mode == kModeResidual && d.d_row >= 0;
    w.Oq = d.O_q;
    w.r = w.has_q ? (float)(d.S_q / d.S_p) : 0.f;
    w.scale = w.has_q ? (float)(1.0 / d.S_q) : (float)(1.0 / d.S_p);
    return w;
}

// Sum of the weights of one lane's 16-byte vector: scale times the fp32 sum
// of the unscaled weights in element order.
template <class E, bool Q>
__device__ __forceinline__ float lane_weight_sum(const float (&fp)[E::kVec], const float (&fq)[E::kVec],
                                                 const WeightFn& wf) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) s += weight_u<Q>(wf, fp[e], fq[e]);
    return s * wf.scale;
}

constexpr int kResolveThreads = kBlock;
constexpr int kMassChunkVecs = 2048;      // 16-byte vectors per mass workgroup
#ifndef SD_MASS_UNROLL
#define SD_MASS_UNROLL 2
#endif
constexpr int kMU = SD_MASS_UNROLL;       // pieces per wave per round of the mass pass
// One workgroup per sequence for the decision, the mass and the final draw,
// when the batch alone fills the device (or one mass chunk covers the row).
#ifndef SD_FUSED_THREADS
#define SD_FUSED_THREADS 512
#endif
#ifndef SD_FUSED_MIN_B
#define SD_FUSED_MIN_B 256
#endif
constexpr int kFusedThreads = SD_FUSED_THREADS;
constexpr int kLdsPieces = 1024;          // piece masses kept in LDS up to this many
constexpr int kFusedMinB = SD_FUSED_MIN_B;

// Weight mass of every piece (64 consecutive 16-byte vectors: 512 bf16 or 256
// fp32 tokens) of tokens [beg, end) of the decision row(s), written to
// pieces[beg / piece_tokens ..]. Coalesced 16-byte loads, the next round in
// flight while the current one is weighed; wave w of round rd, unroll u
// covers piece (rd * U + u) * waves + w of the range. `beg` is a multiple of
// the piece size.
template <class E, bool VEC, int T, bool Q>
__device__ void mass_pass(const typename E::raw* tp, const typename E::raw* dp, int beg, int end,
                          const WeightFn& wf, double* pieces, int npieces) {
    constexpr int EV = E::kVec;
    constexpr int waves = T / kWave;
    constexpr int step = T * kMU;
    constexpr int NR = Q ? 2 : 1;     // rows streamed: target, and draft for the residual
    const int nvec = (end - beg + EV - 1) / EV;
    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int p0 = beg / (kWave * EV);
    const int rounds = (nvec + step - 1) / step;
    const typename E::raw* tb = tp + beg;
    const typename E::raw* db = dp + beg;
    static_assert(kMU == 2 || kMU == 4, "the piece reduction sums two or four pieces at once");
    // loads of one round: kMU vectors of the target row, then kMU of the draft
    // row (only the last, partial round checks the row's end)
    auto fetch = [&](uint4 (&v)[NR * kMU], int rd, bool check) {
#pragma unroll
        for (int u = 0; u < kMU; ++u) {
            const int vi = rd * step + u * T + threadIdx.x;
            if (VEC) {
                const bool in = !check || vi < nvec;
                v[u] = in ? load16(tb, vi) : E::neg_inf();
                if (Q) v[NR * kMU - kMU + u] = in ? load16(db, vi) : E::neg_inf();
            }
        }
    };
    auto weigh = [&](const uint4 (&v)[NR * kMU], int rd) {
        double s[kMU];
#pragma unroll
        for (int u = 0; u < kMU; ++u) {
            float fp[EV], fq[EV];
            if (VEC) {
                E::unpack(v[u], fp);
                if (Q) E::unpack(v[NR * kMU - kMU + u], fq);
            } else {
                const int vi = rd * step + u * T + threadIdx.x;
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const int j = beg + vi * EV + e;
                    fp[e] = (vi < nvec && j < end) ? E::at(tp, j) : -INFINITY;
                    if (Q) fq[e] = (vi < nvec && j < end) ? E::at(dp, j) : -INFINITY;
                }
            }
            s[u] = (double)lane_weight_sum<E, Q>(fp, fq, wf);
        }
        // kMU wave sums at once (reduce-scatter): halves of the wave trade half
        // of the sums, (with four) quarters one, then a butterfly over the
        // rest; lane (64 / kMU) * i ends with the sum of piece i of the round.
        const bool h32 = (lane & 32) != 0;
        double t;
        int u;
        if (kMU == 4) {
            const bool h16 = (lane & 16) != 0;
            const double r0 = __shfl_xor(h32 ? s[0] : s[kMU / 2], 32, kWave);
            const double r1 = __shfl_xor(h32 ? s[1] : s[kMU - 1], 32, kWave);
            const double a0 = (h32 ? s[kMU / 2] : s[0]) + r0;
            const double a1 = (h32 ? s[kMU - 1] : s[1]) + r1;
            const double r2 = __shfl_xor(h16 ? a0 : a1, 16, kWave);
            t = (h16 ? a1 : a0) + r2;
            u = (h32 ? 2 : 0) + (h16 ? 1 : 0);
        } else {
            const double r0 = __shfl_xor(h32 ? s[0] : s[kMU - 1], 32, kWave);
            t = (h32 ? s[kMU - 1] : s[0]) + r0;
            const double r1 = __shfl_xor(t, 16, kWave);
            t += r1;
            u = h32 ? 1 : 0;
        }
#if SD_MASS_DPP
        t = row_sum_f64(t);                 // the rest within each row of 16 lanes
#else
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) t += __shfl_xor(t, o, kWave);
#endif
        const int piece = p0 + (rd * kMU + u) * waves + w;
        if ((lane & (kWave / kMU - 1)) == 0 && piece < npieces) pieces[piece] = t;
    };
    const int full = VEC ? nvec / step : 0;
    pipelined_steps<NR * kMU>(
        full, [&](uint4 (&v)[NR * kMU], int rd) { fetch(v, rd, false); }, weigh);
    for (int rd = full; rd < rounds; ++rd) {
        uint4 v[NR * kMU];
        fetch(v, rd, true);
        weigh(v, rd);
    }
}

// Scans one piece (64 lanes x one 16-byte vector, tokens e0 ..) from cumulative
// mass `before`: the first token whose running mass exceeds `target`, or the
// last token of the piece with positive weight. One wave (all lanes active).
template <class E, bool VEC, bool Q>
__device__ int scan_piece(const typename E::raw* tp, const typename E::raw* dp, int e0, int V,
                          const WeightFn& wf, double before, double target, bool take_last) {
    constexpr int EV = E::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int j0 = e0 + lane * EV;
    float fp[EV], fq[EV];
    if (VEC) {                  // (e0 is a multiple of the piece size, V of the vector size)
        const bool in = j0 < V;
        E::unpack(in ? load16_cached(tp, j0 / EV) : E::neg_inf(), fp);
        if (Q) E::unpack(in ? load16_cached(dp, j0 / EV) : E::neg_inf(), fq);
    } else {
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const int j = j0 + e;
            fp[e] = (j < V) ? E::at(tp, j) : -INFINITY;
            fq[e] = (Q && j < V) ? E::at(dp, j) : -INFINITY;
        }
    }
    float w[EV];
    float us = 0.f;
    int lastpos = -1;
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const float uw = weight_u<Q>(wf, fp[e], fq[e]);
        us += uw;
        w[e] = uw * wf.scale;
        if (w[e] > 0.f) lastpos = j0 + e;
    }
    const float ls = us * wf.scale;         // the lane sum exactly as the mass pass formed it
    const int last_any = (int)wave_max_u32((uint32_t)(lastpos + 1)) - 1;
    if (take_last) return last_any;
    const double incl = wave_incl_scan_f64((double)ls);
    const double start = before + (incl - (double)ls);
    const unsigned long long m = __ballot(start + (double)ls > target);
    if (!m) return last_any;
    const int L = __ffsll(m) - 1;
    int pick = -1;
    if (lane == L) {
        double run = start;
        int lp = -1;
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            run += (double)w[e];
            if (w[e] > 0.f) lp = j0 + e;
            if (pick < 0 && run > target && w[e] > 0.f) pick = j0 + e;
        }
        if (pick < 0) pick = lp;
    }
    pick = __shfl(pick, L, kWave);
    return pick >= 0 ? pick : last_any;
}

// Inverse CDF in token order from the piece masses: the first token whose
// running mass exceeds u * total. One wave. Returns -1 when total is 0.
template <class E, bool VEC, bool Q>
__device__ int sample_from_pieces(const double* S, int npieces, const typename E::raw* tp,
                                  const typename E::raw* dp, int V, const WeightFn& wf, double u,
                                  double* total_out, int p_base = 0) {
    constexpr int EV = E::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int per = (npieces + kWave - 1) / kWave;
    const int s0 = min(npieces, lane * per), s1 = min(npieces, s0 + per);
    double mine = 0.0;
    int lastpos = -1;
    for (int i = s0; i < s1; ++i) {
        mine += S[i];
        if (S[i] > 0.0) lastpos = i;
    }
    const double incl = wave_incl_scan_f64(mine);
    const double excl = incl - mine;
    const double total = __shfl(incl, kWave - 1, kWave);
    *total_out = total;
    if (!(total > 0.0)) return -1;
    const double target = u * total;
    int hit = -1;
    double before = 0.0, run = excl;
    for (int i = s0; i < s1; ++i) {
        if (run + S[i] > target && S[i] > 0.0) {
            hit = i;
            before = run;
            break;
        }
        run += S[i];
    }
    const unsigned long long m = __ballot(hit >= 0);
    bool take_last = false;
    int piece;
    if (m) {
        const int L = __ffsll(m) - 1;
        piece = __shfl(hit, L, kWave);
        before = __shfl(before, L, kWave);
    } else {
        piece = (int)wave_max_u32((uint32_t)(lastpos + 1)) - 1;   // rounding left the point past the end
        take_last = true;
    }
    return scan_piece<E, VEC, Q>(tp, dp, (p_base + piece) * kWave * EV, V, wf, before, target, take_last);
}

// The chunk of an extra-token row that holds its draw, from the row's chunk
// partials: the chunk masses relative to the row reference O (as the row's
// sum combines them), their running sum in chunk order, and the first chunk
// whose running mass passes u times the total. *frac gets the draw's place
// within that chunk (in [0, 1]); -1 when no chunk has mass. One wave.
__device__ int extra_chunk(const Partial* p, int n_chunks, float O, double u, double* frac) {
    const int lane = threadIdx.x & (kWave - 1);
    auto mass = [&](int i) -> double {
        if (i >= n_chunks) return 0.0;
        const Partial q = p[i];
        return q.S > 0.0 ? ldexp(q.S, (int)fmaxf(q.o - O, -4096.f)) : 0.0;
    };
    double total = 0.0;
    for (int base = 0; base < n_chunks; base += kWave) total += wave_sum(mass(base + lane));
    const double target = u * total;
    double run = 0.0;
    int last = -1;
    for (int base = 0; base < n_chunks; base += kWave) {
        const double m = mass(base + lane);
        const double incl = wave_incl_scan_f64(m);
        const double start = run + (incl - m);
        const unsigned long long hit = __ballot(m > 0.0 && start + m > target);
        if (hit) {
            const int L = __ffsll(hit) - 1;
            const double ms = __shfl(m, L, kWave), st = __shfl(start, L, kWave);
            const double f = (target - st) / ms;
            *frac = f < 0.0 ? 0.0 : (f > 1.0 ? 1.0 : f);
            return base + L;
        }
        last = max(last, (int)wave_max_u32((uint32_t)(m > 0.0 ? base + lane + 1 : 0)) - 1);
        run += __shfl(incl, kWave - 1, kWave);
    }
    *frac = 1.0;                        // rounding left the point past the end
    return last;
}

// Inverse CDF over the whole decision row with the piece masses computed on
// the fly by one wave (used only when the residual came out with no mass).
template <class E>
__device__ int sample_by_rescan(const typename E::raw* tp, int V, const WeightFn& wf, double u) {
    constexpr int EV = E::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int pe = kWave * EV;
    const int np = (V + pe - 1) / pe;
    auto piece_mass = [&](int i) -> double {
        const int j0 = i * pe + lane * EV;
        float fp[EV], fq[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            fp[e] = (j0 + e < V) ? E::at(tp, j0 + e) : -INFINITY;
            fq[e] = -INFINITY;
        }
        return wave_sum((double)lane_weight_sum<E, false>(fp, fq, wf));
    };
    double total = 0.0;
    int last = -1;
    for (int i = 0; i < np; ++i) {
        const double m = piece_mass(i);
        total += m;
        if (m > 0.0) last = i;
    }
    if (!(total > 0.0)) return -1;
    const double target = u * total;
    double run = 0.0;
    for (int i = 0; i < np; ++i) {
        const double m = piece_mass(i);
        if (run + m > target && m > 0.0) return scan_piece<E, false, false>(tp, tp, i * pe, V, wf, run, target, false);
        run += m;
    }
    return scan_piece<E, false, false>(tp, tp, last * pe, V, wf, 0.0, target, true);
}

#ifndef SD_DECIDE_SEQS
#define SD_DECIDE_SEQS 2
#endif
constexpr int kSeqPerBlock = SD_DECIDE_SEQS;     // decide / sample: one wave per sequence

// Inputs and outputs of the per-sequence decision.
struct DecideArgs {
    const Partial* part_t;
    const Partial* part_d;
    const SlotRec* rec;
    const float* uni;
    const int32_t* cu;
    int K_max, V, n_chunks, chunk;
    float c;
    int32_t* A_out;
    float* probs_out;
    int32_t* status_out;
    const int32_t* cap;
    int32_t* A_full_out;
    int hi;             // slots streamed so far (the phase's upper bound)
    int32_t* alive;     // per-sequence flag across phases, or null
};

// The decision of sequence b from the row partials (one wave): combines the
// partials of each row, evaluates p_i(y_i) and q_i(y_i) in fp64, the accept
// bits and A (wave ballot); stores A, the status bits and the probabilities,
// and returns in d the descriptor of the row(s) the final token is drawn
// from. Returns false, with the sequence marked alive, when every position
// streamed so far passed and later slots remain.
__device__ __forceinline__ bool decide_sequence(const DecideArgs& g, int b, ChainDesc& d) {
    const Partial* __restrict__ part_t = g.part_t;
    const Partial* __restrict__ part_d = g.part_d;
    const SlotRec* __restrict__ rec = g.rec;
    const float* __restrict__ uni = g.uni;
    const int K_max = g.K_max, n_chunks = g.n_chunks, hi = g.hi;
    const float c = g.c;
    float* __restrict__ probs_out = g.probs_out;
    int32_t* __restrict__ alive = g.alive;
    const int lane = threadIdx.x & (kWave - 1);
    const int slots = K_max + 1;
    const int64_t slot0 = (int64_t)b * slots;
    // Lane s combines the partials of slot s (target, and draft below K_max)
    // and reads the slot's record, for every slot streamed so far. Every lane
    // issues its loads at once, with no branch between them (a lane past the
    // streamed slots reads the last one's, a slot without a draft row reads
    // memory it never uses), and none of them waits for cu: one round trip.
    const int ns = slots < hi ? slots : hi;
    const int ls = lane < ns ? lane : ns - 1;
    Partial qt[kRegChunks], qd[kRegChunks];
    load_partials(part_t + (slot0 + ls) * n_chunks, n_chunks, qt);
    load_partials(part_d + (slot0 + ls) * n_chunks, n_chunks, qd);
    const SlotRec r_ls = rec[slot0 + ls];
    int d0, k;
    seq_range(g.cu, b, K_max, d0, k);
    RowStat rp{-INFINITY, 0.0, false}, rq{-INFINITY, 0.0, false};
    SlotRec r{0.f, 0.f, 0.f, 0};
    if (lane < ns) {
        rp = combine_loaded(qt, part_t + (slot0 + lane) * n_chunks, n_chunks);
        r = r_ls;
        if (lane < K_max) rq = combine_loaded(qd, part_d + (slot0 + lane) * n_chunks, n_chunks);
    }
    // positions evaluated so far: those of the slots streamed up to this phase
    const int kk = k < hi ? k : hi;
    // uniform of position `lane` (streamed slots; lane k_b's is the final draw's
    // for an uncapped window)
    const float u_lane = (lane <= k && lane < ns) ? r.u : 0.f;
    const float xt = r.xt, xd = r.xd;
    bool acc = true;
    int st = 0;
    if (lane < kk) {
        const bool yok = r.yok != 0;
        double py = 0.0, qy = 0.0;
        // the summed terms' fp32 reference, evaluated exactly in fp64
        if (yok && rp.valid) py = exp2((double)xt * (double)c - (double)rp.O) / rp.S;
        if (yok && rq.valid) qy = exp2((double)xd * (double)c - (double)rq.O) / rq.S;
        const double u = (double)u_lane;
        acc = rp.valid && rq.valid && yok && py > 0.0 && u * qy <= py;
        st = (yok ? 0 : 1) | ((rp.valid && rq.valid) ? 0 : 2);
        if (probs_out) {
            probs_out[2 * (int64_t)(d0 + lane)] = (float)py;
            probs_out[2 * (int64_t)(d0 + lane) + 1] = (float)qy;
        }
    }
    const unsigned long long rej = __ballot(!acc);
    if (rej == 0ull && k >= hi) {                       // every position so far passed: next phase
        if (lane == 0) alive[b] = 1;
        return false;
    }
    if (alive != nullptr && lane == 0) alive[b] = 0;
    const int A_full = rej ? (__ffsll(rej) - 1) : k;
    const int kc = committed_len(g.cap, b, k);
    const int A = A_full < kc ? A_full : kc;
    int mine = (lane < kc && lane <= A) ? st : 0;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) mine |= __shfl_xor(mine, o, kWave);
    d.A = A;
    // the final draw's uniform: from its slot's record when that slot was
    // streamed (and is a lane), else from the uniforms (a window rejected
    // before its later slots were streamed, or a 64-position window)
    d.u = (kc < ns && kc < kWave) ? __shfl(u_lane, kc, kWave) : uni[d0 + b + kc];
    d.slot = -1;
    if (A < kc) {
        const float Op = __shfl(rp.O, A, kWave);
        const double Sp = __shfl(rp.S, A, kWave);
        const bool vp = __shfl((int)rp.valid, A, kWave) != 0;
        const float Oq = __shfl(rq.O, A, kWave);
        const double Sq = __shfl(rq.S, A, kWave);
        const bool vq = __shfl((int)rq.valid, A, kWave) != 0;
        d.mode = vp ? kModeResidual : kModeNone;
        d.t_row = d0 + b + A;
        d.d_row = vq ? d0 + A : -1;
        d.O_p = Op;
        d.S_p = Sp;
        d.O_q = Oq;
        d.S_q = Sq;
    } else {
        // the extra-token row: slot kc, streamed in this phase (kc <= k < hi)
        RowStat rb;
        if (kc < kWave) {
            rb.O = __shfl(rp.O, kc, kWave);
            rb.S = __shfl(rp.S, kc, kWave);
            rb.valid = __shfl((int)rp.valid, kc, kWave) != 0;
        } else {
            rb = combine_row(part_t + (slot0 + kc) * n_chunks, n_chunks);
        }
        d.mode = rb.valid ? kModeExtra : kModeNone;
        if (!rb.valid) mine |= 2;
        d.slot = (int32_t)(slot0 + kc);
        d.t_row = d0 + b + kc;
        d.d_row = -1;
        d.O_p = rb.O;
        d.S_p = rb.S;
        d.O_q = 0.f;
        d.S_q = 0.0;
    }
    if (lane == 0) {
        g.A_out[b] = A;
        if (g.A_full_out) g.A_full_out[b] = A_full;
        if (g.status_out) g.status_out[b] = mine;
    }
    return true;
}

// One wave per sequence: the decision after a phase; the descriptor goes to
// the workspace for the launches that draw the final token.
__global__ __launch_bounds__(kSeqPerBlock * kWave) void k_chain_decide(DecideArgs g, int B, int alive_in,
                                                         ChainDesc* __restrict__ desc) {
    const int b = blockIdx.x * kSeqPerBlock + threadIdx.x / kWave;
    if (b >= B) return;
    if (alive_in && g.alive[b] == 0) return;            // decided in an earlier phase
    ChainDesc d;
    if (decide_sequence(g, b, d) && (threadIdx.x & (kWave - 1)) == 0) desc[b] = d;
}

// grid (sequence, chunk of 16-byte vectors: 4096 per workgroup): re-reads only
// the decision row(s) of the sequence and writes the weight mass of the
// residual (or of p for the extra token) per 512-token piece.
template <class E, bool VEC>
__global__ __launch_bounds__(kResolveThreads) void k_chain_mass(
    const typename E::raw* __restrict__ tgt, const typename E::raw* __restrict__ dft,
    const ChainDesc* __restrict__ desc, int V, int mchunk, int n_mchunks, float c,
    double* __restrict__ piece_ws) {
    constexpr int EV = E::kVec;
    const int b = blockIdx.x / n_mchunks;
    const int mc = blockIdx.x % n_mchunks;
    const ChainDesc d = desc[b];
    if (d.mode == kModeNone) return;
    const int npieces = (V + kWave * EV - 1) / (kWave * EV);
    const typename E::raw* tp = tgt + (int64_t)d.t_row * V;
    const WeightFn wf = weight_fn(d, c, false);
    const typename E::raw* dp = wf.has_q ? dft + (int64_t)d.d_row * V : tp;
    const int beg = mc * mchunk;
    const int end = min(V, beg + mchunk);
    double* pieces = piece_ws + (int64_t)b * npieces;
    if (wf.has_q) mass_pass<E, VEC, kResolveThreads, true>(tp, dp, beg, end, wf, pieces, npieces);
    else mass_pass<E, VEC, kResolveThreads, false>(tp, dp, beg, end, wf, pieces, npieces);
}

// One wave per sequence: the final token from the piece masses (inverse CDF in
// token order at u_k times the total). The rare case of a residual with no
// mass (rounding) is redrawn from p of the decision row by the same wave.
template <class E, bool VEC>
__global__ __launch_bounds__(kSeqPerBlock * kWave) void k_chain_sample(
    const typename E::raw* __restrict__ tgt, const typename E::raw* __restrict__ dft,
    const ChainDesc* __restrict__ desc, const double* __restrict__ piece_ws, int B, int V,
    float c, int32_t* __restrict__ next_out, float* __restrict__ R_out) {
    constexpr int EV = E::kVec;
    const int b = blockIdx.x * kSeqPerBlock + threadIdx.x / kWave;
    if (b >= B) return;
    const int lane = threadIdx.x & (kWave - 1);
    const ChainDesc d = desc[b];
    int next = -1;
    double total = 0.0;
    if (d.mode != kModeNone) {
        const int npieces = (V + kWave * EV - 1) / (kWave * EV);
        const typename E::raw* tp = tgt + (int64_t)d.t_row * V;
        const WeightFn wf = weight_fn(d, c, false);
        const typename E::raw* dp = wf.has_q ? dft + (int64_t)d.d_row * V : tp;
        const double* pieces = piece_ws + (int64_t)b * npieces;
        next = wf.has_q ? sample_from_pieces<E, VEC, true>(pieces, npieces, tp, dp, V, wf, (double)d.u, &total)
                        : sample_from_pieces<E, VEC, false>(pieces, npieces, tp, dp, V, wf, (double)d.u, &total);
        if (d.mode == kModeResidual && !(total > 0.0))
            next = sample_by_rescan<E>(tp, V, weight_fn(d, c, true), (double)d.u);
    }
    if (lane == 0) {
        next_out[b] = next;
        if (R_out) R_out[b] = (d.mode == kModeResidual) ? (float)total : 0.f;
    }
}

// One workgroup per sequence, after the last phase: the decision (wave 0, or
// the descriptor of an earlier phase), the weight mass per piece of the
// decision row(s) by every wave, then the final draw by wave 0. The piece
// masses stay in LDS (or, for a very long row, go through the workspace: the
// workgroup's own stores are visible to it after the barrier).
template <class E, bool VEC>
__global__ __launch_bounds__(kFusedThreads) void k_chain_resolve(
    const typename E::raw* __restrict__ tgt, const typename E::raw* __restrict__ dft,
    DecideArgs g, int alive_in, const ChainDesc* __restrict__ desc,
    double* __restrict__ piece_ws, int32_t* __restrict__ next_out, float* __restrict__ R_out) {
    constexpr int EV = E::kVec;
    __shared__ ChainDesc sdesc;
    __shared__ double spieces[kLdsPieces];
    __shared__ int s_xc;
    __shared__ double s_frac;
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    if (threadIdx.x < kWave) {
        ChainDesc d;
        if (alive_in && g.alive[b] == 0) d = desc[b];   // decided in an earlier phase
        else decide_sequence(g, b, d);                  // the window ends here: always decides
        // an extra token is drawn from p of one row: the row's chunk partials
        // say which chunk holds the draw, and only that chunk is weighed (a
        // row of one chunk is weighed whole)
        int xc = -1;
        double fr = 0.0;
        if (d.mode == kModeExtra && g.n_chunks > 1)
            xc = extra_chunk(g.part_t + (int64_t)d.slot * g.n_chunks, g.n_chunks, d.O_p, (double)d.u, &fr);
        if (lane == 0) {
            sdesc = d;
            s_xc = xc;
            s_frac = fr;
        }
    }
    __syncthreads();
    const ChainDesc d = sdesc;
    const int xc = s_xc;
    if (d.mode == kModeNone) {
        if (threadIdx.x == 0) {
            next_out[b] = -1;
            if (R_out) R_out[b] = 0.f;
        }
        return;
    }
    const int V = g.V;
    const int npieces = (V + kWave * EV - 1) / (kWave * EV);
    const typename E::raw* tp = tgt + (int64_t)d.t_row * V;
    const WeightFn wf = weight_fn(d, g.c, false);
    const typename E::raw* dp = wf.has_q ? dft + (int64_t)d.d_row * V : tp;
    double* pieces = npieces <= kLdsPieces ? spieces : piece_ws + (int64_t)b * npieces;
    if (xc >= 0) {
        // (a chunk is a whole number of pieces)
        const int beg = xc * g.chunk;
        const int end = min(V, beg + g.chunk);
        mass_pass<E, VEC, kFusedThreads, false>(tp, dp, beg, end, wf, pieces, (end + kWave * EV - 1) / (kWave * EV));
    } else if (wf.has_q) {
        mass_pass<E, VEC, kFusedThreads, true>(tp, dp, 0, V, wf, pieces, npieces);
    } else {
        mass_pass<E, VEC, kFusedThreads, false>(tp, dp, 0, V, wf, pieces, npieces);
    }
    __syncthreads();
    if (threadIdx.x >= kWave) return;
    double total = 0.0;
    int next;
    if (xc >= 0) {
        const int p0 = xc * g.chunk / (kWave * EV);
        const int p1 = (min(V, (xc + 1) * g.chunk) + kWave * EV - 1) / (kWave * EV);
        next = sample_from_pieces<E, VEC, false>(pieces + p0, p1 - p0, tp, dp, V, wf, s_frac, &total, p0);
        // no fp32 weight in the chunk (its mass is below fp32's range): the
        // whole row, one wave
        if (next < 0) next = sample_by_rescan<E>(tp, V, wf, (double)d.u);
    } else {
        next = wf.has_q ? sample_from_pieces<E, VEC, true>(pieces, npieces, tp, dp, V, wf, (double)d.u, &total)
                        : sample_from_pieces<E, VEC, false>(pieces, npieces, tp, dp, V, wf, (double)d.u, &total);
        if (d.mode == kModeResidual && !(total > 0.0))
            next = sample_by_rescan<E>(tp, V, weight_fn(d, g.c, true), (double)d.u);
    }
    if (lane == 0) {
        next_out[b] = next;
        if (R_out) R_out[b] = (d.mode == kModeResidual) ? (float)total : 0.f;
    }
}

}  // namespace

size_t chain_full_ws_bytes(int B, int K_max, int V, int dtype) {
    const int nc = n_chunks_for(V, dtype);
    const size_t slots = (size_t)B * (K_max + 1);
    const int ev = dtype == 1 ? 8 : 4;
    const size_t npieces = (size_t)(V + 64 * ev - 1) / (64 * ev);
    Carve cv;
    cv.take(slots * nc * sizeof(Partial));          // part_t
    cv.take(slots * nc * sizeof(Partial));          // part_d
    cv.take(slots * sizeof(SlotRec));               // slot records
    cv.take((size_t)B * npieces * sizeof(double));  // piece masses
    cv.take((size_t)B * sizeof(ChainDesc));         // decisions
    cv.take((size_t)B * sizeof(int32_t));           // still undecided after a phase
    return cv.off;
}

template <class E, bool VEC>
static hipError_t chain_full_impl(const ChainArgs& a) {
    const int nc = n_chunks_for(a.V, a.dtype);
    const int chunk = chunk_elems(a.dtype);
    const size_t slots = (size_t)a.B * (a.K_max + 1);
    const size_t npieces = (size_t)(a.V + 64 * E::kVec - 1) / (64 * E::kVec);
    Carve cv;
    char* ws = static_cast<char*>(a.ws);
    Partial* part_t = reinterpret_cast<Partial*>(ws + cv.take(slots * nc * sizeof(Partial)));
    Partial* part_d = reinterpret_cast<Partial*>(ws + cv.take(slots * nc * sizeof(Partial)));
    SlotRec* rec = reinterpret_cast<SlotRec*>(ws + cv.take(slots * sizeof(SlotRec)));
    double* pieces = reinterpret_cast<double*>(ws + cv.take((size_t)a.B * npieces * sizeof(double)));
    ChainDesc* desc = reinterpret_cast<ChainDesc*>(ws + cv.take((size_t)a.B * sizeof(ChainDesc)));
    int32_t* alive = reinterpret_cast<int32_t*>(ws + cv.take((size_t)a.B * sizeof(int32_t)));
    const int mchunk = kMassChunkVecs * E::kVec;
    const int n_mchunks = (a.V + mchunk - 1) / mchunk;
    const float c = (float)(1.4426950408889634 / (double)a.temperature);
    using raw = typename E::raw;
    const raw* tgt = static_cast<const raw*>(a.target);
    const raw* dft = static_cast<const raw*>(a.draft);
    // Positions are verified in phases: a sequence whose draft is rejected in
    // an early phase never streams its later rows. One phase when every
    // position's p(y), q(y) or the full-window rejection is asked for.
    // (only for batches large enough to be bandwidth-bound: below that the
    // extra launches cost more than the rows they save)
    const bool phased = a.probs_out == nullptr && a.cap == nullptr && a.accepted_full == nullptr &&
                        (size_t)a.B * (a.K_max + 1) * a.V >= kPhaseMinElems;
    const unsigned seq_blocks = (unsigned)((a.B + kSeqPerBlock - 1) / kSeqPerBlock);
    int bounds[kMaxPhases + 1];
    int n_phases = 0;
    bounds[0] = 0;
    if (phased)
        for (int i = 0; i < kMaxPhases - 1; ++i)
            if (kPhaseBounds[i] > bounds[n_phases] && kPhaseBounds[i] < a.K_max + 1)
                bounds[++n_phases] = kPhaseBounds[i];
    bounds[++n_phases] = a.K_max + 1;
    // The last phase's decision, the mass and the final draw run as one
    // workgroup per sequence when that fills the device, else as a decision
    // launch, a chunked mass launch and a one-wave-per-sequence draw.
    const bool fused = a.B >= kFusedMinB || n_mchunks == 1;
    DecideArgs g;
    g.part_t = part_t;
    g.part_d = part_d;
    g.rec = rec;
    g.uni = a.uniforms;
    g.cu = a.cu;
    g.K_max = a.K_max;
    g.V = a.V;
    g.n_chunks = nc;
    g.chunk = chunk;
    g.c = c;
    g.A_out = a.accepted_len;
    g.probs_out = a.probs_out;
    g.status_out = a.seq_status;
    g.cap = a.cap;
    g.A_full_out = a.accepted_full;
    g.alive = n_phases > 1 ? alive : nullptr;
    for (int ph = 0; ph < n_phases; ++ph) {
        const int lo = bounds[ph], hi = bounds[ph + 1];
        // The first phase streams every sequence's rows with one row per
        // workgroup; later phases keep a slot's two rows in one workgroup, so
        // that half as many workgroups exit at once for decided sequences.
        const bool split = ph == 0 && n_phases > 1 && kSplitFirstPhase;
        const unsigned grid1 = (unsigned)((size_t)a.B * (hi - lo) * nc * (split ? 2 : 1));
        if (ph == 0)
            PassTimer::launch(split ? k_chain_stats<E, VEC, true> : k_chain_stats<E, VEC, false>, dim3(grid1),
                              dim3(kBlock), a.stream, tgt, dft, a.tokens, a.uniforms, a.cu, a.K_max, a.V, chunk,
                              nc, c, part_t, part_d, rec, lo, hi - lo, (int32_t*)nullptr);
        else
            hipLaunchKernelGGL((k_chain_stats<E, VEC, false>), dim3(grid1), dim3(kBlock), 0, a.stream, tgt,
                               dft, a.tokens, a.uniforms, a.cu, a.K_max, a.V, chunk, nc, c, part_t, part_d, rec,
                               lo, hi - lo, alive);
        g.hi = hi;
        if (fused && ph == n_phases - 1) {
            hipLaunchKernelGGL((k_chain_resolve<E, VEC>), dim3((unsigned)a.B), dim3(kFusedThreads), 0,
                               a.stream, tgt, dft, g, ph > 0 ? 1 : 0, desc, pieces, a.next_token,
                               a.resid_mass_out);
            return hipGetLastError();
        }
        hipLaunchKernelGGL(k_chain_decide, dim3(seq_blocks), dim3(kSeqPerBlock * kWave), 0, a.stream, g, a.B,
                           ph > 0 ? 1 : 0, desc);
    }
    hipLaunchKernelGGL((k_chain_mass<E, VEC>), dim3((unsigned)((size_t)a.B * n_mchunks)),
                       dim3(kResolveThreads), 0, a.stream, tgt, dft, desc, a.V, mchunk, n_mchunks, c,
                       pieces);
    hipLaunchKernelGGL((k_chain_sample<E, VEC>), dim3(seq_blocks), dim3(kSeqPerBlock * kWave), 0, a.stream, tgt,
                       dft, desc, pieces, a.B, a.V, c, a.next_token, a.resid_mass_out);
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
